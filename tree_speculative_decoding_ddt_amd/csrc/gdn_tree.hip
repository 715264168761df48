// Branch-local short conv + Gated DeltaNet over the draft tree.
// Sources: "DDTree on vLLM: candid research notes", section "Why hybrid attention
// makes it hard": every node reads the recurrent (GDN) state and the short-conv
// state of its parent and writes its own to scratch, never to committed state;
// "The architecture of speculation", section "The DDTree Integration Challenge":
// recurrent state is per branch, not shared.
//
// Per node i (parent p; the committed state when p < 0), per head h:
//   window = [conv state of p (W-1 rows), x_i];  y = SiLU(sum_j w[c][j] window[j][c])
//   q = y[q-channels of h] * dk^-1/2;  k = y[k-channels of h] / sqrt(|k|^2 + 1e-6)
//   S_i = g S_p + beta (v - g S_p k) k^T;  o_i = S_i q = g (S_p q) + beta (v - g S_p k) (k.q)
//
// Layout of the work: a block owns one (sequence, head) and R consecutive rows of
// the [dv][dk] state; a thread owns 4 consecutive columns of one row, so the two
// row dot products (S_p k, S_p q) reduce across dk/4 lanes.  Rows of S evolve
// independently, so the tree dependency never crosses blocks.  Nodes are visited in
// depth-first order: the parent's state is then always the newest one written at
// depth d-1, so each thread keeps a private stack of (L+1) float4 slots in LDS,
// indexed by depth -- no state is re-read from memory.  Every node's state still
// goes to S_scratch (the scratch contract), as 16-byte stores.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

constexpr int kGdnThreads = 256;
constexpr int kGdnMaxW = 8;
constexpr int kGdnMaxT = 128;

template <typename A, int DK>
__global__ void __launch_bounds__(kGdnThreads) gdn_tree_kernel(const A* __restrict__ x, const float* __restrict__ conv_w,
                                                               const A* __restrict__ conv_state, A* __restrict__ conv_scratch,
                                                               const A* __restrict__ v, const float* __restrict__ beta,
                                                               const float* __restrict__ g, const float* __restrict__ S,
                                                               float* __restrict__ S_scratch, A* __restrict__ o,
                                                               const int32_t* __restrict__ parent, int Tn, int L, int H,
                                                               int C, int W) {
  constexpr int DV = DK;
  constexpr int LPR = DK / 4;              // lanes per state row
  constexpr int R = kGdnThreads / LPR;     // state rows per block
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = blockIdx.y * R + tid / LPR;
  const int c0 = (tid % LPR) * 4;
  const bool conv_writer = blockIdx.y == 0;

  extern __shared__ float4 stack[];        // [(L+1)][256]
  __shared__ float qk[2][2 * DK];
  __shared__ int par[kGdnMaxT], dep[kGdnMaxT], order[kGdnMaxT], first[kGdnMaxT], nxt[kGdnMaxT], stk[kGdnMaxT];
  __shared__ int hrow[kGdnMaxT][kGdnMaxW];  // back b from node: tree row (>= 0) or -(1 + committed row)
  __shared__ int n_order;

  for (int i = tid; i < Tn; i += kGdnThreads) {
    par[i] = parent[(size_t)s * Tn + i];
    first[i] = -1;
    nxt[i] = -1;
  }
  __syncthreads();
  if (tid == 0) {
    // child lists in increasing row order; a row whose parent is not an earlier row
    // reads the committed state (the root, and rows left unused by the build)
    for (int i = Tn - 1; i >= 1; --i) {
      const int p = par[i];
      if (p >= 0 && p < i) {
        nxt[i] = first[p];
        first[p] = i;
      }
    }
    int cnt = 0;
    for (int rt = 0; rt < Tn; ++rt) {
      const int p = par[rt];
      if (p >= 0 && p < rt) continue;
      int sp = 0;
      stk[sp++] = rt;
      dep[rt] = 0;
      for (int b = 1; b < W; ++b) hrow[rt][b] = -(1 + (W - 1 - b));
      while (sp > 0) {
        const int u = stk[--sp];
        if (dep[u] > L) continue;  // deeper than the stated bound: not processed
        order[cnt++] = u;
        for (int c = first[u]; c >= 0; c = nxt[c]) {
          dep[c] = dep[u] + 1;
          hrow[c][1] = u;
          for (int b = 2; b < W; ++b) hrow[c][b] = hrow[u][b - 1];
          stk[sp++] = c;
        }
      }
    }
    n_order = cnt;
  }

  // this thread's conv channel and taps (threads < 2*DK)
  const bool conv_thread = tid < 2 * DK;
  const int ch = tid < DK ? h * DK + tid : H * DK + h * DK + (tid - DK);
  float wt[kGdnMaxW];
#pragma unroll
  for (int j = 0; j < kGdnMaxW; ++j) wt[j] = (conv_thread && j < W) ? conv_w[(size_t)ch * W + j] : 0.f;
  __syncthreads();

  const float qscale = rsqrtf((float)DK);
  const int norder = n_order;
  for (int k = 0; k < norder; ++k) {
    const int u = order[k];
    const int d = dep[u];
    const int buf = k & 1;
    if (conv_thread) {
      float acc = 0.f;
      A win[kGdnMaxW];
#pragma unroll
      for (int j = 0; j < kGdnMaxW; ++j) {
        if (j < W) {
          const int back = W - 1 - j;
          A val;
          if (back == 0) {
            val = x[((size_t)s * Tn + u) * C + ch];
          } else {
            const int hr = hrow[u][back];
            val = hr >= 0 ? x[((size_t)s * Tn + hr) * C + ch]
                          : conv_state[((size_t)s * (W - 1) + (-hr - 1)) * C + ch];
          }
          win[j] = val;
          acc += wt[j] * Elem<A>::load(&val, 0);
        }
      }
      qk[buf][tid] = acc / (1.f + __expf(-acc));
      if (conv_writer) {
#pragma unroll
        for (int j = 1; j < kGdnMaxW; ++j)
          if (j < W) conv_scratch[(((size_t)s * Tn + u) * (W - 1) + (j - 1)) * C + ch] = win[j];
      }
    }
    __syncthreads();

    // |k|^2 and k.q over the head (every wave computes them)
    float kk = 0.f, kq = 0.f;
    for (int c = lane; c < DK; c += 64) {
      const float kv = qk[buf][DK + c], qv = qk[buf][c];
      kk += kv * kv;
      kq += kv * qv;
    }
    kk = wave_sum(kk);
    kq = wave_sum(kq);
    const float rn = 1.f / sqrtf(kk + 1e-6f);
    const float kqn = kq * rn * qscale;

    const float4 kr = *reinterpret_cast<const float4*>(&qk[buf][DK + c0]);
    const float4 qr = *reinterpret_cast<const float4*>(&qk[buf][c0]);
    const float k4[4] = {kr.x * rn, kr.y * rn, kr.z * rn, kr.w * rn};
    const float q4[4] = {qr.x * qscale, qr.y * qscale, qr.z * qscale, qr.w * qscale};
    const float4 spv = d == 0 ? *reinterpret_cast<const float4*>(&S[(((size_t)s * H + h) * DV + r) * DK + c0])
                              : stack[(d - 1) * kGdnThreads + tid];
    const float sp[4] = {spv.x, spv.y, spv.z, spv.w};
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a += sp[e] * k4[e];
      b += sp[e] * q4[e];
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) {
      a += __shfl_xor(a, off, 64);
      b += __shfl_xor(b, off, 64);
    }
    const size_t ti = ((size_t)s * Tn + u) * H + h;
    const float gi = g[ti], bi = beta[ti];
    const float vr = Elem<A>::load(v, ti * DV + r);
    const float delta = bi * (vr - gi * a);
    float4 sn;
    sn.x = gi * sp[0] + delta * k4[0];
    sn.y = gi * sp[1] + delta * k4[1];
    sn.z = gi * sp[2] + delta * k4[2];
    sn.w = gi * sp[3] + delta * k4[3];
    stack[d * kGdnThreads + tid] = sn;
    *reinterpret_cast<float4*>(&S_scratch[((ti * DV) + r) * DK + c0]) = sn;
    if (c0 == 0) Elem<A>::store(o, ti * DV + r, gi * b + delta * kqn);
  }
}

hipError_t launch_gdn_tree_step(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch,
                                const void* v, const float* beta, const float* g, const float* S, float* S_scratch,
                                void* o, const int32_t* parent, int n, int T, int L, int H, int dk, int C, int W,
                                int act_dt, hipStream_t st) {
  const size_t smem = (size_t)(L + 1) * kGdnThreads * sizeof(float4);
#define DDT_GDN(TY, DKV)                                                                                      \
  do {                                                                                                        \
    const dim3 grid(n * H, DKV / (kGdnThreads / (DKV / 4)));                                                  \
    hipFuncSetAttribute(reinterpret_cast<const void*>(&gdn_tree_kernel<TY, DKV>),                              \
                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);                               \
    hipLaunchKernelGGL((gdn_tree_kernel<TY, DKV>), grid, dim3(kGdnThreads), smem, st,                        \
                       static_cast<const TY*>(x), conv_w, static_cast<const TY*>(conv_state),                \
                       static_cast<TY*>(conv_scratch), static_cast<const TY*>(v), beta, g, S, S_scratch,      \
                       static_cast<TY*>(o), parent, T, L, H, C, W);                                           \
  } while (0)
  if (act_dt == DDT_BF16) {
    if (dk == 32) DDT_GDN(uint16_t, 32);
    else if (dk == 64) DDT_GDN(uint16_t, 64);
    else DDT_GDN(uint16_t, 128);
  } else {
    if (dk == 32) DDT_GDN(float, 32);
    else if (dk == 64) DDT_GDN(float, 64);
    else DDT_GDN(float, 128);
  }
#undef DDT_GDN
  return hipGetLastError();
}

}  // namespace ddt
