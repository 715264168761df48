// GDN replay on commit: the committed recurrent and conv state advanced along the
// accepted path, instead of copied from a per-node scratch of every tree node.
// Sources: "DDTree on vLLM: candid research notes", sections "Why hybrid attention
// makes it hard" (the accepted path's state is what the committed buffers receive) and
// "Where the next step is" (scratch-buffer GDN and conv replay); "The architecture of
// speculation", section "The DDTree Integration Challenge" (recomputing or compacting
// recurrent state instead of keeping one copy per branch).
//
// For sequence s with a = acc_len[s] >= 0 and path rows r_0 (the root), ..., r_a:
//   for j = 0..a:  window of r_j = [committed conv rows ..., x[r_0], ..., x[r_j]] (last W)
//                  k = SiLU(conv of the k channels) / sqrt(|k|^2 + 1e-6)
//                  S = g S + beta (v - g S k) k^T          (per head, rows of S independent)
//   conv_state = the last W-1 rows of the window of r_a
// The tree walk applies exactly these updates to the same inputs, so the result equals
// the stored state of row r_a up to fp32 rounding order.
//
// Two kernels per group of layers:
//   replay_state  grid (n*H, dv/R, layers): a block owns R rows of one head's state in
//                 registers (a thread 8 columns of one row, as in the tree walk); the
//                 path's inputs are read into LDS first, all at once; per path node the
//                 block computes the head's dk k-channels, then every row takes its
//                 rank-1 update.  Reads the committed conv rows.
//   replay_conv   grid (n, layers, C/256): one thread per channel rebuilds the W-1
//                 committed conv rows (exact copies), after every state block has read
//                 them (stream order).
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

constexpr int kReplayLayers = 16;
constexpr int kReplayMaxW = 8;

struct ReplayTable {
  const uint8_t* x[kReplayLayers];
  const float* conv_w[kReplayLayers];
  const uint8_t* v[kReplayLayers];
  const float* beta[kReplayLayers];
  const float* g[kReplayLayers];
  float* S[kReplayLayers];
  uint8_t* conv_state[kReplayLayers];
};

// Path rows of sequence s into LDS; false (for the whole block) if the sequence is not
// to be committed or a row is out of range.
__device__ bool load_path(const int32_t* acc_rows, const int32_t* acc_len, int s, int Tn, int Lp1, int* rows,
                          int& a) {
  __shared__ int bad;
  a = acc_len[s];
  if (a < 0 || a >= Lp1) return false;  // uniform: every thread read the same value
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  if ((int)threadIdx.x <= a) {
    const int r = acc_rows[(size_t)s * Lp1 + threadIdx.x];
    rows[threadIdx.x] = r;
    if (r < 0 || r >= Tn) bad = 1;
  }
  __syncthreads();
  return bad == 0;
}

template <typename A, int DK>
__global__ void __launch_bounds__(256) replay_state_kernel(ReplayTable tab, const int32_t* __restrict__ acc_rows,
                                                           const int32_t* __restrict__ acc_len, int Tn, int Lp1,
                                                           int H, int C, int W) {
  constexpr int DV = DK;
  constexpr int CPT = DK >= 64 ? 8 : 4;  // columns per thread, as in the tree walk
  constexpr int LPR = DK / CPT;          // lanes per state row
  constexpr int R = 256 / LPR;           // state rows per block
  constexpr int GS = DK / (CPT / 4);     // stride between a thread's column groups
  const int s = blockIdx.x / H, h = blockIdx.x % H, layer = blockIdx.z;
  const int tid = threadIdx.x;
  const int rl = tid / LPR, r = blockIdx.y * R + rl;
  const int c0 = (tid % LPR) * 4;
  __shared__ int rows[64];
  __shared__ float ks[DK];
  __shared__ float red[DK / 64 + 1];
  __shared__ float gbs[2][64];  // g and beta of every path node (this head)
  __shared__ float vs[64][R];   // v of every path node (this block's rows)
  extern __shared__ float xk[];  // [(W-1) + a+1][DK]: the k channels' committed conv rows, then path rows
  int a;
  if (!load_path(acc_rows, acc_len, s, Tn, Lp1, rows, a)) return;

  const A* x = reinterpret_cast<const A*>(tab.x[layer]);
  const float* w = tab.conv_w[layer];
  const A* v = reinterpret_cast<const A*>(tab.v[layer]);
  const float* beta = tab.beta[layer];
  const float* g = tab.g[layer];
  float* S = tab.S[layer];
  const A* cs = reinterpret_cast<const A*>(tab.conv_state[layer]);

  float st[CPT];  // this thread's columns of its state row
  float* srow = S + (((size_t)s * H + h) * DV + r) * DK + c0;
#pragma unroll
  for (int e = 0; e < CPT; ++e) st[e] = srow[(e / 4) * GS + (e % 4)];

  // Every input of the path is read up front, all loads in flight together (they depend
  // on the path rows only, not on the state): the window values of the head's k channels
  // (the W-1 committed conv rows, then the path rows in order, so that node j's window is
  // entries j .. j+W-1), each node's g, beta and v, and this channel's weights.
  const int nw = (W - 1) + (a + 1);
  for (int i = tid; i < nw * DK; i += 256) {
    const int q = i / DK, kc = H * DK + h * DK + (i % DK);
    const A val = q < W - 1 ? cs[((size_t)s * (W - 1) + q) * C + kc]
                            : x[((size_t)s * Tn + rows[q - (W - 1)]) * C + kc];
    xk[i] = Elem<A>::load(&val, 0);
  }
  for (int j = tid; j <= a; j += 256) {
    const size_t ti = ((size_t)s * Tn + rows[j]) * H + h;
    gbs[0][j] = g[ti];
    gbs[1][j] = beta[ti];
  }
  for (int i = tid; i < (a + 1) * R; i += 256) {
    const int j = i / R, q = i % R;
    vs[j][q] = Elem<A>::load(v, (((size_t)s * Tn + rows[j]) * H + h) * DV + blockIdx.y * R + q);
  }
  const int kc = H * DK + h * DK + tid;  // k channel computed by thread tid < DK
  float wk[kReplayMaxW];                 // wk[b]: the weight of back b (tap W-1-b)
#pragma unroll
  for (int b = 0; b < kReplayMaxW; ++b) wk[b] = tid < DK && b < W ? w[(size_t)kc * W + (W - 1 - b)] : 0.f;
  __syncthreads();

  for (int j = 0; j <= a; ++j) {
    float y = 0.f;
    if (tid < DK) {
      // back b: entry j + W-1 - b of the window (path row r_{j-b}, or past the root the
      // committed conv row W-1-(b-j))
      float acc = 0.f;
#pragma unroll
      for (int b = 0; b < kReplayMaxW; ++b)
        if (b < W) acc += wk[b] * xk[(j + W - 1 - b) * DK + tid];
      y = acc / (1.f + __expf(-acc));
      ks[tid] = y;
    }
    if (tid < (DK + 63) / 64 * 64) {  // whole waves: lanes past DK add zeros
      const float kk = wave_sum(y * y);
      if ((tid & 63) == 0) red[tid >> 6] = kk;
    }
    __syncthreads();
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < (DK + 63) / 64; ++i) sum += red[i];
    const float rn = 1.f / sqrtf(sum + 1e-6f);
    float kv[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) kv[e] = ks[c0 + (e / 4) * GS + (e % 4)] * rn;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < CPT; ++e) dot += st[e] * kv[e];
    dot = group_sum<LPR>(dot);
    const float gi = gbs[0][j], bi = gbs[1][j];
    const float delta = bi * (vs[j][rl] - gi * dot);
#pragma unroll
    for (int e = 0; e < CPT; ++e) st[e] = gi * st[e] + delta * kv[e];
    __syncthreads();  // ks and red are rewritten by the next node
  }
#pragma unroll
  for (int e = 0; e < CPT; ++e) srow[(e / 4) * GS + (e % 4)] = st[e];
}

template <typename A>
__global__ void __launch_bounds__(256) replay_conv_kernel(ReplayTable tab, const int32_t* __restrict__ acc_rows,
                                                          const int32_t* __restrict__ acc_len, int Tn, int Lp1,
                                                          int C, int W) {
  const int s = blockIdx.x, layer = blockIdx.y;
  const int c = blockIdx.z * 256 + threadIdx.x;
  __shared__ int rows[64];
  int a;
  if (!load_path(acc_rows, acc_len, s, Tn, Lp1, rows, a)) return;
  if (c >= C) return;
  const A* x = reinterpret_cast<const A*>(tab.x[layer]);
  A* cs = reinterpret_cast<A*>(tab.conv_state[layer]);
  // slot t (oldest first) of the deepest row's window is back b = W-2-t
  A nv[kReplayMaxW - 1];
#pragma unroll
  for (int t = 0; t < kReplayMaxW - 1; ++t) {
    if (t < W - 1) {
      const int b = W - 2 - t;
      nv[t] = b <= a ? x[((size_t)s * Tn + rows[a - b]) * C + c]
                     : cs[((size_t)s * (W - 1) + (W - 1 - (b - a))) * C + c];
    }
  }
#pragma unroll
  for (int t = 0; t < kReplayMaxW - 1; ++t)
    if (t < W - 1) cs[((size_t)s * (W - 1) + t) * C + c] = nv[t];
}

template <typename A, int DK>
static void launch_replay_dk(const ReplayTable& tab, int cnt, const int32_t* acc_rows, const int32_t* acc_len, int n,
                             int T, int Lp1, int H, int C, int W, hipStream_t st) {
  constexpr int R = 256 / (DK / (DK >= 64 ? 8 : 4));
  const size_t smem = (size_t)((W - 1) + Lp1) * DK * sizeof(float);  // the path's window values (<= 36 KB)
  hipLaunchKernelGGL((replay_state_kernel<A, DK>), dim3(n * H, DK / R, cnt), dim3(256), smem, st, tab, acc_rows,
                     acc_len, T, Lp1, H, C, W);
}

hipError_t launch_gdn_replay(const int32_t* acc_rows, const int32_t* acc_len, const ddt_gdn_replay_layer* layers,
                             int n_layers, int H, int dk, int C, int W, int act_dt, int n, int T, int L,
                             hipStream_t st) {
  const int Lp1 = L + 1;
  for (int l0 = 0; l0 < n_layers; l0 += kReplayLayers) {
    const int cnt = n_layers - l0 < kReplayLayers ? n_layers - l0 : kReplayLayers;
    ReplayTable tab = {};
    for (int j = 0; j < cnt; ++j) {
      const ddt_gdn_replay_layer& y = layers[l0 + j];
      tab.x[j] = static_cast<const uint8_t*>(y.x);
      tab.conv_w[j] = y.conv_w;
      tab.v[j] = static_cast<const uint8_t*>(y.v);
      tab.beta[j] = y.beta;
      tab.g[j] = y.g;
      tab.S[j] = y.S;
      tab.conv_state[j] = static_cast<uint8_t*>(y.conv_state);
    }
#define DDT_REPLAY(TY)                                                                                      \
  do {                                                                                                      \
    if (dk == 32) launch_replay_dk<TY, 32>(tab, cnt, acc_rows, acc_len, n, T, Lp1, H, C, W, st);            \
    else if (dk == 64) launch_replay_dk<TY, 64>(tab, cnt, acc_rows, acc_len, n, T, Lp1, H, C, W, st);       \
    else launch_replay_dk<TY, 128>(tab, cnt, acc_rows, acc_len, n, T, Lp1, H, C, W, st);                    \
    hipLaunchKernelGGL((replay_conv_kernel<TY>), dim3(n, cnt, cdiv(C, 256)), dim3(256), 0, st, tab, acc_rows, \
                       acc_len, T, Lp1, C, W);                                                              \
  } while (0)
    if (act_dt == DDT_BF16) DDT_REPLAY(uint16_t);
    else DDT_REPLAY(float);
#undef DDT_REPLAY
  }
  return hipGetLastError();
}

}  // namespace ddt
