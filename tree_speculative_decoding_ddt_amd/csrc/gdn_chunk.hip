// Short conv + Gated DeltaNet tree step without stored node states, in chunk form on the
// matrix cores.
// Sources: "DDTree on vLLM: candid research notes", section "Where the next step is"
// (scratch-buffer GDN replay instead of one state per branch); "The architecture of
// speculation", section "The DDTree Integration Challenge" (recompute rather than keep a
// recurrent state per branch).
//
// The step of node t with parent p (the committed S0 when t has no parent row) is
//   S_t = g_t S_p + w_t k_t^T,   w_t = beta_t (v_t - g_t S_p k_t),   o_t = S_t q_t.
// Along t's root path (t and its ancestors, path(t)) this unrolls to
//   S_t = G_t S0 + sum_{j in path(t)} r_tj w_j k_j^T,
// with G_t the product of g over path(t) and r_tj = G_t / G_j the product of g over the
// nodes of path(t) below j (r_tt = 1).  Hence, for every node, ancestors first:
//   w_t = beta_t (v_t - G_t (S0 k_t)) - sum_{j in anc(t)} beta_t r_tj (k_j . k_t) w_j
//   o_t = G_t (S0 q_t) + sum_{j in path(t)} r_tj (k_j . q_t) w_j
// so the dense work is S0 [K | Q] (T x dv from dk x dv) and the Gram products K K^T and
// Q K^T (T x T), on the matrix cores, and what remains is a triangular solve over the
// tree with dv right-hand sides, in which the nodes of one depth are independent.  No
// node state is formed.
//
// One block per (sequence, head), 4 waves.  Every global load of a phase is issued
// before any of its results is used (unconditional loads at clamped addresses), so each
// phase waits for memory once:
//   P0  the head's x channels (q and k part) of every node and the committed conv rows
//       staged in LDS, node scalars, each node's conv window (the node, its parent chain,
//       then the committed conv rows), depth and G_t; the depth order by a
//       histogram; the short conv and SiLU from LDS, k L2-normalised and q scaled, kept
//       as bf16 high and low parts (x = hi + lo to 2^-17); then, the stage being dead,
//       r_tj (products of g along the parent chain, so a zero g is exact too) and each
//       node's ancestor at every depth.  The wave's S0 operands and v values are loaded
//       into registers at the start, beside the stage.
//   P1  S0 [K|Q] and the lower block triangle of K K^T and Q K^T with
//       v_mfma_f32_16x16x32_bf16 as hi*hi + hi*lo + lo*hi (fp32 accumulation; the
//       dropped lo*lo term is 2^-18 relative)
//   P2  right-hand sides beta_t (v_t - G_t S0 k_t), the base G_t S0 q_t, and per node and
//       ancestor depth the record (ancestor row, solve coefficient, output coefficient)
//   P3  the solve, depth by depth: a wave owns dv/4 columns (so it needs no barrier: the
//       w it reads are its own), 512/dv nodes of one depth at a time, 2 columns per
//       lane; a node at depth d has exactly d ancestors, one per shallower depth.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

namespace {
typedef __bf16 cbf16x8 __attribute__((ext_vector_type(8)));
typedef float cf32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void split8(const float (&x)[8], cbf16x8& hi, cbf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(x[e]);
    hi[e] = h;
    lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
  }
}
// acc += a * b with a, b given as bf16 high and low parts
__device__ __forceinline__ cf32x4 mfma3(const cbf16x8& ah, const cbf16x8& al, const cbf16x8& bh, const cbf16x8& bl,
                                        cf32x4 acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
}
// 8 consecutive activations as fp32
template <typename A> __device__ __forceinline__ void load8(const A* p, float (&x)[8]);
template <> __device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&x)[8]) {
  const uint4 w = *reinterpret_cast<const uint4*>(p);
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
}  // namespace

constexpr int kChunkMaxTT = 5;   // 16-row tiles of nodes: T <= 80
constexpr int kChunkMaxW = 8;    // conv width
constexpr int kChunkMaxT = 65;   // nodes (budget <= 64 plus the root)

// LDS layout (bytes) for T nodes (row stride RSB = 2*dk + 16 for bf16 rows):
//   KQ     K hi, K lo, Q hi, Q lo: [T+1] rows each (row T stays zero: the rows of a
//          16-row tile past the last node read it); after P1 the right-hand sides / w
//          [T][dv] and the o base [T][dv] (fp32) take this area
//   scalars parent, g, beta, G, M_tt, depth, depth order, depth histogram/fill [T];
//          depth starts [T+1]; conv windows [T][8] int
//   big    during the conv: the x stage [T + W-1][2*dk] (act); then R [T][TS] fp32
//          (r_tj, TS = T rounded up to 4) and the records [T][T] x 16 B (P2 on)
struct ChunkLayout {
  int TS, rows, off_sc, off_win, off_big, off_rec, total;
};
__host__ __device__ inline ChunkLayout chunk_layout(int T, int dk, int W, int esize) {
  ChunkLayout c;
  const int RSB = 2 * dk + 16;
  c.TS = (T + 3) / 4 * 4;
  c.rows = T + 1;
  const int kq = 4 * c.rows * RSB, st = 2 * T * dk * 4;
  c.off_sc = ((kq > st ? kq : st) + 15) / 16 * 16;
  c.off_win = c.off_sc + ((8 * T + T + 1) * 4 + 15) / 16 * 16;
  c.off_big = c.off_win + T * kChunkMaxW * 4;
  const int stage = (T + W - 1) * 2 * dk * esize;
  c.off_rec = c.off_big + (T * c.TS * 4 + 15) / 16 * 16;
  const int after = c.off_rec + T * T * 16;
  c.total = (c.off_big + stage > after) ? c.off_big + stage : after;
  return c;
}

template <typename A, int DK>
__global__ void __launch_bounds__(256) gdn_chunk_kernel(const A* __restrict__ x, const float* __restrict__ conv_w,
                                                        const A* __restrict__ conv_state, const A* __restrict__ v,
                                                        const float* __restrict__ beta, const float* __restrict__ g,
                                                        const float* __restrict__ S, A* __restrict__ o,
                                                        const int32_t* __restrict__ parent, int Tn, int H, int W) {
  constexpr int DV = DK, RSB = 2 * DK + 16, NCS = DK / 32, NRT = DV / 16;
  constexpr int RTW = (NRT + 3) / 4;  // 16-column tiles of S0 per wave
  constexpr int NG = DK / 8;          // lanes per (node, q or k) in the conv: 8 channels each
  constexpr int NPR = 256 / (2 * NG); // nodes per conv round
  constexpr int CPW = DV / 4;         // solve: columns a wave owns
  constexpr int LPN = CPW / 2;        // lanes per node (2 columns per lane)
  constexpr int NPW = 64 / LPN;       // nodes of one depth per wave step
  constexpr int ROW8 = 2 * DK / 8;    // 16-byte chunks (8 activations) of a staged row
  extern __shared__ __align__(16) uint8_t lds[];
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int C = 2 * H * DK;
  const ChunkLayout L = chunk_layout(Tn, DK, W, (int)sizeof(A));
  const int NTT = (Tn + 15) / 16, TS = L.TS, RW = L.rows;
  int* par = reinterpret_cast<int*>(lds + L.off_sc);
  float* gg = reinterpret_cast<float*>(par + Tn);
  float* be = gg + Tn;
  float* Gam = be + Tn;
  float* Md = Gam + Tn;
  int* dep = reinterpret_cast<int*>(Md + Tn);
  int* ord = dep + Tn;
  int* cnt = ord + Tn;     // depth histogram, then the fill counters
  int* lstart = cnt + Tn;  // [Tn + 1]
  int* win = reinterpret_cast<int*>(lds + L.off_win);
  A* stage = reinterpret_cast<A*>(lds + L.off_big);  // [Tn + W-1][2*DK]: x rows, then conv rows
  float* Rm = reinterpret_cast<float*>(lds + L.off_big);
  float4* rec = reinterpret_cast<float4*>(lds + L.off_rec);  // [t][depth]: (row, A_tj, M_tj, -)

  // ---- P0: every global load of the block first (addresses clamped into range)
  const float* S0 = S + ((size_t)s * H + h) * DV * DK;
  float sop[RTW][NCS][8];
#pragma unroll
  for (int w = 0; w < RTW; ++w) {
    const int rt = min(wave + 4 * w, NRT - 1);
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs) load8<float>(S0 + (size_t)(16 * rt + l16) * DK + 32 * cs + 8 * q4, sop[w][cs]);
  }
  float vv[RTW][kChunkMaxTT][4];
#pragma unroll
  for (int w = 0; w < RTW; ++w) {
    const int rt = min(wave + 4 * w, NRT - 1);
#pragma unroll
    for (int ti = 0; ti < kChunkMaxTT; ++ti)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = min(16 * ti + 4 * q4 + e, Tn - 1);
        vv[w][ti][e] = Elem<A>::load(v, (((size_t)s * Tn + t) * H + h) * DV + 16 * rt + l16);
      }
  }
  // this thread's conv channels: 8 of the head's q (half 0) or k (half 1) channels
  const int cg = tid % NG, half = (tid / NG) & 1, tsub = tid / (2 * NG);
  const int c0 = half * H * DK + h * DK + 8 * cg;  // channel in x
  const int s0 = half * DK + 8 * cg;               // channel in the stage
  float cw[8][kChunkMaxW];
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int c = 0; c < kChunkMaxW; ++c) cw[e][c] = conv_w[(size_t)(c0 + e) * W + min(c, W - 1)];
  // the stage: rows 0..T-1 are x, rows T..T+W-2 the committed conv rows; chunk k of a row
  // is 8 activations of the q part (k < ROW8/2) or the k part
  constexpr int kStageIt = ((kChunkMaxT + kChunkMaxW - 1) * ROW8 + 255) / 256;
  const int nst = (Tn + W - 1) * ROW8;
  uint4 sv[kStageIt * (int)sizeof(A) / 2];  // 16 bytes per chunk for bf16, 32 for fp32
#pragma unroll
  for (int k = 0; k < kStageIt; ++k) {
    const int idx = min(tid + 256 * k, nst - 1);
    const int row = idx / ROW8, ch = idx % ROW8;
    const int chan = ch < ROW8 / 2 ? h * DK + 8 * ch : H * DK + h * DK + 8 * (ch - ROW8 / 2);
    const A* src = row < Tn ? x + ((size_t)s * Tn + row) * C + chan
                            : conv_state + ((size_t)s * (W - 1) + (row - Tn)) * C + chan;
    if constexpr (sizeof(A) == 2) {
      sv[k] = *reinterpret_cast<const uint4*>(src);
    } else {
      sv[2 * k] = *reinterpret_cast<const uint4*>(src);
      sv[2 * k + 1] = *reinterpret_cast<const uint4*>(src + 4);
    }
  }
  int pr = 0;
  float gr = 0.f, br = 0.f;
  if (tid < Tn) {
    const size_t ti = ((size_t)s * Tn + tid) * H + h;
    pr = parent[(size_t)s * Tn + tid];
    gr = g[ti];
    br = beta[ti];
  }
#pragma unroll
  for (int k = 0; k < kStageIt; ++k) {
    const int idx = tid + 256 * k;
    if (idx < nst) {
      if constexpr (sizeof(A) == 2) {
        reinterpret_cast<uint4*>(stage)[idx] = sv[k];
      } else {
        reinterpret_cast<uint4*>(stage)[2 * idx] = sv[2 * k];
        reinterpret_cast<uint4*>(stage)[2 * idx + 1] = sv[2 * k + 1];
      }
    }
  }
  if (tid < Tn) {
    par[tid] = pr;
    gg[tid] = gr;
    be[tid] = br;
    cnt[tid] = 0;
  }
  for (int i = tid; i < 4 * RSB / 16; i += 256)  // row T of K hi, K lo, Q hi, Q lo: zero
    *reinterpret_cast<uint4*>(lds + (i / (RSB / 16)) * RW * RSB + Tn * RSB + (i % (RSB / 16)) * 16) =
        make_uint4(0, 0, 0, 0);
  __syncthreads();
  // per node: conv window (back b: stage row; the committed conv rows come after the
  // node rows, newest last), depth, G_t; the depth histogram
  if (tid < Tn) {
    const int t = tid;
    int cur = t, in_tree = 1, beyond = 0;
    for (int b = 0; b < W; ++b) {
      int r = t;
      if (b > 0) {
        if (in_tree) {
          const int p = par[cur];
          if (p >= 0 && p < cur) cur = p;
          else in_tree = 0;
        }
        r = in_tree ? cur : Tn + (W - 1 - (++beyond));
      }
      win[t * kChunkMaxW + b] = r;
    }
    float prod = 1.f;
    int a = t, d = 0;
    while (true) {
      const int p = par[a];
      if (!(p >= 0 && p < a)) break;
      prod *= gg[a];
      a = p;
      ++d;
    }
    Gam[t] = prod * gg[a];
    dep[t] = d;
    atomicAdd(&cnt[d], 1);
  }
  __syncthreads();
  // depth starts (one thread: at most T depths) while the others run the conv
  if (tid == 0) {
    int acc = 0, d = 0;
    for (; d < Tn && cnt[d] > 0; ++d) {
      lstart[d] = acc;
      acc += cnt[d];
      cnt[d] = 0;  // reused as the fill counter of depth d
    }
    lstart[d] = Tn;
  }
  // the short conv of the head's q and k channels from the stage (NPR nodes per round)
  for (int t0 = 0; t0 < Tn; t0 += NPR) {
    const int t = min(t0 + tsub, Tn - 1);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = 0.f;
#pragma unroll
    for (int c = 0; c < kChunkMaxW; ++c) {  // tap c multiplies the row W-1-c back
      if (c >= W) break;
      const int r = win[t * kChunkMaxW + (W - 1 - c)];
      float xv[8];
      load8<A>(stage + (size_t)r * (2 * DK) + s0, xv);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] += cw[e][c] * xv[e];
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = y[e] / (1.f + __expf(-y[e]));
      ss += y[e] * y[e];
    }
    // k: L2 norm over the head's dk channels (the NG lanes of this node and half)
#pragma unroll
    for (int off = NG / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off, 64);
    const float sc = half ? 1.f / sqrtf(ss + 1e-6f) : rsqrtf((float)DK);
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] *= sc;
    if (t0 + tsub < Tn) {
      cbf16x8 hi, lo;
      split8(y, hi, lo);
      const int base = (half ? 0 : 2) * RW * RSB + t * RSB + cg * 16;  // K hi/lo first, then Q hi/lo
      *reinterpret_cast<cbf16x8*>(lds + base) = hi;
      *reinterpret_cast<cbf16x8*>(lds + base + RW * RSB) = lo;
    }
  }
  __syncthreads();  // the stage is dead: R and the records take its area
  for (int i = tid; i < Tn * TS; i += 256) Rm[i] = 0.f;
  if (tid < Tn) ord[lstart[dep[tid]] + atomicAdd(&cnt[dep[tid]], 1)] = tid;
  __syncthreads();
  // r_tj along each node's parent chain; rec[t][depth of j] starts with the row j
  if (tid < Tn) {
    const int t = tid;
    float prod = 1.f;
    int a = t, d = dep[t];
    Rm[t * TS + t] = 1.f;
    while (true) {
      const int p = par[a];
      if (!(p >= 0 && p < a)) break;
      prod *= gg[a];
      a = p;
      --d;
      Rm[t * TS + a] = prod;
      rec[t * Tn + d] = make_float4(__int_as_float(a), 0.f, 0.f, 0.f);
    }
  }

  // ---- P1: S0 [K|Q] and the Gram products (results stay in registers).  A tile's rows
  // past the last node read row T, which is zero.
  cf32x4 acc[RTW][kChunkMaxTT][2];
#pragma unroll
  for (int w = 0; w < RTW; ++w)
#pragma unroll
    for (int ti = 0; ti < kChunkMaxTT; ++ti) acc[w][ti][0] = acc[w][ti][1] = cf32x4{0.f, 0.f, 0.f, 0.f};
  const uint8_t* Khi = lds;
  const uint8_t* Klo = lds + RW * RSB;
  const uint8_t* Qhi = lds + 2 * RW * RSB;
  const uint8_t* Qlo = lds + 3 * RW * RSB;
#pragma unroll
  for (int w = 0; w < RTW; ++w) {
    if (wave + 4 * w >= NRT) continue;
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs) {
      // B = S0^T: column r = 16*rt + l16, k-range c = 32*cs + 8*q4 .. +7
      cbf16x8 bh, bl;
      split8(sop[w][cs], bh, bl);
#pragma unroll
      for (int ti = 0; ti < kChunkMaxTT; ++ti) {
        if (ti >= NTT) break;
        const int ro = min(16 * ti + l16, Tn) * RSB + 64 * cs + 16 * q4;
        const cbf16x8 kh = *reinterpret_cast<const cbf16x8*>(Khi + ro);
        const cbf16x8 kl = *reinterpret_cast<const cbf16x8*>(Klo + ro);
        const cbf16x8 qh = *reinterpret_cast<const cbf16x8*>(Qhi + ro);
        const cbf16x8 ql = *reinterpret_cast<const cbf16x8*>(Qlo + ro);
        acc[w][ti][0] = mfma3(kh, kl, bh, bl, acc[w][ti][0]);
        acc[w][ti][1] = mfma3(qh, ql, bh, bl, acc[w][ti][1]);
      }
    }
  }
  // Gram blocks (ti, tj), tj <= ti, dealt to the waves: K_t . K_j and Q_t . K_j
  constexpr int kMaxPairs = (kChunkMaxTT * (kChunkMaxTT + 1) / 2 + 3) / 4;  // per wave
  const int NP = NTT * (NTT + 1) / 2;
  cf32x4 gk[kMaxPairs][2];
  int pti[kMaxPairs], ptj[kMaxPairs];
#pragma unroll
  for (int k = 0; k < kMaxPairs; ++k) {
    gk[k][0] = gk[k][1] = cf32x4{0.f, 0.f, 0.f, 0.f};
    const int p = wave + 4 * k;
    int ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= p) ++ti;
    pti[k] = ti;
    ptj[k] = p - ti * (ti + 1) / 2;
    if (p >= NP) continue;
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs) {
      const int ra = min(16 * pti[k] + l16, Tn) * RSB + 64 * cs + 16 * q4;
      const int rb = min(16 * ptj[k] + l16, Tn) * RSB + 64 * cs + 16 * q4;
      const cbf16x8 kh = *reinterpret_cast<const cbf16x8*>(Khi + ra);
      const cbf16x8 kl = *reinterpret_cast<const cbf16x8*>(Klo + ra);
      const cbf16x8 qh = *reinterpret_cast<const cbf16x8*>(Qhi + ra);
      const cbf16x8 ql = *reinterpret_cast<const cbf16x8*>(Qlo + ra);
      const cbf16x8 jh = *reinterpret_cast<const cbf16x8*>(Khi + rb);
      const cbf16x8 jl = *reinterpret_cast<const cbf16x8*>(Klo + rb);
      gk[k][0] = mfma3(kh, kl, jh, jl, gk[k][0]);
      gk[k][1] = mfma3(qh, ql, jh, jl, gk[k][1]);
    }
  }
  __syncthreads();  // every wave is done with q/k: their area now takes w and the o base

  // ---- P2: right-hand sides, o base (D layout: column l16, rows 4*q4 + e) and the
  // records (ancestor row, beta_t r_tj (k_j . k_t), r_tj (k_j . q_t)) by ancestor depth
  float* Wm = reinterpret_cast<float*>(lds);  // [T][DV]: right-hand sides, then w
  float* Ob = Wm + Tn * DV;                   // [T][DV]: G_t S0 q_t
  float bt[kChunkMaxTT][4], Gt[kChunkMaxTT][4];
#pragma unroll
  for (int ti = 0; ti < kChunkMaxTT; ++ti)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = min(16 * ti + 4 * q4 + e, Tn - 1);
      bt[ti][e] = be[t];
      Gt[ti][e] = Gam[t];
    }
#pragma unroll
  for (int w = 0; w < RTW; ++w) {
    const int rt = wave + 4 * w;
    if (rt >= NRT) continue;
    const int r = 16 * rt + l16;
#pragma unroll
    for (int ti = 0; ti < kChunkMaxTT; ++ti) {
      if (ti >= NTT) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 16 * ti + 4 * q4 + e;
        if (t < Tn) {
          Wm[t * DV + r] = bt[ti][e] * (vv[w][ti][e] - Gt[ti][e] * acc[w][ti][0][e]);
          Ob[t * DV + r] = Gt[ti][e] * acc[w][ti][1][e];
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxPairs; ++k) {
    if (wave + 4 * k >= NP) continue;
    const int j = 16 * ptj[k] + l16;
    const int jc = min(j, Tn - 1);
    const int dj = dep[jc];
    float rr[4], bb[4];
    int dt[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = min(16 * pti[k] + 4 * q4 + e, Tn - 1);
      rr[e] = Rm[t * TS + jc];
      bb[e] = be[t];
      dt[e] = dep[t];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * pti[k] + 4 * q4 + e;
      if (t < Tn && j == t) Md[t] = gk[k][1][e];  // r_tt = 1
      // the slot of depth dep[j] < dep[t] holds t's ancestor there: j owns it if it is
      // that row (r_tj may be 0 when a g on the way is 0: then so are both coefficients)
      if (t < Tn && j < t && dj < dt[e]) {
        float4* rp = &rec[t * Tn + dj];
        if (__float_as_int(rp->x) == j) {
          rp->y = bb[e] * rr[e] * gk[k][0][e];
          rp->z = rr[e] * gk[k][1][e];
        }
      }
    }
  }
  __syncthreads();

  // ---- P3: the solve, depth by depth, barrier-free: wave `wave` owns columns
  // [CPW*wave, CPW*(wave+1)), a lane 2 of them, NPW nodes of one depth at once
  {
    const int nsub = lane / LPN;
    const int rc = CPW * wave + 2 * (lane % LPN);
    for (int d = 0;; ++d) {
      const int beg = __builtin_amdgcn_readfirstlane(lstart[d]);
      if (beg >= Tn) break;
      const int end = __builtin_amdgcn_readfirstlane(lstart[d + 1]);
      for (int i0 = beg; i0 < end; i0 += NPW) {
        const int k = i0 + nsub;
        const int t = ord[min(k, end - 1)];
        float aw0 = 0.f, aw1 = 0.f, ao0 = 0.f, ao1 = 0.f;
        // d ancestors, one per shallower depth, four at a time (records first, then rows)
        for (int e0 = 0; e0 < d; e0 += 4) {
          float4 rv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) rv[u] = rec[t * Tn + min(e0 + u, d - 1)];
          float2 wv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) wv[u] = *reinterpret_cast<const float2*>(&Wm[__float_as_int(rv[u].x) * DV + rc]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float sa = e0 + u < d ? rv[u].y : 0.f, sm = e0 + u < d ? rv[u].z : 0.f;
            aw0 += sa * wv[u].x;
            aw1 += sa * wv[u].y;
            ao0 += sm * wv[u].x;
            ao1 += sm * wv[u].y;
          }
        }
        if (k < end) {
          const float2 rh = *reinterpret_cast<const float2*>(&Wm[t * DV + rc]);
          const float2 ob = *reinterpret_cast<const float2*>(&Ob[t * DV + rc]);
          const float md = Md[t];
          const float w0 = rh.x - aw0, w1 = rh.y - aw1;
          *reinterpret_cast<float2*>(&Wm[t * DV + rc]) = make_float2(w0, w1);
          const size_t oi = (((size_t)s * Tn + t) * H + h) * DV + rc;
          Elem<A>::store(o, oi, ob.x + ao0 + md * w0);
          Elem<A>::store(o, oi + 1, ob.y + ao1 + md * w1);
        }
      }
    }
  }
}

size_t gdn_chunk_lds_bytes(int T, int dk, int W, int esize) { return (size_t)chunk_layout(T, dk, W, esize).total; }

template <typename A, int DK>
static void launch_chunk(const void* x, const float* conv_w, const void* conv_state, const void* v,
                         const float* beta, const float* g, const float* S, void* o, const int32_t* parent, int n,
                         int T, int H, int W, hipStream_t st) {
  auto kern = gdn_chunk_kernel<A, DK>;
  // the dynamic LDS limit is raised once per kernel, to the largest size any call uses
  // (a host-side attribute, not a stream operation: calls stay capturable in a graph)
  static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)gdn_chunk_lds_bytes(kChunkMaxT, DK, kChunkMaxW,
                                                                        (int)sizeof(A))) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL(kern, dim3(n * H), dim3(256), gdn_chunk_lds_bytes(T, DK, W, (int)sizeof(A)), st, static_cast<const A*>(x), conv_w,
                     static_cast<const A*>(conv_state), static_cast<const A*>(v), beta, g, S, static_cast<A*>(o),
                     parent, T, H, W);
}

hipError_t launch_gdn_chunk(const void* x, const float* conv_w, const void* conv_state, const void* v,
                            const float* beta, const float* g, const float* S, void* o, const int32_t* parent, int n,
                            int T, int H, int dk, int W, int act_dt, hipStream_t st) {
#define DDT_CHUNK(TY, DKV) launch_chunk<TY, DKV>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, st)
  // bf16 activations only (fp32 ones keep the node-by-node walk); T <= 65, W <= 8
  if (act_dt != DDT_BF16 || T < 1 || T > kChunkMaxT || W < 1 || W > kChunkMaxW) return hipErrorInvalidValue;
  if (dk == 32) DDT_CHUNK(uint16_t, 32);
  else if (dk == 64) DDT_CHUNK(uint16_t, 64);
  else if (dk == 128) DDT_CHUNK(uint16_t, 128);
  else return hipErrorInvalidValue;
#undef DDT_CHUNK
  return hipGetLastError();
}

}  // namespace ddt
