// Short conv + Gated DeltaNet tree step in chunk form on the matrix cores: without stored
// node states, or with them (formed afterwards, each from S0 and its path's terms).
// Sources: "DDTree on vLLM: candid research notes", sections "Why hybrid attention makes
// it hard" (each node's state and conv state written to scratch) and "Where the next step
// is" (scratch-buffer GDN replay instead of one state per branch); "The architecture of
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
// node state is formed here; with states stored (STORE) the kernel also writes the conv
// scratch and leaves k, w and the path records for gdn_states_kernel.
//
// One block per (sequence, head), 8 waves.  Every global load of a phase is issued
// before any of its results is used (unconditional loads at clamped addresses), so each
// phase waits for memory once:
//   P0  the node scalars and, by LDS DMA, the stage (the head's x channels, q and k part,
//       of every node, then the committed conv rows); after the first barrier the wave's
//       S0 operands and v values are issued (they arrive during the walk).  One walk per
//       node up its parent chain gives its conv window (the node, its ancestors, then the
//       committed conv rows), its depth, G_t and its ancestor records (row, r_tj: products
//       of g along the chain, so a zero g is exact too); the depth order by a histogram;
//       the short conv and SiLU from the stage, k L2-normalised and q scaled, kept as
//       bf16 high and low parts (x = hi + lo to 2^-17).  With STORE: G_t, the depths and
//       the records are exported after the walk, the conv scratch and the fp32 k during
//       the conv, and w after the solve.
//   P1  S0 [K|Q] and the lower block triangle of K K^T and Q K^T with
//       v_mfma_f32_16x16x32_bf16 as hi*hi + hi*lo + lo*hi (fp32 accumulation; the
//       dropped lo*lo term is 2^-18 relative)
//   P2  right-hand sides beta_t (v_t - G_t S0 k_t), the base G_t S0 q_t, and per node and
//       ancestor depth the record (ancestor row, solve coefficient, output coefficient)
//   P3  the solve, depth by depth: a wave owns dv/8 columns (so it needs no barrier: the
//       w it reads are its own), 2048/dv nodes of one depth at a time, 4 columns per
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
// 8 consecutive fp32 values
template <typename A> __device__ __forceinline__ void load8(const A* p, float (&x)[8]);
template <> __device__ __forceinline__ void load8<float>(const float* p, float (&x)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
}  // namespace

constexpr int kChunkThreads = 512;                // threads per block (one per (sequence, head))
constexpr int kChunkWaves = kChunkThreads / 64;
constexpr int kChunkMaxTT = 5;   // 16-row tiles of nodes
constexpr int kChunkMaxW = 8;    // conv width
constexpr int kChunkMaxT = 65;   // nodes (budget <= 64 plus the root)

// Node t keeps one record per proper ancestor, nearest first: slot t(t-1)/2 + k holds
// its (k+1)-th ancestor (k = 0: the parent).  Parents precede their children, so t has
// at most t ancestors and T(T-1)/2 slots hold every record.
__host__ __device__ inline int rec_base(int t) { return t * (t - 1) / 2; }

// What the chunk kernel hands to gdn_states_kernel when node states are stored (device
// arrays in the workspace; TRI = rec_base(T) record slots per tree):
//   k [n][T][H][dk], w [n][T][H][dv]  the normalised keys and the solve's w (fp32)
//   gam [n][T][H]                     G_t
//   dep [n][T]                        proper ancestors of t (head independent)
//   rows [n][TRI]                     t's (k+1)-th ancestor at slot rec_base(t) + k
//   rho [n][H][TRI]                   r_tj of that ancestor
// and the conv scratch [n][T][W-1][C], which the chunk kernel writes itself.
struct ChunkStoreOut {
  uint16_t* conv_scratch;
  float* k;
  float* w;
  float* gam;
  int32_t* dep;
  int32_t* rows;
  float* rho;
};

// LDS layout (bytes) for T nodes (bf16 row stride RSB = 2*dk + 16):
//   KQ      K hi, K lo, Q hi, Q lo: [T+1] rows each (row T stays zero: the rows of a
//           16-row tile past the last node read it); from P2 on, w [T][WS] and the o base
//           [T][WS] (fp32, WS = dv + 4) take this area
//   scalars parent, g, beta, G, M_tt, depth, nodes per depth, depth order [T]; first
//           position of each depth [T+1]; the largest depth
//   win     conv windows [T][8]: stage rows, tap W-1-b reads entry b
//   rec     the records [T(T-1)/2] x (ancestor row, r_tj then beta_t r_tj k_j.k_t,
//           r_tj k_j.q_t, unused)
//   stage   x rows [T][2*dk] (q part, k part) then the committed conv rows [W-1][2*dk],
//           padded to whole 4 KB rounds of the block's LDS DMA
struct ChunkLayout {
  int rows, WS, off_sc, off_win, off_rec, off_stage, total;
};
__host__ __device__ inline ChunkLayout chunk_layout(int T, int dk, int W) {
  ChunkLayout c;
  const int RSB = 2 * dk + 16;
  c.rows = T + 1;
  c.WS = dk + 4;
  const int kq = 4 * c.rows * RSB, wo = 2 * T * c.WS * 4;
  c.off_sc = ((kq > wo ? kq : wo) + 15) / 16 * 16;
  c.off_win = c.off_sc + (9 * ((T + 3) & ~3) + 8) * 4;
  c.off_rec = c.off_win + T * kChunkMaxW * 4;
  c.off_stage = c.off_rec + rec_base(T) * 16;
  c.total = c.off_stage + ((T + W - 1) * 2 * dk * 2 + 4095) / 4096 * 4096;  // whole DMA rounds
  return c;
}

// WT = 4: conv width exactly 4; WT = 8: any width up to 8 (taps past W weigh 0).
// STORE: also hand the per-node states to gdn_states_kernel (ChunkStoreOut) and write
// the conv scratch.
template <int DK, int WT, bool STORE>
__global__ void __launch_bounds__(kChunkThreads) gdn_chunk_kernel(const uint16_t* __restrict__ x, const float* __restrict__ conv_w,
                                                        const uint16_t* __restrict__ conv_state,
                                                        const uint16_t* __restrict__ v, const float* __restrict__ beta,
                                                        const float* __restrict__ g, const float* __restrict__ S,
                                                        uint16_t* __restrict__ o, const int32_t* __restrict__ parent,
                                                        int Tn, int H, int W, ChunkStoreOut so) {
  constexpr int DV = DK, RSB = 2 * DK + 16, NCS = DK / 32, NRT = DV / 16;
  constexpr int NTH = kChunkThreads, NWV = kChunkWaves;
  constexpr int RTW = (NRT + NWV - 1) / NWV;  // 16-row tiles of S0 per wave
  constexpr int NG = DK / 8;           // conv: lanes per (node, q or k part), 8 channels each
  constexpr int NPR = NTH / (2 * NG);  // conv: node slots of the block
  // conv: nodes per thread and pass: one pass for any T <= 65 at the fixed width 4; two for
  // the generic widths, whose 8 taps of weights take the registers
  constexpr int NU = WT == 4 ? (kChunkMaxT + NPR - 1) / NPR : ((kChunkMaxT + NPR - 1) / NPR + 1) / 2;
  constexpr int ROW8 = 2 * DK / 8;     // 16-byte chunks of a staged row
  constexpr int kStageIt = ((kChunkMaxT + kChunkMaxW - 1) * ROW8 + NTH - 1) / NTH;
  constexpr int CPW = DV / NWV;        // solve: columns a wave owns
  constexpr int LPN = CPW / 4;         // solve: lanes per node, 4 columns each
  constexpr int NGP = 64 / LPN;        // solve: nodes a wave holds side by side
  constexpr int NS = (kChunkMaxT + NGP - 1) / NGP;  // solve: node slots per lane
  extern __shared__ __align__(16) uint8_t lds[];
  const int s = blockIdx.x / H, h = blockIdx.x % H;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;
  const int C = 2 * H * DK;
  const ChunkLayout L = chunk_layout(Tn, DK, W);
  const int NTT = (Tn + 15) / 16, RW = L.rows, WS = L.WS;
  const int TP4 = (Tn + 3) & ~3;  // scalar arrays start 16-byte aligned
  int* par = reinterpret_cast<int*>(lds + L.off_sc);
  float* gg = reinterpret_cast<float*>(par + TP4);
  float* be = gg + TP4;
  float* Gam = be + TP4;
  float* Md = Gam + TP4;
  int* dep = reinterpret_cast<int*>(Md + TP4);
  int* cnt = dep + TP4;     // nodes per depth, then the fill counters of the depth order
  int* ord = cnt + TP4;     // the nodes by depth
  int* lstart = ord + TP4;  // [T + 1]: position of the first node of each depth in ord
  int* maxdep = lstart + TP4 + 4;
  int* win = reinterpret_cast<int*>(lds + L.off_win);
  float4* rec = reinterpret_cast<float4*>(lds + L.off_rec);
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds + L.off_stage);

  // ---- P0.  The node scalars and, by LDS DMA, the stage first; then (after the first
  // barrier, which waits for those) S0 and v, which arrive during the walk and the conv.
  // Every address is clamped into range.
  const int tn = min(tid, Tn - 1);
  const int pr = parent[(size_t)s * Tn + tn];
  const float gr = g[((size_t)s * Tn + tn) * H + h], br = beta[((size_t)s * Tn + tn) * H + h];
  // the stage, 16-byte chunk idx = NTH*k + tid: a wave fills 1 KB at a time; chunks past
  // the last repeat it into the stage's padding
  const int nst = (Tn + W - 1) * ROW8;
#pragma unroll
  for (int k = 0; k < kStageIt; ++k) {
    if (NTH * k >= nst) break;
    const int idx = min(tid + NTH * k, nst - 1);
    const int row = idx / ROW8, ch = idx % ROW8;
    const int chan = ch < ROW8 / 2 ? h * DK + 8 * ch : H * DK + h * DK + 8 * (ch - ROW8 / 2);
    const uint16_t* src = row < Tn ? x + ((size_t)s * Tn + row) * C + chan
                                   : conv_state + ((size_t)s * (W - 1) + (row - Tn)) * C + chan;
    __builtin_amdgcn_global_load_lds(src, reinterpret_cast<__attribute__((address_space(3))) void*>(
                                              reinterpret_cast<uintptr_t>(stage + (size_t)(NTH * k + 64 * wave) * 8)),
                                     16, 0, 0);
  }
  // this thread's conv channels: 8 of the head's q (half 0) or k (half 1) channels
  const int cg = tid % NG, half = (tid / NG) & 1, tsub = tid / (2 * NG);
  const int c0 = half * H * DK + h * DK + 8 * cg;  // channel in x
  const int s0 = half * DK + 8 * cg;               // channel in a staged row
  float cw[8][WT];
  if constexpr (WT == 4) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float4 q = *reinterpret_cast<const float4*>(conv_w + (size_t)(c0 + e) * 4);
      cw[e][0] = q.x; cw[e][1] = q.y; cw[e][2] = q.z; cw[e][3] = q.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int c = 0; c < WT; ++c) cw[e][c] = conv_w[(size_t)(c0 + e) * W + min(c, W - 1)];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int c = 0; c < WT; ++c) cw[e][c] = c < W ? cw[e][c] : 0.f;
  }
  par[tn] = pr;
  gg[tn] = gr;
  be[tn] = br;
  cnt[tn] = 0;
  if (tid < 4 * (RSB / 16))  // row T of K hi, K lo, Q hi, Q lo: zero
    *reinterpret_cast<uint4*>(lds + (tid / (RSB / 16)) * RW * RSB + Tn * RSB + (tid % (RSB / 16)) * 16) =
        make_uint4(0, 0, 0, 0);
  __syncthreads();
  // S0 rows r = 16*rt + l16, columns 32*cs + 8*q4 .. +7: the A operands of S0 [K|Q]
  const float* S0 = S + ((size_t)s * H + h) * DV * DK;
  float sop[RTW][NCS][8];
#pragma unroll
  for (int w = 0; w < RTW; ++w) {
    const int rt = min(wave + NWV * w, NRT - 1);
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs) load8<float>(S0 + (size_t)(16 * rt + l16) * DK + 32 * cs + 8 * q4, sop[w][cs]);
  }
  // v of node 16*ti + l16, columns 16*rt + 4*q4 .. +3 (the layout of S0 [K|Q]'s result)
  uint2 vv[RTW][kChunkMaxTT];
#pragma unroll
  for (int w = 0; w < RTW; ++w) {
    const int rt = min(wave + NWV * w, NRT - 1);
#pragma unroll
    for (int ti = 0; ti < kChunkMaxTT; ++ti) {
      const int t = min(16 * ti + l16, Tn - 1);
      vv[w][ti] = *reinterpret_cast<const uint2*>(v + (((size_t)s * Tn + t) * H + h) * DV + 16 * rt + 4 * q4);
    }
  }
  // per node, one walk up the parent chain: conv window (the node, its ancestors, then
  // the committed conv rows, newest first), depth, G_t and the records (row, r_tj)
  if (tid < Tn) {
    const int t = tid, rb = rec_base(t);
    int a = t, k = 0;
    float prod = 1.f;
    win[t * kChunkMaxW] = t;
    while (true) {
      const int p = par[a];
      const float ga = gg[a];
      if (!(p >= 0 && p < a)) {
        Gam[t] = prod * ga;
        break;
      }
      prod *= ga;
      a = p;
      rec[rb + k] = make_float4(__int_as_float(a), prod, 0.f, 0.f);
      ++k;
      if (k < W) win[t * kChunkMaxW + k] = a;
    }
    for (int b = k + 1; b < W; ++b) win[t * kChunkMaxW + b] = Tn + W - 1 - (b - k);
    dep[t] = k;
    atomicAdd(&cnt[k], 1);
  }
  __syncthreads();
  if (STORE) {
    // G_t and the depth; every record slot of t (t slots): its (k+1)-th ancestor and r_tj,
    // or past dep[t] a valid row (t) with ratio 0, so that the states kernel may read t's
    // first slots before its depth
    if (tid < Tn) {
      so.gam[((size_t)s * Tn + tid) * H + h] = Gam[tid];
      if (h == 0) so.dep[(size_t)s * Tn + tid] = dep[tid];
    }
    const int TRI = rec_base(Tn);
    constexpr int kRecIt = (kChunkMaxT * (kChunkMaxT - 1) / 2 + NTH - 1) / NTH;
#pragma unroll
    for (int i = 0; i < kRecIt; ++i) {
      const int idx = min(tid + NTH * i, max(TRI - 1, 0));  // slot rec_base(t) + k
      int t = (int)((1.f + sqrtf(1.f + 8.f * (float)idx)) * 0.5f);
      t -= rec_base(t) > idx;
      t += rec_base(t + 1) <= idx;
      const int k = idx - rec_base(t), dt = dep[t];
      const float4 r = rec[rec_base(t) + min(k, max(dt - 1, 0))];
      if (tid + NTH * i < TRI) {
        so.rho[((size_t)s * H + h) * TRI + idx] = k < dt ? r.y : 0.f;
        if (h == 0) so.rows[(size_t)s * TRI + idx] = k < dt ? __float_as_int(r.x) : t;
      }
    }
  }
  if (wave == 0) {  // depth starts: an exclusive scan of the histogram over 64 lanes (+ depth 64)
    int c = lane < Tn ? cnt[lane] : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int u = __shfl_up(c, off, 64);
      if (lane >= off) c += u;
    }
    // c = nodes of depth <= lane
    if (lane < Tn) lstart[lane + 1] = c;
    // the largest depth: the last nonempty one (depth 64 only in a chain of 65)
    const uint64_t nz = __ballot(lane < Tn && cnt[lane] > 0);
    if (lane == 0) {
      lstart[0] = 0;
      lstart[Tn] = Tn;  // depth Tn - 1 (a chain of 65) lies past the 64 lanes
      *maxdep = (Tn > 64 && cnt[64] > 0) ? 64 : 63 - __builtin_clzll(nz);
    }
  }
  // the short conv of the head's q and k channels from the stage, NU nodes per thread and
  // pass; SiLU; k L2-normalised, q scaled; stored as bf16 high and low parts
  for (int t0 = 0; t0 < Tn; t0 += NU * NPR) {
    float y[NU][8];
    int tt[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      tt[u] = min(t0 + tsub + u * NPR, Tn - 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[u][e] = 0.f;
#pragma unroll
      for (int c = 0; c < WT; ++c) {  // tap c multiplies the row W-1-c back
        const int b = WT == 4 ? 3 - c : max(W - 1 - c, 0);
        const int r = win[tt[u] * kChunkMaxW + b];
        const uint4 raw = *reinterpret_cast<const uint4*>(stage + (size_t)r * (2 * DK) + s0);
        // the conv scratch of the node: its window's newest W-1 rows, tap c (1 <= c <= W-1,
        // back W-1-c) in slot c-1; a clamped duplicate node writes the same bytes
        if (STORE && c >= 1 && (WT == 4 || c <= W - 1))
          *reinterpret_cast<uint4*>(so.conv_scratch + (((size_t)s * Tn + tt[u]) * (W - 1) + (c - 1)) * C + c0) = raw;
        const uint32_t rw[4] = {raw.x, raw.y, raw.z, raw.w};
        float xv[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          xv[2 * i] = __uint_as_float(rw[i] << 16);
          xv[2 * i + 1] = __uint_as_float(rw[i] & 0xffff0000u);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) y[u][e] += cw[e][c] * xv[e];
      }
    }
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[u][e] = y[u][e] * __builtin_amdgcn_rcpf(1.f + __expf(-y[u][e]));
        ss += y[u][e] * y[u][e];
      }
      // k: L2 norm over the head's dk channels (the NG lanes of this node and half; DPP)
      ss = group_sum<NG>(ss);
      const float sc = half ? 1.f / sqrtf(ss + 1e-6f) : rsqrtf((float)DK);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[u][e] *= sc;
      if (STORE && half) {  // the normalised k in fp32 (a clamped duplicate node writes the same values)
        float* kd = so.k + (((size_t)s * Tn + tt[u]) * H + h) * DK + 8 * cg;
        *reinterpret_cast<float4*>(kd) = make_float4(y[u][0], y[u][1], y[u][2], y[u][3]);
        *reinterpret_cast<float4*>(kd + 4) = make_float4(y[u][4], y[u][5], y[u][6], y[u][7]);
      }
      cbf16x8 hi, lo;
      split8(y[u], hi, lo);
      const int base = (half ? 0 : 2) * RW * RSB + tt[u] * RSB + cg * 16;  // K hi/lo first, then Q hi/lo
      *reinterpret_cast<cbf16x8*>(lds + base) = hi;
      *reinterpret_cast<cbf16x8*>(lds + base + RW * RSB) = lo;
    }
  }
  __syncthreads();
  if (tid < Tn) cnt[tid] = 0;  // the fill counters (every read of the histogram is done)
  __syncthreads();
  if (tid < Tn) ord[lstart[dep[tid]] + atomicAdd(&cnt[dep[tid]], 1)] = tid;

  // ---- P1: S0 [K|Q] as D[r][t] (lane: node column 16*ti + l16, rows 16*rt + 4*q4 + e)
  // and the Gram products (results stay in registers).  A tile's rows past the last
  // node read row T, which is zero.
  cbf16x8 sh[RTW][NCS], sl[RTW][NCS];
#pragma unroll
  for (int w = 0; w < RTW; ++w)
#pragma unroll
    for (int cs = 0; cs < NCS; ++cs) split8(sop[w][cs], sh[w][cs], sl[w][cs]);
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
  for (int cs = 0; cs < NCS; ++cs) {
#pragma unroll
    for (int ti = 0; ti < kChunkMaxTT; ++ti) {
      if (ti >= NTT) break;
      const int ro = min(16 * ti + l16, Tn) * RSB + 64 * cs + 16 * q4;
      const cbf16x8 kh = *reinterpret_cast<const cbf16x8*>(Khi + ro);
      const cbf16x8 kl = *reinterpret_cast<const cbf16x8*>(Klo + ro);
      const cbf16x8 qh = *reinterpret_cast<const cbf16x8*>(Qhi + ro);
      const cbf16x8 ql = *reinterpret_cast<const cbf16x8*>(Qlo + ro);
#pragma unroll
      for (int w = 0; w < RTW; ++w) {
        if (wave + NWV * w >= NRT) continue;
        acc[w][ti][0] = mfma3(sh[w][cs], sl[w][cs], kh, kl, acc[w][ti][0]);
        acc[w][ti][1] = mfma3(sh[w][cs], sl[w][cs], qh, ql, acc[w][ti][1]);
      }
    }
  }
  // Gram blocks (ti, tj), tj <= ti, dealt to the waves: K_t . K_j and Q_t . K_j as
  // D[t][j] (lane: j = 16*tj + l16, t = 16*ti + 4*q4 + e)
  constexpr int kMaxPairs = (kChunkMaxTT * (kChunkMaxTT + 1) / 2 + NWV - 1) / NWV;  // per wave
  const int NP = NTT * (NTT + 1) / 2;
  cf32x4 gk[kMaxPairs][2];
  int pti[kMaxPairs], ptj[kMaxPairs];
#pragma unroll
  for (int k = 0; k < kMaxPairs; ++k) {
    gk[k][0] = gk[k][1] = cf32x4{0.f, 0.f, 0.f, 0.f};
    const int p = wave + NWV * k;
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

  // ---- P2: right-hand sides beta_t (v_t - G_t S0 k_t), the o base G_t S0 q_t, M_tt, and
  // the records' coefficients
  float* Wm = reinterpret_cast<float*>(lds);  // [T][WS]: right-hand sides, then w
  float* Ob = Wm + Tn * WS;                   // [T][WS]: G_t S0 q_t
  float bt[kChunkMaxTT], Gt[kChunkMaxTT];
#pragma unroll
  for (int ti = 0; ti < kChunkMaxTT; ++ti) {
    const int tc = min(16 * ti + l16, Tn - 1);
    bt[ti] = be[tc];
    Gt[ti] = Gam[tc];
  }
  // the records: every read first (clamped), then the predicated writes.  The four rows
  // t = 16*ti + 4*q4 .. +3 of a pair are one 16-byte read of each scalar array.
  int rix[kMaxPairs][4];
  float bet[kMaxPairs][4];
#pragma unroll
  for (int k = 0; k < kMaxPairs; ++k) {
    const int t0 = 16 * pti[k] + 4 * q4;
    const int4 d4 = *reinterpret_cast<const int4*>(&dep[t0]);
    const float4 b4 = *reinterpret_cast<const float4*>(&be[t0]);
    const int dj = dep[min(16 * ptj[k] + l16, Tn - 1)];
    const int dt[4] = {d4.x, d4.y, d4.z, d4.w};
    bet[k][0] = b4.x; bet[k][1] = b4.y; bet[k][2] = b4.z; bet[k][3] = b4.w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // t's record at distance dep[t] - dep[j] holds t's ancestor at j's depth: j's
      // own when j is an ancestor of t (rows past the last node are never written)
      const int kk = dt[e] - 1 - dj;
      rix[k][e] = (t0 + e < Tn && kk >= 0 && kk < t0 + e) ? rec_base(t0 + e) + kk : -1;
    }
  }
  float4 rr[kMaxPairs][4];
#pragma unroll
  for (int k = 0; k < kMaxPairs; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) rr[k][e] = rec[max(rix[k][e], 0)];
#pragma unroll
  for (int ti = 0; ti < kChunkMaxTT; ++ti) {
    const int t = 16 * ti + l16;
#pragma unroll
    for (int w = 0; w < RTW; ++w) {
      const int rt = wave + NWV * w;
      if (rt >= NRT) continue;
      const uint2 q = vv[w][ti];
      const float v4[4] = {__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                           __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u)};
      float4 wv, ov;
      wv.x = bt[ti] * (v4[0] - Gt[ti] * acc[w][ti][0][0]);
      wv.y = bt[ti] * (v4[1] - Gt[ti] * acc[w][ti][0][1]);
      wv.z = bt[ti] * (v4[2] - Gt[ti] * acc[w][ti][0][2]);
      wv.w = bt[ti] * (v4[3] - Gt[ti] * acc[w][ti][0][3]);
      ov.x = Gt[ti] * acc[w][ti][1][0];
      ov.y = Gt[ti] * acc[w][ti][1][1];
      ov.z = Gt[ti] * acc[w][ti][1][2];
      ov.w = Gt[ti] * acc[w][ti][1][3];
      if (t < Tn) {
        *reinterpret_cast<float4*>(&Wm[t * WS + 16 * rt + 4 * q4]) = wv;
        *reinterpret_cast<float4*>(&Ob[t * WS + 16 * rt + 4 * q4]) = ov;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kMaxPairs; ++k) {
    if (wave + NWV * k >= NP) continue;
    const int j = 16 * ptj[k] + l16;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = 16 * pti[k] + 4 * q4 + e;
      if (t < Tn && j == t) Md[t] = gk[k][1][e];  // r_tt = 1
      if (rix[k][e] >= 0 && __float_as_int(rr[k][e].x) == j) {
        const float r = rr[k][e].y;
        rec[rix[k][e]].y = bet[k][e] * r * gk[k][0][e];
        rec[rix[k][e]].z = r * gk[k][1][e];
      }
    }
  }
  __syncthreads();

  // ---- P3: the solve, depth by depth, without barriers: wave `wave` owns columns
  // [CPW*wave, CPW*(wave+1)), a lane 4 of them for NS nodes (slots), NGP nodes side by
  // side, slot i holding positions NGP*i .. NGP*i + NGP-1 of the depth order.  At depth e
  // the nodes there are final (w written, o stored); then every deeper node takes its
  // depth-e ancestor's term, whose record was fetched one depth ahead.  The depth order
  // makes the slots of one depth a contiguous range and those of deeper nodes a suffix,
  // so whole slots (groups of GS) are skipped where no lane has work.
  {
    constexpr int GS = 3;
    const int ng = lane / LPN, c = CPW * wave + 4 * (lane % LPN);
    const int nd = __builtin_amdgcn_readfirstlane(*maxdep);
    float4 aw[NS], ao[NS], rv[NS];
    float md[NS];
    int dp[NS], tt[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int pos = NGP * i + ng;
      tt[i] = ord[min(pos, Tn - 1)];
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) dp[i] = NGP * i + ng < Tn ? dep[tt[i]] : -1;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      aw[i] = *reinterpret_cast<const float4*>(&Wm[tt[i] * WS + c]);
      ao[i] = *reinterpret_cast<const float4*>(&Ob[tt[i] * WS + c]);
      md[i] = Md[tt[i]];
      rv[i] = rec[rec_base(tt[i]) + max(dp[i] - 1, 0)];
    }
    int lo = 0;  // lstart[e]
    for (int e = 0;; ++e) {
      const int hi = __builtin_amdgcn_readfirstlane(lstart[e + 1]);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (NGP * (i + 1) <= lo || NGP * i >= hi) continue;  // no node of depth e in slot i
        if (dp[i] != e) continue;
        const int t = tt[i];
        *reinterpret_cast<float4*>(&Wm[t * WS + c]) = aw[i];
        uint2 u;
        u.x = (uint32_t)f32_to_bf16(ao[i].x + md[i] * aw[i].x) | ((uint32_t)f32_to_bf16(ao[i].y + md[i] * aw[i].y) << 16);
        u.y = (uint32_t)f32_to_bf16(ao[i].z + md[i] * aw[i].z) | ((uint32_t)f32_to_bf16(ao[i].w + md[i] * aw[i].w) << 16);
        *reinterpret_cast<uint2*>(o + (((size_t)s * Tn + t) * H + h) * DV + c) = u;
      }
      if (e >= nd) break;
      // slots from i0 on hold nodes deeper than e
      const int i0 = hi / NGP;
#pragma unroll
      for (int g0 = 0; g0 < NS; g0 += GS) {
        if (g0 + GS <= i0) continue;
        float4 wv[GS];
        float ca[GS], cm[GS];
#pragma unroll
        for (int u = 0; u < GS; ++u) {
          const int i = g0 + u;
          if (i >= NS) break;
          const bool act = dp[i] > e;
          const int row = act ? __float_as_int(rv[i].x) : tt[i];
          ca[u] = act ? rv[i].y : 0.f;
          cm[u] = act ? rv[i].z : 0.f;
          wv[u] = *reinterpret_cast<const float4*>(&Wm[row * WS + c]);
          rv[i] = rec[rec_base(tt[i]) + max(dp[i] - 2 - e, 0)];  // the record of depth e + 1
        }
#pragma unroll
        for (int u = 0; u < GS; ++u) {
          const int i = g0 + u;
          if (i >= NS) break;
          aw[i].x -= ca[u] * wv[u].x;
          aw[i].y -= ca[u] * wv[u].y;
          aw[i].z -= ca[u] * wv[u].z;
          aw[i].w -= ca[u] * wv[u].w;
          ao[i].x += cm[u] * wv[u].x;
          ao[i].y += cm[u] * wv[u].y;
          ao[i].z += cm[u] * wv[u].z;
          ao[i].w += cm[u] * wv[u].w;
        }
      }
      lo = hi;
    }
    if (STORE) {
      // w of every node, the wave's own columns (its own LDS writes: no barrier needed)
      for (int idx = lane; idx < Tn * (CPW / 4); idx += 64) {
        const int t = idx / (CPW / 4), cc = CPW * wave + 4 * (idx % (CPW / 4));
        *reinterpret_cast<float4*>(so.w + (((size_t)s * Tn + t) * H + h) * DV + cc) =
            *reinterpret_cast<const float4*>(&Wm[t * WS + cc]);
      }
    }
  }
}

// Every node's state S_t = G_t S0 + sum_{i in path(t)} r_ti w_i k_i^T written out by
// short-lived blocks, each R = RB*RPT rows (RPT*4 KB) of one (sequence, node, head)
// state, blocks in the order of S_scratch.  Blocks that each write one small piece and
// end keep the writes in flight over a narrow, advancing address range, as a fill does;
// a block that writes a whole state (or a persistent block walking nodes) spreads them
// over every state in flight.
// The path is t itself (ratio 1) followed by its records, taken NB at a time: the block
// stages each path node's k row and its ratio times the w of the block's rows in LDS
// (one coalesced pass: 256/NB threads per path node), then a thread (4 columns of RPT
// consecutive rows) adds r w k^T from LDS.  Every node's first record slots hold a valid
// row (ratio 0 past its depth), so the first batch's rows and ratios are read with S0,
// before the depth is known: a node less than NB deep waits on memory twice.
constexpr int kStatesNB = 8;  // path nodes staged per batch

template <int DK, int RPT>
__global__ void __launch_bounds__(256) gdn_states_kernel(const float* __restrict__ S, const float* __restrict__ kf,
                                                         const float* __restrict__ wf, const int32_t* __restrict__ rows,
                                                         const float* __restrict__ rho, const float* __restrict__ gam,
                                                         const int32_t* __restrict__ dep, float* __restrict__ S_scratch,
                                                         int Tn, int H) {
  constexpr int DV = DK, LPR = DK / 4, RB = 256 / LPR, R = RB * RPT, BPS = DV / R;
  static_assert(BPS * R == DV, "a block covers whole rows of one state");
  constexpr int NB = kStatesNB, TPN = 256 / NB;  // path nodes per batch; staging threads per node
  constexpr int NK4 = DK / 4, NW4 = R / 4, NP4 = NK4 + NW4;  // 16-byte pieces per path node
  __shared__ float4 kS[NB][NK4];
  __shared__ __align__(16) float wS[NB][R];
  const int TRI = rec_base(Tn);
  const int state = blockIdx.x / BPS, r0 = (blockIdx.x % BPS) * R;  // state = (s*T + t)*H + h
  const int h = state % H, st = state / H, s = st / Tn, t = st % Tn;
  const int tid = threadIdx.x, c4 = tid % LPR, rr = (tid / LPR) * RPT;  // rows r0+rr .. +RPT-1
  const int base = rec_base(t);
  const int d = dep[st];  // t's records: base .. base + d - 1 (d <= t)
  const float G = gam[state];
  const float* S0 = S + ((size_t)s * H + h) * DV * DK;
  float4 acc[RPT];
#pragma unroll
  for (int q = 0; q < RPT; ++q) acc[q] = *reinterpret_cast<const float4*>(S0 + (size_t)(r0 + rr + q) * DK + 4 * c4);
  const int u = tid / TPN, pl = tid % TPN;  // staging: path node u of the batch, piece lane pl
  for (int i0 = 0; i0 <= d; i0 += NB) {
    // path entry i = i0 + u: t itself (i = 0) or record i-1; the first batch clamps to t's
    // own slots (written for any t >= 1; slot 0 for the root), later ones to the depth
    const int i = i0 + u;
    const int kk = i0 == 0 ? min(max(i - 1, 0), max(t - 1, 0)) : min(i - 1, d - 1);
    const bool rec = i > 0 && TRI > 0;
    const int j = rec ? rows[(size_t)s * TRI + base + kk] : t;
    const float cr = rec ? rho[((size_t)s * H + h) * TRI + base + kk] : 1.f;
    const size_t js = ((size_t)s * Tn + j) * H + h;
    float4 pc[(NP4 + TPN - 1) / TPN];
#pragma unroll
    for (int m = 0; m < (NP4 + TPN - 1) / TPN; ++m) {
      const int o = min(pl + TPN * m, NP4 - 1);
      pc[m] = o < NK4 ? *reinterpret_cast<const float4*>(kf + js * DK + 4 * o)
                      : *reinterpret_cast<const float4*>(wf + js * DV + r0 + 4 * (o - NK4));
    }
    const float c = i <= d ? cr : 0.f;  // past t's path: weight 0
    if (i0 > 0) __syncthreads();        // the previous batch's reads are done
#pragma unroll
    for (int m = 0; m < (NP4 + TPN - 1) / TPN; ++m) {
      const int o = pl + TPN * m;
      if (o < NK4) kS[u][o] = pc[m];
      else if (o < NP4) *reinterpret_cast<float4*>(&wS[u][4 * (o - NK4)]) =
          make_float4(c * pc[m].x, c * pc[m].y, c * pc[m].z, c * pc[m].w);
    }
    __syncthreads();
    if (i0 == 0) {
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        acc[q].x *= G;
        acc[q].y *= G;
        acc[q].z *= G;
        acc[q].w *= G;
      }
    }
    const int nv = min(NB, d + 1 - i0);  // path nodes of this batch (uniform)
#pragma unroll
    for (int v = 0; v < NB; ++v) {
      if (v >= nv) break;
      const float4 kv = kS[v][c4];
      float wv[RPT];
      if constexpr (RPT == 4) {
        const float4 w4 = *reinterpret_cast<const float4*>(&wS[v][rr]);
        wv[0] = w4.x; wv[1] = w4.y; wv[2] = w4.z; wv[3] = w4.w;
      } else {
#pragma unroll
        for (int q = 0; q < RPT; ++q) wv[q] = wS[v][rr + q];
      }
#pragma unroll
      for (int q = 0; q < RPT; ++q) {
        acc[q].x += wv[q] * kv.x;
        acc[q].y += wv[q] * kv.y;
        acc[q].z += wv[q] * kv.z;
        acc[q].w += wv[q] * kv.w;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < RPT; ++q) {
    const cf32x4 out = {acc[q].x, acc[q].y, acc[q].z, acc[q].w};
    __builtin_nontemporal_store(out, reinterpret_cast<cf32x4*>(S_scratch + ((size_t)state * DV + r0 + rr + q) * DK + 4 * c4));
  }
}

size_t gdn_chunk_lds_bytes(int T, int dk, int W) { return (size_t)chunk_layout(T, dk, W).total; }

template <int DK, int WT, bool STORE>
static void launch_chunk(const void* x, const float* conv_w, const void* conv_state, const void* v,
                         const float* beta, const float* g, const float* S, void* o, const int32_t* parent, int n,
                         int T, int H, int W, const ChunkStoreOut& so, hipStream_t st) {
  auto kern = gdn_chunk_kernel<DK, WT, STORE>;
  // the dynamic LDS limit is raised once per kernel, to the largest size any call uses
  // (a host-side attribute, not a stream operation: calls stay capturable in a graph)
  static const bool attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                               hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)gdn_chunk_lds_bytes(kChunkMaxT, DK, kChunkMaxW)) == hipSuccess;
  (void)attr;
  hipLaunchKernelGGL(kern, dim3(n * H), dim3(kChunkThreads), gdn_chunk_lds_bytes(T, DK, W), st,
                     static_cast<const uint16_t*>(x), conv_w, static_cast<const uint16_t*>(conv_state),
                     static_cast<const uint16_t*>(v), beta, g, S, static_cast<uint16_t*>(o), parent, T, H, W, so);
}

template <int DK, bool STORE>
static void launch_chunk_w(const void* x, const float* conv_w, const void* conv_state, const void* v,
                           const float* beta, const float* g, const float* S, void* o, const int32_t* parent, int n,
                           int T, int H, int W, const ChunkStoreOut& so, hipStream_t st) {
  if (W == 4)
    launch_chunk<DK, 4, STORE>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, so, st);
  else
    launch_chunk<DK, 8, STORE>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, so, st);
}

static bool chunk_shape_ok(int act_dt, int T, int W, int dk) {
  return act_dt == DDT_BF16 && T >= 1 && T <= kChunkMaxT && W >= 1 && W <= kChunkMaxW &&
         (dk == 32 || dk == 64 || dk == 128);
}

hipError_t launch_gdn_chunk(const void* x, const float* conv_w, const void* conv_state, const void* v,
                            const float* beta, const float* g, const float* S, void* o, const int32_t* parent, int n,
                            int T, int H, int dk, int W, int act_dt, hipStream_t st) {
  // bf16 activations only (fp32 ones keep the node-by-node walk); T <= 65, W <= 8
  if (!chunk_shape_ok(act_dt, T, W, dk)) return hipErrorInvalidValue;
  const ChunkStoreOut none = {};
  if (dk == 32) launch_chunk_w<32, false>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, none, st);
  else if (dk == 64) launch_chunk_w<64, false>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, none, st);
  else launch_chunk_w<128, false>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, none, st);
  return hipGetLastError();
}

constexpr int kStatesRPT = 4;  // 16 KB of states per block

size_t gdn_chunk_store_bytes(int n, int T, int H) {
  const size_t tri = (size_t)rec_base(T);
  return ((size_t)n * tri * 4 + 255) / 256 * 256 + ((size_t)n * H * tri * 4 + 255) / 256 * 256;
}

// The record tables follow one another in `tables`: rows [n][TRI] int32, then rho [n][H][TRI].
static float* rho_table(void* tables, int n, int T) {
  return reinterpret_cast<float*>(static_cast<uint8_t*>(tables) + ((size_t)n * rec_base(T) * 4 + 255) / 256 * 256);
}

hipError_t launch_gdn_chunk_exports(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch,
                                    const void* v, const float* beta, const float* g, const float* S, void* o,
                                    const int32_t* parent, int n, int T, int H, int dk, int W, int act_dt, float* kbuf,
                                    float* wbuf, float* gam, int32_t* dep, void* tables, hipStream_t st) {
  if (!chunk_shape_ok(act_dt, T, W, dk) || W < 2) return hipErrorInvalidValue;
  ChunkStoreOut so;
  so.conv_scratch = static_cast<uint16_t*>(conv_scratch);
  so.k = kbuf;
  so.w = wbuf;
  so.gam = gam;
  so.dep = dep;
  so.rows = static_cast<int32_t*>(tables);
  so.rho = rho_table(tables, n, T);
  if (dk == 32) launch_chunk_w<32, true>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, so, st);
  else if (dk == 64) launch_chunk_w<64, true>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, so, st);
  else launch_chunk_w<128, true>(x, conv_w, conv_state, v, beta, g, S, o, parent, n, T, H, W, so, st);
  return hipGetLastError();
}

hipError_t launch_gdn_states(const float* S, float* S_scratch, int n, int T, int H, int dk, const float* kbuf,
                             const float* wbuf, const float* gam, const int32_t* dep, const void* tables,
                             hipStream_t st) {
  if (T < 1 || T > kChunkMaxT || !(dk == 32 || dk == 64 || dk == 128)) return hipErrorInvalidValue;
  const int32_t* rows = static_cast<const int32_t*>(tables);
  const float* rho = rho_table(const_cast<void*>(tables), n, T);
#define DDT_STATES(DKV)                                                                                          \
  do {                                                                                                           \
    constexpr int RPT = kStatesRPT * 1024 <= DKV * DKV ? kStatesRPT : DKV * DKV / 1024;                          \
    hipLaunchKernelGGL((gdn_states_kernel<DKV, RPT>), dim3((unsigned)((size_t)n * T * H * DKV * DKV / (1024 * RPT))), \
                       dim3(256), 0, st, S, kbuf, wbuf, rows, rho, gam, dep, S_scratch, T, H);                  \
  } while (0)
  if (dk == 32) DDT_STATES(32);
  else if (dk == 64) DDT_STATES(64);
  else DDT_STATES(128);
#undef DDT_STATES
  return hipGetLastError();
}

hipError_t launch_gdn_chunk_stored(const void* x, const float* conv_w, const void* conv_state, void* conv_scratch,
                                   const void* v, const float* beta, const float* g, const float* S, float* S_scratch,
                                   void* o, const int32_t* parent, int n, int T, int H, int dk, int W, int act_dt,
                                   float* kbuf, float* wbuf, float* gam, int32_t* dep, void* tables, hipStream_t st) {
  const hipError_t e = launch_gdn_chunk_exports(x, conv_w, conv_state, conv_scratch, v, beta, g, S, o, parent, n, T, H,
                                                dk, W, act_dt, kbuf, wbuf, gam, dep, tables, st);
  if (e != hipSuccess) return e;
  return launch_gdn_states(S, S_scratch, n, T, H, dk, kbuf, wbuf, gam, dep, tables, st);
}

}  // namespace ddt
