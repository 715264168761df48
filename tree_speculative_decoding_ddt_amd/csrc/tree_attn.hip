// Tree-masked attention: every tree row attends to the committed prefix, the root,
// its ancestors and itself -- never to a sibling.
// Sources: "DDTree on vLLM: candid research notes", section "Why hybrid attention
// makes it hard" (prefix + own ancestors, never siblings); "From DDTree to drafter
// training", section "The Architecture of DDTree" (one verify pass over root + all
// nodes with an ancestor-only mask).
//
// bf16, D in {128, 256}: matrix-core path.
//   Rows of one kv head are the G = Hq/Hkv query heads of all T tree rows, flattened
//   r = t*G + h_local and cut into 16-row tiles; a wave owns up to NT tiles (and runs
//   the products of only those that hold rows), a block (NW = 8 waves) shares each
//   32-key K/V tile in LDS.  Per 32 keys:
//     S^T = K Q^T   v_mfma_f32_16x16x32_bf16, A = K rows from LDS, B = Q from VGPRs;
//                   each lane then holds 8 scores of ONE query row,
//     softmax in the log2 domain (fp32) against a reference fixed for the pass
//                   (a pass is redone once if a score overshoots it),
//     O^T += V^T P^T  A = V^T from LDS, B = P straight from the score registers.
//   Keys are the contraction index of the second product and V sits in LDS key-major
//   as copied, so each A operand (8 keys of one column d) comes from two transposing
//   reads (ds_read_b64_tr_b16), keys 4*q4..+3 and 16+4*q4..+3: the same key order in
//   which S^T leaves a lane's 8 scores, so P feeds the B operand straight from them.
//   The prefix is split across blocks (split-K); one extra split handles the T tree
//   keys under the ancestor mask.  Each split writes (lse, O/l) per row and a combine
//   kernel merges them with log-sum-exp weights.
// fp32 (any D in {64,128,256}) and bf16 D=64: scalar path, one wavefront per
//   (sequence, row, head), prefix then visible tree keys, no workspace.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnNK = 32;      // keys per K/V tile (bf16 path)
constexpr int kAttnStages = 4;   // LDS ring of K/V tiles (bf16 path)
constexpr int kAttnMinSplit = 256;  // fewest prefix keys per split: a split's (lse, O) partials
                                    // cost about the traffic of 400 keys of K/V, but with few
                                    // sequences more splits fill more of the 256 CUs
constexpr float kMaxRowSum = 0x1p64f;  // a pass whose row sum reaches this is redone (see below)
constexpr int kPageTab = 1024;   // block-table entries a paged split stages in LDS

// ------------------------------------------------------------------ scalar path
template <typename T, int D, bool PAGED>
__global__ void __launch_bounds__(64) attn_scalar_kernel(const T* __restrict__ q, const T* __restrict__ k_cache,
                                                         const T* __restrict__ v_cache,
                                                         const int32_t* __restrict__ prefix_len,
                                                         const T* __restrict__ k_tree, const T* __restrict__ v_tree,
                                                         const uint64_t* __restrict__ anc, int Tn, int Hq, int Hkv,
                                                         int Pmax, float scale, PagedKV pg, T* __restrict__ out) {
  constexpr int DPL = D / 64;
  const int bid = blockIdx.x;
  const int h = bid % Hq;
  const int i = (bid / Hq) % Tn;
  const int s = bid / (Hq * Tn);
  const int kvh = h / (Hq / Hkv);
  const int lane = threadIdx.x;
  __shared__ float qs[D];
  for (int d = lane; d < D; d += 64) qs[d] = Elem<T>::load(q, (((size_t)s * Tn + i) * Hq + h) * D + d) * scale;
  __syncthreads();
  float m = -INFINITY, l = 0.f, acc[DPL];
#pragma unroll
  for (int j = 0; j < DPL; ++j) acc[j] = 0.f;

  // element offset of prefix row `key` of this (sequence, kv head) in the cache or page pool
  auto prow = [&](int key) -> size_t {
    if constexpr (PAGED) return pg.row(s, kvh, Hkv, key) * D;
    else return ((size_t)(s * Hkv + kvh) * Pmax + key) * D;
  };
  auto block = [&](float sc, const T* vbase, int vrow0, bool pre) {
    const float mb = wave_max(sc);
    const float mn = fmaxf(m, mb);
    if (mn == -INFINITY) return;
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - mn);
    const float p = (sc == -INFINITY) ? 0.f : expf(sc - mn);
    l = l * alpha + wave_sum(p);
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] *= alpha;
    for (int u = 0; u < 64; ++u) {
      const float pu = __shfl(p, u, 64);
      if (pu != 0.f) {
        const size_t rb = pre ? prow(vrow0 + u) : (size_t)(vrow0 + u) * D;
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] += pu * Elem<T>::load(vbase, rb + lane + 64 * j);
      }
    }
    m = mn;
  };

  const int P = min(max(prefix_len[s], 0), Pmax);
  for (int k0 = 0; k0 < P; k0 += 64) {
    const int key = k0 + lane;
    float sc = -INFINITY;
    if (key < P) {
      const size_t kr = prow(key);
      float d0 = 0.f;
      for (int d = 0; d < D; ++d) d0 += qs[d] * Elem<T>::load(k_cache, kr + d);
      sc = d0;
    }
    block(sc, v_cache, k0, true);
  }
  const uint64_t a = anc[(size_t)s * Tn + i];
  const T* kt = k_tree + (size_t)(s * Hkv + kvh) * Tn * D;
  const T* vt = v_tree + (size_t)(s * Hkv + kvh) * Tn * D;
  for (int j0 = 0; j0 < Tn; j0 += 64) {
    const int j = j0 + lane;
    const bool vis = j < Tn && (j == 0 || ((a >> (j - 1)) & 1ull));
    float sc = -INFINITY;
    if (vis) {
      float d0 = 0.f;
      for (int d = 0; d < D; ++d) d0 += qs[d] * Elem<T>::load(kt, (size_t)j * D + d);
      sc = d0;
    }
    block(sc, vt, j0, false);
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int j = 0; j < DPL; ++j)
    Elem<T>::store(out, (((size_t)s * Tn + i) * Hq + h) * D + lane + 64 * j, acc[j] * inv);
}

// ------------------------------------------------------------------ bf16 matrix-core path
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// 16 bytes per lane from global memory straight into LDS (global_load_lds_dwordx4): lane
// l's bytes land at LDS byte address lds_addr + 16*l.  Written as inline asm so that the
// compiler does not treat the in-flight copy as aliasing every later LDS read (it would
// wait for all outstanding copies before each read); the kernel counts vmcnt itself.
// The source is a wave-uniform row base p plus this lane's byte offset voff, so the
// address sums stay in scalar registers (no per-copy vector arithmetic).  The base is
// first copied into scratch SGPRs by a scalar move inside the asm, so the load reads
// SGPRs last written by a scalar instruction: an SGPR written by a vector instruction
// (e.g. a spill reload with v_readlane) needs 5 wait states before a vector-memory
// instruction reads it, and the compiler does not insert them around inline asm.
__device__ __forceinline__ void dma16s(const void* p, uint32_t voff, uint32_t lds_addr) {
  uint64_t tmp;
  uint32_t saved;
  asm volatile(
      "s_mov_b64 %0, %3\n\ts_mov_b32 %1, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %0 offset:0\n\ts_mov_b32 m0, %1"
      : "=&s"(tmp), "=&s"(saved)
      : "v"(voff), "s"(p), "s"(lds_addr)
      : "memory");
}
// Workgroup barrier without a memory fence: copies into other LDS stages stay in flight.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }
// s_waitcnt with vmcnt = n (0..63) and the other counters left unconstrained.
#define DDT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int N> struct IntC { static constexpr int value = N; };
// f(IntC<min(n, N)>) for a wave-uniform count n >= 0
template <int N, typename F>
__device__ __forceinline__ void dispatch_count(int n, F& f) {
  if constexpr (N == 0) {
    f(IntC<0>{});
  } else {
    if (n >= N) f(IntC<N>{});
    else dispatch_count<N - 1>(n, f);
  }
}

// Block = NW waves (two per SIMD) sharing one ring of K/V tiles in LDS; a wave owns NT
// 16-row tiles of the flattened (tree row, q head) rows of one kv head.  The 4-stage
// ring holds tile it, whose S = K Q^T, softmax and O += V^T P^T all run in iteration it,
// and tiles it+1..it+3 whose copies are in flight (three tiles ahead keep more bytes
// in flight than deferring tile it's P.V to the next iteration and prefetching two).
// The two waves of a SIMD overlap one's softmax with the other's matrix-core products.
template <int D, int NT, int NW, int PK, bool PAGED>
__global__ void __launch_bounds__(NW * 64, 1) attn_mfma_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k_cache,
                                                           const uint16_t* __restrict__ v_cache,
                                                           const int32_t* __restrict__ prefix_len,
                                                           const uint16_t* __restrict__ k_tree,
                                                           const uint16_t* __restrict__ v_tree,
                                                           const uint64_t* __restrict__ anc, int Tn, int Hq,
                                                           int Hkv, int Pmax, float sl2, int nwg, int nsplit,
                                                           int split_len, int units, PagedKV pg,
                                                           float* __restrict__ part_lse, float* __restrict__ part_o,
                                                           uint16_t* __restrict__ out) {
  constexpr int NK = kAttnNK, NST = kAttnStages;
  constexpr int ROWB = D * 2, LPR = ROWB / 16;  // bytes of a key row, DMA lanes per key row
  constexpr int RS = ROWB + 32;                 // LDS row stride (padded, see below)
  constexpr int TILE = NK * RS;                 // bytes of one K (or V) tile in LDS
  constexpr int RPW = NK / NW;                  // key rows each wave copies per K (or V) tile
  constexpr int DS = D / 32, DB = D / 16;
  __shared__ __align__(1024) uint8_t lds[NST * 2 * TILE];

  // XCD-aware placement: block ids are dealt to the 8 XCDs round-robin, so the nwg row
  // groups of one (sequence, kv head, split) get ids 8 apart and share one L2.
  const int jb = blockIdx.x >> 3;
  const int grp = jb % nwg;
  const int u = (jb / nwg) * 8 + (blockIdx.x & 7);
  if (u >= units) return;
  const int split = u % nsplit;
  const int kvh = (u / nsplit) % Hkv;
  const int s = u / (nsplit * Hkv);
  const bool last = split == nsplit - 1;
  const int G = Hq / Hkv, R = Tn * G, ntiles = (R + 15) / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l16 = lane & 15, q4 = lane >> 4;

  // key tiles: this split's slice of the prefix, then (last split) the tree rows.  The
  // split length is this sequence's: its prefix plus the tree keys spread evenly over the
  // nsplit splits in whole tiles (split_len, planned from the cache capacity, bounds it),
  // so a prefix shorter than the capacity does not leave the last split short and the
  // others long
  const int P = min(max(prefix_len[s], 0), Pmax);
  const int ttl = (Tn + NK - 1) / NK * NK;
  const int sl = min(split_len, ((P + ttl + nsplit - 1) / nsplit + NK - 1) / NK * NK);
  const int k_beg = min(split * sl, P);
  const int k_end = last ? P : min(P, k_beg + sl);
  const int n_pre = (k_end - k_beg + NK - 1) / NK;
  const int n_all = n_pre + (last ? (Tn + NK - 1) / NK : 0);
  const size_t hoff = (size_t)s * Hkv + kvh;
  // contiguous: this (sequence, kv head)'s rows; paged: the pool (rows found per page)
  const uint16_t* Kp = PAGED ? k_cache : k_cache + hoff * Pmax * D;
  const uint16_t* Vp = PAGED ? v_cache : v_cache + hoff * Pmax * D;
  const uint16_t* Kt = k_tree + hoff * Tn * D;
  const uint16_t* Vt = v_tree + hoff * Tn * D;

  // LDS layout of a tile: key row r at r*RS, RS = row bytes + 32, so consecutive rows
  // start 32 bytes apart modulo the 256 bytes the banks span, chunks in row order.  The
  // K operand reads (16 bytes per lane) and the transposing V reads then run without bank
  // conflicts (the hardware counter reads zero; an XOR swizzle of the chunks by row,
  // tried first, caused conflicts on a third of the LDS-active cycles), and every read
  // address is a per-lane base plus an immediate offset.
  const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(lds);
  // paged: the block-table entries of this split's pages, staged in LDS once (clamped into
  // the pool) when they fit, so that a prefix row's page is an in-order LDS read instead of
  // a scalar load that may miss the scalar cache; wider splits keep the scalar lookups
  __shared__ int32_t pgtab[PAGED ? kPageTab : 1];
  const int pfirst = PAGED ? k_beg >> pg.lps : 0;
  const int pcount = PAGED && k_end > k_beg ? ((k_end - 1) >> pg.lps) - pfirst + 1 : 0;
  const bool use_tab = PAGED && pcount <= kPageTab;
  if constexpr (PAGED) {
    if (use_tab)
      for (int i = threadIdx.x; i < pcount; i += NW * 64) {
        const int g = pg.bt[(size_t)s * pg.maxb + pfirst + i];
        pgtab[i] = g < 0 ? 0 : (g >= pg.npages ? pg.npages - 1 : g);
      }
  }
  auto issue = [&](int it) {
    const uint32_t kb = lds0 + (uint32_t)((it % NST) * 2 * TILE);
    const bool pre = it < n_pre;
    const int r0 = pre ? k_beg + it * NK : (it - n_pre) * NK;
    const int rows = pre ? k_end - r0 : Tn - r0;  // rows past the end repeat the last one (masked later)
    const uint16_t* Kg = pre ? Kp : Kt;
    const uint16_t* Vg = pre ? Vp : Vt;
    // the lane id is recomputed here: hoisted out of the loop it would be spilled, and a
    // scratch reload waits for every outstanding copy (they share vmcnt)
    int ln;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
    // paged: the pool rows of this wave's RPW key rows (wave-uniform scalar lookups).  With
    // the staged table and pages of at least 4 keys, a wave copies 4 consecutive key rows
    // (tiles start 32 keys apart, so they lie in one page): one lookup, then base + 1, 2, 3
    size_t prow[RPW];
    bool grp4 = false;
    if constexpr (PAGED) {
      static_assert(RPW == 4, "the paged lookup batches four rows per wave");
      if (pre) {
        grp4 = use_tab && pg.lps >= 2;
        if (grp4) {
          const int key0 = r0 + min(4 * wave, rows - 1);
          const int pgid = __builtin_amdgcn_readfirstlane(pgtab[(key0 >> pg.lps) - pfirst]);  // one value for the wave
          const size_t p0 = (((size_t)pgid * Hkv + kvh) << pg.lps) + (key0 & ((1 << pg.lps) - 1));
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const size_t pr = p0 + (size_t)(min(4 * wave + k, rows - 1) - (key0 - r0));
            prow[k] = ((size_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(pr >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)pr);
          }
        } else {
          int keys[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) keys[k] = r0 + min(wave + NW * k, rows - 1);
          if (use_tab) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              prow[k] = (((size_t)pgtab[(keys[k] >> pg.lps) - pfirst] * Hkv + kvh) << pg.lps) +
                        (keys[k] & ((1 << pg.lps) - 1));
          } else {
            pg.rows_uniform4(s, kvh, Hkv, keys, prow);
          }
        }
      }
    }
    if (ln < LPR) {
#pragma unroll
      for (int k = 0; k < RPW; ++k) {
        const int row = grp4 ? 4 * wave + k : wave + NW * k;
        const int key = r0 + min(row, rows - 1);
        size_t e = (size_t)key * D;  // wave-uniform row start
        if constexpr (PAGED)
          if (pre) e = prow[k] * D;
        const uint32_t voff = (uint32_t)ln << 4;  // this lane's 16-byte chunk
        const uint32_t m = kb + (uint32_t)(row * RS);
        dma16s(Kg + e, voff, m);
        dma16s(Vg + e, voff, m + TILE);
      }
    }
  };

  // this wave's tiles and Q fragments (B operand of S^T: row l16, d = 32*st + 8*q4 .. +7)
  // Two row groups and an odd tile count: group 0 holds one tile more.  The slot of
  // group 1 that would hold the tile past the last one recomputes group 0's last tile
  // instead (its result is dropped), so both groups carry the same load per key tile and
  // keep pace: the K/V tiles they share are then read from HBM once and hit in L2.
  const int tdup = (nwg == 2 && (ntiles & 1)) ? ntiles - 1 : -1;
  int tile[NT];
  bf16x8 Qf[NT][DS];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    tile[j] = grp + nwg * (wave + NW * j);
    if (tdup >= 0 && tile[j] == ntiles) tile[j] = tdup;
    const int r = tile[j] * 16 + l16;
    const bool ok = tile[j] < ntiles && r < R;
    const int trow = ok ? r / G : 0;
    const int hl = ok ? r % G : 0;
    const uint16_t* qp = q + (((size_t)s * Tn + trow) * Hq + kvh * G + hl) * D + 8 * q4;
#pragma unroll
    for (int st = 0; st < DS; ++st) {
      uint4 w = ok ? *reinterpret_cast<const uint4*>(qp + 32 * st) : make_uint4(0, 0, 0, 0);
      Qf[j][st] = __builtin_bit_cast(bf16x8, w);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);  // Q and masks in registers before the copy counting starts
  if constexpr (PAGED) __syncthreads();  // the staged page table before the first copy

  // tile it must have landed (tiles it+1, it+2 may stay in flight: 2*RPW copies each,
  // completed in issue order); the barrier also means every wave is done with tile
  // it-1, whose stage is refilled with tile it+3
  auto sync_tile = [&](int it) {
    if (it + 2 < n_all) DDT_WAIT_VMCNT(4 * RPW);
    else if (it + 1 < n_all) DDT_WAIT_VMCNT(2 * RPW);
    else DDT_WAIT_VMCNT(0);
    barrier_nofence();
  };
  // the copies of tile it+3 (into the stage of tile it-1, free since the barrier) are
  // issued after tile it's first products, whose matrix-core time covers their scalar
  // address work
  auto refill = [&](int it) {
    if (it + 3 < n_all) issue(it + 3);
  };

  // per-lane LDS read bases inside a stage (K: key row 16h + l16, chunk 4*st + q4; V:
  // row 16h + 4*q4 + l16/4 of a transposing read, chunk 2*b + (l16 & 3)/2); the step
  // index enters as an immediate offset (64*st for K, 32*b for V)
  int kbase[2], vbase[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = 16 * h + l16;
    kbase[h] = key * RS + (q4 << 4);
    const int vkey = 16 * h + 4 * q4 + (l16 >> 2);
    vbase[h] = TILE + vkey * RS + (((l16 & 3) >> 1) << 4) + (l16 & 1) * 8;
  }

  f32x4 O[NT][DB];
  float m[NT];    // softmax reference of the row (log2 units), fixed for a pass
  float l[NT];    // this lane's share of the row sum (8 of the row's keys per tile)
  float mxs[NT];  // largest exponent argument (score in log2 units - m) of a tracking pass
  bf16x8 Pp[NT];  // P of the current tile, B operand of its P.V product

  // S^T blocks: Sacc[j][h] lane (l16, q4) element e = key 16h + 4*q4 + e of row l16.
  // The 2*DS operand reads are issued PK ahead of the products that use them (the
  // sched_group_barrier sequence pins that order for the machine scheduler).
  auto s_phase = [&](auto NAc, int stage, f32x4 (&Sacc)[NT][2]) {
    constexpr int NA = decltype(NAc)::value;
    if constexpr (NA > 0) {
    const uint8_t* Ks = lds + stage * 2 * TILE;
    constexpr int NOP = 2 * DS;
#pragma unroll
    for (int j = 0; j < NA; ++j) Sacc[j][0] = Sacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 Kop[NOP];
#pragma unroll
    for (int i = 0; i < NOP; ++i) Kop[i] = *reinterpret_cast<const bf16x8*>(Ks + kbase[i & 1] + 64 * (i >> 1));
#pragma unroll
    for (int i = 0; i < NOP; ++i)
#pragma unroll
      for (int j = 0; j < NA; ++j)
        Sacc[j][i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Kop[i], Qf[j][i >> 1], Sacc[j][i & 1], 0, 0, 0);
    if constexpr (PK > 0) {  // PK = 0: leave the order to the scheduler
      __builtin_amdgcn_sched_group_barrier(0x100, PK, 0);  // DS reads
#pragma unroll
      for (int i = 0; i < NOP; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NA, 0);  // MFMA
        if (i + PK < NOP) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    }
  };
  // O^T += V^T P^T: A = V^T (d = 16b + l16; keys 4*q4 + 0..3, then 16 + 4*q4 + 0..3),
  // two transposing reads per block, issued two blocks ahead of their products
  auto pv_phase = [&](auto NAc, int stage) {
    constexpr int NA = decltype(NAc)::value;
    if constexpr (NA > 0) {
    const uint8_t* Vs = lds + stage * 2 * TILE;
    // rolling prefetch: the transposing reads of block b+2 are issued before the
    // products of block b (a sched_barrier after each block keeps that order)
    s16x4 lo[3], hi[3];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      lo[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + vbase[0] + 32 * b));
      hi[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + vbase[1] + 32 * b));
    }
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      if (b + 2 < DB) {
        lo[(b + 2) % 3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + vbase[0] + 32 * (b + 2)));
        hi[(b + 2) % 3] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + vbase[1] + 32 * (b + 2)));
      }
      const bf16x8 A =
          __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[b % 3], hi[b % 3], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int j = 0; j < NA; ++j) O[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Pp[j], O[j][b], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    }
  };
  // ancestor mask of this lane's row in tile j (tree tiles only: read when needed)
  auto anc_row = [&](int j) -> uint64_t {
    const int r = tile[j] * 16 + l16;
    return (tile[j] < ntiles && r < R) ? anc[(size_t)s * Tn + r / G] : 0ull;
  };
  // scores of tile j, invisible keys at -inf when masked (prefix tail or tree tile)
  auto scores = [&](const f32x4 (&Sacc)[NT][2], int j, bool masked, bool tree, int kb, int kend, float (&sv)[8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = Sacc[j][h][e];
        if (masked) {
          const int key = kb + 16 * h + 4 * q4 + e;
          bool vis = key < kend;
          if (tree) vis = vis && (key == 0 || ((anc_row(j) >> (key - 1)) & 1ull));
          x = vis ? x : -INFINITY;
        }
        sv[4 * h + e] = x;
      }
  };
  // P = 2^(score*scale*log2e - m) against the pass's fixed reference.  TRACK (only in a
  // redo, see below) also records the largest exponent argument of each row.
  auto softmax = [&](auto NAc, auto TRc, const f32x4 (&Sacc)[NT][2], bool masked, bool tree, int kb, int kend,
                     bf16x8 (&Pout)[NT]) {
    constexpr int NA = decltype(NAc)::value;
    constexpr bool TRACK = decltype(TRc)::value;
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      float sv[8];
      scores(Sacc, j, masked, tree, kb, kend, sv);
      // the exponent arguments: results of arithmetic, so their maximum needs no NaN
      // canonicalisation of the raw matrix-core outputs
      float a[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] = fmaf(sv[e], sl2, -m[j]);
      if constexpr (TRACK) {
        float mx = a[0];
#pragma unroll
        for (int e = 1; e < 8; ++e) mx = fmaxf(mx, a[e]);
        mxs[j] = fmaxf(mxs[j], mx);
      }
      float r = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = __builtin_amdgcn_exp2f(a[e]);
        r += p;
        Pout[j][e] = static_cast<__bf16>(p);
      }
      l[j] += r;
    }
  };
  // row max of the raw scores of tile j over the 4 lanes that hold the row
  auto row_max = [&](float x) {
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    return fmaxf(x, __shfl_xor(x, 32, 64));
  };

  // key tiles [0, n_full) need no mask; [n_full, n_all) are the prefix tail and the tree
  const int n_full = (k_end - k_beg) / NK;
  __shared__ int redo_vote;
  if (threadIdx.x == 0) redo_vote = 0;
#pragma unroll
  for (int j = 0; j < NT; ++j) {  // a split with no keys writes lse = -inf and O = 0
    m[j] = -INFINITY;
    mxs[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) O[j][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // One pass over this split's key tiles, for a wave that owns NA valid 16-row tiles
  // (its first NA; the rest lie past the last row): tiles past the rows run no products
  // (the K/V operand reads, shared by a wave's tiles, are skipped only when NA = 0), but
  // the wave still copies its share of every K/V tile and meets every barrier.
  auto one_pass = [&](auto NAc, auto TRc, bool first) __attribute__((always_inline)) {
    constexpr int NA = decltype(NAc)::value;
    issue(0);  // every wave enters a pass with no copy in flight
    if (n_all > 1) issue(1);
    if (n_all > 2) issue(2);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      l[j] = 0.f;
      mxs[j] = -INFINITY;
#pragma unroll
      for (int b = 0; b < DB; ++b) O[j][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // tile 0: S, then (first pass) the reference from its exact row max
    {
      sync_tile(0);
      const bool tree = 0 >= n_pre;
      const int kb = tree ? 0 : k_beg;
      const int kend = tree ? Tn : k_end;
      const bool masked = tree || kb + NK > kend;
      f32x4 Sacc[NT][2];
      s_phase(NAc, 0, Sacc);
      refill(0);
      if (first) {
#pragma unroll
        for (int j = 0; j < NA; ++j) {
          float sv[8];
          scores(Sacc, j, masked, tree, kb, kend, sv);
          float mx = sv[0];
#pragma unroll
          for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
          m[j] = row_max(mx) * sl2;  // every row sees at least one key of its first tile
        }
      }
      softmax(NAc, TRc, Sacc, masked, tree, kb, kend, Pp);
      pv_phase(NAc, 0);
    }
    int it = 1;
    for (; it < n_full; ++it) {
      sync_tile(it);
      f32x4 Sacc[NT][2];
      s_phase(NAc, it % NST, Sacc);
      refill(it);
      softmax(NAc, TRc, Sacc, false, false, 0, 0, Pp);
      pv_phase(NAc, it % NST);
    }
    for (; it < n_all; ++it) {  // the prefix tail and the tree tiles, under the mask
      sync_tile(it);
      const bool tree = it >= n_pre;
      const int kb = tree ? (it - n_pre) * NK : k_beg + it * NK;
      const int kend = tree ? Tn : k_end;
      f32x4 Sacc[NT][2];
      s_phase(NAc, it % NST, Sacc);
      refill(it);
      softmax(NAc, TRc, Sacc, true, tree, kb, kend, Pp);
      pv_phase(NAc, it % NST);
    }
  };
  // The reference of a row is the exact maximum of its first key tile, so later keys may
  // lie above it.  A pass whose row sum l reached 2^64 (or overflowed) may have lost
  // precision or range in P and O; it is redone, rarely and only for such inputs: a pass
  // that tracks the largest exponent argument of every row, then a pass with every
  // reference at the true row maximum (all exponents <= 0, so l <= the key count).
  auto passes = [&](auto NAc) {
    constexpr int NA = decltype(NAc)::value;
    if (n_all == 0) return;
    for (int pass = 0; pass < 3; ++pass) {
      // pass 0: first-tile references; 1 (redo only): max tracking; 2: true maxima
      if (pass == 1) one_pass(NAc, IntC<1>{}, false);
      else one_pass(NAc, IntC<0>{}, pass == 0);
      if (pass == 1) {
#pragma unroll
        for (int j = 0; j < NA; ++j) m[j] += fmaxf(row_max(mxs[j]), 0.f);
        __syncthreads();
        continue;
      }
      if (pass == 2) break;
      bool bad = false;
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        float lt = l[j];
        lt += __shfl_xor(lt, 16, 64);
        lt += __shfl_xor(lt, 32, 64);
        bad |= !(lt < kMaxRowSum);
      }
      if (__any(bad)) redo_vote = 1;
      __syncthreads();  // the vote, and every wave done with the last pass's stages
      if (redo_vote == 0) break;
    }
  };
  int na = 0;  // wave-uniform: the valid tiles are a prefix of tile[]
#pragma unroll
  for (int j = 0; j < NT; ++j) na += tile[j] < ntiles;
  dispatch_count<NT>(na, passes);

  // every wave reaches this point with no copy in flight (the last sync waited for all)

  // results: with one split the normalised output directly, else (lse, O/l) partials
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    float lt = l[j];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const int r = tile[j] * 16 + l16;
    if (tile[j] >= ntiles || r >= R || (grp == 1 && tile[j] == tdup)) continue;
    const float lse = lt > 0.f ? m[j] + log2f(lt) : -INFINITY;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (nsplit == 1) {
      const int trow = r / G, hl = r % G;
      uint16_t* op = out + (((size_t)s * Tn + trow) * Hq + kvh * G + hl) * D;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const f32x4 o = O[j][b] * inv;
        const uint32_t lo = (uint32_t)f32_to_bf16(o[0]) | ((uint32_t)f32_to_bf16(o[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(o[2]) | ((uint32_t)f32_to_bf16(o[3]) << 16);
        *reinterpret_cast<uint2*>(&op[16 * b + 4 * q4]) = make_uint2(lo, hi);
      }
    } else {
      const size_t base = ((size_t)(s * Hkv + kvh) * nsplit + split) * R + r;
      if (q4 == 0) part_lse[base] = lse;
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const f32x4 o = O[j][b] * inv;
        *reinterpret_cast<float4*>(&part_o[base * D + 16 * b + 4 * q4]) = make_float4(o[0], o[1], o[2], o[3]);
      }
    }
  }
}

// Merge of the split partials: one lane per 4 output columns of one (sequence, tree
// row, q head); parts are weighted by 2^(lse_p - max lse) and renormalised.  The loads
// do not wait on one another: the parts' lse values first (eight in flight per lane),
// then every part's O row unconditionally (a split that saw no key wrote lse -inf and
// O = 0, so its weight is 0), eight at a time.
template <int D>
__global__ void __launch_bounds__(D / 4) attn_combine_kernel(const float* __restrict__ part_lse,
                                                             const float* __restrict__ part_o, int Tn, int Hq,
                                                             int Hkv, int nparts, uint16_t* __restrict__ out) {
  constexpr int U = 8;
  const int hq = blockIdx.x % Hq;
  const int t = (blockIdx.x / Hq) % Tn;
  const int s = blockIdx.x / (Hq * Tn);
  const int G = Hq / Hkv, R = Tn * G;
  const int d4 = threadIdx.x;
  const size_t base = (size_t)(s * Hkv + hq / G) * nparts * R + t * G + hq % G;
  float M = -INFINITY;
  for (int p0 = 0; p0 < nparts; p0 += U) {
    float ls[U];
#pragma unroll
    for (int u = 0; u < U; ++u) ls[u] = part_lse[base + (size_t)min(p0 + u, nparts - 1) * R];
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, ls[u]);  // a clamped index repeats a part: same max
  }
  float wsum = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = 0; p0 < nparts; p0 += U) {
    float ls[U];
    float4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t pb = base + (size_t)min(p0 + u, nparts - 1) * R;
      ls[u] = part_lse[pb];
      o[u] = *reinterpret_cast<const float4*>(&part_o[pb * D + 4 * d4]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {  // weight 0 (adds exact zeros: the O rows are finite) past the parts
      const float w = (p0 + u < nparts && ls[u] != -INFINITY) ? exp2f(ls[u] - M) : 0.f;
      wsum += w;
      acc.x += w * o[u].x; acc.y += w * o[u].y; acc.z += w * o[u].z; acc.w += w * o[u].w;
    }
  }
  const float inv = 1.f / wsum;
  const uint32_t lo = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
  const uint32_t hi = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
  *reinterpret_cast<uint2*>(&out[(((size_t)s * Tn + t) * Hq + hq) * D + 4 * d4]) = make_uint2(lo, hi);
}

// Tiling of the bf16 path: NT 16-row tiles per wave, NW waves per block.  Q (DS*4
// registers per tile) and the fp32 O accumulators (DB*4 per tile) stay in registers.
#ifndef DDT_ATTN_NT256
#define DDT_ATTN_NT256 2
#endif
#ifndef DDT_ATTN_NW256
#define DDT_ATTN_NW256 8
#endif
#ifndef DDT_ATTN_NT128
#define DDT_ATTN_NT128 4
#endif
#ifndef DDT_ATTN_NW128
#define DDT_ATTN_NW128 8
#endif
#ifndef DDT_ATTN_PK
#define DDT_ATTN_PK 3  // K operand reads pinned ahead of their products (0: scheduler's order)
#endif
constexpr int attn_nt(int D) { return D == 256 ? DDT_ATTN_NT256 : DDT_ATTN_NT128; }
constexpr int attn_nw(int D) { return D == 256 ? DDT_ATTN_NW256 : DDT_ATTN_NW128; }

AttnPlan plan_tree_attn(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt) {
  AttnPlan p = {};
  const int T = B + 1;
  p.mfma = dt == DDT_BF16 && (D == 128 || D == 256);
  p.G = Hq / Hkv;
  p.R = T * p.G;
  p.ntiles = cdiv(p.R, 16);
  if (!p.mfma) return p;
  p.nwg = cdiv(p.ntiles, attn_nw(D) * attn_nt(D));
  // one block per CU: split the prefix so that the grid fills the 256 CUs once
  const int rowblocks = n * Hkv * p.nwg;
  int ns = 256 / rowblocks;
  const int ns_max = Pmax / kAttnMinSplit > 1 ? Pmax / kAttnMinSplit : 1;
  ns = ns < 1 ? 1 : (ns > ns_max ? ns_max : ns);
  int len = cdiv(Pmax > 0 ? Pmax : 1, ns);
  len = cdiv(len, kAttnNK) * kAttnNK;
  p.split_len = len;
  p.nsplit = cdiv(Pmax > 0 ? Pmax : 1, len);
  p.units = n * Hkv * p.nsplit;
  p.grid = cdiv(p.units, 8) * 8 * p.nwg;
  if (p.nsplit == 1) return p;  // the kernel writes the output directly
  const size_t rows = (size_t)n * Hkv * p.nsplit * p.R;
  p.off_lse = 0;
  p.off_o = (rows * sizeof(float) + 255) / 256 * 256;
  p.total = p.off_o + rows * D * sizeof(float);
  return p;
}

hipError_t launch_tree_attn(const void* q, const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                            const void* k_tree, const void* v_tree, const uint64_t* anc, int n, int T, int Hq,
                            int Hkv, int D, int Pmax, float scale, int dt, void* out, const AttnPlan& plan,
                            void* ws, hipStream_t st, const PagedKV& pg) {
  const bool paged = pg.bt != nullptr;
  if (!plan.mfma) {
    const dim3 grid(n * T * Hq);
#define DDT_SCALAR1(TY, DD, PG)                                                                              \
  hipLaunchKernelGGL((attn_scalar_kernel<TY, DD, PG>), grid, dim3(64), 0, st, static_cast<const TY*>(q),      \
                     static_cast<const TY*>(k_cache), static_cast<const TY*>(v_cache), prefix_len,           \
                     static_cast<const TY*>(k_tree), static_cast<const TY*>(v_tree), anc, T, Hq, Hkv, Pmax,  \
                     scale, pg, static_cast<TY*>(out))
#define DDT_SCALAR(TY, DD)            \
  do {                                \
    if (paged) DDT_SCALAR1(TY, DD, true);  \
    else DDT_SCALAR1(TY, DD, false);       \
  } while (0)
    if (dt == DDT_F32) {
      if (D == 64) DDT_SCALAR(float, 64);
      else if (D == 128) DDT_SCALAR(float, 128);
      else DDT_SCALAR(float, 256);
    } else {
      DDT_SCALAR(uint16_t, 64);
    }
#undef DDT_SCALAR
#undef DDT_SCALAR1
    return hipGetLastError();
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* part_lse = plan.total ? reinterpret_cast<float*>(w + plan.off_lse) : nullptr;
  float* part_o = plan.total ? reinterpret_cast<float*>(w + plan.off_o) : nullptr;
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid(plan.grid);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  const auto* kt = static_cast<const uint16_t*>(k_tree);
  const auto* vt = static_cast<const uint16_t*>(v_tree);
  auto* o16 = static_cast<uint16_t*>(out);
#define DDT_MFMA(DD, PG)                                                                                     \
  hipLaunchKernelGGL((attn_mfma_kernel<DD, attn_nt(DD), attn_nw(DD), DDT_ATTN_PK, PG>), grid,      \
                     dim3(64 * attn_nw(DD)), 0, st, qq, kc, vc, prefix_len, kt, vt, anc, T, Hq, Hkv, Pmax, sl2, \
                     plan.nwg, plan.nsplit, plan.split_len, plan.units, pg, part_lse, part_o, o16)
  if (D == 256) {
    if (paged) DDT_MFMA(256, true);
    else DDT_MFMA(256, false);
    if (plan.nsplit > 1)
      hipLaunchKernelGGL((attn_combine_kernel<256>), dim3(n * T * Hq), dim3(64), 0, st, part_lse, part_o, T, Hq, Hkv,
                         plan.nsplit, o16);
  } else {
    if (paged) DDT_MFMA(128, true);
    else DDT_MFMA(128, false);
    if (plan.nsplit > 1)
      hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(n * T * Hq), dim3(32), 0, st, part_lse, part_o, T, Hq, Hkv,
                         plan.nsplit, o16);
  }
#undef DDT_MFMA
  return hipGetLastError();
}

}  // namespace ddt
