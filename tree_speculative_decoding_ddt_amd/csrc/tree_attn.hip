// Tree-masked attention: every tree row attends to the committed prefix, the root,
// its ancestors and itself -- never to a sibling.
// Sources: "DDTree on vLLM: candid research notes", section "Why hybrid attention
// makes it hard" (prefix + own ancestors, never siblings); "From DDTree to drafter
// training", section "The Architecture of DDTree" (one verify pass over root + all
// nodes with an ancestor-only mask).
//
// bf16, D in {128, 256}: matrix-core path.
//   Rows of one kv head are the G = Hq/Hkv query heads of all T tree rows, flattened
//   r = t*G + h_local and cut into 16-row tiles; a wave owns up to NT tiles, a block
//   (4 waves) shares one 32-key K/V tile in LDS.  Per 32 keys:
//     S^T = K Q^T   v_mfma_f32_16x16x32_bf16, A = K rows from LDS, B = Q from VGPRs;
//                   each lane then holds 8 scores of ONE query row,
//     online softmax in the log2 domain (fp32),
//     O^T += V^T P^T  A = V^T from LDS, B = P straight from the score registers.
//   Keys are the MFMA contraction index of the second product, so their order is
//   free: V is written transposed into LDS with keys permuted so that the 8 keys a
//   lane holds are the 8 contiguous bf16 the A operand reads (one ds_read_b128).
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

constexpr int kAttnNK = 32;  // keys per iteration (bf16 path)
constexpr float kLazy = 8.f; // rescale threshold of the online softmax (log2 units)
#ifndef DDT_ATTN_STAGES
#define DDT_ATTN_STAGES 3
#endif
constexpr int kAttnStages = DDT_ATTN_STAGES; // LDS stages of K/V tiles (bf16 path)
#ifndef DDT_HOIST_K
#define DDT_HOIST_K 0           // read all K operands of a tile before its S^T products
#endif
#ifndef DDT_HOIST_V
#define DDT_HOIST_V 0           // V^T operand blocks read before the softmax
#endif

// ------------------------------------------------------------------ scalar path
template <typename T, int D>
__global__ void __launch_bounds__(64) attn_scalar_kernel(const T* __restrict__ q, const T* __restrict__ k_cache,
                                                         const T* __restrict__ v_cache,
                                                         const int32_t* __restrict__ prefix_len,
                                                         const T* __restrict__ k_tree, const T* __restrict__ v_tree,
                                                         const uint64_t* __restrict__ anc, int Tn, int Hq, int Hkv,
                                                         int Pmax, float scale, T* __restrict__ out) {
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

  auto block = [&](float sc, const T* vbase, int vrow0) {
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
        const size_t rb = (size_t)(vrow0 + u) * D;
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] += pu * Elem<T>::load(vbase, rb + lane + 64 * j);
      }
    }
    m = mn;
  };

  const int P = min(max(prefix_len[s], 0), Pmax);
  const T* kc = k_cache + (size_t)(s * Hkv + kvh) * Pmax * D;
  const T* vc = v_cache + (size_t)(s * Hkv + kvh) * Pmax * D;
  for (int k0 = 0; k0 < P; k0 += 64) {
    const int key = k0 + lane;
    float sc = -INFINITY;
    if (key < P) {
      float d0 = 0.f;
      for (int d = 0; d < D; ++d) d0 += qs[d] * Elem<T>::load(kc, (size_t)key * D + d);
      sc = d0;
    }
    block(sc, vc, k0);
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
    block(sc, vt, j0);
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int j = 0; j < DPL; ++j)
    Elem<T>::store(out, (((size_t)s * Tn + i) * Hq + h) * D + lane + 64 * j, acc[j] * inv);
}

// ------------------------------------------------------------------ bf16 matrix-core path
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// K and V tiles live in LDS row-major, one key per row of D bf16, with the 16-byte
// chunks of row `key` permuted by chunk ^ (key mod chunks-per-row): 16 consecutive
// keys then hit 16 different bank groups for both the row reads of K and the
// transposing reads of V.
template <int D>
__device__ __forceinline__ int swz_off(int key, int chunk) {
  constexpr int CH = D / 8;
  return key * (D * 2) + ((chunk ^ (key & (CH - 1))) << 4);
}

// One 16-byte lane-slice per lane per instruction, straight from global memory into
// LDS (no registers): instruction i of a tile covers LDS bytes [1024 i, 1024 i + 1024).
// Rows past `rows` are clamped to the last valid row (finite data, masked later).
template <int D, int NK>
__device__ __forceinline__ void load_tile_async(uint8_t* lds, const uint16_t* src, int row0, int rows, int wave,
                                                int lane) {
  constexpr int ROWB = D * 2, CH = D / 8, INSTR = NK * ROWB / 1024;
#pragma unroll
  for (int i = wave; i < INSTR; i += 4) {
    const int byte = i * 1024 + lane * 16;
    const int row = byte / ROWB;
    const int chunk = (byte % ROWB) >> 4;
    const int gchunk = chunk ^ (row & (CH - 1));
    const int grow = row0 + (row < rows ? row : rows - 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + (size_t)grow * D + gchunk * 8),
                                     reinterpret_cast<void*>(lds + i * 1024), 16, 0, 0);
  }
}

// s_waitcnt with vmcnt = n (0..63) and the other counters left unconstrained.
#define DDT_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))

template <int D, int NT>
__global__ void __launch_bounds__(256, 1) attn_mfma_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ k_cache,
                                                           const uint16_t* __restrict__ v_cache,
                                                           const int32_t* __restrict__ prefix_len,
                                                           const uint16_t* __restrict__ k_tree,
                                                           const uint16_t* __restrict__ v_tree,
                                                           const uint64_t* __restrict__ anc, int Tn, int Hq,
                                                           int Hkv, int Pmax, float scale_log2, int nwg,
                                                           int nsplit, int split_len, float* __restrict__ part_lse,
                                                           float* __restrict__ part_o, uint16_t* __restrict__ out) {
  constexpr int NK = kAttnNK;
  constexpr int NST = kAttnStages;              // LDS stages (tiles in flight = NST - 1)
  constexpr int TILE = NK * D * 2;              // bytes of one K or V tile
  constexpr int DS = D / 32;                    // contraction steps of S^T = K Q^T
  constexpr int DB = D / 16;                    // 16-wide blocks of d in O^T
  constexpr int DMA = 2 * (TILE / 1024) / 4;    // async load instructions per wave per tile
  __shared__ __align__(1024) uint8_t lds[NST][2][TILE];  // [stage][K, V]

  const int G = Hq / Hkv;
  const int R = Tn * G;
  const int ntiles = (R + 15) / 16;
  int bx = blockIdx.x;
  const int grp = bx % nwg;
  bx /= nwg;
  const int kvh = bx % Hkv;
  const int s = bx / Hkv;
  const int split = blockIdx.y;
  const bool last = split == nsplit - 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;

  // key tiles: this split's slice of the prefix, then (last split) the tree rows
  const int P = min(max(prefix_len[s], 0), Pmax);
  const int k_beg = min(split * split_len, P);
  const int k_end = min(P, k_beg + split_len);
  const int n_pre = (k_end - k_beg + NK - 1) / NK;
  const int n_all = n_pre + (last ? (Tn + NK - 1) / NK : 0);
  const uint16_t* Kp = k_cache + (size_t)(s * Hkv + kvh) * Pmax * D;
  const uint16_t* Vp = v_cache + (size_t)(s * Hkv + kvh) * Pmax * D;
  const uint16_t* Kt = k_tree + (size_t)(s * Hkv + kvh) * Tn * D;
  const uint16_t* Vt = v_tree + (size_t)(s * Hkv + kvh) * Tn * D;
  auto issue = [&](int it) {
    const int stage = it % NST;
    if (it < n_pre) {
      const int r0 = k_beg + it * NK;
      load_tile_async<D, NK>(lds[stage][0], Kp, r0, k_end - r0, wave, lane);
      load_tile_async<D, NK>(lds[stage][1], Vp, r0, k_end - r0, wave, lane);
    } else {
      const int r0 = (it - n_pre) * NK;
      load_tile_async<D, NK>(lds[stage][0], Kt, r0, Tn - r0, wave, lane);
      load_tile_async<D, NK>(lds[stage][1], Vt, r0, Tn - r0, wave, lane);
    }
  };

  // this wave's tiles and Q fragments (B operand of S^T: row l16, d = 32*st + 8*q4 .. +7)
  int tile[NT];
  bf16x8 Qf[NT][DS];
  uint64_t arow[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    tile[j] = grp + nwg * (wave + 4 * j);
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
    arow[j] = (ok && last) ? anc[(size_t)s * Tn + trow] : 0ull;
  }
  __builtin_amdgcn_s_waitcnt(0);  // Q in registers before the DMA counting starts
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (i < n_all) issue(i);

  f32x4 O[NT][DB];
  float m[NT], l[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) O[j][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // per-lane LDS offsets of the operands (the swizzle depends on the key row only)
  int koff[2][DS];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int st = 0; st < DS; ++st) koff[b][st] = swz_off<D>(16 * b + l16, 4 * st + q4);
  const int vkey = 4 * q4 + (l16 >> 2);
  const int vintra = (l16 & 1) * 8;

  for (int it = 0; it < n_all; ++it) {
    // wait for tile `it` (later tiles may still be in flight), then make it visible
    const int ahead = n_all - 1 - it;
    if (ahead >= NST - 2) DDT_WAIT_VMCNT((NST - 2) * DMA);
    else if (ahead == 1) DDT_WAIT_VMCNT(DMA);
    else DDT_WAIT_VMCNT(0);
    __syncthreads();
    if (it + NST - 1 < n_all) issue(it + NST - 1);  // refills the stage read in iteration it-1
    const uint8_t* Ks = lds[it % NST][0];
    const uint8_t* Vs = lds[it % NST][1];
    const bool tree = it >= n_pre;
    const int kb = tree ? (it - n_pre) * NK : k_beg + it * NK;
    const int kend = tree ? Tn : k_end;
    const bool full = !tree && kb + NK <= kend;

    // S^T blocks: keys 16b + 4*q4 + e of row l16
    f32x4 Sacc[NT][2];
#pragma unroll
    for (int j = 0; j < NT; ++j) Sacc[j][0] = Sacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#if DDT_HOIST_K
    bf16x8 Ka[2][DS];
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int b = 0; b < 2; ++b) Ka[b][st] = *reinterpret_cast<const bf16x8*>(Ks + koff[b][st]);
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int j = 0; j < NT; ++j)
          Sacc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Ka[b][st], Qf[j][st], Sacc[j][b], 0, 0, 0);
#else
#pragma unroll
    for (int st = 0; st < DS; ++st)
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(Ks + koff[b][st]);
#pragma unroll
        for (int j = 0; j < NT; ++j)
          Sacc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Qf[j][st], Sacc[j][b], 0, 0, 0);
      }
#endif

    // V^T operands (d = 16*b + l16, keys 4*q4 + 0..3 and 16 + 4*q4 + 0..3), read now so
    // that their latency overlaps the softmax
    s16x4 Vlo[DB], Vhi[DB];
#pragma unroll
    for (int b = 0; b < DDT_HOIST_V; ++b) {
      const int chunk = 2 * b + ((l16 & 3) >> 1);
      Vlo[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + swz_off<D>(vkey, chunk) + vintra));
      Vhi[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + swz_off<D>(vkey + 16, chunk) + vintra));
    }

    bf16x8 Pb[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float sv[8];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[4 * b + e] = Sacc[j][b][e] * scale_log2;
      if (!full) {  // tail of the prefix, or the tree under its ancestor mask
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = kb + 16 * b + 4 * q4 + e;
            bool vis = key < kend;
            if (tree) vis = vis && (key == 0 || ((arow[j] >> (key - 1)) & 1ull));
            if (!vis) sv[4 * b + e] = -INFINITY;
          }
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      // Lazy rescaling: the running reference m only moves when a row's max exceeds it
      // by more than kLazy (log2 units), so P <= 2^kLazy and O, l are rescaled rarely.
      if (__any(mx > m[j] + kLazy)) {
        const float mn = fmaxf(m[j], mx);
        const float alpha = (m[j] == -INFINITY) ? (mn == -INFINITY ? 1.f : 0.f) : exp2f(m[j] - mn);
        l[j] *= alpha;
        m[j] = mn;
#pragma unroll
        for (int b = 0; b < DB; ++b) O[j][b] *= alpha;
      }
      const float mref = m[j] == -INFINITY ? 0.f : m[j];
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2f(sv[e] - mref);  // exp2(-inf) = 0 for masked keys
        sv[e] = p;
        rs += p;
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l[j] += rs;
#pragma unroll
      for (int e = 0; e < 8; ++e) Pb[j][e] = static_cast<__bf16>(sv[e]);
    }

    // O^T += V^T P^T
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      if (b >= DDT_HOIST_V) {
        const int chunk = 2 * b + ((l16 & 3) >> 1);
        Vlo[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + swz_off<D>(vkey, chunk) + vintra));
        Vhi[b] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Vs + swz_off<D>(vkey + 16, chunk) + vintra));
      }
      // whole-vector join: the keys 4*q4+0..3 then 16+4*q4+0..3 of column d
      const bf16x8 A = __builtin_bit_cast(bf16x8, __builtin_shufflevector(Vlo[b], Vhi[b], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int j = 0; j < NT; ++j) O[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Pb[j], O[j][b], 0, 0, 0);
    }
  }

  // results: with one split the normalised output directly, else (lse, O/l) partials
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = tile[j] * 16 + l16;
    if (tile[j] >= ntiles || r >= R) continue;
    const float lse = l[j] > 0.f ? m[j] + log2f(l[j]) : -INFINITY;
    const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
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

template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(const float* __restrict__ part_lse,
                                                           const float* __restrict__ part_o, int Tn, int Hq,
                                                           int Hkv, int nparts, uint16_t* __restrict__ out) {
  const int s = blockIdx.x / Tn, t = blockIdx.x % Tn;
  const int G = Hq / Hkv, R = Tn * G;
  for (int idx = threadIdx.x; idx < Hq * (D / 4); idx += blockDim.x) {
    const int hq = idx / (D / 4), d4 = idx % (D / 4);
    const int kvh = hq / G, r = t * G + hq % G;
    const size_t base = (size_t)(s * Hkv + kvh) * nparts * R + r;
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, part_lse[base + (size_t)p * R]);
    float wsum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = 0; p < nparts; ++p) {
      const float ls = part_lse[base + (size_t)p * R];
      if (ls == -INFINITY) continue;
      const float w = exp2f(ls - M);
      const float4 o = *reinterpret_cast<const float4*>(&part_o[(base + (size_t)p * R) * D + 4 * d4]);
      wsum += w;
      acc.x += w * o.x; acc.y += w * o.y; acc.z += w * o.z; acc.w += w * o.w;
    }
    const float inv = 1.f / wsum;
    const uint32_t lo = (uint32_t)f32_to_bf16(acc.x * inv) | ((uint32_t)f32_to_bf16(acc.y * inv) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(acc.z * inv) | ((uint32_t)f32_to_bf16(acc.w * inv) << 16);
    *reinterpret_cast<uint2*>(&out[(((size_t)s * Tn + t) * Hq + hq) * D + 4 * d4]) = make_uint2(lo, hi);
  }
}

// 16-row tiles per wave: Q (2 VGPR/row at D=256) and O (4 AGPR/row) stay in registers.
constexpr int attn_nt(int D) { return D == 256 ? 2 : 3; }

AttnPlan plan_tree_attn(int n, int B, int Hq, int Hkv, int D, int Pmax, int dt) {
  AttnPlan p = {};
  const int T = B + 1;
  p.mfma = dt == DDT_BF16 && (D == 128 || D == 256);
  p.G = Hq / Hkv;
  p.R = T * p.G;
  p.ntiles = cdiv(p.R, 16);
  if (!p.mfma) return p;
  p.nwg = cdiv(p.ntiles, 4 * attn_nt(D));
  // one block per CU: split the prefix so that the grid fills the 256 CUs once
  const int units = n * Hkv * p.nwg;
  int ns = 256 / units;
  const int ns_max = Pmax / 256 > 1 ? Pmax / 256 : 1;
  ns = ns < 1 ? 1 : (ns > ns_max ? ns_max : ns);
  int len = cdiv(Pmax > 0 ? Pmax : 1, ns);
  len = cdiv(len, kAttnNK) * kAttnNK;
  p.split_len = len;
  p.nsplit = cdiv(Pmax > 0 ? Pmax : 1, len);
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
                            void* ws, hipStream_t st) {
  if (!plan.mfma) {
    const dim3 grid(n * T * Hq);
#define DDT_SCALAR(TY, DD)                                                                                   \
  hipLaunchKernelGGL((attn_scalar_kernel<TY, DD>), grid, dim3(64), 0, st, static_cast<const TY*>(q),          \
                     static_cast<const TY*>(k_cache), static_cast<const TY*>(v_cache), prefix_len,           \
                     static_cast<const TY*>(k_tree), static_cast<const TY*>(v_tree), anc, T, Hq, Hkv, Pmax,  \
                     scale, static_cast<TY*>(out))
    if (dt == DDT_F32) {
      if (D == 64) DDT_SCALAR(float, 64);
      else if (D == 128) DDT_SCALAR(float, 128);
      else DDT_SCALAR(float, 256);
    } else {
      DDT_SCALAR(uint16_t, 64);
    }
#undef DDT_SCALAR
    return hipGetLastError();
  }
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* part_lse = plan.total ? reinterpret_cast<float*>(w + plan.off_lse) : nullptr;
  float* part_o = plan.total ? reinterpret_cast<float*>(w + plan.off_o) : nullptr;
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid(n * Hkv * plan.nwg, plan.nsplit);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  const auto* kt = static_cast<const uint16_t*>(k_tree);
  const auto* vt = static_cast<const uint16_t*>(v_tree);
  auto* o16 = static_cast<uint16_t*>(out);
  if (D == 256) {
    hipLaunchKernelGGL((attn_mfma_kernel<256, attn_nt(256)>), grid, dim3(256), 0, st, qq, kc, vc, prefix_len, kt, vt,
                       anc, T, Hq, Hkv, Pmax, sl2, plan.nwg, plan.nsplit, plan.split_len, part_lse, part_o, o16);
    if (plan.nsplit > 1)
      hipLaunchKernelGGL((attn_combine_kernel<256>), dim3(n * T), dim3(256), 0, st, part_lse, part_o, T, Hq, Hkv,
                         plan.nsplit, o16);
  } else {
    hipLaunchKernelGGL((attn_mfma_kernel<128, attn_nt(128)>), grid, dim3(256), 0, st, qq, kc, vc, prefix_len, kt, vt,
                       anc, T, Hq, Hkv, Pmax, sl2, plan.nwg, plan.nsplit, plan.split_len, part_lse, part_o, o16);
    if (plan.nsplit > 1)
      hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(n * T), dim3(256), 0, st, part_lse, part_o, T, Hq, Hkv,
                         plan.nsplit, o16);
  }
  return hipGetLastError();
}

}  // namespace ddt
