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
                                                           float* __restrict__ part_o) {
  constexpr int NK = kAttnNK;
  constexpr int KPAD = D + 8;    // K tile row stride (bf16): keeps 16 consecutive rows on distinct banks
  constexpr int VPAD = NK + 8;   // V^T row stride (bf16)
  constexpr int DS = D / 32;     // contraction steps of S^T = K Q^T
  constexpr int DB = D / 16;     // 16-wide blocks of d in O^T
  __shared__ __align__(16) uint16_t Ks[NK * KPAD];
  __shared__ __align__(16) uint16_t Vt[D * VPAD];

  const int G = Hq / Hkv;
  const int R = Tn * G;
  const int ntiles = (R + 15) / 16;
  int bx = blockIdx.x;
  const int grp = bx % nwg;
  bx /= nwg;
  const int kvh = bx % Hkv;
  const int s = bx / Hkv;
  const int split = blockIdx.y;
  const bool is_tree = split == nsplit;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, q4 = lane >> 4;

  int k_beg, k_end;
  const uint16_t *Kb, *Vb;
  if (is_tree) {
    k_beg = 0;
    k_end = Tn;
    Kb = k_tree + (size_t)(s * Hkv + kvh) * Tn * D;
    Vb = v_tree + (size_t)(s * Hkv + kvh) * Tn * D;
  } else {
    const int P = min(max(prefix_len[s], 0), Pmax);
    k_beg = split * split_len;
    k_end = min(P, k_beg + split_len);
    Kb = k_cache + (size_t)(s * Hkv + kvh) * Pmax * D;
    Vb = v_cache + (size_t)(s * Hkv + kvh) * Pmax * D;
  }

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
    arow[j] = (ok && is_tree) ? anc[(size_t)s * Tn + trow] : 0ull;
  }

  f32x4 O[NT][DB];
  float m[NT], l[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int b = 0; b < DB; ++b) O[j][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int kb = k_beg; kb < k_end; kb += NK) {
    // K tile: rows kb..kb+NK-1 as-is
    for (int v = tid; v < NK * (D / 8); v += 256) {
      const int key = v / (D / 8), dc = (v % (D / 8)) * 8;
      const int kk = kb + key;
      const uint4 w = kk < k_end ? *reinterpret_cast<const uint4*>(Kb + (size_t)kk * D + dc) : make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(&Ks[key * KPAD + dc]) = w;
    }
    // V tile transposed: Vt[d][pos(key)], keys 4g..4g+3 -> positions 8g.. (g<4) or 8(g-4)+4.. (g>=4)
    for (int v = tid; v < (NK / 4) * (D / 8); v += 256) {
      const int kg = v / (D / 8), dc = (v % (D / 8)) * 8;
      uint32_t w[4][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kk = kb + 4 * kg + i;
        const uint4 x = kk < k_end ? *reinterpret_cast<const uint4*>(Vb + (size_t)kk * D + dc) : make_uint4(0, 0, 0, 0);
        w[i][0] = x.x; w[i][1] = x.y; w[i][2] = x.z; w[i][3] = x.w;
      }
      const int pos = kg < 4 ? 8 * kg : 8 * (kg - 4) + 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t a0 = (w[0][e >> 1] >> sh) & 0xffffu, a1 = (w[1][e >> 1] >> sh) & 0xffffu;
        const uint32_t a2 = (w[2][e >> 1] >> sh) & 0xffffu, a3 = (w[3][e >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<uint2*>(&Vt[(dc + e) * VPAD + pos]) = make_uint2(a0 | (a1 << 16), a2 | (a3 << 16));
      }
    }
    __syncthreads();

    // S^T blocks: keys 16b + 4*q4 + e of row l16
    f32x4 Sacc[NT][2];
#pragma unroll
    for (int j = 0; j < NT; ++j) Sacc[j][0] = Sacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < DS; ++st) {
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 A = *reinterpret_cast<const bf16x8*>(&Ks[(16 * b + l16) * KPAD + 32 * st + 8 * q4]);
#pragma unroll
        for (int j = 0; j < NT; ++j) Sacc[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Qf[j][st], Sacc[j][b], 0, 0, 0);
      }
    }

    bf16x8 Pb[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = kb + 16 * b + 4 * q4 + e;
          bool vis = key < k_end;
          if (is_tree) vis = vis && (key == 0 || ((arow[j] >> (key - 1)) & 1ull));
          const float x = vis ? Sacc[j][b][e] * scale_log2 : -INFINITY;
          sv[4 * b + e] = x;
          mx = fmaxf(mx, x);
        }
      }
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
      const float mref = m[j];
      float rs = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = (sv[e] == -INFINITY) ? 0.f : exp2f(sv[e] - mref);
        sv[e] = p;
        rs += p;
      }
      rs += __shfl_xor(rs, 16, 64);
      rs += __shfl_xor(rs, 32, 64);
      l[j] += rs;
#pragma unroll
      for (int e = 0; e < 8; ++e) Pb[j][e] = static_cast<__bf16>(sv[e]);
    }

#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const bf16x8 A = *reinterpret_cast<const bf16x8*>(&Vt[(16 * b + l16) * VPAD + 8 * q4]);
#pragma unroll
      for (int j = 0; j < NT; ++j) O[j][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Pb[j], O[j][b], 0, 0, 0);
    }
    __syncthreads();
  }

  // partial results: lse (log2 domain) and O / l per row
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int r = tile[j] * 16 + l16;
    if (tile[j] >= ntiles || r >= R) continue;
    const size_t base = ((size_t)(s * Hkv + kvh) * (nsplit + 1) + split) * R + r;
    const float lse = l[j] > 0.f ? m[j] + log2f(l[j]) : -INFINITY;
    const float inv = l[j] > 0.f ? 1.f / l[j] : 0.f;
    if (q4 == 0) part_lse[base] = lse;
#pragma unroll
    for (int b = 0; b < DB; ++b) {
      const f32x4 o = O[j][b] * inv;
      *reinterpret_cast<float4*>(&part_o[base * D + 16 * b + 4 * q4]) = make_float4(o[0], o[1], o[2], o[3]);
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

// 16-row tiles per wave: Q (2 VGPR/row at D=256) and O (4 AGPR/row) must stay in registers.
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
  const int units = n * Hkv * p.nwg;
  int ns = cdiv(256, units);
  const int ns_max = Pmax / 512 > 1 ? Pmax / 512 : 1;
  ns = ns < 1 ? 1 : (ns > ns_max ? ns_max : ns);
  int len = cdiv(Pmax > 0 ? Pmax : 1, ns);
  len = cdiv(len, kAttnNK) * kAttnNK;
  p.split_len = len;
  p.nsplit = cdiv(Pmax > 0 ? Pmax : 1, len);
  const size_t rows = (size_t)n * Hkv * (p.nsplit + 1) * p.R;
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
  float* part_lse = reinterpret_cast<float*>(w + plan.off_lse);
  float* part_o = reinterpret_cast<float*>(w + plan.off_o);
  const float sl2 = scale * 1.4426950408889634f;
  const dim3 grid(n * Hkv * plan.nwg, plan.nsplit + 1);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* kc = static_cast<const uint16_t*>(k_cache);
  const auto* vc = static_cast<const uint16_t*>(v_cache);
  const auto* kt = static_cast<const uint16_t*>(k_tree);
  const auto* vt = static_cast<const uint16_t*>(v_tree);
  if (D == 256) {
    hipLaunchKernelGGL((attn_mfma_kernel<256, attn_nt(256)>), grid, dim3(256), 0, st, qq, kc, vc, prefix_len, kt, vt,
                       anc, T, Hq, Hkv, Pmax, sl2, plan.nwg, plan.nsplit, plan.split_len, part_lse, part_o);
    hipLaunchKernelGGL((attn_combine_kernel<256>), dim3(n * T), dim3(256), 0, st, part_lse, part_o, T, Hq, Hkv,
                       plan.nsplit + 1, static_cast<uint16_t*>(out));
  } else {
    hipLaunchKernelGGL((attn_mfma_kernel<128, attn_nt(128)>), grid, dim3(256), 0, st, qq, kc, vc, prefix_len, kt, vt,
                       anc, T, Hq, Hkv, Pmax, sl2, plan.nwg, plan.nsplit, plan.split_len, part_lse, part_o);
    hipLaunchKernelGGL((attn_combine_kernel<128>), dim3(n * T), dim3(256), 0, st, part_lse, part_o, T, Hq, Hkv,
                       plan.nsplit + 1, static_cast<uint16_t*>(out));
  }
  return hipGetLastError();
}

}  // namespace ddt
