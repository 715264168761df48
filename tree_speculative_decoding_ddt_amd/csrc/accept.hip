// Target argmax (or a Gumbel-max draw) + tree walk.
// Source: "From DDTree to drafter training", section "The Architecture of DDTree":
// after the verify pass, walk down from the root while the target's token at the
// current node matches a child; "DDTree on vLLM: candid research notes", section
// "What broke along the way": the bonus token is emitted but kept apart from the
// accepted draft nodes.
//
// Phase 1 (HBM-bound): every (row, chunk) block scans a slice of one target row and
// leaves the slice's best (value desc, token id asc) as one 64-bit key
//   key = float_key(value) << 32 | (0xffffffff - id)
// in the workspace; integer max over keys is exact, so the result does not depend on
// the reduction order.  Phase 2: one wavefront per sequence reduces the chunk keys
// of its T rows and walks the tree (sibling tokens are distinct, so at most one
// child can match; two matches mark the tree malformed).
#include "common.h"
#include "launch.h"

namespace ddt {

// Sampled walk: the Gumbel-max key z * (1/t) + G with each operation rounded once
// (no fused multiply-add), as IEEE float32 arithmetic written out does it.
__device__ __forceinline__ float gumbel_key(float z, float inv, float g) {
#pragma clang fp contract(off)
  const float a = z * inv;
  return a + g;
}

// SAMPLED: the key of element v is z_v * (1/t) + G_v (t = temperature of the row's
// sequence; t <= 0 keeps z_v, the greedy argmax).
template <typename T, int VEC, bool SAMPLED>
__global__ void __launch_bounds__(256) argmax_partial_kernel(const T* __restrict__ logits, int V, int chunk,
                                                             const float* __restrict__ gumbel,
                                                             const float* __restrict__ temperature, int T_rows,
                                                             uint64_t* __restrict__ part) {
  const int row = blockIdx.x, c = blockIdx.y, S = gridDim.y;
  const int beg = c * chunk;
  const int end = min(V, beg + chunk);
  const T* p = logits + (size_t)row * V;
  const float* gp = SAMPLED ? gumbel + (size_t)row * V : nullptr;
  bool sample = false;
  float inv = 1.f;
  if constexpr (SAMPLED) {
    const float t = temperature[row / T_rows];
    sample = t > 0.f;
    inv = sample ? 1.0f / t : 1.f;  // IEEE division (correctly rounded)
  }
  uint64_t best = 0;
  auto consider = [&](float v, float g, int id) {
    if constexpr (SAMPLED) v = sample ? gumbel_key(v, inv, g) : v;
    const uint64_t k = (static_cast<uint64_t>(float_key(v)) << 32) | (0xffffffffu - (uint32_t)id);
    best = k > best ? k : best;
  };
  if constexpr (VEC > 1) {
    // beg and V are multiples of VEC elements: 16-byte loads
    const int nvec = (end - beg) / VEC;
    for (int i = threadIdx.x; i < nvec; i += blockDim.x) {
      const int e0 = beg + i * VEC;
      const uint4 w = *reinterpret_cast<const uint4*>(p + e0);
      float g[VEC];
      if constexpr (SAMPLED) {
#pragma unroll
        for (int j = 0; j < VEC / 4; ++j) {
          const float4 q = reinterpret_cast<const float4*>(gp + e0)[j];
          g[4 * j] = q.x; g[4 * j + 1] = q.y; g[4 * j + 2] = q.z; g[4 * j + 3] = q.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < VEC; ++j) g[j] = 0.f;
      }
      if constexpr (sizeof(T) == 2) {
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          consider(bf16_to_f32(u[j] & 0xffffu), g[2 * j], e0 + 2 * j);
          consider(bf16_to_f32(u[j] >> 16), g[2 * j + 1], e0 + 2 * j + 1);
        }
      } else {
        consider(__uint_as_float(w.x), g[0], e0);
        consider(__uint_as_float(w.y), g[1], e0 + 1);
        consider(__uint_as_float(w.z), g[2], e0 + 2);
        consider(__uint_as_float(w.w), g[3], e0 + 3);
      }
    }
  } else {
    for (int i = beg + threadIdx.x; i < end; i += blockDim.x)
      consider(Elem<T>::load(p, i), SAMPLED ? gp[i] : 0.f, i);
  }
  best = wave_max_u64(best);
  __shared__ uint64_t red[4];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) red[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t b = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) b = red[w] > b ? red[w] : b;
    part[(size_t)row * S + c] = b;
  }
}

// One wavefront per sequence; T <= 65 rows, two per lane.
__global__ void __launch_bounds__(64) walk_kernel(const uint64_t* __restrict__ part, int S,
                                                  const int32_t* __restrict__ tok,
                                                  const int32_t* __restrict__ parent, int T, int L,
                                                  int32_t* __restrict__ acc_rows, int32_t* __restrict__ acc_len,
                                                  int32_t* __restrict__ bonus) {
  const int s = blockIdx.x, lane = threadIdx.x;
  __shared__ int32_t targ[128];
  int my_tok[2], my_par[2], my_row[2];
  bool bad = false;
  for (int j = 0; j < 2; ++j) {
    const int r = lane + 64 * j;
    my_row[j] = r;
    my_tok[j] = -1;
    my_par[j] = -1;
    if (r < T) {
      uint64_t b = 0;
      for (int c = 0; c < S; ++c) {
        const uint64_t k = part[((size_t)s * T + r) * S + c];
        b = k > b ? k : b;
      }
      targ[r] = (int32_t)(0xffffffffu - (uint32_t)(b & 0xffffffffu));
      my_tok[j] = tok[(size_t)s * T + r];
      my_par[j] = parent[(size_t)s * T + r];
      if (r >= 1 && my_tok[j] >= 0 && (my_par[j] < 0 || my_par[j] >= r)) bad = true;
    }
  }
  __syncthreads();
  bad = __any(bad);
  int32_t* out = acc_rows + (size_t)s * (L + 1);
  for (int j = lane; j <= L; j += 64) out[j] = (j == 0) ? 0 : -1;
  int cur = 0, len = 0;
  while (!bad && len < L) {
    const int want = targ[cur];
    int hit = -1, nhit = 0;
    for (int j = 0; j < 2; ++j) {
      const bool m = my_row[j] >= 1 && my_row[j] < T && my_par[j] == cur && my_tok[j] == want;
      const uint64_t bal = __ballot(m);
      nhit += __popcll(bal);
      if (bal && hit < 0) hit = 64 * j + (int)__ffsll((unsigned long long)bal) - 1;
    }
    if (nhit == 0) break;
    if (nhit > 1) { bad = true; break; }
    cur = hit;
    ++len;
    if (lane == 0) out[len] = cur;
  }
  if (lane == 0) {
    acc_len[s] = bad ? -1 : len;
    bonus[s] = targ[cur];
  }
}

AcceptPlan plan_tree_accept(int n, int B, int V) {
  AcceptPlan p;
  const int rows = n * (B + 1);
  int S = cdiv(2048, rows);
  const int smax = V / 4096 > 1 ? V / 4096 : 1;
  S = S < 1 ? 1 : (S > smax ? smax : S);
  p.chunk = (cdiv(V, S) + 7) / 8 * 8;
  p.S = cdiv(V, p.chunk);
  p.total = (size_t)rows * p.S * sizeof(uint64_t);
  return p;
}

hipError_t launch_tree_accept(const void* logits, int dt, const int32_t* tok, const int32_t* parent,
                              int n, int T, int L, int V, int32_t* acc_rows, int32_t* acc_len,
                              int32_t* bonus, const AcceptPlan& plan, void* ws, hipStream_t st,
                              const float* gumbel, const float* temperature) {
  uint64_t* part = static_cast<uint64_t*>(ws);
  const dim3 grid(n * T, plan.S);
  const bool sampled = gumbel != nullptr;
  const bool aligned = (reinterpret_cast<uintptr_t>(logits) % 16) == 0 &&
                       (!sampled || (reinterpret_cast<uintptr_t>(gumbel) % 16) == 0);
#define DDT_ARGMAX(TY, VEC)                                                                                       \
  do {                                                                                                            \
    if (sampled)                                                                                                  \
      hipLaunchKernelGGL((argmax_partial_kernel<TY, VEC, true>), grid, dim3(256), 0, st, p, V, plan.chunk, gumbel, \
                         temperature, T, part);                                                                   \
    else                                                                                                          \
      hipLaunchKernelGGL((argmax_partial_kernel<TY, VEC, false>), grid, dim3(256), 0, st, p, V, plan.chunk,        \
                         nullptr, nullptr, T, part);                                                              \
  } while (0)
  if (dt == DDT_BF16) {
    const uint16_t* p = static_cast<const uint16_t*>(logits);
    if (aligned && V % 8 == 0) DDT_ARGMAX(uint16_t, 8);
    else DDT_ARGMAX(uint16_t, 1);
  } else {
    const float* p = static_cast<const float*>(logits);
    if (aligned && V % 4 == 0) DDT_ARGMAX(float, 4);
    else DDT_ARGMAX(float, 1);
  }
#undef DDT_ARGMAX
  hipLaunchKernelGGL(walk_kernel, dim3(n), dim3(64), 0, st, part, plan.S, tok, parent, T, L, acc_rows,
                     acc_len, bonus);
  return hipGetLastError();
}

}  // namespace ddt
