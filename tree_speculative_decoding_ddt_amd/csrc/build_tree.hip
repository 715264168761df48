// Draft-tree build: per-depth full-vocab log-softmax + exact top-K, then best-first
// expansion into a flattened tree.
// Source: "From DDTree to drafter training", section "The Architecture of DDTree":
// top-K ids and log-probs per drafter position, a max-heap seeded with the best
// depth-1 token, pop the best node, push its next-ranked sibling and its best child,
// stop at the budget; flatten to ids, per-depth positions and an ancestor-only mask.
// "DDTree on vLLM: candid research notes", section "What broke along the way": depth
// logits are not branch-conditioned, so a path's score is the sum of its log-probs.
//
// Kernels
//  1. topk_partial  grid (n*L rows, S chunks).  One HBM pass: each block holds its
//     chunk (<= 16384 logits) in registers as order-preserving integer keys, computes
//     the chunk's (max, sum exp) and selects its exact top-K by (value desc, id asc):
//     a lower bound from the K-th largest per-thread maximum filters the chunk, an
//     LDS radix select over the filtered keys finds the K-th value, and a second
//     radix select over chunk offsets resolves ties at that value.
//  2. topk_merge    grid (n*L).  Bitonic-sorts the S*K chunk candidates as 64-bit
//     (value, -id) keys, keeps the best K, combines the chunk (max, sum) pairs into
//     the row's log-sum-exp and writes lp = z - lse in fp32.
//  3. heap_expand   grid (n), one wavefront.  The frontier (<= B+1 entries) lives in
//     registers, two slots per lane; each pop is a wave-wide max over 64-bit keys
//     (score desc, token asc, parent row asc) -- exact integer comparisons, so the
//     pop order is deterministic.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

constexpr int kTopkThreads = 256;
constexpr int kEmax = 64;                              // keys per thread
constexpr int kChunkMax = kTopkThreads * kEmax;        // 16384 logits per block
constexpr int kSortMax = 2048;                         // merge capacity (S*K)

// --- block-wide digit search over a 256-bin LDS histogram (wave 0 only).
// Finds the bin where the running count (from the top bin down when `desc`, else from
// bin 0 up) first reaches `need`; returns bin, the count strictly before it, and its size.
__device__ __forceinline__ void find_digit(const uint32_t* hist, uint32_t need, bool desc, uint32_t* sel) {
  const int lane = threadIdx.x & 63;
  // lane l owns bins in scan order: positions 4l..4l+3
  uint32_t h[4], tot = 0;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int pos = 4 * lane + b;
    h[b] = hist[desc ? 255 - pos : pos];
    tot += h[b];
  }
  // inclusive prefix over lanes in scan order
  uint32_t inc = tot;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(inc, o, 64);
    if (lane >= o) inc += t;
  }
  const uint32_t before = inc - tot;
  if (before < need && need <= inc) {
    uint32_t acc = before;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      if (acc + h[b] >= need) {
        const int pos = 4 * lane + b;
        sel[0] = desc ? 255 - pos : pos;
        sel[1] = acc;
        sel[2] = h[b];
        break;
      }
      acc += h[b];
    }
  }
}

template <typename T, int KBITS>
__global__ void __launch_bounds__(kTopkThreads) topk_partial_kernel(const T* __restrict__ logits, int V, int chunk,
                                                                    int K, float* __restrict__ cval,
                                                                    int32_t* __restrict__ cid,
                                                                    float2* __restrict__ stat) {
  const int row = blockIdx.x, c = blockIdx.y, S = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int beg = c * chunk;
  const int cnt = min(chunk, V - beg);
  const int keff = min(K, cnt);
  const T* p = logits + (size_t)row * V + beg;

  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmaxs[kTopkThreads];
  __shared__ uint32_t sel[3];
  __shared__ uint32_t tau_s;
  __shared__ float2 red[kTopkThreads / 64];
  __shared__ int out_cnt;

  // 1. load the chunk as keys; online (max, sum exp)
  uint32_t key[kEmax];
  float m = -INFINITY, sum = 0.f;
  uint32_t tmax = 0;
#pragma unroll
  for (int j = 0; j < kEmax; ++j) {
    const int e = tid + kTopkThreads * j;
    uint32_t k = 0;
    if (e < cnt) {
      const float v = Elem<T>::load(p, e);
      k = float_key(v) >> (32 - KBITS);
      if (v > m) {
        sum = sum * __expf(m - v) + 1.f;
        m = v;
      } else if (v != -INFINITY) {
        sum += __expf(v - m);
      }
      tmax = k > tmax ? k : tmax;
    }
    key[j] = k;
  }
  // (max, sum) over the block
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(sum, o, 64);
    const float mm = fmaxf(m, m2);
    sum = (mm == -INFINITY) ? 0.f : sum * __expf(m - mm) + s2 * __expf(m2 - mm);
    m = mm;
  }
  if (lane == 0) red[wave] = make_float2(m, sum);
  tmaxs[tid] = tmax;
  __syncthreads();
  if (tid == 0) {
    float mm = red[0].x, ss = red[0].y;
    for (int w = 1; w < kTopkThreads / 64; ++w) {
      const float m2 = red[w].x, s2 = red[w].y;
      const float mx = fmaxf(mm, m2);
      ss = (mx == -INFINITY) ? 0.f : ss * __expf(mm - mx) + s2 * __expf(m2 - mx);
      mm = mx;
    }
    stat[(size_t)row * S + c] = make_float2(mm, ss);
  }

  // 2. lower bound: the keff-th largest per-thread maximum
  {
    uint32_t rank = 0;
    for (int u = 0; u < kTopkThreads; ++u) {
      const uint32_t o = tmaxs[u];
      rank += (o > tmax) || (o == tmax && u < tid);
    }
    if ((int)rank == keff - 1) tau_s = tmax;
  }
  __syncthreads();
  const uint32_t tau = tau_s;

  // 3. radix select of the keff-th largest key among keys >= tau
  uint32_t prefix = 0, pmask = 0, need = keff, count_eq = 0;
#pragma unroll
  for (int shift = KBITS - 8; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kEmax; ++j) {
      const uint32_t k = key[j];
      if (tid + kTopkThreads * j < cnt && k >= tau && (k & pmask) == prefix)
        atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) find_digit(hist, need, true, sel);
    __syncthreads();
    need -= sel[1];
    count_eq = sel[2];
    prefix |= sel[0] << shift;
    pmask |= 255u << shift;
  }
  const uint32_t kth = prefix;

  // 4. ties at the K-th value: keep the `need` lowest chunk offsets
  uint32_t off_th = 0xffffffffu;
  if (count_eq > need) {
    uint32_t pre2 = 0, msk2 = 0, need2 = need;
#pragma unroll
    for (int shift = 8; shift >= 0; shift -= 8) {
      __syncthreads();
      hist[tid] = 0;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kEmax; ++j) {
        const uint32_t e = tid + kTopkThreads * j;
        if ((int)e < cnt && key[j] == kth && (e & msk2) == pre2) atomicAdd(&hist[(e >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) find_digit(hist, need2, false, sel);
      __syncthreads();
      need2 -= sel[1];
      pre2 |= sel[0] << shift;
      msk2 |= 255u << shift;
    }
    off_th = pre2;
  }

  // 5. emit exactly keff candidates (unordered); pad to K with id -1
  if (tid == 0) out_cnt = 0;
  __syncthreads();
  const size_t base = ((size_t)row * S + c) * K;
#pragma unroll
  for (int j = 0; j < kEmax; ++j) {
    const uint32_t e = tid + kTopkThreads * j;
    const uint32_t k = key[j];
    if ((int)e < cnt && (k > kth || (k == kth && e <= off_th))) {
      const int pos = atomicAdd(&out_cnt, 1);
      if (pos < K) {
        cval[base + pos] = Elem<T>::load(p, e);
        cid[base + pos] = beg + (int)e;
      }
    }
  }
  if (tid >= keff && tid < K) cid[base + tid] = -1;
}

__global__ void __launch_bounds__(256) topk_merge_kernel(const float* __restrict__ cval,
                                                         const int32_t* __restrict__ cid,
                                                         const float2* __restrict__ stat, int S, int K,
                                                         int sortN, int32_t* __restrict__ top_id,
                                                         float* __restrict__ top_lp) {
  const int row = blockIdx.x, tid = threadIdx.x;
  __shared__ uint64_t sk[kSortMax];
  __shared__ float lse_s;
  const int N = S * K;
  for (int i = tid; i < sortN; i += blockDim.x) {
    uint64_t k = 0;
    if (i < N) {
      const int id = cid[(size_t)row * N + i];
      if (id >= 0)
        k = (static_cast<uint64_t>(float_key(cval[(size_t)row * N + i])) << 32) | (0xffffffffu - (uint32_t)id);
    }
    sk[i] = k;
  }
  if (tid == 0) {
    float M = -INFINITY;
    for (int c = 0; c < S; ++c) M = fmaxf(M, stat[(size_t)row * S + c].x);
    float tot = 0.f;
    for (int c = 0; c < S; ++c) {
      const float2 st = stat[(size_t)row * S + c];
      if (st.x != -INFINITY) tot += st.y * __expf(st.x - M);
    }
    lse_s = M + __logf(tot);
  }
  __syncthreads();
  // bitonic sort, descending
  for (int k = 2; k <= sortN; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < sortN; i += blockDim.x) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const uint64_t a = sk[i], b = sk[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            sk[i] = b;
            sk[ixj] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  const float lse = lse_s;
  for (int i = tid; i < K; i += blockDim.x) {
    const uint64_t k = sk[i];
    if (k != 0) {
      top_id[(size_t)row * K + i] = (int32_t)(0xffffffffu - (uint32_t)(k & 0xffffffffu));
      top_lp[(size_t)row * K + i] = key_float((uint32_t)(k >> 32)) - lse;
    } else {
      top_id[(size_t)row * K + i] = -1;
      top_lp[(size_t)row * K + i] = -INFINITY;
    }
  }
}

struct Slot {
  float score;
  int tok, par, dep, rank;
  bool valid;
};

__device__ __forceinline__ uint64_t slot_key(const Slot& s) {
  if (!s.valid) return 0;
  const uint32_t lo = ((0xfffffu - (uint32_t)s.tok) << 7) | (127u - (uint32_t)s.par);
  return (static_cast<uint64_t>(float_key(s.score)) << 32) | lo;
}

// One wavefront per sequence.  T = B+1 <= 65, frontier <= B+1 <= 65 entries.
__global__ void __launch_bounds__(64) heap_expand_kernel(const int32_t* __restrict__ top_id,
                                                         const float* __restrict__ top_lp, int L, int K,
                                                         int T, const int32_t* __restrict__ root_token,
                                                         int32_t* __restrict__ tok, int32_t* __restrict__ parent,
                                                         int32_t* __restrict__ depth, float* __restrict__ score,
                                                         uint64_t* __restrict__ anc) {
  const int s = blockIdx.x, lane = threadIdx.x;
  extern __shared__ uint8_t smem[];
  float* lp = reinterpret_cast<float*>(smem);                  // [L][K]
  int32_t* ids = reinterpret_cast<int32_t*>(lp + L * K);       // [L][K]
  __shared__ float nscore[128];
  __shared__ uint64_t nanc[128];
  for (int i = lane; i < L * K; i += 64) {
    lp[i] = top_lp[(size_t)s * L * K + i];
    ids[i] = top_id[(size_t)s * L * K + i];
  }
  const size_t ob = (size_t)s * T;
  for (int i = lane; i < T; i += 64) {
    tok[ob + i] = (i == 0) ? root_token[s] : -1;
    parent[ob + i] = -1;
    depth[ob + i] = (i == 0) ? 0 : -1;
    score[ob + i] = (i == 0) ? 0.f : -INFINITY;
    anc[ob + i] = 0;
  }
  if (lane == 0) {
    nscore[0] = 0.f;
    nanc[0] = 0;
  }
  __syncthreads();

  Slot s0, s1;  // this lane's frontier slots: index lane and 64 + lane
  s0.valid = s1.valid = false;
  int nslots = 0;
  auto put = [&](int idx, float sc, int tk, int pr, int dp, int rk) {
    if ((idx & 63) == lane) {
      Slot& d = (idx >> 6) ? s1 : s0;
      d.score = sc; d.tok = tk; d.par = pr; d.dep = dp; d.rank = rk; d.valid = true;
    }
  };
  if (T > 1 && L >= 1 && ids[0] >= 0) put(nslots++, 0.f + lp[0], ids[0], 0, 1, 0);

  for (int i = 1; i < T; ++i) {
    const uint64_t k0 = slot_key(s0), k1 = slot_key(s1);
    const uint64_t best = wave_max_u64(k0 > k1 ? k0 : k1);
    if (best == 0) break;
    const uint64_t b0 = __ballot(k0 == best && k0 != 0), b1 = __ballot(k1 == best && k1 != 0);
    const int j = b0 ? 0 : 1;
    const int owner = (int)__ffsll((unsigned long long)(b0 ? b0 : b1)) - 1;
    const int idx = 64 * j + owner;
    const Slot w = j ? s1 : s0;
    const float sc = __shfl(w.score, owner, 64);
    const int tk = __shfl(w.tok, owner, 64), pr = __shfl(w.par, owner, 64);
    const int dp = __shfl(w.dep, owner, 64), rk = __shfl(w.rank, owner, 64);
    const uint64_t a = nanc[pr] | (1ull << (i - 1));
    if (lane == 0) {
      tok[ob + i] = tk; parent[ob + i] = pr; depth[ob + i] = dp; score[ob + i] = sc; anc[ob + i] = a;
      nscore[i] = sc;
      nanc[i] = a;
    }
    // the popped slot takes the next-ranked sibling, or empties
    if (lane == owner) {
      if (j) s1.valid = false;
      else s0.valid = false;
    }
    const int r2 = rk + 1;
    if (r2 < K && ids[(dp - 1) * K + r2] >= 0)
      put(idx, nscore[pr] + lp[(dp - 1) * K + r2], ids[(dp - 1) * K + r2], pr, dp, r2);
    // the best child goes to a fresh slot
    if (dp < L && ids[dp * K] >= 0) put(nslots++, sc + lp[dp * K], ids[dp * K], i, dp + 1, 0);
    __syncthreads();
  }
}

BuildPlan plan_build_tree(int n, int L, int V, int B, int K) {
  BuildPlan p = {};
  p.K = K;
  int S = cdiv(V, kChunkMax);
  const int want = cdiv(512, n * L);
  const int smax_len = V / 2048 > 1 ? V / 2048 : 1;
  if (want > S) S = want < smax_len ? want : (smax_len > S ? smax_len : S);
  if (S * K > kSortMax) S = kSortMax / K;
  p.chunk = (cdiv(V, S) + 7) / 8 * 8;
  p.S = cdiv(V, p.chunk);
  int sn = 1;
  while (sn < p.S * K) sn <<= 1;
  p.sortN = sn;
  const size_t rows = (size_t)n * L;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  p.off_ckey = off; off += al(rows * p.S * K * sizeof(float));
  p.off_cid = off;  off += al(rows * p.S * K * sizeof(int32_t));
  p.off_stat = off; off += al(rows * p.S * sizeof(float2));
  p.off_tid = off;  off += al(rows * K * sizeof(int32_t));
  p.off_tlp = off;  off += al(rows * K * sizeof(float));
  p.total = off;
  return p;
}

hipError_t launch_build_tree(const void* logits, int dt, int n, int L, int V, int B, const BuildPlan& plan,
                             const int32_t* root_token, int32_t* tok, int32_t* parent, int32_t* depth,
                             float* score, uint64_t* anc, void* ws, hipStream_t st) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* cval = reinterpret_cast<float*>(w + plan.off_ckey);
  int32_t* cid = reinterpret_cast<int32_t*>(w + plan.off_cid);
  float2* stat = reinterpret_cast<float2*>(w + plan.off_stat);
  int32_t* tid = reinterpret_cast<int32_t*>(w + plan.off_tid);
  float* tlp = reinterpret_cast<float*>(w + plan.off_tlp);
  const dim3 g1(n * L, plan.S);
  if (dt == DDT_BF16)
    hipLaunchKernelGGL((topk_partial_kernel<uint16_t, 16>), g1, dim3(kTopkThreads), 0, st,
                       static_cast<const uint16_t*>(logits), V, plan.chunk, plan.K, cval, cid, stat);
  else
    hipLaunchKernelGGL((topk_partial_kernel<float, 32>), g1, dim3(kTopkThreads), 0, st,
                       static_cast<const float*>(logits), V, plan.chunk, plan.K, cval, cid, stat);
  hipLaunchKernelGGL(topk_merge_kernel, dim3(n * L), dim3(256), 0, st, cval, cid, stat, plan.S, plan.K,
                     plan.sortN, tid, tlp);
  const size_t smem = (size_t)L * plan.K * (sizeof(float) + sizeof(int32_t));
  hipLaunchKernelGGL(heap_expand_kernel, dim3(n), dim3(64), smem, st, tid, tlp, L, plan.K, B + 1, root_token,
                     tok, parent, depth, score, anc);
  return hipGetLastError();
}

}  // namespace ddt
