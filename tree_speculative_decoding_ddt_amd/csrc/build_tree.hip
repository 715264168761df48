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
//  1. topk_partial  grid (n*L rows, S chunks).  One HBM pass (16-byte loads): each block
//     holds its chunk (<= 16384 logits) in registers as order-preserving integer keys,
//     computes the chunk's (max, sum exp) and selects its exact top-K by (value desc, id asc):
//     a lower bound from the per-thread maxima (per wave, by ballots) filters the chunk;
//     the keys that pass (typically about a hundred) are compacted into LDS as unique
//     64-bit (key, -offset) words and ranked by counting.  When more than 512 pass (many
//     ties near the top), an LDS radix select over the filtered keys finds the K-th value
//     and a second radix select over chunk offsets resolves ties at that value.
//  2. topk_merge    grid (n*L), one thread per compare-exchange.  Bitonic-sorts the S*K
//     chunk candidates as 64-bit (value, -id) keys, keeps the best K, combines the chunk
//     (max, sum) pairs into the row's log-sum-exp and writes lp = z - lse in fp32.
//  3. heap_expand   grid (n), one wavefront.  The frontier (<= B+1 entries) lives in
//     registers, one slot per lane; each pop is a wave-wide max over 64-bit keys
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
constexpr int kCand = 2 * kTopkThreads;                // compacted keys of the usual case

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

template <typename T, int KBITS, bool VECLOAD>
__global__ void __launch_bounds__(kTopkThreads) __attribute__((amdgpu_waves_per_eu(3))) topk_partial_kernel(const T* __restrict__ logits, int V, int chunk,
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
  __shared__ uint32_t tmaxs[kTopkThreads / 64];
  __shared__ uint32_t sel[3];
  __shared__ float2 red[kTopkThreads / 64];
  __shared__ int out_cnt;
  __shared__ uint32_t wpass[kTopkThreads / 64];
  __shared__ uint64_t cand[kCand];

  // chunk offset of register j: element-wise, or VEC consecutive elements per 16-byte load
  constexpr int VEC = 16 / (int)sizeof(T);
  auto elem = [&](int j) -> int {
    if constexpr (VECLOAD) return VEC * (tid + kTopkThreads * (j / VEC)) + (j % VEC);
    else return tid + kTopkThreads * j;
  };

  // 1. load the chunk as keys (exact: KBITS is the width of T), per-thread max key
  uint32_t key[kEmax];
  uint32_t tmax = 0;
  if constexpr (VECLOAD) {
    // the chunk start and the row are 16-byte aligned (V and the chunk length are multiples of VEC)
#pragma unroll
    for (int jv = 0; jv < kEmax / VEC; ++jv) {
      const int e0 = VEC * (tid + kTopkThreads * jv);
      uint4 w = make_uint4(0, 0, 0, 0);
      if (e0 + VEC <= cnt) w = *reinterpret_cast<const uint4*>(p + e0);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        const int e = e0 + i;
        float v;
        if constexpr (sizeof(T) == 2) v = bf16_to_f32(static_cast<uint16_t>(i & 1 ? u[i >> 1] >> 16 : u[i >> 1] & 0xffffu));
        else v = __uint_as_float(u[i]);
        if (e0 + VEC > cnt && e < cnt) v = Elem<T>::load(p, e);  // ragged end of the chunk
        const uint32_t k = e < cnt ? float_key(v) >> (32 - KBITS) : 0u;
        key[jv * VEC + i] = k;
        tmax = k > tmax ? k : tmax;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kEmax; ++j) {
      const int e = elem(j);
      const uint32_t k = e < cnt ? float_key(Elem<T>::load(p, e)) >> (32 - KBITS) : 0u;
      key[j] = k;
      tmax = k > tmax ? k : tmax;
    }
  }
  // the value of a key: the dropped low bits of a 16-bit key are zeros for a positive
  // value and ones for a negative one (the key of a negative value is its complement)
  auto kval = [](uint32_t k) {
    uint32_t kf = k << (32 - KBITS);
    if (KBITS < 32 && !(kf & 0x80000000u)) kf |= (1u << (32 - KBITS)) - 1u;
    return key_float(kf);
  };
  // this thread's (max, sum exp): the max from the largest key, then one exp per element
  float m = -INFINITY, sum = 0.f;
  if (tmax != 0) {
    m = kval(tmax);
    if (m != -INFINITY) {
#pragma unroll
      for (int j = 0; j < kEmax; ++j)
        if (elem(j) < cnt) sum += __expf(kval(key[j]) - m);
    }
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

  // 2. lower bound: each wave finds the c-th largest of its 64 per-thread maxima
  // (c = ceil(keff / waves)) bit by bit with ballots; the smallest of the waves' values
  // is a bound that at least keff thread maxima, hence at least keff keys, reach
  {
    constexpr int NWV = kTopkThreads / 64;
    const uint32_t c = (uint32_t)((keff + NWV - 1) / NWV);
    uint32_t t = 0;
#pragma unroll
    for (int b = KBITS - 1; b >= 0; --b) {
      const uint32_t cand = t | (1u << b);
      if ((uint32_t)__popcll(__ballot(tmax >= cand)) >= c) t = cand;
    }
    if (lane == 0) tmaxs[wave] = t;
  }
  __syncthreads();
  uint32_t tau = tmaxs[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / 64; ++w) tau = tmaxs[w] < tau ? tmaxs[w] : tau;
  const size_t base = ((size_t)row * S + c) * K;

  // 3a. usual case: the keys at or above tau (at least keff of them, typically about a
  // hundred per chunk) fit in LDS.  They are compacted there as unique 64-bit words
  // (key, complement of the chunk offset) and each is ranked by counting the words above
  // it: rank < keff are the chunk's top keff by (value desc, id asc), emitted in order.
  uint32_t npass = 0;
#pragma unroll
  for (int j = 0; j < kEmax; ++j) npass += (elem(j) < cnt && key[j] >= tau) ? 1u : 0u;
  uint32_t incl = npass;  // inclusive prefix over the wave's lanes
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wpass[wave] = incl;
  __syncthreads();
  uint32_t total = 0, off = incl - npass;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const uint32_t x = wpass[w];
    total += x;
    off += w < wave ? x : 0u;
  }
  if (total <= (uint32_t)kCand) {  // block-uniform
#pragma unroll
    for (int j = 0; j < kEmax; ++j) {
      const int e = elem(j);
      if (e < cnt && key[j] >= tau) cand[off++] = (static_cast<uint64_t>(key[j]) << 32) | (0xffffffffu - (uint32_t)e);
    }
    __syncthreads();
    const uint64_t w0 = tid < (int)total ? cand[tid] : 0ull;
    const uint64_t w1 = tid + kTopkThreads < (int)total ? cand[tid + kTopkThreads] : 0ull;
    uint32_t r0 = 0, r1 = 0;
    for (uint32_t i = 0; i < total; ++i) {
      const uint64_t x = cand[i];
      r0 += x > w0 ? 1u : 0u;
      r1 += x > w1 ? 1u : 0u;
    }
    if (tid < (int)total && r0 < (uint32_t)keff) {
      cval[base + r0] = kval(static_cast<uint32_t>(w0 >> 32));
      cid[base + r0] = beg + (int)(0xffffffffu - (uint32_t)w0);
    }
    if (tid + kTopkThreads < (int)total && r1 < (uint32_t)keff) {
      cval[base + r1] = kval(static_cast<uint32_t>(w1 >> 32));
      cid[base + r1] = beg + (int)(0xffffffffu - (uint32_t)w1);
    }
    if (tid >= keff && tid < K) cid[base + tid] = -1;
    return;
  }
  // 3b. otherwise (many keys tied near the top, e.g. a flat row): radix select below

  // 3. radix select of the keff-th largest key among keys >= tau
  uint32_t prefix = 0, pmask = 0, need = keff, count_eq = 0;
#pragma unroll
  for (int shift = KBITS - 8; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kEmax; ++j) {
      const uint32_t k = key[j];
      if (elem(j) < cnt && k >= tau && (k & pmask) == prefix)
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
        const uint32_t e = elem(j);
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
#pragma unroll
  for (int j = 0; j < kEmax; ++j) {
    const uint32_t e = elem(j);
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

__global__ void __launch_bounds__(1024) topk_merge_kernel(const float* __restrict__ cval,
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
  // bitonic sort, descending: in each stage, pair p compares i (bit j of i clear) with i + j
  for (int k = 2; k <= sortN; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int pr = tid; pr < sortN / 2; pr += blockDim.x) {
        const int i = (pr / j) * 2 * j + (pr % j);
        const int ixj = i + j;
        const uint64_t a = sk[i], b = sk[ixj];
        const bool desc = (i & k) == 0;
        if (desc ? (a < b) : (a > b)) {
          sk[i] = b;
          sk[ixj] = a;
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

// One frontier entry: a candidate node (score, token, parent row, depth, rank among the
// depth's top-K) and its next-ranked sibling's (log-prob, token), fetched when the entry
// is made so that a pop reads no LDS on its critical path.
struct Slot {
  float score, nlp;
  int tok, par, dep, rank, ntok;
  bool valid;
};

__device__ __forceinline__ uint64_t slot_key(const Slot& s) {
  if (!s.valid) return 0;
  const uint32_t lo = ((0xfffffu - (uint32_t)s.tok) << 7) | (127u - (uint32_t)s.par);
  return (static_cast<uint64_t>(float_key(s.score)) << 32) | lo;
}

// One wavefront per sequence, T = B+1 <= 65.  The frontier has one slot per lane: the
// seed takes slot 0, pop i puts the popped node's sibling in the popped slot and its best
// child in slot i at most (a fresh slot per pop), and the child of the last pop is never
// popped, so 64 slots suffice.  Every step of a pop is lane-local, a DPP move or a scalar
// read of one lane (readlane): the wave-wide max of the frontier keys, the winner's
// fields, the parent's score and mask (node i's are kept by lane i), and the best child of
// depth d (lane d).  The wave needs no barrier.
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
  __syncthreads();

  // best candidate of depth d + 1 (rank 0) in lane d
  const float blp = lane < L ? lp[lane * K] : -INFINITY;
  const int btok = lane < L ? ids[lane * K] : -1;
  // built nodes: score and ancestor mask of node i held by lane i (i <= 63 are read)
  float nsc = 0.f;
  uint64_t nan = 0ull;

  Slot sl;
  sl.valid = false;
  sl.score = sl.nlp = 0.f;
  sl.tok = sl.par = sl.dep = sl.rank = sl.ntok = 0;
  int nslots = 0;
  // (fields assigned one by one: a reference chosen at run time would put the slot in
  // scratch memory)
  auto put = [&](int idx, float sc, int tk, int pr, int dp, int rk) {
    if (idx == lane) {
      sl.score = sc; sl.tok = tk; sl.par = pr; sl.dep = dp; sl.rank = rk; sl.valid = true;
      const int nx = (dp - 1) * K + rk + 1;
      sl.ntok = rk + 1 < K ? ids[nx] : -1;
      sl.nlp = rk + 1 < K ? lp[nx] : -INFINITY;
    }
  };
  const int tok0 = __builtin_amdgcn_readlane(btok, 0);
  if (T > 1 && L >= 1 && tok0 >= 0)
    put(nslots++, 0.f + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, blp), 0)), tok0,
        0, 1, 0);

  for (int i = 1; i < T; ++i) {
    const uint64_t k = slot_key(sl);
    const uint64_t best = wave_max_u64_uniform(k);
    if (best == 0) break;
    const int owner = __builtin_amdgcn_readfirstlane((int)__ffsll((unsigned long long)__ballot(k == best && k != 0)) - 1);
    const float sc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sl.score), owner));
    const int tk = __builtin_amdgcn_readlane(sl.tok, owner), pr = __builtin_amdgcn_readlane(sl.par, owner);
    const int dp = __builtin_amdgcn_readlane(sl.dep, owner), rk = __builtin_amdgcn_readlane(sl.rank, owner);
    const int ntk = __builtin_amdgcn_readlane(sl.ntok, owner);
    const float nlp = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, sl.nlp), owner));
    const uint64_t a = readlane_u64(nan, pr) | (1ull << (i - 1));
    if (lane == 0) {
      tok[ob + i] = tk; parent[ob + i] = pr; depth[ob + i] = dp; score[ob + i] = sc; anc[ob + i] = a;
    }
    if (lane == i) {  // node 64 (never a parent) is not kept
      nsc = sc;
      nan = a;
    }
    // the popped slot takes the next-ranked sibling, or empties
    if (lane == owner) sl.valid = false;
    if (ntk >= 0) {
      const float psc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, nsc), pr));
      put(owner, psc + nlp, ntk, pr, dp, rk + 1);
    }
    // the best child goes to a fresh slot (none after the last pop)
    if (i + 1 < T && dp < L) {
      const int ctk = __builtin_amdgcn_readlane(btok, dp);
      if (ctk >= 0)
        put(nslots++, sc + __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, blp), dp)), ctk,
            i, dp + 1, 0);
    }
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
  // the merge sorts S*K candidates; above 1024 its cost outgrows what more chunks save
  // in the scan, so stay at 1024 when the chunk size allows
  const int smin = cdiv(V, kChunkMax);
  if (S * K > 1024 && smin * K <= 1024) S = 1024 / K > smin ? 1024 / K : smin;
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
  const int vec = dt == DDT_BF16 ? 8 : 4;
  const bool vload = (reinterpret_cast<uintptr_t>(logits) % 16) == 0 && V % vec == 0 && plan.chunk % vec == 0;
#define DDT_TOPK(TY, KB, VL)                                                                                     \
  hipLaunchKernelGGL((topk_partial_kernel<TY, KB, VL>), g1, dim3(kTopkThreads), 0, st, static_cast<const TY*>(logits), \
                     V, plan.chunk, plan.K, cval, cid, stat)
  if (dt == DDT_BF16) {
    if (vload) DDT_TOPK(uint16_t, 16, true);
    else DDT_TOPK(uint16_t, 16, false);
  } else {
    if (vload) DDT_TOPK(float, 32, true);
    else DDT_TOPK(float, 32, false);
  }
#undef DDT_TOPK
  // one thread per compare-exchange of a sorting stage (sortN / 2 <= 1024)
  hipLaunchKernelGGL(topk_merge_kernel, dim3(n * L), dim3(plan.sortN / 2 < 64 ? 64 : plan.sortN / 2), 0, st, cval,
                     cid, stat, plan.S, plan.K, plan.sortN, tid, tlp);
  const size_t smem = (size_t)L * plan.K * (sizeof(float) + sizeof(int32_t));
  hipLaunchKernelGGL(heap_expand_kernel, dim3(n), dim3(64), smem, st, tid, tlp, L, plan.K, B + 1, root_token,
                     tok, parent, depth, score, anc);
  return hipGetLastError();
}

}  // namespace ddt
