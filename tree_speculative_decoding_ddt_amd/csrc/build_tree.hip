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
//     holds its chunk (<= 8192 logits, 16384 when there are many rows) in registers as raw words, computes the chunk's
//     (max, sum exp) and a lower bound for its top keff from the per-thread maximum keys
//     (per wave, by ballots): at least keff keys reach it.  Every key at or above the
//     bound (typically about a hundred) is written out unordered as a candidate word
//     (order-preserving key, chunk offset).  When more than the chunk's capacity pass
//     (many ties near the top), an LDS radix select over the keys finds the exact keff-th
//     value and a second radix select over chunk offsets resolves ties at that value.
//  2. topk_merge    grid (n*L).  The row's K-th largest key is at least every chunk's
//     bound (of a chunk with K keys above it), so only candidates at or above the largest
//     bound take part; they are ranked by counting as 64-bit (key, complement of the id)
//     words, after a radix select of the K-th word when more than one per thread remain.
//     The chunk (max, sum) pairs give the row's log-sum-exp; lp = z - lse in fp32.
//  3. heap_expand   grid (n), one wavefront.  The frontier (<= B+1 entries) lives in
//     registers, one slot per lane; each pop is a wave-wide max over 64-bit keys
//     (score desc, token asc, parent row asc) -- exact integer comparisons, so the
//     pop order is deterministic.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

constexpr int kTopkThreads = 256;
constexpr int kEmax = 32;                              // logits per thread
constexpr int kChunkMax = kTopkThreads * kEmax;        // 8192 logits per block
constexpr int kCand = 192;                             // candidate words a chunk may write

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

// A chunk candidate: the key in the high bits, the chunk offset (< 2^14) in the low ones.
template <int KBITS> struct CandWord { typedef uint64_t type; };
template <> struct CandWord<16> { typedef uint32_t type; };

// the value of a key: the dropped low bits of a 16-bit key are zeros for a positive
// value and ones for a negative one (the key of a negative value is its complement)
template <int KBITS> __device__ __forceinline__ float key_value(uint32_t k) {
  uint32_t kf = k << (32 - KBITS);
  if (KBITS < 32 && !(kf & 0x80000000u)) kf |= (1u << (32 - KBITS)) - 1u;
  return key_float(kf);
}

template <typename T, int KBITS, bool VECLOAD, int EMAX>
__global__ void __launch_bounds__(kTopkThreads) topk_partial_kernel(const T* __restrict__ logits, int V, int chunk,
                                                                    int K, int cap,
                                                                    typename CandWord<KBITS>::type* __restrict__ cand,
                                                                    int32_t* __restrict__ ccount,
                                                                    uint32_t* __restrict__ ctau,
                                                                    float2* __restrict__ stat) {
  typedef typename CandWord<KBITS>::type CW;
  const int row = blockIdx.x, c = blockIdx.y, S = gridDim.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int beg = c * chunk;
  const int cnt = min(chunk, V - beg);
  const int keff = min(K, cnt);
  const T* p = logits + (size_t)row * V + beg;
  CW* out = cand + ((size_t)row * S + c) * cap;

  __shared__ uint32_t hist[256];
  __shared__ uint32_t tmaxs[kTopkThreads / 64];
  __shared__ uint32_t sel[3];
  __shared__ float2 red[kTopkThreads / 64];
  __shared__ int out_cnt;
  __shared__ uint32_t wpass[kTopkThreads / 64];

  // chunk offset of register j: element-wise, or VEC consecutive elements per 16-byte load
  constexpr int VEC = 16 / (int)sizeof(T);
  auto elem = [&](int j) -> int {
    if constexpr (VECLOAD) return VEC * (tid + kTopkThreads * (j / VEC)) + (j % VEC);
    else return tid + kTopkThreads * j;
  };

  // 1. load the chunk as raw words (two bf16 or one fp32 per dword) and keys on the fly
  constexpr int NW = EMAX * (int)sizeof(T) / 4;
  uint32_t raw[NW];
  // every load is issued unconditionally at a clamped address (no load waits behind a
  // branch); elements past the chunk's end are masked by elem(j) < cnt below
  if constexpr (VECLOAD) {
    // the chunk start and the row are 16-byte aligned and cnt is a multiple of VEC (V and
    // the chunk length are), so a vector starting inside the chunk ends inside it
#pragma unroll
    for (int jv = 0; jv < EMAX / VEC; ++jv) {
      const int e0 = min(VEC * (tid + kTopkThreads * jv), cnt - VEC);
      const uint4 w = *reinterpret_cast<const uint4*>(p + e0);
      raw[4 * jv] = w.x;
      raw[4 * jv + 1] = w.y;
      raw[4 * jv + 2] = w.z;
      raw[4 * jv + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < EMAX; ++j) {
      const int e = min(elem(j), cnt - 1);
      uint32_t b;
      if constexpr (sizeof(T) == 2) b = reinterpret_cast<const uint16_t*>(p)[e];
      else b = reinterpret_cast<const uint32_t*>(p)[e];
      if constexpr (sizeof(T) == 2) {
        if (j & 1) raw[j >> 1] |= b << 16;
        else raw[j >> 1] = b;
      } else {
        raw[j] = b;
      }
    }
  }
  auto val = [&](int j) -> float {
    if constexpr (sizeof(T) == 2) return __uint_as_float((j & 1) ? (raw[j >> 1] & 0xffff0000u) : (raw[j >> 1] << 16));
    else return __uint_as_float(raw[j]);
  };
  // bf16 in 16-byte vectors: the keys of a dword's two logits at once, packed as two
  // 16-bit halves (b ^ 0xffff for a negative b, b | 0x8000 otherwise), the keys of a
  // vector past the chunk's end (cnt is a multiple of VEC) masked to 0
  constexpr bool PK = sizeof(T) == 2 && VECLOAD;
  uint32_t kp[PK ? NW : 1];
  auto vvalid = [&](int jv) { return VEC * (tid + kTopkThreads * jv) < cnt; };
  if constexpr (PK) {
#pragma unroll
    for (int jv = 0; jv < EMAX / VEC; ++jv) {
      const uint32_t vm = vvalid(jv) ? 0xffffffffu : 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t w = raw[4 * jv + q];
        kp[4 * jv + q] = (w ^ (((w >> 15) & 0x10001u) * 0x7fffu + 0x80008000u)) & vm;
      }
    }
  }
  auto key = [&](int j) -> uint32_t {
    if constexpr (PK) return (j & 1) ? kp[j >> 1] >> 16 : kp[j >> 1] & 0xffffu;
    else return elem(j) < cnt ? float_key(val(j)) >> (32 - KBITS) : 0u;
  };

  // this thread's largest key, then (max, sum exp) with one exp per element
  uint32_t tmax = 0;
  if constexpr (PK) {
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 mx = {0, 0};
#pragma unroll
    for (int q = 0; q < NW; ++q) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(us2, kp[q]));
    tmax = max((uint32_t)mx.x, (uint32_t)mx.y);
  } else {
#pragma unroll
    for (int j = 0; j < EMAX; ++j) tmax = max(tmax, key(j));
  }
  float m = -INFINITY, sum = 0.f;
  if (tmax != 0) {
    m = key_value<KBITS>(tmax);
    if (m != -INFINITY) {
      if constexpr (PK) {
#pragma unroll
        for (int jv = 0; jv < EMAX / VEC; ++jv) {  // a vector's 8 terms, kept or dropped whole
          // exp(v - m) as 2^(v log2 e - m log2 e)
          const float ml = m * 1.4426950408889634f;
          float s8 = 0.f;
#pragma unroll
          for (int i = 0; i < VEC; ++i) s8 += __builtin_amdgcn_exp2f(fmaf(val(VEC * jv + i), 1.4426950408889634f, -ml));
          sum += vvalid(jv) ? s8 : 0.f;
        }
      } else {
#pragma unroll
        for (int j = 0; j < EMAX; ++j) {  // branch-free: masked elements add 0
          const float ex = __expf(val(j) - m);
          sum += elem(j) < cnt ? ex : 0.f;
        }
      }
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

  // 2. lower bound: each wave finds the c-th largest of its 64 per-thread maxima
  // (c = ceil(keff / waves)) bit by bit with ballots; the smallest of the waves' values
  // is a bound that at least keff thread maxima, hence at least keff keys, reach
  {
    constexpr int NWV = kTopkThreads / 64;
    const uint32_t cw = (uint32_t)((keff + NWV - 1) / NWV);
    uint32_t t = 0;
#pragma unroll
    for (int b = KBITS - 1; b >= 0; --b) {
      const uint32_t cb = t | (1u << b);
      if ((uint32_t)__popcll(__ballot(tmax >= cb)) >= cw) t = cb;
    }
    if (lane == 0) tmaxs[wave] = t;
  }
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
  uint32_t tau = tmaxs[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / 64; ++w) tau = tmaxs[w] < tau ? tmaxs[w] : tau;

  // 3a. usual case: every key at or above tau (at least keff of them, typically about a
  // hundred per chunk) is a candidate, written unordered; the merge ranks them
  // masked keys are 0: with tau > 0 the key test alone excludes them.  In range:
  // element by element, or (packed keys) vector by vector
  const bool tpos = tau > 0;
  auto inrange = [&](int j) {
    if constexpr (PK) return vvalid(j / VEC);
    else return elem(j) < cnt;
  };
  uint32_t npass = 0;
#pragma unroll
  for (int j = 0; j < EMAX; ++j) npass += ((tpos || inrange(j)) && key(j) >= tau) ? 1u : 0u;
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
  // the bound holds for the row only when the chunk has K keys at or above it
  const uint32_t bound = keff == K ? tau : 0u;
  if (total <= (uint32_t)cap) {  // block-uniform
#pragma unroll
    for (int j = 0; j < EMAX; ++j) {
      const int e = elem(j);
      const uint32_t k = key(j);
      if ((tpos || inrange(j)) && k >= tau) out[off++] = (static_cast<CW>(k) << (KBITS == 16 ? 16 : 32)) | (CW)e;
    }
    if (tid == 0) {
      ccount[(size_t)row * S + c] = (int)total;
      ctau[(size_t)row * S + c] = bound;
    }
    return;
  }
  // 3b. otherwise (many keys tied near the top, e.g. a flat row): the exact top keff by
  // radix select, the keff-th largest key among keys >= tau
  uint32_t prefix = 0, pmask = 0, need = keff, count_eq = 0;
#pragma unroll
  for (int shift = KBITS - 8; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < EMAX; ++j) {
      const uint32_t k = key(j);
      if (elem(j) < cnt && k >= tau && (k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
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
      for (int j = 0; j < EMAX; ++j) {
        const uint32_t e = elem(j);
        if ((int)e < cnt && key(j) == kth && (e & msk2) == pre2) atomicAdd(&hist[(e >> shift) & 255u], 1u);
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

  // 5. emit exactly keff candidates (unordered)
  if (tid == 0) out_cnt = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EMAX; ++j) {
    const uint32_t e = elem(j);
    const uint32_t k = key(j);
    if ((int)e < cnt && (k > kth || (k == kth && e <= off_th))) {
      const int pos = atomicAdd(&out_cnt, 1);
      if (pos < keff) out[pos] = (static_cast<CW>(k) << (KBITS == 16 ? 16 : 32)) | (CW)e;
    }
  }
  if (tid == 0) {
    ccount[(size_t)row * S + c] = keff;
    ctau[(size_t)row * S + c] = keff == K ? kth : 0u;
  }
}

constexpr int kMergeThreads = 512;
constexpr int kMergeMax = 8192;  // candidates of one row (S * cap)
constexpr int kHistBins = 2048;  // key range [bound, largest key] counted bin by bin

// One block per (sequence, depth) row.  The row's K-th largest key is at least every
// chunk's bound (of a chunk with K keys at or above it), so only candidates at or above
// the largest bound take part, as 64-bit words (key, complement of the vocabulary id).
// A radix select over their keys finds the K-th largest key; the words above it and
// the ties at it are ranked by counting (a radix select over the id part first when the
// ties do not fit one per thread).
template <int KBITS>
__global__ void __launch_bounds__(kMergeThreads) topk_merge_kernel(const typename CandWord<KBITS>::type* __restrict__ cand,
                                                                  const int32_t* __restrict__ ccount,
                                                                  const uint32_t* __restrict__ ctau,
                                                                  const float2* __restrict__ stat, int S, int K,
                                                                  int cap, int chunk, int V,
                                                                  int32_t* __restrict__ top_id,
                                                                  float* __restrict__ top_lp) {
  typedef typename CandWord<KBITS>::type CW;
  constexpr int SH = KBITS == 16 ? 16 : 32;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint64_t fk[kMergeMax];
  __shared__ uint64_t top[kMergeThreads];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sel[3];
  __shared__ int nf, ntop;
  __shared__ int cbeg[129];       // first candidate of each chunk in the row's list
  __shared__ uint32_t ctau_s[2];  // largest bound, largest kept key
  __shared__ uint32_t hist2[kHistBins];
  __shared__ float2 st_s[128];
  __shared__ float lse_s;
  // the chunks' counts, bounds and (max, sum) pairs, one chunk per thread (S <= 128)
  if (tid < 64) {
    int nc0 = 0, nc1 = 0;
    uint32_t b = 0;
    if (tid < S) {
      nc0 = ccount[(size_t)row * S + tid];
      b = ctau[(size_t)row * S + tid];
      st_s[tid] = stat[(size_t)row * S + tid];
    }
    if (tid + 64 < S) {
      nc1 = ccount[(size_t)row * S + tid + 64];
      b = max(b, ctau[(size_t)row * S + tid + 64]);
      st_s[tid + 64] = stat[(size_t)row * S + tid + 64];
    }
    // exclusive prefix of the counts over chunk order (lanes hold chunks l and l + 64)
    int inc = nc0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o, 64);
      if (lane >= o) inc += t;
    }
    const int tot0 = __shfl(inc, 63, 64);
    int inc1 = nc1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc1, o, 64);
      if (lane >= o) inc1 += t;
    }
    cbeg[tid] = inc - nc0;
    cbeg[tid + 64] = tot0 + inc1 - nc1;
    if (tid == 63) cbeg[128] = tot0 + inc1;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) b = max(b, (uint32_t)__shfl_xor((int)b, o, 64));
    if (tid == 0) {
      ctau_s[0] = b;
      ctau_s[1] = 0;
      nf = 0;
      ntop = 0;
    }
  }
  __syncthreads();
  if (wave == 0) {  // the row's log-sum-exp from the chunks' (max, sum) pairs
    const float2 a = lane < S ? st_s[lane] : make_float2(-INFINITY, 0.f);
    const float2 b = lane + 64 < S ? st_s[lane + 64] : make_float2(-INFINITY, 0.f);
    float M = fmaxf(a.x, b.x);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
    float tot = (a.x != -INFINITY ? a.y * __expf(a.x - M) : 0.f) + (b.x != -INFINITY ? b.y * __expf(b.x - M) : 0.f);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
    if (lane == 0) lse_s = M + __logf(tot);
  }
  const uint32_t tau = ctau_s[0];
  // gather the candidates at or above tau as (key, complement of the id).  Slot
  // u = c * cap + j holds word j of chunk c; the S * cap <= kMergeMax slots are dealt to
  // the threads, and every load is issued before the first is used.
  constexpr int U = kMergeMax / kMergeThreads;
  CW xs[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int slot = tid + kMergeThreads * u;
    const int c = min(slot / cap, S - 1), j = slot - c * cap;
    xs[u] = cand[((size_t)row * S + c) * cap + min(j, cap - 1)];
  }
  uint32_t kmax = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int slot = tid + kMergeThreads * u;
    const int c = slot / cap, j = slot - c * cap;
    const bool in = c < S && j < cbeg[c + 1] - cbeg[c];
    const uint32_t k = (uint32_t)(xs[u] >> SH);
    const bool keep = in && k >= tau;
    const uint32_t id = (uint32_t)(c * chunk) + (uint32_t)(xs[u] & (((CW)1 << SH) - 1));
    const uint64_t w = (static_cast<uint64_t>(k) << 32) | (0xffffffffu - id);
    kmax = keep ? max(kmax, k) : kmax;
    const uint64_t bal = __ballot(keep);
    if (bal == 0) continue;  // wave-uniform
    int base = 0;
    if (lane == 0) base = atomicAdd(&nf, (int)__popcll(bal));
    base = __shfl(base, 0, 64);
    if (keep) fk[base + __popcll(bal & ((1ull << lane) - 1))] = w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  if (lane == 0) atomicMax(&ctau_s[1], kmax);
  __syncthreads();
  const int M = nf;
  const int keff = min(K, V);
  const float lse = lse_s;
  auto emit = [&](int r, uint64_t w) {
    top_id[(size_t)row * K + r] = (int32_t)(0xffffffffu - (uint32_t)w);
    top_lp[(size_t)row * K + r] = key_value<KBITS>((uint32_t)(w >> 32)) - lse;
  };
  // the keff-th largest key kth: by a histogram over [tau, kmax] when that range is
  // short (the usual case: the top of a row spans few bf16 values), else by 8-bit digits
  uint32_t kth = 0, above = 0;
  const uint32_t krange = ctau_s[1] - tau + 1;
  if (krange <= kHistBins) {
    for (int b = tid; b < (int)krange; b += kMergeThreads) hist2[b] = 0;
    __syncthreads();
    for (int i = tid; i < M; i += kMergeThreads) atomicAdd(&hist2[(uint32_t)(fk[i] >> 32) - tau], 1u);
    __syncthreads();
    if (wave == 0) {  // from the top bin down: the bin where the running count reaches keff
      constexpr int PER = kHistBins / 64;
      const int b0 = (int)krange - 1 - PER * lane;  // lane l scans bins b0, b0 - 1, ...
      uint32_t h[PER], tot = 0;
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        h[q] = b0 - q >= 0 ? hist2[b0 - q] : 0u;
        tot += h[q];
      }
      uint32_t inc = tot;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
      }
      uint32_t acc = inc - tot;
      if (acc < (uint32_t)keff && (uint32_t)keff <= inc) {
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          if (acc + h[q] >= (uint32_t)keff) {
            sel[0] = tau + (uint32_t)(b0 - q);
            sel[1] = acc;  // keys above kth
            break;
          }
          acc += h[q];
        }
      }
    }
    __syncthreads();
    kth = sel[0];
    above = sel[1];
  } else {
    uint32_t kmask = 0, need = keff;
    for (int shift = KBITS - 8; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < M; i += kMergeThreads) {
        const uint32_t k = (uint32_t)(fk[i] >> 32);
        if ((k & kmask) == kth) atomicAdd(&hist[(k >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) find_digit(hist, need, true, sel);
      __syncthreads();
      need -= sel[1];
      kth |= sel[0] << shift;
      kmask |= 255u << shift;
    }
    above = (uint32_t)keff - need;
  }
  // every word with a key above kth, and the ties at kth, ranked by counting among
  // themselves (all other words are smaller)
  for (int i = tid; i < M; i += kMergeThreads) {
    const uint64_t w = fk[i];
    if ((uint32_t)(w >> 32) >= kth) {
      const int at = atomicAdd(&ntop, 1);
      if (at < kMergeThreads) top[at] = w;
    }
  }
  __syncthreads();
  const int C = ntop;
  if (C <= kMergeThreads) {  // block-uniform
    if (tid < C) {
      const uint64_t w = top[tid];
      int r = 0;
      for (int i = 0; i < C; ++i) r += top[i] > w ? 1 : 0;
      if (r < keff) emit(r, w);
    }
  } else {
    // many ties at the keff-th key: the keff-th largest word by 8-bit digits of the
    // id part (the key part is kth), then the words at or above it ranked by counting
    uint32_t prefix = 0, pmask = 0, need2 = (uint32_t)keff - above;  // ties to take
    for (int shift = 24; shift >= 0; shift -= 8) {
      if (tid < 256) hist[tid] = 0;
      __syncthreads();
      for (int i = tid; i < M; i += kMergeThreads) {
        const uint64_t w = fk[i];
        const uint32_t lo = (uint32_t)w;
        if ((uint32_t)(w >> 32) == kth && (lo & pmask) == prefix) atomicAdd(&hist[(lo >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) find_digit(hist, need2, true, sel);
      __syncthreads();
      need2 -= sel[1];
      prefix |= sel[0] << shift;
      pmask |= 255u << shift;
    }
    const uint64_t wth = (static_cast<uint64_t>(kth) << 32) | prefix;
    if (tid == 0) ntop = 0;
    __syncthreads();
    for (int i = tid; i < M; i += kMergeThreads) {
      const uint64_t w = fk[i];
      if (w >= wth) top[atomicAdd(&ntop, 1)] = w;  // exactly keff words
    }
    __syncthreads();
    if (tid < keff) {
      const uint64_t w = top[tid];
      int r = 0;
      for (int i = 0; i < keff; ++i) r += top[i] > w ? 1 : 0;
      emit(r, w);
    }
  }
  for (int r = keff + tid; r < K; r += kMergeThreads) {
    top_id[(size_t)row * K + r] = -1;
    top_lp[(size_t)row * K + r] = -INFINITY;
  }
}

// 64-bit key of a frontier entry: score desc, then token asc, then parent row asc.
__device__ __forceinline__ uint64_t frontier_key(float score, int tok, int par) {
  const uint32_t lo = ((0xfffffu - (uint32_t)tok) << 7) | (127u - (uint32_t)par);
  return (static_cast<uint64_t>(float_key(score)) << 32) | lo;
}

// Largest 32-bit value over the wave, by DPP within rows of 16 and reads of 4 lanes.
__device__ __forceinline__ uint32_t wave_max_u32_uniform(uint32_t v) {
  v = max(v, DDT_DPP_U32(v, 0x128));  // row_ror:8
  v = max(v, DDT_DPP_U32(v, 0x124));  // row_ror:4
  v = max(v, DDT_DPP_U32(v, 0x122));  // row_ror:2
  v = max(v, DDT_DPP_U32(v, 0x121));  // row_ror:1
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0), b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32), d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// One wavefront per sequence, T = B+1 <= 65.  The frontier is kept sorted across the
// lanes by the 64-bit key (score desc, token asc, parent row asc), so a pop reads lane 0
// and needs no reduction.  Of its two successors, the next sibling's score is the parent
// row's score plus the sibling's log-prob (one LDS read), and the best child comes from
// the lanes of the depth (rank 0 of depth d + 1 in lane d); each is placed by one ballot
// of the larger keys, and the other entries shift by DPP.  The pop order is the
// best-first heap's, so the tree is the same.  Node i's row, score and ancestor mask are
// kept by lane i (node 64 in scalars) and stored at the end.
__global__ void __launch_bounds__(64) heap_expand_kernel(const int32_t* __restrict__ top_id,
                                                         const float* __restrict__ top_lp, int L, int K,
                                                         int T, const int32_t* __restrict__ root_token,
                                                         int32_t* __restrict__ tok, int32_t* __restrict__ parent,
                                                         int32_t* __restrict__ depth, float* __restrict__ score,
                                                         uint64_t* __restrict__ anc) {
  const int s = blockIdx.x, lane = threadIdx.x;
  extern __shared__ uint8_t smem[];
  float2* cand = reinterpret_cast<float2*>(smem);  // [L][K]: (log-prob, token bits), one 8-byte read
  for (int i0 = 0; i0 < L * K; i0 += 16 * 64) {  // sixteen loads of each in flight per lane
    float a[16];
    int b[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = min(i0 + 64 * u + lane, L * K - 1);
      a[u] = top_lp[(size_t)s * L * K + i];
      b[u] = top_id[(size_t)s * L * K + i];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = min(i0 + 64 * u + lane, L * K - 1);
      cand[i] = make_float2(a[u], __builtin_bit_cast(float, b[u]));
    }
  }
  __syncthreads();

  // rank 0 of depth d + 1 in lane d
  const float2 c0 = cand[min(lane, L - 1) * K];
  const float bl0 = lane < L ? c0.x : -INFINITY;
  const int bt0 = lane < L ? __builtin_bit_cast(int, c0.y) : -1;
  // node i (i <= 63) in lane i: token, parent, depth, score, ancestor mask
  int o_tok = lane == 0 ? root_token[s] : -1, o_par = -1, o_dep = lane == 0 ? 0 : -1;
  float o_sc = lane == 0 ? 0.f : -INFINITY;
  uint64_t o_anc = 0ull;
  int tok64 = -1, par64 = -1, dep64 = -1;  // node 64
  float sc64 = -INFINITY;
  uint64_t anc64 = 0ull;

  // The frontier, sorted: lane p holds the entry of rank p by frontier key (lane 0 the
  // best; empty lanes have f_tk1 = 0 and sort last).  An entry is its score, token + 1 and
  // the packed (parent row << 16 | depth << 8 | rank); its parent's score is the parent
  // row's (lane `parent` of o_sc) and its next-ranked sibling is read from LDS at its pop.
  // A pop takes lane 0; its two successors (the next sibling, the best child) are placed
  // by counting the lanes whose key is larger (one ballot each), and every other entry
  // moves by 0, 1 or 2 lanes (wave-wide DPP shifts).  An entry pushed past lane 63 ranks
  // below every pop still to come.
  float f_sc = 0.f;
  int f_tk1 = 0, f_pdr = 0;
  const int tok0 = __builtin_amdgcn_readlane(bt0, 0);
  if (T > 1 && L >= 1 && tok0 >= 0 && lane == 0) {
    f_sc = bl0; f_tk1 = tok0 + 1; f_pdr = 1 << 8;  // parent row 0 (the root), depth 1, rank 0
  }
  // wave_shl:1 (lane l reads lane l+1) and wave_shr:1 (lane l reads lane l-1); a lane
  // with no source reads 0 (an empty entry, as f_tk1 = 0)
#define DDT_SHL1(x) __builtin_amdgcn_mov_dpp((x), 0x130, 0xf, 0xf, true)
#define DDT_SHR1(x) __builtin_amdgcn_mov_dpp((x), 0x138, 0xf, 0xf, true)
#define DDT_RLF(x, l) __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, (x)), (l)))
  // pops 1 .. min(T, 64) - 1 (node 64, if any, is popped after the loop); a pop from an
  // empty frontier (a tree of fewer than B nodes) changes nothing
  const int tpop = min(T, 64);
  for (int i = 1; i < tpop; ++i) {
    const int tk = __builtin_amdgcn_readfirstlane(f_tk1) - 1;
    const bool live = tk >= 0;
    const float sc = DDT_RLF(f_sc, 0);
    const int pdr = __builtin_amdgcn_readfirstlane(f_pdr);
    const int pr = pdr >> 16, dp = (pdr >> 8) & 255, rk = pdr & 255;
    // the next sibling: rank rk + 1 of depth dp under the same parent
    const int nx = min(max((dp - 1) * K + rk + 1, 0), L * K - 1);
    const float2 nc = cand[nx];
    const float nlp = nc.x;
    const int ntk = live && rk + 1 < K ? __builtin_bit_cast(int, nc.y) : -1;
    const float psc = DDT_RLF(o_sc, pr);
    // the best child: rank 0 of depth dp + 1 (none after the last pop)
    const int dpc = min(dp, 63);
    const int ctk = __builtin_amdgcn_readlane(bt0, dpc);
    const float clp = DDT_RLF(bl0, dpc);
    const bool sib = ntk >= 0;
    const bool chd = live && i + 1 < T && dp < L && ctk >= 0;
    const float scA = psc + nlp, scB = sc + clp;
    const uint64_t kA = frontier_key(scA, ntk, pr), kB = frontier_key(scB, ctk, i);
    // ranks among the entries left after the pop (lanes 1..63)
    const uint64_t kl = (lane >= 1 && f_tk1 > 0) ? frontier_key(f_sc, f_tk1 - 1, f_pdr >> 16) : 0ull;
    const int cA = __popcll(__ballot(kl > kA)), cB = __popcll(__ballot(kl > kB));
    const int posA = sib ? cA + (chd && kB > kA ? 1 : 0) : 99;
    const int posB = chd ? cB + (sib && kA > kB ? 1 : 0) : 99;
    // entry of lane l after the pop and the insertions: A or B, else the old entry of lane
    // l + 1 - (new entries placed before l)
    const int nb = (lane > posA ? 1 : 0) + (lane > posB ? 1 : 0);
    {
      const int s0 = __builtin_bit_cast(int, f_sc);
      const int a0 = DDT_SHL1(s0), a2 = DDT_SHR1(s0);
      const int b0 = DDT_SHL1(f_tk1), b2 = DDT_SHR1(f_tk1);
      const int c0 = DDT_SHL1(f_pdr), c2 = DDT_SHR1(f_pdr);
      const int ms = nb == 0 ? a0 : (nb == 1 ? s0 : a2);
      f_tk1 = nb == 0 ? b0 : (nb == 1 ? f_tk1 : b2);
      f_pdr = nb == 0 ? c0 : (nb == 1 ? f_pdr : c2);
      f_sc = __builtin_bit_cast(float, ms);
    }
    const bool isA = lane == posA, isB = lane == posB;
    f_sc = isA ? scA : (isB ? scB : f_sc);
    f_tk1 = isA ? ntk + 1 : (isB ? ctk + 1 : f_tk1);
    f_pdr = isA ? pdr + 1 : (isB ? ((i << 16) | ((dp + 1) << 8)) : f_pdr);
    // node i's row
    const uint64_t a = readlane_u64(o_anc, pr) | (1ull << (i - 1));
    const bool me = live && lane == i;
    o_tok = me ? tk : o_tok;
    o_par = me ? pr : o_par;
    o_dep = me ? dp : o_dep;
    o_sc = me ? sc : o_sc;
    o_anc = me ? a : o_anc;
  }
  if (T > 64) {  // the last pop: node 64 (its successors are not needed)
    const int tk = __builtin_amdgcn_readfirstlane(f_tk1) - 1;
    if (tk >= 0) {
      const int pdr = __builtin_amdgcn_readfirstlane(f_pdr);
      tok64 = tk;
      par64 = pdr >> 16;
      dep64 = (pdr >> 8) & 255;
      sc64 = DDT_RLF(f_sc, 0);
      anc64 = readlane_u64(o_anc, par64) | (1ull << 63);
    }
  }
#undef DDT_SHL1
#undef DDT_SHR1
#undef DDT_RLF
  // the rows: node i from lane i (rows not reached keep tok -1, depth -1, score -inf)
  const size_t ob = (size_t)s * T;
  if (lane < T) {
    tok[ob + lane] = o_tok;
    parent[ob + lane] = o_par;
    depth[ob + lane] = o_dep;
    score[ob + lane] = o_sc;
    anc[ob + lane] = o_anc;
  }
  if (T > 64 && lane == 0) {
    tok[ob + 64] = tok64;
    parent[ob + 64] = par64;
    depth[ob + 64] = dep64;
    score[ob + 64] = sc64;
    anc[ob + 64] = anc64;
  }
}

BuildPlan plan_build_tree(int n, int L, int V, int B, int K) {
  BuildPlan p = {};
  p.K = K;
  // chunks of up to 8192 logits; 16384 when the rows alone give the chip several
  // thousand blocks; more, smaller chunks (at least 2048 logits) when the rows are few
  int S = cdiv(V, kChunkMax);
  if ((long)n * L * S >= 8192 && V > kChunkMax) S = cdiv(V, 2 * kChunkMax);
  const int want = cdiv(1024, n * L);
  const int smax_len = V / 2048 > 1 ? V / 2048 : 1;
  if (want > S) S = want < smax_len ? want : (smax_len > S ? smax_len : S);
  if (S > 64) S = 64;
  p.chunk = (cdiv(V, S) + 7) / 8 * 8;
  p.S = cdiv(V, p.chunk);
  // candidate space per chunk: cap 4-byte words (bf16 logits) or cap / 2 8-byte words
  // (fp32).  A row's candidates fit the merge's LDS, and cap / 2 >= 64 >= K (S <= 64).
  // A chunk typically passes about a hundred keys; above its space it takes the exact
  // path, which writes K.
  p.cap = kMergeMax / p.S < kCand ? kMergeMax / p.S : kCand;
  const size_t rows = (size_t)n * L;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  p.off_ckey = off; off += al(rows * p.S * p.cap * 4);
  p.off_cid = off;  off += al(rows * p.S * (sizeof(int32_t) + sizeof(uint32_t)));  // counts, bounds
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
  void* cand = w + plan.off_ckey;
  int32_t* ccount = reinterpret_cast<int32_t*>(w + plan.off_cid);
  uint32_t* ctau = reinterpret_cast<uint32_t*>(ccount + (size_t)n * L * plan.S);
  float2* stat = reinterpret_cast<float2*>(w + plan.off_stat);
  int32_t* tid = reinterpret_cast<int32_t*>(w + plan.off_tid);
  float* tlp = reinterpret_cast<float*>(w + plan.off_tlp);
  const dim3 g1(n * L, plan.S);
  const int vec = dt == DDT_BF16 ? 8 : 4;
  const bool vload = (reinterpret_cast<uintptr_t>(logits) % 16) == 0 && V % vec == 0 && plan.chunk % vec == 0;
  const bool small = plan.chunk <= 16 * kTopkThreads, big = plan.chunk > kChunkMax;
  const int cap = dt == DDT_BF16 ? plan.cap : plan.cap / 2;  // words of 4 or 8 bytes
#define DDT_TOPK(TY, KB, VL)                                                                                     \
  {                                                                                                              \
    auto* cw_ = static_cast<typename CandWord<KB>::type*>(cand);                                                 \
    if (small)                                                                                                   \
      hipLaunchKernelGGL((topk_partial_kernel<TY, KB, VL, 16>), g1, dim3(kTopkThreads), 0, st,                   \
                         static_cast<const TY*>(logits), V, plan.chunk, plan.K, cap, cw_, ccount, ctau, stat);   \
    else if (big)                                                                                                \
      hipLaunchKernelGGL((topk_partial_kernel<TY, KB, VL, 2 * kEmax>), g1, dim3(kTopkThreads), 0, st,            \
                         static_cast<const TY*>(logits), V, plan.chunk, plan.K, cap, cw_, ccount, ctau, stat);   \
    else                                                                                                         \
      hipLaunchKernelGGL((topk_partial_kernel<TY, KB, VL, kEmax>), g1, dim3(kTopkThreads), 0, st,                \
                         static_cast<const TY*>(logits), V, plan.chunk, plan.K, cap, cw_, ccount, ctau, stat);   \
  }
  if (dt == DDT_BF16) {
    if (vload) DDT_TOPK(uint16_t, 16, true) else DDT_TOPK(uint16_t, 16, false)
    hipLaunchKernelGGL(topk_merge_kernel<16>, dim3(n * L), dim3(kMergeThreads), 0, st,
                       static_cast<const uint32_t*>(cand), ccount, ctau, stat, plan.S, plan.K, cap, plan.chunk, V,
                       tid, tlp);
  } else {
    if (vload) DDT_TOPK(float, 32, true) else DDT_TOPK(float, 32, false)
    hipLaunchKernelGGL(topk_merge_kernel<32>, dim3(n * L), dim3(kMergeThreads), 0, st,
                       static_cast<const uint64_t*>(cand), ccount, ctau, stat, plan.S, plan.K, cap, plan.chunk, V,
                       tid, tlp);
  }
#undef DDT_TOPK
  const size_t smem = (size_t)L * plan.K * sizeof(float2);
  hipLaunchKernelGGL(heap_expand_kernel, dim3(n), dim3(64), smem, st, tid, tlp, L, plan.K, B + 1, root_token,
                     tok, parent, depth, score, anc);
  return hipGetLastError();
}

}  // namespace ddt
