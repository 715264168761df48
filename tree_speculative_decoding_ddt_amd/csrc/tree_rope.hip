// Rotary embedding of the tree rows at positions prefix + depth, ahead of the tree
// attention of the same call.
// Sources: "DDTree on vLLM: candid research notes", sections "What broke along the
// way" and "Where the next step is" (positions and RoPE must follow the branch depth;
// tree K/V go to scratch, never to the committed cache); "From DDTree to drafter
// training", section "The Architecture of DDTree" (one pass over the whole tree).
//
// Rotate-half layout: channel pairs (j, j + rot/2), j < rot/2, turn by
// pos * theta^(-2j/rot); channels from rot on pass unchanged.  pos = prefix_len[s] +
// depth[s][t].  One block per (sequence, tree row): the angles are formed in fp64
// (positions reach 10^5 radians at the slowest pair, where an fp32 product would be
// off by 10^-2) and kept as fp32 cos/sin in LDS; the rotation itself is fp32.
//   q      [n][T][Hq][D]  -> q_out  [n][T][Hq][D]   (workspace; the attention's queries)
//   k_new  [n][T][Hkv][D] -> k_tree [n][Hkv][T][D]  (rotated, the commit's source)
//   v_new  [n][T][Hkv][D] -> v_tree [n][Hkv][T][D]  (copied)
// A thread moves 8 channels (16 bytes of bf16, 32 of fp32); rot is a multiple of 16,
// so an 8-channel chunk lies wholly in the first half, the second half or the tail.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace ddt {

template <typename A> struct Chunk8;
template <> struct Chunk8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void store(uint16_t* p) const { *reinterpret_cast<uint4*>(p) = w; }
  __device__ __forceinline__ float get(int e) const {
    const uint32_t u = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
    return __uint_as_float((e & 1) ? (u & 0xffff0000u) : (u << 16));
  }
  __device__ __forceinline__ void set_all(const float* f) {
    uint32_t u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = static_cast<uint32_t>(f32_to_bf16(f[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(f[2 * i + 1])) << 16);
    w = make_uint4(u[0], u[1], u[2], u[3]);
  }
};
template <> struct Chunk8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void store(float* p) const {
    reinterpret_cast<float4*>(p)[0] = a;
    reinterpret_cast<float4*>(p)[1] = b;
  }
  __device__ __forceinline__ float get(int e) const {
    const float4& v = e < 4 ? a : b;
    const int i = e & 3;
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
  }
  __device__ __forceinline__ void set_all(const float* f) {
    a = make_float4(f[0], f[1], f[2], f[3]);
    b = make_float4(f[4], f[5], f[6], f[7]);
  }
};

template <typename A>
__global__ void __launch_bounds__(256) rope_tree_kernel(const A* __restrict__ q, const A* __restrict__ k_new,
                                                        const A* __restrict__ v_new, const int32_t* __restrict__ depth,
                                                        const int32_t* __restrict__ prefix_len, int T, int Hq, int Hkv,
                                                        int D, int rot, double log2_theta, A* __restrict__ q_out,
                                                        A* __restrict__ k_tree, A* __restrict__ v_tree) {
  __shared__ float cs[128], sn[128];
  const int s = blockIdx.x / T, t = blockIdx.x % T;
  const int half = rot / 2;
  const double pos = (double)prefix_len[s] + (double)depth[(size_t)s * T + t];
  for (int j = threadIdx.x; j < half; j += blockDim.x) {
    const double inv_freq = exp2(-(2.0 * j / rot) * log2_theta);
    double sa, ca;
    sincos(pos * inv_freq, &sa, &ca);
    cs[j] = (float)ca;
    sn[j] = (float)sa;
  }
  __syncthreads();
  const int CH = D / 8;
  const int total = (Hq + 2 * Hkv) * CH;
  const size_t tok = (size_t)s * T + t;
  for (int c = threadIdx.x; c < total; c += blockDim.x) {
    const int r = c / CH, e0 = (c % CH) * 8;
    const A* src;
    A* dst;
    bool rotate = true;
    if (r < Hq) {
      src = q + (tok * Hq + r) * D;
      dst = q_out + (tok * Hq + r) * D;
    } else if (r < Hq + Hkv) {
      const int h = r - Hq;
      src = k_new + (tok * Hkv + h) * D;
      dst = k_tree + (((size_t)s * Hkv + h) * T + t) * D;
    } else {
      const int h = r - Hq - Hkv;
      src = v_new + (tok * Hkv + h) * D;
      dst = v_tree + (((size_t)s * Hkv + h) * T + t) * D;
      rotate = false;
    }
    Chunk8<A> x;
    x.load(src + e0);
    if (rotate && e0 < rot) {
      const bool lo = e0 < half;
      const int j0 = lo ? e0 : e0 - half;  // pair index of the chunk's first channel
      Chunk8<A> p;
      p.load(src + (lo ? e0 + half : e0 - half));
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c_ = cs[j0 + e], s_ = sn[j0 + e];
        // first half: x c - x' s;  second half: x c + x' s  (x' the pair's other channel)
        y[e] = lo ? x.get(e) * c_ - p.get(e) * s_ : x.get(e) * c_ + p.get(e) * s_;
      }
      x.set_all(y);
    }
    x.store(dst + e0);
  }
}

hipError_t launch_tree_rope(const void* q, const void* k_new, const void* v_new, const int32_t* depth,
                            const int32_t* prefix_len, int n, int T, int Hq, int Hkv, int D, int rot, float theta,
                            int dt, void* q_out, void* k_tree, void* v_tree, hipStream_t st) {
  const double l2t = log2((double)theta);
  if (dt == DDT_BF16)
    hipLaunchKernelGGL((rope_tree_kernel<uint16_t>), dim3(n * T), dim3(256), 0, st,
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_new),
                       static_cast<const uint16_t*>(v_new), depth, prefix_len, T, Hq, Hkv, D, rot, l2t,
                       static_cast<uint16_t*>(q_out), static_cast<uint16_t*>(k_tree), static_cast<uint16_t*>(v_tree));
  else
    hipLaunchKernelGGL((rope_tree_kernel<float>), dim3(n * T), dim3(256), 0, st, static_cast<const float*>(q),
                       static_cast<const float*>(k_new), static_cast<const float*>(v_new), depth, prefix_len, T, Hq,
                       Hkv, D, rot, l2t, static_cast<float*>(q_out), static_cast<float*>(k_tree),
                       static_cast<float*>(v_tree));
  return hipGetLastError();
}

}  // namespace ddt
