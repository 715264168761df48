// Shared device helpers for the gfx950 kernels of libddt.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ddt.h"

namespace ddt {

// ------------------------------------------------------------------ bf16
// bf16 is carried as its 16-bit pattern; conversions are exact (bf16 -> f32) or
// round-to-nearest-even (f32 -> bf16, the hardware conversion of __bf16).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Element access for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, size_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Order-preserving map of a float to uint32: a < b (as floats, no NaN) <=> key(a) < key(b).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------------ wave helpers (wave64)
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), o, 64);
  uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), o, 64);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = shfl_xor_u64(v, o);
    v = w > v ? w : v;
  }
  return v;
}

// Sum over aligned groups of N lanes (N in {4, 8, 16, 32}): every lane of a group ends
// with the group's sum.  Steps inside a 16-lane row are DPP lane moves folded into the
// adds (row rotations, half-row mirror, quad permutations), not LDS round trips; the
// lanes of a group may differ in the last bit (each adds in its own order).
#define DDT_DPP_F32(x, ctrl) \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, (x)), (ctrl), 0xf, 0xf, false))
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group of 4, 8, 16 or 32 lanes");
  if constexpr (N >= 16) {
    x += DDT_DPP_F32(x, 0x128);  // row_ror:8
    x += DDT_DPP_F32(x, 0x124);  // row_ror:4
    x += DDT_DPP_F32(x, 0x122);  // row_ror:2
    x += DDT_DPP_F32(x, 0x121);  // row_ror:1
    if constexpr (N == 32) x += __shfl_xor(x, 16, 64);
  } else {
    if constexpr (N == 8) x += DDT_DPP_F32(x, 0x141);  // row_half_mirror: lane i + lane 7-i
    x += DDT_DPP_F32(x, 0xB1);                         // quad_perm [1,0,3,2]
    x += DDT_DPP_F32(x, 0x4E);                         // quad_perm [2,3,0,1]
  }
  return x;
}

// Wave-uniform maximum of a 64-bit value over all 64 lanes: DPP row rotations inside each
// 16-lane row, then the four row maxima read as scalars (no LDS round trip).
#define DDT_DPP_U32(x, ctrl) static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), (ctrl), 0xf, 0xf, false))
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64_uniform(uint64_t v) {
#define DDT_MAX_STEP(ctrl)                                                                              \
  {                                                                                                     \
    const uint64_t w = (static_cast<uint64_t>(DDT_DPP_U32(static_cast<uint32_t>(v >> 32), ctrl)) << 32) | \
                       DDT_DPP_U32(static_cast<uint32_t>(v), ctrl);                                      \
    v = w > v ? w : v;                                                                                  \
  }
  DDT_MAX_STEP(0x128)  // row_ror:8
  DDT_MAX_STEP(0x124)  // row_ror:4
  DDT_MAX_STEP(0x122)  // row_ror:2
  DDT_MAX_STEP(0x121)  // row_ror:1
#undef DDT_MAX_STEP
  const uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16), c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  const uint64_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

__host__ __device__ constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace ddt
