// gdn_device.hpp -- small device helpers for the gfx950 kernels: storage
// types, exact bf16 widening, streaming 16-byte memory ops and wave64
// cross-lane sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f4 __attribute__((ext_vector_type(4)));

// bf16 storage tag: the raw 16 bits, never rounded inside the library.
struct bf16 {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) {
  return __uint_as_float(static_cast<uint32_t>(v.bits) << 16);
}

// Inverse of to_f32 for values that came from the same storage type (conv
// windows hold raw inputs), so the round trip is exact.
template <typename T>
__device__ __forceinline__ T from_exact(float v);
template <>
__device__ __forceinline__ float from_exact<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ bf16 from_exact<bf16>(float v) {
  return bf16{static_cast<uint16_t>(__float_as_uint(v) >> 16)};
}

// Streaming (non-temporal) 16-byte accesses for data touched once per call.
__device__ __forceinline__ f4 ld_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f4*>(p));
}
__device__ __forceinline__ void st_stream(float* p, f4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f4*>(p));
}

// DPP lane permutations inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8 lanes

// Sum over aligned groups of N lanes (N = 4 or 8); every lane of the group
// ends with the same bits (each step adds a commuted pair).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8, "group of 4 or 8 lanes");
  v = v + dpp<kDppQuadXor1>(v);
  v = v + dpp<kDppQuadXor2>(v);
  if constexpr (N == 8) v = v + dpp<kDppHalfMirror>(v);
  return v;
}

// Butterfly sum over the 64 lanes of a wave; identical bits in every lane.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = v + __shfl_xor(v, m, 64);
  return v;
}

}  // namespace gdn
