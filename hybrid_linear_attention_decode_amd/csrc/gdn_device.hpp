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

// Raw buffer accesses (gfx9 descriptor, no stride): an access whose 32-bit
// byte offset lies at or past num_records reads zero or is dropped, which
// masks rows or lanes without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// A byte offset past every descriptor here: its loads read zero.
constexpr uint32_t kOutOfRange = 0x80000000u;

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

constexpr int kDppRowMirror = 0x140;  // lane i <- lane 15-i within 16 lanes

// Lane i <- lane i - N of its row of 16 lanes; lanes without one read zero.
template <int N>
__device__ __forceinline__ float row_shr(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + N, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 4, 8 or 16); every lane of the group
// ends with the same bits (each step adds a commuted pair).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(N == 4 || N == 8 || N == 16, "group of 4, 8 or 16 lanes");
  v = v + dpp<kDppQuadXor1>(v);
  v = v + dpp<kDppQuadXor2>(v);
  if constexpr (N >= 8) v = v + dpp<kDppHalfMirror>(v);
  if constexpr (N == 16) v = v + dpp<kDppRowMirror>(v);
  return v;
}

// Sum over the 64 lanes of a wave: DPP sums inside each row of 16 lanes, then
// the four row sums read into scalars and added in a fixed order, so every
// lane (and every wave summing the same data) gets the same bits.
__device__ __forceinline__ float wave_sum(float v) {
  v = group_sum<16>(v);
  const int iv = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(iv, 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(iv, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(iv, 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(iv, 48));
  return (r0 + r1) + (r2 + r3);
}

// Workgroup barrier for LDS traffic only: this wave's LDS accesses complete,
// then all waves meet.  Unlike __syncthreads() it does not wait for global
// memory, which keeps streaming across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// A value the compiler may keep in a scalar register (it is wave-uniform).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace gdn
