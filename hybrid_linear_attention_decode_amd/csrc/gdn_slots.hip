// gdn_slots.hip -- bulk slot operations on both state pools: copy-on-write
// (dst <- src), explicit zeroing, and the speculative commit (slot <- the
// snapshot of the last accepted draft token).  All are bitwise 16-byte
// streaming copies; one workgroup moves a contiguous 16 KiB piece of one
// item's ssm slot followed by its conv slot.  When the snapshots themselves
// live in pool slots, the commit is an index update (commit_index_kernel).
// Pack / unpack move slots to and from a contiguous buffer of (ssm || conv)
// items, bitwise -- the local half of moving state between engines.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kThreads = 256;
constexpr int kVecPerThread = 4;
constexpr int64_t kVecPerBlock = kThreads * kVecPerThread;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u4 ld_u4(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u4*>(p));
}
__device__ __forceinline__ void st_u4(void* p, u4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u4*>(p));
}

template <int MODE>
__global__ void __launch_bounds__(kThreads) slot_kernel(const SlotArgs a) {
  const int item = blockIdx.y;
  const int32_t ia = a.a[item];
  int32_t dst = -1;
  const char* src_ssm = nullptr;
  const char* src_conv = nullptr;
  const int64_t ssm_bytes = a.ssm_vec * 16;
  const int64_t conv_bytes = a.conv_vec * 16;
  if (MODE == kSlotCopy) {
    const int32_t ib = a.b[item];
    if (ia < 0 || ia >= a.num_slots || ib < 0 || ib >= a.num_slots) return;
    dst = ib;
    src_ssm = reinterpret_cast<const char*>(a.ssm) + ia * ssm_bytes;
    src_conv = static_cast<const char*>(a.conv) + ia * conv_bytes;
  } else if (MODE == kSlotZero) {
    if (ia < 0 || ia >= a.num_slots) return;
    dst = ia;
  } else if (MODE == kSlotCommit) {  // item = request, a = slots, b = accepted lengths
    const int32_t L = a.b[item];
    if (ia < 0 || ia >= a.num_slots || L < 1 || L > a.t_max) return;
    dst = ia;
    const int64_t row = static_cast<int64_t>(item) * a.t_max + (L - 1);
    src_ssm = reinterpret_cast<const char*>(a.spec_ssm) + row * ssm_bytes;
    src_conv = static_cast<const char*>(a.spec_conv) + row * conv_bytes;
  } else {  // pack / unpack: item i of the buffer <-> slot a[i]
    if (ia < 0 || ia >= a.num_slots) return;
    char* packed = static_cast<char*>(a.buf) + item * (ssm_bytes + conv_bytes);
    if (MODE == kSlotPack) {
      src_ssm = reinterpret_cast<const char*>(a.ssm) + ia * ssm_bytes;
      src_conv = static_cast<const char*>(a.conv) + ia * conv_bytes;
    } else {
      src_ssm = packed;
      src_conv = packed + ssm_bytes;
      dst = ia;
    }
  }
  char* dst_ssm;
  char* dst_conv;
  if (MODE == kSlotPack) {
    dst_ssm = static_cast<char*>(a.buf) + item * (ssm_bytes + conv_bytes);
    dst_conv = dst_ssm + ssm_bytes;
  } else {
    dst_ssm = reinterpret_cast<char*>(a.ssm) + dst * ssm_bytes;
    dst_conv = static_cast<char*>(a.conv) + dst * conv_bytes;
  }

  const int64_t v0 = static_cast<int64_t>(blockIdx.x) * kVecPerBlock;
  const int64_t total = a.ssm_vec + a.conv_vec;
  u4 buf[kVecPerThread];
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    const int64_t v = v0 + k * kThreads + threadIdx.x;
    buf[k] = u4{0u, 0u, 0u, 0u};
    if (MODE != kSlotZero && v < total)
      buf[k] = v < a.ssm_vec ? ld_u4(src_ssm + v * 16) : ld_u4(src_conv + (v - a.ssm_vec) * 16);
  }
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k) {
    const int64_t v = v0 + k * kThreads + threadIdx.x;
    if (v < total) {
      if (v < a.ssm_vec)
        st_u4(dst_ssm + v * 16, buf[k]);
      else
        st_u4(dst_conv + (v - a.ssm_vec) * 16, buf[k]);
    }
  }
}

// Commit by index: request b's working slot becomes the pool slot holding
// the snapshot of its last accepted draft token; nothing is copied.
__global__ void __launch_bounds__(kThreads) commit_index_kernel(const CommitIndexArgs a) {
  const int b = blockIdx.x * kThreads + threadIdx.x;
  if (b >= a.B) return;
  const int32_t L = a.accepted_len[b];
  int32_t out = -1;
  if (L >= 1 && L <= a.t_max) {
    const int32_t ns = a.spec_slots[static_cast<int64_t>(b) * a.t_max + (L - 1)];
    if (ns >= 0 && ns < a.num_slots) {
      out = a.idx[b];
      a.idx[b] = ns;
    }
  }
  if (a.released) a.released[b] = out;
}

}  // namespace

hipError_t launch_commit_index(const CommitIndexArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(commit_index_kernel, dim3((a.B + kThreads - 1) / kThreads), dim3(kThreads),
                     0, s, a);
  return hipGetLastError();
}

hipError_t launch_slots(const SlotArgs& a, SlotMode mode, hipStream_t s) {
  if (a.n <= 0) return hipSuccess;
  const int64_t total = a.ssm_vec + a.conv_vec;
  const dim3 grid(static_cast<unsigned>((total + kVecPerBlock - 1) / kVecPerBlock), a.n);
  switch (mode) {
    case kSlotCopy:
      hipLaunchKernelGGL(slot_kernel<kSlotCopy>, grid, dim3(kThreads), 0, s, a);
      break;
    case kSlotZero:
      hipLaunchKernelGGL(slot_kernel<kSlotZero>, grid, dim3(kThreads), 0, s, a);
      break;
    case kSlotCommit:
      hipLaunchKernelGGL(slot_kernel<kSlotCommit>, grid, dim3(kThreads), 0, s, a);
      break;
    case kSlotPack:
      hipLaunchKernelGGL(slot_kernel<kSlotPack>, grid, dim3(kThreads), 0, s, a);
      break;
    case kSlotUnpack:
      hipLaunchKernelGGL(slot_kernel<kSlotUnpack>, grid, dim3(kThreads), 0, s, a);
      break;
  }
  return hipGetLastError();
}

}  // namespace gdn
