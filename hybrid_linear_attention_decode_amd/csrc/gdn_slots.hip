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
constexpr uint32_t kPieceBytes = kVecPerBlock * 16;

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Workgroup (x, item): piece x of the item's ssm slot for x < the ssm
// pieces, else a piece of its conv slot.  Every access is a buffer access
// over the piece's segment, so the tail of a segment reads zero and drops its
// stores with no per-vector branch, and all loads of a thread are in flight
// together.
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

  // this workgroup's piece: segment, byte offset in it, bytes left in it
  const int64_t ssm_pieces = (ssm_bytes + kPieceBytes - 1) / kPieceBytes;
  const int64_t x = blockIdx.x;
  const bool in_ssm = x < ssm_pieces;
  const int64_t off = (in_ssm ? x : x - ssm_pieces) * kPieceBytes;
  const int64_t seg = in_ssm ? ssm_bytes : conv_bytes;
  if (off >= seg) return;
  const uint32_t n = static_cast<uint32_t>(seg - off < kPieceBytes ? seg - off : kPieceBytes);
  const rsrc_t d = make_rsrc((in_ssm ? dst_ssm : dst_conv) + off, n);
  u4 buf[kVecPerThread];
  if (MODE == kSlotZero) {
#pragma unroll
    for (int k = 0; k < kVecPerThread; ++k) buf[k] = u4{0u, 0u, 0u, 0u};
  } else {
    const rsrc_t s = make_rsrc((in_ssm ? src_ssm : src_conv) + off, n);
#pragma unroll
    for (int k = 0; k < kVecPerThread; ++k)
      buf[k] = __builtin_amdgcn_raw_buffer_load_b128(s, (k * kThreads + threadIdx.x) * 16u, 0,
                                                     2 /* non-temporal */);
  }
#pragma unroll
  for (int k = 0; k < kVecPerThread; ++k)
    __builtin_amdgcn_raw_buffer_store_b128(buf[k], d, (k * kThreads + threadIdx.x) * 16u, 0,
                                           2 /* non-temporal */);
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
  const int64_t pieces = (a.ssm_vec + kVecPerBlock - 1) / kVecPerBlock +
                         (a.conv_vec + kVecPerBlock - 1) / kVecPerBlock;
  const dim3 grid(static_cast<unsigned>(pieces), a.n);
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
