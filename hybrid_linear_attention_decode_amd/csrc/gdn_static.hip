// gdn_static.hip -- gdn_prefill_chunked_static: the chunked prefill for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  Its workspace is a
// file-scope device array of GDN_PREFILL_STATIC_BYTES, one copy per GPU the
// library runs on, held until the process ends; the call allocates nothing.
//
// In host code the array's name stands for a host-side symbol, not a device
// address, so it is never passed to a kernel or a copy: on the first call on
// each device (with that device current) its device address is looked up
// with hipGetSymbolAddress and kept per device, and that address is what the
// prefill kernels get as their workspace.
#include <mutex>

#include "gdn.h"
#include <hip/hip_runtime.h>

namespace {

__device__ __align__(256) unsigned char scratch[GDN_PREFILL_STATIC_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (null: not yet)

// The scratch array's device address on the current device, or null.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_chunked_static(const gdn_layer* layer, const gdn_pool* pool,
                                      const int32_t* dst_slots, const int32_t* init_slot,
                                      int32_t N, const int32_t* cu_seqlens, int32_t max_seqlen,
                                      int32_t total_tokens, int32_t chunk, const gdn_inputs* in,
                                      float* out, const gdn_prefill_ckpt* ckpt, void* stream) {
  // A call the workspace array cannot hold is refused before anything else
  // (bad arguments make the size query return 0; the prefill itself then
  // reports them).
  const size_t need = gdn_prefill_workspace_size(layer, N, max_seqlen, total_tokens, chunk);
  if (need > static_cast<size_t>(GDN_PREFILL_STATIC_BYTES)) return GDN_ERR_WORKSPACE;
  void* ws = nullptr;
  if (total_tokens > 0 && need > 0) {
    ws = scratch_ptr();
    if (!ws) return GDN_ERR_LAUNCH;
  }
  return gdn_prefill_chunked(layer, pool, dst_slots, init_slot, N, cu_seqlens, max_seqlen,
                             total_tokens, chunk, in, out, ckpt, ws,
                             ws ? static_cast<size_t>(GDN_PREFILL_STATIC_BYTES) : 0, stream);
}

}  // extern "C"
