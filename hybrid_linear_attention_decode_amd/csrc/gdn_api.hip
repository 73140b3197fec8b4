// gdn_api.hip -- the C ABI of libgdn (declared in include/gdn.h): host-side
// validation of every host-checkable argument, then one asynchronous launch
// on the caller's stream.  Nothing is allocated and no state is kept between
// calls.
#include "gdn.h"
#include "gdn_internal.hpp"

#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

namespace {

using gdn::DecodeArgs;
using gdn::SlotArgs;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t channels(const gdn_layer* L) {
  return 2 * static_cast<int64_t>(L->n_k_heads) * L->d_k +
         static_cast<int64_t>(L->n_v_heads) * L->d_v;
}

size_t act_size(const gdn_layer* L) { return L->act_dtype == GDN_BF16 ? 2 : 4; }

// Largest number of elements of one token's row: conv channels C, H_v d_v
// outputs, H_v d_k per-channel decays.
constexpr int64_t kMaxRowElems = int64_t{1} << 22;

gdn_status check_layer(const gdn_layer* L) {
  if (!L) return GDN_ERR_NULL_ARG;
  if (L->gate != GDN_GATE_SCALAR && L->gate != GDN_GATE_CHANNEL) return GDN_ERR_BAD_DTYPE;
  if (L->act_dtype != GDN_F32 && L->act_dtype != GDN_BF16) return GDN_ERR_BAD_DTYPE;
  if (L->n_k_heads <= 0 || L->n_v_heads <= 0) return GDN_ERR_BAD_SHAPE;
  if (L->n_v_heads % L->n_k_heads) return GDN_ERR_BAD_SHAPE;
  if (L->n_k_heads > 65535) return GDN_ERR_BAD_SHAPE;
  if (L->d_k <= 0 || L->d_v <= 0 || L->conv_width < 1) return GDN_ERR_BAD_SHAPE;
  if (L->flags & ~(GDN_F_CONV_SILU | GDN_F_L2NORM_QK)) return GDN_ERR_BAD_SHAPE;
  if (!(L->l2_eps >= 0.f) || !(L->q_scale == L->q_scale)) return GDN_ERR_BAD_SHAPE;
  if (L->d_k != 16 && L->d_k != 32 && L->d_k != 64 && L->d_k != 128) return GDN_ERR_UNSUPPORTED;
  if (L->d_v % 16 || L->d_v > 256) return GDN_ERR_UNSUPPORTED;
  if (L->conv_width > 4) return GDN_ERR_UNSUPPORTED;
  // the kernels address a token's channels, and a chunk's rows of them, with
  // 32-bit offsets
  if (channels(L) > kMaxRowElems || static_cast<int64_t>(L->n_v_heads) * L->d_k > kMaxRowElems)
    return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

gdn_status check_pool(const gdn_layer* L, const gdn_pool* P) {
  if (!P || !P->ssm) return GDN_ERR_NULL_ARG;
  if (L->conv_width > 1 && !P->conv) return GDN_ERR_NULL_ARG;
  if (P->num_slots < 0 || P->num_slots > INT32_MAX) return GDN_ERR_BAD_SHAPE;
  if (!aligned16(P->ssm) || (P->conv && !aligned16(P->conv))) return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

gdn_status check_spec(const gdn_layer* L, const gdn_spec_cache* S) {
  if (S->t_max < 1) return GDN_ERR_BAD_SHAPE;
  if (S->slots) return GDN_OK;  // snapshots in pool slots
  if (!S->ssm) return GDN_ERR_NULL_ARG;
  if (L->conv_width > 1 && !S->conv) return GDN_ERR_NULL_ARG;
  if (!aligned16(S->ssm) || (S->conv && !aligned16(S->conv))) return GDN_ERR_BAD_SHAPE;
  return GDN_OK;
}

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH; }

// ---- Device-side preconditions, checked only when GDN_DEBUG is set (and not
// "0") in the environment at the time of the call: the index arrays are
// copied to the host on the call's stream (which waits for it) and checked
// before anything is enqueued.

bool debug_checks() {
  const char* e = getenv("GDN_DEBUG");
  return e && e[0] && !(e[0] == '0' && e[1] == 0);
}

// n int32 values of a device array (an empty vector for n <= 0 or no array);
// false when the copy fails.
bool fetch(const int32_t* d, int64_t n, hipStream_t s, std::vector<int32_t>& h) {
  h.clear();
  if (!d || n <= 0) return true;
  h.resize(static_cast<size_t>(n));
  if (hipMemcpyAsync(h.data(), d, static_cast<size_t>(n) * sizeof(int32_t),
                     hipMemcpyDeviceToHost, s) != hipSuccess)
    return false;
  return hipStreamSynchronize(s) == hipSuccess;
}

bool in_pool(int32_t v, int64_t num_slots) { return v >= 0 && v < num_slots; }

// The in-pool entries of a, sorted; false if two are equal.
bool distinct(const std::vector<int32_t>& a, int64_t num_slots, std::vector<int32_t>& sorted) {
  sorted.clear();
  for (int32_t v : a)
    if (in_pool(v, num_slots)) sorted.push_back(v);
  std::sort(sorted.begin(), sorted.end());
  return std::adjacent_find(sorted.begin(), sorted.end()) == sorted.end();
}
bool contains(const std::vector<int32_t>& sorted, int32_t v) {
  return std::binary_search(sorted.begin(), sorted.end(), v);
}

// Rows i of a batch write slot dst[i] (skipped when out of the pool) and read
// slot src[i] (the same when src is empty).  Writes must not collide, and no
// row may read a slot that another row writes.
gdn_status check_rows(const std::vector<int32_t>& dst, const std::vector<int32_t>& src,
                      int64_t num_slots, std::vector<int32_t>& written) {
  if (!distinct(dst, num_slots, written)) return GDN_ERR_PRECONDITION;
  for (size_t i = 0; i < src.size(); ++i) {
    if (!in_pool(dst[i], num_slots) || !in_pool(src[i], num_slots) || src[i] == dst[i]) continue;
    if (contains(written, src[i])) return GDN_ERR_PRECONDITION;
  }
  return GDN_OK;
}

// Extra targets (snapshot or checkpoint slots, -1 = none): distinct, and none
// of them a slot that the rows read or write.
gdn_status check_targets(const std::vector<int32_t>& t, const std::vector<int32_t>& dst,
                         const std::vector<int32_t>& src, int64_t num_slots) {
  std::vector<int32_t> ts;
  if (!distinct(t, num_slots, ts)) return GDN_ERR_PRECONDITION;
  for (size_t i = 0; i < dst.size(); ++i) {
    if (!in_pool(dst[i], num_slots)) continue;
    if (contains(ts, dst[i])) return GDN_ERR_PRECONDITION;
    if (!src.empty() && in_pool(src[i], num_slots) && contains(ts, src[i]))
      return GDN_ERR_PRECONDITION;
  }
  return GDN_OK;
}

SlotArgs slot_args(const gdn_layer* L, const gdn_pool* P, int32_t n) {
  SlotArgs a{};
  a.n = n;
  a.num_slots = P->num_slots;
  a.ssm_vec = static_cast<int64_t>(L->n_v_heads) * L->d_v * L->d_k / 4;
  a.conv_vec = static_cast<int64_t>(L->conv_width - 1) * channels(L) *
               static_cast<int64_t>(act_size(L)) / 16;
  a.ssm = P->ssm;
  a.conv = P->conv;
  return a;
}

size_t slot_bytes(const gdn_layer* L) {
  const gdn_pool dummy{nullptr, nullptr, 1};
  const SlotArgs a = slot_args(L, &dummy, 0);
  return static_cast<size_t>((a.ssm_vec + a.conv_vec) * 16);
}

gdn_status pack_common(const gdn_layer* L, const gdn_pool* P, const int32_t* idx, int32_t n,
                       const void* buffer, size_t buffer_bytes, gdn::SlotMode mode, void* stream) {
  gdn_status st = check_layer(L);
  if (st != GDN_OK) return st;
  if ((st = check_pool(L, P)) != GDN_OK) return st;
  if (n < 0 || n > 65535) return GDN_ERR_BAD_SHAPE;
  if (n == 0) return GDN_OK;
  if (!idx || !buffer) return GDN_ERR_NULL_ARG;
  if (!aligned16(buffer)) return GDN_ERR_BAD_SHAPE;
  if (buffer_bytes / static_cast<size_t>(n) < slot_bytes(L)) return GDN_ERR_BAD_SHAPE;
  if (mode == gdn::kSlotUnpack && debug_checks()) {
    std::vector<int32_t> d, written;
    if (!fetch(idx, n, static_cast<hipStream_t>(stream), d)) return GDN_ERR_LAUNCH;
    if (!distinct(d, P->num_slots, written)) return GDN_ERR_PRECONDITION;
  }
  SlotArgs a = slot_args(L, P, n);
  a.a = idx;
  a.buf = const_cast<void*>(buffer);
  return from_hip(gdn::launch_slots(a, mode, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

const char* gdn_status_string(gdn_status status) {
  // A C caller may pass any int: read it as one (an out-of-range value of
  // the enum type must not be loaded as that type).
  int s = 0;
  memcpy(&s, &status, sizeof(s));
  switch (s) {
    case GDN_OK: return "ok";
    case GDN_ERR_NULL_ARG: return "a required pointer is NULL";
    case GDN_ERR_BAD_SHAPE: return "inconsistent or out-of-range sizes or misaligned pointer";
    case GDN_ERR_BAD_DTYPE: return "unknown dtype or gate kind";
    case GDN_ERR_UNSUPPORTED: return "shape not supported by the built kernels";
    case GDN_ERR_WORKSPACE: return "prefill workspace missing or too small";
    case GDN_ERR_LAUNCH: return "HIP kernel launch failed";
    case GDN_ERR_PRECONDITION:
      return "device-side precondition failed (colliding slots or bad cu_seqlens; GDN_DEBUG)";
  }
  return "unknown status";
}

gdn_status gdn_decode_step(const gdn_layer* L, const gdn_pool* P, const int32_t* idx,
                           const int32_t* init_slot, int32_t B, int32_t T, const gdn_inputs* in,
                           float* out, const gdn_spec_cache* spec, uint32_t* work,
                           void* stream) {
  gdn_status st = check_layer(L);
  if (st != GDN_OK) return st;
  if ((st = check_pool(L, P)) != GDN_OK) return st;
  if (B < 0 || B > 65535 || T < 1) return GDN_ERR_BAD_SHAPE;
  if (!idx || !in || !out) return GDN_ERR_NULL_ARG;
  if (!in->x || !in->alpha || !in->beta || !in->conv_w) return GDN_ERR_NULL_ARG;
  if (spec) {
    if ((st = check_spec(L, spec)) != GDN_OK) return st;
    if (T > spec->t_max) return GDN_ERR_BAD_SHAPE;
  }
  const int G = L->n_v_heads / L->n_k_heads;
  if (!gdn::decode_rows_per_wave(L->d_k, G, L->d_v, L->conv_width - 1,
                                 L->gate == GDN_GATE_CHANNEL))
    return GDN_ERR_UNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(work) & 3u) return GDN_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(B) * L->n_k_heads > INT32_MAX) return GDN_ERR_BAD_SHAPE;
  // a request's T rows of x, out and the decays are addressed with 32-bit offsets
  const int64_t row = std::max({channels(L), static_cast<int64_t>(L->n_v_heads) * L->d_v,
                                static_cast<int64_t>(L->n_v_heads) * L->d_k});
  if (static_cast<int64_t>(T) * row > INT32_MAX) return GDN_ERR_BAD_SHAPE;
  if (B == 0) return GDN_OK;
  if (debug_checks()) {
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    std::vector<int32_t> d, src, tab, written;
    if (!fetch(idx, B, hs, d) || !fetch(init_slot, B, hs, src)) return GDN_ERR_LAUNCH;
    if ((st = check_rows(d, src, P->num_slots, written)) != GDN_OK) return st;
    if (spec && spec->slots) {
      if (!fetch(spec->slots, static_cast<int64_t>(B) * spec->t_max, hs, tab)) return GDN_ERR_LAUNCH;
      std::vector<int32_t> used;  // the snapshot slots of tokens 0..T-1
      for (int32_t b = 0; b < B; ++b)
        if (in_pool(d[b], P->num_slots))
          for (int32_t t = 0; t < T; ++t) used.push_back(tab[static_cast<size_t>(b) * spec->t_max + t]);
      if ((st = check_targets(used, d, src, P->num_slots)) != GDN_OK) return st;
    }
  }

  DecodeArgs a{};
  a.Hk = L->n_k_heads;
  a.Hv = L->n_v_heads;
  a.dv = L->d_v;
  a.W = L->conv_width;
  a.C = static_cast<int32_t>(channels(L));
  a.G = G;
  a.B = B;
  a.T = T;
  a.num_slots = P->num_slots;
  a.silu = (L->flags & GDN_F_CONV_SILU) ? 1 : 0;
  a.l2norm = (L->flags & GDN_F_L2NORM_QK) ? 1 : 0;
  a.q_scale = L->q_scale;
  a.eps = L->l2_eps;
  a.ssm = P->ssm;
  a.conv = P->conv;
  a.idx = idx;
  a.init = init_slot;
  a.x = in->x;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.w = in->conv_w;
  a.bias = in->conv_b;
  a.out = out;
  a.spec_slots = spec ? spec->slots : nullptr;
  a.spec_ssm = spec && !spec->slots ? spec->ssm : nullptr;
  a.spec_conv = spec && !spec->slots ? spec->conv : nullptr;
  a.t_max = spec ? spec->t_max : 0;
  a.work = work;
  return from_hip(gdn::launch_decode(a, L->d_k, L->act_dtype == GDN_BF16,
                                     L->gate == GDN_GATE_CHANNEL,
                                     static_cast<hipStream_t>(stream)));
}

gdn_status gdn_spec_decode_commit(const gdn_layer* L, const gdn_pool* P, const int32_t* idx,
                                  const gdn_spec_cache* spec, const int32_t* accepted_len,
                                  int32_t B, void* stream) {
  gdn_status st = check_layer(L);
  if (st != GDN_OK) return st;
  if ((st = check_pool(L, P)) != GDN_OK) return st;
  if (!spec || !idx || !accepted_len) return GDN_ERR_NULL_ARG;
  if ((st = check_spec(L, spec)) != GDN_OK) return st;
  if (spec->slots) return GDN_ERR_BAD_SHAPE;  // pool-slot snapshots commit by index
  if (B < 0 || B > 65535) return GDN_ERR_BAD_SHAPE;
  if (debug_checks() && B > 0) {
    std::vector<int32_t> d, written;
    if (!fetch(idx, B, static_cast<hipStream_t>(stream), d)) return GDN_ERR_LAUNCH;
    if (!distinct(d, P->num_slots, written)) return GDN_ERR_PRECONDITION;
  }
  SlotArgs a = slot_args(L, P, B);
  a.a = idx;
  a.b = accepted_len;
  a.spec_ssm = spec->ssm;
  a.spec_conv = spec->conv;
  a.t_max = spec->t_max;
  return from_hip(gdn::launch_slots(a, gdn::kSlotCommit, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_spec_commit_index(const gdn_pool* P, const gdn_spec_cache* spec,
                                 const int32_t* accepted_len, int32_t* idx, int32_t* released,
                                 int32_t B, void* stream) {
  if (!P || !spec || !accepted_len || !idx) return GDN_ERR_NULL_ARG;
  if (!spec->slots) return GDN_ERR_NULL_ARG;
  if (spec->t_max < 1 || B < 0 || B > 65535 || P->num_slots < 1) return GDN_ERR_BAD_SHAPE;
  gdn::CommitIndexArgs a{};
  a.B = B;
  a.t_max = spec->t_max;
  a.num_slots = P->num_slots;
  a.spec_slots = spec->slots;
  a.accepted_len = accepted_len;
  a.idx = idx;
  a.released = released;
  return from_hip(gdn::launch_commit_index(a, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_slot_copy(const gdn_layer* L, const gdn_pool* P, const int32_t* src,
                         const int32_t* dst, int32_t n, void* stream) {
  gdn_status st = check_layer(L);
  if (st != GDN_OK) return st;
  if ((st = check_pool(L, P)) != GDN_OK) return st;
  if (n < 0 || n > 65535) return GDN_ERR_BAD_SHAPE;
  if (n > 0 && (!src || !dst)) return GDN_ERR_NULL_ARG;
  if (debug_checks() && n > 0) {
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    std::vector<int32_t> d, sv, written;
    if (!fetch(dst, n, hs, d) || !fetch(src, n, hs, sv)) return GDN_ERR_LAUNCH;
    for (int32_t i = 0; i < n; ++i)  // a row with a source outside the pool is skipped
      if (!in_pool(sv[i], P->num_slots)) d[i] = -1;
    if ((st = check_rows(d, sv, P->num_slots, written)) != GDN_OK) return st;
  }
  SlotArgs a = slot_args(L, P, n);
  a.a = src;
  a.b = dst;
  return from_hip(gdn::launch_slots(a, gdn::kSlotCopy, static_cast<hipStream_t>(stream)));
}

size_t gdn_slot_bytes(const gdn_layer* L) {
  if (check_layer(L) != GDN_OK) return 0;
  return slot_bytes(L);
}


gdn_status gdn_slot_pack(const gdn_layer* L, const gdn_pool* P, const int32_t* idx, int32_t n,
                         void* buffer, size_t buffer_bytes, void* stream) {
  return pack_common(L, P, idx, n, buffer, buffer_bytes, gdn::kSlotPack, stream);
}

gdn_status gdn_slot_unpack(const gdn_layer* L, const gdn_pool* P, const void* buffer,
                           size_t buffer_bytes, const int32_t* idx, int32_t n, void* stream) {
  return pack_common(L, P, idx, n, buffer, buffer_bytes, gdn::kSlotUnpack, stream);
}

gdn_status gdn_slot_zero(const gdn_layer* L, const gdn_pool* P, const int32_t* idx, int32_t n,
                         void* stream) {
  gdn_status st = check_layer(L);
  if (st != GDN_OK) return st;
  if ((st = check_pool(L, P)) != GDN_OK) return st;
  if (n < 0 || n > 65535) return GDN_ERR_BAD_SHAPE;
  if (n > 0 && !idx) return GDN_ERR_NULL_ARG;
  SlotArgs a = slot_args(L, P, n);
  a.a = idx;
  return from_hip(gdn::launch_slots(a, gdn::kSlotZero, static_cast<hipStream_t>(stream)));
}

size_t gdn_prefill_workspace_size(const gdn_layer* L, int32_t N, int32_t max_seqlen,
                                  int32_t total_tokens, int32_t chunk) {
  if (check_layer(L) != GDN_OK || N < 0 || max_seqlen < 0 || total_tokens < 0 || chunk != 64)
    return 0;
  // The scalar-decay prefill stores the prepared q / k rows (computed once
  // per key head); the per-channel one the diagonal blocks of each chunk.
  if (L->gate != GDN_GATE_CHANNEL)
    return gdn::qk_workspace_bytes(L->n_k_heads, L->d_k, total_tokens);
  return gdn::kda_workspace_bytes(L->n_v_heads, N, total_tokens);
}

gdn_status gdn_prefill_chunked(const gdn_layer* L, const gdn_pool* P, const int32_t* dst,
                               const int32_t* init_slot, int32_t N, const int32_t* cu_seqlens,
                               int32_t max_seqlen, int32_t total_tokens, int32_t chunk,
                               const gdn_inputs* in, float* out, const gdn_prefill_ckpt* ckpt,
                               void* workspace, size_t workspace_bytes, void* stream) {
  gdn_status st = check_layer(L);
  if (st != GDN_OK) return st;
  if ((st = check_pool(L, P)) != GDN_OK) return st;
  if (N < 0 || N > 65535 || max_seqlen < 0 || total_tokens < 0) return GDN_ERR_BAD_SHAPE;
  if (chunk != 64) return GDN_ERR_UNSUPPORTED;
  if (!gdn::prefill_supported(L->d_k, L->gate == GDN_GATE_CHANNEL)) return GDN_ERR_UNSUPPORTED;
  const int32_t nblk = (L->d_v + 63) / 64;
  if (static_cast<int64_t>(N) * L->n_v_heads * nblk > INT32_MAX) return GDN_ERR_BAD_SHAPE;
  if (ckpt) {
    if (ckpt->per_seq < 0 || ckpt->per_seq > 65534) return GDN_ERR_BAD_SHAPE;
    if (ckpt->every < 64 || ckpt->every % 64) return GDN_ERR_BAD_SHAPE;
    if (ckpt->per_seq > 0 && !ckpt->slots) return GDN_ERR_NULL_ARG;
  }
  if (N == 0) return GDN_OK;
  if (!dst || !cu_seqlens || !in) return GDN_ERR_NULL_ARG;
  if (total_tokens > 0 && (!in->x || !in->alpha || !in->beta || !in->conv_w || !out))
    return GDN_ERR_NULL_ARG;
  if (in->x && !aligned16(in->x)) return GDN_ERR_BAD_SHAPE;
  if (out && !aligned16(out)) return GDN_ERR_BAD_SHAPE;
  if (debug_checks()) {
    // cu_seqlens: 0, non-decreasing, ending at total_tokens, no sequence
    // longer than max_seqlen; destination writes distinct; no sequence reading
    // a slot another one writes; used checkpoint slots distinct and apart
    // from every destination and source
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    std::vector<int32_t> cu, d, src, tab, written;
    if (!fetch(cu_seqlens, static_cast<int64_t>(N) + 1, hs, cu) || !fetch(dst, N, hs, d) ||
        !fetch(init_slot, N, hs, src))
      return GDN_ERR_LAUNCH;
    if (cu[0] != 0 || cu[N] != total_tokens) return GDN_ERR_PRECONDITION;
    for (int32_t i = 0; i < N; ++i)
      if (cu[i + 1] < cu[i] || cu[i + 1] - cu[i] > max_seqlen) return GDN_ERR_PRECONDITION;
    if ((st = check_rows(d, src, P->num_slots, written)) != GDN_OK) return st;
    if (ckpt && ckpt->per_seq > 0) {
      if (!fetch(ckpt->slots, static_cast<int64_t>(N) * ckpt->per_seq, hs, tab))
        return GDN_ERR_LAUNCH;
      std::vector<int32_t> used;  // checkpoints that fall inside their sequence
      for (int32_t i = 0; i < N; ++i) {
        if (!in_pool(d[i], P->num_slots)) continue;
        const int32_t n_ck = std::min((cu[i + 1] - cu[i]) / ckpt->every, ckpt->per_seq);
        for (int32_t k = 0; k < n_ck; ++k)
          used.push_back(tab[static_cast<size_t>(i) * ckpt->per_seq + k]);
      }
      if ((st = check_targets(used, d, src, P->num_slots)) != GDN_OK) return st;
    }
  }
  const bool kda = L->gate == GDN_GATE_CHANNEL;
  if (kda && total_tokens > 0 && in->alpha && !aligned16(in->alpha)) return GDN_ERR_BAD_SHAPE;
  if (total_tokens > 0) {
    const size_t need = kda ? gdn::kda_workspace_bytes(L->n_v_heads, N, total_tokens)
                            : gdn::qk_workspace_bytes(L->n_k_heads, L->d_k, total_tokens);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255))
      return GDN_ERR_WORKSPACE;
  }

  gdn::PrefillArgs a{};
  a.Hk = L->n_k_heads;
  a.Hv = L->n_v_heads;
  a.dv = L->d_v;
  a.W = L->conv_width;
  a.C = static_cast<int32_t>(channels(L));
  a.G = L->n_v_heads / L->n_k_heads;
  a.N = N;
  a.nblk = nblk;
  a.total = total_tokens;
  a.num_slots = P->num_slots;
  a.silu = (L->flags & GDN_F_CONV_SILU) ? 1 : 0;
  a.l2norm = (L->flags & GDN_F_L2NORM_QK) ? 1 : 0;
  a.q_scale = L->q_scale;
  a.eps = L->l2_eps;
  a.ssm = P->ssm;
  a.conv = P->conv;
  a.dst = dst;
  a.init = init_slot;
  a.cu = cu_seqlens;
  a.x = in->x;
  a.alpha = in->alpha;
  a.beta = in->beta;
  a.w = in->conv_w;
  a.bias = in->conv_b;
  a.out = out;
  a.ws = workspace;
  if (ckpt && ckpt->per_seq > 0) {
    a.ckpt = ckpt->slots;
    a.ckpt_every = ckpt->every;
    a.ckpt_per_seq = ckpt->per_seq;
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (kda)
    return from_hip(gdn::launch_prefill_kda(a, L->d_k, L->act_dtype == GDN_BF16, max_seqlen, hs));
  return from_hip(gdn::launch_prefill(a, L->d_k, L->act_dtype == GDN_BF16, max_seqlen, hs));
}

}  // extern "C"
