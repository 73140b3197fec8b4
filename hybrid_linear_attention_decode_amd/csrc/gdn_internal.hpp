// gdn_internal.hpp -- argument blocks shared by the C-ABI entry points
// (gdn_api.hip) and the kernel launchers (gdn_decode.hip, gdn_slots.hip,
// gdn_prefill.hip, kda_prefill.hip).  Host-visible only; no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// One decode call: T tokens for B requests of one layer.
struct DecodeArgs {
  int32_t Hk, Hv, dv, W, C, G;
  int32_t B, T;
  int32_t tchunk;             // tokens prepared per LDS chunk (1..T)
  int64_t num_slots;
  int32_t silu, l2norm;
  float q_scale, eps;
  float* ssm;                // [slots][Hv][dv][dk]
  void* conv;                // [slots][W-1][C]
  const int32_t* idx;        // [B]
  const int32_t* init;       // [B] or nullptr (= idx): source slot, < 0 = zero start
  const void* x;             // [B*T][C]
  const void* alpha;         // [B*T][Hv] or [B*T][Hv][dk]
  const void* beta;          // [B*T][Hv]
  const void* w;             // [C][W]
  const void* bias;          // [C] or nullptr
  float* out;                // [B*T][Hv][dv]
  float* spec_ssm;           // [B][t_max][Hv][dv][dk] or nullptr
  void* spec_conv;           // [B][t_max][W-1][C]
  const int32_t* spec_slots; // [B][t_max] pool slots taking the snapshots, or nullptr
  int32_t t_max;
  uint32_t* work;            // the caller's work counter (zero between calls), or nullptr
  int32_t nstatic;           // units run by the workgroup of the same index (work given)
  int32_t nticket;           // workgroups that draw a ticket each (work given)
};

// Bulk slot operations (copy, zero, commit of a snapshot).
struct SlotArgs {
  int32_t n;                 // items
  int64_t num_slots;
  int64_t ssm_vec;           // 16-byte vectors per ssm slot
  int64_t conv_vec;          // 16-byte vectors per conv slot
  float* ssm;
  void* conv;
  const int32_t* a;          // copy: src; zero: idx; commit: mamba_pool_indices
  const int32_t* b;          // copy: dst; commit: accepted_len
  const float* spec_ssm;     // commit only
  const void* spec_conv;
  int32_t t_max;
  void* buf;                 // pack / unpack: n items of (ssm slot || conv slot)
};

enum SlotMode { kSlotCopy = 0, kSlotZero = 1, kSlotCommit = 2, kSlotPack = 3, kSlotUnpack = 4 };

// Commit by index (snapshots in pool slots).
struct CommitIndexArgs {
  int32_t B, t_max;
  int64_t num_slots;
  const int32_t* spec_slots;    // [B][t_max]
  const int32_t* accepted_len;  // [B]
  int32_t* idx;                 // [B] mamba_pool_indices, updated
  int32_t* released;            // [B] or nullptr
};

// One chunked prefill call over N sequences.
struct PrefillArgs {
  int32_t Hk, Hv, dv, W, C, G;
  int32_t N;
  int32_t nblk;              // workgroups per (sequence, value head): ceil(dv / 64)
  int32_t total;             // cu_seqlens[N]
  int64_t num_slots;
  int32_t silu, l2norm;
  float q_scale, eps;
  float* ssm;                // [slots][Hv][dv][dk]
  void* conv;                // [slots][W-1][C]
  const int32_t* dst;        // [N]
  const int32_t* init;       // [N] or nullptr (= dst)
  const int32_t* cu;         // [N+1]
  const void* x;             // [total][C]
  const void* alpha;         // [total][Hv] or [total][Hv][dk]
  const void* beta;          // [total][Hv]
  const void* w;             // [C][W]
  const void* bias;          // [C] or nullptr
  float* out;                // [total][Hv][dv]
  void* ws;                  // workspace: prepared q / k rows (scalar decay) or
                             // diagonal-block records (per-channel decay)
  const int32_t* ckpt;       // [N][ckpt_per_seq] checkpoint slots, or nullptr
  int32_t ckpt_every;        // tokens between checkpoints (a multiple of the chunk)
  int32_t ckpt_per_seq;
};

// Launchers: return hipSuccess or the launch error.  The caller has validated
// every host-checkable argument.
hipError_t launch_decode(const DecodeArgs& a, int dk, int act_bf16, int kda, hipStream_t s);
hipError_t launch_slots(const SlotArgs& a, SlotMode mode, hipStream_t s);
hipError_t launch_commit_index(const CommitIndexArgs& a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, int dk, int act_bf16, int max_seqlen,
                          hipStream_t s);
hipError_t launch_prefill_kda(const PrefillArgs& a, int dk, int act_bf16, int max_seqlen,
                              hipStream_t s);
// Workspace bytes of the per-channel-decay prefill for N sequences of total tokens.
size_t kda_workspace_bytes(int Hv, int64_t N, int64_t total);
// Workspace bytes of the scalar-decay prefill: the prepared q / k rows.
size_t qk_workspace_bytes(int Hk, int dk, int64_t total);

// Rows of state per wave of the decode kernel for a shape; 0 when unsupported.
int decode_rows_per_wave(int dk, int G, int dv, int W1, int kda);
// Nonzero when the chunked prefill kernels cover this key width and gate kind.
int prefill_supported(int dk, int kda);

}  // namespace gdn
