/*
 * gdn.h -- C ABI of libgdn: the per-request recurrent-state step of the
 * linear-attention layers of hybrid models (Gated DeltaNet, and the KDA
 * variant with a per-key-channel gate), on AMD Instinct MI355X (gfx950).
 *
 * What the calls compute.  For every request b with slot s = mamba_pool_indices[b]
 * and every token t:
 *   1. causal depthwise conv update of the conv window of slot s:
 *        win = (conv[s][0..W-2][c], x_t[c]),  y_c = sum_j conv_w[c][j] win[j] (+ conv_b[c]),
 *        conv[s] <- win[1..W-1],  a = SiLU(y)               (GDN_F_CONV_SILU)
 *   2. head prep: a = q | k | v (head-major), q^ = q (|q|^2+eps)^-1/2 q_scale,
 *      k^ = k (|k|^2+eps)^-1/2 (GDN_F_L2NORM_QK); value head h reads key head
 *      h / (H_v/H_k);
 *   3. gated delta rule, in place on the fp32 state S (d_v x d_k) of slot s:
 *        S' = alpha S (GDN)  or  S' = S diag(alpha) (KDA, alpha in R^{d_k}),
 *        u = beta (v - S' k^),  S <- S' + u k^T,  o = S q^
 *      i.e. S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *      o_t = S_t q_t.
 * The pages behind this library name the layers (Gated DeltaNet in Qwen3.5,
 * KDA in Kimi K3) and describe the state machinery these calls serve, but
 * print no formula:
 *   - aitujian.cn, "TokenSpeed" AICon talk, section "Why agentic inference
 *     needs a new engine": the context of these layers is a continuously
 *     iterated SSM state plus a conv state that must be updated, saved and
 *     restored;
 *   - "TokenSpeed alcanza 580 tps con Qwen3.5-397B-A17B en GPU", section
 *     "Scheduler dual": per-request mamba_pool_indices, state updated in place
 *     every decode step, a spec_cache of per-speculative-step Conv/SSM
 *     snapshots for rollback, prefill populating the state;
 *   - same page, section "Ciclo de vida de slots": working vs checkpoint slots;
 *   - same page, section "Riesgo de correctitud: estado obsoleto": the slot
 *     allocator never clears memory, so a fresh working slot is safe only by
 *     copy-on-write from a clean checkpoint or by explicit zeroing.
 *
 * Conventions for every entry point.
 *   - Pointers are DEVICE pointers unless marked (host).  The caller owns and
 *     allocates every buffer; the library allocates nothing, keeps no state
 *     between calls and is safe to call from several host threads, on any
 *     streams (hipStreamPerThread included) and under graph capture.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Returning GDN_OK means "validated and enqueued".
 *   - Host-checkable errors (NULL pointers, shapes, dtypes, unsupported sizes,
 *     T > t_max, workspace too small) return a GDN_ERR_* code with nothing
 *     enqueued.  A failed launch returns GDN_ERR_LAUNCH.
 *   - Device-resident indices are not range-checked on the host.  A slot index
 *     < 0 or >= num_slots skips that row (no read, no write, output untouched);
 *     an accepted length outside [0, t_max] is treated as 0.  Destination slots
 *     of one call must be distinct (two rows updating one slot race), no row
 *     may read a slot that another row of the call writes, and snapshot /
 *     checkpoint slots must be distinct and apart from both.
 *   - With the environment variable GDN_DEBUG set (and not "0") at the time of
 *     a call, the call first copies its device index arrays (and cu_seqlens)
 *     to the host on `stream`, waiting for the stream, and returns
 *     GDN_ERR_PRECONDITION with nothing enqueued if any of the rules above or
 *     the cu_seqlens contract is broken.  For debugging only: it synchronises.
 *   - `out` must not alias any input or either pool.
 *
 * Layouts (row-major; act = gdn_layer.act_dtype, C = 2 H_k d_k + H_v d_v):
 *   pool.ssm   [num_slots][H_v][d_v][d_k] fp32  (row = value index, contiguous
 *                                                over key index)
 *   pool.conv  [num_slots][W-1][C]        act   (oldest input first)
 *   x          [rows][C]                  act   (channel order q | k | v)
 *   alpha      [rows][H_v]  or  [rows][H_v][d_k] (KDA)   act, values in (0, 1]
 *   beta       [rows][H_v]                act
 *   conv_w     [C][W] act;  conv_b [C] act or NULL
 *   out        [rows][H_v][d_v]           fp32
 *   spec.ssm   [B][t_max][H_v][d_v][d_k]  fp32;  spec.conv [B][t_max][W-1][C] act
 * Decode rows are b*T + t; prefill rows are token positions given by cu_seqlens.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL_ARG = 1,    /* a required pointer is NULL */
  GDN_ERR_BAD_SHAPE = 2,   /* inconsistent or out-of-range sizes */
  GDN_ERR_BAD_DTYPE = 3,   /* unknown dtype / gate enum */
  GDN_ERR_UNSUPPORTED = 4, /* valid but not built (e.g. d_k not in {16,32,64,128}) */
  GDN_ERR_WORKSPACE = 5,   /* prefill workspace missing or too small */
  GDN_ERR_LAUNCH = 6,      /* the HIP launch failed */
  GDN_ERR_PRECONDITION = 7 /* a device-side precondition failed (only with GDN_DEBUG set) */
} gdn_status;

typedef enum { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

typedef enum {
  GDN_GATE_SCALAR = 0, /* GDN: one alpha per (token, value head) */
  GDN_GATE_CHANNEL = 1 /* KDA: alpha[d_k] per (token, value head) */
} gdn_gate;

enum {
  GDN_F_CONV_SILU = 1u << 0, /* SiLU after the conv */
  GDN_F_L2NORM_QK = 1u << 1  /* L2-normalise q and k per head */
};

/* (host) layer description.  The conv channels C = 2 H_k d_k + H_v d_v and
 * H_v d_k are at most 2^22 (else GDN_ERR_BAD_SHAPE from every entry point). */
typedef struct {
  int32_t n_k_heads, n_v_heads; /* H_v % H_k == 0 */
  int32_t d_k, d_v;             /* d_k in {16, 32, 64, 128}; d_v a multiple of 16, <= 256 */
  int32_t conv_width;           /* W in 1..4; W == 1 means no conv state */
  int32_t gate;                 /* gdn_gate */
  int32_t act_dtype;            /* gdn_dtype of x, alpha, beta, conv_w, conv_b, conv state */
  uint32_t flags;               /* GDN_F_* */
  float q_scale;                /* usually 1/sqrt(d_k) */
  float l2_eps;                 /* usually 1e-6 */
} gdn_layer;

/* (host) struct of device pointers: the state pools */
typedef struct {
  float* ssm;
  void* conv; /* may be NULL when conv_width == 1 */
  int64_t num_slots;
} gdn_pool;

/* (host) struct of device pointers: per-draft-token snapshots, either in
 * their own buffers (ssm [B][t_max][H_v][d_v][d_k], conv [B][t_max][W-1][C])
 * or, when slots != NULL, in pool slots: slots [B][t_max] int32 names the
 * pool slot (both pools) that receives the snapshot of request b after draft
 * token t (ssm and conv are then ignored; an entry outside the pool drops
 * that snapshot).  Snapshot slots must be distinct and must not be any
 * request's working or source slot. */
typedef struct {
  float* ssm;
  void* conv;
  int32_t t_max;
  const int32_t* slots;
} gdn_spec_cache;

/* (host) struct of device pointers: per-token inputs */
typedef struct {
  const void* x;
  const void* alpha;
  const void* beta;
  const void* conv_w;
  const void* conv_b; /* NULL: no bias */
} gdn_inputs;

/*
 * Decode T >= 1 tokens per request ("Scheduler dual": the state of the slot
 * named by mamba_pool_indices is updated in place every decode step; with a
 * spec cache, per-speculative-step Conv/SSM snapshots are kept for rollback).
 * One workgroup per (request, key head) unit.  With G = H_v / H_k, the
 * unit's G * d_v state rows go to w <= 8 waves of r rows each, r in {32, 16,
 * 8} dividing d_v and a multiple of 4 (d_k >= 64) or of 256 / d_k, and the
 * workgroup's 64 w threads must cover the 2 d_k + G d_v conv channels and the
 * G (scalar decay) or G d_k (KDA) gate values plus G betas; a shape with no
 * such r returns GDN_ERR_UNSUPPORTED before anything is enqueued (the
 * Qwen3.5 and KDA shapes: r = 32 and 16, 8 waves).
 *   mamba_pool_indices [B] int32 (device); B >= 0; 1 <= T, with T C, T H_v d_v
 *     and T H_v d_k at most 2^31 - 1 (else GDN_ERR_BAD_SHAPE).
 *   init_slot [B] int32 (device) or NULL -- slot preparation fused into the
 *     step ("Riesgo de correctitud": a fresh working slot must start clean):
 *     NULL or init_slot[b] == mamba_pool_indices[b]: start from the slot
 *     itself; init_slot[b] < 0: start from zero state and zero conv window
 *     (nothing read); any other s: copy-on-write, start from slot s (only
 *     read) and write the working slot.  s >= num_slots skips the row.
 *   out [B][T][H_v][d_v] fp32: o_t for every token.
 *   spec == NULL: conv and ssm of each working slot are written after T tokens.
 *   spec != NULL: T <= spec->t_max; the state after token t (0-based) goes to
 *     snapshot t of request b (see gdn_spec_cache); working slots are not
 *     written.
 *   work: NULL, or one uint32 word of device memory owned by the caller,
 *     zero before its first use; every call leaves it at zero.  With it the
 *     last quarter of the units is handed out at run time (an atomic ticket
 *     per workgroup), so the XCDs that stream faster take more of the tail;
 *     without it every unit has a fixed workgroup.  Calls that may run at the
 *     same time (on different streams, or graph replays beside other work)
 *     need distinct words; calls on one stream may share one.
 */
gdn_status gdn_decode_step(const gdn_layer* layer, const gdn_pool* pool,
                           const int32_t* mamba_pool_indices, const int32_t* init_slot,
                           int32_t B, int32_t T, const gdn_inputs* in, float* out,
                           const gdn_spec_cache* spec, uint32_t* work, void* stream);

/*
 * Rollback / commit after verification ("Scheduler dual": rollback from the
 * spec_cache when verification fails).  For each b with L = accepted_len[b]:
 * L > 0 copies snapshot L-1 (ssm and conv) into slot mamba_pool_indices[b];
 * L == 0 leaves the slot as it was before the draft.  Bitwise copy.
 *   accepted_len [B] int32 (device), each in [0, spec->t_max].
 *   spec->slots must be NULL (snapshots in pool slots commit by index).
 */
gdn_status gdn_spec_decode_commit(const gdn_layer* layer, const gdn_pool* pool,
                                  const int32_t* mamba_pool_indices,
                                  const gdn_spec_cache* spec, const int32_t* accepted_len,
                                  int32_t B, void* stream);

/* (host) checkpoints a prefill emits on the way (mechatronicstore.cl note,
 * section on slot lifecycles: checkpoint slots at block-aligned positions for
 * prefix reuse): slots [N][per_seq] int32 (device); checkpoint k of sequence
 * s is the state (ssm and conv window) after its first (k+1)*every tokens,
 * written to pool slot slots[s][k] when (k+1)*every <= the sequence's
 * length; entries outside the pool are skipped.  every is a multiple of the
 * chunk (64).  Checkpoint slots must be distinct and must not be any
 * sequence's destination or initial slot. */
typedef struct {
  const int32_t* slots;
  int32_t every;
  int32_t per_seq;
} gdn_prefill_ckpt;

/*
 * Chunked prefill of N variable-length sequences ("Scheduler dual": prefill
 * populates the initial state; "Riesgo de correctitud": a fresh working slot
 * starts from a clean checkpoint copy or from zeros).  Both gate kinds: the
 * scalar decay (GDN) and the per-channel decay (KDA, the fine-grained gate of
 * the Kimi K3 layers the pages name).
 *   dst_slots [N] int32 (device): the working slot each sequence writes.
 *   init_slot [N] int32 (device) or NULL: -1 = start from zero state and zero
 *     conv window; s >= 0 = start from slot s (s == dst continues in place,
 *     any other s is a copy-on-write source that is only read).  NULL means
 *     init_slot == dst_slots.  No init slot may be another sequence's dst.
 *   cu_seqlens [N+1] int32 (device), cu_seqlens[0] == 0, non-decreasing;
 *     max_seqlen (host) >= every length (it sizes a launch grid; a smaller
 *     value stays correct, only slower); total_tokens (host) == cu_seqlens[N].
 *   chunk: 64, the only value accepted: the granularity of checkpoints (the
 *     scalar-decay kernel steps through 32-token blocks internally; results
 *     do not depend on it beyond rounding).  d_k in {16, 32, 64, 128}
 *     (16 runs in the d_k = 32 layout, its upper channels zero padding).
 *   in->alpha: [total][H_v] (scalar decay) or [total][H_v][d_k] (per-channel
 *     decay, 16-byte aligned).
 *   out [total][H_v][d_v] fp32.
 *   ckpt: NULL, or the checkpoints to emit (gdn_prefill_ckpt).  A later
 *     prefill that starts from a checkpoint (init_slot = its slot) continues
 *     the sequence bit for bit.
 *   workspace: device scratch of at least gdn_prefill_workspace_size() bytes,
 *     256-byte aligned, owned by the caller and free again when the call's
 *     stream work has finished.  The scalar decay stores there the
 *     normalised q and k rows (conv, SiLU, L2 norm; split into two bf16
 *     halves), computed once per key head by a first kernel; the per-channel
 *     decay its diagonal blocks.  Missing, short or misaligned (with
 *     total_tokens > 0): GDN_ERR_WORKSPACE, nothing enqueued.
 */
gdn_status gdn_prefill_chunked(const gdn_layer* layer, const gdn_pool* pool,
                               const int32_t* dst_slots, const int32_t* init_slot, int32_t N,
                               const int32_t* cu_seqlens, int32_t max_seqlen,
                               int32_t total_tokens, int32_t chunk, const gdn_inputs* in,
                               float* out, const gdn_prefill_ckpt* ckpt, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Chunked prefill that allocates nothing, for callers that cannot allocate
 * device memory (code under graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): gdn_prefill_chunked with the same arguments except
 * the workspace, which is a device array of GDN_PREFILL_STATIC_BYTES inside
 * the library -- one per GPU the library runs on, held until the process
 * ends.  A call that would need more workspace than that
 * (gdn_prefill_workspace_size) returns GDN_ERR_WORKSPACE with nothing
 * enqueued; GDN_ERR_LAUNCH if the array's address cannot be looked up.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (different streams, graph replays beside other work) race and
 * must not be issued.  The array keeps the last call's contents; nothing in
 * it needs to start at zero.  64 MiB holds, e.g., the scalar-decay workspace
 * of 4096 tokens of a 16-key-head, d_k = 128 layer (16 KiB per token).
 */
#define GDN_PREFILL_STATIC_BYTES (64u * 1024u * 1024u)
gdn_status gdn_prefill_chunked_static(const gdn_layer* layer, const gdn_pool* pool,
                                      const int32_t* dst_slots, const int32_t* init_slot,
                                      int32_t N, const int32_t* cu_seqlens, int32_t max_seqlen,
                                      int32_t total_tokens, int32_t chunk, const gdn_inputs* in,
                                      float* out, const gdn_prefill_ckpt* ckpt, void* stream);

/* Bytes of workspace gdn_prefill_chunked needs for these sizes: for the
 * scalar decay 8 * total * H_k * d_k; for the per-channel decay 2048 * H_v *
 * (floor(total/16) + 4 * min(N, total)).  0 on bad arguments. */
size_t gdn_prefill_workspace_size(const gdn_layer* layer, int32_t N, int32_t max_seqlen,
                                  int32_t total_tokens, int32_t chunk);

/*
 * Commit by index, for snapshots kept in pool slots (talk page, section
 * "Kernel：让 MLA 真正跑满 GPU", on linear models: at a cut-off an index moves,
 * not the state block): for each b with L =
 * accepted_len[b] in [1, t_max] and s = spec->slots[b][L-1] inside the pool,
 * mamba_pool_indices[b] <- s; nothing is copied.  released [B] (device) or
 * NULL receives the slot each request no longer references (its previous
 * working slot), or -1 where nothing changed; the caller returns released
 * and rejected snapshot slots to its free list.
 */
gdn_status gdn_spec_commit_index(const gdn_pool* pool, const gdn_spec_cache* spec,
                                 const int32_t* accepted_len, int32_t* mamba_pool_indices,
                                 int32_t* released, int32_t B, void* stream);

/*
 * Copy-on-write of n slots ("Riesgo de correctitud": a fresh working slot is
 * made clean by copying a known-clean checkpoint): dst[i] <- src[i], both
 * pools, bitwise.  src / dst [n] int32 (device).  The dst slots must be
 * distinct and must not appear among the src slots.
 */
gdn_status gdn_slot_copy(const gdn_layer* layer, const gdn_pool* pool, const int32_t* src,
                         const int32_t* dst, int32_t n, void* stream);

/*
 * Explicit zeroing of n slots ("Riesgo de correctitud": the other way to make
 * a fresh working slot clean): ssm and conv rows <- +0.0.  idx [n] (device).
 */
gdn_status gdn_slot_zero(const gdn_layer* layer, const gdn_pool* pool, const int32_t* idx,
                         int32_t n, void* stream);

/*
 * Slot pack / unpack: the local half of moving working state between engines
 * (mechatronicstore.cl note, section on prefill / decode disaggregation: slot
 * indices become byte offsets become contiguous blocks).  A packed item is
 * one slot's ssm bytes followed by its conv bytes, bitwise, gdn_slot_bytes()
 * long; item i of the buffer is slot idx[i].
 *   pack: buffer[i] <- slot idx[i];  unpack: slot idx[i] <- buffer[i].
 *   idx [n] int32 (device); an index outside the pool skips its item (the
 *   buffer item, or the slot, is left as it was).  buffer (device, 16-byte
 *   aligned) holds at least n * gdn_slot_bytes() bytes, else
 *   GDN_ERR_BAD_SHAPE.  Unpack targets must be distinct.
 */
size_t gdn_slot_bytes(const gdn_layer* layer);
gdn_status gdn_slot_pack(const gdn_layer* layer, const gdn_pool* pool, const int32_t* idx,
                         int32_t n, void* buffer, size_t buffer_bytes, void* stream);
gdn_status gdn_slot_unpack(const gdn_layer* layer, const gdn_pool* pool, const void* buffer,
                           size_t buffer_bytes, const int32_t* idx, int32_t n, void* stream);

/* Static string for a status code (never NULL). */
const char* gdn_status_string(gdn_status status);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
