/*
 * gdn_oracle.h -- plain fp64 CPU oracle for the gated-delta-rule state step.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the checker, not the product:
 * only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load or call it.  It shares no code, header, table or helper with the HIP
 * library (hybrid_linear_attention_decode_amd/csrc) and never includes it.
 *
 * What it computes (sources: "TokenSpeed alcanza 580 tps con Qwen3.5-397B-A17B
 * en GPU", sections "Scheduler dual" and "Riesgo de correctitud: estado
 * obsoleto" for the slot / snapshot / rollback semantics; the recurrence
 * itself is the gated delta rule
 *     S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * which the pages name (Gated DeltaNet in Qwen3.5, KDA in Kimi K3:
 * aitujian.cn talk, section "Why agentic inference needs a new engine") but
 * never write out; the readings taken where they are silent are listed in the
 * design notes of the repository):
 *
 *   D1 conv update, per channel c and token t:
 *        win = (state[0..W-2][c], x_t[c]),  y = sum_j w[c][j] win[j] + b[c],
 *        state <- win[1..W-1] (newest last),  a = SiLU(y) when enabled.
 *   D2 head prep: a is split q | k | v (head-major); q^ = q / sqrt(|q|^2+eps)
 *        * q_scale, k^ = k / sqrt(|k|^2+eps) when L2 normalisation is on;
 *        value head h reads key head floor(h / (H_v/H_k)).
 *   D3 GDN step (scalar alpha per value head):
 *        S' = alpha S;  p = S' k^;  u = beta (v - p);  S <- S' + u k^T;
 *        o = S q^.
 *   D4 KDA step: as D3 with S' = S diag(alpha), alpha in R^{d_k}.
 *   D5 multi-token / speculative: D1-D4 for t = 1..T in order; snapshot t
 *        is (S, conv window) after token t; commit(L) makes the working slot
 *        equal to snapshot L (unchanged when L = 0).
 *   D6 slot copy / zero of both pools.
 *   D7 prefill: the D1-D4 recurrence token by token over each sequence from
 *        the initial slot (or zeros); final S and conv window go to the
 *        destination slot.  This is the authority for the chunked form.
 *   D8 chunked prefill in fp64 (WY/UT-transform form, GDN gate only): a
 *        self-check of the chunk algebra, never the authority.
 *
 * Layouts (row-major, all fp64 here):
 *   ssm  [num_slots][H_v][d_v][d_k]      conv [num_slots][W-1][C]
 *   x    [rows][C],  C = 2 H_k d_k + H_v d_v, channel order q | k | v
 *   alpha [rows][H_v] (GDN) or [rows][H_v][d_k] (KDA);  beta [rows][H_v]
 *   out  [rows][H_v][d_v]
 *   spec_ssm [B][t_max][H_v][d_v][d_k],  spec_conv [B][t_max][W-1][C]
 * Decode rows are b*T + t; prefill rows are token positions (cu_seqlens).
 *
 * Return value of every entry point: 0 on success, negative on bad arguments.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_k_heads, n_v_heads; /* H_v % H_k == 0 */
  int32_t d_k, d_v;
  int32_t conv_width;           /* W >= 1 */
  int32_t gate;                 /* 0: scalar alpha (GDN), 1: alpha[d_k] (KDA) */
  int32_t conv_silu;            /* SiLU after the conv */
  int32_t l2norm;               /* L2-normalise q and k */
  double q_scale;
  double eps;
} orc_layer;

int orc_decode(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
               const int32_t* mamba_pool_indices, int32_t B, int32_t T,
               const double* x, const double* alpha, const double* beta,
               const double* conv_w, const double* conv_b,
               double* out, double* spec_ssm, double* spec_conv, int32_t t_max,
               int32_t nthreads);

int orc_spec_commit(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                    const int32_t* mamba_pool_indices, const double* spec_ssm,
                    const double* spec_conv, int32_t t_max,
                    const int32_t* accepted_len, int32_t B);

int orc_slot_copy(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                  const int32_t* src, const int32_t* dst, int32_t n);

int orc_slot_zero(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                  const int32_t* idx, int32_t n);

int orc_prefill(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                const int32_t* dst, const int32_t* init_slot, int32_t N,
                const int32_t* cu_seqlens, const double* x, const double* alpha,
                const double* beta, const double* conv_w, const double* conv_b,
                double* out, int32_t nthreads);

int orc_prefill_chunked(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                        const int32_t* dst, const int32_t* init_slot, int32_t N,
                        const int32_t* cu_seqlens, int32_t chunk, const double* x,
                        const double* alpha, const double* beta, const double* conv_w,
                        const double* conv_b, double* out, int32_t nthreads);

#ifdef __cplusplus
}
#endif
#endif
