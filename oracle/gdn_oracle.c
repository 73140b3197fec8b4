/*
 * gdn_oracle.c -- plain fp64 CPU oracle (TEST INFRASTRUCTURE ONLY).
 *
 * Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
 * load this library.  It is deliberately slow and literal: every loop below
 * follows the definitions D1-D8 listed in gdn_oracle.h in their written
 * order, with no blocking, fusion or reordering.  Threads only split
 * independent (request or sequence, value head) units.
 *
 * Build: gcc -O2 -fPIC -shared -pthread gdn_oracle.c -o libgdn_oracle.so -lm
 */
#include "gdn_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* shape helpers                                                             */

static int64_t n_channels(const orc_layer* L) {
  return 2 * (int64_t)L->n_k_heads * L->d_k + (int64_t)L->n_v_heads * L->d_v;
}
static int64_t ssm_slot_elems(const orc_layer* L) {
  return (int64_t)L->n_v_heads * L->d_v * L->d_k;
}
static int64_t conv_slot_elems(const orc_layer* L) {
  return (int64_t)(L->conv_width - 1) * n_channels(L);
}
static int64_t alpha_per_row(const orc_layer* L) {
  return L->gate ? (int64_t)L->n_v_heads * L->d_k : L->n_v_heads;
}

static int check_layer(const orc_layer* L) {
  if (!L) return -1;
  if (L->n_k_heads <= 0 || L->n_v_heads <= 0) return -1;
  if (L->n_v_heads % L->n_k_heads) return -1;
  if (L->d_k <= 0 || L->d_v <= 0 || L->conv_width < 1) return -1;
  if (L->gate != 0 && L->gate != 1) return -1;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* a minimal static work split over threads                                 */

typedef void (*unit_fn)(void* ctx, int64_t u);
typedef struct {
  unit_fn fn;
  void* ctx;
  int64_t n;
  int tid, nth;
} worker_arg;

static void* worker(void* p) {
  worker_arg* a = (worker_arg*)p;
  for (int64_t u = a->tid; u < a->n; u += a->nth) a->fn(a->ctx, u);
  return NULL;
}

static void run_units(unit_fn fn, void* ctx, int64_t n, int nth) {
  if (nth > n) nth = (int)n;
  if (nth <= 1) {
    for (int64_t u = 0; u < n; ++u) fn(ctx, u);
    return;
  }
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * nth);
  worker_arg* args = (worker_arg*)malloc(sizeof(worker_arg) * nth);
  for (int i = 0; i < nth; ++i) {
    args[i].fn = fn;
    args[i].ctx = ctx;
    args[i].n = n;
    args[i].tid = i;
    args[i].nth = nth;
    pthread_create(&th[i], NULL, worker, &args[i]);
  }
  for (int i = 0; i < nth; ++i) pthread_join(th[i], NULL);
  free(th);
  free(args);
}

/* ------------------------------------------------------------------------ */
/* D1: causal depthwise conv of one channel for one token.
 * win[0..W-2] are the previous inputs, oldest first; w[0..W-1] the taps,
 * w[W-1] multiplying the current input.  The window shifts in place.       */
static double conv_channel(const orc_layer* L, double* win, double xt, const double* w,
                           double bias) {
  const int W = L->conv_width;
  double y = bias;
  for (int j = 0; j < W - 1; ++j) y += w[j] * win[j];
  y += w[W - 1] * xt;
  for (int j = 0; j + 1 < W - 1; ++j) win[j] = win[j + 1];
  if (W > 1) win[W - 2] = xt;
  if (L->conv_silu) y = y / (1.0 + exp(-y)); /* SiLU: y * sigmoid(y) */
  return y;
}

/* Per-head conv windows: q and k channels of the key head, v channels of the
 * value head, each [n][W-1].                                                 */
typedef struct {
  double *wq, *wk, *wv;
} head_windows;

static void windows_alloc(const orc_layer* L, head_windows* hw) {
  int Wm = L->conv_width > 1 ? L->conv_width - 1 : 1;
  hw->wq = (double*)calloc((size_t)L->d_k * Wm, sizeof(double));
  hw->wk = (double*)calloc((size_t)L->d_k * Wm, sizeof(double));
  hw->wv = (double*)calloc((size_t)L->d_v * Wm, sizeof(double));
}
static void windows_free(head_windows* hw) {
  free(hw->wq);
  free(hw->wk);
  free(hw->wv);
}

/* channel offsets of D2: q | k | v, head-major within each part */
static int64_t q_off(const orc_layer* L, int kh) { return (int64_t)kh * L->d_k; }
static int64_t k_off(const orc_layer* L, int kh) {
  return (int64_t)L->n_k_heads * L->d_k + (int64_t)kh * L->d_k;
}
static int64_t v_off(const orc_layer* L, int h) {
  return 2 * (int64_t)L->n_k_heads * L->d_k + (int64_t)h * L->d_v;
}
static int key_head_of(const orc_layer* L, int h) {
  return h / (L->n_v_heads / L->n_k_heads);
}

/* Load the initial windows of value head h from a [W-1][C] window block
 * (NULL means all-zero history).                                           */
static void windows_load(const orc_layer* L, int h, const double* win0, head_windows* hw) {
  const int W1 = L->conv_width - 1;
  const int64_t C = n_channels(L);
  const int kh = key_head_of(L, h);
  if (!win0 || W1 == 0) return; /* calloc'd: zeros */
  for (int j = 0; j < L->d_k; ++j)
    for (int r = 0; r < W1; ++r) {
      hw->wq[j * W1 + r] = win0[r * C + q_off(L, kh) + j];
      hw->wk[j * W1 + r] = win0[r * C + k_off(L, kh) + j];
    }
  for (int i = 0; i < L->d_v; ++i)
    for (int r = 0; r < W1; ++r) hw->wv[i * W1 + r] = win0[r * C + v_off(L, h) + i];
}

/* D1 + D2 for value head h and one token x_t[C]: returns q^, k^, v. */
static void head_token_prep(const orc_layer* L, int h, head_windows* hw, const double* xt,
                            const double* w, const double* b, double* q, double* k,
                            double* v) {
  const int W = L->conv_width;
  const int W1 = W - 1;
  const int Ws = W1 > 0 ? W1 : 1;
  const int kh = key_head_of(L, h);
  for (int j = 0; j < L->d_k; ++j) {
    int64_t c = q_off(L, kh) + j;
    q[j] = conv_channel(L, hw->wq + j * Ws, xt[c], w + c * W, b ? b[c] : 0.0);
  }
  for (int j = 0; j < L->d_k; ++j) {
    int64_t c = k_off(L, kh) + j;
    k[j] = conv_channel(L, hw->wk + j * Ws, xt[c], w + c * W, b ? b[c] : 0.0);
  }
  for (int i = 0; i < L->d_v; ++i) {
    int64_t c = v_off(L, h) + i;
    v[i] = conv_channel(L, hw->wv + i * Ws, xt[c], w + c * W, b ? b[c] : 0.0);
  }
  double rq = 1.0, rk = 1.0;
  if (L->l2norm) {
    double nq = 0.0, nk = 0.0;
    for (int j = 0; j < L->d_k; ++j) nq += q[j] * q[j];
    for (int j = 0; j < L->d_k; ++j) nk += k[j] * k[j];
    rq = 1.0 / sqrt(nq + L->eps);
    rk = 1.0 / sqrt(nk + L->eps);
  }
  for (int j = 0; j < L->d_k; ++j) q[j] = q[j] * rq * L->q_scale;
  for (int j = 0; j < L->d_k; ++j) k[j] = k[j] * rk;
}

/* D3 / D4: one token of the gated delta rule on one head, rank-1 form.
 * a[j] is the decay of key column j (all equal for the scalar GDN gate).   */
static void state_step(const orc_layer* L, double* S, const double* q, const double* k,
                       const double* v, const double* a, double beta, double* o) {
  const int dk = L->d_k, dv = L->d_v;
  for (int i = 0; i < dv; ++i) {
    double* row = S + (int64_t)i * dk;
    double p = 0.0;
    for (int j = 0; j < dk; ++j) {
      row[j] = row[j] * a[j]; /* S' = S diag(a) */
      p += row[j] * k[j];     /* (S' k^)_i */
    }
    double u = beta * (v[i] - p);
    double oi = 0.0;
    for (int j = 0; j < dk; ++j) {
      row[j] = row[j] + u * k[j]; /* S <- S' + u k^T */
      oi += row[j] * q[j];        /* o = S q^ */
    }
    o[i] = oi;
  }
}

/* Fill a[d_k] with the decay of token row `t` for value head h. */
static void gate_of(const orc_layer* L, const double* alpha_rows, int64_t t, int h, double* a) {
  if (L->gate == 0) {
    double al = alpha_rows[t * L->n_v_heads + h];
    for (int j = 0; j < L->d_k; ++j) a[j] = al;
  } else {
    const double* src = alpha_rows + (t * L->n_v_heads + h) * (int64_t)L->d_k;
    for (int j = 0; j < L->d_k; ++j) a[j] = src[j];
  }
}

/* Run value head h over T consecutive token rows, updating S in place.
 * snap (optional) receives the state after each token, stride snap_stride. */
static void run_head(const orc_layer* L, int h, double* S, const double* win0,
                     const double* x, const double* alpha, const double* beta, int64_t T,
                     const double* w, const double* b, double* out, double* snap,
                     int64_t snap_stride) {
  const int dk = L->d_k, dv = L->d_v, Hv = L->n_v_heads;
  const int64_t C = n_channels(L);
  head_windows hw;
  windows_alloc(L, &hw);
  windows_load(L, h, win0, &hw);
  double* q = (double*)malloc(sizeof(double) * dk);
  double* k = (double*)malloc(sizeof(double) * dk);
  double* a = (double*)malloc(sizeof(double) * dk);
  double* v = (double*)malloc(sizeof(double) * dv);
  double* o = (double*)malloc(sizeof(double) * dv);
  for (int64_t t = 0; t < T; ++t) {
    head_token_prep(L, h, &hw, x + t * C, w, b, q, k, v);
    gate_of(L, alpha, t, h, a);
    state_step(L, S, q, k, v, a, beta[t * Hv + h], o);
    memcpy(out + (t * Hv + h) * (int64_t)dv, o, sizeof(double) * dv);
    if (snap) memcpy(snap + t * snap_stride + (int64_t)h * dv * dk, S, sizeof(double) * dv * dk);
  }
  free(q);
  free(k);
  free(a);
  free(v);
  free(o);
  windows_free(&hw);
}

/* Window after `t_end` tokens (t_end >= 1) of the sequence
 * z = (win0[0..W-2], x[0..T-1]): rows z[t_end .. t_end+W-2].  All channels. */
static void window_after(const orc_layer* L, const double* win0, const double* x,
                         int64_t t_end, double* dst) {
  const int W1 = L->conv_width - 1;
  const int64_t C = n_channels(L);
  for (int r = 0; r < W1; ++r) {
    int64_t zi = t_end + r; /* index into z */
    for (int64_t c = 0; c < C; ++c) {
      double val;
      if (zi < W1)
        val = win0 ? win0[zi * C + c] : 0.0;
      else
        val = x[(zi - W1) * C + c];
      dst[r * C + c] = val;
    }
  }
}

/* ------------------------------------------------------------------------ */
/* D3-D5: decode (in place) or speculative draft (snapshots)                 */

typedef struct {
  const orc_layer* L;
  double* ssm;
  double* conv;
  const int32_t* idx;
  int32_t T;
  const double *x, *alpha, *beta, *w, *b;
  double* out;
  double* spec_ssm;
  int32_t t_max;
} decode_ctx;

static void decode_unit(void* p, int64_t u) {
  decode_ctx* c = (decode_ctx*)p;
  const orc_layer* L = c->L;
  const int Hv = L->n_v_heads, dk = L->d_k, dv = L->d_v;
  const int64_t b = u / Hv;
  const int h = (int)(u % Hv);
  const int32_t slot = c->idx[b];
  if (slot < 0) return;
  const int64_t C = n_channels(L);
  const int64_t T = c->T;
  double* S = c->ssm + slot * ssm_slot_elems(L) + (int64_t)h * dv * dk;
  double* work = S;
  double* snap = NULL;
  int64_t snap_stride = 0;
  if (c->spec_ssm) { /* the working slot is left untouched */
    work = (double*)malloc(sizeof(double) * dv * dk);
    memcpy(work, S, sizeof(double) * dv * dk);
    snap = c->spec_ssm + b * c->t_max * ssm_slot_elems(L);
    snap_stride = ssm_slot_elems(L);
  }
  const double* win0 = L->conv_width > 1 ? c->conv + slot * conv_slot_elems(L) : NULL;
  run_head(L, h, work, win0, c->x + b * T * C, c->alpha + b * T * alpha_per_row(L),
           c->beta + b * T * Hv, T, c->w, c->b, c->out + b * T * Hv * (int64_t)dv, snap,
           snap_stride);
  if (work != S) free(work);
}

int orc_decode(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
               const int32_t* idx, int32_t B, int32_t T, const double* x, const double* alpha,
               const double* beta, const double* conv_w, const double* conv_b, double* out,
               double* spec_ssm, double* spec_conv, int32_t t_max, int32_t nthreads) {
  if (check_layer(L) || !ssm || (L->conv_width > 1 && !conv) || !idx || B < 0 || T < 0)
    return -1;
  if (T > 0 && (!x || !alpha || !beta || !conv_w || !out)) return -1;
  if (spec_ssm && (T > t_max || (L->conv_width > 1 && !spec_conv))) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (idx[b] >= num_slots) return -1;
  if (T == 0) return 0;

  decode_ctx c = {L, ssm, conv, idx, T, x, alpha, beta, conv_w, conv_b, out, spec_ssm, t_max};
  run_units(decode_unit, &c, (int64_t)B * L->n_v_heads, nthreads);

  /* conv windows: after every token into the snapshots, or after the last
   * token into the pool.  All head units have read the old window already. */
  if (L->conv_width > 1) {
    const int64_t C = n_channels(L);
    const int64_t cs = conv_slot_elems(L);
    double* tmp = (double*)malloc(sizeof(double) * cs);
    for (int32_t b = 0; b < B; ++b) {
      const int32_t slot = idx[b];
      if (slot < 0) continue;
      const double* win0 = conv + slot * cs;
      const double* xb = x + (int64_t)b * T * C;
      if (spec_ssm) {
        for (int32_t t = 0; t < T; ++t)
          window_after(L, win0, xb, t + 1, spec_conv + ((int64_t)b * t_max + t) * cs);
      } else {
        window_after(L, win0, xb, T, tmp);
        memcpy(conv + slot * cs, tmp, sizeof(double) * cs);
      }
    }
    free(tmp);
  }
  return 0;
}

/* D5 commit: working slot <- snapshot accepted_len - 1 (nothing when 0). */
int orc_spec_commit(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                    const int32_t* idx, const double* spec_ssm, const double* spec_conv,
                    int32_t t_max, const int32_t* acc, int32_t B) {
  if (check_layer(L) || !ssm || !idx || !spec_ssm || !acc || B < 0) return -1;
  if (L->conv_width > 1 && (!conv || !spec_conv)) return -1;
  for (int32_t b = 0; b < B; ++b)
    if (idx[b] >= num_slots || acc[b] < 0 || acc[b] > t_max) return -1;
  const int64_t ss = ssm_slot_elems(L), cs = conv_slot_elems(L);
  for (int32_t b = 0; b < B; ++b) {
    const int32_t slot = idx[b];
    const int32_t n = acc[b];
    if (slot < 0 || n == 0) continue;
    memcpy(ssm + slot * ss, spec_ssm + ((int64_t)b * t_max + n - 1) * ss, sizeof(double) * ss);
    if (cs)
      memcpy(conv + slot * cs, spec_conv + ((int64_t)b * t_max + n - 1) * cs,
             sizeof(double) * cs);
  }
  return 0;
}

/* D6 */
int orc_slot_copy(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                  const int32_t* src, const int32_t* dst, int32_t n) {
  if (check_layer(L) || !ssm || !src || !dst || n < 0) return -1;
  if (L->conv_width > 1 && !conv) return -1;
  for (int32_t i = 0; i < n; ++i)
    if (src[i] >= num_slots || dst[i] >= num_slots) return -1;
  const int64_t ss = ssm_slot_elems(L), cs = conv_slot_elems(L);
  for (int32_t i = 0; i < n; ++i) {
    if (src[i] < 0 || dst[i] < 0) continue;
    memcpy(ssm + (int64_t)dst[i] * ss, ssm + (int64_t)src[i] * ss, sizeof(double) * ss);
    if (cs) memcpy(conv + (int64_t)dst[i] * cs, conv + (int64_t)src[i] * cs, sizeof(double) * cs);
  }
  return 0;
}

int orc_slot_zero(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                  const int32_t* idx, int32_t n) {
  if (check_layer(L) || !ssm || !idx || n < 0) return -1;
  if (L->conv_width > 1 && !conv) return -1;
  for (int32_t i = 0; i < n; ++i)
    if (idx[i] >= num_slots) return -1;
  const int64_t ss = ssm_slot_elems(L), cs = conv_slot_elems(L);
  for (int32_t i = 0; i < n; ++i) {
    if (idx[i] < 0) continue;
    for (int64_t e = 0; e < ss; ++e) ssm[(int64_t)idx[i] * ss + e] = 0.0;
    for (int64_t e = 0; e < cs; ++e) conv[(int64_t)idx[i] * cs + e] = 0.0;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* D7 / D8: prefill over variable-length sequences.
 * All initial states are read before any destination is written, so a
 * sequence may start from a slot that another sequence writes.             */

typedef struct {
  const orc_layer* L;
  const int32_t* cu;
  const int32_t* dst;
  int32_t chunk;
  const double *x, *alpha, *beta, *w, *b;
  double* out;
  double* S0;   /* [N][H_v][d_v][d_k] initial -> final states */
  double* win0; /* [N][W-1][C] initial windows */
  int has_win;
} prefill_ctx;

static void prefill_seq_unit(void* p, int64_t u) {
  prefill_ctx* c = (prefill_ctx*)p;
  const orc_layer* L = c->L;
  const int Hv = L->n_v_heads;
  const int64_t s = u / Hv;
  const int h = (int)(u % Hv);
  if (c->dst[s] < 0) return;
  const int64_t C = n_channels(L);
  const int64_t t0 = c->cu[s], T = c->cu[s + 1] - c->cu[s];
  double* S = c->S0 + s * ssm_slot_elems(L) + (int64_t)h * L->d_v * L->d_k;
  const double* win0 = c->has_win ? c->win0 + s * conv_slot_elems(L) : NULL;
  run_head(L, h, S, win0, c->x + t0 * C, c->alpha + t0 * alpha_per_row(L),
           c->beta + t0 * Hv, T, c->w, c->b, c->out + t0 * Hv * (int64_t)L->d_v, NULL, 0);
}

/* D8: the WY/UT-transform chunk form (GDN scalar gate).  For a chunk of c
 * tokens with rows K, Q, V (k^, q^, v) and S0 the state before the chunk:
 *   g_r = sum_{i<=r} log alpha_i,
 *   A_ri = beta_r e^{g_r - g_i} (k_r . k_i) for i < r,
 *   (I + A) T = diag(beta)          (forward substitution),
 *   W = T diag(e^g) K,  U~ = T V,  U = U~ - W S0^T,
 *   O = diag(e^g) Q S0^T + P U,  P_ri = e^{g_r - g_i} (q_r . k_i), i <= r,
 *   S <- e^{g_c} S0 + U^T diag(e^{g_c - g}) K.                             */
static void prefill_chunk_unit(void* p, int64_t u) {
  prefill_ctx* c = (prefill_ctx*)p;
  const orc_layer* L = c->L;
  const int Hv = L->n_v_heads, dk = L->d_k, dv = L->d_v;
  const int64_t s = u / Hv;
  const int h = (int)(u % Hv);
  if (c->dst[s] < 0) return;
  const int64_t C = n_channels(L);
  const int64_t t0 = c->cu[s], T = c->cu[s + 1] - c->cu[s];
  double* S = c->S0 + s * ssm_slot_elems(L) + (int64_t)h * dv * dk;
  const double* win0 = c->has_win ? c->win0 + s * conv_slot_elems(L) : NULL;
  if (T == 0) return;

  /* activations of the whole sequence for this head (D1, D2) */
  double* Q = (double*)malloc(sizeof(double) * T * dk);
  double* K = (double*)malloc(sizeof(double) * T * dk);
  double* V = (double*)malloc(sizeof(double) * T * dv);
  head_windows hw;
  windows_alloc(L, &hw);
  windows_load(L, h, win0, &hw);
  for (int64_t t = 0; t < T; ++t)
    head_token_prep(L, h, &hw, c->x + (t0 + t) * C, c->w, c->b, Q + t * dk, K + t * dk,
                    V + t * dv);
  windows_free(&hw);

  const int cmax = c->chunk;
  double* g = (double*)malloc(sizeof(double) * cmax);
  double* bet = (double*)malloc(sizeof(double) * cmax);
  double* A = (double*)malloc(sizeof(double) * cmax * cmax);
  double* Tm = (double*)malloc(sizeof(double) * cmax * cmax);
  double* Wm = (double*)malloc(sizeof(double) * cmax * dk);
  double* Ut = (double*)malloc(sizeof(double) * cmax * dv);
  double* U = (double*)malloc(sizeof(double) * cmax * dv);
  double* Snew = (double*)malloc(sizeof(double) * dv * dk);

  for (int64_t c0 = 0; c0 < T; c0 += cmax) {
    const int n = (int)(T - c0 < cmax ? T - c0 : cmax);
    const double* Kc = K + c0 * dk;
    const double* Qc = Q + c0 * dk;
    const double* Vc = V + c0 * dv;
    for (int r = 0; r < n; ++r) {
      double la = log(c->alpha[(t0 + c0 + r) * Hv + h]);
      if (la < -80.0) la = -80.0;
      g[r] = (r ? g[r - 1] : 0.0) + la;
      bet[r] = c->beta[(t0 + c0 + r) * Hv + h];
    }
    for (int r = 0; r < n; ++r)
      for (int i = 0; i < n; ++i) {
        double a = 0.0;
        if (i < r) {
          double kk = 0.0;
          for (int j = 0; j < dk; ++j) kk += Kc[r * dk + j] * Kc[i * dk + j];
          a = bet[r] * exp(g[r] - g[i]) * kk;
        }
        A[r * n + i] = a;
      }
    /* forward substitution, one column m at a time */
    for (int m = 0; m < n; ++m)
      for (int r = 0; r < n; ++r) {
        double t = (r == m) ? bet[r] : 0.0;
        for (int i = 0; i < r; ++i) t -= A[r * n + i] * Tm[i * n + m];
        Tm[r * n + m] = t;
      }
    for (int r = 0; r < n; ++r) {
      for (int j = 0; j < dk; ++j) {
        double acc = 0.0;
        for (int i = 0; i < n; ++i) acc += Tm[r * n + i] * exp(g[i]) * Kc[i * dk + j];
        Wm[r * dk + j] = acc;
      }
      for (int e = 0; e < dv; ++e) {
        double acc = 0.0;
        for (int m = 0; m < n; ++m) acc += Tm[r * n + m] * Vc[m * dv + e];
        Ut[r * dv + e] = acc;
      }
    }
    for (int r = 0; r < n; ++r)
      for (int e = 0; e < dv; ++e) {
        double ws = 0.0;
        for (int j = 0; j < dk; ++j) ws += Wm[r * dk + j] * S[e * dk + j];
        U[r * dv + e] = Ut[r * dv + e] - ws;
      }
    for (int r = 0; r < n; ++r)
      for (int e = 0; e < dv; ++e) {
        double qs = 0.0;
        for (int j = 0; j < dk; ++j) qs += Qc[r * dk + j] * S[e * dk + j];
        double pu = 0.0;
        for (int m = 0; m <= r; ++m) {
          double qk = 0.0;
          for (int j = 0; j < dk; ++j) qk += Qc[r * dk + j] * Kc[m * dk + j];
          pu += exp(g[r] - g[m]) * qk * U[m * dv + e];
        }
        c->out[((t0 + c0 + r) * Hv + h) * (int64_t)dv + e] = exp(g[r]) * qs + pu;
      }
    const double gc = g[n - 1];
    for (int e = 0; e < dv; ++e)
      for (int j = 0; j < dk; ++j) {
        double acc = exp(gc) * S[e * dk + j];
        for (int r = 0; r < n; ++r) acc += U[r * dv + e] * exp(gc - g[r]) * Kc[r * dk + j];
        Snew[e * dk + j] = acc;
      }
    memcpy(S, Snew, sizeof(double) * dv * dk);
  }
  free(g);
  free(bet);
  free(A);
  free(Tm);
  free(Wm);
  free(Ut);
  free(U);
  free(Snew);
  free(Q);
  free(K);
  free(V);
}

static int prefill_common(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                          const int32_t* dst, const int32_t* init, int32_t N,
                          const int32_t* cu, int32_t chunk, const double* x,
                          const double* alpha, const double* beta, const double* w,
                          const double* b, double* out, int32_t nthreads, unit_fn fn) {
  if (check_layer(L) || !ssm || (L->conv_width > 1 && !conv) || !dst || !cu || N < 0)
    return -1;
  if (cu[0] != 0) return -1;
  for (int32_t s = 0; s < N; ++s) {
    if (cu[s + 1] < cu[s]) return -1;
    if (dst[s] >= num_slots) return -1;
    if (init && init[s] >= num_slots) return -1;
  }
  if (cu[N] > 0 && (!x || !alpha || !beta || !w || !out)) return -1;
  const int64_t ss = ssm_slot_elems(L), cs = conv_slot_elems(L), C = n_channels(L);
  double* S0 = (double*)calloc((size_t)(N ? N : 1) * ss, sizeof(double));
  double* W0 = (double*)calloc((size_t)(N ? N : 1) * (cs ? cs : 1), sizeof(double));
  for (int32_t s = 0; s < N; ++s) {
    const int32_t src = init ? init[s] : dst[s];
    if (src >= 0) {
      memcpy(S0 + s * ss, ssm + (int64_t)src * ss, sizeof(double) * ss);
      if (cs) memcpy(W0 + s * cs, conv + (int64_t)src * cs, sizeof(double) * cs);
    }
  }
  prefill_ctx c = {L, cu, dst, chunk, x, alpha, beta, w, b, out, S0, W0, cs > 0};
  run_units(fn, &c, (int64_t)N * L->n_v_heads, nthreads);
  double* tmp = (double*)malloc(sizeof(double) * (cs ? cs : 1));
  for (int32_t s = 0; s < N; ++s) {
    if (dst[s] < 0) continue;
    memcpy(ssm + (int64_t)dst[s] * ss, S0 + s * ss, sizeof(double) * ss);
    if (cs) {
      const int64_t T = cu[s + 1] - cu[s];
      if (T == 0)
        memcpy(tmp, W0 + s * cs, sizeof(double) * cs);
      else
        window_after(L, W0 + s * cs, x + (int64_t)cu[s] * C, T, tmp);
      memcpy(conv + (int64_t)dst[s] * cs, tmp, sizeof(double) * cs);
    }
  }
  free(tmp);
  free(S0);
  free(W0);
  return 0;
}

int orc_prefill(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                const int32_t* dst, const int32_t* init, int32_t N, const int32_t* cu,
                const double* x, const double* alpha, const double* beta, const double* w,
                const double* b, double* out, int32_t nthreads) {
  return prefill_common(L, ssm, conv, num_slots, dst, init, N, cu, 0, x, alpha, beta, w, b,
                        out, nthreads, prefill_seq_unit);
}

int orc_prefill_chunked(const orc_layer* L, double* ssm, double* conv, int64_t num_slots,
                        const int32_t* dst, const int32_t* init, int32_t N, const int32_t* cu,
                        int32_t chunk, const double* x, const double* alpha,
                        const double* beta, const double* w, const double* b, double* out,
                        int32_t nthreads) {
  if (!L || L->gate != 0 || chunk < 1) return -2; /* chunk form: scalar gate only */
  return prefill_common(L, ssm, conv, num_slots, dst, init, N, cu, chunk, x, alpha, beta, w,
                        b, out, nthreads, prefill_chunk_unit);
}
