// gdn_decode.hip -- fused decode step for Gated DeltaNet / KDA on gfx950.
//
// Work unit: one (request b, key head kh).  A unit owns the q and k conv
// channels of kh, the v channels of its G = H_v/H_k value heads and the
// G*d_v state rows of those heads, so it is the only reader and writer of
// every conv-window channel it touches: no cross-workgroup ordering exists.
//
// Persistent schedule.  The grid is H_k * m workgroups (m about CUs / H_k),
// so workgroup x always serves key head x % H_k and walks the requests
// x / H_k, + m, + 2m, ...  Its conv taps and bias are therefore loaded once.
// For each unit the state rows and the unit's first-token inputs (x, conv
// window, gates, betas) stream from HBM straight into LDS with
// global_load_lds (no registers involved), issued while the previous unit is
// computed and stored; each wave copies its own rows into its own LDS stage.
// Nothing the compute reads is ever a register load in flight, so the only
// wait on vector memory is one explicit drain per unit (vm_wait<0>) before
// the staged rows are pulled into registers.  HBM reads of the next unit
// thus overlap the compute and the writes of the current one.
//
// Per unit, per token (state in registers across all T tokens of the call):
//   conv update + SiLU of the unit's channels          -> LDS
//   |q|^2, |k|^2, q.k per token (DPP + readlane sums)  -> LDS scales
//   per state row i (value index), per lane CPL*4 key columns:
//     s' = s * a_j                    (a_j = alpha, or alpha_j for KDA)
//     pk = sum_j s'_j k^_j,  pq = sum_j s'_j q^_j     (DPP row-group sums)
//     u  = beta (v_i - pk);  o_i = pq + u (k^.q^);  s = s' + u k^_j
// which is S_t = alpha S (I - beta k k^T) + beta v k^T, o_t = S_t q_t, with
// o_t formed as S' q^ + u (k^.q^) (equal to S_t q^ by definition).
//
// Memory: a state row (d_k fp32) is split over LPR lanes x CPL 16-byte
// chunks and a lane group owns NR consecutive rows, so each copy instruction
// of a wave covers whole 128-byte lines and every state access of a lane is
// one base address plus an immediate offset.  State traffic is
// non-temporal: each slot is touched once per call.
//
// Bitwise contract: the in-place path (spec_ssm == nullptr) and the snapshot
// path run the same instantiation and the same per-token arithmetic (built
// with -ffp-contract=off, explicit fmaf), so a draft of T tokens followed by
// a commit of L equals an in-place decode of L tokens bit for bit.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kMaxW1 = 3;                 // conv_width <= 4
constexpr int kBatch = 2;                 // later tokens whose x are loaded together
constexpr int kMaxUnitsPerCta = 512;      // slot-table entries per workgroup
constexpr int kRawIt = 6;                 // raw-input copies per lane with precomputed offsets
constexpr size_t kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU

// Lane layout of a state row of d_k fp32: LPR lanes, each holding CPL 16-byte
// chunks (chunk n*LPR + lc in lane lc); one copy instruction of a wave covers
// RPP rows x LPR*16 contiguous bytes.
template <int DK>
struct RowMap {
  static constexpr int LPR = DK >= 64 ? 16 : DK / 4;  // lanes per state row
  static constexpr int CPL = DK / (4 * LPR);          // 16-byte chunks per lane
  static constexpr int RPP = 64 / LPR;                // rows per wave per pass
};

// LDS plan of a workgroup, in dwords: per-wave state stages | two raw-input
// buffers (the next unit's copies land while this unit reads its own) | one
// activation buffer | slot table of the workgroup's units (destination and
// source slot of each).
struct LdsPlan {
  int stage_per_wave, raw_len, act_len;
  int raw, act, slots, total;
};
__host__ __device__ inline LdsPlan lds_plan(int dk, int rpw, int waves, int Cg, int W1, int GA,
                                            int G, int tchunk, int units = kMaxUnitsPerCta) {
  LdsPlan p;
  const int rpp = dk >= 64 ? 4 : 256 / dk;
  const int cpl = dk >= 64 ? dk / 64 : 1;
  p.stage_per_wave = (rpw / rpp) * cpl * 256;
  p.raw_len = Cg * (1 + W1) + GA + G;
  p.act_len = tchunk * (Cg + GA + G + 4);
  p.raw = waves * p.stage_per_wave;
  p.act = p.raw + 2 * p.raw_len;
  p.slots = p.act + p.act_len;
  p.total = p.slots + 2 * units;
  return p;
}

template <int DK, int RPW, typename Act, bool KDA>
struct DecodeCta {
  using M = RowMap<DK>;
  static constexpr int LPR = M::LPR, CPL = M::CPL, RPP = M::RPP;
  static_assert(RPW % RPP == 0, "whole passes per wave");
  static constexpr int NR = RPW / RPP;      // rows per lane
  static constexpr int DKA = KDA ? DK : 1;  // gate values per (token, value head)

  const DecodeArgs& a;
  int tid, lane, wave, nwaves, NT, lr, lc;
  int dv, G, R, Cg, GA, W, W1, lead, C, T, TC, Hv, Hk, per_tok;
  int kh, b0, m;  // this workgroup's key head, first request, request stride
  bool spec;        // snapshots per token instead of an in-place update
  bool spec_pool;   // ... into pool slots named by a.spec_slots
  int64_t slot_elems;
  uint32_t lane_off;  // this lane's first state element within a unit
  uint32_t chan;      // global conv channel of this thread (tid < Cg)
  LdsPlan plan;
  // element offset, within its source block (x row | conv window | gates |
  // betas), of raw input j*64 + lane for this wave's first kRawIt values of j
  uint32_t roff[kRawIt];

  __device__ __forceinline__ DecodeCta(const DecodeArgs& args) : a(args) {
    tid = threadIdx.x;
    lane = tid & 63;
    wave = uniform(tid >> 6);
    nwaves = blockDim.x >> 6;
    NT = blockDim.x;
    lr = lane / LPR;
    lc = lane % LPR;
    dv = a.dv;
    G = a.G;
    R = G * dv;
    Cg = 2 * DK + R;
    GA = G * DKA;
    W = a.W;
    W1 = W - 1;
    lead = kMaxW1 - W1;
    C = a.C;
    T = a.T;
    TC = a.tchunk;
    Hv = a.Hv;
    Hk = a.Hk;
    per_tok = Cg + GA + G + 4;
    kh = static_cast<int>(blockIdx.x) % Hk;
    b0 = static_cast<int>(blockIdx.x) / Hk;
    m = static_cast<int>(gridDim.x) / Hk;
    spec_pool = a.spec_slots != nullptr;
    spec = spec_pool || a.spec_ssm != nullptr;
    slot_elems = static_cast<int64_t>(Hv) * dv * DK;
    lane_off = static_cast<uint32_t>(wave * RPW + lr * NR) * DK + 4 * lc;
    chan = channel(tid < Cg ? tid : 0);
    plan = lds_plan(DK, RPW, nwaves, Cg, W1, GA, G, TC);
#pragma unroll
    for (int i = 0; i < kRawIt; ++i) roff[i] = raw_offset((wave + i * nwaves) * 64 + lane);
  }

  // Offset of raw input d within its source block (see copy_unit).
  __device__ __forceinline__ uint32_t raw_offset(int d) const {
    const int nx = Cg * (1 + W1);
    if (d < Cg) return channel(d);
    if (d < nx) {
      const int r = (d - Cg) / Cg;
      return static_cast<uint32_t>(r) * C + channel(d - Cg - r * Cg);
    }
    return d < nx + GA ? d - nx : d - nx - GA;
  }

  // global conv channel of local channel c (q | k | v of this key head)
  __device__ __forceinline__ uint32_t channel(int c) const {
    return c < DK       ? kh * DK + c
           : c < 2 * DK ? Hk * DK + kh * DK + (c - DK)
                        : 2 * Hk * DK + kh * R + (c - 2 * DK);
  }
  // state of this unit's key-head group in a slot (uniform)
  __device__ __forceinline__ float* state(float* base, int64_t row) const {
    return base + row * slot_elems + static_cast<int64_t>(kh) * R * DK;
  }
  __device__ __forceinline__ static float raw_f32(uint32_t d) {
    if constexpr (sizeof(Act) == 2)
      return __uint_as_float(d << 16);
    else
      return __uint_as_float(d);
  }

  // Issue the copies of unit (b, source slot) into LDS: this wave's state
  // rows into its stage -- instruction (p, n) as 64 lanes x 16 B at stage +
  // (p*CPL + n)*256, lane i's bytes at 16*i, exactly what a register load
  // would give -- and, shared by the waves, the raw first-token inputs into
  // raw: [x: Cg][window: W1 x Cg][gates: GA][betas: G], one dword per element.
  // A negative source (a fresh start) copies no state and zeroes the window.
  __device__ __forceinline__ void copy_unit(int b, int32_t slot, float* stage,
                                            uint32_t* raw) const {
    if (slot >= 0) {
      const float* src = state(a.ssm, slot) + lane_off;
#pragma unroll
      for (int p = 0; p < NR; ++p)
#pragma unroll
        for (int n = 0; n < CPL; ++n)
          lds_dma16(src + p * DK + 4 * n * LPR, stage + (p * CPL + n) * 256);
    }

    const Act* x0 = static_cast<const Act*>(a.x) + static_cast<int64_t>(b) * T * C;
    const Act* cs =
        static_cast<const Act*>(a.conv) + static_cast<int64_t>(slot >= 0 ? slot : 0) * W1 * C;
    const int64_t th = static_cast<int64_t>(b) * T * Hv + static_cast<int64_t>(kh) * G;
    const Act* al = static_cast<const Act*>(a.alpha) + th * DKA;
    const Act* be = static_cast<const Act*>(a.beta) + th;
    const int nx = Cg * (1 + W1);
    int i = 0;
    for (int j = wave; j * 64 < plan.raw_len; j += nwaves, ++i) {
      const int d = j * 64 + lane;
      if (d < plan.raw_len) {
        uint32_t off = 0;
#pragma unroll
        for (int q = 0; q < kRawIt; ++q)
          if (q == i) off = roff[q];
        if (i >= kRawIt) off = raw_offset(d);
        const Act* base = d < Cg ? x0 : d < nx ? cs : d < nx + GA ? al : be;
        if (slot < 0 && d >= Cg && d < nx)
          raw[j * 64 + lane] = 0u;
        else
          lds_dma<sizeof(Act)>(base + off, raw + j * 64);
      }
    }
  }

  __device__ __forceinline__ void stage_read(const float* stage, f4 (&s)[NR][CPL]) const {
#pragma unroll
    for (int p = 0; p < NR; ++p)
#pragma unroll
      for (int n = 0; n < CPL; ++n)
        s[p][n] = *reinterpret_cast<const f4*>(stage + (p * CPL + n) * 256 + 4 * lane);
  }

  // Where token t's snapshot goes (null: nowhere): a row of the spec cache,
  // or the pool slot the spec slot table names for it (skipped when outside
  // the pool).
  __device__ __forceinline__ int32_t spec_slot(int b, int t) const {
    const int32_t sl = a.spec_slots[static_cast<int64_t>(b) * a.t_max + t];
    return (sl < 0 || static_cast<int64_t>(sl) >= a.num_slots) ? -1 : sl;
  }
  __device__ __forceinline__ Act* snap_conv(int b, int t) const {
    if (spec_pool) {
      const int32_t sl = spec_slot(b, t);
      return sl < 0 ? nullptr : static_cast<Act*>(a.conv) + static_cast<int64_t>(sl) * W1 * C;
    }
    return static_cast<Act*>(a.spec_conv) + (static_cast<int64_t>(b) * a.t_max + t) * W1 * C;
  }
  __device__ __forceinline__ float* snap_ssm(int b, int t) const {
    if (spec_pool) {
      const int32_t sl = spec_slot(b, t);
      return sl < 0 ? nullptr : state(a.ssm, sl);
    }
    return state(a.spec_ssm, static_cast<int64_t>(b) * a.t_max + t);
  }

  // D1 for one token t of this thread's channel: conv over the window and
  // x, window shift, SiLU; the activation goes to act[tid]; the shifted
  // window goes to the snapshot of token t (spec) or, after the last token,
  // back to the slot.
  __device__ __forceinline__ void conv_token(int b, int t, float xv, const float (&wt)[kMaxW1 + 1],
                                             float (&win)[kMaxW1], float bias, float* act,
                                             Act* conv_slot) const {
    float y = bias;
#pragma unroll
    for (int j = 0; j < kMaxW1; ++j) y = fmaf(wt[j], win[j], y);
    y = fmaf(wt[kMaxW1], xv, y);
#pragma unroll
    for (int j = 0; j + 1 < kMaxW1; ++j) win[j] = j >= lead ? win[j + 1] : 0.f;
    win[kMaxW1 - 1] = xv;
    if (a.silu) y = y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
    act[tid] = y;
    Act* wdst = nullptr;
    if (spec)
      wdst = snap_conv(b, t);
    else if (t == T - 1)
      wdst = conv_slot;
    if (wdst) {
#pragma unroll
      for (int j = 0; j < kMaxW1; ++j)
        if (j >= lead) wdst[static_cast<uint32_t>(j - lead) * C + chan] = from_exact<Act>(win[j]);
    }
  }

  // Run the T tokens of unit (b, slot) on its state rows s.  raw holds the
  // unit's copied first-token inputs; act is the unit's activation buffer.
  __device__ __forceinline__ void run(int b, int32_t slot, f4 (&s)[NR][CPL],
                                      const float (&wt)[kMaxW1 + 1], float bias,
                                      const uint32_t* raw, float* act, bool wait_next) const {
    const int64_t tok0 = static_cast<int64_t>(b) * T;
    const Act* const x_req = static_cast<const Act*>(a.x) + tok0 * C;
    Act* const conv_slot = static_cast<Act*>(a.conv) + static_cast<int64_t>(slot) * W1 * C;
    const Act* const al_req =
        static_cast<const Act*>(a.alpha) + (tok0 * Hv + static_cast<int64_t>(kh) * G) * DKA;
    const Act* const be_req =
        static_cast<const Act*>(a.beta) + tok0 * Hv + static_cast<int64_t>(kh) * G;
    float* const out_req = a.out + (tok0 * Hv + static_cast<int64_t>(kh) * G) * dv;
    const int nx = Cg * (1 + W1);

    // conv window of this thread's channel, from the copied inputs
    float win[kMaxW1];
#pragma unroll
    for (int j = 0; j < kMaxW1; ++j)
      win[j] = (tid < Cg && j >= lead) ? raw_f32(raw[Cg + (j - lead) * Cg + tid]) : 0.f;

    for (int t0 = 0; t0 < T; t0 += TC) {
      const int nt = T - t0 < TC ? T - t0 : TC;

      // ---- D1: conv update + activation of the unit's channels for the nt
      // tokens of this chunk, into LDS; gates and betas alongside.
      // token 0 from the copied inputs (no global load on this path)
      const int first = t0 == 0 ? 1 : 0;
      if (first) {
        if (tid < Cg)
          conv_token(b, 0, raw_f32(raw[tid]), wt, win, bias, act, conv_slot);
        if (tid < GA + G) act[Cg + tid] = raw_f32(raw[nx + tid]);
      }
      // later tokens of the chunk from global memory
      if (tid < Cg) {
        for (int tb = first; tb < nt; tb += kBatch) {
          float xr[kBatch];
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            const int tt = tb + k < nt ? tb + k : nt - 1;
            xr[k] = to_f32(x_req[static_cast<uint32_t>(t0 + tt) * C + chan]);
          }
#pragma unroll
          for (int k = 0; k < kBatch; ++k) {
            if (tb + k >= nt) break;
            conv_token(b, t0 + tb + k, xr[k], wt, win, bias, act + (tb + k) * per_tok, conv_slot);
          }
        }
      }
      for (int e = tid + first * (GA + G); e < nt * (GA + G); e += NT) {
        const int tt = e / (GA + G);
        const int k = e - tt * (GA + G);
        const uint32_t tq = static_cast<uint32_t>(t0 + tt) * Hv;
        act[tt * per_tok + Cg + k] =
            k < GA ? to_f32(al_req[tq * DKA + k]) : to_f32(be_req[tq + (k - GA)]);
      }
      lds_barrier();

      // ---- D2: per token, norms of q and k and q.k; wave w takes tokens w,
      // w + nwaves, ... and leaves (|k|^-1, |q|^-1 q_scale, k^.q^) in LDS.
      for (int tt = wave; tt < nt; tt += nwaves) {
        const float* ab = act + tt * per_tok;
        float sq = 0.f, sk = 0.f, sqk = 0.f;
#pragma unroll
        for (int j0 = 0; j0 < DK; j0 += 64) {
          if (j0 + lane < DK) {
            const float qv = ab[j0 + lane];
            const float kv = ab[DK + j0 + lane];
            sq = fmaf(qv, qv, sq);
            sk = fmaf(kv, kv, sk);
            sqk = fmaf(qv, kv, sqk);
          }
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        sqk = wave_sum(sqk);
        const float rq = a.l2norm ? rsqrtf(sq + a.eps) : 1.0f;
        const float rk = a.l2norm ? rsqrtf(sk + a.eps) : 1.0f;
        const float qs = rq * a.q_scale;
        if (lane == 0) {
          float* sc = act + tt * per_tok + Cg + GA + G;
          sc[0] = rk;
          sc[1] = qs;
          sc[2] = sqk * rk * qs;  // k^ . q^
        }
      }
      lds_barrier();

      // ---- D3 / D4: the gated delta rule on this lane's rows, token by
      // token.  All RPW rows of a wave lie in one value head (RPW | d_v).
      const int hl = (wave * RPW) / dv;               // value head within the unit
      const int i0 = wave * RPW - hl * dv + lr * NR;  // value index of row p = 0
      for (int tt = 0; tt < nt; ++tt) {
        const int t = t0 + tt;
        const float* ab = act + tt * per_tok;
        const float* gl = ab + Cg;
        const float* bl = gl + GA;
        const float rk = bl[G + 0], qs = bl[G + 1], kq = bl[G + 2];
        f4 kk[CPL], qq[CPL];
#pragma unroll
        for (int n = 0; n < CPL; ++n) {
          const int col = 4 * (n * LPR + lc);
          kk[n] = *reinterpret_cast<const f4*>(ab + DK + col) * rk;
          qq[n] = *reinterpret_cast<const f4*>(ab + col) * qs;
        }
        const float be = bl[hl];
        f4 ga[CPL];
        if constexpr (KDA) {
#pragma unroll
          for (int n = 0; n < CPL; ++n)
            ga[n] = *reinterpret_cast<const f4*>(gl + hl * DK + 4 * (n * LPR + lc));
        } else {
          const float al = gl[hl];
#pragma unroll
          for (int n = 0; n < CPL; ++n) ga[n] = f4{al, al, al, al};
        }
#pragma unroll
        for (int p = 0; p < NR; ++p) {
          const int i = i0 + p;  // value index of this lane's row
          float pk = 0.f, pq = 0.f;
#pragma unroll
          for (int n = 0; n < CPL; ++n) {
            f4 v = s[p][n] * ga[n];
            s[p][n] = v;
            pk = fmaf(v.x, kk[n].x, pk);
            pk = fmaf(v.y, kk[n].y, pk);
            pk = fmaf(v.z, kk[n].z, pk);
            pk = fmaf(v.w, kk[n].w, pk);
            pq = fmaf(v.x, qq[n].x, pq);
            pq = fmaf(v.y, qq[n].y, pq);
            pq = fmaf(v.z, qq[n].z, pq);
            pq = fmaf(v.w, qq[n].w, pq);
          }
          pk = group_sum<LPR>(pk);
          pq = group_sum<LPR>(pq);
          const float u = be * (ab[2 * DK + hl * dv + i] - pk);
          const float o = fmaf(u, kq, pq);
#pragma unroll
          for (int n = 0; n < CPL; ++n) {
            s[p][n].x = fmaf(u, kk[n].x, s[p][n].x);
            s[p][n].y = fmaf(u, kk[n].y, s[p][n].y);
            s[p][n].z = fmaf(u, kk[n].z, s[p][n].z);
            s[p][n].w = fmaf(u, kk[n].w, s[p][n].w);
          }
          if (lc == 0) out_req[static_cast<uint32_t>(t) * Hv * dv + hl * dv + i] = o;
        }
        if (spec) {
          float* dst = snap_ssm(b, t);
          if (dst) {
            dst += lane_off;
#pragma unroll
            for (int p = 0; p < NR; ++p)
#pragma unroll
              for (int n = 0; n < CPL; ++n) st_stream(dst + p * DK + 4 * n * LPR, s[p][n]);
          }
        }
      }
      if (t0 + TC < T) lds_barrier();  // the next chunk rewrites this buffer
    }

    if (!spec) {
      // The next unit's copies are waited for here, before this unit's state
      // stores are issued: the wait then covers the copies and the few output
      // and window stores, and the state stores drain while the next unit is
      // computed.
      if (wait_next) vm_wait<0>();
      float* dst = state(a.ssm, slot) + lane_off;
#pragma unroll
      for (int p = 0; p < NR; ++p)
#pragma unroll
        for (int n = 0; n < CPL; ++n) st_stream(dst + p * DK + 4 * n * LPR, s[p][n]);
    }
  }
};

// Units of at most 16 rows per wave (single-head groups such as KDA's) have
// 64 KiB stages, so two workgroups share a CU when the registers allow four
// waves per SIMD.
template <int DK, int RPW, typename Act, bool KDA>
__global__ void __launch_bounds__(512, RPW <= 16 ? 4 : 2) decode_kernel(const DecodeArgs a) {
  using Cta = DecodeCta<DK, RPW, Act, KDA>;
  const Cta cta(a);
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const LdsPlan& P = cta.plan;
  float* const stage = lds + cta.wave * P.stage_per_wave;
  uint32_t* const raw0 = reinterpret_cast<uint32_t*>(lds + P.raw);
  float* const act0 = lds + P.act;
  int32_t* const slot_tab = reinterpret_cast<int32_t*>(lds + P.slots);

  // This workgroup serves key head kh for requests b0 + k*m, k < mine.
  const int mine = (a.B - cta.b0 + cta.m - 1) / cta.m;
  if (mine <= 0) return;

  // Once per workgroup: the slots of its units -- destination (an index
  // outside the pool marks a unit as skipped) and source (the destination
  // itself, a copy-on-write source, or negative for a zero start; a source
  // past the pool skips the unit) -- and the conv taps and bias of its
  // channels.
  for (int k = cta.tid; k < mine; k += cta.NT) {
    const int bk = cta.b0 + k * cta.m;
    int32_t sl = a.idx[bk];
    int32_t sr = a.init ? a.init[bk] : sl;
    if (sl < 0 || static_cast<int64_t>(sl) >= a.num_slots || static_cast<int64_t>(sr) >= a.num_slots)
      sl = -1;
    slot_tab[2 * k] = sl;
    slot_tab[2 * k + 1] = sr < 0 ? -1 : sr;
  }
  float wt[kMaxW1 + 1];
  float bias = 0.f;
  {
    const Act* wg = static_cast<const Act*>(a.w);
    const Act* bg = static_cast<const Act*>(a.bias);
#pragma unroll
    for (int j = 0; j <= kMaxW1; ++j)
      wt[j] = (cta.tid < cta.Cg && j >= cta.lead)
                  ? to_f32(wg[cta.chan * static_cast<uint32_t>(cta.W) + (j - cta.lead)])
                  : 0.f;
    if (bg && cta.tid < cta.Cg) bias = to_f32(bg[cta.chan]);
  }
  lds_barrier();

  int32_t sl = uniform(slot_tab[0]), sr = uniform(slot_tab[1]);
  if (sl >= 0) cta.copy_unit(cta.b0, sr, stage, raw0);
  f4 s[Cta::NR][Cta::CPL];
  bool waited = false;  // this unit's copies were waited for inside the previous run
  for (int k = 0; k < mine; ++k) {
    const int b = cta.b0 + k * cta.m;
    uint32_t* const raw = raw0 + (k & 1) * P.raw_len;
    // one activation buffer: the barrier above ends every wave's reads of
    // the previous unit's activations before this unit writes them
    float* const act = act0;
    // drain: this unit's copies (and the previous unit's stores) are done
    if (!waited) vm_wait<0>();
    if (sl >= 0) {
      if (sr >= 0) {
        cta.stage_read(stage, s);
        lgkm_wait();  // the stage is read before the next copy overwrites it
      } else {
#pragma unroll
        for (int p = 0; p < Cta::NR; ++p)
#pragma unroll
          for (int n = 0; n < Cta::CPL; ++n) s[p][n] = f4{0.f, 0.f, 0.f, 0.f};
      }
    }
    lds_barrier();  // every wave's copies of the shared raw inputs have landed
    int32_t sn = -1, srn = -1;
    if (k + 1 < mine) {
      sn = uniform(slot_tab[2 * (k + 1)]);
      srn = uniform(slot_tab[2 * (k + 1) + 1]);
    }
    if (sn >= 0) cta.copy_unit(b + cta.m, srn, stage, raw0 + ((k + 1) & 1) * P.raw_len);
    const bool early = sl >= 0 && sn >= 0 && !cta.spec;
    if (sl >= 0) cta.run(b, sl, s, wt, bias, raw, act, early);
    waited = early;
    sl = sn;
    sr = srn;
  }
}

// Dynamic LDS bytes of the decode kernel for a shape and token chunk.
size_t decode_lds_bytes(int dk, int rpw, int G, int dv, int W1, int kda, int tchunk,
                        int units = kMaxUnitsPerCta) {
  const int waves = G * dv / rpw;
  const int Cg = 2 * dk + G * dv;
  const LdsPlan p = lds_plan(dk, rpw, waves, Cg, W1, G * (kda ? dk : 1), G, tchunk, units);
  return sizeof(float) * static_cast<size_t>(p.total);
}

template <typename K>
hipError_t launch_one(K kernel, dim3 grid, int threads, size_t lds, hipStream_t s,
                      const DecodeArgs& a) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, grid, dim3(threads), lds, s, a);
  return hipGetLastError();
}

template <int DK, typename Act, bool KDA>
hipError_t launch_rpw(const DecodeArgs& a, int rpw, dim3 grid, size_t lds, hipStream_t s) {
  const int threads = 64 * (a.G * a.dv / rpw);
  switch (rpw) {
    case 32:
      if constexpr (32 % RowMap<DK>::RPP == 0)
        return launch_one(decode_kernel<DK, 32, Act, KDA>, grid, threads, lds, s, a);
      else
        return hipErrorInvalidValue;
    case 16:
      return launch_one(decode_kernel<DK, 16, Act, KDA>, grid, threads, lds, s, a);
    case 8:
      if constexpr (8 % RowMap<DK>::RPP == 0)
        return launch_one(decode_kernel<DK, 8, Act, KDA>, grid, threads, lds, s, a);
      else
        return hipErrorInvalidValue;
    default:
      return hipErrorInvalidValue;
  }
}

template <typename Act, bool KDA>
hipError_t launch_dk(const DecodeArgs& a, int dk, int rpw, dim3 grid, size_t lds,
                     hipStream_t s) {
  switch (dk) {
    case 16: return launch_rpw<16, Act, KDA>(a, rpw, grid, lds, s);
    case 32: return launch_rpw<32, Act, KDA>(a, rpw, grid, lds, s);
    case 64: return launch_rpw<64, Act, KDA>(a, rpw, grid, lds, s);
    case 128: return launch_rpw<128, Act, KDA>(a, rpw, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

int rows_per_pass(int dk) { return dk >= 64 ? 4 : 256 / dk; }

}  // namespace

// Rows of state per wave (32, 16 or 8; a divisor of d_v, so a wave stays in
// one value head) such that the group's G*d_v rows take at most 8 waves and
// there is a thread for every conv channel and every gate value of the
// group, with one token of LDS buffers fitting next to the state stages; 0
// when the shape is not supported.
int decode_rows_per_wave(int dk, int G, int dv, int W1, int kda) {
  const int rows = G * dv;
  const int channels = 2 * dk + rows;
  const int gates = G * (kda ? dk : 1);
  for (int rpw = 32; rpw >= 8; rpw >>= 1) {
    if (rpw % rows_per_pass(dk) || dv % rpw) continue;
    const int waves = rows / rpw;
    if (waves < 1 || waves > 8) continue;
    if (64 * waves < channels || 64 * waves < gates) continue;
    if (decode_lds_bytes(dk, rpw, G, dv, W1, kda, 1) > kLdsBytes) continue;
    return rpw;
  }
  return 0;
}

hipError_t launch_decode(const DecodeArgs& args, int dk, int act_bf16, int kda, hipStream_t s) {
  const int W1 = args.W - 1;
  const int rpw = decode_rows_per_wave(dk, args.G, args.dv, W1, kda);
  if (!rpw) return hipErrorInvalidValue;
  // persistent grid: H_k * m workgroups, m ~ 2 * (workgroups per CU) * CUs
  // / H_k -- twice what fits at once, so the dispatcher hands the second half
  // to whichever CUs finish first (per-XCD bandwidth differs from call to
  // call); at least one request per workgroup, at most kMaxUnitsPerCta units
  // each.  Workgroups per CU: what the LDS plan allows (2 for single-head
  // units such as KDA's 64 KiB stages, else 1).
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess || cus <= 0) return e != hipSuccess ? e : hipErrorInvalidDevice;
  const int per_cu =
      args.T == 1 && 2 * decode_lds_bytes(dk, rpw, args.G, args.dv, W1, kda, 1,
                                          (args.B + cus - 1) / cus) <= kLdsBytes
          ? 2
          : 1;
  int64_t m = 2 * per_cu * static_cast<int64_t>(cus) / args.Hk;
  if (m < 1) m = 1;
  const int64_t m_min = (args.B + kMaxUnitsPerCta - 1) / kMaxUnitsPerCta;
  if (m < m_min) m = m_min;
  if (m > args.B) m = args.B;
  // slot-table entries: the units of the busiest workgroup (a small table
  // lets two workgroups share a CU when the state stages allow it)
  const int units = static_cast<int>((args.B + m - 1) / m);
  // tokens whose activations are staged in LDS at once: what fits next to
  // the stages, raw buffers and slot table
  DecodeArgs a = args;
  int tc = 1;
  while (tc < args.T &&
         decode_lds_bytes(dk, rpw, args.G, args.dv, W1, kda, tc + 1, units) <= kLdsBytes)
    ++tc;
  a.tchunk = tc;
  const size_t lds = decode_lds_bytes(dk, rpw, args.G, args.dv, W1, kda, tc, units);
  const int64_t ctas = m * args.Hk;
  if (ctas < 1 || ctas > INT32_MAX) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(ctas));
  if (act_bf16)
    return kda ? launch_dk<bf16, true>(a, dk, rpw, grid, lds, s)
               : launch_dk<bf16, false>(a, dk, rpw, grid, lds, s);
  return kda ? launch_dk<float, true>(a, dk, rpw, grid, lds, s)
             : launch_dk<float, false>(a, dk, rpw, grid, lds, s);
}

}  // namespace gdn
