// gdn_decode.hip -- fused decode step for Gated DeltaNet / KDA on gfx950.
//
// Work unit: one (request b, key head kh), one workgroup.  A unit owns the q
// and k conv channels of kh, the v channels of its G = H_v/H_k value heads
// and the G*d_v state rows of those heads, so it is the only reader and
// writer of every conv-window channel it touches: no cross-workgroup
// ordering exists.
//
// Schedule.  Each workgroup is small in LDS (the activations of a few
// tokens) and in registers.  The first three quarters of the units are
// fixed, a block of requests per XCD; with the caller's work counter the
// rest go out by ticket to the workgroups that start next, so XCDs that
// stream faster take more of them (decode_unit); without it every unit is
// fixed.  Units of up to 64 KiB of state run two per CU (one's stores drain
// while the other's loads stream in); larger ones one per CU, which keeps
// fewer requests queued at HBM and measures faster.
// Within a unit the slot lookups and the first-token inputs (x, taps,
// gates, betas, then the source slot's conv window) are issued first and
// the state rows, straight into registers, right after them; loads complete
// in order, so the conv and the norms run while the state streams in.
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
// chunks and a lane group owns NR consecutive rows, so each load or store
// instruction of a wave covers whole 128-byte lines and every state access
// of a lane is one base address plus an immediate offset.  State traffic is
// non-temporal: each slot is touched once per call.
//
// Bitwise contract: the in-place path (no snapshots) and the snapshot paths
// run the same instantiation and the same per-token arithmetic (built with
// -ffp-contract=off, explicit fmaf), so a draft of T tokens followed by a
// commit of L equals an in-place decode of L tokens bit for bit.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kMaxW1 = 3;     // conv_width <= 4
constexpr int kBatch = 2;     // later tokens whose x are loaded together
constexpr int kMaxChunk = 8;  // tokens whose activations sit in LDS at once
constexpr size_t kHalfLds = 80 * 1024;  // half the LDS of a gfx950 CU

// Lane layout of a state row of d_k fp32: LPR lanes, each holding CPL 16-byte
// chunks (chunk n*LPR + lc in lane lc); one instruction of a wave covers
// RPP rows x LPR*16 contiguous bytes.
template <int DK>
struct RowMap {
  static constexpr int LPR = DK >= 64 ? 16 : DK / 4;  // lanes per state row
  static constexpr int CPL = DK / (4 * LPR);          // 16-byte chunks per lane
  static constexpr int RPP = 64 / LPR;                // rows per wave per pass
};

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
  int kh, b;        // this workgroup's unit: key head kh of request b
  bool spec;        // snapshots per token instead of an in-place update
  bool spec_pool;   // ... into pool slots named by a.spec_slots
  int64_t slot_elems;
  uint32_t lane_off;  // this lane's first state element within a unit
  uint32_t chan;      // global conv channel of this thread (tid < Cg)

  __device__ __forceinline__ DecodeCta(const DecodeArgs& args, int unit) : a(args) {
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
    per_tok = (Cg + GA + G + 4 + 3) & ~3;  // 16-byte aligned token records
    kh = unit % Hk;
    b = unit / Hk;
    spec_pool = a.spec_slots != nullptr;
    spec = spec_pool || a.spec_ssm != nullptr;
    slot_elems = static_cast<int64_t>(Hv) * dv * DK;
    lane_off = static_cast<uint32_t>(wave * RPW + lr * NR) * DK + 4 * lc;
    chan = channel(tid < Cg ? tid : 0);
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

  // First-token inputs of this thread as raw bits (zero-extended storage
  // words): conv taps, bias, window and x of its channel (tid < Cg), and
  // the gate or beta value of index tid (tid < GA + G).  Every load is a
  // buffer load; whatever does not apply (a lane past the channels or gates,
  // a tap or window column before the first, no bias, a fresh start) reads
  // past its descriptor and so is zero, with no branch or select in the way
  // of the loads.
  struct Raw {
    uint32_t wt[kMaxW1 + 1], bias, win[kMaxW1], x0, al, be;
  };
  static constexpr uint32_t kAct = sizeof(Act);
  __device__ __forceinline__ static uint32_t raw_word(rsrc_t r, uint32_t off) {
    if constexpr (sizeof(Act) == 2)
      return static_cast<uint16_t>(__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
    else
      return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
  __device__ __forceinline__ static float raw_f32(uint32_t d) {
    if constexpr (sizeof(Act) == 2)
      return __uint_as_float(d << 16);
    else
      return __uint_as_float(d);
  }
  // Everything but the window (whose slot is not known yet).
  __device__ __forceinline__ void load_fixed(Raw& r) const {
    const bool ch = tid < Cg;
    const rsrc_t w = make_rsrc(a.w, static_cast<uint32_t>(C) * W * kAct);
    const rsrc_t bs = make_rsrc(a.bias ? a.bias : a.w, a.bias ? static_cast<uint32_t>(C) * kAct : 0u);
    const rsrc_t x = make_rsrc(static_cast<const Act*>(a.x) + static_cast<int64_t>(b) * T * C,
                               static_cast<uint32_t>(C) * kAct);
    const int64_t th = static_cast<int64_t>(b) * T * Hv + static_cast<int64_t>(kh) * G;
    const rsrc_t al = make_rsrc(static_cast<const Act*>(a.alpha) + th * DKA,
                                static_cast<uint32_t>(GA) * kAct);
    const rsrc_t be = make_rsrc(static_cast<const Act*>(a.beta) + th, static_cast<uint32_t>(G) * kAct);
#pragma unroll
    for (int j = 0; j <= kMaxW1; ++j)
      r.wt[j] = raw_word(w, (ch && j >= lead) ? (chan * W + (j - lead)) * kAct : kOutOfRange);
    r.bias = raw_word(bs, ch ? chan * kAct : kOutOfRange);
    r.x0 = raw_word(x, ch ? chan * kAct : kOutOfRange);
    r.al = raw_word(al, tid < GA ? tid * kAct : kOutOfRange);
    r.be = raw_word(be, (tid >= GA && tid < GA + G) ? (tid - GA) * kAct : kOutOfRange);
  }
  // The window of the source slot.
  __device__ __forceinline__ void load_window(int32_t src, Raw& r) const {
    const bool on = src >= 0 && W1 > 0;
    const rsrc_t cw = make_rsrc(
        on ? static_cast<const Act*>(a.conv) + static_cast<int64_t>(src) * W1 * C : a.x,
        on ? static_cast<uint32_t>(W1) * C * kAct : 0u);
#pragma unroll
    for (int j = 0; j < kMaxW1; ++j)
      r.win[j] = raw_word(cw, (tid < Cg && j >= lead)
                                  ? (static_cast<uint32_t>(j - lead) * C + chan) * kAct
                                  : kOutOfRange);
  }
  // The raw words as values.
  __device__ __forceinline__ void inputs(const Raw& r, float (&wt)[kMaxW1 + 1], float& bias,
                                         float (&win)[kMaxW1], float& x0, float& g0) const {
#pragma unroll
    for (int j = 0; j <= kMaxW1; ++j) wt[j] = raw_f32(r.wt[j]);
    bias = raw_f32(r.bias);
#pragma unroll
    for (int j = 0; j < kMaxW1; ++j) win[j] = raw_f32(r.win[j]);
    x0 = raw_f32(r.x0);
    g0 = raw_f32(r.al | r.be);  // at most one of the two is non-zero
  }

  // This lane's state rows of the unit's source slot; a fresh start reads
  // past an empty descriptor, i.e. zeros, with no memory traffic.
  __device__ __forceinline__ void load_state(int32_t src, f4 (&s)[NR][CPL]) const {
    const rsrc_t st = make_rsrc(state(a.ssm, src >= 0 ? src : 0),
                                src >= 0 ? static_cast<uint32_t>(R) * DK * 4u : 0u);
#pragma unroll
    for (int r = 0; r < NR; ++r)
#pragma unroll
      for (int n = 0; n < CPL; ++n)
        s[r][n] = __builtin_bit_cast(
            f4, __builtin_amdgcn_raw_buffer_load_b128(
                    st, (lane_off + r * DK + 4 * n * LPR) * 4u, 0, 2 /* non-temporal */));
  }

  // Where token t's snapshot goes (null: nowhere): a row of the spec cache,
  // or the pool slot the spec slot table names for it (skipped when outside
  // the pool).
  __device__ __forceinline__ int32_t spec_slot(int t) const {
    const int32_t sl = a.spec_slots[static_cast<int64_t>(b) * a.t_max + t];
    return (sl < 0 || static_cast<int64_t>(sl) >= a.num_slots) ? -1 : sl;
  }
  __device__ __forceinline__ Act* snap_conv(int t) const {
    if (spec_pool) {
      const int32_t sl = spec_slot(t);
      return sl < 0 ? nullptr : static_cast<Act*>(a.conv) + static_cast<int64_t>(sl) * W1 * C;
    }
    return static_cast<Act*>(a.spec_conv) + (static_cast<int64_t>(b) * a.t_max + t) * W1 * C;
  }
  __device__ __forceinline__ float* snap_ssm(int t) const {
    if (spec_pool) {
      const int32_t sl = spec_slot(t);
      return sl < 0 ? nullptr : state(a.ssm, sl);
    }
    return state(a.spec_ssm, static_cast<int64_t>(b) * a.t_max + t);
  }

  // D1 for one token t of this thread's channel: conv over the window and
  // x, window shift, SiLU; the activation goes to act[tid]; the shifted
  // window goes to the snapshot of token t (spec) or, after the last token,
  // back to the slot.
  __device__ __forceinline__ void conv_token(int t, float xv, const float (&wt)[kMaxW1 + 1],
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
      wdst = snap_conv(t);
    else if (t == T - 1)
      wdst = conv_slot;
    if (wdst) {
#pragma unroll
      for (int j = 0; j < kMaxW1; ++j)
        if (j >= lead) wdst[static_cast<uint32_t>(j - lead) * C + chan] = from_exact<Act>(win[j]);
    }
  }

  // Run the T tokens of the unit on its state rows s and write the state to
  // slot (in place) or the snapshots.  x0 / win / g0 are this thread's
  // first-token inputs; act is the unit's activation buffer in LDS.
  __device__ __forceinline__ void run(int32_t slot, f4 (&s)[NR][CPL],
                                      const float (&wt)[kMaxW1 + 1], float bias, float x0,
                                      float (&win)[kMaxW1], float g0, float* act) const {
    const int64_t tok0 = static_cast<int64_t>(b) * T;
    const Act* const x_req = static_cast<const Act*>(a.x) + tok0 * C;
    Act* const conv_slot = static_cast<Act*>(a.conv) + static_cast<int64_t>(slot) * W1 * C;
    const Act* const al_req =
        static_cast<const Act*>(a.alpha) + (tok0 * Hv + static_cast<int64_t>(kh) * G) * DKA;
    const Act* const be_req =
        static_cast<const Act*>(a.beta) + tok0 * Hv + static_cast<int64_t>(kh) * G;
    float* const out_req = a.out + (tok0 * Hv + static_cast<int64_t>(kh) * G) * dv;

    for (int t0 = 0; t0 < T; t0 += TC) {
      const int nt = T - t0 < TC ? T - t0 : TC;

      // ---- D1: conv update + activation of the unit's channels for the nt
      // tokens of this chunk, into LDS; gates and betas alongside.
      // token 0 from the inputs already in registers
      const int first = t0 == 0 ? 1 : 0;
      if (first) {
        if (tid < Cg) conv_token(0, x0, wt, win, bias, act, conv_slot);
        if (tid < GA + G) act[Cg + tid] = g0;
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
            conv_token(t0 + tb + k, xr[k], wt, win, bias, act + (tb + k) * per_tok, conv_slot);
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
        // where the rows go after this token: the snapshot of token t (spec),
        // the slot after the last token (in place), or nowhere yet; each row
        // is stored as soon as it is updated
        float* rows_dst = nullptr;
        if (spec)
          rows_dst = snap_ssm(t);
        else if (t == T - 1)
          rows_dst = state(a.ssm, slot);
        if (rows_dst) rows_dst += lane_off;
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
          if (rows_dst) {
#pragma unroll
            for (int n = 0; n < CPL; ++n) st_stream(rows_dst + p * DK + 4 * n * LPR, s[p][n]);
          }
        }
      }
      if (t0 + TC < T) lds_barrier();  // the next chunk rewrites this buffer
    }
  }
};

// The unit of this workgroup, or -1 for none.  Workgroup x runs on XCD
// x mod 8 (the dispatcher deals workgroups out round-robin over the XCDs).
// The first nstatic units are fixed: XCD k is given the k-th eighth of them
// (a block of requests with all their key heads), in order.  With the
// caller's work counter, the rest are handed out by ticket: each of the
// nticket workgroups after them draws one when it starts, so XCDs that run
// ahead take more of the tail (XCDs of one MI355X differ by up to ~10 % in
// how fast they stream); the workgroup that draws the last ticket puts the
// counter back to zero, and those past the last unit exit.  Without a
// counter every unit is fixed.
__device__ __forceinline__ int decode_unit(const DecodeArgs& a, int& drawn) {
  const unsigned x = blockIdx.x;
  const unsigned nfix = a.work ? static_cast<unsigned>(a.nstatic) : gridDim.x;
  if (x < nfix) {
    const unsigned q = nfix >> 3;
    return static_cast<int>(x < 8 * q ? (x & 7) * q + (x >> 3) : x);
  }
  if (threadIdx.x == 0) {
    const unsigned t = atomicAdd(a.work, 1u);
    if (t == static_cast<unsigned>(a.nticket) - 1) atomicExch(a.work, 0u);
    const int64_t u = static_cast<int64_t>(a.nstatic) + t;
    drawn = u < static_cast<int64_t>(a.B) * a.Hk ? static_cast<int>(u) : -1;
  }
  __syncthreads();
  return uniform(drawn);
}

// At most 128 registers per lane: room for two 8-wave workgroups per CU
// (units of 128 KiB of state run one per CU, see launch_decode).
template <int DK, int RPW, typename Act, bool KDA>
__global__ void __launch_bounds__(512, 4) decode_kernel(const DecodeArgs a) {
  using Cta = DecodeCta<DK, RPW, Act, KDA>;
  extern __shared__ __attribute__((aligned(16))) float act[];
  __shared__ int drawn;
  const int unit = decode_unit(a, drawn);
  if (unit < 0) return;

  // The unit's destination slot (an index outside the pool skips the unit)
  // and source slot (the destination itself, a copy-on-write source, or
  // negative for a zero start; a source past the pool skips the unit).
  // Both lookups go out first and together, as scalar loads (the index
  // arrays are only read here), then the inputs that need no slot; the
  // workgroup waits for the lookups alone.
  typedef const __attribute__((address_space(4))) int32_t* const_i32;
  const int b = unit / a.Hk;
  const int32_t* srcs = a.init ? a.init : a.idx;
  const int32_t sl = ((const_i32)a.idx)[b];
  const int32_t sr_in = ((const_i32)srcs)[b];
  const Cta cta(a, unit);
  typename Cta::Raw raw;
  cta.load_fixed(raw);
  asm volatile("" ::: "memory");
  if (sl < 0 || static_cast<int64_t>(sl) >= a.num_slots ||
      static_cast<int64_t>(sr_in) >= a.num_slots)
    return;
  const int32_t sr = sr_in < 0 ? -1 : sr_in;
  cta.load_window(sr, raw);
  // The state loads follow the inputs (loads complete in order, so the conv
  // waits for the inputs alone); the conv and the norms run while the state
  // streams in.
  asm volatile("" ::: "memory");
  f4 s[Cta::NR][Cta::CPL];
  cta.load_state(sr, s);
  asm volatile("" ::: "memory");
  float wt[kMaxW1 + 1], win[kMaxW1], bias, x0, g0;
  cta.inputs(raw, wt, bias, win, x0, g0);
  cta.run(sl, s, wt, bias, x0, win, g0, act);
}

// Dynamic LDS bytes of the decode kernel: the activations of tchunk tokens.
size_t decode_lds_bytes(int dk, int G, int dv, int kda, int tchunk) {
  const int per_tok = (2 * dk + G * dv + G * (kda ? dk : 1) + G + 4 + 3) & ~3;
  return sizeof(float) * static_cast<size_t>(tchunk) * per_tok;
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
// group; 0 when the shape is not supported.
int decode_rows_per_wave(int dk, int G, int dv, int W1, int kda) {
  const int rows = G * dv;
  const int channels = 2 * dk + rows;
  const int gates = G * (kda ? dk : 1);
  if (W1 < 0 || W1 > kMaxW1) return 0;
  for (int rpw = 32; rpw >= 8; rpw >>= 1) {
    if (rpw % rows_per_pass(dk) || dv % rpw) continue;
    const int waves = rows / rpw;
    if (waves < 1 || waves > 8) continue;
    if (64 * waves < channels || 64 * waves < gates + G) continue;
    return rpw;
  }
  return 0;
}

hipError_t launch_decode(const DecodeArgs& args, int dk, int act_bf16, int kda, hipStream_t s) {
  const int W1 = args.W - 1;
  const int rpw = decode_rows_per_wave(dk, args.G, args.dv, W1, kda);
  if (!rpw) return hipErrorInvalidValue;
  const int64_t units = static_cast<int64_t>(args.B) * args.Hk;
  if (units < 1 || units > INT32_MAX) return hipErrorInvalidValue;
  DecodeArgs a = args;
  a.tchunk = args.T < kMaxChunk ? args.T : kMaxChunk;
  // Units of 128 KiB of state or more run one workgroup per CU, reserved
  // through LDS: two such units per CU queue more requests than HBM serves
  // well (Qwen3.5 shape, B=64: 50.5 us against 51.9 us with two); 64 KiB
  // units are fastest two per CU (51.9 us against 54.9 us with one).
  const int64_t unit_bytes = static_cast<int64_t>(args.G) * args.dv * dk * 4;
  size_t lds = decode_lds_bytes(dk, args.G, args.dv, kda, a.tchunk);
  if (unit_bytes >= 128 * 1024 && lds < kHalfLds + 16) lds = kHalfLds + 16;
  // With the caller's work counter the last quarter of the units goes out by
  // ticket (Qwen3.5 shape, B=64: 49.4-50.1 us against 50.6-51.2 us with every
  // unit fixed), with half again as many ticket workgroups as tail units so
  // that fast XCDs can take up to 1.5x their share.
  int64_t nwg = units;
  if (a.work) {
    a.nstatic = static_cast<int32_t>((units - units / 4) / 8 * 8);
    const int64_t tail = units - a.nstatic;
    a.nticket = static_cast<int32_t>(tail + tail / 2);
    nwg = a.nstatic + a.nticket;
    if (nwg > INT32_MAX) return hipErrorInvalidValue;
  }
  const dim3 grid(static_cast<unsigned>(nwg));
  if (act_bf16)
    return kda ? launch_dk<bf16, true>(a, dk, rpw, grid, lds, s)
               : launch_dk<bf16, false>(a, dk, rpw, grid, lds, s);
  return kda ? launch_dk<float, true>(a, dk, rpw, grid, lds, s)
             : launch_dk<float, false>(a, dk, rpw, grid, lds, s);
}

}  // namespace gdn
