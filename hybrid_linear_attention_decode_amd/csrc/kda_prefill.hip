// kda_prefill.hip -- chunked prefill of the delta rule with a per-channel
// decay (Kimi Delta Attention) on gfx950.
//
// The recurrence S_t = S_{t-1} diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = S_t q_t, a_t in [0, 1]^{d_k} (one decay per key channel), evaluated
// 64 tokens at a time in the WY / UT form of the delta rule (Yang et al.,
// "Parallelizing Linear Transformers with the Delta Rule over Sequence
// Length", 2024, sec. 3) with the fine-grained gate of Kimi Delta Attention.
// With g_t = sum_{s <= t} log a_s (per channel, inside the chunk):
//   A_ri = b_r sum_c k_rc k_ic e^{g_rc - g_ic}          (i < r)
//   P_ri =     sum_c q_rc k_ic e^{g_rc - g_ic}          (i <= r)
//   (I + A) U = diag(b) (V - (K o e^g) S0^T)
//   O = (Q o e^g) S0^T + P U
//   S^T = diag(e^{g_c}) S0^T + (K o e^{g_c - g})^T U
// A per-channel decay does not factor out of the products as a row scale,
// and e^{-g} overflows fp32 after a few strongly decaying tokens, so every
// factor is taken relative to a 16-token block boundary and stays <= 1:
// for token t in block R (boundary b_R = the token before the block),
//   E_t = prod_{b_R < s <= t} a_s,  F_t = prod_{t < s <= last of R} a_s,
//   Lam_R = prod over the whole block R;
//   KE = K o E, QE = Q o E, KF = K o F (bf16 hi/lo planes in LDS);
//   off-diagonal block pair (R, I), I < R:
//     A_RI = diag(b_R) KE_R diag(D_RI) KF_I^T,  P_RI = QE_R diag(D_RI) KF_I^T,
//     D_RI = prod_{I < J < R} Lam_J;
//   K o e^g on block R = KE_R diag(e^{G_R}), e^{G_R} = prod_{J < R} Lam_J,
//     applied to S0^T instead (a per-channel scale of the contraction);
//   K o e^{g_c - g} on block I = KF_I diag(f_I), f_I = prod_{J > I} Lam_J,
//     applied to the block's partial sum of the state update.
// The four diagonal 16 x 16 blocks need e^{g_r - g_i} inside one block, which
// has no bounded factorisation; they are formed exactly, with products of
// the decays, by a first kernel (kda_diag_kernel) that also inverts each
// block of I + A with the nilpotent product series on MFMA that the
// scalar-decay kernel uses.  The second kernel
// (kda_chunk_kernel) has the work split and pipeline of the scalar-decay
// kernel (gdn_prefill.hip): producers prepare the next chunk (conv1d, SiLU,
// L2 norm, the decay products and the three planes), all waves form the six
// off-diagonal blocks, and four consumer waves carry 16 value columns each.
#include "prefill_common.hpp"

namespace gdn {
namespace {

constexpr int kBlk = 16;           // tokens per diagonal block
constexpr int kWsBlockBytes = 2048;  // one diagonal block: X, P as (hi, lo)

// Workspace block of token block jb of sequence s (start t0): sequences are
// laid out at floor(t0 / 16) + 4 min(s, t0) blocks, which leaves room for
// their 4 ceil(T / 64) blocks whatever the lengths; the whole call needs
// floor(total / 16) + 4 min(N, total) blocks per value head.
__device__ __forceinline__ int64_t ws_block(int s, int t0, int jb) {
  return static_cast<int64_t>(t0 / kBlk) + 4 * static_cast<int64_t>(s < t0 ? s : t0) + jb;
}

// =====================================================================
// Kernel 1: the diagonal 16 x 16 blocks, workgroups of four waves per
// (sequence, value head); workgroup y of gridDim.y takes the token blocks y,
// y + gridDim.y, ... of its sequence in turn.  Workspace record (2 KiB): lane
// l = 4 r + q holds columns 4q..4q+3 of row r as X hi, X lo, P hi, P lo (4
// bf16 each), where X = (I + N)^{-1}, N_ri = b_r sum_c k_rc k_ic
// prod_{i < s <= r} a_sc (i < r), and P_ri = sum_c q_rc k_ic
// prod_{i < s <= r} a_sc (i <= r).
// =====================================================================
constexpr int kDiagThreads = 256;
// Token blocks per workgroup: the workgroup's set-up (taps and bias into
// LDS, the pair stage's addresses) is paid once for all of them.  4 x 8192
// tokens of a KDA layer, whole call: 1, 2, 4, 8 blocks per workgroup took
// 2.13-2.14, 2.06-2.08, 2.07-2.08, 2.03 ms on one MI355X; 8, 16, 32 took
// 2.07, 2.08-2.10, 2.09 ms on another.
constexpr int kDiagPer = 8;
constexpr int kDiagMinGroups = 2048;   // ... unless that leaves fewer workgroups

// Rows of q, k and the decays in LDS: DK floats, the 16-byte chunk index of
// odd rows XOR 8 (d_k >= 64), so two consecutive rows read at the same
// chunk fall in opposite halves of the banks.
template <int DK>
__device__ __forceinline__ int diag_at(int r, int c) {
  if constexpr (DK >= 64)
    return r * DK + (((c >> 2) ^ ((r & 1) << 3)) << 2) + (c & 3);
  else
    return r * DK + c;
}

template <int DK>
struct DiagPlan {
  static constexpr int kRow = DK;                // fp32 per row of q, k, a
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + kBlk * kRow * 4;
  static constexpr int oA = oK + kBlk * kRow * 4;
  static constexpr int oN = oA + kBlk * kRow * 4;  // fp32 [16][16]
  static constexpr int oP = oN + kBlk * kBlk * 4;
  static constexpr int oRed = oP + kBlk * kBlk * 4;  // fp32 [4 waves][2][17][8] partial sums
  static constexpr int oBeta = oRed + 4 * 2 * 17 * 8 * 4;
  // conv taps (f4) and bias of the head's q and k channels, [m][octet]
  static constexpr int oW = oBeta + kBlk * 4;
  static constexpr int oB = oW + 2 * DK * 16;
  static constexpr int kBytes = oB + 2 * DK * 4;
};

// DKR: the layer's d_k; DK the layout it runs in (32 for d_k = 16, whose
// channels from DKR on are padding: zero q, k, taps and bias, decay 1).
template <int DK, typename Act, int DKR>
__global__ void __launch_bounds__(kDiagThreads, 4) kda_diag_kernel(PrefillArgs a) {
  using DP = DiagPlan<DK>;
  constexpr int kGrp = DK / 8;        // channel octets per head
  constexpr int kItems = 2 * kGrp * kBlk;   // (q|k octet, token) conv items
  constexpr int kNg = DK / 4;         // groups of 4 channels in the pair stage
  constexpr int kWaves = (kNg + 7) / 8;     // waves taking part in the pair stage
  __shared__ __align__(16) unsigned char lds[DP::kBytes];
  float* yq = reinterpret_cast<float*>(lds + DP::oQ);
  float* yk = reinterpret_cast<float*>(lds + DP::oK);
  float* al = reinterpret_cast<float*>(lds + DP::oA);
  float* nm = reinterpret_cast<float*>(lds + DP::oN);
  float* pm = reinterpret_cast<float*>(lds + DP::oP);
  float* red = reinterpret_cast<float*>(lds + DP::oRed);
  float* bt = reinterpret_cast<float*>(lds + DP::oBeta);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = blockIdx.x / a.Hv, h = blockIdx.x % a.Hv;
  const int t0 = a.cu[s], t1 = a.cu[s + 1];
  const int32_t dst = a.dst[s];
  const int32_t init = a.init ? a.init[s] : dst;
  if (t0 < 0 || t1 < t0 || t1 > a.total || dst < 0 || dst >= a.num_slots || init >= a.num_slots)
    return;
  const int T = t1 - t0;
  const int nb = 4 * ((T + kC - 1) / kC);
  if (static_cast<int>(blockIdx.y) >= nb) return;

  PrefillCore<DK, Act> core{a, lds};
  core.t0 = t0;
  core.T = T;
  core.init = init;
  core.h = h;
  core.hk = h / a.G;

  // conv stage: item = co + 2 kGrp * token (co: channel octet of q | k), so
  // the kGrp octets of one head and token are consecutive lanes
  const int co = tid % (2 * kGrp);
  const bool isk = co >= kGrp;
  const int oc = isk ? co - kGrp : co;
  const int ch = (isk ? a.Hk * DKR : 0) + core.hk * DKR + 8 * oc;
  constexpr bool kPad = DKR < DK;
  const bool pad_item = kPad && 8 * oc >= DKR;   // an octet of padding: its rows read zero
  // decay stage: item = (token r, channel octet)
  // pair stage: lane = (column pair cp, channel group cg of 4 channels);
  // columns cp and 15 - cp take 17 (row, column) steps in all
  const int cp = (tid >> 3) & 7, cg = (tid & 7) + 8 * wave;
  for (int i = tid; i < 2 * kBlk * kBlk; i += kDiagThreads) nm[i] = 0.f;  // upper parts stay 0
  float* wl = reinterpret_cast<float*>(lds + DP::oW);
  float* bl = reinterpret_cast<float*>(lds + DP::oB);
  for (int i = tid; i < 2 * DK; i += kDiagThreads) {
    const int ih = i < DK ? i : i - DK;
    const int c = i < DK ? core.hk * DKR + i : a.Hk * DKR + core.hk * DKR + (i - DK);
    const int at = (i & 7) * (2 * kGrp) + (i >> 3);
    const bool on = !kPad || ih < DKR;
    *reinterpret_cast<f4*>(wl + 4 * at) =
        on ? f4{core.tap(c, 0), core.tap(c, 1), core.tap(c, 2), core.tap(c, 3)}
           : f4{0.f, 0.f, 0.f, 0.f};
    bl[at] = (on && a.bias) ? to_f32(static_cast<const Act*>(a.bias)[c]) : 0.f;
  }

  lds_barrier();                // taps and bias in LDS
  for (int jb = blockIdx.y; jb < nb; jb += gridDim.y) {
    const int tb = jb * kBlk;   // first token of the block
    const int n = T - tb < kBlk ? (T > tb ? T - tb : 0) : kBlk;
    // ---- conv1d + SiLU + L2 norm of q and k, one token per item ----
    {
      const rsrc_t rx = core.x_rows(tb);
      const rsrc_t rw = core.win_rows();
#pragma unroll
      for (int it = 0; it < (kItems + kDiagThreads - 1) / kDiagThreads; ++it) {
        const int item = tid + it * kDiagThreads;
        if (item < kItems) {    // whole waves: kItems is a multiple of 64 or all of one wave
          const int tok = item / (2 * kGrp);
          Row8<Act> raw[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            raw[r].load(rx, pad_item ? static_cast<int>(kOutOfRange)
                                     : core.x_off(tb, tb + tok - 3 + r, ch));
            if (tb == 0) {
              Row8<Act> wr;
              wr.load(rw, pad_item ? static_cast<int>(kOutOfRange)
                                   : core.win_off(tok - 3 + r, ch));
              raw[r].merge(wr);
            }
          }
          float y[8], ss = 0.f;
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            const f4 wt = *reinterpret_cast<const f4*>(wl + 4 * (m * 2 * kGrp + co));
            float v = bl[m * 2 * kGrp + co];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) v = fmaf(wt[jj], raw[jj].get(m), v);
            v = core.act(v);
            y[m] = v;
            ss = fmaf(v, v, ss);
          }
          const float sum = group_sum<kGrp>(ss);
          float sc = a.l2norm ? rsqrtf(sum + a.eps) : 1.0f;
          if (!isk) sc *= a.q_scale;
          if (tb + tok >= T) sc = 0.f;
          float* yb = isk ? yk : yq;
          *reinterpret_cast<f4*>(yb + diag_at<DK>(tok, 8 * oc)) = f4{y[0], y[1], y[2], y[3]} * sc;
          *reinterpret_cast<f4*>(yb + diag_at<DK>(tok, 8 * oc + 4)) = f4{y[4], y[5], y[6], y[7]} * sc;
        }
      }
    }
    // ---- decays (1 past the sequence) and b ----
    {
      const int64_t rowe = static_cast<int64_t>(a.Hv) * DKR;
      const rsrc_t ra = make_rsrc(static_cast<const Act*>(a.alpha) + (t0 + static_cast<int64_t>(tb)) * rowe,
                                  static_cast<uint32_t>(n * rowe * sizeof(Act)));
      if (tid < kBlk * (DK / 8)) {
        const int r = tid / (DK / 8), c = 8 * (tid % (DK / 8));
        const bool real = !kPad || c < DKR;   // padding decays by 1
        const bool on = r < n && real;
        Row8<Act> v;
        v.load(ra, real ? static_cast<int>(((r * a.Hv + h) * DKR + c) * sizeof(Act))
                        : static_cast<int>(kOutOfRange));
        f4 lo4, hi4;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          lo4[m] = on ? v.get(m) : 1.f;
          hi4[m] = on ? v.get(m + 4) : 1.f;
        }
        *reinterpret_cast<f4*>(al + diag_at<DK>(r, c)) = lo4;
        *reinterpret_cast<f4*>(al + diag_at<DK>(r, c + 4)) = hi4;
      }
      if (tid < kBlk)
        bt[tid] = tid < n ? to_f32(static_cast<const Act*>(a.beta)[(t0 + static_cast<int64_t>(tb) + tid) * a.Hv + h])
                          : 0.f;
    }
    lds_barrier();
    // ---- N and P by products of the decays; partial sums per wave, per
    // step straight to LDS (no accumulator arrays held across the steps) ----
    if (wave < kWaves) {
      const bool on = cg < kNg;
      f4 w = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int st = 0; st < 17; ++st) {
        const bool first = st < 16 - cp;
        const int i = first ? cp : 15 - cp;
        const int r = first ? cp + st : st - 1;
        const int off = diag_at<DK>(r, 4 * (on ? cg : 0));
        const f4 kv = *reinterpret_cast<const f4*>(yk + off);
        const f4 qv = *reinterpret_cast<const f4*>(yq + off);
        const f4 av = *reinterpret_cast<const f4*>(al + off);
        const bool start = r == i;
        float sn = 0.f, sp = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          w[m] = start ? kv[m] : w[m] * av[m];
          sn = fmaf(kv[m], w[m], sn);
          sp = fmaf(qv[m], w[m], sp);
        }
        sn = group_sum<8>(on ? sn : 0.f);
        sp = group_sum<8>(on ? sp : 0.f);
        if ((tid & 7) == 0) {
          red[((wave * 2 + 0) * 17 + st) * 8 + cp] = sn;
          red[((wave * 2 + 1) * 17 + st) * 8 + cp] = sp;
        }
      }
    }
    lds_barrier();
    // ---- totals over the waves -> N (times b_r) and P ----
    for (int e = tid; e < 2 * 17 * 8; e += kDiagThreads) {
      const int which = e / (17 * 8), st = (e / 8) % 17, cpe = e % 8;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red[((w * 2 + which) * 17 + st) * 8 + cpe];
      const bool first = st < 16 - cpe;
      const int i = first ? cpe : 15 - cpe;
      const int r = first ? cpe + st : st - 1;
      if (which == 0) {
        if (r > i) nm[r * kBlk + i] = bt[r] * v;
      } else {
        pm[r * kBlk + i] = v;
      }
    }
    lds_barrier();
    // ---- X = (I + N)^{-1} on MFMA, and the record (wave 0) ----
    if (wave == 0) {
      const int lr = lane & 15, lg = lane >> 4;
      f4 na, nbv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        na[v] = nm[lr * kBlk + 4 * lg + v];
        nbv[v] = nm[(4 * lg + v) * kBlk + lr];
      }
      const f4 xv = unit_lower_inverse(na, nbv, lr, lg);      // X[lr][4 lg + v]
      const f4 pv = *reinterpret_cast<const f4*>(pm + lr * kBlk + 4 * lg);
      s4 xh, xl, ph, pl;
      split4(xv, xh, xl);
      split4(pv, ph, pl);
      typedef uint32_t u4 __attribute__((ext_vector_type(4)));
      unsigned char* rec = static_cast<unsigned char*>(a.ws) +
                           (ws_block(s, t0, jb) * a.Hv + h) * kWsBlockBytes + (4 * lr + lg) * 32;
      *reinterpret_cast<u4*>(rec) = __builtin_bit_cast(u4, cat(xh, xl));
      *reinterpret_cast<u4*>(rec + 16) = __builtin_bit_cast(u4, cat(ph, pl));
    }
    lds_barrier();  // the next block reuses the LDS
  }
}

// =====================================================================
// Kernel 2: the chunk scan.
// =====================================================================
// LDS plan (bytes).  KE, QE, KF planes ([token][d_k] bf16 hi and lo, rows
// per QkRow, staggered by 64 bytes); P and A ([token][token] bf16 hi and lo,
// rows padded by 16 bytes); b per token; per-channel fp32 vectors: block
// decays Lam_0..3, then e^{G_1..3}, e^{G_4} (the chunk's decay), f_0..2;
// conv taps and bias of the key head's q and k channels.
template <int DK>
struct KdaPlan {
  static constexpr int kRowQK = QkRow<DK>::kElems;
  static constexpr int kRowT = kC + 8;
  static constexpr int kQK = 2 * kC * kRowQK + 64;
  static constexpr int kSq = 2 * kC * kRowT;
  static constexpr int oEKh = 0, oEKl = oEKh + kQK, oEQh = oEKl + kQK, oEQl = oEQh + kQK;
  static constexpr int oFKh = oEQl + kQK, oFKl = oFKh + kQK;
  static constexpr int oPh = oFKl + kQK, oPl = oPh + kSq, oAh = oPl + kSq, oAl = oAh + kSq;
  static constexpr int oBeta = oAl + kSq;
  static constexpr int oLam = oBeta + kC * 4;       // fp32 [4][DK]
  static constexpr int oVec = oLam + 4 * DK * 4;    // fp32 [7][DK]
  static constexpr int kVecG = 0, kVecC = 3, kVecF = 4;
  static constexpr int oW = oVec + 7 * DK * 4;
  static constexpr int oB = oW + 2 * DK * 16;
  static constexpr int kBytes = oB + 2 * DK * 4;
};

template <int DK, typename Act, int DKR>
struct KdaChunk : PrefillCore<DK, Act> {
  GDN_PREFILL_CORE(DK, Act);
  // DKR: the layer's d_k.  Below DK (d_k = 16 in the d_k = 32 layout) the
  // upper half of every octet (channels 16 + 4j..) is padding: zero rows,
  // taps and bias, decay 1, so KE, QE and KF are zero there and the rows
  // DKR.. of S^T stay zero.
  static constexpr bool kPad = DKR < DK;
  using P = KdaPlan<DK>;
  static constexpr int kSl = DK / 32;
  static constexpr int kDt = DK / 16;
  static constexpr int kNco = DK / 4;
  static constexpr int kGrp = DK / 8;
  static constexpr bool kBf = sizeof(Act) == 2;

  int s;   // sequence index (workspace addressing)

  __device__ __forceinline__ static int qk(int r, int sl) { return QkRow<DK>::at(r, sl); }
  __device__ __forceinline__ static float bfx(short v) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(v)) << 16);
  }

  // ================= producers =================
  // Thread (co, tau): channel octet co of q|k (q first), tokens 8 tau..+7.
  // Octet oc of a head is the 8 channels of storage chunk oc of the K / Q
  // rows, 32 (oc / 4) + 4 (oc % 4) + {0..3, 16..19} (see slot()), so each
  // row of a thread is stored as one 16-byte chunk.
  __device__ __forceinline__ static int oct_base(int oc) { return 32 * (oc >> 2) + 4 * (oc & 3); }
  struct Prod {
    Row8<Act> raw[11];        // rows 8 tau - 3 .. 8 tau + 7 of a chunk
    Row8<Act> dec[8];         // decays of tokens 8 tau .. +7 at the 8 channels
    s8 eh[8], el[8];          // KE (k) or QE (q) rows, not yet stored
    s8 fh[4], fl[4];          // KF rows: tokens 0..3 of the octet (k thread), 4..7 (q thread)
    float lam[8];             // decay over the whole 16-token block
    uint32_t diag[8];         // this thread's 32 bytes of a diagonal-block record
    float beta;               // wave 3: b of token = lane
    int co, tau, ch, oc;
    bool isk, on;
  };

  __device__ void prod_init(Prod& p) const {
    p.on = tid < 8 * kNco;
    p.co = tid % kNco;
    p.tau = tid / kNco;
    p.isk = p.co >= kGrp;
    p.oc = p.isk ? p.co - kGrp : p.co;
    p.ch = (p.isk ? a.Hk * DKR : 0) + hk * DKR + oct_base(p.oc);
  }

  // Taps and bias of the key head's q and k channels, stored [m][octet] (m =
  // channel within the octet) so that the lanes of one wave, one octet each,
  // read 16 consecutive bytes apiece at every m.
  __device__ void load_taps() const {
    float* wt = fp(P::oW);
    float* bs = fp(P::oB);
    for (int i = tid; i < 2 * DK; i += kThreads) {
      const int ih = i < DK ? i : i - DK;
      const int ch = i < DK ? hk * DKR + i : a.Hk * DKR + hk * DKR + (i - DK);
      // channel r of a 32-block: octet 4 (block) + (r % 16) / 4, place
      // r % 4 (+ 4 in the block's upper half)
      const int r = i & 31, oc = 4 * (i >> 5) + ((r & 15) >> 2), m = (r & 3) + 4 * (r >> 4);
      const int at = m * kNco + oc;
      const bool on = !kPad || ih < DKR;
      *reinterpret_cast<f4*>(wt + 4 * at) =
          on ? f4{tap(ch, 0), tap(ch, 1), tap(ch, 2), tap(ch, 3)} : f4{0.f, 0.f, 0.f, 0.f};
      bs[at] = (on && a.bias) ? to_f32(static_cast<const Act*>(a.bias)[ch]) : 0.f;
    }
  }

  // Row8::load_split, except that with padding the octet's upper half is
  // not read but set to fill (0 for inputs, the bits of 1.0 for decays).
  __device__ __forceinline__ static void load_oct(Row8<Act>& r, rsrc_t rs, int off, uint32_t fill) {
    if constexpr (!kPad) {
      r.load_split(rs, off);
    } else {
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      typedef uint32_t u4 __attribute__((ext_vector_type(4)));
      constexpr int kH = Row8<Act>::kWords / 2;
      if constexpr (kH == 2) {
        const u2 u = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
        r.w[0] = u[0], r.w[1] = u[1];
      } else {
        const u4 u = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
        r.w[0] = u[0], r.w[1] = u[1], r.w[2] = u[2], r.w[3] = u[3];
      }
#pragma unroll
      for (int i = kH; i < 2 * kH; ++i) r.w[i] = fill;
    }
  }

  __device__ __forceinline__ void prod_load(Prod& p, int c0) const {
    const int tau = opaque(p.tau), ch = opaque(p.ch), oc = opaque(p.oc);
    if (p.on) {
      const rsrc_t rx = x_rows(c0);
#pragma unroll
      for (int r = 0; r < 11; ++r) load_oct(p.raw[r], rx, x_off(c0, c0 + 8 * tau - 3 + r, ch), 0u);
      const int n = T - c0 < kC ? T - c0 : kC;
      const int64_t rowe = static_cast<int64_t>(a.Hv) * DKR;
      const rsrc_t ra = make_rsrc(static_cast<const Act*>(a.alpha) + (t0 + static_cast<int64_t>(c0)) * rowe,
                                  static_cast<uint32_t>(n * rowe * sizeof(Act)));
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        load_oct(p.dec[tt], ra,
                 static_cast<int>((((8 * tau + tt) * a.Hv + h) * DKR + oct_base(oc)) * sizeof(Act)),
                 sizeof(Act) == 2 ? 0x3F803F80u : 0x3F800000u);
      if (c0 == 0) {
        const rsrc_t rw = win_rows();
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          Row8<Act> wr;
          load_oct(wr, rw, win_off(8 * tau - 3 + r, ch), 0u);
          p.raw[r].merge(wr);
        }
      }
    }
  }

  // The chunk's diagonal-block records (thread = block R, lane): loaded when
  // its preparation starts, stored with its planes.
  __device__ __forceinline__ void load_diag(Prod& p, int c0) const {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const int R = tid >> 6, l = tid & 63;
    const unsigned char* rec = static_cast<const unsigned char*>(a.ws) +
                               (ws_block(s, t0, c0 / kBlk + R) * a.Hv + h) * kWsBlockBytes + l * 32;
    const u4 w0 = *reinterpret_cast<const u4*>(rec);
    const u4 w1 = *reinterpret_cast<const u4*>(rec + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p.diag[i] = w0[i];
      p.diag[4 + i] = w1[i];
    }
  }

  // Decay of token 8 tau + tt at channel m of the thread's octet, unpacked
  // from an opaque copy of its word: the backward pass's 64 unpacked values
  // are then not held until the forward pass unpacks them again.
  __device__ __forceinline__ float dec(const Prod& p, int tt, int m) const {
    Row8<Act> r;
#pragma unroll
    for (int i = 0; i < Row8<Act>::kWords; ++i) r.w[i] = 0;
    r.w[m * Row8<Act>::kWords / 8] = static_cast<uint32_t>(opaque(static_cast<int>(p.dec[tt].w[m * Row8<Act>::kWords / 8])));
    return r.get(m);
  }

  // conv + SiLU + L2 norm (+ q scale), the decay products and the planes of
  // chunk c0, in one forward pass over the octet's tokens.  A backward pass
  // over the decays first gives the octet's total and the suffix products
  // F the thread needs (a k thread keeps tokens 0..3 of the KF rows, its q
  // partner kGrp lanes away -- same channels, same decays -- takes 4..7 and
  // receives those k rows by shuffle); the partner octet of the 16-token
  // block (kNco lanes away) supplies the missing factor of E and F.
  __device__ void prod_prep(Prod& p, int c0) const {
    const float* wl = fp(P::oW);
    const float* bl = fp(P::oB);
    load_diag(p, c0);
    if (p.on) {
      const int tbase = c0 + 8 * p.tau;
      if (tbase + 8 > T) {      // decays of tokens past the sequence read 1
        constexpr uint32_t kOne = sizeof(Act) == 2 ? 0x3F803F80u : 0x3F800000u;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
#pragma unroll
          for (int i = 0; i < Row8<Act>::kWords; ++i)
            p.dec[tt].w[i] = tbase + tt < T ? p.dec[tt].w[i] : kOne;
      }
      float fs[4][8], run[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) run[m] = 1.f;
#pragma unroll
      for (int tt = 7; tt >= 0; --tt) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          if (tt >= 4)
            fs[tt - 4][m] = run[m];
          else
            fs[tt][m] = p.isk ? run[m] : fs[tt][m];
          run[m] = run[m] * dec(p, tt, m);
        }
      }
      const bool odd = p.tau & 1;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const float pt = __shfl_xor(run[m], kNco);   // the partner octet's total
        p.lam[m] = pt * run[m];
#pragma unroll
        for (int j = 0; j < 4; ++j) fs[j][m] = odd ? fs[j][m] : fs[j][m] * pt;
        run[m] = odd ? pt : 1.f;                      // E starts at the partner's total
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const bool in = tbase + tt < T;
        float y[8], ss = 0.f;
        const int cw = opaque(p.co);   // taps re-read per token, not held
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const f4 wt = *reinterpret_cast<const f4*>(wl + 4 * (m * kNco + cw));
          float v = bl[m * kNco + cw];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v = fmaf(wt[jj], p.raw[tt + jj].get(m), v);
          v = act(v);
          y[m] = v;
          ss = fmaf(v, v, ss);
        }
        const float sum = group_sum<kGrp>(ss);
        float sc = a.l2norm ? rsqrtf(sum + a.eps) : 1.0f;
        if (!p.isk) sc *= a.q_scale;
        if (!in) sc = 0.f;
        f4 ve[2], vf[2];
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          const float yv = y[m] * sc;
          run[m] = run[m] * p.dec[tt].get(m);
          ve[m >> 2][m & 3] = yv * run[m];
          const float kv = tt < 4 ? yv : __shfl_xor(yv, kGrp);
          vf[m >> 2][m & 3] = kv * fs[tt & 3][m];
        }
        s4 h0, l0, h1, l1;
        split4(ve[0], h0, l0);
        split4(ve[1], h1, l1);
        p.eh[tt] = cat(h0, h1);
        p.el[tt] = cat(l0, l1);
        split4(vf[0], h0, l0);
        split4(vf[1], h1, l1);
        if (tt < 4 || !p.isk) {
          p.fh[tt & 3] = cat(h0, h1);
          p.fl[tt & 3] = cat(l0, l1);
        }
      }
    }
    if (wave == 3)
      p.beta = c0 + lane < T ? to_f32(static_cast<const Act*>(a.beta)[(static_cast<int64_t>(t0) + c0 + lane) * a.Hv + h])
                             : 0.f;
  }

  __device__ void prod_store(const Prod& p) const {
    if (p.on) {
      short* eh = sp(p.isk ? P::oEKh : P::oEQh);
      short* el = sp(p.isk ? P::oEKl : P::oEQl);
      const int tau = opaque(p.tau);
      const int sb = 8 * opaque(p.oc);   // the octet's storage chunk
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int o = qk(8 * tau + tt, sb);
        *reinterpret_cast<s8*>(eh + o) = p.eh[tt];
        *reinterpret_cast<s8*>(el + o) = p.el[tt];
      }
      {
        short* fh = sp(P::oFKh);
        short* fl = sp(P::oFKl);
        const int t4 = 8 * tau + (p.isk ? 0 : 4);
#pragma unroll
        for (int jx = 0; jx < 4; ++jx) {
          const int o = qk(t4 + jx, sb);
          *reinterpret_cast<s8*>(fh + o) = p.fh[jx];
          *reinterpret_cast<s8*>(fl + o) = p.fl[jx];
        }
      }
      if (p.isk) {
        if (tau & 1) {
          float* lam = fp(P::oLam) + (tau >> 1) * DK + oct_base(opaque(p.oc));
          *reinterpret_cast<f4*>(lam) = f4{p.lam[0], p.lam[1], p.lam[2], p.lam[3]};
          *reinterpret_cast<f4*>(lam + 16) = f4{p.lam[4], p.lam[5], p.lam[6], p.lam[7]};
        }
      }
    }
    {
      const int l = lane_now();
      const int R = wave, r = 16 * R + (l >> 2), q4 = l & 3;
      const int o = r * P::kRowT + slot(16 * R + 4 * q4);
      typedef uint32_t u2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u2*>(sp(P::oAh) + o) = u2{p.diag[0], p.diag[1]};
      *reinterpret_cast<u2*>(sp(P::oAl) + o) = u2{p.diag[2], p.diag[3]};
      *reinterpret_cast<u2*>(sp(P::oPh) + o) = u2{p.diag[4], p.diag[5]};
      *reinterpret_cast<u2*>(sp(P::oPl) + o) = u2{p.diag[6], p.diag[7]};
    }
    if (wave == 3) fp(P::oBeta)[lane] = p.beta;
  }

  // ================= all waves: the off-diagonal blocks of A and P =====
  __device__ __forceinline__ void op_bases(int (&ob)[kSl]) const {
    const int l = lane_now(), r = l & 15, g = l >> 4;
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) ob[sl] = qk(r, 32 * sl + 8 * g);
  }

  // Block pair (IB, JB), IB > JB + 0, computed transposed: A operand KF rows
  // JB (times D = prod_{JB < J < IB} Lam_J on its channels), B operands KE
  // and QE rows IB; lane holds row r = 16 IB + lr at columns 16 JB + 4 lg + v.
  template <int IB, int JB>
  __device__ __forceinline__ void pair(const int (&ob)[kSl]) const {
    const short* fh = sp(P::oFKh);
    const short* fl = sp(P::oFKl);
    const short* kh = sp(P::oEKh);
    const short* kl = sp(P::oEKl);
    const short* qh = sp(P::oEQh);
    const short* ql = sp(P::oEQl);
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    f4 g = {0.f, 0.f, 0.f, 0.f}, pq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      const int oa = 16 * JB * P::kRowQK + ob[sl], obr = 16 * IB * P::kRowQK + ob[sl];
      s8 ah = *reinterpret_cast<const s8*>(fh + oa);
      s8 al = *reinterpret_cast<const s8*>(fl + oa);
      if constexpr (IB - JB > 1) {
        // channels 32 sl + 4 lg + j (slots 0..3) and 32 sl + 16 + 4 lg + j (4..7)
        const float* lam = fp(P::oLam);
        f4 d0 = *reinterpret_cast<const f4*>(lam + (JB + 1) * DK + 32 * sl + 4 * lg);
        f4 d1 = *reinterpret_cast<const f4*>(lam + (JB + 1) * DK + 32 * sl + 16 + 4 * lg);
        if constexpr (IB - JB > 2) {
          d0 = d0 * *reinterpret_cast<const f4*>(lam + (JB + 2) * DK + 32 * sl + 4 * lg);
          d1 = d1 * *reinterpret_cast<const f4*>(lam + (JB + 2) * DK + 32 * sl + 16 + 4 * lg);
        }
        f4 x0, x1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          x0[j] = (bfx(ah[j]) + bfx(al[j])) * d0[j];
          x1[j] = (bfx(ah[4 + j]) + bfx(al[4 + j])) * d1[j];
        }
        s4 h0, l0, h1, l1;
        split4(x0, h0, l0);
        split4(x1, h1, l1);
        ah = cat(h0, h1);
        al = cat(l0, l1);
      }
      const s8 bkh = *reinterpret_cast<const s8*>(kh + obr);
      const s8 bkl = *reinterpret_cast<const s8*>(kl + obr);
      const s8 bqh = *reinterpret_cast<const s8*>(qh + obr);
      const s8 bql = *reinterpret_cast<const s8*>(ql + obr);
      g = mma32(al, bkh, g);
      pq = mma32(al, bqh, pq);
      g = mma32(ah, bkl, g);
      pq = mma32(ah, bql, pq);
      g = mma32(ah, bkh, g);
      pq = mma32(ah, bqh, pq);
    }
    const int r = 16 * IB + lr;
    const int o = r * P::kRowT + slot(16 * JB + 4 * lg);
    s4 h, lo;
    split4(pq, h, lo);
    *reinterpret_cast<s4*>(sp(P::oPh) + o) = h;
    *reinterpret_cast<s4*>(sp(P::oPl) + o) = lo;
    split4(fp(P::oBeta)[r] * g, h, lo);
    *reinterpret_cast<s4*>(sp(P::oAh) + o) = h;
    *reinterpret_cast<s4*>(sp(P::oAl) + o) = lo;
  }

  // Per-channel chunk vectors from the block decays: e^{G_R} = prod_{J<R}
  // Lam_J (R = 1..3), e^{G_4}, and f_I = prod_{J>I} Lam_J (I = 0..2).
  __device__ void vectors() const {
    const int c = (wave - 6) * 64 + lane_now();
    if (c >= DK) return;
    const float* lam = fp(P::oLam);
    float* vec = fp(P::oVec);
    const float l0 = lam[c], l1 = lam[DK + c], l2 = lam[2 * DK + c], l3 = lam[3 * DK + c];
    const float g1 = l0, g2 = g1 * l1, g3 = g2 * l2;
    vec[(P::kVecG + 0) * DK + c] = g1;
    vec[(P::kVecG + 1) * DK + c] = g2;
    vec[(P::kVecG + 2) * DK + c] = g3;
    vec[P::kVecC * DK + c] = g3 * l3;
    const float f2 = l3, f1 = l2 * f2, f0 = l1 * f1;
    vec[(P::kVecF + 0) * DK + c] = f0;
    vec[(P::kVecF + 1) * DK + c] = f1;
    vec[(P::kVecF + 2) * DK + c] = f2;
  }

  __device__ void gram_phase() const {
    int ob[kSl];
    op_bases(ob);
    switch (wave) {
      case 0: pair<1, 0>(ob); break;
      case 1: pair<2, 1>(ob); break;
      case 2: pair<3, 2>(ob); break;
      case 3: pair<2, 0>(ob); break;
      case 4: pair<3, 1>(ob); break;
      case 5: pair<3, 0>(ob); break;
      default: vectors(); break;
    }
  }

  // ================= consumers =================
  // The value conv of the wave's 16 columns: lane (lr, lg) needs tokens
  // 16 b + 4 lg + v (v < 4), i.e. raw rows 16 b + 4 lg - 3 .. + 3.
  struct Cons {
    uint32_t vx[4][7];
    float vw[4], vb;
    int vch;
    bool von;
  };

  __device__ void cons_init(Cons& c) const {
    c.vch = 2 * a.Hk * DKR + h * a.dv + e0 + lr;
    c.von = e0 + lr < a.dv;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) c.vw[jj] = c.von ? tap(c.vch, jj) : 0.f;
    c.vb = (c.von && a.bias) ? to_f32(static_cast<const Act*>(a.bias)[c.vch]) : 0.f;
  }

  __device__ __forceinline__ void cons_load(Cons& c, int c0) const {
    const rsrc_t rx = x_rows(c0);
    const int l = lane_now(), lgg = l >> 4, vch = opaque(c.vch);
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 7; ++i) {
        const int off = x_off(c0, c0 + 16 * b + 4 * lgg - 3 + i, vch);
        if constexpr (kBf)
          c.vx[b][i] = __builtin_amdgcn_raw_buffer_load_b16(rx, off, 0, 0);
        else
          c.vx[b][i] = __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0);
      }
    if (c0 == 0) {
      const rsrc_t rw = win_rows();
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        const int off = win_off(4 * lgg - 3 + i, vch);
        if constexpr (kBf)
          c.vx[0][i] |= __builtin_amdgcn_raw_buffer_load_b16(rw, off, 0, 0);
        else
          c.vx[0][i] |= __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0);
      }
    }
  }

  __device__ __forceinline__ float vraw(uint32_t u) const {
    return kBf ? __uint_as_float(u << 16) : __uint_as_float(u);
  }

  // The wave's 16 value columns for chunk c0.  S[d] holds rows
  // 16d + 4 lg + v (key index) of S^T at column e0 + lr (value index).
  __device__ void columns(int c0, f4 (&S)[kDt], Cons& cv, bool next) const {
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    // value conv of this chunk, then the next chunk's raw rows
    f4 V[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = cv.vb;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) y = fmaf(cv.vw[jj], vraw(cv.vx[b][v + jj]), y);
        V[b][v] = c0 + 16 * b + 4 * lg + v < T ? act(y) : 0.f;
      }
    if (next) cons_load(cv, c0 + kC);
    const float* vec = fp(P::oVec);
    const short* kh = sp(P::oEKh);
    const short* kl = sp(P::oEKl);
    const short* qh = sp(P::oEQh);
    const short* ql = sp(P::oEQl);
    // K E_b diag(e^{G_b}) S0^T and the same for Q, rows 16 tb + 4 lg + v
    f4 ks[4], qs[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      ks[tb] = f4{0.f, 0.f, 0.f, 0.f};
      qs[tb] = f4{0.f, 0.f, 0.f, 0.f};
    }
    int ob[kSl];
    op_bases(ob);
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      s8 xh[4], xl[4], yh[4], yl[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int ra = 16 * tb * P::kRowQK + ob[sl];
        xh[tb] = *reinterpret_cast<const s8*>(kh + ra);
        xl[tb] = *reinterpret_cast<const s8*>(kl + ra);
        yh[tb] = *reinterpret_cast<const s8*>(qh + ra);
        yl[tb] = *reinterpret_cast<const s8*>(ql + ra);
      }
      s8 sbh[4], sbl[4];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        f4 s0 = S[2 * sl], s1 = S[2 * sl + 1];
        if (tb > 0) {
          const float* gv = vec + (P::kVecG + tb - 1) * DK + 32 * sl + 4 * lg;
          s0 = s0 * *reinterpret_cast<const f4*>(gv);
          s1 = s1 * *reinterpret_cast<const f4*>(gv + 16);
        }
        s4 h0, l0, h1, l1;
        split4(s0, h0, l0);
        split4(s1, h1, l1);
        sbh[tb] = cat(h0, h1);
        sbl[tb] = cat(l0, l1);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        ks[tb] = mma32(xl[tb], sbh[tb], ks[tb]);
        qs[tb] = mma32(yl[tb], sbh[tb], qs[tb]);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        ks[tb] = mma32(xh[tb], sbl[tb], ks[tb]);
        qs[tb] = mma32(yh[tb], sbl[tb], qs[tb]);
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        ks[tb] = mma32(xh[tb], sbh[tb], ks[tb]);
        qs[tb] = mma32(yh[tb], sbh[tb], qs[tb]);
      }
    }
    // U_b = X_bb (b_b R_b - sum_{j<b} A_bj U_j),  R = V - (K o e^g) S0^T
    const float* bt = fp(P::oBeta);
    f4 U[4];
    s4 uh[4], ul[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = (16 * b + lr) * P::kRowT;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      if (b > 0) {
        s4 ah[3], al[3];
#pragma unroll
        for (int jb = 0; jb < b; ++jb) {
          const int o = row + slot(16 * jb + 4 * lg);
          ah[jb] = *reinterpret_cast<const s4*>(sp(P::oAh) + o);
          al[jb] = *reinterpret_cast<const s4*>(sp(P::oAl) + o);
        }
#pragma unroll
        for (int jb = 0; jb < b; ++jb) acc = mma16(al[jb], uh[jb], acc);
#pragma unroll
        for (int jb = 0; jb < b; ++jb) acc = mma16(ah[jb], ul[jb], acc);
#pragma unroll
        for (int jb = 0; jb < b; ++jb) acc = mma16(ah[jb], uh[jb], acc);
      }
      const int o = row + slot(16 * b + 4 * lg);
      const s4 xh = *reinterpret_cast<const s4*>(sp(P::oAh) + o);
      const s4 xl = *reinterpret_cast<const s4*>(sp(P::oAl) + o);
      const f4 bb = *reinterpret_cast<const f4*>(bt + 16 * b + 4 * lg);
      s4 zh, zl;
      split4(bb * (V[b] - ks[b]) - acc, zh, zl);
      U[b] = mma16x3(xh, xl, zh, zl, f4{0.f, 0.f, 0.f, 0.f});
      split4(U[b], uh[b], ul[b]);
    }
    // O = (Q o e^g) S0^T + P U
    {
      constexpr int kB[6] = {0, 1, 2, 2, 3, 3}, kU[6] = {0, 0, 0, 1, 0, 1};
      s8 ph[6], pl[6];
#pragma unroll
      for (int i = 0; i < 6; ++i) {
        const int off = (16 * kB[i] + lr) * P::kRowT + 32 * kU[i] + 8 * lg;
        ph[i] = *reinterpret_cast<const s8*>(sp(P::oPh) + off);
        pl[i] = *reinterpret_cast<const s8*>(sp(P::oPl) + off);
      }
      f4 o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) o[b] = qs[b];
      const s8 u0h = cat(uh[0], uh[1]), u0l = cat(ul[0], ul[1]);
      const s8 u1h = cat(uh[2], uh[3]), u1l = cat(ul[2], ul[3]);
#pragma unroll
      for (int i = 0; i < 6; ++i) o[kB[i]] = mma32(pl[i], kU[i] ? u1h : u0h, o[kB[i]]);
#pragma unroll
      for (int i = 0; i < 6; ++i) o[kB[i]] = mma32(ph[i], kU[i] ? u1l : u0l, o[kB[i]]);
#pragma unroll
      for (int i = 0; i < 6; ++i) o[kB[i]] = mma32(ph[i], kU[i] ? u1h : u0h, o[kB[i]]);
      const int rs = a.Hv * a.dv;
      const int n = T - c0 < kC ? T - c0 : kC;
      const rsrc_t ro =
          make_rsrc(a.out + ((static_cast<int64_t>(t0) + c0) * a.Hv + h) * a.dv + e0,
                    static_cast<uint32_t>(n) * static_cast<uint32_t>(rs) * 4u);
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[b][v]), ro,
                                                ((16 * b + 4 * lg + v) * rs + lr) * 4, 0, 0);
    }
    // S^T <- diag(e^{G_4}) S^T + sum_I diag(f_I) KF_I^T U_I: per key tile d,
    // one 16-token product per block I from transposing reads of the KF rows.
    int tb0[kSl];
    {
      const int r = l & 15, g = l >> 4;
#pragma unroll
      for (int D = 0; D < kSl; ++D) tb0[D] = qk(4 * g + (r >> 2), 32 * D + 8 * (r & 3));
    }
    const short* fh = sp(P::oFKh);
    const short* fl = sp(P::oFKl);
#pragma unroll
    for (int d = 0; d < kDt; ++d) {
      s4 th[4], tl[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        const int r0 = tb0[d >> 1] + (16 * I) * P::kRowQK + 4 * (d & 1);
        th[I] = ld_tr(fh + r0);
        tl[I] = ld_tr(fl + r0);
      }
      f4 acc[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) acc[I] = mma16(tl[I], uh[I], f4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int I = 0; I < 4; ++I) acc[I] = mma16(th[I], ul[I], acc[I]);
#pragma unroll
      for (int I = 0; I < 4; ++I) acc[I] = mma16(th[I], uh[I], acc[I]);
      const int key = 16 * d + 4 * lg;
      f4 s = *reinterpret_cast<const f4*>(vec + P::kVecC * DK + key) * S[d] + acc[3];
#pragma unroll
      for (int I = 0; I < 3; ++I)
        s = s + *reinterpret_cast<const f4*>(vec + (P::kVecF + I) * DK + key) * acc[I];
      S[d] = s;
    }
  }
};

template <int DK, typename Act, int DKR>
__global__ void __launch_bounds__(kThreads, 1) kda_chunk_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  using K = KdaChunk<DK, Act, DKR>;
  using P = KdaPlan<DK>;
  K k{{a, lds_raw}};
  k.tid = threadIdx.x;
  k.wave = __builtin_amdgcn_readfirstlane(k.tid >> 6);
  k.lane = k.tid & 63;
  k.lr = k.lane & 15;
  k.lg = k.lane >> 4;

  // Units (sequence, value head, column block), value heads of one key head
  // consecutive, dealt so that consecutive units share an XCD.
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int u = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int j = u % a.nblk;
  k.h = (u / a.nblk) % a.Hv;
  const int s = u / a.nblk / a.Hv;
  k.s = s;
  k.hk = k.h / a.G;

  const int t0 = a.cu[s], t1 = a.cu[s + 1];
  const int32_t dst = a.dst[s];
  k.init = a.init ? a.init[s] : dst;
  if (t0 < 0 || t1 < t0 || t1 > a.total || dst < 0 || dst >= a.num_slots ||
      k.init >= a.num_slots)
    return;
  k.t0 = t0;
  k.T = t1 - t0;
  const int nch = (k.T + kC - 1) / kC;

  // P and A planes: the blocks above the diagonal stay zero.
  for (int i = k.tid; i < 4 * P::kSq / 16; i += kThreads)
    reinterpret_cast<uint4*>(lds_raw + P::oPh)[i] = uint4{0u, 0u, 0u, 0u};
  k.e0 = j * kCols;
  k.load_taps();

  if (k.tid < kProd) {
    typename K::Prod p;
    k.prod_init(p);
    if (nch > 0) k.prod_load(p, 0);
    lds_barrier();            // planes zeroed, taps loaded
    // A chunk's raw rows and decays are fetched when its preparation starts:
    // the preparation runs beside the consumers' pass over the chunk before,
    // which is longer by more than the fetch takes, and fetched any earlier
    // (while the stored rows or the off-diagonal operands hold registers)
    // they were spilled, each spill waiting for the whole fetch inside the
    // serial store and off-diagonal phases.
    if (nch > 0) {
      k.prod_prep(p, 0);
      k.prod_store(p);
      lds_barrier();
      k.gram_phase();
      lds_barrier();
    }
    for (int c = 0; c < nch; ++c) {
      const bool next = c + 1 < nch;
      if (next) {
        k.prod_load(p, (c + 1) * kC);
        k.prod_prep(p, (c + 1) * kC);
      }
      lds_barrier();          // consumers are done with chunk c
      if (next) {
        k.prod_store(p);
        lds_barrier();
        k.gram_phase();
        lds_barrier();
      }
    }
  } else {
    k.e0 = j * kCols + (k.wave - 4) * 16;
    const bool cols = k.e0 < a.dv;
    typename K::Cons cv;
    k.cons_init(cv);
    if (cols && nch > 0) k.cons_load(cv, 0);
    f4 S[K::kDt];
    // rows of S^T in the slots: d_k = DKR floats per value index
    const int64_t head = static_cast<int64_t>(k.h) * a.dv * DKR;
    const int64_t slot_elems = static_cast<int64_t>(a.Hv) * a.dv * DKR;
    constexpr int kDtR = DKR / 16;   // 16-row tiles that exist in the slots
#pragma unroll
    for (int d = 0; d < K::kDt; ++d) {
      S[d] = f4{0.f, 0.f, 0.f, 0.f};
      if (d < kDtR && cols && k.init >= 0)
        S[d] = *reinterpret_cast<const f4*>(a.ssm + k.init * slot_elems + head +
                                           static_cast<int64_t>(k.e0 + k.lr) * DKR + 16 * d +
                                           4 * k.lg);
    }
    lds_barrier();            // planes zeroed, taps loaded
    if (nch > 0) {
      lds_barrier();          // producers stored chunk 0
      k.gram_phase();
      lds_barrier();
    }
    for (int c = 0; c < nch; ++c) {
      const bool next = c + 1 < nch;
      if (cols) k.columns(c * kC, S, cv, next);
      const int32_t cs = __builtin_amdgcn_readfirstlane(ckpt_slot(a, s, (c + 1) * kC, k.T));
      if (cols && cs >= 0) {  // the state after (c + 1) * 64 tokens, to a checkpoint slot
        const int l = k.lane_now();
        float* o = a.ssm + cs * slot_elems + head + static_cast<int64_t>(k.e0 + (l & 15)) * DKR;
#pragma unroll
        for (int d = 0; d < kDtR; ++d) *reinterpret_cast<f4*>(o + 16 * d + 4 * (l >> 4)) = S[d];
      }
      lds_barrier();          // chunk c consumed
      if (next) {
        lds_barrier();        // producers stored chunk c + 1
        k.gram_phase();
        lds_barrier();
      }
    }
    if (cols) {
      float* out = a.ssm + dst * slot_elems + head + static_cast<int64_t>(k.e0 + k.lr) * DKR;
#pragma unroll
      for (int d = 0; d < kDtR; ++d) *reinterpret_cast<f4*>(out + 16 * d + 4 * k.lg) = S[d];
    }
  }
}

template <int DK, typename Act, int DKR = DK>
hipError_t launch_kda(const PrefillArgs& a, int max_seqlen, hipStream_t st) {
  // diagonal blocks: grid y strides over the token blocks of a sequence,
  // kDiagPer of them per workgroup while that leaves kDiagMinGroups
  // workgroups, fewer (down to one) when it would not
  const int64_t want = 4 * ((static_cast<int64_t>(max_seqlen) + kC - 1) / kC);
  const int64_t heads = static_cast<int64_t>(a.N) * a.Hv;
  int64_t g = (want + kDiagPer - 1) / kDiagPer;
  const int64_t enough = (kDiagMinGroups + heads - 1) / heads;
  if (g < enough) g = enough < want ? enough : want;
  const int gy = static_cast<int>(g < 1 ? 1 : (g > 65535 ? 65535 : g));
  hipLaunchKernelGGL((kda_diag_kernel<DK, Act, DKR>), dim3(a.N * a.Hv, gy), dim3(kDiagThreads), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int bytes = KdaPlan<DK>::kBytes;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&kda_chunk_kernel<DK, Act, DKR>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((kda_chunk_kernel<DK, Act, DKR>), dim3(a.N * a.Hv * a.nblk), dim3(kThreads),
                     bytes, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.W < 2) return e;
  hipLaunchKernelGGL((prefill_conv_tail<Act>), conv_tail_grid(a), dim3(256), 0, st, a);
  return hipGetLastError();
}

static_assert(KdaPlan<128>::kBytes <= 160 * 1024, "LDS plan exceeds 160 KiB");

}  // namespace

size_t kda_workspace_bytes(int Hv, int64_t N, int64_t total) {
  const int64_t blocks = total / kBlk + 4 * (N < total ? N : total);
  return static_cast<size_t>(blocks) * static_cast<size_t>(Hv) * kWsBlockBytes;
}

hipError_t launch_prefill_kda(const PrefillArgs& a, int dk, int act_bf16, int max_seqlen,
                              hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  switch (dk) {
    case 16: return act_bf16 ? launch_kda<32, bf16, 16>(a, max_seqlen, s) : launch_kda<32, float, 16>(a, max_seqlen, s);
    case 32: return act_bf16 ? launch_kda<32, bf16>(a, max_seqlen, s) : launch_kda<32, float>(a, max_seqlen, s);
    case 64: return act_bf16 ? launch_kda<64, bf16>(a, max_seqlen, s) : launch_kda<64, float>(a, max_seqlen, s);
    case 128: return act_bf16 ? launch_kda<128, bf16>(a, max_seqlen, s) : launch_kda<128, float>(a, max_seqlen, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
