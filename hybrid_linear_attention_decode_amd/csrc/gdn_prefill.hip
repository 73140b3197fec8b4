// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The recurrence S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = S_t q_t is evaluated 32 tokens at a time in its WY / UT-transform
// form (Yang et al., "Parallelizing Linear Transformers with the Delta Rule
// over Sequence Length", 2024, sec. 3; with the scalar decay of "Gated Delta
// Networks", 2025, sec. 3).  For a chunk with rows K, Q (normalised keys and
// queries), V, log-decay prefix sums g and state S0 before the chunk:
//   A_ri = b_r e^{g_r - g_i} k_r . k_i            (i < r)
//   (I + A) U = diag(b) (V - diag(e^g) K S0^T)    (U: the chunk's updates)
//   O = diag(e^g) Q S0^T + P U,  P_ri = e^{g_r - g_i} q_r . k_i   (i <= r)
//   S = e^{g_c} S0 + U^T diag(e^{g_c - g}) K       (g_c: the chunk's last g)
// The triangular system is solved blockwise: the two 16x16 diagonal blocks
// of (I + A) are inverted in fp32, and U is formed block row by block row,
// U_b = X_bb (b_b R_b - sum_{j<b} A_bj U_j).
//
// Two kernels.  The first prepares q and k once per key head: conv1d +
// SiLU + L2 norm (+ q scale), split into bf16 (hi, lo) rows in a workspace.
// In the second, rows of S are independent through the whole recurrence
// (row i of S, U and O depend only on row i of S0), so a workgroup owns one
// (sequence, value head, 64 value columns) and walks that sequence's chunks
// in order, its 64 x d_k slice of S^T held in MFMA accumulators across
// chunks.  Its 8 waves form a pipeline over LDS buffers that rotate by chunk
// (K, Q, V^T and gates: three; P and A: two), with one barrier per chunk.
// Between barriers c - 1 and c:
//   consumers (waves 4-7), 16 value columns each, run chunk c: K S0^T,
//     Q S0^T, U, O and the state update;
//   producers (waves 0-3) copy chunk c + 2's prepared K, Q rows into LDS with
//     its value conv (wave 1 also its gates, the log-decay prefix sums, from
//     inputs loaded a chunk ahead), and form chunk c + 1's A and P from the
//     lower 16x16 tiles of K K^T and Q K^T, with the inverses of the diagonal
//     blocks of (I + A): for N strictly lower triangular, (I + N)^{-1} =
//     (I - N)(I + N^2)(I + N^4)(I + N^8), and K K^T is symmetric, so both
//     operand layouts of N come from the one accumulator tile.
// Each kernel also writes the destination's and the checkpoints' conv
// windows of the channels it reads (q, k in the first, the value columns in
// the second): a destination window by the threads that alone read the
// initial window, after those reads (see load_window_out, vwin_load).
// Every product runs on v_mfma_f32_16x16x{32,16}_bf16 with each fp32
// operand split as x ~= hi + lo (two bf16), and a*b ~= ah*bh + ah*bl + al*bh
// accumulated in fp32: about 16 significant bits per operand, which keeps
// the chunked result within a few 1e-5 of the fp64 recurrence, where plain
// bf16 operands would not meet a 2e-3 bound.
//
// Contraction index order.  An MFMA sums over its k index in any order, so
// operands that feed the k side are stored with a fixed permutation of each
// block of 32 indices ("slot", below) chosen so that two accumulator tiles
// of a previous product (rows 4*(lane/16)+0..3 of each) are directly the
// k-operand of a 16x16x32 MFMA.  K, Q and P (and K^T) in LDS use the same
// permutation, so every 16-byte LDS read lines up with register tiles.
#include "prefill_common.hpp"

namespace gdn {
namespace {

constexpr int kT = 32;         // chunk length (tokens)
constexpr int kNb = kT / 16;   // 16-token blocks per chunk
constexpr int kTpt = kT / 8;   // tokens per producer thread
// The producer wave that writes the gates: one of the two that form the
// block inverses (the other two run the value conv).
constexpr int kGateWave = 1;

// LDS plan (bytes).  Chunk c's planes sit in buffer c % 3 (K, Q, V^T and
// gates) or c % 2 (P and A): while the consumers read chunk c, the producers
// form chunk c + 1's P and A from its K, Q and gates (stored an iteration
// earlier) and store chunk c + 2's K, Q and V^T.  P, A and V^T rows are
// padded by 16 bytes so that 16 lanes reading 16 consecutive rows hit
// distinct banks; K and Q rows follow QkRow; K and Q planes are staggered by
// 64 bytes.
template <int DK>
struct Plan {
  static constexpr int kRowQK = QkRow<DK>::kElems;  // bf16 per row of K, Q   [token][dk]
  static constexpr int kRowT = kT + 8;   // bf16 per row of P, A   [token][token]
  static constexpr int kRowV = kT + 4;   // fp32 per row of V^T    [value column][token]
  static constexpr int kQK = 2 * kT * kRowQK + 64;   // one K or Q plane
  static constexpr int kSq = 2 * kT * kRowT;         // one P or A plane
  static constexpr int kVt = kCols * kRowV * 4;      // V^T
  static constexpr int kGt = 4 * kT * 4;             // fp32 [4][kT]: g, b, e^g, e^{g_c - g}
  static constexpr int oKQ = 0;                      // [3][Kh, Kl, Qh, Ql]
  static constexpr int oPA = oKQ + 3 * 4 * kQK;      // [2][Ph, Pl, Ah, Al]
  static constexpr int oV = oPA + 2 * 4 * kSq;       // [3]
  static constexpr int oG = oV + 3 * kVt;            // [3]
  // conv taps (4, left-padded) and bias of the workgroup's 64 value columns
  static constexpr int kWch = kCols;
  static constexpr int oW = oG + 3 * kGt;
  static constexpr int oB = oW + kWch * 16;
  static constexpr int kBytes = oB + kWch * 4;
  enum { Kh = 0, Kl = 1, Qh = 2, Ql = 3 };   // planes of a K / Q buffer
  enum { Ph = 0, Pl = 1, Ah = 2, Al = 3 };   // planes of a P / A buffer
  __device__ static int kq(int c, int plane) { return oKQ + ((c % 3) * 4 + plane) * kQK; }
  __device__ static int pa(int c, int plane) { return oPA + ((c & 1) * 4 + plane) * kSq; }
  __device__ static int v(int c) { return oV + (c % 3) * kVt; }
  __device__ static int gate(int c) { return oG + (c % 3) * kGt; }
};

// Prepared q / k rows in the workspace: [token][H_k][q | k][hi | lo][DK]
// bf16, each row in storage-slot order (the order of K and Q rows in LDS
// before the swizzle).  A descriptor covers the rows of one chunk of a
// sequence (rows past the sequence read zero); offsets are in bytes.
template <int DK>
__device__ __forceinline__ rsrc_t qk_rows(const PrefillArgs& a, int t0, int T, int c0, int n) {
  const int64_t row = static_cast<int64_t>(a.Hk) * 4 * DK;   // bf16 per token
  const int rows = T - c0 < n ? (T > c0 ? T - c0 : 0) : n;
  return make_rsrc(static_cast<const short*>(a.ws) + (static_cast<int64_t>(t0) + c0) * row,
                   static_cast<uint32_t>(rows * row * 2));
}
template <int DK>
__device__ __forceinline__ int qk_off(const PrefillArgs& a, int r, int hk, bool isk, int lo,
                                      int sl) {
  return (((r * a.Hk + hk) * 4 + (isk ? 2 : 0) + lo) * DK + sl) * 2;
}

// The q / k preparation pass (its own kernel, before the main one): one
// workgroup per (sequence, key head, every n-th 32-token chunk), thread
// (co, tau): channel group co of q | k (q first), tokens 4 tau..+3 -- conv1d
// + SiLU + L2 norm (+ q scale), split into bf16 (hi, lo).  Once per key
// head, where the main kernel's workgroups that share the key head would
// each repeat it.  Group oc of a head holds channels 4j..4j+3 and
// 4j+16..4j+19 of 32-block b (oc = 4b + j): exactly the channels of storage
// slots 8 oc..8 oc+7, so each row half goes out as one 16-byte store.
template <int DK, typename Act, int DKR>
struct QkPrep : PrefillCore<DK, Act> {
  GDN_PREFILL_CORE(DK, Act);
  // DKR: the layer's d_k.  Below DK (d_k = 16 runs the d_k = 32 layout) the
  // channels from DKR on are padding: read as zero with zero taps and bias,
  // so their prepared rows are zero and add nothing to any product.
  static constexpr bool kPad = DKR < DK;
  int s;          // sequence (checkpoint table row)
  int32_t dst;    // destination slot
  static constexpr int kNco = DK / 4;   // channel groups of q and k
  static constexpr int kGrp = DK / 8;   // groups per head (lanes of one norm)
  static constexpr int kRaw = kTpt + 3; // raw rows per thread
  static constexpr int kE = static_cast<int>(sizeof(Act));

  // Channel m (0..7) of group oc, relative to the head.
  __device__ __forceinline__ static int chan(int oc, int m) {
    return 32 * (oc >> 2) + 4 * (oc & 3) + (m < 4 ? m : 12 + m);
  }

  // The group's 8 channels of one raw row: the two 4-channel halves.
  __device__ __forceinline__ static void load_row(Row8<Act>& r, rsrc_t rs, int off) {
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    // the second half (16 channels on) lies in the padding when d_k = 16
    const uint32_t off1 = kPad ? kOutOfRange : static_cast<uint32_t>(off + 16 * kE);
    if constexpr (kE == 2) {
      const u2 a0 = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
      const u2 a1 = __builtin_amdgcn_raw_buffer_load_b64(rs, off1, 0, 0);
      r.w[0] = a0[0], r.w[1] = a0[1], r.w[2] = a1[0], r.w[3] = a1[1];
    } else {
      const u4 a0 = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
      const u4 a1 = __builtin_amdgcn_raw_buffer_load_b128(rs, off1, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) r.w[i] = a0[i], r.w[4 + i] = a1[i];
    }
  }

  // Raw rows 4 tau - 3 .. 4 tau + 3 of chunk c0 for the group starting at
  // channel c (its first half; the second is 16 channels on).
  __device__ __forceinline__ void load(Row8<Act> (&raw)[kRaw], int c0, int tau, int c) const {
    const rsrc_t rx = x_rows(c0);
#pragma unroll
    for (int r = 0; r < kRaw; ++r) load_row(raw[r], rx, x_off(c0, c0 + kTpt * tau - 3 + r, c));
    if (c0 == 0) {
      // rows -3..-1 (thread tokens 0..2 of token group 0) from the window;
      // every other offset lies past the window and reads zero
      const rsrc_t rw = win_rows();
#pragma unroll
      for (int r = 0; r < 3; ++r) {
        Row8<Act> wr;
        load_row(wr, rw, win_off(kTpt * tau - 3 + r, c));
        raw[r].merge(wr);
      }
    }
  }

  // The group's 8 channels of raw row r to a conv-state row (channel c's
  // element at p): the two 4-channel halves, the second not in the padding.
  __device__ __forceinline__ static void put_row(Act* p, const Row8<Act>& r) {
    if constexpr (kE == 2) {
      *reinterpret_cast<uint2*>(p) = uint2{r.w[0], r.w[1]};
      if constexpr (!kPad) *reinterpret_cast<uint2*>(p + 16) = uint2{r.w[2], r.w[3]};
    } else {
      *reinterpret_cast<uint4*>(p) = uint4{r.w[0], r.w[1], r.w[2], r.w[3]};
      if constexpr (!kPad) *reinterpret_cast<uint4*>(p + 16) = uint4{r.w[4], r.w[5], r.w[6], r.w[7]};
    }
  }
  // Row jj of the destination window of the group (first channel c): input
  // T - (W-1) + jj of the sequence, or of the initial window before it.
  __device__ __forceinline__ void load_window_out(Row8<Act> (&nw)[3], int c) const {
    const int W1 = a.W - 1;
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      if (jj < W1) {
        const int rho = T - W1 + jj;   // uniform
        if (rho >= 0)
          load_row(nw[jj], seq_row(rho), c * kE);
        else
          load_row(nw[jj], win_rows(), win_off(rho, c));
      }
    }
  }
  __device__ __forceinline__ Act* conv_row(int32_t slot, int jj, int c) const {
    return static_cast<Act*>(a.conv) + (static_cast<int64_t>(slot) * (a.W - 1) + jj) * a.C + c;
  }

  // Taps (4, left-padded) and bias of the group's channels (first at c): for
  // a width-4 conv with aligned arrays one 4-tap load per channel and one
  // load per 4 biases, else element by element.
  __device__ __forceinline__ void taps8(int c, f4 (&wt)[8], float (&bias)[8]) const {
    const Act* w = static_cast<const Act*>(a.w);
    const Act* b = static_cast<const Act*>(a.bias);
    const uintptr_t wa = reinterpret_cast<uintptr_t>(w), ba = reinterpret_cast<uintptr_t>(b);
    if (a.W == 4 && wa % (4 * kE) == 0) {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const Act* t = w + static_cast<int64_t>(c + (m < 4 ? m : 12 + m)) * 4;
        if constexpr (kE == 2) {
          const uint2 u = *reinterpret_cast<const uint2*>(t);
          wt[m] = f4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
        } else {
          wt[m] = *reinterpret_cast<const f4*>(t);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int cm = c + (m < 4 ? m : 12 + m);
        wt[m] = f4{tap(cm, 0), tap(cm, 1), tap(cm, 2), tap(cm, 3)};
      }
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) bias[m] = 0.f;
    if (b) {
      if (kE == 2 && ba % 8 == 0) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint2 u = *reinterpret_cast<const uint2*>(b + c + 16 * hf);
          bias[4 * hf + 0] = __uint_as_float(u.x << 16);
          bias[4 * hf + 1] = __uint_as_float(u.x & 0xffff0000u);
          bias[4 * hf + 2] = __uint_as_float(u.y << 16);
          bias[4 * hf + 3] = __uint_as_float(u.y & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 8; ++m) bias[m] = to_f32(b[c + (m < 4 ? m : 12 + m)]);
      }
    }
    if constexpr (kPad) {
      // the second half's taps and bias were read from the channels that
      // follow (in bounds); the padding has none
#pragma unroll
      for (int m = 4; m < 8; ++m) {
        wt[m] = f4{0.f, 0.f, 0.f, 0.f};
        bias[m] = 0.f;
      }
    }
  }

  // Chunks first, first + step, ... of the sequence, the next one's rows
  // loaded while the current one is computed.
  __device__ void run(int first, int step) const {
    if (tid >= 8 * kNco) return;        // whole 16-lane groups drop out together
    const int co = tid % kNco, tau = tid / kNco;
    const bool isk = co >= kGrp;
    const int oc = isk ? co - kGrp : co;
    const int c = (isk ? a.Hk * DKR : 0) + hk * DKR + chan(oc, 0);
    // The destination window of the group's channels is written by the
    // threads that alone read the initial window (token group 0 of the
    // workgroup that takes chunk 0), once their reads of it are done.
    const int W1 = a.W - 1;
    const bool win = W1 > 0 && first == 0 && tau == 0;
    Row8<Act> nw[3];
    if (win) load_window_out(nw, c);
    if (first * kT >= T) {   // an empty sequence: its window only
      if (win)
#pragma unroll
        for (int jj = 0; jj < 3; ++jj)
          if (jj < W1) put_row(conv_row(dst, jj, c), nw[jj]);
      return;
    }
    f4 wt[8];
    float bias[8];
    taps8(c, wt, bias);
    short* ws = static_cast<short*>(a.ws);
    Row8<Act> raw[kRaw], nxt[kRaw];
    load(raw, first * kT, tau, c);
    for (int cc = first; cc * kT < T; cc += step) {
      const int c0 = cc * kT;
      const bool more = (cc + step) * kT < T;
      if (more) load(nxt, (cc + step) * kT, tau, c);
#pragma unroll
      for (int tt = 0; tt < kTpt; ++tt) {
        float y[8], ss = 0.f;
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          float v = bias[m];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) v = fmaf(wt[m][jj], raw[tt + jj].get(m), v);
          v = act(v);
          y[m] = v;
          ss = fmaf(v, v, ss);
        }
        const float sum = group_sum<kGrp>(ss);
        float sc = a.l2norm ? rsqrtf(sum + a.eps) : 1.0f;
        if (!isk) sc *= a.q_scale;
        const int tok = c0 + kTpt * tau + tt;
        if (tok < T) {
          s4 h0, l0, h1, l1;
          split4(f4{y[0], y[1], y[2], y[3]} * sc, h0, l0);
          split4(f4{y[4], y[5], y[6], y[7]} * sc, h1, l1);
          short* hi = ws + ((static_cast<int64_t>(t0) + tok) * a.Hk + hk) * 4 * DK +
                      (isk ? 2 : 0) * DK + 8 * oc;
          *reinterpret_cast<s8*>(hi) = cat(h0, h1);
          *reinterpret_cast<s8*>(hi + DK) = cat(l0, l1);
        }
      }
      if (win && cc == 0) {     // the initial window's rows in raw have been used
#pragma unroll
        for (int jj = 0; jj < 3; ++jj)
          if (jj < W1) put_row(conv_row(dst, jj, c), nw[jj]);
      }
      // A checkpoint after this chunk: its window is the chunk's last W-1
      // rows, the last raw rows of the last token group.
      if (a.ckpt && W1 > 0 && tau == kT / kTpt - 1 && (c0 + kT) % a.ckpt_every == 0) {
        const int32_t cs = ckpt_slot(a, s, c0 + kT, T);
        if (cs >= 0) {
          if (W1 == 3) {
            put_row(conv_row(cs, 0, c), raw[kRaw - 3]);
            put_row(conv_row(cs, 1, c), raw[kRaw - 2]);
            put_row(conv_row(cs, 2, c), raw[kRaw - 1]);
          } else if (W1 == 2) {
            put_row(conv_row(cs, 0, c), raw[kRaw - 2]);
            put_row(conv_row(cs, 1, c), raw[kRaw - 1]);
          } else {
            put_row(conv_row(cs, 0, c), raw[kRaw - 1]);
          }
        }
      }
      if (more) {
#pragma unroll
        for (int r = 0; r < kRaw; ++r) raw[r] = nxt[r];
      }
    }
  }
};

template <int DK, typename Act, int DKR>
struct Prefill : PrefillCore<DK, Act> {
  GDN_PREFILL_CORE(DK, Act);
  // DKR: the layer's d_k (DK but for d_k = 16, run in the d_k = 32 layout;
  // the padded K, Q channels are zero, so rows DKR.. of S^T stay zero and
  // are neither read nor written).
  using P = Plan<DK>;
  int s;          // sequence (checkpoint table row)
  int32_t dst;    // destination slot
  static constexpr int kSl = DK / 32;   // 32-wide slices of d_k
  static constexpr int kDt = DK / 16;   // 16-row tiles of d_k
  static constexpr int kNco = DK / 4;   // channel octets of q and k
  static constexpr int kGrp = DK / 8;   // octets per head (lanes of one norm)
  static constexpr int kVt = 8;          // tokens per value-conv thread
  static constexpr int kVRaw = kVt + 3;  // raw rows per value-conv thread

  // Element offset of storage slot sl of row r in a K or Q plane.
  __device__ __forceinline__ static int qk(int r, int sl) { return QkRow<DK>::at(r, sl); }

  // ================= producers =================
  // The prepared K, Q rows of a chunk are copied as 16-byte pieces: piece x
  // = tid + 256 i of the chunk is token x / (4 kNc), workspace plane
  // (x / kNc) % 4 (q hi, q lo, k hi, k lo), chunk x % kNc -- a wave reads
  // whole workspace rows, and each 8 lanes of a store write 8 chunks of one
  // row, which the swizzle keeps in distinct banks.  A thread's pieces are
  // one plane and chunk at tokens t_0 + i kTs, so their addresses are a
  // per-thread base plus a uniform or immediate offset.
  static constexpr int kNc = QkRow<DK>::kChunks;   // 16-byte chunks per K / Q row
  static constexpr int kCopy = kNc / 2;            // pieces per producer thread and chunk
  static constexpr int kTs = 64 / kNc;             // token step between a thread's pieces
  struct Prod {
    u4 row[kCopy];              // the next chunk's prepared pieces, not yet stored
    int qoff;                   // workspace bytes of piece 0 from the chunk's first row
    int lds[2];                 // LDS bytes of piece 0 (pieces with bit 1 of i set: [1])
                                //   within a K / Q buffer
    // value conv (waves 2, 3, which carry no block inverse): channels 2 vp,
    // 2 vp + 1 of the column block, tokens 8 vt..+7
    uint32_t vraw[kVRaw][sizeof(Act) == 2 ? 1 : 2];
    f4 vo[2][2];                // [channel][token half], not yet stored
    uint32_t vwin[3][sizeof(Act) == 2 ? 1 : 2];   // destination window rows (vt == 0)
    int vp, vt, vch;
    bool von;
  };

  __device__ void prod_init(Prod& p) const {
    const int u = tid % (4 * kNc), t = tid / (4 * kNc), pp = u / kNc, cl = u % kNc;
    p.qoff = qk_off<DK>(a, t, hk, pp >> 1, pp & 1, 8 * cl);
    // the swizzle of token t + kTs i differs from token t's only by bit 1
    // (i >> 1 odd: rows 8..15 of the 16-row block; d_k = 128, t < 4)
    const int plane = (pp ^ 2) * P::kQK;   // q hi, q lo, k hi, k lo -> Qh, Ql, Kh, Kl
    p.lds[0] = plane + 2 * qk(t, 8 * cl);
    p.lds[1] = QkRow<DK>::kSwz ? plane + 2 * qk(t, 8 * (cl ^ 2)) : p.lds[0];
    const int vtid = tid >= kProd / 2 ? tid - kProd / 2 : 0;
    p.vp = vtid % 32;
    p.vt = vtid / 32;
    p.von = tid >= kProd / 2 && e0 + 2 * p.vp < a.dv;
    p.vch = 2 * a.Hk * DKR + h * a.dv + e0 + 2 * p.vp;
  }

  // Taps and bias of the workgroup's value columns into LDS (all threads).
  __device__ void load_taps() const {
    float* wt = fp(P::oW);
    float* bs = fp(P::oB);
    for (int i = tid; i < P::kWch; i += kThreads) {
      const int ch = 2 * a.Hk * DKR + h * a.dv + e0 + i;
      const bool ok = e0 + i < a.dv;
      f4 t = {0.f, 0.f, 0.f, 0.f};
      if (ok) t = f4{tap(ch, 0), tap(ch, 1), tap(ch, 2), tap(ch, 3)};
      *reinterpret_cast<f4*>(wt + 4 * i) = t;
      bs[i] = (ok && a.bias) ? to_f32(static_cast<const Act*>(a.bias)[ch]) : 0.f;
    }
  }

  __device__ __forceinline__ static s4 ld8(rsrc_t r, int off) {
    return __builtin_bit_cast(s4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  }

  // Window rows of the thread's two value channels: row jj of the window
  // ending before token `end`.  The destination's are loaded at the start by
  // token group 0 (the only threads that read the initial window) -- input
  // T - (W-1) + jj of the sequence, or of the initial window before it --
  // and stored once those threads' chunk-0 reads are done.
  static constexpr int kVw = sizeof(Act) == 2 ? 1 : 2;   // words per row of two channels
  __device__ __forceinline__ void vwin_load(Prod& p) const {
    const int W1 = a.W - 1, vch = opaque(p.vch);
#pragma unroll
    for (int jj = 0; jj < 3; ++jj) {
      if (jj < W1) {
        const int rho = T - W1 + jj;   // uniform
        const rsrc_t r = rho >= 0 ? seq_row(rho) : win_rows();
        const int off = rho >= 0 ? vch * static_cast<int>(sizeof(Act)) : win_off(rho, vch);
        if constexpr (kVw == 1) {
          p.vwin[jj][0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
        } else {
          typedef uint32_t u2 __attribute__((ext_vector_type(2)));
          const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
          p.vwin[jj][0] = v[0];
          p.vwin[jj][1] = v[1];
        }
      }
    }
  }
  __device__ __forceinline__ void vrow_put(int32_t slot, int jj, int vch, const uint32_t* w) const {
    Act* d = static_cast<Act*>(a.conv) + (static_cast<int64_t>(slot) * (a.W - 1) + jj) * a.C + vch;
    if constexpr (kVw == 1)
      *reinterpret_cast<uint32_t*>(d) = w[0];
    else
      *reinterpret_cast<uint2*>(d) = uint2{w[0], w[1]};
  }
  __device__ __forceinline__ void vwin_store(const Prod& p) const {
#pragma unroll
    for (int jj = 0; jj < 3; ++jj)
      if (jj < a.W - 1) vrow_put(dst, jj, p.vch, p.vwin[jj]);
  }

  // Prepared q / k pieces of chunk c0 and the raw value inputs.
  __device__ __forceinline__ void prod_load(Prod& p, int c0) const {
    const int vt = opaque(p.vt), vch = opaque(p.vch);
    const rsrc_t rq = qk_rows<DK>(a, t0, T, c0, kT);
    const int step = kTs * a.Hk * 4 * DK * 2;   // workspace bytes between a thread's pieces
#pragma unroll
    for (int i = 0; i < kCopy; ++i)
      p.row[i] = __builtin_amdgcn_raw_buffer_load_b128(rq, p.qoff, i * step, 0);
    const rsrc_t rx = x_rows(c0);
    if (p.von) {
#pragma unroll
      for (int r = 0; r < kVRaw; ++r) {
        const int off = x_off(c0, c0 + kVt * vt - 3 + r, vch);
        if constexpr (sizeof(Act) == 2) {
          p.vraw[r][0] = __builtin_amdgcn_raw_buffer_load_b32(rx, off, 0, 0);
        } else {
          typedef uint32_t u2 __attribute__((ext_vector_type(2)));
          const u2 v = __builtin_amdgcn_raw_buffer_load_b64(rx, off, 0, 0);
          p.vraw[r][0] = v[0];
          p.vraw[r][1] = v[1];
        }
      }
    }
    if (c0 == 0) {
      // rows -3..-1 (thread tokens 0..2 of token group 0) from the window;
      // every other offset lies past the window and reads zero
      const rsrc_t rw = win_rows();
      if (p.von) {
#pragma unroll
        for (int r = 0; r < 3; ++r) {
          const int off = win_off(kVt * vt - 3 + r, vch);
          if constexpr (sizeof(Act) == 2) {
            p.vraw[r][0] |= __builtin_amdgcn_raw_buffer_load_b32(rw, off, 0, 0);
          } else {
            typedef uint32_t u2 __attribute__((ext_vector_type(2)));
            const u2 v = __builtin_amdgcn_raw_buffer_load_b64(rw, off, 0, 0);
            p.vraw[r][0] |= v[0];
            p.vraw[r][1] |= v[1];
          }
        }
      }
    }
  }

  // The value conv (+ SiLU) of the prefetched inputs of chunk c0.
  __device__ void prod_prep(Prod& p, int c0) const {
    const float* wl = fp(P::oW);
    const float* bl = fp(P::oB);
    if (p.von) {
      float xr[kVRaw][2];
#pragma unroll
      for (int r = 0; r < kVRaw; ++r) {
        if constexpr (sizeof(Act) == 2) {
          xr[r][0] = __uint_as_float(p.vraw[r][0] << 16);
          xr[r][1] = __uint_as_float(p.vraw[r][0] & 0xffff0000u);
        } else {
          xr[r][0] = __uint_as_float(p.vraw[r][0]);
          xr[r][1] = __uint_as_float(p.vraw[r][1]);
        }
      }
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const f4 vw = *reinterpret_cast<const f4*>(wl + 4 * (2 * p.vp + m));
        const float vb = bl[2 * p.vp + m];
#pragma unroll
        for (int tt = 0; tt < kVt; ++tt) {
          float y = vb;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) y = fmaf(vw[jj], xr[tt + jj][m], y);
          p.vo[m][tt / 4][tt % 4] = c0 + kVt * p.vt + tt < T ? act(y) : 0.f;
        }
      }
      // A checkpoint after this chunk: its window is the chunk's last W-1
      // rows, the last raw rows of the last token group.
      const int W1 = a.W - 1;
      if (a.ckpt && W1 > 0 && p.vt == kT / kVt - 1 && (c0 + kT) % a.ckpt_every == 0) {
        const int32_t cs = ckpt_slot(a, s, c0 + kT, T);
        if (cs >= 0) {
          if (W1 == 3) {
            vrow_put(cs, 0, p.vch, p.vraw[kVRaw - 3]);
            vrow_put(cs, 1, p.vch, p.vraw[kVRaw - 2]);
            vrow_put(cs, 2, p.vch, p.vraw[kVRaw - 1]);
          } else if (W1 == 2) {
            vrow_put(cs, 0, p.vch, p.vraw[kVRaw - 2]);
            vrow_put(cs, 1, p.vch, p.vraw[kVRaw - 1]);
          } else {
            vrow_put(cs, 0, p.vch, p.vraw[kVRaw - 1]);
          }
        }
      }
    }
  }

  // Raw bits of the gate inputs a, b of chunk c0 (token = lane < kT),
  // loaded a chunk ahead of their use through descriptors over the
  // sequence's rows (rows past it read zero); converted only where used, so
  // the loads are not waited for here.
  struct GateIn {
    uint32_t al, bt;
    int c0;
  };
  __device__ __forceinline__ GateIn gate_load(int c0) const {
    constexpr int kE = static_cast<int>(sizeof(Act));
    const uint32_t bytes = static_cast<uint32_t>(T) * static_cast<uint32_t>(a.Hv) * kE;
    const int64_t base = static_cast<int64_t>(t0) * a.Hv;
    const rsrc_t ra = make_rsrc(static_cast<const Act*>(a.alpha) + base, bytes);
    const rsrc_t rb = make_rsrc(static_cast<const Act*>(a.beta) + base, bytes);
    const uint32_t off =
        lane < kT ? static_cast<uint32_t>(((c0 + lane) * a.Hv + h) * kE) : kOutOfRange;
    GateIn r;
    r.c0 = c0;
    if constexpr (kE == 2) {
      r.al = __builtin_amdgcn_raw_buffer_load_b16(ra, off, 0, 0);
      r.bt = __builtin_amdgcn_raw_buffer_load_b16(rb, off, 0, 0);
    } else {
      r.al = __builtin_amdgcn_raw_buffer_load_b32(ra, off, 0, 0);
      r.bt = __builtin_amdgcn_raw_buffer_load_b32(rb, off, 0, 0);
    }
    return r;
  }

  // The gates of chunk c into its buffer (one wave, token = lane < kT):
  // g = prefix sums of log a over the chunk, b, e^g and e^{g_c - g}; tokens
  // past the sequence take a = 1, b = 0 and add nothing.  The scan runs
  // inside each row of 16 lanes (DPP shifts, zero filled), then row 1 adds
  // row 0's total.
  __device__ void gates(const GateIn& in, int c) const {
    const bool valid = lane < kT && in.c0 + lane < T;
    const float al = valid ? __uint_as_float(sizeof(Act) == 2 ? in.al << 16 : in.al) : 1.f;
    const float bt = valid ? __uint_as_float(sizeof(Act) == 2 ? in.bt << 16 : in.bt) : 0.f;
    float g = fmaxf(logf(al), -80.0f);
    g += row_shr<1>(g);
    g += row_shr<2>(g);
    g += row_shr<4>(g);
    g += row_shr<8>(g);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), 15));
    if (lane >= 16) g += r0;
    const float gc = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g), kT - 1));
    if (lane < kT) {
      float* gt = fp(P::gate(c));
      gt[lane] = g;
      gt[kT + lane] = bt;
      gt[2 * kT + lane] = expf(g);
      gt[3 * kT + lane] = expf(gc - g);
    }
  }

  // Store prepared chunk c: the K, Q pieces and the value columns.
  __device__ void prod_store(const Prod& p, int c) const {
    unsigned char* buf = lds + P::kq(c, 0);
#pragma unroll
    for (int i = 0; i < kCopy; ++i)
      *reinterpret_cast<u4*>(buf + p.lds[(i >> 1) & 1] + 2 * kTs * i * P::kRowQK) = p.row[i];
    if (p.von) {
      float* vt = fp(P::v(c));
      const int vp = opaque(p.vp), vtk = opaque(p.vt);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
          *reinterpret_cast<f4*>(vt + (2 * vp + m) * P::kRowV + kVt * vtk + 4 * hf) = p.vo[m][hf];
    }
  }

  // ================= producers, second half: A, P and the inverses ======
  // Element offsets, for rows 16 blk + lr, of the 16x16x32 operand slots
  // 32 sl + 8 lg: a per-slice base plus 16 blk rows (the swizzle depends on
  // the row only through lr).
  __device__ __forceinline__ void op_bases(int (&ob)[kSl]) const {
    const int l = lane_now(), r = l & 15, g = l >> 4;
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) ob[sl] = qk(r, 32 * sl + 8 * g);
  }

  // Tiles of token blocks (IB, JB), IB >= JB, of K K^T (G) and / or Q K^T
  // (PQ), computed transposed (A operand K rows JB, B operands K and Q rows
  // IB) so that each lane holds row r = 16 IB + lr at the four columns
  // 16 JB + 4 lg + v: they store as one 8-byte (hi, lo) group each.
  template <int IB, int JB, bool G, bool PQ>
  __device__ __forceinline__ void tiles(f4& g, f4& pq, const int (&ob)[kSl], int c) const {
    const short* kh = sp(P::kq(c, P::Kh));
    const short* kl = sp(P::kq(c, P::Kl));
    const short* qh = sp(P::kq(c, P::Qh));
    const short* ql = sp(P::kq(c, P::Ql));
    // two accumulators per product (even and odd slices) halve the chain
    // of dependent MFMAs; every operand read is issued first
    f4 gs[2], ps[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      gs[i] = f4{0.f, 0.f, 0.f, 0.f};
      ps[i] = f4{0.f, 0.f, 0.f, 0.f};
    }
    s8 ah[kSl], al[kSl], bkh[kSl], bkl[kSl], bqh[kSl], bql[kSl];
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      const int oa = 16 * JB * P::kRowQK + ob[sl], obr = 16 * IB * P::kRowQK + ob[sl];
      ah[sl] = *reinterpret_cast<const s8*>(kh + oa);
      al[sl] = *reinterpret_cast<const s8*>(kl + oa);
      if constexpr (G && IB != JB) {
        bkh[sl] = *reinterpret_cast<const s8*>(kh + obr);
        bkl[sl] = *reinterpret_cast<const s8*>(kl + obr);
      }
      if constexpr (PQ) {
        bqh[sl] = *reinterpret_cast<const s8*>(qh + obr);
        bql[sl] = *reinterpret_cast<const s8*>(ql + obr);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      if constexpr (G) {
        if constexpr (IB == JB)
          gs[sl & 1] = mma32x3(ah[sl], al[sl], ah[sl], al[sl], gs[sl & 1]);
        else
          gs[sl & 1] = mma32x3(ah[sl], al[sl], bkh[sl], bkl[sl], gs[sl & 1]);
      }
      if constexpr (PQ) ps[sl & 1] = mma32x3(ah[sl], al[sl], bqh[sl], bql[sl], ps[sl & 1]);
    }
    g = gs[0] + gs[1];
    pq = ps[0] + ps[1];
  }

  // Decays e^{g_r - g_i} of a transposed tile: r = 16 IB + lr, i = 16 JB +
  // 4 lg + v.
  template <int IB, int JB>
  __device__ __forceinline__ f4 decays(const float* gt) const {
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    const float gr = gt[16 * IB + lr];
    const f4 gi = *reinterpret_cast<const f4*>(gt + 16 * JB + 4 * lg);
    f4 dec;
#pragma unroll
    for (int v = 0; v < 4; ++v) dec[v] = __expf(gr - gi[v]);
    return dec;
  }

  // P_ri = e^{g_r - g_i} q_r.k_i (i <= r) from a transposed Q K^T tile.
  template <int IB, int JB>
  __device__ __forceinline__ void store_p(const f4& pq, int c) const {
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    const float* gt = fp(P::gate(c));
    const int o = (16 * IB + lr) * P::kRowT + slot(16 * JB + 4 * lg);
    f4 pv = decays<IB, JB>(gt) * pq;
    if (IB == JB) {
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (4 * lg + v > lr) pv[v] = 0.f;
    }
    s4 h, lo;
    split4(pv, h, lo);
    *reinterpret_cast<s4*>(sp(P::pa(c, P::Ph)) + o) = h;
    *reinterpret_cast<s4*>(sp(P::pa(c, P::Pl)) + o) = lo;
  }

  // A_ri = b_r e^{g_r - g_i} k_r.k_i (IB > JB) from a transposed K K^T tile.
  template <int IB, int JB>
  __device__ __forceinline__ void store_a(const f4& g, int c) const {
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    const float* gt = fp(P::gate(c));
    const int r = 16 * IB + lr;
    const int o = r * P::kRowT + slot(16 * JB + 4 * lg);
    s4 h, lo;
    split4(gt[kT + r] * decays<IB, JB>(gt) * g, h, lo);
    *reinterpret_cast<s4*>(sp(P::pa(c, P::Ah)) + o) = h;
    *reinterpret_cast<s4*>(sp(P::pa(c, P::Al)) + o) = lo;
  }

  // Diagonal block b from its raw K K^T tile G: N = the strictly lower block
  // of A, X = (I + N)^{-1}, stored in A layout (X[lr][4 lg + v]) in the
  // diagonal block of the A planes.
  __device__ void diag_inverse(int b, const f4& G, int c) const {
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    const float* gt = fp(P::gate(c));
    const float gi = gt[16 * b + lr], bi = gt[kT + 16 * b + lr];
    const f4 gr = *reinterpret_cast<const f4*>(gt + 16 * b + 4 * lg);
    const f4 br = *reinterpret_cast<const f4*>(gt + kT + 16 * b + 4 * lg);
    f4 nb, na;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int rv = 4 * lg + v;
      nb[v] = lr < rv ? br[v] * __expf(gr[v] - gi) * G[v] : 0.f;  // N[rv][lr]
      na[v] = rv < lr ? bi * __expf(gi - gr[v]) * G[v] : 0.f;     // N[lr][rv]
    }
    const f4 xt = unit_lower_inverse(na, nb, lr, lg);
    s4 xh, xl;
    split4(xt, xh, xl);
    const int o = (16 * b + lr) * P::kRowT + slot(16 * b + 4 * lg);
    *reinterpret_cast<s4*>(sp(P::pa(c, P::Ah)) + o) = xh;
    *reinterpret_cast<s4*>(sp(P::pa(c, P::Al)) + o) = xl;
  }

  // A, P and the inverses of chunk c over the 4 producer waves: waves 0 and 1 the
  // diagonal K K^T tiles and their inverses, wave 2 the diagonal Q K^T
  // tiles, wave 3 the off-diagonal pair.
  __device__ void gram_phase(int c) const {
    int ob[kSl];
    op_bases(ob);
    f4 g, pq;
    switch (wave) {
      case 0:
        tiles<0, 0, true, false>(g, pq, ob, c);
        diag_inverse(0, g, c);
        break;
      case 1:
        tiles<1, 1, true, false>(g, pq, ob, c);
        diag_inverse(1, g, c);
        break;
      case 2:
        tiles<0, 0, false, true>(g, pq, ob, c);
        store_p<0, 0>(pq, c);
        tiles<1, 1, false, true>(g, pq, ob, c);
        store_p<1, 1>(pq, c);
        break;
      default:
        tiles<1, 0, true, true>(g, pq, ob, c);
        store_a<1, 0>(g, c);
        store_p<1, 0>(pq, c);
        break;
    }
  }

  // ================= consumers =================
  // The loop-carried chain of a consumer is S -> K S0^T -> U -> S; Q S0^T and
  // the outputs hang off it.  So S enters a chunk already split into bf16
  // (hi, lo) operands (split at the end of the previous chunk, where it
  // overlaps the state update), K S0^T comes first, and Q S0^T follows the
  // serial U chain, whose MFMA gaps it fills.
  //
  // S[d] holds rows 16d + 4 lg + v (key index) of S^T at column e0 + lr
  // (value index); Sh[sl], Sl[sl] its 32-row slice sl as 16x16x32 B
  // operands.  U[b] and qs[b] hold rows 16 b + 4 lg + v (token) at that
  // column.
  __device__ __forceinline__ static void split_state(const f4 (&S)[kDt], s8 (&Sh)[kSl],
                                                     s8 (&Sl)[kSl]) {
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      s4 h0, l0, h1, l1;
      split4(S[2 * sl], h0, l0);
      split4(S[2 * sl + 1], h1, l1);
      Sh[sl] = cat(h0, h1);
      Sl[sl] = cat(l0, l1);
    }
  }

  // X S0^T for the chunk's rows X (K or Q planes), rows 16 tb + 4 lg + v.
  __device__ __forceinline__ void rows_times_state(const short* xh_, const short* xl_,
                                                   const s8 (&Sh)[kSl], const s8 (&Sl)[kSl],
                                                   f4 (&r)[kNb]) const {
#pragma unroll
    for (int tb = 0; tb < kNb; ++tb) r[tb] = f4{0.f, 0.f, 0.f, 0.f};
    int ob[kSl];
    op_bases(ob);
    // every operand read is issued before the first product, so their LDS
    // latencies overlap instead of each one stalling its MFMA
    s8 xh[kSl][kNb], xl[kSl][kNb];
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl)
#pragma unroll
      for (int tb = 0; tb < kNb; ++tb) {
        const int ra = 16 * tb * P::kRowQK + ob[sl];
        xh[sl][tb] = *reinterpret_cast<const s8*>(xh_ + ra);
        xl[sl][tb] = *reinterpret_cast<const s8*>(xl_ + ra);
      }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
#pragma unroll
      for (int tb = 0; tb < kNb; ++tb) r[tb] = mma32(xl[sl][tb], Sh[sl], r[tb]);
#pragma unroll
      for (int tb = 0; tb < kNb; ++tb) r[tb] = mma32(xh[sl][tb], Sl[sl], r[tb]);
#pragma unroll
      for (int tb = 0; tb < kNb; ++tb) r[tb] = mma32(xh[sl][tb], Sh[sl], r[tb]);
    }
  }

  // First half of chunk c for the wave's 16 value columns: K S0^T, the
  // updates U (and their (hi, lo) split), then Q S0^T.
  __device__ void updates(const s8 (&Sh)[kSl], const s8 (&Sl)[kSl], f4 (&U)[kNb],
                          s4 (&uh)[kNb], s4 (&ul)[kNb], f4 (&qs)[kNb], int c) const {
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    const float* gt = fp(P::gate(c));
    f4 ks[kNb];
    rows_times_state(sp(P::kq(c, P::Kh)), sp(P::kq(c, P::Kl)), Sh, Sl, ks);
    // U_b = X_bb (b_b R_b - sum_{j<b} A_bj U_j),  R = V - e^g (K S0^T)
    const float* vt = fp(P::v(c)) + (e0 % kCols + lr) * P::kRowV;
    const short* ah_ = sp(P::pa(c, P::Ah));
    const short* al_ = sp(P::pa(c, P::Al));
#pragma unroll
    for (int b = 0; b < kNb; ++b) {
      const int row = (16 * b + lr) * P::kRowT;
      f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jb = 0; jb < b; ++jb) {
        const int o = row + slot(16 * jb + 4 * lg);
        acc = mma16x3(*reinterpret_cast<const s4*>(ah_ + o), *reinterpret_cast<const s4*>(al_ + o),
                      uh[jb], ul[jb], acc);
      }
      const int o = row + slot(16 * b + 4 * lg);
      const s4 xh = *reinterpret_cast<const s4*>(ah_ + o);
      const s4 xl = *reinterpret_cast<const s4*>(al_ + o);
      const f4 V = *reinterpret_cast<const f4*>(vt + 16 * b + 4 * lg);
      const f4 gam = *reinterpret_cast<const f4*>(gt + 2 * kT + 16 * b + 4 * lg);
      const f4 bt = *reinterpret_cast<const f4*>(gt + kT + 16 * b + 4 * lg);
      s4 zh, zl;
      split4(bt * (V - gam * ks[b]) - acc, zh, zl);
      U[b] = mma16x3(xh, xl, zh, zl, f4{0.f, 0.f, 0.f, 0.f});
      split4(U[b], uh[b], ul[b]);
    }
    rows_times_state(sp(P::kq(c, P::Qh)), sp(P::kq(c, P::Ql)), Sh, Sl, qs);
  }

  // Second half: O = e^g (Q S0^T) + P U to the output rows of chunk c
  // (rows past the sequence lie past the descriptor and are dropped), then
  // S^T <- e^{g_c} S^T + K^T diag(e^{g_c - g}) U, and its split for the
  // next chunk.
  __device__ void outputs_and_state(f4 (&S)[kDt], s8 (&Sh)[kSl], s8 (&Sl)[kSl],
                                    const f4 (&U)[kNb], const s4 (&uh)[kNb],
                                    const s4 (&ul)[kNb], const f4 (&qs)[kNb], int c) const {
    const int c0 = c * kT;
    const int l = lane_now(), lr = l & 15, lg = l >> 4;
    const float* gt = fp(P::gate(c));
    const s8 u0h = cat(uh[0], uh[1]), u0l = cat(ul[0], ul[1]);
    {
      const short* ph_ = sp(P::pa(c, P::Ph));
      const short* pl_ = sp(P::pa(c, P::Pl));
      f4 o[kNb];
#pragma unroll
      for (int b = 0; b < kNb; ++b) {
        const int off = (16 * b + lr) * P::kRowT + 8 * lg;
        const s8 ph = *reinterpret_cast<const s8*>(ph_ + off);
        const s8 pl = *reinterpret_cast<const s8*>(pl_ + off);
        o[b] = *reinterpret_cast<const f4*>(gt + 2 * kT + 16 * b + 4 * lg) * qs[b];
        o[b] = mma32x3(ph, pl, u0h, u0l, o[b]);
      }
      const int rs = a.Hv * a.dv;
      const int n = T - c0 < kT ? T - c0 : kT;
      const rsrc_t ro =
          make_rsrc(a.out + ((static_cast<int64_t>(t0) + c0) * a.Hv + h) * a.dv + e0,
                    static_cast<uint32_t>(n) * static_cast<uint32_t>(rs) * 4u);
#pragma unroll
      for (int b = 0; b < kNb; ++b)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[b][v]), ro,
                                                ((16 * b + 4 * lg + v) * rs + lr) * 4, 0, 0);
    }
    // The state update: K^T tiles by transposing reads of the K rows.
    const short* kh = sp(P::kq(c, P::Kh));
    const short* kl = sp(P::kq(c, P::Kl));
    s8 wh, wl;
    {
      const f4 g0 = *reinterpret_cast<const f4*>(gt + 3 * kT + 4 * lg);
      const f4 g1 = *reinterpret_cast<const f4*>(gt + 3 * kT + 16 + 4 * lg);
      s4 h0, l0, h1, l1;
      split4(g0 * U[0], h0, l0);
      split4(g1 * U[1], h1, l1);
      wh = cat(h0, h1);
      wl = cat(l0, l1);
    }
    const float ec = gt[2 * kT + kT - 1];
    // K^T tile d, half hf: rows 16hf + 4 lg + lr/4, slots 32 (d>>1) + 4 (d&1)
    // + 8 (lr&3); a base per pair D = d >> 1 plus 16hf rows and 4 (d&1) slots.
    int tb0[kSl];
    {
      const int l2 = lane_now(), r = l2 & 15, g = l2 >> 4;
#pragma unroll
      for (int D = 0; D < kSl; ++D) tb0[D] = qk(4 * g + (r >> 2), 32 * D + 8 * (r & 3));
    }
    // all transposing reads first (their latencies overlap), then the products
    s8 th[kDt], tl[kDt];
#pragma unroll
    for (int d = 0; d < kDt; ++d) {
      const int r0 = tb0[d >> 1] + 4 * (d & 1);
      const int r1 = r0 + 16 * P::kRowQK;
      th[d] = cat(ld_tr(kh + r0), ld_tr(kh + r1));
      tl[d] = cat(ld_tr(kl + r0), ld_tr(kl + r1));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int d = 0; d < kDt; ++d) S[d] = ec * S[d];
#pragma unroll
    for (int d = 0; d < kDt; ++d) S[d] = mma32(tl[d], wh, S[d]);
#pragma unroll
    for (int d = 0; d < kDt; ++d) S[d] = mma32(th[d], wl, S[d]);
#pragma unroll
    for (int d = 0; d < kDt; ++d) S[d] = mma32(th[d], wh, S[d]);
    split_state(S, Sh, Sl);
  }
};

template <int DK, typename Act, int DKR>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  using K = Prefill<DK, Act, DKR>;
  using P = Plan<DK>;
  K k{{a, lds_raw}};
  k.tid = threadIdx.x;
  k.wave = __builtin_amdgcn_readfirstlane(k.tid >> 6);  // uniform: offsets from it stay scalar
  k.lane = k.tid & 63;
  k.lr = k.lane & 15;
  k.lg = k.lane >> 4;

  // Units (sequence, value head, column block) in that order; consecutive
  // units -- the value heads sharing a key head -- go to one XCD, whose L2
  // then serves their common q / k reads (workgroups are dealt to the 8
  // XCDs round robin).
  const int nb = gridDim.x;
  const int bid = blockIdx.x;
  const int u = (nb % 8 == 0) ? (bid % 8) * (nb / 8) + bid / 8 : bid;
  const int j = u % a.nblk;
  k.h = (u / a.nblk) % a.Hv;
  const int s = u / a.nblk / a.Hv;
  k.hk = k.h / a.G;

  const int t0 = a.cu[s], t1 = a.cu[s + 1];
  const int32_t dst = a.dst[s];
  k.init = a.init ? a.init[s] : dst;
  if (t0 < 0 || t1 < t0 || t1 > a.total || dst < 0 || dst >= a.num_slots ||
      k.init >= a.num_slots)
    return;
  k.t0 = t0;
  k.T = t1 - t0;
  k.s = s;
  k.dst = dst;
  const int nch = (k.T + kT - 1) / kT;

  // P and A planes of both buffers: the tiles above the diagonal stay zero.
  for (int i = k.tid; i < 2 * 4 * P::kSq / 16; i += kThreads)
    reinterpret_cast<uint4*>(lds_raw + P::oPA)[i] = uint4{0u, 0u, 0u, 0u};
  k.e0 = j * kCols;
  k.load_taps();

  // One barrier per chunk.  Between barriers c - 1 and c the consumers run
  // chunk c while the producers store chunk c + 2 (wave 1: its gates too) and
  // form chunk c + 1's A, P and inverses (its K, Q and gates were stored an
  // iteration earlier).
  if (k.tid < kProd) {
    // ---------------- producers ----------------
    typename K::Prod p;
    k.prod_init(p);
    // the destination window of the value channels (see vwin_load)
    const bool vwin = a.W > 1 && p.von && p.vt == 0;
    if (vwin) k.vwin_load(p);
    if (nch > 0) k.prod_load(p, 0);
    if (vwin && nch == 0) k.vwin_store(p);
    lds_barrier();            // planes zeroed, taps loaded
    typename K::GateIn gin{0u, 0u, 0};
    if (k.wave == kGateWave) {
      for (int c = 0; c < 2 && c < nch; ++c) k.gates(k.gate_load(c * kT), c);
      if (nch > 2) gin = k.gate_load(2 * kT);
    }
    // (the prepared rows are loaded straight into the registers they are
    // stored from: each chunk's store comes before the next chunk's load)
    for (int c = 0; c < 2 && c < nch; ++c) {
      k.prod_prep(p, c * kT);
      if (vwin && c == 0) k.vwin_store(p);   // chunk 0's reads of the initial window are used
      k.prod_store(p, c);
      if (c + 1 < nch) k.prod_load(p, (c + 1) * kT);
    }
    lds_barrier();            // chunks 0 and 1 stored, their gates written
    if (nch > 0) k.gram_phase(0);
    lds_barrier();            // chunk 0 complete
    for (int c = 0; c < nch; ++c) {
      if (c + 2 < nch) {
        k.prod_prep(p, (c + 2) * kT);
        k.prod_store(p, c + 2);
        if (c + 3 < nch) k.prod_load(p, (c + 3) * kT);
      }
      if (c + 1 < nch) k.gram_phase(c + 1);
      if (k.wave == kGateWave && c + 2 < nch) {
        k.gates(gin, c + 2);
        if (c + 3 < nch) gin = k.gate_load((c + 3) * kT);
      }
      lds_barrier();          // chunk c consumed
    }
  } else {
    // ---------------- consumers ----------------
    k.e0 = j * kCols + (k.wave - 4) * 16;
    const bool cols = k.e0 < a.dv;
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
    s8 Sh[K::kSl], Sl[K::kSl];
    K::split_state(S, Sh, Sl);
    lds_barrier();            // planes zeroed, taps loaded
    lds_barrier();            // chunks 0 and 1 stored, their gates written
    lds_barrier();            // chunk 0 complete
    for (int c = 0; c < nch; ++c) {
      f4 U[kNb], qs[kNb];
      s4 uh[kNb], ul[kNb];
      if (cols) k.updates(Sh, Sl, U, uh, ul, qs, c);
      if (cols) k.outputs_and_state(S, Sh, Sl, U, uh, ul, qs, c);
      const int32_t cs = __builtin_amdgcn_readfirstlane(ckpt_slot(a, s, (c + 1) * kT, k.T));
      if (cols && cs >= 0) {  // the state after (c + 1) * kT tokens, to a checkpoint slot
        const int l = k.lane_now();
        float* o = a.ssm + cs * slot_elems + head + static_cast<int64_t>(k.e0 + (l & 15)) * DKR;
#pragma unroll
        for (int d = 0; d < kDtR; ++d) *reinterpret_cast<f4*>(o + 16 * d + 4 * (l >> 4)) = S[d];
      }
      lds_barrier();          // chunk c consumed
    }
    if (cols) {
      float* out = a.ssm + dst * slot_elems + head + static_cast<int64_t>(k.e0 + k.lr) * DKR;
#pragma unroll
      for (int d = 0; d < kDtR; ++d) *reinterpret_cast<f4*>(out + 16 * d + 4 * k.lg) = S[d];
    }
  }
}


template <int DK, typename Act, int DKR>
__global__ void __launch_bounds__(256) qk_prep_kernel(PrefillArgs a, int nchunk) {
  const int hk = blockIdx.x % a.Hk;
  const int first = (blockIdx.x / a.Hk) % nchunk;
  const int s = blockIdx.x / a.Hk / nchunk;
  const int t0 = a.cu[s], t1 = a.cu[s + 1];
  const int32_t dst = a.dst[s];
  const int32_t init = a.init ? a.init[s] : dst;
  if (t0 < 0 || t1 < t0 || t1 > a.total || dst < 0 || dst >= a.num_slots || init >= a.num_slots)
    return;
  QkPrep<DK, Act, DKR> q{{a, nullptr}};
  q.s = s;
  q.dst = dst;
  q.tid = threadIdx.x;
  q.wave = __builtin_amdgcn_readfirstlane(q.tid >> 6);
  q.lane = q.tid & 63;
  q.lr = q.lane & 15;
  q.lg = q.lane >> 4;
  q.h = q.e0 = 0;
  q.hk = hk;
  q.t0 = t0;
  q.T = t1 - t0;
  q.init = init;
  // chunks first, first + nchunk, ...: every chunk is covered whatever the
  // grid assumed of the longest sequence
  q.run(first, nchunk);
}

// DKR: the layer's d_k; DK the layout it runs in (32 for d_k = 16).
template <int DK, typename Act, int DKR = DK>
hipError_t launch_one(const PrefillArgs& a, int max_seqlen, hipStream_t st) {
  // About 8 workgroups per CU: each covers every nchunk-th chunk of its
  // (sequence, key head), prefetching the next while computing one.
  const int64_t per = static_cast<int64_t>(a.N) * a.Hk;
  const int64_t want = 2048 / per > 0 ? 2048 / per : 1;
  const int64_t most = max_seqlen > 0 ? (max_seqlen + kT - 1) / kT : 1;
  const int64_t nchunk = want < most ? want : most;
  hipLaunchKernelGGL((qk_prep_kernel<DK, Act, DKR>), dim3(static_cast<uint32_t>(nchunk * per)),
                     dim3(256), 0, st, a, static_cast<int>(nchunk));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int bytes = Plan<DK>::kBytes;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<DK, Act, DKR>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const int grid = a.N * a.Hv * a.nblk;
  hipLaunchKernelGGL((prefill_kernel<DK, Act, DKR>), dim3(grid), dim3(kThreads), bytes, st, a);
  return hipGetLastError();
}

static_assert(Plan<128>::kBytes <= 160 * 1024, "LDS plan exceeds 160 KiB");
static_assert(kT == 32, "the tile code assumes two 16-token blocks per chunk");

}  // namespace

int prefill_supported(int dk, int kda) {
  (void)kda;
  return dk == 16 || dk == 32 || dk == 64 || dk == 128;   // 16 in the 32 layout
}

size_t qk_workspace_bytes(int Hk, int dk, int64_t total) {
  const int dk_layout = dk < 32 ? 32 : dk;   // d_k = 16 runs the d_k = 32 layout
  return static_cast<size_t>(total) * Hk * dk_layout * 8;
}

hipError_t launch_prefill(const PrefillArgs& a, int dk, int act_bf16, int max_seqlen,
                          hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  switch (dk) {
    case 16:
      return act_bf16 ? launch_one<32, bf16, 16>(a, max_seqlen, s)
                      : launch_one<32, float, 16>(a, max_seqlen, s);
    case 32:
      return act_bf16 ? launch_one<32, bf16>(a, max_seqlen, s)
                      : launch_one<32, float>(a, max_seqlen, s);
    case 64:
      return act_bf16 ? launch_one<64, bf16>(a, max_seqlen, s)
                      : launch_one<64, float>(a, max_seqlen, s);
    case 128:
      return act_bf16 ? launch_one<128, bf16>(a, max_seqlen, s)
                      : launch_one<128, float>(a, max_seqlen, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
