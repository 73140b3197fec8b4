// gdn_prefill.hip -- chunked prefill of the gated delta rule on gfx950.
//
// The recurrence S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,
// o_t = S_t q_t is evaluated 64 tokens at a time in its WY / UT-transform
// form (Yang et al., "Parallelizing Linear Transformers with the Delta Rule
// over Sequence Length", 2024, sec. 3; with the scalar decay of "Gated Delta
// Networks", 2025, sec. 3).  For a chunk with rows K, Q (normalised keys and
// queries), V, log-decay prefix sums g and state S0 before the chunk:
//   A_ri = b_r e^{g_r - g_i} k_r . k_i            (i < r)
//   (I + A) U = diag(b) (V - diag(e^g) K S0^T)    (U: the chunk's updates)
//   O = diag(e^g) Q S0^T + P U,  P_ri = e^{g_r - g_i} q_r . k_i   (i <= r)
//   S = e^{g_c} S0 + U^T diag(e^{g_c - g}) K       (g_c: the chunk's last g)
// The triangular system is solved blockwise: the four 16x16 diagonal blocks
// of (I + A) are inverted by forward substitution in fp32, and U is formed
// block row by block row, U_b = X_bb (b_b R_b - sum_{j<b} A_bj U_j).
//
// Work split.  Rows of S are independent through the whole recurrence (row
// i of S, U and O depend only on row i of S0), so a workgroup owns one
// (sequence, value head, 64 value columns) and walks that sequence's chunks
// in order, its 64x d_k slice of S^T held in MFMA accumulators across
// chunks.  Per chunk its 4 waves:
//   1. conv1d + SiLU + L2 norm of the chunk's q and k (8 channels x 8 tokens
//      per thread), stored as bf16 (hi, lo) pairs; gates and prefix sums;
//   2. the 20 lower 16x16 tiles of K K^T and Q K^T  -> A, P;
//   3. inverses of the diagonal blocks of (I + A);
//   4. per wave, 16 value columns: K S0^T, Q S0^T, the value conv, U, O and
//      the state update.
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
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef short s8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

constexpr int kC = 64;         // chunk length
constexpr int kThreads = 256;  // 4 waves
constexpr int kCols = 64;      // value columns per workgroup (16 per wave)

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi) (round to nearest even).
__device__ __forceinline__ void split(float x, short& hi, short& lo) {
  const __bf16 h = static_cast<__bf16>(x);
  const __bf16 l = static_cast<__bf16>(x - static_cast<float>(h));
  hi = __builtin_bit_cast(short, h);
  lo = __builtin_bit_cast(short, l);
}
__device__ __forceinline__ void split4(f4 x, s4& hi, s4& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    short h, l;
    split(x[i], h, l);
    hi[i] = h;
    lo[i] = l;
  }
}

__device__ __forceinline__ f4 mma32(s8 a, s8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8, a),
                                                 __builtin_bit_cast(b8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f4 mma16(s4 a, s4 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// c + a*b with both operands given as (hi, lo) pairs.
__device__ __forceinline__ f4 mma32x3(s8 ah, s8 al, s8 bh, s8 bl, f4 c) {
  c = mma32(al, bh, c);
  c = mma32(ah, bl, c);
  return mma32(ah, bh, c);
}
__device__ __forceinline__ f4 mma16x3(s4 ah, s4 al, s4 bh, s4 bl, f4 c) {
  c = mma16(al, bh, c);
  c = mma16(ah, bl, c);
  return mma16(ah, bh, c);
}
__device__ __forceinline__ s8 cat(s4 x, s4 y) {
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Storage slot of contraction index i: inside each block of 32, index
// 16h + 4g + j (h < 2, g < 4, j < 4) sits at 8g + 4h + j.  Lane group g of a
// 16x16x32 operand then reads 8 consecutive slots holding rows 4g..4g+3 of
// the two 16-row tiles of the block.
__device__ __forceinline__ int slot(int i) {
  return (i & ~31) | (((i >> 2) & 3) << 3) | (((i >> 4) & 1) << 2) | (i & 3);
}

// LDS plan (bytes).  Rows are padded by 16 bytes so that 16 lanes reading
// 16 consecutive rows hit distinct banks.
template <int DK>
struct Plan {
  static constexpr int kRowQK = DK + 8;  // bf16 per row of K, Q   [token][dk]
  static constexpr int kRowT = kC + 8;   // bf16 per row of K^T [dk][token], P, A [token][token]
  static constexpr int kQK = 2 * kC * kRowQK;
  static constexpr int kKT = 2 * DK * kRowT;
  static constexpr int kSq = 2 * kC * kRowT;
  static constexpr int oKh = 0, oKl = oKh + kQK, oQh = oKl + kQK, oQl = oQh + kQK;
  static constexpr int oTh = oQl + kQK, oTl = oTh + kKT;
  static constexpr int oPh = oTl + kKT, oPl = oPh + kSq, oAh = oPl + kSq, oAl = oAh + kSq;
  static constexpr int kAdRow = 17;  // fp32 diagonal blocks of A: [4][16][17]
  static constexpr int oAd = oAl + kSq;
  static constexpr int oGate = oAd + 4 * 16 * kAdRow * 4;  // fp32 [4][64]: g, b, e^g, e^{g_c-g}
  static constexpr int kBytes = oGate + 4 * kC * 4;
};

// Raw input loads (bf16 or fp32 storage -> fp32).
template <typename Act>
__device__ __forceinline__ void load8(const Act* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
  const f4 x = *reinterpret_cast<const f4*>(p);
  const f4 y = *reinterpret_cast<const f4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = x[i];
    v[4 + i] = y[i];
  }
}

template <int DK, typename Act>
struct Prefill {
  using P = Plan<DK>;
  static constexpr int kSl = DK / 32;   // 32-wide slices of d_k
  static constexpr int kDt = DK / 16;   // 16-row tiles of d_k
  static constexpr int kNco = DK / 4;   // channel octets of q and k
  static constexpr int kGrp = DK / 8;   // octets per head (lanes of one norm)

  const PrefillArgs& a;
  unsigned char* lds;
  int tid, wave, lane, lr, lg;
  int s, h, hk, e0;
  int t0, T;
  int32_t dst, init;

  __device__ short* sp(int off) const { return reinterpret_cast<short*>(lds + off); }
  __device__ float* fp(int off) const { return reinterpret_cast<float*>(lds + off); }

  // Row rho of the sequence (rho < 0: the conv window of the initial slot)
  // at channel ch, 8 channels; zero outside the sequence and its window.
  __device__ __forceinline__ void row8(int rho, int ch, float (&v)[8]) const {
    const int W1 = a.W - 1;
    if (rho >= 0 && rho < T) {
      load8<Act>(static_cast<const Act*>(a.x) + (static_cast<int64_t>(t0) + rho) * a.C + ch, v);
    } else if (rho < 0 && rho >= -W1 && init >= 0) {
      load8<Act>(static_cast<const Act*>(a.conv) +
                     (static_cast<int64_t>(init) * W1 + (W1 + rho)) * a.C + ch,
                 v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
  }
  __device__ __forceinline__ float row1(int rho, int ch) const {
    const int W1 = a.W - 1;
    if (rho >= 0 && rho < T)
      return to_f32(static_cast<const Act*>(a.x)[(static_cast<int64_t>(t0) + rho) * a.C + ch]);
    if (rho < 0 && rho >= -W1 && init >= 0)
      return to_f32(static_cast<const Act*>(
          a.conv)[(static_cast<int64_t>(init) * W1 + (W1 + rho)) * a.C + ch]);
    return 0.f;
  }
  // Conv tap jj (0..3, the last on the current token) of channel ch; taps of
  // a narrower conv are left-padded with zeros.
  __device__ __forceinline__ float tap(int ch, int jj) const {
    const int lead = 4 - a.W;
    return jj >= lead ? to_f32(static_cast<const Act*>(a.w)[static_cast<int64_t>(ch) * a.W + jj - lead])
                      : 0.f;
  }
  __device__ __forceinline__ float act(float y) const {
    return a.silu ? y / (1.0f + expf(-y)) : y;
  }

  // ---- step 1: conv + SiLU + L2 norm of q and k for tokens 8*tau..+7 of
  // the chunk at c0, 8 channels (octet co).  Writes K, Q as (hi, lo) rows
  // and K^T as (hi, lo) columns.
  __device__ void prep_qk(int c0, int co, int tau, const float (&wt)[8][4],
                          const float (&bias)[8]) const {
    const bool isk = co >= kGrp;
    const int oc = isk ? co - kGrp : co;
    const int ch = (isk ? a.Hk * DK : 0) + hk * DK + 8 * oc;
    float raw[11][8];
#pragma unroll
    for (int r = 0; r < 11; ++r) row8(c0 + 8 * tau - 3 + r, ch, raw[r]);
    float y[8][8];
    float ss[8];
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      ss[tt] = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        float v = bias[m];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) v = fmaf(wt[m][jj], raw[tt + jj][m], v);
        v = act(v);
        y[tt][m] = v;
        ss[tt] = fmaf(v, v, ss[tt]);
      }
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const float sum = group_sum<kGrp>(ss[tt]);
      float sc = a.l2norm ? rsqrtf(sum + a.eps) : 1.0f;
      if (!isk) sc *= a.q_scale;
      if (c0 + 8 * tau + tt >= T) sc = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) y[tt][m] *= sc;
    }
    // rows: token t, two groups of 4 channels at slot(8*oc) and +8
    short* hi = sp(isk ? P::oKh : P::oQh);
    short* lo = sp(isk ? P::oKl : P::oQl);
    const int sb = slot(8 * oc);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      s4 h0, l0, h1, l1;
      split4(f4{y[tt][0], y[tt][1], y[tt][2], y[tt][3]}, h0, l0);
      split4(f4{y[tt][4], y[tt][5], y[tt][6], y[tt][7]}, h1, l1);
      const int row = (8 * tau + tt) * P::kRowQK + sb;
      *reinterpret_cast<s4*>(hi + row) = h0;
      *reinterpret_cast<s4*>(hi + row + 8) = h1;
      *reinterpret_cast<s4*>(lo + row) = l0;
      *reinterpret_cast<s4*>(lo + row + 8) = l1;
    }
    if (isk) {
      // columns: channel 8*oc+m, tokens at slot(8*tau) and +8
      short* th = sp(P::oTh);
      short* tl = sp(P::oTl);
      const int tb = slot(8 * tau);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        s4 h0, l0, h1, l1;
        split4(f4{y[0][m], y[1][m], y[2][m], y[3][m]}, h0, l0);
        split4(f4{y[4][m], y[5][m], y[6][m], y[7][m]}, h1, l1);
        const int row = (8 * oc + m) * P::kRowT + tb;
        *reinterpret_cast<s4*>(th + row) = h0;
        *reinterpret_cast<s4*>(th + row + 8) = h1;
        *reinterpret_cast<s4*>(tl + row) = l0;
        *reinterpret_cast<s4*>(tl + row + 8) = l1;
      }
    }
  }

  // ---- step 1 (one wave): log-decay prefix sums and gates of the chunk.
  __device__ void gates(int c0) const {
    float la = 0.f, bt = 0.f;
    if (c0 + lane < T) {
      const int64_t row = (static_cast<int64_t>(t0) + c0 + lane) * a.Hv + h;
      la = fmaxf(logf(to_f32(static_cast<const Act*>(a.alpha)[row])), -80.0f);
      bt = to_f32(static_cast<const Act*>(a.beta)[row]);
    }
    float g = la;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(g, off);
      if (lane >= off) g += o;
    }
    const float gc = __shfl(g, 63);
    float* gt = fp(P::oGate);
    gt[lane] = g;
    gt[kC + lane] = bt;
    gt[2 * kC + lane] = expf(g);
    gt[3 * kC + lane] = expf(gc - g);
  }

  // ---- step 2: tile q of the 20 lower tiles (10 of K K^T, then 10 of
  // Q K^T), scaled into A (off-diagonal: (hi, lo); diagonal: fp32) and P.
  __device__ void gram_tile(int q) const {
    const bool isp = q >= 10;
    const int p = isp ? q - 10 : q;
    const int ib = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
    const int jb = p - ib * (ib + 1) / 2;
    const short* ah = sp(isp ? P::oQh : P::oKh);
    const short* al = sp(isp ? P::oQl : P::oKl);
    const short* bh = sp(P::oKh);
    const short* bl = sp(P::oKl);
    f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      const int ra = (16 * ib + lr) * P::kRowQK + 32 * sl + 8 * lg;
      const int rb = (16 * jb + lr) * P::kRowQK + 32 * sl + 8 * lg;
      acc = mma32x3(*reinterpret_cast<const s8*>(ah + ra), *reinterpret_cast<const s8*>(al + ra),
                    *reinterpret_cast<const s8*>(bh + rb), *reinterpret_cast<const s8*>(bl + rb),
                    acc);
    }
    const float* gt = fp(P::oGate);
    const int i = 16 * jb + lr;
    const float gi = gt[i];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = 16 * ib + 4 * lg + v;
      const float dec = expf(gt[r] - gi);
      if (isp) {
        const float val = i <= r ? dec * acc[v] : 0.f;
        short vh, vl;
        split(val, vh, vl);
        sp(P::oPh)[r * P::kRowT + slot(i)] = vh;
        sp(P::oPl)[r * P::kRowT + slot(i)] = vl;
      } else {
        const float val = i < r ? gt[kC + r] * dec * acc[v] : 0.f;
        if (ib == jb) {
          fp(P::oAd)[(ib * 16 + (r & 15)) * P::kAdRow + (i & 15)] = val;
        } else {
          short vh, vl;
          split(val, vh, vl);
          sp(P::oAh)[r * P::kRowT + slot(i)] = vh;
          sp(P::oAl)[r * P::kRowT + slot(i)] = vl;
        }
      }
    }
  }

  // ---- step 3 (16 lanes of wave b): column c of X_bb = (I + A_bb)^{-1} by
  // forward substitution; stored as (hi, lo) in the diagonal block of A.
  __device__ void diag_inverse(int b, int c) const {
    const float* ad = fp(P::oAd) + b * 16 * P::kAdRow;
    float x[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float acc = r == c ? 1.f : 0.f;
#pragma unroll
      for (int i = 0; i < r; ++i) acc = fmaf(-ad[r * P::kAdRow + i], x[i], acc);
      x[r] = acc;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      short vh, vl;
      split(x[r], vh, vl);
      sp(P::oAh)[(16 * b + r) * P::kRowT + slot(16 * b + c)] = vh;
      sp(P::oAl)[(16 * b + r) * P::kRowT + slot(16 * b + c)] = vl;
    }
  }

  // ---- step 4: the wave's 16 value columns.  S[d] holds rows
  // 16d + 4*lg + v (key index) of S^T at column e0 + lr (value index).
  __device__ void columns(int c0, f4 (&S)[kDt], const float (&wv)[4], float bv) const {
    const float* gt = fp(P::oGate);
    // S^T as k-operand pairs of 16x16x32 MFMAs
    s8 sbh[kSl], sbl[kSl];
#pragma unroll
    for (int sl = 0; sl < kSl; ++sl) {
      s4 h0, l0, h1, l1;
      split4(S[2 * sl], h0, l0);
      split4(S[2 * sl + 1], h1, l1);
      sbh[sl] = cat(h0, h1);
      sbl[sl] = cat(l0, l1);
    }
    // K S0^T and Q S0^T, rows 16 tb + 4 lg + v
    f4 ks[4], qs[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      ks[tb] = f4{0.f, 0.f, 0.f, 0.f};
      qs[tb] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < kSl; ++sl) {
        const int ra = (16 * tb + lr) * P::kRowQK + 32 * sl + 8 * lg;
        ks[tb] = mma32x3(*reinterpret_cast<const s8*>(sp(P::oKh) + ra),
                         *reinterpret_cast<const s8*>(sp(P::oKl) + ra), sbh[sl], sbl[sl], ks[tb]);
        qs[tb] = mma32x3(*reinterpret_cast<const s8*>(sp(P::oQh) + ra),
                         *reinterpret_cast<const s8*>(sp(P::oQl) + ra), sbh[sl], sbl[sl], qs[tb]);
      }
    }
    // value conv at this lane's column, R = V - e^g (K S0^T)
    const int vch = 2 * a.Hk * DK + h * a.dv + e0 + lr;
    f4 R[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      float xr[7];
#pragma unroll
      for (int r = 0; r < 7; ++r) xr[r] = row1(c0 + 16 * tb + 4 * lg - 3 + r, vch);
      const f4 gam = *reinterpret_cast<const f4*>(gt + 2 * kC + 16 * tb + 4 * lg);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float y = bv;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) y = fmaf(wv[jj], xr[v + jj], y);
        y = act(y);
        if (c0 + 16 * tb + 4 * lg + v >= T) y = 0.f;
        R[tb][v] = y - gam[v] * ks[tb][v];
      }
    }
    // U_b = X_bb (b_b R_b - sum_{j<b} A_bj U_j)
    f4 U[4];
    s4 uh[4], ul[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      f4 acc = {0.f, 0.f, 0.f, 0.f};
      const int row = (16 * b + lr) * P::kRowT;
#pragma unroll
      for (int jb = 0; jb < b; ++jb) {
        const int o = row + slot(16 * jb + 4 * lg);
        acc = mma16x3(*reinterpret_cast<const s4*>(sp(P::oAh) + o),
                      *reinterpret_cast<const s4*>(sp(P::oAl) + o), uh[jb], ul[jb], acc);
      }
      const f4 bt = *reinterpret_cast<const f4*>(gt + kC + 16 * b + 4 * lg);
      s4 zh, zl;
      split4(bt * R[b] - acc, zh, zl);
      const int o = row + slot(16 * b + 4 * lg);
      U[b] = mma16x3(*reinterpret_cast<const s4*>(sp(P::oAh) + o),
                     *reinterpret_cast<const s4*>(sp(P::oAl) + o), zh, zl,
                     f4{0.f, 0.f, 0.f, 0.f});
      split4(U[b], uh[b], ul[b]);
    }
    // O = e^g (Q S0^T) + P U
    const int n = T - c0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f4 gam = *reinterpret_cast<const f4*>(gt + 2 * kC + 16 * b + 4 * lg);
      f4 o = gam * qs[b];
      const int row = (16 * b + lr) * P::kRowT;
#pragma unroll
      for (int u = 0; 2 * u <= b; ++u) {
        const int off = row + 32 * u + 8 * lg;
        o = mma32x3(*reinterpret_cast<const s8*>(sp(P::oPh) + off),
                    *reinterpret_cast<const s8*>(sp(P::oPl) + off), cat(uh[2 * u], uh[2 * u + 1]),
                    cat(ul[2 * u], ul[2 * u + 1]), o);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = 16 * b + 4 * lg + v;
        if (t < n)
          a.out[(static_cast<int64_t>(t0) + c0 + t) * a.Hv * a.dv + static_cast<int64_t>(h) * a.dv +
                e0 + lr] = o[v];
      }
    }
    // S^T <- e^{g_c} S^T + K^T diag(e^{g_c - g}) U
    s4 wh[4], wl[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const f4 gp = *reinterpret_cast<const f4*>(gt + 3 * kC + 16 * b + 4 * lg);
      split4(gp * U[b], wh[b], wl[b]);
    }
    const float ec = gt[2 * kC + kC - 1];
#pragma unroll
    for (int d = 0; d < kDt; ++d) {
      f4 acc = ec * S[d];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int off = (16 * d + lr) * P::kRowT + 32 * u + 8 * lg;
        acc = mma32x3(*reinterpret_cast<const s8*>(sp(P::oTh) + off),
                      *reinterpret_cast<const s8*>(sp(P::oTl) + off),
                      cat(wh[2 * u], wh[2 * u + 1]), cat(wl[2 * u], wl[2 * u + 1]), acc);
      }
      S[d] = acc;
    }
  }
};

template <int DK, typename Act>
__global__ void __launch_bounds__(kThreads, 1) prefill_kernel(PrefillArgs a) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  using K = Prefill<DK, Act>;
  using P = Plan<DK>;
  K k{a, lds_raw};
  k.tid = threadIdx.x;
  k.wave = k.tid >> 6;
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
  k.s = u / a.nblk / a.Hv;
  k.hk = k.h / a.G;
  k.e0 = j * kCols + k.wave * 16;

  const int t0 = a.cu[k.s], t1 = a.cu[k.s + 1];
  k.dst = a.dst[k.s];
  k.init = a.init ? a.init[k.s] : k.dst;
  if (t0 < 0 || t1 < t0 || t1 > a.total || k.dst < 0 || k.dst >= a.num_slots ||
      k.init >= a.num_slots)
    return;
  k.t0 = t0;
  k.T = t1 - t0;
  const bool cols = k.e0 < a.dv;

  // P and A planes: the blocks above the diagonal stay zero.
  for (int i = k.tid; i < 4 * P::kSq / 16; i += kThreads)
    reinterpret_cast<uint4*>(lds_raw + P::oPh)[i] = uint4{0u, 0u, 0u, 0u};

  // This thread's q / k conv channels (octet co, token octet tau) and the
  // wave's value column.
  const bool prep = k.tid < 8 * K::kNco;
  const int co = k.tid % K::kNco, tau = k.tid / K::kNco;
  float wt[8][4], bias[8];
  {
    const int oc = co >= K::kGrp ? co - K::kGrp : co;
    const int ch = (co >= K::kGrp ? a.Hk * DK : 0) + k.hk * DK + 8 * oc;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) wt[m][jj] = prep ? k.tap(ch + m, jj) : 0.f;
      bias[m] = (prep && a.bias) ? to_f32(static_cast<const Act*>(a.bias)[ch + m]) : 0.f;
    }
  }
  float wv[4], bv = 0.f;
  const int vch = 2 * a.Hk * DK + k.h * a.dv + k.e0 + k.lr;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) wv[jj] = cols ? k.tap(vch, jj) : 0.f;
  if (cols && a.bias) bv = to_f32(static_cast<const Act*>(a.bias)[vch]);

  f4 S[K::kDt];
  const int64_t head = static_cast<int64_t>(k.h) * a.dv * DK;
  const int64_t slot_elems = static_cast<int64_t>(a.Hv) * a.dv * DK;
#pragma unroll
  for (int d = 0; d < K::kDt; ++d) {
    S[d] = f4{0.f, 0.f, 0.f, 0.f};
    if (cols && k.init >= 0)
      S[d] = *reinterpret_cast<const f4*>(a.ssm + k.init * slot_elems + head +
                                         static_cast<int64_t>(k.e0 + k.lr) * DK + 16 * d +
                                         4 * k.lg);
  }

  for (int c0 = 0; c0 < k.T; c0 += kC) {
    if (prep) k.prep_qk(c0, co, tau, wt, bias);
    if (k.wave == 3) k.gates(c0);
    lds_barrier();
    for (int q = k.wave; q < 20; q += 4) k.gram_tile(q);
    lds_barrier();
    if (k.lane < 16) k.diag_inverse(k.wave, k.lane);
    lds_barrier();
    if (cols) k.columns(c0, S, wv, bv);
    lds_barrier();
  }

  if (cols) {
    float* out = a.ssm + k.dst * slot_elems + head + static_cast<int64_t>(k.e0 + k.lr) * DK;
#pragma unroll
    for (int d = 0; d < K::kDt; ++d) *reinterpret_cast<f4*>(out + 16 * d + 4 * k.lg) = S[d];
  }
}

// The destination conv window: the last W-1 inputs of the sequence (taken
// from the initial window when the sequence is shorter).  Runs after the
// main kernel, so an in-place sequence (init == dst) has read its window.
// Each thread reads its channel's rows before writing any.
template <typename Act>
__global__ void __launch_bounds__(256) prefill_conv_tail(PrefillArgs a) {
  const int s = blockIdx.y;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= a.C) return;
  const int t0 = a.cu[s], t1 = a.cu[s + 1];
  const int32_t dst = a.dst[s];
  const int32_t init = a.init ? a.init[s] : dst;
  if (t0 < 0 || t1 < t0 || t1 > a.total || dst < 0 || dst >= a.num_slots || init >= a.num_slots)
    return;
  const int T = t1 - t0, W1 = a.W - 1;
  const Act* x = static_cast<const Act*>(a.x);
  Act* conv = static_cast<Act*>(a.conv);
  Act v[3];
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    v[jj] = from_exact<Act>(0.f);
    if (jj < W1) {
      const int rho = T - W1 + jj;
      if (rho >= 0)
        v[jj] = x[(static_cast<int64_t>(t0) + rho) * a.C + c];
      else if (init >= 0)
        v[jj] = conv[(static_cast<int64_t>(init) * W1 + W1 + rho) * a.C + c];
    }
  }
#pragma unroll
  for (int jj = 0; jj < 3; ++jj)
    if (jj < W1) conv[(static_cast<int64_t>(dst) * W1 + jj) * a.C + c] = v[jj];
}

template <int DK, typename Act>
hipError_t launch_one(const PrefillArgs& a, hipStream_t st) {
  const int bytes = Plan<DK>::kBytes;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&prefill_kernel<DK, Act>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const int grid = a.N * a.Hv * a.nblk;
  hipLaunchKernelGGL((prefill_kernel<DK, Act>), dim3(grid), dim3(kThreads), bytes, st, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.W < 2) return e;
  hipLaunchKernelGGL((prefill_conv_tail<Act>), dim3((a.C + 255) / 256, a.N), dim3(256), 0, st, a);
  return hipGetLastError();
}

static_assert(Plan<128>::kBytes <= 160 * 1024, "LDS plan exceeds 160 KiB");

}  // namespace

int prefill_supported(int dk, int kda) { return !kda && (dk == 32 || dk == 64 || dk == 128); }

hipError_t launch_prefill(const PrefillArgs& a, int dk, int act_bf16, hipStream_t s) {
  if (a.N == 0) return hipSuccess;
  switch (dk) {
    case 32: return act_bf16 ? launch_one<32, bf16>(a, s) : launch_one<32, float>(a, s);
    case 64: return act_bf16 ? launch_one<64, bf16>(a, s) : launch_one<64, float>(a, s);
    case 128: return act_bf16 ? launch_one<128, bf16>(a, s) : launch_one<128, float>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gdn
