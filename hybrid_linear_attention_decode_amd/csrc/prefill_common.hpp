// prefill_common.hpp -- device pieces shared by the chunked prefill kernels
// (scalar decay: gdn_prefill.hip; per-channel decay: kda_prefill.hip):
// bf16 (hi, lo) operand splitting, the MFMA wrappers, the permuted
// contraction order of K / Q planes, raw buffer descriptors, 8-channel raw
// input rows, the per-unit addressing, and the destination conv-window copy.
#pragma once

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

typedef short s4 __attribute__((ext_vector_type(4)));
typedef short s8 __attribute__((ext_vector_type(8)));
typedef __bf16 b8 __attribute__((ext_vector_type(8)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;         // chunk length
constexpr int kThreads = 512;  // 4 producer + 4 consumer waves
constexpr int kProd = 256;     // producer threads
constexpr int kCols = 64;      // value columns per workgroup (16 per consumer wave)

typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// x ~= hi + lo with hi = bf16(x), lo = bf16(x - hi) (round to nearest even),
// two values at a time: one packed conversion per pair, and the pair's hi
// words are already the packed operand halves.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{x0, x1}, bf2));
  const f2 r = {x0 - __uint_as_float(h << 16), x1 - __uint_as_float(h & 0xffff0000u)};
  hi = h;
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf2));
}
__device__ __forceinline__ void split4(f4 x, s4& hi, s4& lo) {
  uint32_t h0, l0, h1, l1;
  split2(x[0], x[1], h0, l0);
  split2(x[2], x[3], h1, l1);
  hi = __builtin_bit_cast(s4, u2{h0, h1});
  lo = __builtin_bit_cast(s4, u2{l0, l1});
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

// ds_read_b64_tr_b16: in each group of 16 lanes, lane j receives element
// (j mod 4) of the 64-bit words read by lanes 4e + j/4, e = 0..3.  Lanes
// 4e + q reading row r0 + e, columns c0 + 4q..4q+3 thus hand lane j the
// column c0 + j of rows r0..r0+3.
__device__ __forceinline__ s4 ld_tr(const short* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s4*)(const_cast<short*>(p)));
}

// SiLU with the hardware exp2 / reciprocal.
__device__ __forceinline__ float silu(float y) {
  return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// Raw 8-channel rows: 16 bytes of bf16 or 32 bytes of fp32.
template <typename Act>
struct Row8 {
  static constexpr int kWords = sizeof(Act) == 2 ? 4 : 8;
  uint32_t w[kWords];
  __device__ __forceinline__ void load(rsrc_t r, int off) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    const u4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    w[0] = u[0], w[1] = u[1], w[2] = u[2], w[3] = u[3];
    if constexpr (kWords == 8) {
      const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
      w[4] = v[0], w[5] = v[1], w[6] = v[2], w[7] = v[3];
    }
  }
  // Channels c..c+3 and c+16..c+19 (the channels of one 16-byte storage
  // chunk of K / Q rows): off is c's byte offset.
  __device__ __forceinline__ void load_split(rsrc_t r, int off) {
    typedef uint32_t u4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u2 __attribute__((ext_vector_type(2)));
    if constexpr (kWords == 4) {
      const u2 u = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
      const u2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 32, 0, 0);
      w[0] = u[0], w[1] = u[1], w[2] = v[0], w[3] = v[1];
    } else {
      const u4 u = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
      const u4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 64, 0, 0);
      w[0] = u[0], w[1] = u[1], w[2] = u[2], w[3] = u[3];
      w[4] = v[0], w[5] = v[1], w[6] = v[2], w[7] = v[3];
    }
  }
  __device__ __forceinline__ void merge(const Row8& o) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] |= o.w[i];
  }
  __device__ __forceinline__ float get(int m) const {
    if constexpr (kWords == 4)
      return __uint_as_float((m & 1) ? (w[m >> 1] & 0xffff0000u) : (w[m >> 1] << 16));
    else
      return __uint_as_float(w[m]);
  }
};

// Bl(X Y) from X in A-operand layout (X[lr][4 lg + v]) and Y in B-operand
// layout (Y[4 lg + v][lr]) of 16x16 tiles; the result is in B layout.  N
// independent products at once, their MFMAs interleaved, each on (hi, lo)
// split operands.
template <int N>
__device__ __forceinline__ void mm_split(const f4 (&x)[N], const f4 (&y)[N], f4 (&r)[N]) {
  s4 xh[N], xl[N], yh[N], yl[N];
#pragma unroll
  for (int n = 0; n < N; ++n) {
    split4(x[n], xh[n], xl[n]);
    split4(y[n], yh[n], yl[n]);
    r[n] = f4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int n = 0; n < N; ++n) r[n] = mma16(xl[n], yh[n], r[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) r[n] = mma16(xh[n], yl[n], r[n]);
#pragma unroll
  for (int n = 0; n < N; ++n) r[n] = mma16(xh[n], yh[n], r[n]);
}

// X = (I + N)^{-1} for a strictly lower triangular 16x16 N given in both
// layouts (na[v] = N[lr][4 lg + v], nb[v] = N[4 lg + v][lr]); returns
// X[lr][4 lg + v].  N is nilpotent (N^16 = 0), so
// X = (I - N)(I + N^2)(I + N^4)(I + N^8); all factors are polynomials in N
// and commute, so X^T is built in B layout: X^T = Q2 + (N^8)^T Q2,
// Q2 = Q1 + (N^4)^T Q1, Q1 = I - N^T + (N^2)^T - N^T (N^2)^T.
__device__ __forceinline__ f4 unit_lower_inverse(const f4& na, const f4& nb, int lr, int lg) {
  f4 id;
#pragma unroll
  for (int v = 0; v < 4; ++v) id[v] = 4 * lg + v == lr ? 1.f : 0.f;
  f4 l1[2];                                   // N^2 in B and A layout
  mm_split<2>({na, nb}, {nb, na}, l1);
  f4 l2[3];                                   // N^4 (B, A), N^T (N^2)^T
  mm_split<3>({l1[1], l1[0], nb}, {l1[0], l1[1], l1[1]}, l2);
  const f4 q1 = id - na + l1[1] - l2[2];
  f4 l3[2];                                   // N^8 (B), (N^4)^T Q1
  mm_split<2>({l2[1], l2[0]}, {l2[0], q1}, l3);
  const f4 q2 = q1 + l3[1];
  f4 l4[1];
  mm_split<1>({l3[0]}, {q2}, l4);
  return q2 + l4[0];
}

// Element offset of storage slot sl of row r in a [token][d_k] bf16 plane.
// Rows of d_k = 128 (256 bytes: one pass over the 64 four-byte banks) are
// swizzled: 16-byte chunk c of row r sits at chunk c ^ f(r), f(r) =
// 4 (r & 3) + 2 ((r >> 3) & 1).  How gfx950 serves LDS reads (measured per
// lane pair with SQ_LDS_BANK_CONFLICT): a 16-byte read splits each half-wave
// into two sets of 16 lanes by the parity of lane bits 2..4, a set being
// conflict-free when its 16 chunks are distinct; an 8-byte read (the
// transposing one too) takes 32 consecutive lanes over 64 banks.  With f the
// MFMA operand reads (lane 16 g + r: row r, chunk 4 s + g) are conflict-free
// -- the rows of each set map to all the even chunks, XOR 0 or 1 -- and the
// transposing reads (rows 4 g + r / 4, chunks 4 D + r % 4) cover every
// chunk twice, their minimum.  f depends on r mod 16 only, so offsets may
// be moved by whole 16-row blocks.  Narrower rows are padded by 16 bytes.
template <int DK>
struct QkRow {
  static constexpr bool kSwz = DK == 128;
  static constexpr int kElems = kSwz ? DK : DK + 8;   // bf16 per row
  static constexpr int kChunks = DK / 8;              // 16-byte chunks per row
  __device__ __forceinline__ static int swz(int r) { return ((r & 3) << 2) | (((r >> 3) & 1) << 1); }
  __device__ __forceinline__ static int at(int r, int sl) {
    if constexpr (kSwz)
      return r * DK + (((sl >> 3) ^ swz(r)) << 3) + (sl & 7);
    else
      return r * kElems + sl;
  }
};

// What every prefill workgroup knows about its unit (sequence, value head,
// 64 value columns) and the raw-input addressing both kernels share.
template <int DK, typename Act>
struct PrefillCore {
  const PrefillArgs& a;
  unsigned char* lds;
  int tid, wave, lane, lr, lg;
  int h, hk, e0;
  int t0, T;
  int32_t init;

  __device__ short* sp(int off) const { return reinterpret_cast<short*>(lds + off); }
  __device__ float* fp(int off) const { return reinterpret_cast<float*>(lds + off); }
  // The lane id, opaque to the compiler: offsets derived from it inside a
  // phase are recomputed there (a few VALU ops) instead of being hoisted
  // out of the chunk loop and kept live (or spilled) across all phases.
  __device__ __forceinline__ static int opaque(int v) {
    asm volatile("" : "+v"(v));
    return v;
  }
  __device__ __forceinline__ int lane_now() const { return opaque(lane); }

  // Raw input rows for chunk c0: a descriptor over rows b0.. of the
  // sequence (b0 = c0 - 8, or 0), ending at the sequence's last row (empty
  // when b0 lies past it), so rows past the end (and before row 0) read zero.  The initial conv window
  // (W-1 rows before row 0) has its own descriptor, empty when the sequence
  // starts from zeros.
  __device__ __forceinline__ int chunk_base(int c0) const { return c0 >= 8 ? c0 - 8 : 0; }
  __device__ __forceinline__ rsrc_t x_rows(int c0) const {
    const int b0 = chunk_base(c0);
    const int64_t rowb = static_cast<int64_t>(a.C) * sizeof(Act);
    const int64_t n = T - b0 < 80 ? (T > b0 ? T - b0 : 0) : 80;
    return make_rsrc(static_cast<const Act*>(a.x) + (static_cast<int64_t>(t0) + b0) * a.C,
                     static_cast<uint32_t>(n * rowb));
  }
  __device__ __forceinline__ rsrc_t win_rows() const {
    const int W1 = a.W - 1;
    const bool on = init >= 0 && W1 > 0;
    return make_rsrc(on ? static_cast<const Act*>(a.conv) + static_cast<int64_t>(init) * W1 * a.C
                        : a.x,
                     on ? static_cast<uint32_t>(W1 * a.C * sizeof(Act)) : 0u);
  }
  // Row rho (0 <= rho < T, uniform) of the sequence alone: channel ch at
  // byte offset ch * sizeof(Act).
  __device__ __forceinline__ rsrc_t seq_row(int rho) const {
    return make_rsrc(static_cast<const Act*>(a.x) + (static_cast<int64_t>(t0) + rho) * a.C,
                     static_cast<uint32_t>(a.C * sizeof(Act)));
  }
  // Byte offsets of row rho at channel ch in the two descriptors.
  __device__ __forceinline__ int x_off(int c0, int rho, int ch) const {
    return (rho - chunk_base(c0)) * a.C * static_cast<int>(sizeof(Act)) +
           ch * static_cast<int>(sizeof(Act));
  }
  __device__ __forceinline__ int win_off(int rho, int ch) const {
    return (a.W - 1 + rho) * a.C * static_cast<int>(sizeof(Act)) +
           ch * static_cast<int>(sizeof(Act));
  }
  // Conv tap jj (0..3, the last on the current token) of channel ch; taps of
  // a narrower conv are left-padded with zeros.
  __device__ __forceinline__ float tap(int ch, int jj) const {
    const int lead = 4 - a.W;
    return jj >= lead ? to_f32(static_cast<const Act*>(a.w)[static_cast<int64_t>(ch) * a.W + jj - lead])
                      : 0.f;
  }
  __device__ __forceinline__ float act(float y) const { return a.silu ? silu(y) : y; }
};

// The using-declarations a kernel struct deriving from PrefillCore needs.
#define GDN_PREFILL_CORE(DK, Act)                                                         \
  using Core = PrefillCore<DK, Act>;                                                      \
  using Core::a; using Core::lds; using Core::tid; using Core::wave; using Core::lane;    \
  using Core::lr; using Core::lg; using Core::h; using Core::hk; using Core::e0;          \
  using Core::t0; using Core::T; using Core::init; using Core::sp; using Core::fp;        \
  using Core::opaque; using Core::lane_now; using Core::chunk_base; using Core::x_rows;  \
  using Core::win_rows; using Core::x_off; using Core::win_off; using Core::tap;          \
  using Core::seq_row;                                                                   \
  using Core::act

// Pool slot of checkpoint k = tok / every - 1 of sequence s, taken after its
// first tok tokens, or -1 when there is none (no checkpoint table, tok past
// the sequence or not a multiple of the interval, k past the table's
// columns, an entry outside the pool).
__device__ __forceinline__ int32_t ckpt_slot(const PrefillArgs& a, int s, int tok, int T) {
  if (!a.ckpt || tok > T || tok % a.ckpt_every) return -1;
  const int k = tok / a.ckpt_every - 1;
  if (k < 0 || k >= a.ckpt_per_seq) return -1;
  const int32_t sl = a.ckpt[static_cast<int64_t>(s) * a.ckpt_per_seq + k];
  return (sl < 0 || sl >= a.num_slots) ? -1 : sl;
}

// Conv windows written after the main kernel (the per-channel-decay
// prefill's; the scalar-decay kernels write theirs themselves).  z = 0: the
// destination's, the last W-1 inputs of the sequence (taken from the initial
// window when the sequence is shorter; the main kernel has read an in-place
// sequence's old window by now, and each thread reads its channel's rows
// before writing any).  z = k + 1: checkpoint k's, the W-1 inputs before its
// token.
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
  int end = T;              // the window ends before row `end`
  int32_t to = dst;
  if (blockIdx.z > 0) {
    end = static_cast<int>(blockIdx.z) * a.ckpt_every;
    to = ckpt_slot(a, s, end, T);
    if (to < 0) return;
  }
  const Act* x = static_cast<const Act*>(a.x);
  Act* conv = static_cast<Act*>(a.conv);
  Act v[3];
#pragma unroll
  for (int jj = 0; jj < 3; ++jj) {
    v[jj] = from_exact<Act>(0.f);
    if (jj < W1) {
      const int rho = end - W1 + jj;
      if (rho >= 0)
        v[jj] = x[(static_cast<int64_t>(t0) + rho) * a.C + c];
      else if (init >= 0)
        v[jj] = conv[(static_cast<int64_t>(init) * W1 + W1 + rho) * a.C + c];
    }
  }
#pragma unroll
  for (int jj = 0; jj < 3; ++jj)
    if (jj < W1) conv[(static_cast<int64_t>(to) * W1 + jj) * a.C + c] = v[jj];
}

// Grid of prefill_conv_tail: channel blocks x sequences x (1 + checkpoints).
inline dim3 conv_tail_grid(const PrefillArgs& a) {
  return dim3((a.C + 255) / 256, a.N, 1 + (a.ckpt ? a.ckpt_per_seq : 0));
}

}  // namespace
}  // namespace gdn
