// gdn_decode.hip -- fused decode step for Gated DeltaNet / KDA on gfx950.
//
// One workgroup owns one (request b, key head kh): the q and k conv channels
// of kh, the v channels of its G = H_v/H_k value heads and the G*d_v state
// rows of those heads.  It is therefore the only reader and writer of every
// conv-window channel it touches, and no cross-workgroup ordering exists.
//
// Per token (state held in registers across all T tokens of the call):
//   conv update + SiLU of the group's channels  -> LDS
//   q/k squared norms and q.k (each wave, wave64 butterfly sums)
//   per state row i (value index), per lane 16 contiguous key columns:
//     s' = s * a_j                    (a_j = alpha, or alpha_j for KDA)
//     pk = sum_j s'_j k^_j,  pq = sum_j s'_j q^_j     (8-lane DPP sums)
//     u  = beta (v_i - pk);  o_i = pq + u (k^.q^);  s = s' + u k^_j
// which is S_t = alpha S (I - beta k k^T) + beta v k^T, o_t = S_t q_t with
// o_t computed from S' q^ + u (k^.q^) (equal to S_t q^ by definition).
//
// Memory: a state row (d_k fp32) is split over LPR lanes x CPL 16-byte
// chunks, with chunk n*LPR + lc in lane lc of the row group, so every load
// instruction of a wave covers whole 128-byte lines (8 rows x 128 B for
// d_k >= 32).  Loads and stores of the state are non-temporal: each slot is
// touched once per call.
//
// Bitwise contract: the in-place path (spec_ssm == nullptr) and the snapshot
// path run the same instantiation with the same per-token instruction
// sequence (built with -ffp-contract=off, explicit fmaf), so a draft of T
// tokens followed by a commit of L equals an in-place decode of L tokens bit
// for bit.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {

namespace {

constexpr int kMaxW1 = 3;   // conv_width <= 4
constexpr int kMaxCPT = 2;  // conv channels per thread

template <int DK>
struct RowMap {
  static constexpr int LPR = DK >= 32 ? 8 : 4;   // lanes per state row
  static constexpr int CPL = DK / (4 * LPR);     // 16-byte chunks per lane
  static constexpr int RPP = 64 / LPR;           // rows per wave per pass
};

template <int DK, int NR, typename Act, bool KDA>
__global__ void __launch_bounds__(512) decode_kernel(const DecodeArgs a) {
  using M = RowMap<DK>;
  constexpr int LPR = M::LPR, CPL = M::CPL, RPP = M::RPP;
  constexpr int RPW = NR * RPP;

  const int kh = blockIdx.x;
  const int b = blockIdx.y;
  const int32_t slot = a.idx[b];
  if (slot < 0 || static_cast<int64_t>(slot) >= a.num_slots) return;  // whole group

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane / LPR;
  const int lc = lane % LPR;
  const int NT = blockDim.x;
  const int dv = a.dv;
  const int G = a.G;
  const int R = G * dv;           // state rows of the group
  const int Cg = 2 * DK + R;      // conv channels of the group
  const int W = a.W;
  const int W1 = W - 1;
  const int C = a.C;
  const int T = a.T;
  const bool spec = a.spec_ssm != nullptr;

  extern __shared__ float act[];  // [2][Cg], double buffered over tokens

  const Act* xg = static_cast<const Act*>(a.x);
  const Act* wg = static_cast<const Act*>(a.w);
  const Act* bg = static_cast<const Act*>(a.bias);
  Act* convg = static_cast<Act*>(a.conv);
  const Act* alg = static_cast<const Act*>(a.alpha);
  const Act* beg = static_cast<const Act*>(a.beta);

  // ---- conv channels of this thread: taps, bias and window, issued first and
  // without branches (clamped indices, selects after the loads) so that all
  // of them are in flight together.  Taps and window are right-aligned in a
  // 4-tap frame: tap 3 multiplies the current input, missing older taps of a
  // narrower conv are zero, so the shift below is the same for every width.
  int64_t gch[kMaxCPT];
  bool has[kMaxCPT];
  float wt[kMaxCPT][kMaxW1 + 1];
  float bias[kMaxCPT];
  float win[kMaxCPT][kMaxW1];
  const int lead = kMaxW1 - W1;  // zero taps in front of a narrower conv
#pragma unroll
  for (int m = 0; m < kMaxCPT; ++m) {
    const int c0 = tid + m * NT;
    has[m] = c0 < Cg;
    const int c = has[m] ? c0 : 0;
    int64_t g;
    if (c < DK)
      g = static_cast<int64_t>(kh) * DK + c;
    else if (c < 2 * DK)
      g = static_cast<int64_t>(a.Hk) * DK + static_cast<int64_t>(kh) * DK + (c - DK);
    else
      g = 2 * static_cast<int64_t>(a.Hk) * DK + static_cast<int64_t>(kh) * R + (c - 2 * DK);
    gch[m] = g;
    Act raw_w[kMaxW1 + 1];
#pragma unroll
    for (int j = 0; j <= kMaxW1; ++j) raw_w[j] = wg[g * W + (j >= lead ? j - lead : 0)];
    const Act raw_b = bg ? bg[g] : wg[g * W];
    Act raw_s[kMaxW1];
    if (W1 > 0) {
#pragma unroll
      for (int j = 0; j < kMaxW1; ++j)
        raw_s[j] = convg[(static_cast<int64_t>(slot) * W1 + (j >= lead ? j - lead : 0)) * C + g];
    }
#pragma unroll
    for (int j = 0; j <= kMaxW1; ++j) wt[m][j] = j >= lead ? to_f32(raw_w[j]) : 0.f;
    bias[m] = bg ? to_f32(raw_b) : 0.f;
#pragma unroll
    for (int j = 0; j < kMaxW1; ++j) win[m][j] = (W1 > 0 && j >= lead) ? to_f32(raw_s[j]) : 0.f;
  }

  // ---- state rows of this lane (NR rows x CPL chunks of 4 floats)
  const int64_t slot_elems = static_cast<int64_t>(a.Hv) * dv * DK;
  const int64_t grp_off = static_cast<int64_t>(kh) * R * DK;
  const float* src = a.ssm + static_cast<int64_t>(slot) * slot_elems + grp_off;
  f4 s[NR][CPL];
  int rowp[NR];
#pragma unroll
  for (int p = 0; p < NR; ++p) {
    rowp[p] = wave * RPW + p * RPP + lr;
#pragma unroll
    for (int n = 0; n < CPL; ++n)
      s[p][n] = ld_stream(src + static_cast<int64_t>(rowp[p]) * DK + 4 * (n * LPR + lc));
  }

  for (int t = 0; t < T; ++t) {
    float* buf = act + (t & 1) * Cg;
    const int64_t tok = static_cast<int64_t>(b) * T + t;

    // ---- D1: conv update + activation of the group's channels
#pragma unroll
    for (int m = 0; m < kMaxCPT; ++m) {
      if (!has[m]) continue;
      const float xv = to_f32(xg[tok * C + gch[m]]);
      float y = bias[m];
#pragma unroll
      for (int j = 0; j < kMaxW1; ++j) y = fmaf(wt[m][j], win[m][j], y);
      y = fmaf(wt[m][kMaxW1], xv, y);
#pragma unroll
      for (int j = 0; j + 1 < kMaxW1; ++j) win[m][j] = j >= lead ? win[m][j + 1] : 0.f;
      win[m][kMaxW1 - 1] = xv;
      if (a.silu) y = y / (1.0f + expf(-y));
      buf[tid + m * NT] = y;
      if (spec) {
        Act* sc = static_cast<Act*>(a.spec_conv) +
                  (static_cast<int64_t>(b) * a.t_max + t) * W1 * C + gch[m];
#pragma unroll
        for (int j = 0; j < kMaxW1; ++j)
          if (j >= lead) sc[static_cast<int64_t>(j - lead) * C] = from_exact<Act>(win[m][j]);
      }
    }
    __syncthreads();

    // ---- D2: norms of q and k of the key head, and q.k (redundant per wave)
    float sq = 0.f, sk = 0.f, sqk = 0.f;
    for (int j = lane; j < DK; j += 64) {
      const float qv = buf[j];
      const float kv = buf[DK + j];
      sq = fmaf(qv, qv, sq);
      sk = fmaf(kv, kv, sk);
      sqk = fmaf(qv, kv, sqk);
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    sqk = wave_sum(sqk);
    const float rq = a.l2norm ? rsqrtf(sq + a.eps) : 1.0f;
    const float rk = a.l2norm ? rsqrtf(sk + a.eps) : 1.0f;
    const float qs = rq * a.q_scale;
    const float kq = sqk * rk * qs;  // k^ . q^

    f4 kk[CPL], qq[CPL];
#pragma unroll
    for (int n = 0; n < CPL; ++n) {
      const int col = 4 * (n * LPR + lc);
      kk[n] = *reinterpret_cast<const f4*>(buf + DK + col) * rk;
      qq[n] = *reinterpret_cast<const f4*>(buf + col) * qs;
    }

    // ---- D3 / D4: the gated delta rule on this lane's rows
#pragma unroll
    for (int p = 0; p < NR; ++p) {
      const int r = rowp[p];
      const int g = r / dv;
      const int i = r - g * dv;
      const int h = kh * G + g;
      const int64_t th = tok * a.Hv + h;
      const float be = to_f32(beg[th]);
      f4 ga[CPL];
      if constexpr (KDA) {
#pragma unroll
        for (int n = 0; n < CPL; ++n) {
          const int col = 4 * (n * LPR + lc);
          const Act* ap = alg + th * DK + col;
          ga[n] = f4{to_f32(ap[0]), to_f32(ap[1]), to_f32(ap[2]), to_f32(ap[3])};
        }
      } else {
        const float al = to_f32(alg[th]);
#pragma unroll
        for (int n = 0; n < CPL; ++n) ga[n] = f4{al, al, al, al};
      }
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
      const float u = be * (buf[2 * DK + r] - pk);
      const float o = fmaf(u, kq, pq);
#pragma unroll
      for (int n = 0; n < CPL; ++n) {
        s[p][n].x = fmaf(u, kk[n].x, s[p][n].x);
        s[p][n].y = fmaf(u, kk[n].y, s[p][n].y);
        s[p][n].z = fmaf(u, kk[n].z, s[p][n].z);
        s[p][n].w = fmaf(u, kk[n].w, s[p][n].w);
      }
      if (lc == 0) a.out[th * dv + i] = o;
    }

    if (spec) {
      float* dst = a.spec_ssm + (static_cast<int64_t>(b) * a.t_max + t) * slot_elems + grp_off;
#pragma unroll
      for (int p = 0; p < NR; ++p)
#pragma unroll
        for (int n = 0; n < CPL; ++n)
          st_stream(dst + static_cast<int64_t>(rowp[p]) * DK + 4 * (n * LPR + lc), s[p][n]);
    }
  }

  if (!spec) {
    float* dst = a.ssm + static_cast<int64_t>(slot) * slot_elems + grp_off;
#pragma unroll
    for (int p = 0; p < NR; ++p)
#pragma unroll
      for (int n = 0; n < CPL; ++n)
        st_stream(dst + static_cast<int64_t>(rowp[p]) * DK + 4 * (n * LPR + lc), s[p][n]);
#pragma unroll
    for (int m = 0; m < kMaxCPT; ++m) {
      if (!has[m]) continue;
#pragma unroll
      for (int j = 0; j < kMaxW1; ++j)
        if (j >= lead)
          convg[(static_cast<int64_t>(slot) * W1 + (j - lead)) * C + gch[m]] =
              from_exact<Act>(win[m][j]);
    }
  }
}

template <int DK, typename Act, bool KDA>
hipError_t launch_nr(const DecodeArgs& a, int nr, hipStream_t s) {
  const int R = a.G * a.dv;
  const int threads = decode_threads(DK, nr, R);
  const dim3 grid(a.Hk, a.B);
  const size_t lds = 2 * sizeof(float) * (2 * DK + R);
  switch (nr) {
    case 4:
      hipLaunchKernelGGL((decode_kernel<DK, 4, Act, KDA>), grid, dim3(threads), lds, s, a);
      break;
    case 2:
      hipLaunchKernelGGL((decode_kernel<DK, 2, Act, KDA>), grid, dim3(threads), lds, s, a);
      break;
    case 1:
      hipLaunchKernelGGL((decode_kernel<DK, 1, Act, KDA>), grid, dim3(threads), lds, s, a);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename Act, bool KDA>
hipError_t launch_dk(const DecodeArgs& a, int dk, int nr, hipStream_t s) {
  switch (dk) {
    case 16: return launch_nr<16, Act, KDA>(a, nr, s);
    case 32: return launch_nr<32, Act, KDA>(a, nr, s);
    case 64: return launch_nr<64, Act, KDA>(a, nr, s);
    case 128: return launch_nr<128, Act, KDA>(a, nr, s);
    default: return hipErrorInvalidValue;
  }
}

int rows_per_pass(int dk) { return dk >= 32 ? 8 : 16; }

}  // namespace

int decode_threads(int dk, int nr, int rows_per_group) {
  return 64 * (rows_per_group / (nr * rows_per_pass(dk)));
}

// Largest rows-per-lane count in {4, 2, 1} that tiles the group's rows into
// at most 8 waves and leaves at most two conv channels per thread.
int decode_rows_per_lane(int dk, int rows_per_group, int channels_per_group) {
  const int rpp = rows_per_pass(dk);
  for (int nr = 4; nr >= 1; nr >>= 1) {
    if (rows_per_group % (nr * rpp)) continue;
    const int waves = rows_per_group / (nr * rpp);
    if (waves < 1 || waves > 8) continue;
    if (kMaxCPT * 64 * waves < channels_per_group) continue;
    return nr;
  }
  return 0;
}

hipError_t launch_decode(const DecodeArgs& a, int dk, int act_bf16, int kda, hipStream_t s) {
  const int nr = decode_rows_per_lane(dk, a.G * a.dv, 2 * dk + a.G * a.dv);
  if (!nr) return hipErrorInvalidValue;
  if (act_bf16)
    return kda ? launch_dk<bf16, true>(a, dk, nr, s) : launch_dk<bf16, false>(a, dk, nr, s);
  return kda ? launch_dk<float, true>(a, dk, nr, s) : launch_dk<float, false>(a, dk, nr, s);
}

}  // namespace gdn
