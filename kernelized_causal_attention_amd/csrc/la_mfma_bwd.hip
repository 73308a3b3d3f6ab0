// bf16 MFMA kernels for the cumulative-sum backward (gfx950).
//
// Gradients of L = sum(dout * out) ("[Paper walkthrough] Transformers are
// RNNs", wkq9411.github.io, section 3.1: a prefix matrix for phi(Q),
// eq:gq; a suffix matrix for phi(K) and V, up to eq:gv).  The page leaves
// the denominator to autograd; by the chain rule through out = num / den,
// with g_i = dout_i / den_i and c_i = -(dout_i . out_i) / den_i:
//   grad phi(Q_i) = S_i g_i + c_i Z_i
//   grad phi(K_j) = R_j V_j + r_j,   grad V_j = R_j^T phi(K_j)
//   R_j = sum_{i>=j} phi(Q_i) g_i^T,  r_j = sum_{i>=j} c_i phi(Q_i)
// and dq = grad phi(Q) * phi'(q), dk = grad phi(K) * phi'(k).
//
// Chunked (T = 64 tokens), per chunk with prefix state (S, Z) before it and
// suffix state (R, r) after it:
//   grad phi(Q_i) = S g_i + c_i Z + sum_{j<=i in chunk} (g_i.V_j + c_i) phi(K_j)
//   grad phi(K_j) = R V_j + r + sum_{i>=j in chunk} (g_i.V_j + c_i) phi(Q_i)
//   grad V_j      = R^T phi(K_j) + sum_{i>=j in chunk} (phi(Q_i).phi(K_j)) g_i
// k_bwd_dq_mfma walks a segment forwards (S, Z carried in fp32 MFMA
// accumulators, bf16 copy of S in LDS) and, as a by-product, sums the
// segment's own (R, r) for the suffix scan; k_bwd_dkdv_mfma walks a segment
// backwards carrying (R, r).  As in the forward kernels, the chunk's score
// tiles are computed transposed so that the accumulator layout is directly
// the next MFMA's B operand (keys or queries permuted consistently on the
// other operand, read with LDS transpose loads), scores are carried as bf16
// hi + lo pairs, and Z and r are accumulated in fp32 through MFMAs against a
// ones / c operand.
#include <algorithm>

#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

using namespace mf;

constexpr int NT = kNT;
constexpr int T = kT;

// Split a masked fp32 score tile into bf16 hi + lo.
__device__ __forceinline__ void split(const f32x4_t& acc, i16x4& hi, i16x4& lo) {
  hi = pack4(acc);
  lo = pack4(acc - unpack4(hi));
}

// Each row's c as a bf16 hi + lo pair in LDS (sCh[i], sCh[T + i]), written
// once per chunk by the wave that owns the row.
__device__ __forceinline__ void put_c(uint16_t* sCh, int i, float c) {
  const short hi = bf(c);
  sCh[i] = static_cast<uint16_t>(hi);
  sCh[kT + i] = static_cast<uint16_t>(bf(c - fb(hi)));
}

// Per-wave state layout used by both kernels: X^T accumulators (X = S or R)
// for the wave's column tiles mt = w*DT + a, all row tiles n:
//   lane holds X[d = 16n + li][m = 16mt + 4g + u];
// vector accumulators (Z or r) for the wave's row tiles dt = w*DT + b:
//   lane holds x[16dt + li] (the same in all four u).
// NW waves share the state: DT = D / 16 / NW tiles each (two at D = 128 with
// four waves, one with eight).
template <int DIM, int NW = 4>
__device__ __forceinline__ void init_xt(f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)], f32x4_t (&x)[(Geo<DIM, NW>::DT)],
                                        const float* __restrict__ src, int w, int g, int li) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int a = 0; a < G::DT; ++a) {
    const int mt = w * G::DT + a;
#pragma unroll
    for (int n = 0; n < G::NTL; ++n)
#pragma unroll
      for (int u = 0; u < 4; ++u) X[a][n][u] = src ? src[(16 * n + li) * DIM + 16 * mt + 4 * g + u] : 0.f;
    const float z = src ? src[DIM * DIM + 16 * mt + li] : 0.f;
    x[a] = f32x4_t{z, z, z, z};
  }
}

// The suffix state entering segment `seg` (of P) from the later segments'
// aggregate records recs[P - 1], recs[P - 2], ..., recs[seg + 1] -- summed in
// that order from zero, as the reverse exclusive scan of the records forms
// it -- in the layout of init_xt.
template <int DIM, int NW = 4>
__device__ __forceinline__ void init_xt_suffix(f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)], f32x4_t (&x)[(Geo<DIM, NW>::DT)],
                                               const float* __restrict__ recs, int seg, int P, int w, int g,
                                               int li) {
  using G = Geo<DIM, NW>;
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
#pragma unroll
  for (int a = 0; a < G::DT; ++a) {
    x[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < G::NTL; ++n) X[a][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  for (int p = P - 1; p > seg; --p) {
    const float* rec = recs + p * E;
#pragma unroll
    for (int a = 0; a < G::DT; ++a) {
      const int mt = w * G::DT + a;
#pragma unroll
      for (int n = 0; n < G::NTL; ++n)
#pragma unroll
        for (int u = 0; u < 4; ++u) X[a][n][u] += rec[(16 * n + li) * DIM + 16 * mt + 4 * g + u];
      const float z = rec[DIM * DIM + 16 * mt + li];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[a][u] += z;
    }
  }
}

// bf16 row-major copy X[d][m] and fp32 vector x[d] into LDS.
template <int DIM, int NW = 4>
__device__ __forceinline__ void write_xt(uint16_t* sX, float* sx, const f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)],
                                         const f32x4_t (&x)[(Geo<DIM, NW>::DT)], int w, int g, int li) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int a = 0; a < G::DT; ++a) {
    const int mt = w * G::DT + a;
#pragma unroll
    for (int n = 0; n < G::NTL; ++n)
      *reinterpret_cast<i16x4*>(sX + (16 * n + li) * G::LD + 16 * mt + 4 * g) = pack4(X[a][n]);
    if (g == 0) sx[16 * mt + li] = x[a][0];
  }
}

template <int DIM, int NW = 4>
__device__ __forceinline__ void store_xt(float* __restrict__ rec, const f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)],
                                         const f32x4_t (&x)[(Geo<DIM, NW>::DT)], int w, int g, int li) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int a = 0; a < G::DT; ++a) {
    const int mt = w * G::DT + a;
#pragma unroll
    for (int n = 0; n < G::NTL; ++n)
#pragma unroll
      for (int u = 0; u < 4; ++u) rec[(16 * n + li) * DIM + 16 * mt + 4 * g + u] = X[a][n][u];
    if (g == 0) rec[DIM * DIM + 16 * mt + li] = x[a][0];
  }
}

// X^T[m][d] += sum_j A[j][m] B[j][d] over the chunk's 64 tokens, and
// x[d] += sum_j w_j B[j][d] (w = ones, or c as the hi + lo pair in sCh when
// WC; every row of that A operand is the same, so the MFMA result is
// sum_j c_j B[j][col]).
template <int DIM, bool WC, int NW = 4>
__device__ __forceinline__ void outer_update(f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)], f32x4_t (&x)[(Geo<DIM, NW>::DT)],
                                             const uint16_t* sA, const uint16_t* sB, const uint16_t* sCh, int w,
                                             int g, int li) {
  using G = Geo<DIM, NW>;
  const short one = 0x3f80;
  const i16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int s = 0; s < T / 32; ++s) {
    const int jr = 32 * s + 8 * g + li / 4;
    const int cc = 4 * (li % 4);
    i16x8 chi = ones, clo = ones;
    if (WC) {
      chi = lds8(sCh + 32 * s + 8 * g);
      clo = lds8(sCh + T + 32 * s + 8 * g);
    }
    i16x8 aop[G::DT];
#pragma unroll
    for (int a = 0; a < G::DT; ++a) {
      const int mt = w * G::DT + a;
      aop[a] = cat(lds_tr(sA + jr * G::LD + 16 * mt + cc), lds_tr(sA + (jr + 4) * G::LD + 16 * mt + cc));
    }
#pragma unroll
    for (int n = 0; n < G::NTL; ++n) {
      const i16x8 b = cat(lds_tr(sB + jr * G::LD + 16 * n + cc), lds_tr(sB + (jr + 4) * G::LD + 16 * n + cc));
#pragma unroll
      for (int a = 0; a < G::DT; ++a) X[a][n] = mfma(aop[a], b, X[a][n]);
      if (n / G::DT == w) {
        const int b_ = n % G::DT;
        x[b_] = mfma(chi, b, x[b_]);
        if (WC) x[b_] = mfma(clo, b, x[b_]);
      }
    }
  }
}

// Variants of the helpers above for the forward sweep, which writes
// phi = mu + E (mu per feature, chosen per segment: mu_rule) and keeps the
// prefix state split as
//   S = mu U^T + S',  Z = n mu + Z'.
// The split is exact for any U and n; it pays when S' and Z' are small, i.e.
// when U and n carry the mu direction of S and Z.  Within the sweep the
// kernel keeps U = sum_j V_j, n = number of tokens, S' = sum_j E(K_j) V_j^T,
// Z' = sum_j E(K_j); for a carried-in state (S, Z) it takes the least-squares
// U = sum_d mu_d S[d][:] / smu2 and n = sum_d mu_d Z[d] / smu2 (smu2 = mu.mu;
// for a state built from tokens these leave S', Z' no larger than the token
// sums do, and they need nothing but S and Z; with mu = 0, U = 0 and n = 0).
// y holds, for the wave's column tiles, a vector over m in the X^T
// accumulator layout: lane holds y[16mt + 4g + u].
template <int DIM, int NW = 4>
__device__ __forceinline__ float init_split(f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)], f32x4_t (&x)[(Geo<DIM, NW>::DT)],
                                            f32x4_t (&y)[(Geo<DIM, NW>::DT)], const float* __restrict__ rec,
                                            const float* sMuF, float smu2, int w, int g, int li) {
  using G = Geo<DIM, NW>;
  const float inv = smu2 > 0.f ? 1.f / smu2 : 0.f;
  // n = mu.Z / mu.mu: every wave sums all D entries (lane l reads Z[l],
  // Z[l + 64])
  float n = 0.f;
  if (rec) {
#pragma unroll
    for (int d0 = 0; d0 < DIM; d0 += 64) n += sMuF[d0 + (threadIdx.x & 63)] * rec[DIM * DIM + d0 + (threadIdx.x & 63)];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) n += __shfl_xor(n, off, 64);
    n *= inv;
  }
  float mud[G::NTL];  // mu of this lane's rows d = 16 n_ + li
#pragma unroll
  for (int n_ = 0; n_ < G::NTL; ++n_) mud[n_] = sMuF[16 * n_ + li];
#pragma unroll
  for (int a = 0; a < G::DT; ++a) {
    const int mt = w * G::DT + a;
#pragma unroll
    for (int n_ = 0; n_ < G::NTL; ++n_)
#pragma unroll
      for (int u = 0; u < 4; ++u) X[a][n_][u] = rec ? rec[(16 * n_ + li) * DIM + 16 * mt + 4 * g + u] : 0.f;
    // U[m] = sum_d mu_d S[d][m] / mu.mu over d = 16 n_ + li: in-lane over n_,
    // then over the 16 li
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float s_ = 0.f;
#pragma unroll
      for (int n_ = 0; n_ < G::NTL; ++n_) s_ += mud[n_] * X[a][n_][u];
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) s_ += __shfl_xor(s_, off, 64);
      y[a][u] = s_ * inv;
#pragma unroll
      for (int n_ = 0; n_ < G::NTL; ++n_) X[a][n_][u] -= mud[n_] * y[a][u];
    }
    const float z = rec ? rec[DIM * DIM + 16 * mt + li] - sMuF[16 * mt + li] * n : 0.f;
    x[a] = f32x4_t{z, z, z, z};
  }
  return n;
}

// For every lane: mu.mu over the DIM features, and whether every mu is 1.
template <int DIM>
__device__ __forceinline__ float mu_sq_sum(const float* sMuF, bool* all_one) {
  float m = 0.f, off1 = 0.f;
#pragma unroll
  for (int d0 = 0; d0 < DIM; d0 += 64) {
    const float mu = sMuF[d0 + (threadIdx.x & 63)];
    m += mu * mu;
    off1 += mu != 1.f ? 1.f : 0.f;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    m += __shfl_xor(m, off, 64);
    off1 += __shfl_xor(off1, off, 64);
  }
  *all_one = off1 == 0.f;
  return m;
}

template <int DIM, int NW = 4>
__device__ __forceinline__ void write_y(float* sy, const f32x4_t (&y)[(Geo<DIM, NW>::DT)], int w, int g, int li) {
#pragma unroll
  for (int a = 0; a < Geo<DIM, NW>::DT; ++a)
    if (li == 0) *reinterpret_cast<f32x4_t*>(sy + 16 * (w * Geo<DIM, NW>::DT + a) + 4 * g) = y[a];
}

// outer_update plus y[m] += sum_j A[j][m] (column sums of the A side).
template <int DIM, bool WC, int NW = 4>
__device__ __forceinline__ void outer_update_y(f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)], f32x4_t (&x)[(Geo<DIM, NW>::DT)],
                                               f32x4_t (&y)[(Geo<DIM, NW>::DT)], const uint16_t* sA, const uint16_t* sB,
                                               const uint16_t* sCh, int w, int g, int li) {
  using G = Geo<DIM, NW>;
  const short one = 0x3f80;
  const i16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int s = 0; s < T / 32; ++s) {
    const int jr = 32 * s + 8 * g + li / 4;
    const int cc = 4 * (li % 4);
    i16x8 chi = ones, clo = ones;
    if (WC) {
      chi = lds8(sCh + 32 * s + 8 * g);
      clo = lds8(sCh + T + 32 * s + 8 * g);
    }
    i16x8 aop[G::DT];
#pragma unroll
    for (int a = 0; a < G::DT; ++a) {
      const int mt = w * G::DT + a;
      aop[a] = cat(lds_tr(sA + jr * G::LD + 16 * mt + cc), lds_tr(sA + (jr + 4) * G::LD + 16 * mt + cc));
      y[a] = mfma(aop[a], ones, y[a]);
    }
#pragma unroll
    for (int n = 0; n < G::NTL; ++n) {
      const i16x8 b = cat(lds_tr(sB + jr * G::LD + 16 * n + cc), lds_tr(sB + (jr + 4) * G::LD + 16 * n + cc));
#pragma unroll
      for (int a = 0; a < G::DT; ++a) X[a][n] = mfma(aop[a], b, X[a][n]);
      if (n / G::DT == w) {
        const int b_ = n % G::DT;
        x[b_] = mfma(chi, b, x[b_]);
        if (WC) x[b_] = mfma(clo, b, x[b_]);
      }
    }
  }
}

// Suffix record (R, r) from R = R' + mu G^T, r = r' + C mu.
template <int DIM, int NW = 4>
__device__ __forceinline__ void store_r(float* __restrict__ rec, const f32x4_t (&X)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)],
                                        const f32x4_t (&x)[(Geo<DIM, NW>::DT)], const f32x4_t (&y)[(Geo<DIM, NW>::DT)], float C,
                                        const float* sMuF, int w, int g, int li) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int a = 0; a < G::DT; ++a) {
    const int mt = w * G::DT + a;
#pragma unroll
    for (int n = 0; n < G::NTL; ++n) {
      const float mu = sMuF[16 * n + li];
#pragma unroll
      for (int u = 0; u < 4; ++u) rec[(16 * n + li) * DIM + 16 * mt + 4 * g + u] = X[a][n][u] + mu * y[a][u];
    }
    if (g == 0) rec[DIM * DIM + 16 * mt + li] = x[a][0] + sMuF[16 * mt + li] * C;
  }
}

// ---------------------------------------------------------------------------
// Forward sweep: dq, the per-row c and den for the reverse sweep, and the
// segment's (R, r) aggregate when r_agg != null.
//
// grad phi(Q_i) = sum_{j<=i} phi(K_j) b_ij with b_ij = g_i.V_j + c_i, and
// sum_{j<=i} A_ij b_ij = 0 exactly (that is what out_i is): where phi(K) ~ 1
// the gradient is what is left after that ones direction cancels, a few
// times smaller than its terms.  Rounding phi(K), S or b to bf16 puts an
// error into that direction which the cancellation then amplifies, so this
// kernel writes phi = mu + E, with mu per feature (the segment's mean phi of
// its first chunk of keys, or 1 where that is close to 1: mu_rule) and E
// carried as bf16, and keeps every mu-direction term in fp32:
//   grad phi(Q_i) = beta_i mu + S' g_i + c_i Z' + sum_{j<=i in chunk} E_j b_ij
//   beta_i = sum_{j<=i} b_ij = g_i.U + n_i c_i + sum_{j in chunk} g_i.V_j
// with (S', Z', U) the state before the chunk (split as above), n_i the
// number of keys j <= i, and g_i = bf16(dout_i / den_i).  The same split of
// phi(Q_i) = mu + E_i gives the scores and the denominator in fp32 from
// bf16 E's (smu2 = mu.mu):
//   A_ij = smu2 + mu.E_i + mu.E_j + E_i.E_j
//   den_i = sum_{j in chunk} A_ij + n0 (smu2 + mu.E_i) + sum_d (mu + E_i) Z'
// and c_i = -(g_i . num_i) / den_i from the same pieces:
//   g_i . num_i = sum_j A_ij (g_i.V_j) + (smu2 + mu.E_i)(g_i.U)
//                 + sum_d (mu + E_i)[d] (S' g_i)[d].
// With the aggregate fused (D = 64) the query, g and c tiles are
// double-buffered so that the (R, r) aggregate of a chunk is summed after
// the chunk's last barrier: two barriers per chunk (three with eight waves,
// whose pairs exchange half sums of the c numerator).  R and r are accumulated the same way, R = mu G^T + sum_i E_i g_i^T
// and r = C mu + sum_i c_i E_i with G = sum_i g_i, C = sum_i c_i.
// ---------------------------------------------------------------------------
// FUSED_R: the (R, r) aggregate is summed here (D = 64).  At D = 128 the
// second fp32 128 x 128 state costs each of the eight waves 40 more
// registers than the two waves per SIMD leave (the fused variant spilled
// and ran 0.555 ms against 0.495 for the sweep and the separate pass on
// B=1 H=16 N=65536), and k_bwd_ragg_mfma sums the aggregate in a pass of
// its own.
// The sweep for one query row tile RW of the chunk: every branch on the
// row tile (the triangle of key tiles) resolves at compile time, and the
// chunk body becomes one stretch of code to schedule (the dq sweep is
// bound by its instruction issue; 162 -> 153 us at B=8 H=16 N=8192 D=64).
// MU1: every mu of the segment is 1 (the usual case: centred inputs), and
// the mu terms are compile-time constants; otherwise they come from LDS
// (dq_decide_mu ran first in either case).
// Waves per workgroup of the two sweeps.  D = 64: four, two workgroups per
// CU.  D = 128: with four waves each wave held two 16-column slabs of the
// fp32 128 x 128 state besides its chunk work (~420 registers: one wave per
// SIMD, nothing to hide its waits), so the sweeps run eight waves in one
// workgroup per CU: every wave owns one state slab, and the two waves of a
// pair take the same 16 rows of the chunk and half of the output columns
// each (both form the rows' scores, den and c).
template <int DIM>
constexpr int kBwdWaves = DIM == 128 ? 8 : 4;

// LDS of the dq sweep (byte offsets): E(K), V and E(Q) tiles (E(Q) twice and
// the g tile twice when the (R, r) aggregate is fused, so that it is summed
// after the chunk's last barrier), bf16 S', fp32 Z' and U, four floats of
// c sums, with eight waves the pair's partial dot products (2 x T floats),
// c hi/lo pairs (two buffers of 2T), per-wave output staging (16 rows of the
// wave's SC columns), and mu as fp32 and bf16.
template <int DIM>
struct DqLds {
  static constexpr int NW = kBwdWaves<DIM>, LD = DIM + kLdsPad;
  static constexpr int NQ = DIM == 64 ? 2 : 1, NG = DIM == 64 ? 2 : 0;  // E(Q), g buffers
  static constexpr int SC = 4 * DIM / NW;                               // output columns per wave
  static constexpr int TILE = T * LD * 2;
  static constexpr int KE = 0, V = TILE, QE = 2 * TILE, G = QE + NQ * TILE, S = G + NG * TILE;
  static constexpr int Z = S + DIM * LD * 2, U = Z + DIM * 4, RED = U + DIM * 4, DOT = RED + 4 * 4;
  static constexpr int CH = DOT + (NW == 8 ? 2 * T * 4 : 0), STAGE = CH + 4 * T * 2;
  static constexpr int MUF = STAGE + NW * 16 * (SC + kLdsPad) * 2, MUB = MUF + DIM * 4, BYTES = MUB + DIM * 2;
  static_assert(Z % 16 == 0 && DOT % 16 == 0 && STAGE % 16 == 0 && MUF % 16 == 0, "16-byte LDS accesses");
};

// Where the dq sweep keeps mu in LDS (the layout above).
template <int DIM>
__device__ __forceinline__ float* dq_mu_lds(uint16_t* smem) {
  return reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(smem) + DqLds<DIM>::MUF);
}

// The split constant mu of one segment's dq sweep into LDS (fp32 and bf16):
// decide_mu over the segment's first chunk of keys (causal), or mu_rule on
// the mean phi(K) of the carried totals, Z / N (non-causal).  Returns whether
// every mu is 1.  Ends with a barrier.
template <int DIM, bool CAUSAL>
__device__ __forceinline__ bool dq_decide_mu(const bf16_t* __restrict__ k, const float* __restrict__ carry_s,
                                              int64_t N, int P, int seg_len, int64_t bh, int seg) {
  constexpr int NW = kBwdWaves<DIM>;
  using G = Geo<DIM, NW>;
  extern __shared__ __align__(16) uint16_t smem[];
  float* sMuF = dq_mu_lds<DIM>(smem);
  uint16_t* sMuB = reinterpret_cast<uint16_t*>(sMuF + DIM);
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  if constexpr (CAUSAL) {
    i32x4 kraw[G::PC];
    bload_tile<DIM, NW>(kraw, make_rsrc(k + bh * N * DIM, N * DIM * 2), static_cast<int>(r0 * DIM * 2));
    store_tile_e<DIM, NW>(smem, kraw);  // the E(K) tile's place; the sweep overwrites it
    __syncthreads();
    decide_mu<DIM, G::LD>(smem, static_cast<int>(min(static_cast<int64_t>(T), r1 - r0)), sMuF, sMuB);
  } else if (threadIdx.x < DIM) {
    constexpr int64_t ER = static_cast<int64_t>(DIM) * DIM + DIM;
    const float* cs = carry_s ? carry_s + bh * ER : nullptr;
    const float mu = cs ? mu_rule(cs[DIM * DIM + threadIdx.x] / static_cast<float>(N)) : 1.f;
    sMuF[threadIdx.x] = mu;
    sMuB[threadIdx.x] = static_cast<uint16_t>(bf(mu));
  }
  __syncthreads();
  bool all_one = false;
  mu_sq_sum<DIM>(sMuF, &all_one);
  return all_one;
}

template <int DIM, bool CAUSAL, bool FUSED_R, int RW, int H, bool MU1>
__device__ __forceinline__ void dq_body(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                        const bf16_t* __restrict__ dout, const float* __restrict__ carry_s,
                                        bf16_t* __restrict__ dq, float* __restrict__ r_agg, float* __restrict__ c_out,
                                        float* __restrict__ den_out, int64_t N, int P, int seg_len, int64_t bh,
                                        int seg) {
  using L = DqLds<DIM>;
  constexpr int NW = L::NW, SC = L::SC;
  using G = Geo<DIM, NW>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  // this wave's output column tiles NB .. NB + NH - 1: all of them with four
  // waves, half H of them with eight
  constexpr int NH = SC / 16, NB = H * NH;
  static_assert(!(FUSED_R && NW != 4), "the fused aggregate runs with four waves");
  extern __shared__ __align__(16) uint16_t smem[];
  unsigned char* lds = reinterpret_cast<unsigned char*>(smem);
  uint16_t* sKe = reinterpret_cast<uint16_t*>(lds + L::KE);   // E(K) chunk tile
  uint16_t* sV = reinterpret_cast<uint16_t*>(lds + L::V);
  uint16_t* sQe2 = reinterpret_cast<uint16_t*>(lds + L::QE);  // E(Q), NQ buffers
  uint16_t* sG2 = reinterpret_cast<uint16_t*>(lds + L::G);    // g, NG buffers
  uint16_t* sS = reinterpret_cast<uint16_t*>(lds + L::S);     // bf16 S'
  float* sZ = reinterpret_cast<float*>(lds + L::Z);           // Z'
  float* sU = reinterpret_cast<float*>(lds + L::U);           // U
  float* sRed = reinterpret_cast<float*>(lds + L::RED);       // 4 floats: per-wave sums of c
  float* sDot = reinterpret_cast<float*>(lds + L::DOT);       // eight waves: the halves' dots
  uint16_t* sCh2 = reinterpret_cast<uint16_t*>(lds + L::CH);  // c hi/lo, two buffers of 2T
  uint16_t* sStage = reinterpret_cast<uint16_t*>(lds + L::STAGE);  // per-wave dq staging
  const float* sMuF = reinterpret_cast<const float*>(lds + L::MUF);  // the split constant mu (dq_decide_mu)
  const uint16_t* sMuB = reinterpret_cast<const uint16_t*>(lds + L::MUB);  // and as bf16
  (void)sDot;

  // w is made wave-uniform (an SGPR) so that branches on it are scalar: an
  // MFMA under an EXEC-masked branch still writes every lane.
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int rw = RW;  // query row tile (chosen by the calling kernel)
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t ER = static_cast<int64_t>(DIM) * DIM + DIM;  // S, Z (or R, r) record
  const float* cs = carry_s ? (CAUSAL ? carry_s + (bh * P + seg) * ER : carry_s + bh * ER) : nullptr;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               rg = make_rsrc(dout + hoff, hbytes), rdq = make_rsrc(dq + hoff, hbytes);
  float* ch = c_out + bh * N;
  float* dh = den_out + bh * N;
  const bool want_r = FUSED_R && r_agg != nullptr;
  const int i = 16 * rw + li;
  const int cc = 4 * (li % 4);
  uint16_t* sDQ = sStage + w * 16 * (SC + kLdsPad);
  // causal mask of key j = 16t + 4g + u against query i = 16w + li, as 0 / 1
  // factors (kept in VGPRs: as per-(t, u) lane masks they would not fit in
  // the scalar registers)
  f32x4_t mt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) mt[t][u] = (t < rw || (t == rw && 4 * g + u <= li)) ? 1.f : 0.f;

  int64_t c0 = r0;
  int nrow = static_cast<int>(min(static_cast<int64_t>(T), r1 - c0));
  i32x4 kraw[PC], vraw[PC], qraw[PC], graw[KS];
  auto fetch = [&](int soff) {
    if (CAUSAL) {
      bload_tile<DIM, NW>(kraw, rk, soff);
      bload_tile<DIM, NW>(vraw, rv, soff);
    }
    bload_tile<DIM, NW>(qraw, rq, soff);
    bload_q<DIM>(graw, rg, soff, i, g);
  };
  fetch(static_cast<int>(c0 * DIM * 2));

  bool all_one_;
  const float smu2 = MU1 ? static_cast<float>(DIM) : mu_sq_sum<DIM>(sMuF, &all_one_);
  MuOff moff;
  if constexpr (!MU1) moff = mu_offsets<DIM, NW>(sMuF);
  const short one = 0x3f80;  // bf16 1.0
  const i16x8 ones = {one, one, one, one, one, one, one, one};

  f32x4_t Sacc[DT][NTL], zacc[DT], uacc[DT];
  // n0: the mu-direction count of the state before the current chunk
  float n0 = init_split<DIM, NW>(Sacc, zacc, uacc, cs, sMuF, smu2, w, g, li);
  f32x4_t Racc[FUSED_R ? DT : 1][FUSED_R ? NTL : 1], racc[FUSED_R ? DT : 1], gacc[FUSED_R ? DT : 1];
  if constexpr (FUSED_R) init_split<DIM>(Racc, racc, gacc, nullptr, sMuF, smu2, w, g, li);
  write_xt<DIM, NW>(sS, sZ, Sacc, zacc, w, g, li);
  write_y<DIM, NW>(sU, uacc, w, g, li);
  float csum = 0.f;

  int buf = 0;
  while (c0 < r1) {
    uint16_t* sQe = sQe2 + (L::NQ == 2 ? buf : 0) * T * LD;
    uint16_t* sG = sG2 + (L::NG == 2 ? buf : 0) * T * LD;
    uint16_t* sCh = sCh2 + buf * 2 * T;
    // rows past the head's end were loaded as zero (elu(0) = 0)
    if constexpr (MU1) {
      if (CAUSAL) store_tile_e<DIM, NW>(sKe, kraw);
      store_tile_e<DIM, NW>(sQe, qraw);
    } else {
      if (CAUSAL) store_tile_emu<DIM, NW>(sKe, kraw, nrow, moff);
      store_tile_emu<DIM, NW>(sQe, qraw, nrow, moff);
    }
    if (CAUSAL) store_tile_v<DIM, NW>(sV, vraw);
    __syncthreads();
    const bool valid = i < nrow;
    i32x4 gcur[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) gcur[s] = graw[s];
    const int64_t c1 = c0 + T;
    const int nrow1 = c1 < r1 ? static_cast<int>(min(static_cast<int64_t>(T), r1 - c1)) : 0;
    if (nrow1 > 0) fetch(static_cast<int>(c1 * DIM * 2));
    // The chunk's compute runs at raised wave priority (back to 0 before
    // its stores): with two resident workgroups per CU, the wave that is in
    // its dependent MFMA / VALU chains issues ahead of one that is staging
    // (dq 153 -> 142 us on the B=8 H=16 N=8192 D=64 step).
    __builtin_amdgcn_s_setprio(2);
    const int soff = static_cast<int>(c0 * DIM * 2);

    // E(Q_i) in the MFMA B layout (features 8g + 32s + e) and, unpacked once,
    // in the accumulator layout (features 16n + 4g + u)
    i16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = lds8(sQe + i * LD + 8 * g + 32 * s);
    f32x4_t qd[NTL];
#pragma unroll
    for (int n = 0; n < NTL; ++n) qd[n] = unpack4(*reinterpret_cast<const i16x4*>(sQe + i * LD + 16 * n + 4 * g));
    // phi(Q_i) = mu + E in the accumulator layout (an arithmetic result, so
    // the min below needs no NaN canonicalisation)
    f32x4_t pq[NTL];
#pragma unroll
    for (int n = 0; n < NTL; ++n)
      pq[n] = (MU1 ? f32x4_t{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4_t*>(sMuF + 16 * n + 4 * g)) + qd[n];
    // mu as an MFMA operand (features 8g + 32s + e, the same in every row)
    i16x8 mub[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) mub[s] = MU1 ? ones : lds8(sMuB + 8 * g + 32 * s);
    // sum_d mu_d phi(Q_i) = smu2 + sum_d mu_d E(Q_i), through the MFMA against mu
    f32x4_t sq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) sq = mfma(mub[s], qf[s], sq);
    const float dq_i = smu2 + sq[0];
    // --- scores A^T[j][i] = (smu2 + sq_i) + sk_j + E_j.E_i, masked j <= i:
    // sk_j = sum_d mu_d E(K_j) from the same MFMA chain against mu
    f32x4_t at[4];
    float rs = 0.f;
    if (CAUSAL) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        at[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (t <= rw) {
          at[t] = f32x4_t{dq_i, dq_i, dq_i, dq_i};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            const i16x8 ka = lds8(sKe + (16 * t + li) * LD + 8 * g + 32 * s);
            at[t] = mfma(ka, mub[s], at[t]);
            at[t] = mfma(ka, qf[s], at[t]);
          }
          at[t] *= mt[t];
#pragma unroll
          for (int u = 0; u < 4; ++u) rs += at[t][u];
        }
      }
    }
    // --- den_i = sum_j A_ij + n0 (D + sq_i) + sum_d (1 + E_i)[d] Z'[d]
    float di = 0.f;
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
      const f32x4_t z = *reinterpret_cast<const f32x4_t*>(sZ + 16 * n + 4 * g);
#pragma unroll
      for (int u = 0; u < 4; ++u) di += pq[n][u] * z[u];
    }
    const float den = shfl_sum_groups(rs + di) + n0 * dq_i;
    const float inv = valid ? __builtin_amdgcn_rcpf(den) : 0.f;  // the reverse sweep forms the same g
    // --- g_i = bf16(dout_i / den_i): registers (B operand) and sG (for R);
    // g_i . U in fp32 from the rounded g
    i16x8 gq[KS];
    float gu = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      gq[s] = pack8(unpack8(__builtin_bit_cast(i16x8, gcur[s])) * inv);
      if constexpr (FUSED_R) *reinterpret_cast<i16x8*>(sG + i * LD + 8 * g + 32 * s) = gq[s];
      const f32x8_t gv = unpack8(gq[s]);
      const f32x8_t uv = *reinterpret_cast<const f32x8_t*>(sU + 8 * g + 32 * s);
#pragma unroll
      for (int e = 0; e < 8; ++e) gu += gv[e] * uv[e];
    }
    gu = shfl_sum_groups(gu);
    // --- S' g_i  (dQ^T[d][i] inter term, this wave's columns) and
    // Bv^T[j][i] = g_i . V_j
    f32x4_t o[NH];
#pragma unroll
    for (int a = 0; a < NH; ++a) {
      o[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) o[a] = mfma(lds8(sS + (16 * (NB + a) + li) * LD + 8 * g + 32 * s), gq[s], o[a]);
    }
    f32x4_t bv[4];
    if (CAUSAL) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        bv[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (t <= rw) {
#pragma unroll
          for (int s = 0; s < KS; ++s) bv[t] = mfma(lds8(sV + (16 * t + li) * LD + 8 * g + 32 * s), gq[s], bv[t]);
        }
      }
    }
    // --- c_i = -(sum_j A_ij bv_ij + (D + sq_i) g.U + sum_d (1 + E_i) (S'g)) / den_i
    float dot = 0.f, sbv = 0.f;
#pragma unroll
    for (int a = 0; a < NH; ++a)
#pragma unroll
      for (int u = 0; u < 4; ++u) dot += pq[NB + a][u] * o[a][u];
    if constexpr (NW == 8) {
      // the pair's two halves of sum_d phi(Q_i)[d] (S'g)[d], added in half
      // order so that both waves form the same c
      const float half = shfl_sum_groups(dot);
      if (g == 0) sDot[H * T + i] = half;
      dot = 0.f;
      __syncthreads();
    }
    if (CAUSAL) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (t <= rw) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            dot += at[t][u] * bv[t][u];  // at is masked
            sbv += mt[t][u] * bv[t][u];
          }
        }
    }
    const float dsum = NW == 8 ? (sDot[i] + sDot[T + i]) + shfl_sum_groups(dot) : shfl_sum_groups(dot);
    const float c = -(dsum + dq_i * gu) * inv;
    // beta_i = g.U + n_i c_i + sum_{j in chunk} g.V_j, n_i = n0 + (i + 1)
    const float beta = gu + c * (n0 + (CAUSAL ? static_cast<float>(i + 1) : 0.f)) + shfl_sum_groups(sbv);
    csum += c;
    if (g == 0 && H == 0) {
      if constexpr (FUSED_R) put_c(sCh, i, c);
      if (valid) {
        ch[c0 + i] = c;
        dh[c0 + i] = den;
      }
    }
    // --- grad phi(Q)^T[d][i] = mu_d beta + S'g + c Z'[d] + E(K)^T b, times phi'(q)
    if (CAUSAL) {
      i16x4 bt[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) bt[t] = pack4((bv[t] + c) * mt[t]);
#pragma unroll
      for (int a_ = 0; a_ < NH; ++a_) {
        const int n = NB + a_;
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          if (2 * tp <= rw) {
            const int jr = 32 * tp + 4 * g + li / 4;
            const i16x8 a = cat(lds_tr(sKe + jr * LD + 16 * n + cc), lds_tr(sKe + (jr + 16) * LD + 16 * n + cc));
            o[a_] = mfma(a, cat(bt[2 * tp], bt[2 * tp + 1]), o[a_]);
          }
        }
      }
    }
#pragma unroll
    for (int a = 0; a < NH; ++a) {
      const int n = NB + a;
      const f32x4_t z = *reinterpret_cast<const f32x4_t*>(sZ + 16 * n + 4 * g);
      const f32x4_t mu4 = MU1 ? f32x4_t{1.f, 1.f, 1.f, 1.f} : *reinterpret_cast<const f32x4_t*>(sMuF + 16 * n + 4 * g);
      f32x4_t r;
      // phi'(q) = min(phi(q), 1)
#pragma unroll
      for (int u = 0; u < 4; ++u) r[u] = (mu4[u] * beta + o[a][u] + c * z[u]) * fminf(pq[n][u], 1.f);
      stage_piece<SC>(sDQ, pack4(r), li, g, a);
    }
    __builtin_amdgcn_s_setprio(0);
    store_staged<SC, DIM>(sDQ, rdq, 16 * rw, SC * H, soff);
    if (CAUSAL) outer_update_y<DIM, false, NW>(Sacc, zacc, uacc, sV, sKe, nullptr, w, g, li);
    __syncthreads();
    // this chunk's g, E(Q) and c rows are complete: sum its (R, r) part
    if constexpr (FUSED_R)
      if (want_r) outer_update_y<DIM, true>(Racc, racc, gacc, sG, sQe, sCh, w, g, li);
    if (CAUSAL) {
      write_xt<DIM, NW>(sS, sZ, Sacc, zacc, w, g, li);
      write_y<DIM, NW>(sU, uacc, w, g, li);
    }
    if (CAUSAL) n0 += static_cast<float>(nrow);
    c0 = c1;
    nrow = nrow1;
    buf ^= 1;
  }
  if constexpr (FUSED_R) {
    if (want_r) {
      // C = sum of c over the segment's rows (csum is the same in all four
      // 16-lane groups of a wave: sum over li, then over the row tiles in
      // their order, whichever wave holds which)
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) csum += __shfl_xor(csum, off, 64);
      if (l == 0) sRed[rw] = csum;
      __syncthreads();
      const float C = sRed[0] + sRed[1] + sRed[2] + sRed[3];
      store_r<DIM>(r_agg + (bh * P + seg) * ER, Racc, racc, gacc, C, sMuF, w, g, li);
    }
  }
}

template <int DIM, bool CAUSAL, bool FUSED_R>
__global__ __launch_bounds__(64 * kBwdWaves<DIM>, DIM == 64 ? 2 : 1) void k_bwd_dq_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ carry_s, bf16_t* __restrict__ dq,
    float* __restrict__ r_agg, float* __restrict__ c_out, float* __restrict__ den_out, int64_t N, int P,
    int seg_len) {
  // The triangular intra-chunk work grows with a wave's row tile (tile t
  // does t + 1 key tiles).  Four waves: odd workgroups map wave w to tile
  // 3 - w, so two workgroups sharing a CU give every SIMD the same total.
  // Eight waves (one workgroup per CU, waves w and w + 4 on one SIMD): wave
  // w < 4 takes tile w and the first half of the columns, wave w >= 4 tile
  // 7 - w and the second half, so every SIMD pairs a short and a long
  // triangle and the two waves on tile t are t and 7 - t.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bh = blockIdx.x / P;
  const int seg = static_cast<int>(blockIdx.x % P);
  // the same value in every thread (read from LDS after a barrier)
  const bool mu1 = __builtin_amdgcn_readfirstlane(dq_decide_mu<DIM, CAUSAL>(k, carry_s, N, P, seg_len, bh, seg) ? 1 : 0) != 0;
#define LA_DQ_BODY(CASE_, RW_, H_)                                                                               \
  case CASE_:                                                                                                    \
    if (mu1)                                                                                                     \
      dq_body<DIM, CAUSAL, FUSED_R, RW_, H_, true>(q, k, v, dout, carry_s, dq, r_agg, c_out, den_out, N, P,     \
                                                   seg_len, bh, seg);                                            \
    else                                                                                                         \
      dq_body<DIM, CAUSAL, FUSED_R, RW_, H_, false>(q, k, v, dout, carry_s, dq, r_agg, c_out, den_out, N, P,    \
                                                    seg_len, bh, seg);                                           \
    break
  if constexpr (kBwdWaves<DIM> == 4) {
    switch ((blockIdx.x & 1) ? 3 - w : w) {
      LA_DQ_BODY(0, 0, 0);
      LA_DQ_BODY(1, 1, 0);
      LA_DQ_BODY(2, 2, 0);
      LA_DQ_BODY(3, 3, 0);
    }
  } else {
    switch (w) {
      LA_DQ_BODY(0, 0, 0);
      LA_DQ_BODY(1, 1, 0);
      LA_DQ_BODY(2, 2, 0);
      LA_DQ_BODY(3, 3, 0);
      LA_DQ_BODY(4, 3, 1);
      LA_DQ_BODY(5, 2, 1);
      LA_DQ_BODY(6, 1, 1);
      LA_DQ_BODY(7, 0, 1);
    }
  }
#undef LA_DQ_BODY
}

// ---------------------------------------------------------------------------
// The segment's (R, r) aggregate as its own pass (used at D = 128): the same
// g_i = bf16(dout_i / den_i) and c_i the forward sweep used (den, c read from
// its outputs), summed as the fused version sums them, with R = mu G^T +
// sum_i E(Q_i) g_i^T for a split constant mu chosen from the segment's first
// chunk of queries (the aggregate is a whole record, so any mu gives it).
// ---------------------------------------------------------------------------
template <int DIM>
__global__ __launch_bounds__(NT, 2) void k_bwd_ragg_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ dout,
                                                         const float* __restrict__ den_in,
                                                         const float* __restrict__ c_in, float* __restrict__ r_agg,
                                                         int64_t N, int P, int seg_len) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sQe = smem;
  uint16_t* sG = sQe + T * LD;
  float* sRed = reinterpret_cast<float*>(sG + T * LD);
  uint16_t* sCh = reinterpret_cast<uint16_t*>(sRed + 4);
  float* sMuF = reinterpret_cast<float*>(sCh + 2 * T);
  uint16_t* sMuB = reinterpret_cast<uint16_t*>(sMuF + DIM);
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t ER = static_cast<int64_t>(DIM) * DIM + DIM;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rg = make_rsrc(dout + hoff, hbytes);
  const float* denh = den_in + bh * N;
  const float* chh = c_in + bh * N;
  const int i = 16 * w + li;
  i32x4 qraw[PC], graw[KS];
  {
    // the split constant from the first chunk of queries
    bload_tile<DIM>(qraw, rq, static_cast<int>(r0 * DIM * 2));
    store_tile_e<DIM>(sQe, qraw);
    __syncthreads();
    decide_mu<DIM, LD>(sQe, static_cast<int>(min(static_cast<int64_t>(T), r1 - r0)), sMuF, sMuB);
    __syncthreads();
  }
  const MuOff moff = mu_offsets<DIM>(sMuF);
  f32x4_t Racc[DT][NTL], racc[DT], gacc[DT];
  init_split<DIM>(Racc, racc, gacc, nullptr, sMuF, 0.f, w, g, li);  // no carried record: zeros
  float csum = 0.f;
  // the next chunk's q tile, g rows, den and c are loaded while this one is
  // summed (rows past the segment read as zero, den as 1)
  float dn = 1.f, cn = 0.f;
  auto fetch = [&](int64_t cc0) {
    const int soff = static_cast<int>(cc0 * DIM * 2);
    bload_tile<DIM>(qraw, rq, soff);
    bload_q<DIM>(graw, rg, soff, i, g);
    const bool ok = cc0 + i < r1;
    dn = ok ? denh[cc0 + i] : 1.f;
    cn = ok ? chh[cc0 + i] : 0.f;
  };
  fetch(r0);
  for (int64_t c0 = r0; c0 < r1; c0 += T) {
    const int nrow = static_cast<int>(min(static_cast<int64_t>(T), r1 - c0));
    const bool valid = i < nrow;
    const float inv = valid ? __builtin_amdgcn_rcpf(dn) : 0.f;  // as in the forward sweep
    const float c = valid ? cn : 0.f;
    store_tile_emu<DIM>(sQe, qraw, nrow, moff);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      *reinterpret_cast<i16x8*>(sG + i * LD + 8 * g + 32 * s) = pack8(unpack8(__builtin_bit_cast(i16x8, graw[s])) * inv);
    if (g == 0) put_c(sCh, i, c);
    csum += c;
    __syncthreads();
    if (c0 + T < r1) fetch(c0 + T);
    outer_update_y<DIM, true>(Racc, racc, gacc, sG, sQe, sCh, w, g, li);
    __syncthreads();
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) csum += __shfl_xor(csum, off, 64);
  if (l == 0) sRed[w] = csum;
  __syncthreads();
  const float C = sRed[0] + sRed[1] + sRed[2] + sRed[3];
  store_r<DIM>(r_agg + (bh * P + seg) * ER, Racc, racc, gacc, C, sMuF, w, g, li);
}

// ---------------------------------------------------------------------------
// Reverse sweep: dk, dv with the suffix state (R, r) carried in.
// ---------------------------------------------------------------------------
// poison: the suffix carry could not be formed (a hand-off that timed out in
// the fused kernel): the carry is NaN, so every dk, dv row of the segment is.
template <int DIM, bool CAUSAL>
__device__ __forceinline__ void dkdv_body(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                          const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                                          const float* __restrict__ den_in, const float* __restrict__ c_in,
                                          const float* __restrict__ carry_r, bf16_t* __restrict__ dk,
                                          bf16_t* __restrict__ dv, int64_t N, int P, int seg_len, int carry_raw,
                                          int64_t bh, int seg, int rw, int h, bool poison) {
  constexpr int NW = kBwdWaves<DIM>;
  using G = Geo<DIM, NW>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  // this wave's output column tiles nb .. nb + NH - 1 (all of them with four
  // waves; half h of them with eight, h = 0 also staging the rows' g and c)
  constexpr int SC = 4 * DIM / NW, NH = SC / 16;
  const int nb = h * NH;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sKf = smem;
  uint16_t* sV = sKf + T * LD;
  uint16_t* sQf = sV + T * LD;
  uint16_t* sG = sQf + T * LD;
  uint16_t* sR = sG + T * LD;
  float* sRv = reinterpret_cast<float*>(sR + DIM * LD);
  float* sC = sRv + DIM;
  uint16_t* sCh = reinterpret_cast<uint16_t*>(sC + T);

  // w is made wave-uniform (an SGPR) so that branches on it are scalar: an
  // MFMA under an EXEC-masked branch still writes every lane.
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  (void)l;
  // this wave's staging tiles for its dv and dk rows and columns
  uint16_t* sDV = sCh + 2 * T + w * 2 * 16 * (SC + kLdsPad);
  uint16_t* sDK = sDV + 16 * (SC + kLdsPad);
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;  // R, r record
  const float* cr = carry_r ? (CAUSAL ? carry_r + (bh * P + seg) * E : carry_r + bh * E) : nullptr;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               rg = make_rsrc(dout + hoff, hbytes), rdk = make_rsrc(dk + hoff, hbytes),
               rdv = make_rsrc(dv + hoff, hbytes);
  const float* denh = den_in + bh * N;
  const float* chh = c_in + bh * N;
  const int j = 16 * rw + li;  // this lane's key row (outputs); also its query row for g, c
  // causal mask of query i = 16t + 4g + u against key j = 16w + li (i >= j)
  // as 0 / 1 factors
  f32x4_t mt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) mt[t][u] = (t > rw || (t == rw && 4 * g + u >= li)) ? 1.f : 0.f;

  f32x4_t Racc[DT][NTL], racc[DT];
  if (CAUSAL && carry_raw && carry_r)
    // carry_r holds the raw suffix aggregates: the carry is summed here (no
    // separate scan launch)
    init_xt_suffix<DIM, NW>(Racc, racc, carry_r + bh * P * E, seg, P, w, g, li);
  else
    init_xt<DIM, NW>(Racc, racc, cr, w, g, li);
  if (poison) {
    const float nan = __builtin_nanf("");
#pragma unroll
    for (int a = 0; a < DT; ++a) {
      racc[a] = f32x4_t{nan, nan, nan, nan};
#pragma unroll
      for (int n = 0; n < NTL; ++n) Racc[a][n] = racc[a];
    }
  }
  write_xt<DIM, NW>(sR, sRv, Racc, racc, w, g, li);

  const int64_t nch = (r1 - r0 + T - 1) / T;
  int64_t ci = nch - 1;
  int64_t c0 = r0 + ci * T;
  int nrow = static_cast<int>(min(static_cast<int64_t>(T), r1 - c0));
  i32x4 kraw[PC], vraw[PC], qraw[PC], graw[KS];
  float dnr = 1.f, cnr = 0.f;
  auto fetch = [&](int64_t cc0, int nr) {
    const int soff = static_cast<int>(cc0 * DIM * 2);
    bload_tile<DIM, NW>(kraw, rk, soff);
    bload_tile<DIM, NW>(vraw, rv, soff);
    if (CAUSAL) {
      bload_tile<DIM, NW>(qraw, rq, soff);
      if (h == 0) {
        bload_q<DIM>(graw, rg, soff, j, g);
        dnr = j < nr ? denh[cc0 + j] : 1.f;
        cnr = j < nr ? chh[cc0 + j] : 0.f;
      }
    }
  };
  fetch(c0, nrow);

  while (ci >= 0) {
    store_tile<DIM, true, NW>(sKf, kraw, nrow);
    store_tile_v<DIM, NW>(sV, vraw);
    if (CAUSAL) {
      // the same g_i = bf16(dout_i / den_i) and c_i as the forward sweep used
      store_tile<DIM, true, NW>(sQf, qraw, nrow);
      if (h == 0) {
        const float inv = j < nrow ? __builtin_amdgcn_rcpf(dnr) : 0.f;  // as in the forward sweep
#pragma unroll
        for (int s = 0; s < KS; ++s)
          *reinterpret_cast<i16x8*>(sG + j * LD + 8 * g + 32 * s) =
              pack8(unpack8(__builtin_bit_cast(i16x8, graw[s])) * inv);
        if (g == 0) {
          sC[j] = cnr;
          put_c(sCh, j, cnr);
        }
      }
    }
    __syncthreads();
    const int soff = static_cast<int>(c0 * DIM * 2);

    const int64_t cp = c0 - T;
    const int nrowp = ci > 0 ? T : 0;  // earlier chunks of a segment are always full
    if (ci > 0) fetch(cp, nrowp);

    i16x8 kreg[KS], vreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kreg[s] = lds8(sKf + j * LD + 8 * g + 32 * s);
      vreg[s] = lds8(sV + j * LD + 8 * g + 32 * s);
    }
    // A[i][j] = phi(Q_i).phi(K_j) and Bm[i][j] = g_i.V_j + c_i for query
    // tiles t >= w, masked i >= j; A as hi + lo
    i16x4 ahi[4], alo[4], bm[4];
    if (CAUSAL) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        ahi[t] = alo[t] = bm[t] = i16x4{0, 0, 0, 0};
        if (t >= rw) {
          f32x4_t a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            a = mfma(lds8(sQf + (16 * t + li) * LD + 8 * g + 32 * s), kreg[s], a);
            b = mfma(lds8(sG + (16 * t + li) * LD + 8 * g + 32 * s), vreg[s], b);
          }
          const f32x4_t cv = *reinterpret_cast<const f32x4_t*>(sC + 16 * t + 4 * g);
          split(a * mt[t], ahi[t], alo[t]);
          bm[t] = pack4((b + cv) * mt[t]);
        }
      }
    }
    const int cc = 4 * (li % 4);
#pragma unroll
    for (int a_ = 0; a_ < NH; ++a_) {
      const int n = nb + a_;
      // grad V^T[m][j] = R^T phi(K_j) (+ g^T A)
      f32x4_t ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int dr = 32 * s + 8 * g + li / 4;
        const i16x8 a = cat(lds_tr(sR + dr * LD + 16 * n + cc), lds_tr(sR + (dr + 4) * LD + 16 * n + cc));
        ov = mfma(a, kreg[s], ov);
      }
      // grad phi(K)^T[d][j] = R V_j (+ phi(Q)^T Bm) + r[d]
      f32x4_t ok = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) ok = mfma(lds8(sR + (16 * n + li) * LD + 8 * g + 32 * s), vreg[s], ok);
      if (CAUSAL) {
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
          if (2 * tp + 1 >= rw) {
            const int ir = 32 * tp + 4 * g + li / 4;
            const i16x8 ag = cat(lds_tr(sG + ir * LD + 16 * n + cc), lds_tr(sG + (ir + 16) * LD + 16 * n + cc));
            ov = mfma(ag, cat(ahi[2 * tp], ahi[2 * tp + 1]), ov);
            ov = mfma(ag, cat(alo[2 * tp], alo[2 * tp + 1]), ov);
            const i16x8 aq = cat(lds_tr(sQf + ir * LD + 16 * n + cc), lds_tr(sQf + (ir + 16) * LD + 16 * n + cc));
            ok = mfma(aq, cat(bm[2 * tp], bm[2 * tp + 1]), ok);
          }
        }
      }
      // rows past the head's end fall outside the buffer range: dropped
      const f32x4_t kv = unpack4(*reinterpret_cast<const i16x4*>(sKf + j * LD + 16 * n + 4 * g));
      const f32x4_t rr = *reinterpret_cast<const f32x4_t*>(sRv + 16 * n + 4 * g);
      f32x4_t rk;
#pragma unroll
      for (int u = 0; u < 4; ++u) rk[u] = (ok[u] + rr[u]) * fminf(kv[u], 1.f);
      stage_piece<SC>(sDV, pack4(ov), li, g, a_);
      stage_piece<SC>(sDK, pack4(rk), li, g, a_);
    }
    store_staged<SC, DIM>(sDV, rdv, 16 * rw, SC * h, soff);
    store_staged<SC, DIM>(sDK, rdk, 16 * rw, SC * h, soff);
    if (CAUSAL) outer_update<DIM, true, NW>(Racc, racc, sG, sQf, sCh, w, g, li);
    __syncthreads();
    if (CAUSAL) write_xt<DIM, NW>(sR, sRv, Racc, racc, w, g, li);
    --ci;
    c0 = cp;
    nrow = nrowp;
  }
}

template <int DIM, bool CAUSAL>
__global__ __launch_bounds__(64 * kBwdWaves<DIM>, DIM == 64 ? 2 : 1) void k_bwd_dkdv_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                                                      const float* __restrict__ den_in,
                                                      const float* __restrict__ c_in,
                                                      const float* __restrict__ carry_r, bf16_t* __restrict__ dk,
                                                      bf16_t* __restrict__ dv, int64_t N, int P, int seg_len,
                                                      int carry_raw) {
  // The triangular intra-chunk work grows with a wave's row tile (tile t
  // does 4 - t query tiles): the row tiles and column halves are mapped to
  // the waves as in the dq sweep.
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rt = kBwdWaves<DIM> == 4 ? ((blockIdx.x & 1) ? 3 - w : w) : (w < 4 ? w : 7 - w);
  const int h = kBwdWaves<DIM> == 4 ? 0 : w >> 2;
  dkdv_body<DIM, CAUSAL>(q, k, v, dout, den_in, c_in, carry_r, dk, dv, N, P, seg_len, carry_raw, blockIdx.x / P,
                         static_cast<int>(blockIdx.x % P), rt, h, false);
}

// ---------------------------------------------------------------------------
// The causal backward in one launch (D = 64): each workgroup runs the
// forward sweep over its segment (dq, c, den and the segment's (R, r)
// aggregate), publishes the aggregate, waits for the aggregates of every
// later segment of its sequence, sums them into its suffix carry (in the
// reverse-scan order, as the split sweeps do) and runs the reverse sweep
// over the same segment (dk, dv).  The reverse sweep re-reads the tokens the
// forward sweep has just read, last chunk first, so most of those reads
// come from the last-level cache instead of HBM.  Results are bit for bit
// those of k_bwd_dq_mfma followed by k_bwd_dkdv_mfma.
//
// Hand-off.  Workgroup b serves sequence b / P, segment P - 1 - b % P: the
// later segments of a sequence have the lower workgroup indices, so a
// workgroup only ever waits for workgroups dispatched before it (which hold
// their slots and finish without waiting on anything later), and the host
// launches it only when every workgroup of the grid can be resident at once
// besides.  flags[bh * P + seg] (cleared before the launch) becomes `want`
// once the aggregate is in memory: every thread's stores are released at
// agent scope (written back past this XCD's L2) before a barrier, after which
// one thread sets the flag with a vector atomic store.  The waiting thread
// polls the flags with agent-scope atomic loads (sleeping between polls),
// then every thread acquires at agent scope before reading the records.
// Each wait is bounded by `spin_ticks` of the 100 MHz real-time counter; a
// workgroup whose wait runs out sets *err (la_device_error reports it),
// poisons its dk, dv with NaN and still runs to its end, so the grid always
// drains.
// ---------------------------------------------------------------------------
template <int DIM>
__global__ __launch_bounds__(NT, 2) void k_bwd_fused_mfma(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ carry_s, bf16_t* __restrict__ dq,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ r_agg, float* __restrict__ c_ws,
    float* __restrict__ den_ws, unsigned* __restrict__ flags, unsigned* __restrict__ err, unsigned want,
    long long spin_ticks, int64_t N, int P, int seg_len) {
  __shared__ int s_ok;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t bh = blockIdx.x / P;
  const int seg = P - 1 - static_cast<int>(blockIdx.x % P);
  const int rw = (blockIdx.x & 1) ? 3 - w : w;
  // segment 0's aggregate would only feed the total, which is not needed
  float* ragg = seg > 0 ? r_agg : nullptr;
  const bool mu1 = __builtin_amdgcn_readfirstlane(dq_decide_mu<DIM, true>(k, carry_s, N, P, seg_len, bh, seg) ? 1 : 0) != 0;
  switch (rw) {
#define LA_FUSED_DQ(RW_)                                                                                           \
  case RW_:                                                                                                        \
    if (mu1)                                                                                                       \
      dq_body<DIM, true, true, RW_, 0, true>(q, k, v, dout, carry_s, dq, ragg, c_ws, den_ws, N, P, seg_len, bh,  \
                                             seg);                                                               \
    else                                                                                                           \
      dq_body<DIM, true, true, RW_, 0, false>(q, k, v, dout, carry_s, dq, ragg, c_ws, den_ws, N, P, seg_len, bh, \
                                              seg);                                                              \
    break
    LA_FUSED_DQ(0);
    LA_FUSED_DQ(1);
    LA_FUSED_DQ(2);
    LA_FUSED_DQ(3);
#undef LA_FUSED_DQ
  }
  // publish this segment's aggregate (and make c, den visible)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  if (threadIdx.x == 0) {
    if (seg > 0) __hip_atomic_store(flags + bh * P + seg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int ok = 1;
    if (seg + 1 < P) {
      const long long t0 = static_cast<long long>(wall_clock64());
      for (int p = P - 1; p > seg && ok; --p) {
        while (__hip_atomic_load(flags + bh * P + p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != want) {
          if (static_cast<long long>(wall_clock64()) - t0 > spin_ticks) {
            ok = 0;
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
      }
      if (!ok) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_ok = ok;
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  dkdv_body<DIM, true>(q, k, v, dout, den_ws, c_ws, r_agg, dk, dv, N, P, seg_len, 1, bh, seg, rw, 0, s_ok == 0);
}

__global__ __launch_bounds__(256) void k_fill_u32(unsigned* __restrict__ p, int64_t n, unsigned val) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = val;
}

size_t lds_bwd(int dim) {
  const int nw = dim == 128 ? kBwdWaves<128> : kBwdWaves<64>, sc = 4 * dim / nw;
  return (4 * T * (dim + kLdsPad) + dim * (dim + kLdsPad)) * sizeof(uint16_t) + (dim + T) * sizeof(float) +
         2 * T * sizeof(uint16_t) + nw * 2 * 16 * (sc + kLdsPad) * sizeof(uint16_t);  // + output staging
}
// (+ the split constant mu as fp32 and bf16)
size_t lds_ragg(int dim) {
  return 2 * T * (dim + kLdsPad) * sizeof(uint16_t) + 4 * sizeof(float) + 2 * T * sizeof(uint16_t) +
         dim * (sizeof(float) + sizeof(uint16_t));
}
size_t lds_dq(int dim) { return dim == 128 ? DqLds<128>::BYTES : DqLds<64>::BYTES; }

#define LA_MLAUNCH(kernel, threads, grid, lds, st, ...)                                                     \
  do {                                                                                                      \
    hipError_t e_ = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),                              \
                                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)); \
    if (e_ != hipSuccess) return e_;                                                                        \
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(threads), lds, st, __VA_ARGS__);     \
    return hipGetLastError();                                                                               \
  } while (0)

}  // namespace

hipError_t launch_bwd_dq_mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                              const void* dout, const float* carry_s, void* dq, float* r_agg, float* c_out,
                              float* den_out, hipStream_t st) {
  const int64_t grid = g.BH * g.P;
#define LA_DQ(D, C, F)                                                                                       \
  LA_MLAUNCH((k_bwd_dq_mfma<D, C, F>), 64 * kBwdWaves<D>, grid, lds_dq(D), st,                              \
             static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),   \
             static_cast<const bf16_t*>(dout), carry_s, static_cast<bf16_t*>(dq), r_agg, c_out, den_out, g.N, g.P, g.seg_len)
  if (g.D == 64) {
    if (causal) LA_DQ(64, true, true);
    LA_DQ(64, false, true);
  }
  if (g.D != 128) return hipErrorNotSupported;
  const hipError_t e = [&]() -> hipError_t {
    if (causal) LA_DQ(128, true, false);
    LA_DQ(128, false, false);
  }();
  if (e != hipSuccess || !r_agg) return e;
  LA_MLAUNCH((k_bwd_ragg_mfma<128>), NT, grid, lds_ragg(128), st, static_cast<const bf16_t*>(q),
             static_cast<const bf16_t*>(dout), den_out, c_out, r_agg, g.N, g.P, g.seg_len);
#undef LA_DQ
}

int bwd_fused_supported(int causal, int D) { return causal && D == 64; }

size_t lds_bwd_fused(int dim) { return lds_dq(dim) > lds_bwd(dim) ? lds_dq(dim) : lds_bwd(dim); }

// Workgroups of the fused kernel that can be resident at once on this
// device (0 on error).
int64_t bwd_fused_resident(int dim) {
  static int64_t cached[64] = {};  // per device; the answer does not change
  int dev = 0, cus = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64 && cached[dev] > 0) return cached[dev];
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dim != 64) return 0;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_bwd_fused_mfma<64>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds_bwd_fused(64))) != hipSuccess)
    return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_bwd_fused_mfma<64>, NT, lds_bwd_fused(64)) != hipSuccess)
    return 0;
  const int64_t n = static_cast<int64_t>(per) * cus;
  if (dev >= 0 && dev < 64) cached[dev] = n;
  return n;
}

hipError_t launch_bwd_fused_mfma(const SegGeom& g, const void* q, const void* k, const void* v, const void* dout,
                                 const float* carry_s, void* dq, void* dk, void* dv, float* r_agg, float* c_ws,
                                 float* den_ws, unsigned* flags, unsigned* err, unsigned want, long long spin_ticks,
                                 hipStream_t st) {
  if (g.D != 64) return hipErrorNotSupported;
  const int64_t nflags = g.BH * g.P;
  hipLaunchKernelGGL(k_fill_u32, dim3(static_cast<unsigned>(std::min<int64_t>((nflags + 255) / 256, 1024))),
                     dim3(256), 0, st, flags, nflags, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  LA_MLAUNCH((k_bwd_fused_mfma<64>), NT, g.BH * g.P, lds_bwd_fused(64), st, static_cast<const bf16_t*>(q),
             static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout),
             carry_s, static_cast<bf16_t*>(dq), static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), r_agg, c_ws,
             den_ws, flags, err, want, spin_ticks, g.N, g.P, g.seg_len);
}

hipError_t launch_bwd_dkdv_mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                                const void* dout, const float* den, const float* c, const float* carry_r,
                                void* dk, void* dv, hipStream_t st, int carry_raw) {
  const int64_t grid = g.BH * g.P;
#define LA_KV(D, C)                                                                                          \
  LA_MLAUNCH((k_bwd_dkdv_mfma<D, C>), 64 * kBwdWaves<D>, grid, lds_bwd(D), st,                              \
             static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),   \
             static_cast<const bf16_t*>(dout), den, c, carry_r, static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), g.N, g.P, g.seg_len, carry_raw)
  if (g.D == 64) {
    if (causal) LA_KV(64, true);
    LA_KV(64, false);
  }
  if (g.D == 128) {
    if (causal) LA_KV(128, true);
    LA_KV(128, false);
  }
#undef LA_KV
  return hipErrorNotSupported;
}

}  // namespace la
