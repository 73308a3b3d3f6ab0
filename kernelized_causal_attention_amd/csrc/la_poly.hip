// Linear attention with the degree-2 polynomial kernel on gfx950: bf16 MFMA
// kernels, D = M in {64, 128}.
//
// "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io), section
// 2, "feature map and computation cost", item (3): sim(q, k) = (q^T k)^2,
// whose explicit feature map has C = D^2 coordinates; the attention is
// eq:common with that kernel, causally masked as in eq:mask:
//   out_i = sum_{j<=i} (q_i . k_j)^2 v_j / den_i,  den_i = sum_{j<=i} (q_i . k_j)^2
// (0/0 read as 0: the denominator vanishes only when every weight does).
//
// These kernels evaluate the masked sum directly, block by block, without
// materialising the D^2 features: per query-key pair the cost is 2D + 2M
// flops here against 4 D^2 M / (pairs per query) for the explicit-feature
// linear form, so for causal sequences up to N ~ 4 D^2 M / (D + M) (8192 at
// D = M = 64, 32768 at 128) this form does less work, keeps no D^2 x M
// state, and is bound by the MFMA pipe rather than by HBM.
//
// Forward: a workgroup (4 waves) owns 128 queries (wave w: rows 32w ..
// 32w + 31, two 16-row tiles); key blocks of 64 are staged in LDS, scores
// are computed transposed (S^T = K Q^T, so a lane holds four consecutive keys
// of one query), squared and masked in fp32, rounded to bf16 and fed
// straight to O^T += V^T P^T as the B operand.  The output is normalised by
// the sum of those same rounded weights, so it is an exact convex combination
// of the values (a row with one key reads exactly that key's value, which the
// backward's cancellation relies on); the returned denominator is the sum of
// the fp32 weights.  Every K / V fragment read from LDS serves both query
// tiles of the wave.
#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

using namespace mf;

constexpr int NT = kNT;
constexpr int T = kT;     // keys per block
constexpr int QT = 2;     // 16-row query tiles per wave
constexpr int BQ = 128;   // queries per workgroup (4 waves x QT x 16)

template <int DIM, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void k_poly_fwd(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                    const bf16_t* __restrict__ v, bf16_t* __restrict__ out,
                                                    float* __restrict__ den, int64_t N, int nqb, int64_t BH) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC;
  __shared__ __align__(16) uint16_t sK[T * LD];
  __shared__ __align__(16) uint16_t sV[T * LD];
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // the causal blocks with the most keys go first
  const int64_t bh = blockIdx.x % BH;
  const int qb = CAUSAL ? nqb - 1 - static_cast<int>(blockIdx.x / BH) : static_cast<int>(blockIdx.x / BH);
  const int64_t q0 = static_cast<int64_t>(qb) * BQ;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               ro = make_rsrc(out + hoff, hbytes);
  const int qoff = static_cast<int>(q0 * DIM * 2);

  i16x8 qf[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[qt][s] = __builtin_bit_cast(i16x8, bload16(rq, ((32 * w + 16 * qt + li) * DIM + 8 * g + 32 * s) * 2, qoff));

  f32x4_t o[QT][NTL];
  // sums of the fp32 weights (lane partials) and of the bf16-rounded ones
  // (an MFMA against ones beside O^T: every row of rsum[qt] holds the sum
  // for query li)
  float dacc[QT];
  f32x4_t rsum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    dacc[qt] = 0.f;
    rsum[qt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < NTL; ++n) o[qt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const short one = 0x3f80;  // bf16 1.0
  const i16x8 ones = {one, one, one, one, one, one, one, one};

  const int64_t kend = CAUSAL ? min(N, q0 + BQ) : N;
  const int nkb = static_cast<int>((kend + T - 1) / T);
  i32x4 kraw[PC], vraw[PC];
  auto fetch = [&](int kb) {
    const int soff = kb * T * DIM * 2;
    bload_tile<DIM>(kraw, rk, soff);
    bload_tile<DIM>(vraw, rv, soff);
  };
  fetch(0);
  const int cc = 4 * (li % 4);
  for (int kb = 0; kb < nkb; ++kb) {
    store_tile_v<DIM>(sK, kraw);
    store_tile_v<DIM>(sV, vraw);
    __syncthreads();
    if (kb + 1 < nkb) fetch(kb + 1);
    const int64_t k0 = static_cast<int64_t>(kb) * T;

    // weights P^T[j][i] = (k_j . q_i)^2, masked j <= i
    i16x4 pt[QT][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      i16x8 ka[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[s] = lds8(sK + (16 * t + li) * LD + 8 * g + 32 * s);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int64_t r0 = q0 + 32 * w + 16 * qt;  // first query row of the tile (wave-uniform)
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
        if (!CAUSAL || k0 + 16 * t <= r0 + 15) {
#pragma unroll
          for (int s = 0; s < KS; ++s) acc = mfma(ka[s], qf[qt][s], acc);
          const bool diag = CAUSAL && k0 + 16 * t + 15 > r0;
          // key 16t + 4g + u of the block against query li of the tile, in
          // 32 bits relative to the (wave-uniform) row offset
          const int rel = static_cast<int>(r0 - k0) - 16 * t;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float p = acc[u] * acc[u];
            if (diag) p = (4 * g + u - li <= rel) ? p : 0.f;
            acc[u] = p;
            dacc[qt] += p;
          }
        }
        pt[qt][t] = pack4(acc);
      }
    }
    // O^T += V^T P^T
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const int jr = 32 * tp + 4 * g + li / 4;
#pragma unroll
      for (int n = 0; n < NTL; ++n) {
        const i16x8 a = cat(lds_tr(sV + jr * LD + 16 * n + cc), lds_tr(sV + (jr + 16) * LD + 16 * n + cc));
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int64_t r0 = q0 + 32 * w + 16 * qt;
          if (!CAUSAL || k0 + 32 * tp <= r0 + 15) o[qt][n] = mfma(a, cat(pt[qt][2 * tp], pt[qt][2 * tp + 1]), o[qt][n]);
        }
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int64_t r0 = q0 + 32 * w + 16 * qt;
        if (!CAUSAL || k0 + 32 * tp <= r0 + 15) rsum[qt] = mfma(ones, cat(pt[qt][2 * tp], pt[qt][2 * tp + 1]), rsum[qt]);
      }
    }
    __syncthreads();
  }

  // out = num / den (0 where den = 0); rows past the end are dropped
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float d = shfl_sum_groups(dacc[qt]);
    const float dr = rsum[qt][0];
    const float inv = dr > 0.f ? 1.f / dr : 0.f;
    const int row = 32 * w + 16 * qt + li;
#pragma unroll
    for (int n = 0; n < NTL; ++n) bstore8(ro, pack4(o[qt][n] * inv), (row * DIM + 16 * n + 4 * g) * 2, qoff);
    if (den && g == 0 && q0 + row < N) den[bh * N + q0 + row] = d;
  }
}

// ---------------------------------------------------------------------------
// Backward of L = sum(dout * out), by the chain rule through the masked sum
// (the page gives no gradients).  With s_ij = q_i . k_j, w_ij = s_ij^2:
//   g_i = dout_i / den_i,  c_i = -(dout_i . out_i) / den_i,
//   dS_ij = 2 s_ij (g_i . v_j + c_i)  (masked),
//   dq_i = sum_j dS_ij k_j,  dk_j = sum_i dS_ij q_i,  dv_j = sum_i w_ij g_i;
// rows with den_i = 0 have g_i = c_i = 0.  Two sweeps, no atomics: dq by
// query blocks (recomputing s and g.v per key block; it also leaves c_i for
// the second sweep), dk and dv by key blocks (recomputing s and g.v per
// query block).  g is rounded to bf16 once per row and used by both, and c_i
// is formed from that same rounded g (c_i = -g_i . out_i), so that
// g_i . v_j + c_i = g_i . (v_j - out_i) cancels exactly where the exact
// gradient vanishes (a row whose weight sits on one key).
// ---------------------------------------------------------------------------

// 16-row tiles per wave in the backward sweeps: two at D = 64, one at D = 128
// (two would not fit the accumulators in registers).
__host__ __device__ constexpr int poly_bwd_tiles(int dim) { return dim == 64 ? 2 : 1; }

// bf16 g row pieces: dout features 8g' + 32s .. + 7 of one row, times inv.
template <int DIM>
__device__ __forceinline__ i16x8 scale8(i32x4 raw, float inv) {
  return pack8(unpack8(__builtin_bit_cast(i16x8, raw)) * inv);
}

template <int DIM, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void k_poly_dq(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                   const bf16_t* __restrict__ v, const bf16_t* __restrict__ out,
                                                   const bf16_t* __restrict__ dout, const float* __restrict__ den,
                                                   bf16_t* __restrict__ dq, float* __restrict__ cvec, int64_t N,
                                                   int nqb, int64_t BH) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC;
  constexpr int QTD = poly_bwd_tiles(DIM), BQD = 64 * QTD;
  __shared__ __align__(16) uint16_t sK[T * LD];
  __shared__ __align__(16) uint16_t sV[T * LD];
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x % BH;
  const int qb = CAUSAL ? nqb - 1 - static_cast<int>(blockIdx.x / BH) : static_cast<int>(blockIdx.x / BH);
  const int64_t q0 = static_cast<int64_t>(qb) * BQD;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               ro = make_rsrc(out + hoff, hbytes), rg = make_rsrc(dout + hoff, hbytes),
               rdq = make_rsrc(dq + hoff, hbytes), rden = make_rsrc(den + bh * N, N * 4);
  const int qoff = static_cast<int>(q0 * DIM * 2);

  // this lane's rows: q, g = dout / den (bf16), c = -(dout . out) / den
  i16x8 qf[QTD][KS], gf[QTD][KS];
  float cq[QTD];
#pragma unroll
  for (int qt = 0; qt < QTD; ++qt) {
    const int row = 16 * QTD * w + 16 * qt + li;
    const float d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rden, row * 4, static_cast<int>(q0 * 4), 0));
    const float inv = d > 0.f ? 1.f / d : 0.f;
    float dot = 0.f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = (row * DIM + 8 * g + 32 * s) * 2;
      qf[qt][s] = __builtin_bit_cast(i16x8, bload16(rq, off, qoff));
      gf[qt][s] = scale8<DIM>(bload16(rg, off, qoff), inv);
      const f32x8_t gv = unpack8(gf[qt][s]);
      const f32x8_t ov = unpack8(__builtin_bit_cast(i16x8, bload16(ro, off, qoff)));
#pragma unroll
      for (int e = 0; e < 8; ++e) dot += gv[e] * ov[e];
    }
    cq[qt] = -shfl_sum_groups(dot);
    if (g == 0 && q0 + row < N) cvec[bh * N + q0 + row] = cq[qt];
  }

  f32x4_t o[QTD][NTL];
#pragma unroll
  for (int qt = 0; qt < QTD; ++qt)
#pragma unroll
    for (int n = 0; n < NTL; ++n) o[qt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int64_t kend = CAUSAL ? min(N, q0 + BQD) : N;
  const int nkb = static_cast<int>((kend + T - 1) / T);
  i32x4 kraw[PC], vraw[PC];
  auto fetch = [&](int kb) {
    const int soff = kb * T * DIM * 2;
    bload_tile<DIM>(kraw, rk, soff);
    bload_tile<DIM>(vraw, rv, soff);
  };
  fetch(0);
  const int cc = 4 * (li % 4);
  for (int kb = 0; kb < nkb; ++kb) {
    store_tile_v<DIM>(sK, kraw);
    store_tile_v<DIM>(sV, vraw);
    __syncthreads();
    if (kb + 1 < nkb) fetch(kb + 1);
    const int64_t k0 = static_cast<int64_t>(kb) * T;
    // dS^T[j][i] = 2 s (v_j . g_i + c_i), masked j <= i
    i16x4 dt[QTD][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      i16x8 ka[KS], va[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        ka[s] = lds8(sK + (16 * t + li) * LD + 8 * g + 32 * s);
        va[s] = lds8(sV + (16 * t + li) * LD + 8 * g + 32 * s);
      }
#pragma unroll
      for (int qt = 0; qt < QTD; ++qt) {
        const int64_t r0 = q0 + 16 * QTD * w + 16 * qt;
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
        if (!CAUSAL || k0 + 16 * t <= r0 + 15) {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            sc = mfma(ka[s], qf[qt][s], sc);
            dp = mfma(va[s], gf[qt][s], dp);
          }
          const bool diag = CAUSAL && k0 + 16 * t + 15 > r0;
          const int rel = static_cast<int>(r0 - k0) - 16 * t;  // 32-bit mask test, as in k_poly_fwd
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float x = 2.f * sc[u] * (dp[u] + cq[qt]);
            if (diag) x = (4 * g + u - li <= rel) ? x : 0.f;
            sc[u] = x;
          }
        }
        dt[qt][t] = pack4(sc);
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const int jr = 32 * tp + 4 * g + li / 4;
#pragma unroll
      for (int n = 0; n < NTL; ++n) {
        const i16x8 a = cat(lds_tr(sK + jr * LD + 16 * n + cc), lds_tr(sK + (jr + 16) * LD + 16 * n + cc));
#pragma unroll
        for (int qt = 0; qt < QTD; ++qt) {
          const int64_t r0 = q0 + 16 * QTD * w + 16 * qt;
          if (!CAUSAL || k0 + 32 * tp <= r0 + 15) o[qt][n] = mfma(a, cat(dt[qt][2 * tp], dt[qt][2 * tp + 1]), o[qt][n]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int qt = 0; qt < QTD; ++qt) {
    const int row = 16 * QTD * w + 16 * qt + li;
#pragma unroll
    for (int n = 0; n < NTL; ++n) bstore8(rdq, pack4(o[qt][n]), (row * DIM + 16 * n + 4 * g) * 2, qoff);
  }
}

// Key-block sweep: a workgroup owns 64 KT keys (wave w: KT 16-key tiles, k
// and v as B operands in registers); query blocks of 64 (q, g and c staged in
// LDS) from the diagonal to the end.

template <int DIM, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void k_poly_dkdv(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                                                     const float* __restrict__ den, const float* __restrict__ cvec,
                                                     bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, int64_t N,
                                                     int64_t BH) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, ROW8 = G::ROW8;
  constexpr int KT = poly_bwd_tiles(DIM), BKD = 64 * KT;
  __shared__ __align__(16) uint16_t sQ[T * LD];
  __shared__ __align__(16) uint16_t sG[T * LD];
  __shared__ __align__(16) float sC[T];
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x % BH;
  const int64_t k0 = static_cast<int64_t>(blockIdx.x / BH) * BKD;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               rg = make_rsrc(dout + hoff, hbytes), rdk = make_rsrc(dk + hoff, hbytes),
               rdv = make_rsrc(dv + hoff, hbytes), rden = make_rsrc(den + bh * N, N * 4),
               rc = make_rsrc(cvec + bh * N, N * 4);
  const int koff = static_cast<int>(k0 * DIM * 2);
  i16x8 kf[KT][KS], vf[KT][KS];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int off = ((16 * KT * w + 16 * kt + li) * DIM + 8 * g + 32 * s) * 2;
      kf[kt][s] = __builtin_bit_cast(i16x8, bload16(rk, off, koff));
      vf[kt][s] = __builtin_bit_cast(i16x8, bload16(rv, off, koff));
    }
  f32x4_t ak[KT][NTL], av[KT][NTL];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt)
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
      ak[kt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      av[kt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

  const int64_t qbeg = CAUSAL ? (k0 / T) * T : 0;
  const int nqblk = static_cast<int>((N - qbeg + T - 1) / T);
  i32x4 qraw[PC], graw[PC];
  float dinv[PC], cval = 0.f;
  auto fetch = [&](int64_t i0) {
    const int soff = static_cast<int>(i0 * DIM * 2);
    bload_tile<DIM>(qraw, rq, soff);
    bload_tile<DIM>(graw, rg, soff);
#pragma unroll
    for (int r = 0; r < PC; ++r) {
      const int row = (tid + NT * r) / ROW8;
      const float d = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rden, row * 4, static_cast<int>(i0 * 4), 0));
      dinv[r] = d > 0.f ? 1.f / d : 0.f;
    }
    if (tid < T) cval = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rc, tid * 4, static_cast<int>(i0 * 4), 0));
  };
  fetch(qbeg);
  const int cc = 4 * (li % 4);
  for (int qi = 0; qi < nqblk; ++qi) {
    const int64_t i0 = qbeg + static_cast<int64_t>(qi) * T;
    store_tile_v<DIM>(sQ, qraw);
#pragma unroll
    for (int r = 0; r < PC; ++r) {
      const int p = tid + NT * r;
      *reinterpret_cast<i16x8*>(sG + (p / ROW8) * LD + (p % ROW8) * 8) = scale8<DIM>(graw[r], dinv[r]);
    }
    if (tid < T) sC[tid] = cval;
    __syncthreads();
    if (qi + 1 < nqblk) fetch(i0 + T);
    // P[i][j] = s^2, dS[i][j] = 2 s (g_i . v_j + c_i), masked i >= j
    i16x4 pm[KT][4], dm[KT][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      i16x8 qa[KS], ga[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        qa[s] = lds8(sQ + (16 * t + li) * LD + 8 * g + 32 * s);
        ga[s] = lds8(sG + (16 * t + li) * LD + 8 * g + 32 * s);
      }
      const f32x4_t cv = *reinterpret_cast<const f32x4_t*>(sC + 16 * t + 4 * g);
#pragma unroll
      for (int kt = 0; kt < KT; ++kt) {
        const int64_t j0 = k0 + 16 * KT * w + 16 * kt;  // first key of the tile (wave-uniform)
        f32x4_t sc = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
        if (!CAUSAL || i0 + 16 * t + 15 >= j0) {
#pragma unroll
          for (int s = 0; s < KS; ++s) {
            sc = mfma(qa[s], kf[kt][s], sc);
            dp = mfma(ga[s], vf[kt][s], dp);
          }
          const bool diag = CAUSAL && i0 + 16 * t < j0 + 15;
          // query 16t + 4g + u of the block against key li of the tile, in
          // 32 bits relative to the (wave-uniform) offset
          const int rel = static_cast<int>(j0 - i0) - 16 * t;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float pw = sc[u] * sc[u];
            float x = 2.f * sc[u] * (dp[u] + cv[u]);
            if (diag && 4 * g + u - li < rel) {
              pw = 0.f;
              x = 0.f;
            }
            sc[u] = pw;
            dp[u] = x;
          }
        }
        pm[kt][t] = pack4(sc);
        dm[kt][t] = pack4(dp);
      }
    }
    // dV^T += G^T P, dK^T += Q^T dS
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      const int ir = 32 * tp + 4 * g + li / 4;
#pragma unroll
      for (int n = 0; n < NTL; ++n) {
        const i16x8 ga = cat(lds_tr(sG + ir * LD + 16 * n + cc), lds_tr(sG + (ir + 16) * LD + 16 * n + cc));
        const i16x8 qa = cat(lds_tr(sQ + ir * LD + 16 * n + cc), lds_tr(sQ + (ir + 16) * LD + 16 * n + cc));
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const int64_t j0 = k0 + 16 * KT * w + 16 * kt;
          if (!CAUSAL || i0 + 32 * tp + 31 >= j0) {
            av[kt][n] = mfma(ga, cat(pm[kt][2 * tp], pm[kt][2 * tp + 1]), av[kt][n]);
            ak[kt][n] = mfma(qa, cat(dm[kt][2 * tp], dm[kt][2 * tp + 1]), ak[kt][n]);
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int row = 16 * KT * w + 16 * kt + li;
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
      bstore8(rdk, pack4(ak[kt][n]), (row * DIM + 16 * n + 4 * g) * 2, koff);
      bstore8(rdv, pack4(av[kt][n]), (row * DIM + 16 * n + 4 * g) * 2, koff);
    }
  }
}

// ---------------------------------------------------------------------------
// The linear form's state after a prefix: S[c][m] = sum_t phi(k_t)_c v_t[m],
// Z[c] = sum_t phi(k_t)_c, c = a D + b, phi(k)_c = k_a k_b (D^2 x M fp32 per
// head, the recurrence's S_N, Z_N).  A workgroup owns the 64 rows
// c = a D + b0 .. a D + b0 + 63 (wave w: 16 of them) for all M columns; per
// 64-token chunk the A operand phi(K)^T[c][t] is the transposed K fragment
// of columns b scaled by k_t[a] (one bf16 rounding), V the B operand; Z sums
// the same products in fp32.
// ---------------------------------------------------------------------------
template <int DIM>
__global__ __launch_bounds__(NT, 2) void k_poly_state(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                      float* __restrict__ S, float* __restrict__ Z, int64_t N) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, PC = G::PC;
  constexpr int NB = DIM / 64;  // workgroups per value of a
  __shared__ __align__(16) uint16_t sK[T * LD];
  __shared__ __align__(16) uint16_t sV[T * LD];
  __shared__ __align__(16) float sKa[T];
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / (DIM * NB);
  const int rem = static_cast<int>(blockIdx.x % (DIM * NB));
  const int a = rem / NB, b0 = (rem % NB) * 64;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rk = make_rsrc(k + bh * N * DIM, hbytes), rv = make_rsrc(v + bh * N * DIM, hbytes);
  f32x4_t acc[NTL];
#pragma unroll
  for (int n = 0; n < NTL; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;
  const int nch = static_cast<int>((N + T - 1) / T);
  i32x4 kraw[PC], vraw[PC];
  auto fetch = [&](int c) {
    bload_tile<DIM>(kraw, rk, c * T * DIM * 2);
    bload_tile<DIM>(vraw, rv, c * T * DIM * 2);
  };
  fetch(0);
  const int cc = 4 * (li % 4);
  for (int c = 0; c < nch; ++c) {
    store_tile_v<DIM>(sK, kraw);
    store_tile_v<DIM>(sV, vraw);
    __syncthreads();
    if (tid < T) sKa[tid] = fb(static_cast<short>(sK[tid * LD + a]));
    if (c + 1 < nch) fetch(c + 1);
    __syncthreads();
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      const int jr = 32 * s + 8 * g + li / 4;
      const int col = b0 + 16 * w + cc;
      const f32x8_t kt = unpack8(cat(lds_tr(sK + jr * LD + col), lds_tr(sK + (jr + 4) * LD + col)));
      const f32x4_t ka0 = *reinterpret_cast<const f32x4_t*>(sKa + 32 * s + 8 * g);
      const f32x4_t ka1 = *reinterpret_cast<const f32x4_t*>(sKa + 32 * s + 8 * g + 4);
      f32x8_t ph;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ph[e] = kt[e] * ka0[e];
        ph[e + 4] = kt[e + 4] * ka1[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) zacc += ph[e];
      const i16x8 af = pack8(ph);
#pragma unroll
      for (int n = 0; n < NTL; ++n) {
        const i16x8 bb = cat(lds_tr(sV + jr * LD + 16 * n + cc), lds_tr(sV + (jr + 4) * LD + 16 * n + cc));
        acc[n] = mfma(af, bb, acc[n]);
      }
    }
    __syncthreads();
  }
  const int64_t C = static_cast<int64_t>(DIM) * DIM;
  float* Sh = S + bh * C * DIM;
  const int64_t crow = static_cast<int64_t>(a) * DIM + b0 + 16 * w;
#pragma unroll
  for (int n = 0; n < NTL; ++n)
#pragma unroll
    for (int u = 0; u < 4; ++u) Sh[(crow + 4 * g + u) * DIM + 16 * n + li] = acc[n][u];
  zacc = shfl_sum_groups(zacc);
  if (g == 0) Z[bh * C + crow + li] = zacc;
}

}  // namespace

int poly_supported(int64_t D, int64_t M, int dtype) { return dtype == 1 && D == M && (D == 64 || D == 128); }

hipError_t launch_poly_forward(int64_t BH, int64_t N, int D, const void* q, const void* k, const void* v, void* out,
                               float* den, int causal, hipStream_t st) {
  const int nqb = static_cast<int>((N + BQ - 1) / BQ);
  const dim3 grid(static_cast<unsigned>(BH * nqb)), block(NT);
  const bf16_t* Q = static_cast<const bf16_t*>(q);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  bf16_t* O = static_cast<bf16_t*>(out);
#define LA_PFWD(DIMV, C) hipLaunchKernelGGL((k_poly_fwd<DIMV, C>), grid, block, 0, st, Q, K, V, O, den, N, nqb, BH)
  if (D == 64) {
    if (causal) LA_PFWD(64, true); else LA_PFWD(64, false);
  } else if (D == 128) {
    if (causal) LA_PFWD(128, true); else LA_PFWD(128, false);
  } else {
    return hipErrorNotSupported;
  }
#undef LA_PFWD
  return hipGetLastError();
}

}  // namespace la

namespace la {

hipError_t launch_poly_state(int64_t BH, int64_t N, int D, const void* k, const void* v, float* S, float* Z,
                             hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(BH * D * (D / 64))), block(NT);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  if (D == 64)
    hipLaunchKernelGGL((k_poly_state<64>), grid, block, 0, st, K, V, S, Z, N);
  else if (D == 128)
    hipLaunchKernelGGL((k_poly_state<128>), grid, block, 0, st, K, V, S, Z, N);
  else
    return hipErrorNotSupported;
  return hipGetLastError();
}

hipError_t launch_poly_bwd(int pass, int64_t BH, int64_t N, int D, const void* q, const void* k, const void* v,
                           const void* out, const void* dout, const float* den, void* dq, void* dk, void* dv,
                           float* cvec, int causal, hipStream_t st) {
  // pass 0: the dq sweep (also writes c); pass 1: the dk / dv sweep
  const int bq = 64 * poly_bwd_tiles(D);
  const int nb = static_cast<int>((N + bq - 1) / bq);
  const dim3 grid(static_cast<unsigned>(BH * nb)), block(NT);
  const bf16_t* Q = static_cast<const bf16_t*>(q);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  const bf16_t* O = static_cast<const bf16_t*>(out);
  const bf16_t* dO = static_cast<const bf16_t*>(dout);
  bf16_t* dQ = static_cast<bf16_t*>(dq);
  bf16_t* dK = static_cast<bf16_t*>(dk);
  bf16_t* dV = static_cast<bf16_t*>(dv);
#define LA_PBWD(DIMV, C)                                                                                     \
  do {                                                                                                       \
    if (pass == 0)                                                                                           \
      hipLaunchKernelGGL((k_poly_dq<DIMV, C>), grid, block, 0, st, Q, K, V, O, dO, den, dQ, cvec, N, nb, BH); \
    else                                                                                                     \
      hipLaunchKernelGGL((k_poly_dkdv<DIMV, C>), grid, block, 0, st, Q, K, V, dO, den, cvec, dK, dV, N, BH); \
  } while (0)
  if (D == 64) {
    if (causal) LA_PBWD(64, true); else LA_PBWD(64, false);
  } else if (D == 128) {
    if (causal) LA_PBWD(128, true); else LA_PBWD(128, false);
  } else {
    return hipErrorNotSupported;
  }
#undef LA_PBWD
  return hipGetLastError();
}

}  // namespace la
