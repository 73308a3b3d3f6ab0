// Softmax attention on gfx950, the comparison baseline: a blockwise
// (online-softmax) forward on bf16 MFMA and a KV-cache decode step.
//
// "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io), section
// 1, eq:softmax: out = softmax(Q K^T / sqrt(D)) V, causal per eq:mask.
// "Transformer study notes (4)" (developer.cloud.tencent.cn), section
// "FlashAttention": per block of scores s^(b) with values V^(b), the running
// maximum m, the denominator l and the unnormalised sum a are updated as
//   m' = max(m, max_j s_j),  r = exp(m - m'),
//   l' = r l + sum_j exp(s_j - m'),  a' = r a + sum_j exp(s_j - m') v_j,
// and out = a / l after the last block.
//
// Forward: the same blocking as the polynomial-kernel forward (128 queries
// per workgroup, two 16-row tiles per wave, 64-key blocks in LDS, transposed
// scores feeding O^T += V^T P^T).  A lane holds four consecutive keys of one
// query per tile, so a row's block maximum is an in-lane max over its 16
// raw scores and two cross-lane steps, and the rescale multiplies that
// lane's output column directly.  Each weight is one FMA and one hardware
// exp2: exp2((s - m) log2(e) / sqrt(D)).  The reference maximum m of a row
// moves only when a block raises it by more than kSlack (in log2 units):
// the weights then stay <= 2^kSlack, harmless in bf16 and fp32, and the
// rescale of the output (a wave-uniform decision) is skipped for most
// blocks.  Any common reference gives the same quotient a / l.
#include "la_device.h"
#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

using namespace mf;

constexpr int NT = kNT;
constexpr int T = kT;
constexpr int QT = 2;
constexpr int BQ = 128;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kSlack = 8.f;  // log2 of the largest weight allowed before m moves

// 2^x on the hardware unit (no denormal range reduction: every argument here
// is <= kSlack, and results below 2^-126 are weights that do not matter).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float max_groups(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

template <int DIM, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void k_sm_fwd(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                  const bf16_t* __restrict__ v, bf16_t* __restrict__ out,
                                                  float* __restrict__ lse, int64_t N, int nqb, int64_t BH,
                                                  float scale2) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC;
  __shared__ __align__(16) uint16_t sK[T * LD];
  __shared__ __align__(16) uint16_t sV[T * LD];
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  float mrow[QT], lsum[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    mrow[qt] = kNegInf;
    lsum[qt] = 0.f;
#pragma unroll
    for (int n = 0; n < NTL; ++n) o[qt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

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
    // raw scores s^T[j][i], masked entries -inf
    f32x4_t sc[QT][4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      i16x8 ka[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) ka[s] = lds8(sK + (16 * t + li) * LD + 8 * g + 32 * s);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int64_t r0 = q0 + 32 * w + 16 * qt;
        f32x4_t acc = {kNegInf, kNegInf, kNegInf, kNegInf};
        if (!CAUSAL || k0 + 16 * t <= r0 + 15) {
          f32x4_t x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) x = mfma(ka[s], qf[qt][s], x);
          const bool diag = CAUSAL && k0 + 16 * t + 15 > r0;
          const bool tail = !CAUSAL && k0 + 16 * t + 15 >= N;
          // key 16t + 4g + u of the block, tested in 32 bits against the
          // (wave-uniform) query offset and the keys left in the head
          const int rd = static_cast<int>(r0 - k0);
          const int rn = static_cast<int>(min(N - k0, static_cast<int64_t>(1) << 30));
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int jr = 16 * t + 4 * g + u;
            const bool keep = (!diag || jr <= rd + li) && (!tail || jr < rn);
            acc[u] = keep ? x[u] : kNegInf;
          }
        }
        sc[qt][t] = acc;
      }
    }
    // running maximum, rescale, weights
    i16x4 pt[QT][4];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float mb = kNegInf;
#pragma unroll
      for (int t = 0; t < 4; ++t) mb = fmaxf(mb, fmaxf(fmaxf(sc[qt][t][0], sc[qt][t][1]), fmaxf(sc[qt][t][2], sc[qt][t][3])));
      const float mcand = fmaxf(mrow[qt], max_groups(mb));
      // move the reference only when some row of the wave outgrows it
      if (__any((mcand - mrow[qt]) * scale2 > kSlack)) {
        // a row whose keys so far are all masked keeps m = -inf and r = 0
        const float r = mcand == kNegInf ? 1.f : exp2_hw((mrow[qt] - mcand) * scale2);
        mrow[qt] = mcand;
        lsum[qt] *= r;
#pragma unroll
        for (int n = 0; n < NTL; ++n) o[qt][n] *= r;
      }
      const float msc = mrow[qt] == kNegInf ? 0.f : -mrow[qt] * scale2;
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4_t p;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          p[u] = exp2_hw(__builtin_fmaf(sc[qt][t][u], scale2, msc));
          ps += p[u];
        }
        pt[qt][t] = pack4(p);
      }
      lsum[qt] += ps;
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
    }
    __syncthreads();
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = shfl_sum_groups(lsum[qt]);
    const float inv = 1.f / lt;
    const int row = 32 * w + 16 * qt + li;
#pragma unroll
    for (int n = 0; n < NTL; ++n) bstore8(ro, pack4(o[qt][n] * inv), (row * DIM + 16 * n + 4 * g) * 2, qoff);
    if (lse && g == 0 && q0 + row < N)
      lse[bh * N + q0 + row] = mrow[qt] * scale2 * 0.69314718055994531f + __logf(lt);
  }
}

// ---------------------------------------------------------------------------
// KV-cache decode step ("The deep link between Transformer and RNN",
// section 3): append (k, v) at position L of each head's cache, then attend
// with q over positions 0 .. L.  HBM-bound: every step reads the whole cache
// (L (D + M) elements per head).  One workgroup per head; the L cached keys
// are split across the four waves in contiguous runs; a wave takes 16 keys
// per pass, four lanes per key (each a quarter of the features), reduces the
// partial dot products across the four lanes, and keeps a wave-uniform
// running maximum, so every lane's partial weighted sum (its quarter of the
// value columns, for the keys of its lane slot) is on one scale.  The new
// token's (score, value) is folded in at the end from registers -- it is
// written to the cache but never read back within the step.
// ---------------------------------------------------------------------------
// CNT consecutive elements (16-byte aligned, CNT * size a multiple of 16
// bytes) as fp32, in 16-byte loads.
template <int CNT>
__device__ __forceinline__ void load_row(float (&dst)[CNT], const float* p) {
#pragma unroll
  for (int c = 0; c < CNT / 4; ++c) {
    const f32x4_t x = *reinterpret_cast<const f32x4_t*>(p + 4 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[4 * c + e] = x[e];
  }
}
template <int CNT>
__device__ __forceinline__ void load_row(float (&dst)[CNT], const bf16_t* p) {
#pragma unroll
  for (int c = 0; c < CNT / 8; ++c) {
    const f32x8_t x = unpack8(*reinterpret_cast<const i16x8*>(p + 8 * c));
#pragma unroll
    for (int e = 0; e < 8; ++e) dst[8 * c + e] = x[e];
  }
}

template <typename TIn, int DIM>
__global__ __launch_bounds__(NT) void k_sm_decode(TIn* __restrict__ kc, TIn* __restrict__ vc,
                                                  const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                  const TIn* __restrict__ v, TIn* __restrict__ out, int64_t L,
                                                  int64_t cap, float scale2) {
  constexpr int DQ = DIM / 4;  // features per lane
  __shared__ float sq[DIM], sk[DIM], sv[DIM];
  __shared__ float wm[4], wl[4], wa[4][DIM];
  const int tid = threadIdx.x, l = tid & 63;
  const int w = tid >> 6;
  const int kq = l >> 2, part = l & 3;
  const int64_t bh = blockIdx.x;
  TIn* kh = kc + bh * cap * DIM;
  TIn* vh = vc + bh * cap * DIM;
  for (int d = tid; d < DIM; d += NT) {
    sq[d] = ld(q, bh * DIM + d);
    sk[d] = ld(k, bh * DIM + d);
    sv[d] = ld(v, bh * DIM + d);
    // append the new token (read back by later steps only)
    kh[L * DIM + d] = k[bh * DIM + d];
    vh[L * DIM + d] = v[bh * DIM + d];
  }
  __syncthreads();
  float qv[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) qv[e] = sq[part * DQ + e];
  float m = kNegInf, ls = 0.f, acc[DQ];
#pragma unroll
  for (int e = 0; e < DQ; ++e) acc[e] = 0.f;
  const int64_t per = ((L + 3) / 4 + 15) / 16 * 16;
  const int64_t jb = w * per, je = min(L, jb + per);
  for (int64_t j0 = jb; j0 < je; j0 += 16) {
    const int64_t j = j0 + kq;
    const bool live = j < je;
    float s = 0.f, vv[DQ];
    if (live) {
      float kk[DQ];
      load_row<DQ>(kk, kh + j * DIM + part * DQ);
      load_row<DQ>(vv, vh + j * DIM + part * DQ);
#pragma unroll
      for (int e = 0; e < DQ; ++e) s += qv[e] * kk[e];
    } else {
#pragma unroll
      for (int e = 0; e < DQ; ++e) vv[e] = 0.f;
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    const float s2 = live ? s * scale2 : kNegInf;
    float mb = s2;
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) mb = fmaxf(mb, __shfl_xor(mb, off, 64));
    const float mnew = fmaxf(m, mb);  // finite: key j0 is live
    const float r = exp2_hw(m - mnew);
    const float p = exp2_hw(s2 - mnew);
    float psum = p;
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) psum += __shfl_xor(psum, off, 64);
    ls = ls * r + psum;
#pragma unroll
    for (int e = 0; e < DQ; ++e) acc[e] = acc[e] * r + p * vv[e];
    m = mnew;
  }
  // this wave's (m, l, a): a summed over the 16 lane slots with the same part
#pragma unroll
  for (int e = 0; e < DQ; ++e) {
    float x = acc[e];
#pragma unroll
    for (int off = 4; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    acc[e] = x;
  }
  if (l < 4) {
#pragma unroll
    for (int e = 0; e < DQ; ++e) wa[w][part * DQ + e] = acc[e];
  }
  if (l == 0) {
    wm[w] = m;
    wl[w] = ls;
  }
  __syncthreads();
  // combine the waves and the new token (score from LDS, in fixed order)
  if (tid < 64) {
    float sn = 0.f;
    for (int d = l; d < DIM; d += 64) sn += sq[d] * sk[d];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sn += __shfl_xor(sn, off, 64);
    const float s2n = sn * scale2;
    const float mt = fmaxf(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3])), s2n);
    float f[4], lt = exp2_hw(s2n - mt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f[u] = exp2_hw(wm[u] - mt);
      lt += f[u] * wl[u];
    }
    const float inv = 1.f / lt, fn = exp2_hw(s2n - mt);
    for (int c = l; c < DIM; c += 64) {
      const float a = ((f[0] * wa[0][c] + f[1] * wa[1][c]) + (f[2] * wa[2][c] + f[3] * wa[3][c])) + fn * sv[c];
      st(out, bh * DIM + c, a * inv);
    }
  }
}

}  // namespace

int softmax_supported(int64_t D, int64_t M, int dtype) { return dtype == 1 && D == M && (D == 64 || D == 128); }

hipError_t launch_softmax_forward(int64_t BH, int64_t N, int D, const void* q, const void* k, const void* v,
                                  void* out, float* lse, int causal, hipStream_t st) {
  const int nqb = static_cast<int>((N + BQ - 1) / BQ);
  const dim3 grid(static_cast<unsigned>(BH * nqb)), block(NT);
  const float scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
  const bf16_t* Q = static_cast<const bf16_t*>(q);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  bf16_t* O = static_cast<bf16_t*>(out);
#define LA_SFWD(DIMV, C) \
  hipLaunchKernelGGL((k_sm_fwd<DIMV, C>), grid, block, 0, st, Q, K, V, O, lse, N, nqb, BH, scale2)
  if (D == 64) {
    if (causal) LA_SFWD(64, true); else LA_SFWD(64, false);
  } else if (D == 128) {
    if (causal) LA_SFWD(128, true); else LA_SFWD(128, false);
  } else {
    return hipErrorNotSupported;
  }
#undef LA_SFWD
  return hipGetLastError();
}

hipError_t launch_softmax_decode(int dtype, int64_t BH, int D, void* kc, void* vc, const void* q, const void* k,
                                 const void* v, void* out, int64_t L, int64_t cap, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(BH)), block(NT);
  const float scale2 = 1.4426950408889634f / sqrtf(static_cast<float>(D));
#define LA_SDEC(TT, DIMV)                                                                                      \
  hipLaunchKernelGGL((k_sm_decode<TT, DIMV>), grid, block, 0, st, static_cast<TT*>(kc), static_cast<TT*>(vc), \
                     static_cast<const TT*>(q), static_cast<const TT*>(k), static_cast<const TT*>(v),         \
                     static_cast<TT*>(out), L, cap, scale2)
  if (dtype == 0) {
    if (D == 64) LA_SDEC(float, 64); else if (D == 128) LA_SDEC(float, 128); else return hipErrorNotSupported;
  } else {
    if (D == 64) LA_SDEC(bf16_t, 64); else if (D == 128) LA_SDEC(bf16_t, 128); else return hipErrorNotSupported;
  }
#undef LA_SDEC
  return hipGetLastError();
}

}  // namespace la
