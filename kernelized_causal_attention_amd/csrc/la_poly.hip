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
// straight to O^T += V^T P^T as the B operand; the row sums of the fp32
// weights give the denominator.  Every K / V fragment read from LDS serves
// both query tiles of the wave.
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
  float dacc[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    dacc[qt] = 0.f;
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
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float p = acc[u] * acc[u];
            if (diag) p = (k0 + 16 * t + 4 * g + u <= r0 + li) ? p : 0.f;
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
    }
    __syncthreads();
  }

  // out = num / den (0 where den = 0); rows past the end are dropped
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float d = shfl_sum_groups(dacc[qt]);
    const float inv = d > 0.f ? 1.f / d : 0.f;
    const int row = 32 * w + 16 * qt + li;
#pragma unroll
    for (int n = 0; n < NTL; ++n) bstore8(ro, pack4(o[qt][n] * inv), (row * DIM + 16 * n + 4 * g) * 2, qoff);
    if (den && g == 0 && q0 + row < N) den[bh * N + q0 + row] = d;
  }
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
