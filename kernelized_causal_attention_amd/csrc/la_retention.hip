// Decayed / gated linear attention ("retention") on gfx950: bf16 MFMA
// kernels, D = M in {64, 128}.
//
// "08 - Transformer and Variants" (by-xin.github.io), section 1.3.4: RetNet
// keeps H_t = gamma H_{t-1} + v_t k_t^T and reads y_t = H_t q_t; gated
// retention makes gamma_t time-varying.  As printed, there is no feature
// map and no normaliser.  The state is kept as S = H^T ([D][M], the same
// orientation as the linear-attention state): S_t = gamma_t S_{t-1} + k_t
// v_t^T, y_t = S_t^T q_t.  The gate enters as log gamma_t <= 0 per token.
//
// Chunked form (T = 64 tokens; b_i = sum of log gamma over the chunk's
// tokens up to and including i; S the state before the chunk):
//   y_i   = exp(b_i) S^T q_i + sum_{j <= i in chunk} exp(b_i - b_j)(q_i.k_j) v_j
//   S_new = exp(b_T) S + sum_j exp(b_T - b_j) k_j v_j^T
// Every exponent is <= 0, so no factor overflows whatever the gates.  b is
// an inclusive scan over the chunk's 64 tokens done in each wave's lanes.
// Segments: a segment's aggregate is its own S_new from zero and the sum of
// its log gammas, Lambda; the carry into segment p is the decayed scan
// C_{p+1} = exp(Lambda_p) C_p + dS_p, starting from the carried-in S0.
#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

using namespace mf;

constexpr int NT = kNT;
constexpr int T = kT;

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int l = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(x, off, 64);
    if (l >= off) x += y;
  }
  return x;
}

// log gamma of token cc0 + l (zero past the head's end: no decay there);
// values below -80 are taken as -80 (gamma ~ 2e-35, i.e. 0) so that a full
// reset never forms -inf - (-inf); NaN passes through.
__device__ __forceinline__ float gate(rsrc_t rl, int l, int64_t cc0) {
  const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, l * 4, static_cast<int>(cc0 * 4), 0));
  return x < -80.f ? -80.f : x;
}

// Registers -> LDS with each row scaled: row j of the tile times f(j), where
// the staging thread gets b_j from its own wave's scan (lanes hold b_0..b_63).
template <int DIM>
__device__ __forceinline__ void store_tile_scaled(uint16_t* lds, const i32x4 (&raw)[Geo<DIM>::PC], float b,
                                                  float bT) {
  using G = Geo<DIM>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + NT * r;
    const int j = p / G::ROW8, c8 = p % G::ROW8;
    const float s = __expf(bT - __shfl(b, j, 64));
    *reinterpret_cast<i16x8*>(lds + j * G::LD + c8 * 8) = pack8(unpack8(__builtin_bit_cast(i16x8, raw[r])) * s);
  }
}

// S (fp32, this wave's DT row tiles of the state) and its bf16 S^T copy.
template <int DIM>
__device__ __forceinline__ void write_st(uint16_t* sST, const f32x4_t (&Sacc)[Geo<DIM>::DT][Geo<DIM>::NTL], int w,
                                         int g, int li) {
  using G = Geo<DIM>;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    const int d0 = 16 * (w * G::DT + dt);
#pragma unroll
    for (int n = 0; n < G::NTL; ++n)
      *reinterpret_cast<i16x4*>(sST + (16 * n + li) * G::LD + d0 + 4 * g) = pack4(Sacc[dt][n]);
  }
}

// Sacc[dt][n] holds S[d0 + 4g + u][16n + li], d0 = 16 (w DT + dt).
template <int DIM>
__device__ __forceinline__ void init_s(f32x4_t (&Sacc)[Geo<DIM>::DT][Geo<DIM>::NTL], const float* __restrict__ cs,
                                       int w, int g, int li) {
  using G = Geo<DIM>;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = 16 * (w * G::DT + dt) + 4 * g + u;
#pragma unroll
      for (int n = 0; n < G::NTL; ++n) Sacc[dt][n][u] = cs ? cs[d * DIM + 16 * n + li] : 0.f;
    }
}

// S <- exp(bT) S + Ks^T V  (Ks: the chunk's keys already scaled by
// exp(bT - b_j)).
template <int DIM>
__device__ __forceinline__ void decay_update(f32x4_t (&Sacc)[Geo<DIM>::DT][Geo<DIM>::NTL], float bT,
                                             const uint16_t* sKs, const uint16_t* sV, int w, int g, int li) {
  using G = Geo<DIM>;
  const float dk = __expf(bT);
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt)
#pragma unroll
    for (int n = 0; n < G::NTL; ++n) Sacc[dt][n] *= dk;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    const int d0 = 16 * (w * G::DT + dt);
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      const int jr = 32 * s + 8 * g + li / 4;
      const int cc = 4 * (li % 4);
      const i16x8 a = cat(lds_tr(sKs + jr * G::LD + d0 + cc), lds_tr(sKs + (jr + 4) * G::LD + d0 + cc));
#pragma unroll
      for (int n = 0; n < G::NTL; ++n) {
        const i16x8 bb = cat(lds_tr(sV + jr * G::LD + 16 * n + cc), lds_tr(sV + (jr + 4) * G::LD + 16 * n + cc));
        Sacc[dt][n] = mfma(a, bb, Sacc[dt][n]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Forward.  Wave w owns query rows 16w .. 16w + 15 of each chunk.  carry:
// this segment's incoming state record (S in its first D*M floats), or null.
// ---------------------------------------------------------------------------
template <int DIM>
__global__ __launch_bounds__(NT, DIM == 64 ? 2 : 1) void k_ret_fwd_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                       const bf16_t* __restrict__ v, const float* __restrict__ lg,
                                                       bf16_t* __restrict__ y, const float* __restrict__ carry,
                                                       int64_t N, int P, int seg_len) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sK = smem;
  uint16_t* sV = sK + T * LD;
  uint16_t* sKs = sV + T * LD;
  uint16_t* sST = sKs + T * LD;

  // w is wave-uniform (an SGPR) so that branches on it are scalar: an MFMA
  // under an EXEC-masked branch still writes every lane.
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  const float* cs = carry ? carry + (bh * P + seg) * E : nullptr;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               ry = make_rsrc(y + hoff, hbytes), rl = make_rsrc(lg + bh * N, N * 4);
  const int i = 16 * w + li;
  // causal mask of key j = 16t + 4g + u against query i, as 0 / 1 factors
  f32x4_t mt[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int u = 0; u < 4; ++u) mt[t][u] = (t < w || (t == w && 4 * g + u <= li)) ? 1.f : 0.f;

  f32x4_t Sacc[DT][NTL];
  init_s<DIM>(Sacc, cs, w, g, li);
  write_st<DIM>(sST, Sacc, w, g, li);

  i32x4 kraw[PC], vraw[PC], qraw[KS];
  float lgv;
  auto fetch = [&](int64_t cc0) {
    const int soff = static_cast<int>(cc0 * DIM * 2);
    bload_tile<DIM>(kraw, rk, soff);
    bload_tile<DIM>(vraw, rv, soff);
    bload_q<DIM>(qraw, rq, soff, i, g);
    // rows past the head's end read as zero: no decay there
    lgv = gate(rl, l, cc0);
  };
  fetch(r0);
  for (int64_t c0 = r0; c0 < r1; c0 += T) {
    const float b = wave_incl_scan(lgv);  // lane l: b_l
    const float bT = __shfl(b, 63, 64);
    store_tile_v<DIM>(sK, kraw);
    store_tile_v<DIM>(sV, vraw);
    store_tile_scaled<DIM>(sKs, kraw, b, bT);
    i16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = __builtin_bit_cast(i16x8, qraw[s]);
    __syncthreads();
    const int soff = static_cast<int>(c0 * DIM * 2);
    if (c0 + T < r1) fetch(c0 + T);

    const float bi = __shfl(b, i, 64);
    // scores A^T[j][i] = (k_j . q_i) exp(b_i - b_j), key tiles t <= w, masked
    i16x4 at[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      at[t] = i16x4{0, 0, 0, 0};
      if (t <= w) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma(lds8(sK + (16 * t + li) * LD + 8 * g + 32 * s), qf[s], acc);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] *= __expf(fminf(bi - __shfl(b, 16 * t + 4 * g + u, 64), 0.f)) * mt[t][u];
        at[t] = pack4(acc);
      }
    }
    // Y^T = exp(b_i) S^T q_i + V^T A^T
    const float di = __expf(bi);
    f32x4_t o[NTL];
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
      o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) o[n] = mfma(lds8(sST + (16 * n + li) * LD + 8 * g + 32 * s), qf[s], o[n]);
      o[n] *= di;
    }
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      if (2 * tp <= w) {
        const i16x8 bb = cat(at[2 * tp], at[2 * tp + 1]);
        const int jr = 32 * tp + 4 * g + li / 4;
        const int cc = 4 * (li % 4);
#pragma unroll
        for (int n = 0; n < NTL; ++n) {
          const i16x8 a = cat(lds_tr(sV + jr * LD + 16 * n + cc), lds_tr(sV + (jr + 16) * LD + 16 * n + cc));
          o[n] = mfma(a, bb, o[n]);
        }
      }
    }
    // rows past the head's end fall outside the buffer range: dropped
#pragma unroll
    for (int n = 0; n < NTL; ++n) bstore8(ry, pack4(o[n]), (i * DIM + 16 * n + 4 * g) * 2, soff);
    decay_update<DIM>(Sacc, bT, sKs, sV, w, g, li);
    __syncthreads();
    write_st<DIM>(sST, Sacc, w, g, li);
  }
}

// Segment aggregates: dS = the segment's state from zero, and Lambda = the
// sum of its log gammas (stored in the record's first Z slot).
template <int DIM>
__global__ __launch_bounds__(NT, 2) void k_ret_seg_state(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                         const float* __restrict__ lg, float* __restrict__ recs,
                                                         int64_t N, int P, int seg_len) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, PC = G::PC, DT = G::DT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sKs = smem;
  uint16_t* sV = sKs + T * LD;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rk = make_rsrc(k + bh * N * DIM, hbytes), rv = make_rsrc(v + bh * N * DIM, hbytes),
               rl = make_rsrc(lg + bh * N, N * 4);
  f32x4_t Sacc[DT][NTL];
  init_s<DIM>(Sacc, nullptr, w, g, li);
  float lam = 0.f;
  i32x4 kraw[PC], vraw[PC];
  float lgv;
  auto fetch = [&](int64_t cc0) {
    bload_tile<DIM>(kraw, rk, static_cast<int>(cc0 * DIM * 2));
    bload_tile<DIM>(vraw, rv, static_cast<int>(cc0 * DIM * 2));
    lgv = gate(rl, l, cc0);
  };
  fetch(r0);
  for (int64_t c0 = r0; c0 < r1; c0 += T) {
    const float b = wave_incl_scan(lgv);
    const float bT = __shfl(b, 63, 64);
    lam += bT;
    store_tile_v<DIM>(sV, vraw);
    store_tile_scaled<DIM>(sKs, kraw, b, bT);
    __syncthreads();
    if (c0 + T < r1) fetch(c0 + T);
    decay_update<DIM>(Sacc, bT, sKs, sV, w, g, li);
    __syncthreads();
  }
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  float* rec = recs + (bh * P + seg) * E;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = 16 * (w * DT + dt) + 4 * g + u;
#pragma unroll
      for (int n = 0; n < NTL; ++n) rec[d * DIM + 16 * n + li] = Sacc[dt][n][u];
    }
  if (tid == 0) rec[DIM * DIM] = lam;
}

// Decayed exclusive scan over segments, in place on the S part of the
// records: C_0 = S0 (or 0), C_{p+1} = exp(Lambda_p) C_p + dS_p; record p
// receives C_p; the total C_P goes to tot (when not null; tot may be S0).
__global__ __launch_bounds__(NT) void k_ret_scan(float* __restrict__ recs, int P, int64_t E, int64_t DM, int64_t nb,
                                                 const float* init, float* tot) {
  const int64_t bh = blockIdx.x / nb;
  const int64_t e = (blockIdx.x % nb) * NT + threadIdx.x;
  if (e >= DM) return;
  float carry = init ? init[bh * DM + e] : 0.f;
  for (int p = 0; p < P; ++p) {
    float* rec = recs + (bh * P + p) * E;
    const float x = rec[e];
    const float lam = rec[DM];
    rec[e] = carry;
    carry = __expf(lam) * carry + x;
  }
  if (tot) tot[bh * DM + e] = carry;
}

size_t lds_ret_fwd(int dim) { return (3 * T * (dim + 8) + dim * (dim + 8)) * sizeof(uint16_t); }
size_t lds_ret_seg(int dim) { return 2 * T * (dim + 8) * sizeof(uint16_t); }

#define LA_RLAUNCH(kernel, grid, lds, st, ...)                                                               \
  do {                                                                                                       \
    hipError_t e_ = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),                               \
                                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));  \
    if (e_ != hipSuccess) return e_;                                                                         \
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(NT), lds, st, __VA_ARGS__);           \
    return hipGetLastError();                                                                                \
  } while (0)

}  // namespace

int retention_supported(int64_t D, int64_t M, int dtype) { return dtype == 1 && D == M && (D == 64 || D == 128); }

hipError_t launch_ret_seg_state(const SegGeom& g, const void* k, const void* v, const float* lg, float* recs,
                                hipStream_t st) {
  const int64_t grid = g.BH * g.P;
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  if (g.D == 64) LA_RLAUNCH((k_ret_seg_state<64>), grid, lds_ret_seg(64), st, K, V, lg, recs, g.N, g.P, g.seg_len);
  if (g.D == 128) LA_RLAUNCH((k_ret_seg_state<128>), grid, lds_ret_seg(128), st, K, V, lg, recs, g.N, g.P, g.seg_len);
  return hipErrorNotSupported;
}

hipError_t launch_ret_scan(float* recs, int64_t BH, int P, int D, int M, const float* init, float* tot,
                           hipStream_t st) {
  const int64_t DM = static_cast<int64_t>(D) * M;
  const int64_t nb = (DM + NT - 1) / NT;
  hipLaunchKernelGGL(k_ret_scan, dim3(static_cast<unsigned>(BH * nb)), dim3(NT), 0, st, recs, P, state_elems(D, M),
                     DM, nb, init, tot);
  return hipGetLastError();
}

hipError_t launch_ret_forward(const SegGeom& g, const void* q, const void* k, const void* v, const float* lg, void* y,
                              const float* carry, hipStream_t st) {
  const int64_t grid = g.BH * g.P;
  const bf16_t* Q = static_cast<const bf16_t*>(q);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  bf16_t* Y = static_cast<bf16_t*>(y);
  if (g.D == 64) LA_RLAUNCH((k_ret_fwd_mfma<64>), grid, lds_ret_fwd(64), st, Q, K, V, lg, Y, carry, g.N, g.P, g.seg_len);
  if (g.D == 128)
    LA_RLAUNCH((k_ret_fwd_mfma<128>), grid, lds_ret_fwd(128), st, Q, K, V, lg, Y, carry, g.N, g.P, g.seg_len);
  return hipErrorNotSupported;
}

}  // namespace la
