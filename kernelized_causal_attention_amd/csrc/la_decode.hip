// Batched RNN decode step on gfx950.
//
// "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io), section
// 4: s_i = s_{i-1} + phi(k_i) v_i^T, z_i = z_{i-1} + phi(k_i), and the
// readout phi(q_i)^T s_i / phi(q_i)^T z_i; the state is written before it is
// read (the RNN-mode loop of "The deep link between Transformer and RNN",
// xxqk.cn, section 3).
//
// The step is HBM-bound (about half a flop per byte: every element of S is
// read once, updated with one FMA, written once and multiplied once into the
// readout).  One workgroup owns one (b,h) state: it streams the D x M fp32
// matrix in 16-byte vectors with non-temporal hints (the state is far
// larger than the caches and is not reused within a step), applies the
// rank-1 update, writes it back and folds phi(q)^T S into per-thread column
// partials, which an LDS pass reduces in a fixed order.  The denominator
// phi(q)^T Z is a wavefront reduction.
//
// The same kernels take two more recurrences (MODE):
// * kRet, the decayed recurrence ("08 - Transformer and Variants",
//   by-xin.github.io, section 1.3.4): S <- gamma S + k v^T and y = S^T q,
//   with no feature map and no normaliser, gamma = exp(log gamma) per (b,h)
//   (log gamma below -80 taken as -80, as in the chunked kernels; NaN passes
//   through);
// * kPoly, the degree-2 polynomial feature map ("[Paper walkthrough]
//   Transformers are RNNs", section 2, "feature map and computation cost",
//   item (3)): C = D^2 state rows, phi(x)[a D + b] = x_a x_b formed on the fly
//   from the D raw values in LDS (D a power of two), and out = 0 where the
//   denominator is 0.
#include "la_device.h"
#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

constexpr int NT = 256;
constexpr int kLin = 0, kRet = 1, kPoly = 2;
constexpr int kNonTemporal = 2;  // buffer cache-policy bits: non-temporal
using mf::make_rsrc;
using mf::rsrc_t;
using mf::u32x4;

// Feature c of the row: phi(x)_c from LDS (kLin: phi stored; kRet: x stored;
// kPoly: x stored, c = a D + b -> x_a x_b).
template <int MODE>
__device__ __forceinline__ float feat(const float* f_s, int c, int lgD) {
  if (MODE == kPoly) return f_s[c >> lgD] * f_s[c & ((1 << lgD) - 1)];
  return f_s[c];
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Phase 1, shared by both kernels: phi(q), phi(k) (kLin) or q, k (kRet,
// kPoly) and v into LDS, Z updated in place over the C state rows, and
// den = phi(q)^T Z' (fixed-order reduction; 1 for kRet, which has no Z).
template <int MODE, typename TIn>
__device__ __forceinline__ float decode_prologue(float* qf_s, float* kf_s, float* v_s, float* wden,
                                                 float* __restrict__ Z, const TIn* __restrict__ q,
                                                 const TIn* __restrict__ k, const TIn* __restrict__ v,
                                                 int64_t bh, int D, int C, int lgD, int M) {
  const int t = threadIdx.x;
  for (int d = t; d < D; d += NT) {
    kf_s[d] = MODE == kLin ? phi(ld(k, bh * D + d)) : ld(k, bh * D + d);
    qf_s[d] = MODE == kLin ? phi(ld(q, bh * D + d)) : ld(q, bh * D + d);
  }
  for (int m = t; m < M; m += NT) v_s[m] = ld(v, bh * M + m);
  if (MODE == kPoly) __syncthreads();  // the features read other threads' entries
  float part = 0.f;
  if (MODE != kRet) {
    for (int c = t; c < C; c += NT) {
      const float z = Z[bh * C + c] + feat<MODE>(kf_s, c, lgD);
      Z[bh * C + c] = z;
      part += feat<MODE>(qf_s, c, lgD) * z;
    }
  }
  part = wave_sum(part);
  if ((t & 63) == 0) wden[t >> 6] = part;
  __syncthreads();
  return MODE == kRet ? 1.f : ((wden[0] + wden[1]) + wden[2]) + wden[3];
}

template <int MODE>
__device__ __forceinline__ float readout(float o, float den) {
  if (MODE == kRet) return o;
  if (MODE == kPoly) return den > 0.f ? o / den : 0.f;
  return o / den;
}

__device__ __forceinline__ float decay_of(const float* __restrict__ lg, int64_t bh) {
  const float x = lg[bh];
  return __expf(x < -80.f ? -80.f : x);
}

// Prologue of the vector path for kLin / kRet (D, M <= NT): thread t holds
// entry t of q, k, v and Z.  Split from its use so that the S fetch can be
// issued between the two halves and overlap the prologue's dependent steps.
struct RawIn {
  float q, k, v, z;
};

template <int MODE, typename TIn>
__device__ __forceinline__ RawIn load_raw(const float* __restrict__ Z, const TIn* __restrict__ q,
                                          const TIn* __restrict__ k, const TIn* __restrict__ v, int64_t bh, int D,
                                          int M) {
  const int t = threadIdx.x;
  RawIn r = {0.f, 0.f, 0.f, 0.f};
  if (t < D) {
    r.q = ld(q, bh * D + t);
    r.k = ld(k, bh * D + t);
    if (MODE == kLin) r.z = Z[bh * D + t];
  }
  if (t < M) r.v = ld(v, bh * M + t);
  return r;
}

// Second half: features into LDS, Z' = Z + phi(k) stored, den = phi(q)^T Z'
// (same fixed-order reduction as decode_prologue).
template <int MODE>
__device__ __forceinline__ float finish_raw(const RawIn& r, float* qf_s, float* kf_s, float* v_s, float* wden,
                                            float* __restrict__ Z, int64_t bh, int D, int M) {
  const int t = threadIdx.x;
  float part = 0.f;
  if (t < D) {
    const float kf = MODE == kLin ? phi(r.k) : r.k;
    const float qf = MODE == kLin ? phi(r.q) : r.q;
    kf_s[t] = kf;
    qf_s[t] = qf;
    if (MODE == kLin) {
      const float z = r.z + kf;
      Z[bh * D + t] = z;
      part = qf * z;
    }
  }
  if (t < M) v_s[t] = r.v;
  part = wave_sum(part);
  if ((t & 63) == 0) wden[t >> 6] = part;
  __syncthreads();
  return MODE == kRet ? 1.f : ((wden[0] + wden[1]) + wden[2]) + wden[3];
}

// Vector path: M/4 threads per row, NT/(M/4) rows per pass, U rows in flight.
// The first U rows of each thread are requested before the prologue's
// features and Z update (kLin / kRet after their raw loads, so that waiting
// for those does not wait for S), and each later batch right after the
// previous one is consumed.
template <typename TIn, int TPR, int MODE>
__global__ __launch_bounds__(NT) void k_decode_vec(float* __restrict__ S, float* __restrict__ Z,
                                                   const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                   const TIn* __restrict__ v, const float* __restrict__ lg,
                                                   TIn* __restrict__ out, int D, int C, int lgD) {
  constexpr int M = TPR * 4;
  constexpr int RPI = NT / TPR;
  constexpr int U = 16;
  __shared__ float qf_s[256], kf_s[256], v_s[256], wden[4];
  __shared__ float red[RPI * M];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const int c4 = t % TPR, rg = t / TPR;
  // Buffer access over this head's C x M state: per-lane offset plus a
  // wave-uniform row offset, non-temporal (the state is far larger than the
  // caches and is not reused within a step).  Rows past C read as zero and
  // their stores are dropped by the range check.
  const rsrc_t Sr = make_rsrc(S + bh * static_cast<int64_t>(C) * M, static_cast<int64_t>(C) * M * 4);
  const int voff = (rg * M + 4 * c4) * 4;
  f32x4 sv[U];
  // Always U loads, so the count of loads in flight is fixed and waiting for
  // the prologue's own loads does not wait for S.
  auto fetch = [&](int r0) {
#pragma unroll
    for (int u = 0; u < U; ++u)
      sv[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(Sr, voff, (r0 + u * RPI) * M * 4, kNonTemporal));
  };
  float den;
  if (MODE == kPoly) {
    fetch(0);
    den = decode_prologue<MODE>(qf_s, kf_s, v_s, wden, Z, q, k, v, bh, D, C, lgD, M);
  } else {
    const RawIn r = load_raw<MODE>(Z, q, k, v, bh, D, M);
    fetch(0);
    den = finish_raw<MODE>(r, qf_s, kf_s, v_s, wden, Z, bh, D, M);
  }
  const float gam = MODE == kRet ? decay_of(lg, bh) : 1.f;
  const f32x4 vv = {v_s[4 * c4], v_s[4 * c4 + 1], v_s[4 * c4 + 2], v_s[4 * c4 + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto consume = [&](int r0, bool guard) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int d = r0 + rg + u * RPI;
      const int dc = guard ? min(d, C - 1) : d;
      const f32x4 s = (MODE == kRet ? gam * sv[u] : sv[u]) + feat<MODE>(kf_s, dc, lgD) * vv;
      // (all of the offset in the VGPR, none in the SGPR: the compiler then
      // keeps the stored VGPRs from being overwritten before the store has
      // read them, which it does not do for a store with an SGPR offset)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, s), Sr, voff + (r0 + u * RPI) * M * 4, 0,
                                             kNonTemporal);
      if (!guard || d < C) acc += feat<MODE>(qf_s, dc, lgD) * s;
    }
  };
  for (int r0 = 0; r0 < C; r0 += RPI * U) {
    if (r0) fetch(r0);
    if (r0 + RPI * U <= C)  // wave-uniform: every row of the batch exists
      consume(r0, false);
    else
      consume(r0, true);
  }
  red[rg * M + 4 * c4 + 0] = acc.x;
  red[rg * M + 4 * c4 + 1] = acc.y;
  red[rg * M + 4 * c4 + 2] = acc.z;
  red[rg * M + 4 * c4 + 3] = acc.w;
  __syncthreads();
  for (int m = t; m < M; m += NT) {
    float o = 0.f;
#pragma unroll
    for (int r = 0; r < RPI; ++r) o += red[r * M + m];
    st(out, bh * M + m, readout<MODE>(o, den));
  }
}

// Scalar path for any M <= 256: one thread per column, NT/M rows per pass.
template <typename TIn, int MODE>
__global__ __launch_bounds__(NT) void k_decode_scalar(float* __restrict__ S, float* __restrict__ Z,
                                                      const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                      const TIn* __restrict__ v, const float* __restrict__ lg,
                                                      TIn* __restrict__ out, int D, int C, int lgD, int M) {
  __shared__ float qf_s[256], kf_s[256], v_s[256], wden[4];
  __shared__ float red[NT];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const float den = decode_prologue<MODE>(qf_s, kf_s, v_s, wden, Z, q, k, v, bh, D, C, lgD, M);
  const float gam = MODE == kRet ? decay_of(lg, bh) : 1.f;
  const int rpi = NT / M;
  const int m = t % M, rg = t / M;
  float acc = 0.f;
  if (rg < rpi) {
    float* Sh = S + bh * static_cast<int64_t>(C) * M + m;
    const float vm = v_s[m];
    for (int d = rg; d < C; d += rpi) {
      const float s0 = Sh[static_cast<int64_t>(d) * M];
      const float s = (MODE == kRet ? gam * s0 : s0) + feat<MODE>(kf_s, d, lgD) * vm;
      Sh[static_cast<int64_t>(d) * M] = s;
      acc += feat<MODE>(qf_s, d, lgD) * s;
    }
    red[rg * M + m] = acc;
  }
  __syncthreads();
  for (int mm = t; mm < M; mm += NT) {
    float o = 0.f;
    for (int r = 0; r < rpi; ++r) o += red[r * M + mm];
    st(out, bh * M + mm, readout<MODE>(o, den));
  }
}

template <int MODE>
hipError_t launch_decode(int dtype, int64_t BH, int D, int M, float* S, float* Z, const void* q, const void* k,
                         const void* v, const float* lg, void* out, hipStream_t st) {
  int lgD = 0;
  while ((1 << lgD) < D) ++lgD;
  const int C = MODE == kPoly ? D * D : D;
  const dim3 grid(static_cast<unsigned>(BH)), block(NT);
  const bool aligned = (reinterpret_cast<uintptr_t>(S) & 15u) == 0;
#define LA_DEC_VEC(T, TPR)                                                                              \
  hipLaunchKernelGGL((k_decode_vec<T, TPR, MODE>), grid, block, 0, st, S, Z, static_cast<const T*>(q),  \
                     static_cast<const T*>(k), static_cast<const T*>(v), lg, static_cast<T*>(out), D, C, lgD); \
  return hipGetLastError()
#define LA_DEC(T)                                                                                        \
  if (aligned && M % 4 == 0) {                                                                           \
    switch (M / 4) {                                                                                     \
      case 1: LA_DEC_VEC(T, 1);                                                                          \
      case 2: LA_DEC_VEC(T, 2);                                                                          \
      case 4: LA_DEC_VEC(T, 4);                                                                          \
      case 8: LA_DEC_VEC(T, 8);                                                                          \
      case 16: LA_DEC_VEC(T, 16);                                                                        \
      case 32: LA_DEC_VEC(T, 32);                                                                        \
      case 64: LA_DEC_VEC(T, 64);                                                                        \
      default: break;                                                                                    \
    }                                                                                                    \
  }                                                                                                      \
  hipLaunchKernelGGL((k_decode_scalar<T, MODE>), grid, block, 0, st, S, Z, static_cast<const T*>(q),     \
                     static_cast<const T*>(k), static_cast<const T*>(v), lg, static_cast<T*>(out), D, C, lgD, M); \
  return hipGetLastError()
  if (dtype == 0) {
    LA_DEC(float);
  } else {
    LA_DEC(bf16_t);
  }
#undef LA_DEC
#undef LA_DEC_VEC
}

}  // namespace

hipError_t launch_decode_step(int dtype, int64_t BH, int D, int M, float* S, float* Z, const void* q,
                              const void* k, const void* v, void* out, hipStream_t st) {
  return launch_decode<kLin>(dtype, BH, D, M, S, Z, q, k, v, nullptr, out, st);
}

hipError_t launch_ret_decode_step(int dtype, int64_t BH, int D, int M, float* S, const void* q, const void* k,
                                  const void* v, const float* lg, void* y, hipStream_t st) {
  return launch_decode<kRet>(dtype, BH, D, M, S, nullptr, q, k, v, lg, y, st);
}

hipError_t launch_poly_decode_step(int dtype, int64_t BH, int D, int M, float* S, float* Z, const void* q,
                                   const void* k, const void* v, void* out, hipStream_t st) {
  return launch_decode<kPoly>(dtype, BH, D, M, S, Z, q, k, v, nullptr, out, st);
}

}  // namespace la
