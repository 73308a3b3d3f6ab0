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
// The same kernels take the decayed recurrence ("08 - Transformer and
// Variants", by-xin.github.io, section 1.3.4) when RET is set: S <- gamma S +
// k v^T and y = S^T q, with no feature map and no normaliser, gamma =
// exp(log gamma) per (b,h) (log gamma below -80 taken as -80, as in the
// chunked kernels; NaN passes through).
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int NT = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Phase 1, shared by both kernels: phi(q), phi(k) and v into LDS, Z updated
// in place, and den = phi(q)^T Z' (fixed-order reduction).  RET: q, k as
// given, no Z, den = 1.
template <bool RET, typename TIn>
__device__ __forceinline__ float decode_prologue(float* qf_s, float* kf_s, float* v_s, float* wden,
                                                 float* __restrict__ Z, const TIn* __restrict__ q,
                                                 const TIn* __restrict__ k, const TIn* __restrict__ v,
                                                 int64_t bh, int D, int M) {
  const int t = threadIdx.x;
  float part = 0.f;
  for (int d = t; d < D; d += NT) {
    const float kf = RET ? ld(k, bh * D + d) : phi(ld(k, bh * D + d));
    const float qf = RET ? ld(q, bh * D + d) : phi(ld(q, bh * D + d));
    kf_s[d] = kf;
    qf_s[d] = qf;
    if (!RET) {
      const float z = Z[bh * D + d] + kf;
      Z[bh * D + d] = z;
      part += qf * z;
    }
  }
  for (int m = t; m < M; m += NT) v_s[m] = ld(v, bh * M + m);
  part = wave_sum(part);
  if ((t & 63) == 0) wden[t >> 6] = part;
  __syncthreads();
  return RET ? 1.f : ((wden[0] + wden[1]) + wden[2]) + wden[3];
}

__device__ __forceinline__ float decay_of(const float* __restrict__ lg, int64_t bh) {
  const float x = lg[bh];
  return __expf(x < -80.f ? -80.f : x);
}

// Vector path: M/4 threads per row, NT/(M/4) rows per pass, U rows in flight.
template <typename TIn, int TPR, bool RET>
__global__ __launch_bounds__(NT) void k_decode_vec(float* __restrict__ S, float* __restrict__ Z,
                                                   const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                   const TIn* __restrict__ v, const float* __restrict__ lg,
                                                   TIn* __restrict__ out, int D) {
  constexpr int M = TPR * 4;
  constexpr int RPI = NT / TPR;
  constexpr int U = 16;
  __shared__ float qf_s[256], kf_s[256], v_s[256], wden[4];
  __shared__ float red[RPI * M];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const float den = decode_prologue<RET>(qf_s, kf_s, v_s, wden, Z, q, k, v, bh, D, M);
  const float gam = RET ? decay_of(lg, bh) : 1.f;
  const int c4 = t % TPR, rg = t / TPR;
  const f32x4 vv = {v_s[4 * c4], v_s[4 * c4 + 1], v_s[4 * c4 + 2], v_s[4 * c4 + 3]};
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4* Sh = reinterpret_cast<f32x4*>(S + bh * static_cast<int64_t>(D) * M) + c4;
  for (int d0 = rg; d0 < D; d0 += RPI * U) {
    f32x4 sv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int d = d0 + u * RPI;
      if (d < D) sv[u] = __builtin_nontemporal_load(Sh + static_cast<int64_t>(d) * TPR);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int d = d0 + u * RPI;
      if (d < D) {
        const f32x4 s = (RET ? gam * sv[u] : sv[u]) + kf_s[d] * vv;
        __builtin_nontemporal_store(s, Sh + static_cast<int64_t>(d) * TPR);
        acc += qf_s[d] * s;
      }
    }
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
    st(out, bh * M + m, RET ? o : o / den);
  }
}

// Scalar path for any M <= 256: one thread per column, NT/M rows per pass.
template <typename TIn, bool RET>
__global__ __launch_bounds__(NT) void k_decode_scalar(float* __restrict__ S, float* __restrict__ Z,
                                                      const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                      const TIn* __restrict__ v, const float* __restrict__ lg,
                                                      TIn* __restrict__ out, int D, int M) {
  __shared__ float qf_s[256], kf_s[256], v_s[256], wden[4];
  __shared__ float red[NT];
  const int64_t bh = blockIdx.x;
  const int t = threadIdx.x;
  const float den = decode_prologue<RET>(qf_s, kf_s, v_s, wden, Z, q, k, v, bh, D, M);
  const float gam = RET ? decay_of(lg, bh) : 1.f;
  const int rpi = NT / M;
  const int m = t % M, rg = t / M;
  float acc = 0.f;
  if (rg < rpi) {
    float* Sh = S + bh * static_cast<int64_t>(D) * M + m;
    const float vm = v_s[m];
    for (int d = rg; d < D; d += rpi) {
      const float s0 = Sh[static_cast<int64_t>(d) * M];
      const float s = (RET ? gam * s0 : s0) + kf_s[d] * vm;
      Sh[static_cast<int64_t>(d) * M] = s;
      acc += qf_s[d] * s;
    }
    red[rg * M + m] = acc;
  }
  __syncthreads();
  for (int mm = t; mm < M; mm += NT) {
    float o = 0.f;
    for (int r = 0; r < rpi; ++r) o += red[r * M + mm];
    st(out, bh * M + mm, RET ? o : o / den);
  }
}

template <bool RET>
hipError_t launch_decode(int dtype, int64_t BH, int D, int M, float* S, float* Z, const void* q, const void* k,
                         const void* v, const float* lg, void* out, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(BH)), block(NT);
  const bool aligned = (reinterpret_cast<uintptr_t>(S) & 15u) == 0;
#define LA_DEC_VEC(T, TPR)                                                                              \
  hipLaunchKernelGGL((k_decode_vec<T, TPR, RET>), grid, block, 0, st, S, Z, static_cast<const T*>(q),   \
                     static_cast<const T*>(k), static_cast<const T*>(v), lg, static_cast<T*>(out), D); \
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
  hipLaunchKernelGGL((k_decode_scalar<T, RET>), grid, block, 0, st, S, Z, static_cast<const T*>(q),      \
                     static_cast<const T*>(k), static_cast<const T*>(v), lg, static_cast<T*>(out), D, M); \
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
  return launch_decode<false>(dtype, BH, D, M, S, Z, q, k, v, nullptr, out, st);
}

hipError_t launch_ret_decode_step(int dtype, int64_t BH, int D, int M, float* S, const void* q, const void* k,
                                  const void* v, const float* lg, void* y, hipStream_t st) {
  return launch_decode<true>(dtype, BH, D, M, S, nullptr, q, k, v, lg, y, st);
}

}  // namespace la
