// fp32 MFMA kernels for the chunked forward and the segment states (gfx950),
// D = M = 64 (forward and segment states) and D = M = 128 (segment states),
// fp32 inputs and outputs.
//
// Same method and schedule as the bf16 kernels ("[Paper walkthrough]
// Transformers are RNNs", wkq9411.github.io, sections 2 and 3: phi = elu + 1,
// S_i, Z_i, eq:output; non-causal eq:linear), on v_mfma_f32_16x16x4_f32, so
// every operand stays fp32 and nothing is rounded to a narrower type.
// Lane layout (l = lane, g = l / 16, li = l % 16; measured on the hardware):
//   A operand A[li][g], B operand B[g][li] (one fp32 each),
//   C / D     C[4g + u][li], u = 0..3.
// The contraction index of each product is permuted freely (the same on
// both operands): along D, the MFMA step s and lane group g take feature
// 16g + s, so a lane's 16 features sit contiguously in LDS; along tokens the
// scores' accumulator layout (four consecutive keys per lane) is used as is.
#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

using namespace mf;

constexpr int NT = kNT;
constexpr int T = kT;
constexpr int DF = 64;        // D = M
constexpr int LDF = DF + 4;   // fp32 LDS row stride (keeps 16-byte rows aligned)

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float phi_f(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// Global fp32 [T x 64] tile -> LDS (phi applied when asked); rows past nrow
// are zero.  NTH threads, T * 16 / NTH 16-byte pieces each.
template <bool PHI, int NTH = NT>
__device__ __forceinline__ void stage_f32(float* lds, int nrow, const f32x4 (&raw)[T * 16 / NTH]) {
#pragma unroll
  for (int r = 0; r < T * 16 / NTH; ++r) {
    const int p = threadIdx.x + NTH * r;
    const int j = p / 16, c4 = p % 16;
    f32x4 x = raw[r];
    if (j < nrow) {
      if (PHI) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = phi_f(x[e]);
      }
    } else {
      x = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    *reinterpret_cast<f32x4*>(lds + j * LDF + 4 * c4) = x;
  }
}

template <int NTH = NT>
__device__ __forceinline__ void load_f32(f32x4 (&raw)[T * 16 / NTH], const float* __restrict__ src, int64_t c0,
                                         int nrow) {
#pragma unroll
  for (int r = 0; r < T * 16 / NTH; ++r) {
    const int p = threadIdx.x + NTH * r;
    const int j = p / 16, c4 = p % 16;
    raw[r] = j < nrow ? *reinterpret_cast<const f32x4*>(src + (c0 + j) * DF + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// ---------------------------------------------------------------------------
// Forward.  Eight waves, two per SIMD: wave w takes query rows 16 rt .. + 15
// of each 64-token chunk (rt = w for the first four, 3 - (w & 3) for the
// rest, so that the two waves of a SIMD carry one short and one long
// triangle) and output columns 32 ch .. + 31 (ch = w >> 2), and owns state
// rows 16 (w & 3) .. + 15, columns 32 ch .. + 31 (the Z part of those rows
// in the ch = 0 waves).  The two waves of a query tile both form its scores.
//
// Every MFMA operand read from LDS comes four at a time (16-byte reads along
// the contraction index): phi(K) is staged twice, token-major for the scores
// (contraction over features) and feature-major for the state update
// (contraction over tokens); V and S only feature-major (S^T), the layouts
// their products contract over.  One-element reads would put an LDS round
// trip in front of every other MFMA.
// ---------------------------------------------------------------------------
constexpr int NTF = 512;  // threads of the forward
constexpr int PCF = T * 16 / NTF;  // 16-byte pieces per thread per T x 64 fp32 tile

// A tile's pieces into a feature-major LDS tile ldsT[feature][token] (phi
// applied when asked, rows past nrow zero), and, when given, the same values
// token-major into lds[token][feature].
template <bool PHI>
__device__ __forceinline__ void stage_f32_fm(float* ldsT, float* lds, int nrow, const f32x4 (&raw)[PCF]) {
#pragma unroll
  for (int r = 0; r < PCF; ++r) {
    const int p = threadIdx.x + NTF * r;
    const int j = p / 16, c4 = p % 16;
    f32x4 x = raw[r];
    if (j < nrow) {
      if (PHI) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = phi_f(x[e]);
      }
    } else {
      x = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (lds) *reinterpret_cast<f32x4*>(lds + j * LDF + 4 * c4) = x;
#pragma unroll
    for (int e = 0; e < 4; ++e) ldsT[(4 * c4 + e) * LDF + j] = x[e];
  }
}

template <bool CAUSAL>
__global__ __launch_bounds__(NTF, 1) void k_fwd_f32mfma(const float* __restrict__ q, const float* __restrict__ k,
                                                        const float* __restrict__ v, float* __restrict__ out,
                                                        float* __restrict__ den_out, const float* __restrict__ carry,
                                                        int64_t N, int P, int seg_len, int raw_carry) {
  extern __shared__ __align__(16) float smf[];
  float* sKf = smf;                // phi(K), token-major
  float* sKT = sKf + T * LDF;      // phi(K), feature-major
  float* sVT = sKT + DF * LDF;     // V, feature-major
  float* sQf = sVT + DF * LDF;     // phi(Q), token-major
  float* sST = sQf + T * LDF;      // S^T
  float* sZ = sST + DF * LDF;
  // w is wave-uniform (an SGPR): an MFMA under an EXEC-masked branch would
  // still write every lane.
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rt = w < 4 ? w : 3 - (w & 3);  // query row tile
  const int ch = w >> 2;                   // column half (output and state)
  const int sl = w & 3;                    // state row slab
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DF) * DF + DF;
  // raw_carry (causal): `carry` holds the segments' own aggregates, and this
  // segment's carry-in is their sum over the segments before it, added in
  // segment order as the scan adds them (the same bits as the scanned record)
  const float* cs = carry ? (CAUSAL ? carry + (bh * P + (raw_carry ? 0 : seg)) * E : carry + bh * E) : nullptr;
  const int nadd = !cs ? 0 : (CAUSAL && raw_carry) ? seg : 1;
  const float* qh = q + bh * N * DF;
  const float* kh = k + bh * N * DF;
  const float* vh = v + bh * N * DF;
  float* oh = out ? out + bh * N * DF : nullptr;
  float* dh = den_out ? den_out + bh * N : nullptr;
  const int i = 16 * rt + li;

  // this wave's state part: Sacc[nn] holds S[16 sl + 4g + u][32 ch + 16 nn + li],
  // zacc Z[16 sl + 4g + u]
  f32x4_t Sacc[2], zacc;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    Sacc[0][u] = Sacc[1][u] = 0.f;
    zacc[u] = 0.f;
  }
#pragma unroll 4
  for (int t = 0; t < nadd; ++t) {
    const float* rec = cs + t * E;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = 16 * sl + 4 * g + u;
#pragma unroll
      for (int nn = 0; nn < 2; ++nn) Sacc[nn][u] += rec[d * DF + 32 * ch + 16 * nn + li];
      zacc[u] += rec[DF * DF + d];
    }
  }
  auto write_state = [&]() {
#pragma unroll
    for (int nn = 0; nn < 2; ++nn)
      *reinterpret_cast<f32x4_t*>(sST + (32 * ch + 16 * nn + li) * LDF + 16 * sl + 4 * g) = Sacc[nn];
    if (ch == 0 && li == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) sZ[16 * sl + 4 * g + u] = zacc[u];
    }
  };
  write_state();

  int64_t c0 = r0;
  int nrow = static_cast<int>(min(static_cast<int64_t>(T), r1 - c0));
  f32x4 kraw[PCF], vraw[PCF], qraw[PCF];
  if (CAUSAL) {
    load_f32<NTF>(kraw, kh, c0, nrow);
    load_f32<NTF>(vraw, vh, c0, nrow);
  }
  load_f32<NTF>(qraw, qh, c0, nrow);
  while (c0 < r1) {
    if (CAUSAL) {
      stage_f32_fm<true>(sKT, sKf, nrow, kraw);
      stage_f32_fm<false>(sVT, nullptr, nrow, vraw);
    }
    stage_f32<true, NTF>(sQf, nrow, qraw);
    __syncthreads();
    const int64_t c1 = c0 + T;
    const int nrow1 = c1 < r1 ? static_cast<int>(min(static_cast<int64_t>(T), r1 - c1)) : 0;
    if (nrow1 > 0) {
      if (CAUSAL) {
        load_f32<NTF>(kraw, kh, c1, nrow1);
        load_f32<NTF>(vraw, vh, c1, nrow1);
      }
      load_f32<NTF>(qraw, qh, c1, nrow1);
    }
    // this lane's phi(Q_i) features 16g .. 16g + 15
    float qv[16];
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(sQf + i * LDF + 16 * g + 4 * s4);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[4 * s4 + e] = x[e];
    }
    // scores A^T[j][i] for key tiles t <= rt, masked j <= i
    f32x4_t at[4];
    float rs = 0.f;
    if (CAUSAL) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        at[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (t <= rt) {
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4) {
            const f32x4 kx = *reinterpret_cast<const f32x4*>(sKf + (16 * t + li) * LDF + 16 * g + 4 * s4);
#pragma unroll
            for (int e = 0; e < 4; ++e) at[t] = mfma4(kx[e], qv[4 * s4 + e], at[t]);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (t == rt && 4 * g + u > li) at[t][u] = 0.f;
            rs += at[t][u];
          }
        }
      }
    }
    // den = sum_j A_ij + phi(Q_i) . Z
    float di = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) di += qv[s] * sZ[16 * g + s];
    const float den = shfl_sum_groups(rs + di);
    // O^T[m][i] = sum_d S[d][m] phi(Q_i)[d] + sum_j V[j][m] A^T[j][i], m in this wave's half
    f32x4_t o[2];
#pragma unroll
    for (int nn = 0; nn < 2; ++nn) {
      o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const float* srow = sST + (32 * ch + 16 * nn + li) * LDF + 16 * g;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f32x4 sx = *reinterpret_cast<const f32x4*>(srow + 4 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[nn] = mfma4(sx[e], qv[4 * s4 + e], o[nn]);
      }
    }
    if (CAUSAL) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t <= rt) {
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) {
            const f32x4 vx = *reinterpret_cast<const f32x4*>(sVT + (32 * ch + 16 * nn + li) * LDF + 16 * t + 4 * g);
#pragma unroll
            for (int u = 0; u < 4; ++u) o[nn] = mfma4(vx[u], at[t][u], o[nn]);
          }
        }
      }
    }
    if (i < nrow) {
      if (oh) {
        const float inv = 1.f / den;
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
          *reinterpret_cast<f32x4*>(oh + (c0 + i) * DF + 32 * ch + 16 * nn + 4 * g) = o[nn] * inv;
      }
      if (dh && ch == 0 && g == 0) dh[c0 + i] = den;
    }
    if (CAUSAL) {
      // S[d][m] += sum_j phi(K_j)[d] V_j[m], Z[d] += sum_j phi(K_j)[d] (64 keys, j = 16g + s)
      const float* krow = sKT + (16 * sl + li) * LDF + 16 * g;
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(krow + 4 * s4);
        f32x4 b[2];
#pragma unroll
        for (int nn = 0; nn < 2; ++nn)
          b[nn] = *reinterpret_cast<const f32x4*>(sVT + (32 * ch + 16 * nn + li) * LDF + 16 * g + 4 * s4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (ch == 0) zacc = mfma4(a[e], 1.f, zacc);
#pragma unroll
          for (int nn = 0; nn < 2; ++nn) Sacc[nn] = mfma4(a[e], b[nn][e], Sacc[nn]);
        }
      }
    }
    __syncthreads();
    if (CAUSAL) write_state();
    c0 = c1;
    nrow = nrow1;
  }
}

// Segment aggregates dS = phi(K)^T V, dZ = colsum phi(K) over one segment,
// at D = M = DIM (64 or 128).  Wave w owns the RT = DIM / 64 state row tiles
// 16 (RT w + rt) .. + 15 and every column tile; the chunk's phi(K) and V
// rows are staged in LDS (row stride DIM + 4 floats).
template <int DIM>
__global__ __launch_bounds__(NT, 2) void k_seg_state_f32mfma(const float* __restrict__ k, const float* __restrict__ v,
                                                             float* __restrict__ s_out, int64_t s_stride,
                                                             float* __restrict__ z_out, int64_t z_stride, int64_t N,
                                                             int P, int nseg, int seg_len) {
  constexpr int LDD = DIM + 4;
  constexpr int RT = DIM / 64;     // 16-row state tiles per wave
  constexpr int CT = DIM / 16;     // 16-column state tiles
  constexpr int PR = DIM / 4;      // 16-byte pieces per token row
  constexpr int PC = T * PR / NT;  // pieces per thread per chunk tile
  extern __shared__ __align__(16) float smf[];
  float* sKf = smf;
  float* sV = sKf + T * LDD;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / nseg;
  const int seg = blockIdx.x % nseg;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const float* kh = k + bh * N * DIM;
  const float* vh = v + bh * N * DIM;
  f32x4_t Sacc[RT][CT], zacc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    zacc[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < CT; ++n) Sacc[rt][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // piece p of a T x DIM tile: row p / PR, features 4 (p % PR) .. + 3
  auto load = [&](f32x4 (&raw)[PC], const float* __restrict__ src, int64_t c0, int nrow) {
#pragma unroll
    for (int r = 0; r < PC; ++r) {
      const int p = tid + NT * r, j = p / PR, c4 = p % PR;
      raw[r] = j < nrow ? *reinterpret_cast<const f32x4*>(src + (c0 + j) * DIM + 4 * c4) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  // rows past nrow were loaded as zero; phi is applied to the valid rows only
  auto stage = [&](float* lds, const f32x4 (&raw)[PC], int nrow, bool phi) {
#pragma unroll
    for (int r = 0; r < PC; ++r) {
      const int p = tid + NT * r, j = p / PR, c4 = p % PR;
      f32x4 x = raw[r];
      if (phi && j < nrow) {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = phi_f(x[e]);
      }
      *reinterpret_cast<f32x4*>(lds + j * LDD + 4 * c4) = x;
    }
  };
  int64_t c0 = r0;
  int nrow = static_cast<int>(min(static_cast<int64_t>(T), r1 - c0));
  f32x4 kraw[PC], vraw[PC];
  load(kraw, kh, c0, nrow);
  load(vraw, vh, c0, nrow);
  while (c0 < r1) {
    stage(sKf, kraw, nrow, true);
    stage(sV, vraw, nrow, false);
    __syncthreads();
    const int64_t c1 = c0 + T;
    const int nrow1 = c1 < r1 ? static_cast<int>(min(static_cast<int64_t>(T), r1 - c1)) : 0;
    if (nrow1 > 0) {
      load(kraw, kh, c1, nrow1);
      load(vraw, vh, c1, nrow1);
    }
    // S[d][m] += sum_j phi(K_j)[d] V_j[m], Z[d] += sum_j phi(K_j)[d] over the
    // chunk's 64 keys (step s, lane group g: key 16 g + s)
#pragma unroll
    for (int s_ = 0; s_ < 16; ++s_) {
      const int j = 16 * g + s_;
      float a[RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        a[rt] = sKf[j * LDD + 16 * (RT * w + rt) + li];
        zacc[rt] = mfma4(a[rt], 1.f, zacc[rt]);
      }
#pragma unroll
      for (int n = 0; n < CT; ++n) {
        const float b = sV[j * LDD + 16 * n + li];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) Sacc[rt][n] = mfma4(a[rt], b, Sacc[rt][n]);
      }
    }
    __syncthreads();
    c0 = c1;
    nrow = nrow1;
  }
  const int64_t rec = bh * P + seg;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = 16 * (RT * w + rt) + 4 * g + u;
#pragma unroll
      for (int n = 0; n < CT; ++n) s_out[rec * s_stride + d * DIM + 16 * n + li] = Sacc[rt][n][u];
      if (li == 0) z_out[rec * z_stride + d] = zacc[rt][u];
    }
}

constexpr size_t kLdsFwd = (2 * T * LDF + 3 * DF * LDF + DF) * sizeof(float);  // phi(K) twice, V^T, phi(Q), S^T, Z
constexpr size_t lds_seg_f32(int dim) { return 2 * T * (dim + 4) * sizeof(float); }

}  // namespace

hipError_t launch_forward_f32mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                                  void* out, float* den_out, const float* carry, hipStream_t st, int raw_carry) {
  if (g.D != DF || g.M != DF) return hipErrorNotSupported;
  const dim3 grid(static_cast<unsigned>(g.BH * g.P));
  const float* Q = static_cast<const float*>(q);
  const float* K = static_cast<const float*>(k);
  const float* V = static_cast<const float*>(v);
  float* O = static_cast<float*>(out);
  const void* kern = causal ? reinterpret_cast<const void*>(k_fwd_f32mfma<true>)
                            : reinterpret_cast<const void*>(k_fwd_f32mfma<false>);
  const hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsFwd));
  if (e != hipSuccess) return e;
  if (causal)
    hipLaunchKernelGGL((k_fwd_f32mfma<true>), grid, dim3(NTF), kLdsFwd, st, Q, K, V, O, den_out, carry, g.N, g.P,
                       g.seg_len, raw_carry);
  else
    hipLaunchKernelGGL((k_fwd_f32mfma<false>), grid, dim3(NTF), kLdsFwd, st, Q, K, V, O, den_out, carry, g.N, g.P,
                       g.seg_len, 0);
  return hipGetLastError();
}

hipError_t launch_seg_state_f32mfma(const SegGeom& g, const void* k, const void* v, float* s_out, int64_t s_stride,
                                    float* z_out, int64_t z_stride, hipStream_t st) {
  if (g.D != g.M || (g.D != 64 && g.D != 128)) return hipErrorNotSupported;
  const int nseg = g.nseg > 0 ? g.nseg : g.P;
  const dim3 grid(static_cast<unsigned>(g.BH * nseg));
  const float* K = static_cast<const float*>(k);
  const float* V = static_cast<const float*>(v);
  if (g.D == 64) {
    hipLaunchKernelGGL((k_seg_state_f32mfma<64>), grid, dim3(NT), lds_seg_f32(64), st, K, V, s_out, s_stride, z_out,
                       z_stride, g.N, g.P, nseg, g.seg_len);
    return hipGetLastError();
  }
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_seg_state_f32mfma<128>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds_seg_f32(128)));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_seg_state_f32mfma<128>), grid, dim3(NT), lds_seg_f32(128), st, K, V, s_out, s_stride, z_out,
                     z_stride, g.N, g.P, nseg, g.seg_len);
  return hipGetLastError();
}

}  // namespace la
