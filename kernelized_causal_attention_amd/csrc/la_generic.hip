// Generic chunked kernels for causal / non-causal linear attention on gfx950.
//
// These cover every (D, M) with D*M <= 16384 and fp32 or bf16 inputs, in
// plain fp32 FMA arithmetic with LDS-staged tiles.  The bf16 MFMA kernels
// (la_mfma.hip) take over the common shapes; these stay as the general path.
//
// Method ("[Paper walkthrough] Transformers are RNNs", wkq9411.github.io):
//   section 2: phi = elu + 1; non-causal phi(Q)(phi(K)^T V) (eq:linear)
//   section 3: S_i = sum_{j<=i} phi(K_j) V_j^T, Z_i = sum_{j<=i} phi(K_j),
//              out_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i (eq:mask, eq:output)
//   section 3.1: gradients through a prefix matrix (eq:gq) and a suffix
//              matrix (the phi(K) equation and eq:gv).
//
// Chunking.  Each sequence is cut into P segments of `seg_len` tokens and
// each segment into chunks of TC tokens.  For a chunk starting after state
// (S, Z), the inclusive causal sums split exactly into the carried state and
// a lower-triangular TC x TC tile (the sums are associative; the chunk is
// the block-matrix product of the masked quadratic form):
//   num_i = phi(Q_i)^T S + sum_{j<=i in chunk} (phi(Q_i).phi(K_j)) V_j
//   den_i = phi(Q_i)^T Z + sum_{j<=i in chunk}  phi(Q_i).phi(K_j)
// A segment's carried-in state is the exclusive scan of the per-segment
// aggregates (k_seg_state + k_seg_scan).  One workgroup walks one segment.
#include "la_device.h"
#include "la_internal.h"

namespace la {
namespace {

constexpr int NT = 256;  // threads per workgroup (4 wave64s)

// Stage rows [row0, row0 + nrow) of a [*, F] tensor into an LDS tile with
// row stride `stride`; rows past nrow are zero (so they add nothing to any
// sum), and phi is applied to valid rows when asked.
template <typename TIn, int TC>
__device__ __forceinline__ void stage(float* dst, int stride, const TIn* __restrict__ src, int64_t row0,
                                      int nrow, int F, bool apply_phi) {
  for (int e = threadIdx.x; e < TC * F; e += NT) {
    const int i = e / F, f = e - i * F;
    float x = 0.f;
    if (i < nrow) {
      x = ld(src, (row0 + i) * F + f);
      if (apply_phi) x = phi(x);
    }
    dst[i * stride + f] = x;
  }
}

// S[d][m] += sum_j Kf[j][d] V[j][m];  Z[d] += sum_j Kf[j][d]
__device__ __forceinline__ void state_update(float* S, int SP, float* Z, const float* Kf, int DP,
                                             const float* V, int MP, int nrow, int D, int M) {
  if ((D & 3) == 0 && (M & 3) == 0) {
    // 4 x 4 register tiles: thread tile (dt, mt) holds S[dt + a D/4][mt + b M/4],
    // a, b < 4, for the whole chunk -- 16 FMAs per 8 LDS reads; consecutive
    // threads take consecutive mt (conflict-free V reads, broadcast K reads)
    const int D4 = D >> 2, M4 = M >> 2;
    for (int t = threadIdx.x; t < D4 * M4; t += NT) {
      const int dt = t / M4, mt = t - dt * M4;
      float acc[4][4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = S[(dt + a * D4) * SP + mt + b * M4];
      for (int j = 0; j < nrow; ++j) {
        float kk[4], vv[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) kk[a] = Kf[j * DP + dt + a * D4];
#pragma unroll
        for (int b = 0; b < 4; ++b) vv[b] = V[j * MP + mt + b * M4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int b = 0; b < 4; ++b) acc[a][b] += kk[a] * vv[b];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) S[(dt + a * D4) * SP + mt + b * M4] = acc[a][b];
    }
  } else {
    for (int e = threadIdx.x; e < D * M; e += NT) {
      const int d = e / M, m = e - d * M;
      float acc = S[d * SP + m];
      for (int j = 0; j < nrow; ++j) acc += Kf[j * DP + d] * V[j * MP + m];
      S[d * SP + m] = acc;
    }
  }
  for (int d = threadIdx.x; d < D; d += NT) {
    float z = Z[d];
    for (int j = 0; j < nrow; ++j) z += Kf[j * DP + d];
    Z[d] = z;
  }
}

// ---------------------------------------------------------------------------
// Segment aggregates: dS = sum_{j in segment} phi(K_j) V_j^T, dZ = sum phi(K_j).
// ---------------------------------------------------------------------------
template <typename TIn, int TC>
__global__ __launch_bounds__(NT) void k_seg_state(const TIn* __restrict__ k, const TIn* __restrict__ v,
                                                  float* __restrict__ s_out, int64_t s_stride,
                                                  float* __restrict__ z_out, int64_t z_stride, int64_t N, int D,
                                                  int M, int P, int seg_len) {
  extern __shared__ float sm[];
  const int SP = M + 1, DP = D + 1, MP = M + 1;
  float* S = sm;
  float* Z = S + D * SP;
  float* Kf = Z + D;
  float* V = Kf + TC * DP;
  const int64_t bh = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(s) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const TIn* kh = k + bh * N * D;
  const TIn* vh = v + bh * N * M;
  for (int e = threadIdx.x; e < D * M; e += NT) S[(e / M) * SP + e % M] = 0.f;
  for (int d = threadIdx.x; d < D; d += NT) Z[d] = 0.f;
  for (int64_t c0 = r0; c0 < r1; c0 += TC) {
    const int nrow = static_cast<int>(min(static_cast<int64_t>(TC), r1 - c0));
    __syncthreads();
    stage<TIn, TC>(Kf, DP, kh, c0, nrow, D, true);
    stage<TIn, TC>(V, MP, vh, c0, nrow, M, false);
    __syncthreads();
    state_update(S, SP, Z, Kf, DP, V, MP, nrow, D, M);
  }
  __syncthreads();
  const int64_t rec = bh * P + s;
  for (int e = threadIdx.x; e < D * M; e += NT) s_out[rec * s_stride + e] = S[(e / M) * SP + e % M];
  for (int d = threadIdx.x; d < D; d += NT) z_out[rec * z_stride + d] = Z[d];
}

// ---------------------------------------------------------------------------
// Exclusive scan of per-segment records along the segment axis, fixed order.
// ---------------------------------------------------------------------------
constexpr int kScanBatch = 8;

__global__ __launch_bounds__(NT) void k_seg_scan(float* __restrict__ agg, int P, int64_t E, int64_t nb,
                                                 int reverse, int64_t DM, const float* init_s, const float* init_z,
                                                 float* tot_s, int64_t ts_stride, float* tot_z, int64_t tz_stride) {
  const int64_t bh = blockIdx.x / nb;
  const int64_t e = (blockIdx.x % nb) * NT + threadIdx.x;
  if (e >= E) return;
  // (init and tot may be the same memory: each element is read here, by the
  // thread that writes its total below)
  float carry = init_s ? (e < DM ? init_s[bh * DM + e] : init_z[bh * (E - DM) + (e - DM)]) : 0.f;
  // Records are read kScanBatch at a time before any of them is overwritten:
  // the compiler cannot order a record's load ahead of the previous record's
  // store by itself (it cannot rule out that they alias), so a one-record
  // loop would wait out a memory round trip per segment.
  for (int p0 = 0; p0 < P; p0 += kScanBatch) {
    float x[kScanBatch];
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      const int p = p0 + j;
      const int s = reverse ? P - 1 - p : p;
      // without a total the last record's aggregate is never needed (and
      // may not have been computed): it is not read
      x[j] = (p < P && (tot_s || p + 1 < P)) ? agg[(bh * P + s) * E + e] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kScanBatch; ++j) {
      const int p = p0 + j;
      if (p < P) {
        const int s = reverse ? P - 1 - p : p;
        agg[(bh * P + s) * E + e] = carry;
        carry += x[j];
      }
    }
  }
  if (tot_s) {
    if (e < DM)
      tot_s[bh * ts_stride + e] = carry;
    else
      tot_z[bh * tz_stride + (e - DM)] = carry;
  }
}

// ---------------------------------------------------------------------------
// Forward.  CAUSAL: carry = exclusive prefix record of this segment (or
// null = zero state).  Non-causal: carry = the head's total (S_N, Z_N) and
// the state is not updated.
// ---------------------------------------------------------------------------
template <typename TIn, int TC, bool CAUSAL>
__global__ __launch_bounds__(NT) void k_forward(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                const TIn* __restrict__ v, TIn* __restrict__ out,
                                                float* __restrict__ den_out, const float* __restrict__ carry,
                                                int64_t N, int D, int M, int P, int seg_len) {
  extern __shared__ float sm[];
  const int SP = M + 1, DP = D + 1, MP = M + 1, AP = TC + 1;
  float* S = sm;
  float* Z = S + D * SP;
  float* Qf = Z + D;
  float* Kf = Qf + TC * DP;
  float* V = Kf + TC * DP;
  float* A = V + TC * MP;
  float* den = A + TC * AP;
  const int t = threadIdx.x;
  const int64_t bh = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(s) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const int64_t E = state_elems(D, M);
  const float* cs = nullptr;
  if (carry) cs = CAUSAL ? carry + (bh * P + s) * E : carry + bh * E;
  for (int e = t; e < D * M; e += NT) S[(e / M) * SP + e % M] = cs ? cs[e] : 0.f;
  for (int d = t; d < D; d += NT) Z[d] = cs ? cs[D * M + d] : 0.f;
  const TIn* qh = q + bh * N * D;
  const TIn* kh = k + bh * N * D;
  const TIn* vh = v + bh * N * M;
  TIn* oh = out ? out + bh * N * M : nullptr;
  float* dh = den_out ? den_out + bh * N : nullptr;

  for (int64_t c0 = r0; c0 < r1; c0 += TC) {
    const int nrow = static_cast<int>(min(static_cast<int64_t>(TC), r1 - c0));
    __syncthreads();
    stage<TIn, TC>(Qf, DP, qh, c0, nrow, D, true);
    if (CAUSAL) stage<TIn, TC>(Kf, DP, kh, c0, nrow, D, true);
    if (CAUSAL) stage<TIn, TC>(V, MP, vh, c0, nrow, M, false);
    __syncthreads();
    if (CAUSAL) {
      // masked scores A_ij = phi(Q_i).phi(K_j), j <= i
      for (int e = t; e < TC * TC; e += NT) {
        const int i = e / TC, j = e - i * TC;
        float a = 0.f;
        if (j <= i && i < nrow)
          for (int d = 0; d < D; ++d) a += Qf[i * DP + d] * Kf[j * DP + d];
        A[i * AP + j] = a;
      }
      __syncthreads();
    }
    if (t < TC) {
      float dd = 0.f;
      for (int d = 0; d < D; ++d) dd += Qf[t * DP + d] * Z[d];
      if (CAUSAL)
        for (int j = 0; j <= t; ++j) dd += A[t * AP + j];
      den[t] = dd;
      if (dh && t < nrow) dh[c0 + t] = dd;
    }
    __syncthreads();
    if (oh) {
      for (int e = t; e < TC * M; e += NT) {
        const int i = e / M, m = e - i * M;
        if (i >= nrow) continue;
        float num = 0.f;
        for (int d = 0; d < D; ++d) num += Qf[i * DP + d] * S[d * SP + m];
        if (CAUSAL)
          for (int j = 0; j <= i; ++j) num += A[i * AP + j] * V[j * MP + m];
        st(oh, (c0 + i) * M + m, num / den[i]);
      }
    }
    if (CAUSAL) {
      __syncthreads();
      state_update(S, SP, Z, Kf, DP, V, MP, nrow, D, M);
    }
  }
}

// Stage the per-row backward inputs of one chunk for the reverse sweep:
//   g_i = dout_i / den_i, with den_i and c_i = -(dout_i . out_i) / den_i as
// the forward sweep formed them (from the fp32 numerator, not the stored out).
// G holds g afterwards.
template <typename TIn, int TC>
__device__ __forceinline__ void stage_grad_rows(float* G, int MP, float* cvec, float* dn,
                                                const TIn* __restrict__ gh, const float* __restrict__ denh,
                                                const float* __restrict__ ch, int64_t c0, int nrow, int M) {
  stage<TIn, TC>(G, MP, gh, c0, nrow, M, false);
  for (int i = threadIdx.x; i < TC; i += NT) {
    dn[i] = i < nrow ? denh[c0 + i] : 1.f;
    cvec[i] = i < nrow ? ch[c0 + i] : 0.f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < TC * M; e += NT) {
    const int i = e / M, m = e - i * M;
    G[i * MP + m] = G[i * MP + m] / dn[i];
  }
}

// ---------------------------------------------------------------------------
// Backward, forward sweep:
//   grad phi(Q_i) = S_i g_i + c_i Z_i
// chunked as  sum_{j<=i in chunk} (g_i.V_j + c_i) phi(K_j) + S g_i + c_i Z,
// then dq = grad phi(Q) * phi'(q).  The sweep first forms num_i and den_i of
// its rows in fp32, exactly as the forward does, and takes
//   g_i = dout_i / den_i,  c_i = -(dout_i . num_i) / den_i^2
// from them: the bf16-rounded out would do for c only up to its 2^-9
// rounding, and with phi ~ 1 the two terms of grad phi(Q) cancel in the
// all-ones direction, which multiplies that rounding several times over.
// den and c go to the reverse sweep (den_out, c_out).  The same pass
// accumulates the segment's suffix aggregates R = sum phi(Q_i) g_i^T,
// r = sum c_i phi(Q_i).
// ---------------------------------------------------------------------------
template <typename TIn, int TC, bool CAUSAL, int RPT>
__global__ __launch_bounds__(NT) void k_bwd_dq(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                               const TIn* __restrict__ v, const TIn* __restrict__ dout,
                                               const float* __restrict__ carry_s, TIn* __restrict__ dq,
                                               float* __restrict__ r_agg, float* __restrict__ c_out,
                                               float* __restrict__ den_out, int64_t N, int D, int M, int P,
                                               int seg_len) {
  extern __shared__ float sm[];
  const int SP = M + 1, DP = D + 1, MP = M + 1, AP = TC + 1;
  const int WSZ = (TC * MP > TC * AP) ? TC * MP : TC * AP;
  float* S = sm;
  float* Z = S + D * SP;
  float* Qf = Z + D;
  float* Kf = Qf + TC * DP;
  float* V = Kf + TC * DP;
  float* G = V + TC * MP;
  float* W = G + TC * MP;
  float* A = W + WSZ;
  float* cvec = A + TC * AP;
  float* dn = cvec + TC;
  const int t = threadIdx.x;
  const int64_t bh = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(s) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const int DM = D * M;
  const int64_t E = state_elems(D, M);
  const float* cs = nullptr;
  if (carry_s) cs = CAUSAL ? carry_s + (bh * P + s) * E : carry_s + bh * E;
  for (int e = t; e < DM; e += NT) S[(e / M) * SP + e % M] = cs ? cs[e] : 0.f;
  for (int d = t; d < D; d += NT) Z[d] = cs ? cs[DM + d] : 0.f;
  const TIn* qh = q + bh * N * D;
  const TIn* kh = k + bh * N * D;
  const TIn* vh = v + bh * N * M;
  const TIn* gh = dout + bh * N * M;
  TIn* dqh = dq + bh * N * D;
  float* ch = c_out + bh * N;
  float* dh = den_out + bh * N;
  float racc[RPT];
#pragma unroll
  for (int r = 0; r < RPT; ++r) racc[r] = 0.f;
  float rz = 0.f;

  for (int64_t c0 = r0; c0 < r1; c0 += TC) {
    const int nrow = static_cast<int>(min(static_cast<int64_t>(TC), r1 - c0));
    __syncthreads();
    stage<TIn, TC>(Qf, DP, qh, c0, nrow, D, true);
    if (CAUSAL) stage<TIn, TC>(Kf, DP, kh, c0, nrow, D, true);
    if (CAUSAL) stage<TIn, TC>(V, MP, vh, c0, nrow, M, false);
    stage<TIn, TC>(G, MP, gh, c0, nrow, M, false);
    __syncthreads();
    if (CAUSAL) {
      // masked scores A_ij = phi(Q_i).phi(K_j), j <= i
      for (int e = t; e < TC * TC; e += NT) {
        const int i = e / TC, j = e - i * TC;
        float a = 0.f;
        if (j <= i && i < nrow)
          for (int d = 0; d < D; ++d) a += Qf[i * DP + d] * Kf[j * DP + d];
        A[i * AP + j] = a;
      }
      __syncthreads();
    }
    // num_i into W, den_i into dn (rows past nrow: num 0, den 1)
    for (int e = t; e < TC * M; e += NT) {
      const int i = e / M, m = e - i * M;
      float num = 0.f;
      if (i < nrow) {
        for (int d = 0; d < D; ++d) num += Qf[i * DP + d] * S[d * SP + m];
        if (CAUSAL)
          for (int j = 0; j <= i; ++j) num += A[i * AP + j] * V[j * MP + m];
      }
      W[i * MP + m] = num;
    }
    if (t < TC) {
      float dd = 1.f;
      if (t < nrow) {
        dd = 0.f;
        for (int d = 0; d < D; ++d) dd += Qf[t * DP + d] * Z[d];
        if (CAUSAL)
          for (int j = 0; j <= t; ++j) dd += A[t * AP + j];
      }
      dn[t] = dd;
    }
    __syncthreads();
    if (t < TC) {
      float dot = 0.f;
      for (int m = 0; m < M; ++m) dot += G[t * MP + m] * W[t * MP + m];
      const float c = t < nrow ? -(dot / dn[t]) / dn[t] : 0.f;
      cvec[t] = c;
      if (t < nrow) {
        ch[c0 + t] = c;
        dh[c0 + t] = dn[t];
      }
    }
    __syncthreads();
    for (int e = t; e < TC * M; e += NT) {
      const int i = e / M, m = e - i * M;
      G[i * MP + m] = G[i * MP + m] / dn[i];
    }
    __syncthreads();
    if (CAUSAL) {
      // B_ij = g_i.V_j + c_i for j <= i (W now holds B)
      for (int e = t; e < TC * TC; e += NT) {
        const int i = e / TC, j = e - i * TC;
        float b = 0.f;
        if (j <= i && i < nrow) {
          for (int m = 0; m < M; ++m) b += G[i * MP + m] * V[j * MP + m];
          b += cvec[i];
        }
        W[i * AP + j] = b;
      }
      __syncthreads();
    }
    for (int e = t; e < TC * D; e += NT) {
      const int i = e / D, d = e - i * D;
      if (i >= nrow) continue;
      float acc = cvec[i] * Z[d];
      for (int m = 0; m < M; ++m) acc += G[i * MP + m] * S[d * SP + m];
      if (CAUSAL)
        for (int j = 0; j <= i; ++j) acc += W[i * AP + j] * Kf[j * DP + d];
      st(dqh, (c0 + i) * D + d, acc * phi_prime_from_phi(Qf[i * DP + d]));
    }
    // suffix aggregates of this segment
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int e = t + r * NT;
      if (e < DM) {
        const int d = e / M, m = e - d * M;
        float a = racc[r];
        for (int i = 0; i < nrow; ++i) a += Qf[i * DP + d] * G[i * MP + m];
        racc[r] = a;
      }
    }
    if (t < D)
      for (int i = 0; i < nrow; ++i) rz += cvec[i] * Qf[i * DP + t];
    if (CAUSAL) {
      __syncthreads();
      state_update(S, SP, Z, Kf, DP, V, MP, nrow, D, M);
    }
  }
  if (r_agg) {
    float* rec = r_agg + (bh * P + s) * E;
#pragma unroll
    for (int r = 0; r < RPT; ++r) {
      const int e = t + r * NT;
      if (e < DM) rec[e] = racc[r];
    }
    if (t < D) rec[DM + t] = rz;
  }
}

// ---------------------------------------------------------------------------
// Backward, reverse sweep over the chunks of a segment, suffix state (R, r):
//   grad phi(K_j) = R_j V_j + r_j,  grad V_j = R_j^T phi(K_j),
// chunked as  sum_{i>=j in chunk} (g_i.V_j + c_i) phi(Q_i) + R V_j + r  and
//             sum_{i>=j in chunk} (phi(Q_i).phi(K_j)) g_i + R^T phi(K_j),
// then dk = grad phi(K) * phi'(k).
// ---------------------------------------------------------------------------
template <typename TIn, int TC, bool CAUSAL>
__global__ __launch_bounds__(NT) void k_bwd_dkdv(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                 const TIn* __restrict__ v, const TIn* __restrict__ dout,
                                                 const float* __restrict__ den_in, const float* __restrict__ c_in,
                                                 const float* __restrict__ carry_r, TIn* __restrict__ dk,
                                                 TIn* __restrict__ dv, int64_t N, int D, int M, int P,
                                                 int seg_len) {
  extern __shared__ float sm[];
  const int SP = M + 1, DP = D + 1, MP = M + 1, AP = TC + 1;
  const int WSZ = (TC * MP > TC * AP) ? TC * MP : TC * AP;
  float* R = sm;
  float* rv = R + D * SP;
  float* Qf = rv + D;
  float* Kf = Qf + TC * DP;
  float* V = Kf + TC * DP;
  float* G = V + TC * MP;
  float* W = G + TC * MP;
  float* A = W + WSZ;
  float* cvec = A + TC * AP;
  float* dn = cvec + TC;
  const int t = threadIdx.x;
  const int64_t bh = blockIdx.x / P;
  const int s = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(s) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const int DM = D * M;
  const int64_t E = state_elems(D, M);
  const float* cr = nullptr;
  if (carry_r) cr = CAUSAL ? carry_r + (bh * P + s) * E : carry_r + bh * E;
  for (int e = t; e < DM; e += NT) R[(e / M) * SP + e % M] = cr ? cr[e] : 0.f;
  for (int d = t; d < D; d += NT) rv[d] = cr ? cr[DM + d] : 0.f;
  const TIn* qh = q + bh * N * D;
  const TIn* kh = k + bh * N * D;
  const TIn* vh = v + bh * N * M;
  const TIn* gh = dout + bh * N * M;
  const float* denh = den_in + bh * N;
  const float* chh = c_in + bh * N;
  TIn* dkh = dk + bh * N * D;
  TIn* dvh = dv + bh * N * M;
  const int64_t nch = (r1 - r0 + TC - 1) / TC;

  for (int64_t ci = nch - 1; ci >= 0; --ci) {
    const int64_t c0 = r0 + ci * TC;
    const int nrow = static_cast<int>(min(static_cast<int64_t>(TC), r1 - c0));
    __syncthreads();
    stage<TIn, TC>(Kf, DP, kh, c0, nrow, D, true);
    stage<TIn, TC>(V, MP, vh, c0, nrow, M, false);
    if (CAUSAL) stage<TIn, TC>(Qf, DP, qh, c0, nrow, D, true);
    if (CAUSAL) stage_grad_rows<TIn, TC>(G, MP, cvec, dn, gh, denh, chh, c0, nrow, M);
    __syncthreads();
    if (CAUSAL) {
      for (int e = t; e < TC * TC; e += NT) {
        const int i = e / TC, j = e - i * TC;
        float a = 0.f, b = 0.f;
        if (j <= i && i < nrow) {
          for (int d = 0; d < D; ++d) a += Qf[i * DP + d] * Kf[j * DP + d];
          for (int m = 0; m < M; ++m) b += G[i * MP + m] * V[j * MP + m];
          b += cvec[i];
        }
        A[i * AP + j] = a;
        W[i * AP + j] = b;
      }
      __syncthreads();
    }
    for (int e = t; e < TC * M; e += NT) {
      const int j = e / M, m = e - j * M;
      if (j >= nrow) continue;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += Kf[j * DP + d] * R[d * SP + m];
      if (CAUSAL)
        for (int i = j; i < nrow; ++i) acc += A[i * AP + j] * G[i * MP + m];
      st(dvh, (c0 + j) * M + m, acc);
    }
    for (int e = t; e < TC * D; e += NT) {
      const int j = e / D, d = e - j * D;
      if (j >= nrow) continue;
      float acc = rv[d];
      for (int m = 0; m < M; ++m) acc += R[d * SP + m] * V[j * MP + m];
      if (CAUSAL)
        for (int i = j; i < nrow; ++i) acc += W[i * AP + j] * Qf[i * DP + d];
      st(dkh, (c0 + j) * D + d, acc * phi_prime_from_phi(Kf[j * DP + d]));
    }
    if (CAUSAL) {
      __syncthreads();
      for (int e = t; e < DM; e += NT) {
        const int d = e / M, m = e - d * M;
        float a = R[d * SP + m];
        for (int i = 0; i < nrow; ++i) a += Qf[i * DP + d] * G[i * MP + m];
        R[d * SP + m] = a;
      }
      for (int d = t; d < D; d += NT) {
        float a = rv[d];
        for (int i = 0; i < nrow; ++i) a += cvec[i] * Qf[i * DP + d];
        rv[d] = a;
      }
    }
  }
}

// ------------------------------------------------------------ launchers ----
size_t lds_fwd(int TC, int D, int M) {
  return sizeof(float) * (static_cast<size_t>(D) * (M + 1) + D + 2 * TC * (D + 1) + TC * (M + 1) +
                          TC * (TC + 1) + TC);
}
size_t lds_seg(int TC, int D, int M) {
  return sizeof(float) * (static_cast<size_t>(D) * (M + 1) + D + TC * (D + 1) + TC * (M + 1));
}
size_t lds_bwd_dq(int TC, int D, int M) {
  const size_t wsz = std::max<size_t>(TC * (M + 1), TC * (TC + 1));
  return sizeof(float) * (static_cast<size_t>(D) * (M + 1) + D + 2 * TC * (D + 1) + 2 * TC * (M + 1) +
                          wsz + TC * (TC + 1) + 2 * TC);
}
size_t lds_bwd_dkdv(int TC, int D, int M) {
  const size_t wsz = std::max<size_t>(TC * (M + 1), TC * (TC + 1));
  return sizeof(float) * (static_cast<size_t>(D) * (M + 1) + D + 2 * TC * (D + 1) + 2 * TC * (M + 1) +
                          wsz + TC * (TC + 1) + 2 * TC);
}

#define LA_LAUNCH(kernel, grid, lds, st, ...)                                                     \
  do {                                                                                            \
    hipError_t e_ = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),                    \
                                        hipFuncAttributeMaxDynamicSharedMemorySize,               \
                                        static_cast<int>(lds));                                   \
    if (e_ != hipSuccess) return e_;                                                              \
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(NT), lds, st, __VA_ARGS__); \
    return hipGetLastError();                                                                     \
  } while (0)

}  // namespace

int generic_chunk_for(int D, int M, int which) {
  // which: 0 forward, 1 seg state, 2 bwd dq, 3 bwd dkdv; largest TC whose
  // LDS footprint fits the 160 KiB of a gfx950 CU.
  const size_t cap = 160 * 1024;
  for (int tc : {32, 16}) {
    size_t b = which == 0 ? lds_fwd(tc, D, M)
               : which == 1 ? lds_seg(tc, D, M)
               : which == 2 ? lds_bwd_dq(tc, D, M)
                            : lds_bwd_dkdv(tc, D, M);
    if (b <= cap) return tc;
  }
  return 0;
}

hipError_t launch_seg_state_generic(int dtype, const SegGeom& g, const void* k, const void* v, float* s_out,
                                    int64_t s_stride, float* z_out, int64_t z_stride, hipStream_t st) {
  const int64_t grid = g.BH * g.P;
#define LA_SEG(T, TC)                                                                             \
  LA_LAUNCH((k_seg_state<T, TC>), grid, lds_seg(TC, g.D, g.M), st, static_cast<const T*>(k),     \
            static_cast<const T*>(v), s_out, s_stride, z_out, z_stride, g.N, g.D, g.M, g.P, g.seg_len)
  if (dtype == 0) {
    if (g.chunk == 32) LA_SEG(float, 32);
    LA_SEG(float, 16);
  } else {
    if (g.chunk == 32) LA_SEG(bf16_t, 32);
    LA_SEG(bf16_t, 16);
  }
#undef LA_SEG
}

hipError_t launch_seg_scan(float* agg, int64_t BH, int P, int D, int M, int reverse, const float* init_s,
                           const float* init_z, float* tot_s, int64_t ts_stride, float* tot_z, int64_t tz_stride,
                           hipStream_t st) {
  const int64_t E = state_elems(D, M);
  const int64_t nb = (E + NT - 1) / NT;
  hipLaunchKernelGGL(k_seg_scan, dim3(static_cast<unsigned>(BH * nb)), dim3(NT), 0, st, agg, P, E, nb, reverse,
                     static_cast<int64_t>(D) * M, init_s, init_z, tot_s, ts_stride, tot_z, tz_stride);
  return hipGetLastError();
}

hipError_t launch_forward_generic(int dtype, int causal, const SegGeom& g, const void* q, const void* k,
                                  const void* v, void* out, float* den_out, const float* carry,
                                  hipStream_t st) {
  const int64_t grid = g.BH * g.P;
#define LA_FWD(T, TC, C)                                                                          \
  LA_LAUNCH((k_forward<T, TC, C>), grid, lds_fwd(TC, g.D, g.M), st, static_cast<const T*>(q),    \
            static_cast<const T*>(k), static_cast<const T*>(v), static_cast<T*>(out), den_out, carry, \
            g.N, g.D, g.M, g.P, g.seg_len)
#define LA_FWD_C(T, TC) \
  if (causal) LA_FWD(T, TC, true); \
  LA_FWD(T, TC, false)
  if (dtype == 0) {
    if (g.chunk == 32) { LA_FWD_C(float, 32); }
    LA_FWD_C(float, 16);
  } else {
    if (g.chunk == 32) { LA_FWD_C(bf16_t, 32); }
    LA_FWD_C(bf16_t, 16);
  }
#undef LA_FWD_C
#undef LA_FWD
}

hipError_t launch_bwd_dq_generic(int dtype, int causal, const SegGeom& g, const void* q, const void* k,
                                 const void* v, const void* dout, const float* carry_s, void* dq, float* r_agg,
                                 float* c_out, float* den_out, hipStream_t st) {
  const int64_t grid = g.BH * g.P;
  const bool big = g.D * g.M > 16 * NT;
#define LA_DQ(T, TC, C, R)                                                                        \
  LA_LAUNCH((k_bwd_dq<T, TC, C, R>), grid, lds_bwd_dq(TC, g.D, g.M), st, static_cast<const T*>(q), \
            static_cast<const T*>(k), static_cast<const T*>(v), static_cast<const T*>(dout),       \
            carry_s, static_cast<T*>(dq), r_agg, c_out, den_out, g.N, g.D, g.M, g.P, g.seg_len)
#define LA_DQ_R(T, TC, C) \
  if (big) LA_DQ(T, TC, C, 64); \
  LA_DQ(T, TC, C, 16)
#define LA_DQ_C(T, TC) \
  if (causal) { LA_DQ_R(T, TC, true); } \
  LA_DQ_R(T, TC, false)
  if (dtype == 0) {
    if (g.chunk == 32) { LA_DQ_C(float, 32); }
    LA_DQ_C(float, 16);
  } else {
    if (g.chunk == 32) { LA_DQ_C(bf16_t, 32); }
    LA_DQ_C(bf16_t, 16);
  }
#undef LA_DQ_C
#undef LA_DQ_R
#undef LA_DQ
}

hipError_t launch_bwd_dkdv_generic(int dtype, int causal, const SegGeom& g, const void* q, const void* k,
                                   const void* v, const void* dout, const float* den, const float* c,
                                   const float* carry_r, void* dk, void* dv, hipStream_t st) {
  const int64_t grid = g.BH * g.P;
#define LA_KV(T, TC, C)                                                                           \
  LA_LAUNCH((k_bwd_dkdv<T, TC, C>), grid, lds_bwd_dkdv(TC, g.D, g.M), st, static_cast<const T*>(q), \
            static_cast<const T*>(k), static_cast<const T*>(v), static_cast<const T*>(dout),       \
            den, c, carry_r, static_cast<T*>(dk), static_cast<T*>(dv), g.N, g.D, g.M, g.P,         \
            g.seg_len)
#define LA_KV_C(T, TC) \
  if (causal) LA_KV(T, TC, true); \
  LA_KV(T, TC, false)
  if (dtype == 0) {
    if (g.chunk == 32) { LA_KV_C(float, 32); }
    LA_KV_C(float, 16);
  } else {
    if (g.chunk == 32) { LA_KV_C(bf16_t, 32); }
    LA_KV_C(bf16_t, 16);
  }
#undef LA_KV_C
#undef LA_KV
}

}  // namespace la
