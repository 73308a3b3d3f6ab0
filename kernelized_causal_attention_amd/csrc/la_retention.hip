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

// x moved across lanes by a DPP control (CTRL), into the rows of ROW_MASK;
// lanes with no source, and rows outside the mask, receive 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_or_zero(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xf, false));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS
// round trips): shifts by 1, 2, 4, 8 within each 16-lane row, then row 0's
// total into row 1 and row 2's into row 3 (row_bcast:15), then the total of
// rows 0-1 into rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ float wave_incl_scan(float x) {
  x += dpp_or_zero<0x111, 0xf>(x);  // row_shr:1
  x += dpp_or_zero<0x112, 0xf>(x);  // row_shr:2
  x += dpp_or_zero<0x114, 0xf>(x);  // row_shr:4
  x += dpp_or_zero<0x118, 0xf>(x);  // row_shr:8
  x += dpp_or_zero<0x142, 0xa>(x);  // row_bcast:15
  x += dpp_or_zero<0x143, 0xc>(x);  // row_bcast:31
  return x;
}

// Lane 63's value (the chunk's total log decay), wave-uniform.
__device__ __forceinline__ float last_lane(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// log gamma of token cc0 + l (zero past the head's end: no decay there);
// values below -80 are taken as -80 (gamma ~ 2e-35, i.e. 0) so that a full
// reset never forms -inf - (-inf); NaN passes through.
__device__ __forceinline__ float gate(rsrc_t rl, int l, int64_t cc0) {
  const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, l * 4, static_cast<int>(cc0 * 4), 0));
  return x < -80.f ? -80.f : x;
}

// The kernels keep a chunk's running log decay in base-2 units
// (b = sum of log2 gamma = sum of log gamma / ln 2), so that every decay
// factor is a single hardware 2^x; sums handed to other passes (Lambda) are
// converted back to natural log.
constexpr float kLog2e = 1.44269504088896341f;
constexpr float kLn2 = 0.693147180559945309f;
__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

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
    const float s = ex2(bT - __shfl(b, j, 64));
    *reinterpret_cast<i16x8*>(lds + j * G::LD + c8 * 8) = pack8(unpack8(__builtin_bit_cast(i16x8, raw[r])) * s);
  }
}

// Registers -> LDS with row j times 2^(b_j) (<= 1).
template <int DIM>
__device__ __forceinline__ void store_tile_decay(uint16_t* lds, const i32x4 (&raw)[Geo<DIM>::PC], float b) {
  using G = Geo<DIM>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + NT * r;
    const int j = p / G::ROW8, c8 = p % G::ROW8;
    const float s = ex2(__shfl(b, j, 64));
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

// S <- 2^(bT) S + Ks^T V  (Ks: the chunk's keys already scaled by
// 2^(bT - b_j)).
template <int DIM>
__device__ __forceinline__ void decay_update(f32x4_t (&Sacc)[Geo<DIM>::DT][Geo<DIM>::NTL], float bT,
                                             const uint16_t* sKs, const uint16_t* sV, int w, int g, int li) {
  using G = Geo<DIM>;
  const float dk = ex2(bT);
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
  // query (key) row tile of this wave; odd workgroups take the tiles in
  // reverse so that two workgroups on a CU give each SIMD the same
  // triangular intra-chunk work
  const int rw = (blockIdx.x & 1) ? 3 - w : w;
  uint16_t* sOut = sST + DIM * LD + w * 16 * LD;  // this wave's output staging tile
  float* sB = reinterpret_cast<float*>(sST + DIM * LD + 4 * 16 * LD) + 64 * w;  // this wave's copy of b
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
  const int i = 16 * rw + li;

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
    const float b = wave_incl_scan(lgv * kLog2e);  // lane l: b_l
    const float bT = last_lane(b);
    sB[l] = b;
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
    // scores A^T[j][i] = (k_j . q_i) 2^(b_i - b_j) over key tiles t <= rw;
    // below the diagonal tile every key precedes the query (b_i - b_j <= 0),
    // on it keys j > i are selected away (their 2^x may be +inf)
    i16x4 at[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      at[t] = i16x4{0, 0, 0, 0};
      if (t <= rw) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma(lds8(sK + (16 * t + li) * LD + 8 * g + 32 * s), qf[s], acc);
        const f32x4_t bj = *reinterpret_cast<const f32x4_t*>(sB + 16 * t + 4 * g);
        if (t < rw) {
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] *= ex2(bi - bj[u]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] = 4 * g + u <= li ? acc[u] * ex2(bi - bj[u]) : 0.f;
        }
        at[t] = pack4(acc);
      }
    }
    // Y^T = 2^(b_i) S^T q_i + V^T A^T
    const float di = ex2(bi);
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
      if (2 * tp <= rw) {
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
    for (int n = 0; n < NTL; ++n) stage_piece<DIM>(sOut, pack4(o[n]), li, g, n);
    store_staged<DIM, DIM>(sOut, ry, 16 * rw, 0, soff);
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
                                                         int64_t N, int P, int nseg, int seg_len) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, PC = G::PC, DT = G::DT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sKs = smem;
  uint16_t* sV = sKs + T * LD;
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / nseg;  // segments 0 .. nseg - 1 of each head
  const int seg = blockIdx.x % nseg;
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
    const float b = wave_incl_scan(lgv * kLog2e);
    const float bT = last_lane(b);
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
  if (tid == 0) rec[DIM * DIM] = lam * kLn2;
}

// Segment aggregates at D = 64 with wave-private chunks (the layout of the
// linear-attention segment pass).  The workgroup first sums the log decay
// (base 2) of every chunk of the segment and scans those totals from the
// end, so that each key can be weighted when staged by its decay to the
// segment's end, 2^(Lambda - L_j) = 2^((b_T - b_j) + later) <= 1 (b the
// in-chunk scan, later the summed decay of the chunks after it); wave w
// then sums chunks w, w + 4, ... into a 64 x 64 partial of its own with no
// rescaling between chunks, and the four partials are added in wave order.
// Segments of more than kRetSegWaveChunks chunks use k_ret_seg_state.
constexpr int kRetSegWaveChunks = NT;
__global__ __launch_bounds__(NT, 2) void k_ret_seg_wave64(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                         const float* __restrict__ lg, float* __restrict__ recs,
                                                         int64_t N, int P, int nseg, int seg_len) {
  constexpr int DIM = 64, LD = DIM + kLdsPad;
  constexpr int PW = T * DIM / 8 / 64;  // 16-byte pieces per lane per chunk tile
  constexpr int RP = DIM + 4;           // fp32 row stride of the partials in LDS
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* sK = smem + w * 2 * T * LD;
  uint16_t* sV = sK + T * LD;
  float* sLater = reinterpret_cast<float*>(smem + 4 * 2 * T * LD);  // [chunk]: decay of the later chunks
  float* sW = sLater + kRetSegWaveChunks + 4 + 64 * w;              // this wave's key weights
  float* wsum = sLater + kRetSegWaveChunks;                         // 4 floats
  const int64_t bh = blockIdx.x / nseg;
  const int seg = blockIdx.x % nseg;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const int nch = static_cast<int>((r1 - r0 + T - 1) / T);
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rk = make_rsrc(k + bh * N * DIM, hbytes), rv = make_rsrc(v + bh * N * DIM, hbytes),
               rl = make_rsrc(lg + bh * N, N * 4);
  // chunk totals (tokens past the head's end read 0: no decay), then their
  // exclusive suffix sums: thread tid holds chunk nch - 1 - tid, so a scan
  // over the threads runs from the segment's end
  for (int c = w; c < nch; c += 4) {
    float x = gate(rl, l, r0 + static_cast<int64_t>(c) * T) * kLog2e;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    if (l == 0) sLater[c] = x;
  }
  __syncthreads();
  float lam = 0.f;  // the segment's log2 decay (all chunks)
  {
    const int c = nch - 1 - tid;
    const float t = c >= 0 ? sLater[c] : 0.f;
    const float incl = wave_incl_scan(t);
    if (l == 63) wsum[w] = incl;
    const float up = __shfl_up(incl, 1, 64);
    __syncthreads();
    float before = 0.f;
    for (int u = 0; u < w; ++u) before += wsum[u];
    if (l > 0) before += up;
    lam = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    if (c >= 0) sLater[c] = before;
  }
  __syncthreads();

  f32x4_t S[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) S[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // piece p of lane l: row (64 p + l) / 8, features 8 ((64 p + l) % 8) ..
  i32x4 kr[PW], vr[PW];
  float lgv = 0.f;
  auto fetch = [&](int c) {
    const int64_t cc0 = r0 + static_cast<int64_t>(c) * T;
    const int soff = static_cast<int>(cc0 * DIM * 2);
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      kr[p] = bload16(rk, (64 * p + l) * 16, soff);
      vr[p] = bload16(rv, (64 * p + l) * 16, soff);
    }
    lgv = gate(rl, l, cc0);
  };
  if (w < nch) fetch(w);
  for (int c = w; c < nch; c += 4) {
    // weight of key l of this chunk: 2^((b_T - b_l) + later)
    const float b = wave_incl_scan(lgv * kLog2e);
    sW[l] = ex2(last_lane(b) - b + sLater[c]);
    wave_lds_sync();
    // rows past the head's end loaded as zero
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const int e = 64 * p + l;
      const float wt = sW[e >> 3];
      *reinterpret_cast<i16x8*>(sK + (e >> 3) * LD + (e & 7) * 8) =
          pack8(unpack8(__builtin_bit_cast(i16x8, kr[p])) * wt);
      *reinterpret_cast<i16x8*>(sV + (e >> 3) * LD + (e & 7) * 8) = __builtin_bit_cast(i16x8, vr[p]);
    }
    if (c + 4 < nch) fetch(c + 4);
    // the tiles are private to this wave: its LDS operations complete in
    // order, so only the compiler has to be kept from reordering them
    wave_lds_sync();
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      const int jr = 32 * s + 8 * g + li / 4;
      const int cc = 4 * (li % 4);
      i16x8 a[4], bb[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        a[n] = cat(lds_tr(sK + jr * LD + 16 * n + cc), lds_tr(sK + (jr + 4) * LD + 16 * n + cc));
        bb[n] = cat(lds_tr(sV + jr * LD + 16 * n + cc), lds_tr(sV + (jr + 4) * LD + 16 * n + cc));
      }
#pragma unroll
      for (int dn = 0; dn < 4; ++dn)
#pragma unroll
        for (int mn = 0; mn < 4; ++mn) S[dn][mn] = mfma(a[dn], bb[mn], S[dn][mn]);
    }
    wave_lds_sync();
  }
  // partials to LDS (over the chunk tiles): Sp[w][d][m], rows padded to RP
  __syncthreads();
  float* Sp = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int dn = 0; dn < 4; ++dn)
#pragma unroll
    for (int mn = 0; mn < 4; ++mn)
#pragma unroll
      for (int u = 0; u < 4; ++u) Sp[(w * DIM + 16 * dn + 4 * g + u) * RP + 16 * mn + li] = S[dn][mn][u];
  __syncthreads();
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  float* rec = recs + (bh * P + seg) * E;
  const int m = tid & 63;
  for (int d = tid >> 6; d < DIM; d += 4)
    rec[d * DIM + m] = ((Sp[d * RP + m] + Sp[(DIM + d) * RP + m]) + Sp[(2 * DIM + d) * RP + m]) +
                       Sp[(3 * DIM + d) * RP + m];
  if (tid == 0) rec[DIM * DIM] = lam * kLn2;
}

constexpr int kRetScanBatch = 8;

// Decayed exclusive scan over segments, in place on the S part of the
// records: C_0 = S0 (or 0), C_{p+1} = exp(Lambda_p) C_p + dS_p; record p
// receives C_p; the total C_P goes to tot (when not null; tot may be S0).
__global__ __launch_bounds__(NT) void k_ret_scan(float* __restrict__ recs, int P, int64_t E, int64_t DM, int64_t nb,
                                                 const float* init, float* tot) {
  const int64_t bh = blockIdx.x / nb;
  const int64_t e = (blockIdx.x % nb) * NT + threadIdx.x;
  if (e >= DM) return;
  float carry = init ? init[bh * DM + e] : 0.f;
  // records read kRetScanBatch at a time before any is overwritten (the
  // compiler cannot move a load past the previous record's store itself)
  for (int p0 = 0; p0 < P; p0 += kRetScanBatch) {
    float x[kRetScanBatch], lam[kRetScanBatch];
#pragma unroll
    for (int j = 0; j < kRetScanBatch; ++j) {
      const int p = p0 + j;
      // without a total the last record's aggregate is never needed (and
      // may not have been computed): it is not read
      const bool rd = p < P && (p + 1 < P || tot);
      x[j] = rd ? recs[(bh * P + p) * E + e] : 0.f;
      lam[j] = rd ? recs[(bh * P + p) * E + DM] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kRetScanBatch; ++j) {
      const int p = p0 + j;
      if (p < P) {
        recs[(bh * P + p) * E + e] = carry;
        carry = __expf(lam[j]) * carry + x[j];
      }
    }
  }
  if (tot) tot[bh * DM + e] = carry;
}

// ===========================================================================
// Backward of L = sum(dy * y), by the chain rule through the recurrence:
//   dq_i = S_i dy_i,  R_j = sum_{i>=j} exp(L_i - L_j) q_i dy_i^T,
//   dk_j = R_j v_j,   dv_j = R_j^T k_j,   dS0 = the suffix sum decayed to
//   before the first token,  d log gamma_t = sum_{m>=t} (q_m.dq_m - k_m.dk_m)
// (L_m enters row m's terms with + and column m's with -).  Chunked:
//   dq_i = exp(b_i) S dy_i + sum_{j<=i} exp(b_i - b_j)(dy_i.v_j) k_j
//   dk_j = exp(b_T - b_j) R v_j + sum_{i>=j} exp(b_i - b_j)(dy_i.v_j) q_i
//   dv_j = exp(b_T - b_j) R^T k_j + sum_{i>=j} exp(b_i - b_j)(q_i.k_j) dy_i
//   R (passed to the previous chunk) = exp(b_T) R + sum_i exp(b_i) q_i dy_i^T
// with S the state before the chunk and R the suffix state decayed to the
// chunk's last token.
//
// d log gamma_t is the sum of the pair terms w_ij = exp(L_i - L_j)(q_i.k_j)
// (dy_i.v_j) over the pairs i >= t > j that straddle t.  Summing
// q.dq - k.dk over all later tokens would cancel long runs of large terms
// computed through different bf16 roundings, so it is formed as
//   d log gamma_t = Y + sum_{t <= m < segment end} a_m,
//   a_m = p_m + rowsum_m - colsum_m - r_m,
// Y = <S, R> at the segment's end (the straddling pairs there, from the fp32
// state records), p_m = exp(b_m) q_m^T S dy_m (pairs into the chunk from
// before it), r_m = exp(b_T - b_m) k_m^T R v_m (pairs out of the chunk), and
// the in-chunk pairs' row and column sums from fp32 w_ij.
// ===========================================================================

// X^T layout for the suffix state (as in the linear-attention backward):
// lane holds X[d = 16n + li][m = 16mt + 4g + u], mt = w DT + a.
// X^T[m][d] += sum_j A[j][m] B[j][d] over the chunk's 64 tokens.
template <int DIM>
__device__ __forceinline__ void outer_xt(f32x4_t (&X)[Geo<DIM>::DT][Geo<DIM>::NTL], const uint16_t* sA,
                                         const uint16_t* sB, int w, int g, int li) {
  using G = Geo<DIM>;
#pragma unroll
  for (int s = 0; s < T / 32; ++s) {
    const int jr = 32 * s + 8 * g + li / 4;
    const int cc = 4 * (li % 4);
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
    }
  }
}

// bf16 row-major X[d][m] into LDS from the X^T accumulators.
template <int DIM>
__device__ __forceinline__ void write_x(uint16_t* sX, const f32x4_t (&X)[Geo<DIM>::DT][Geo<DIM>::NTL], int w, int g,
                                        int li) {
  using G = Geo<DIM>;
#pragma unroll
  for (int a = 0; a < G::DT; ++a)
#pragma unroll
    for (int n = 0; n < G::NTL; ++n)
      *reinterpret_cast<i16x4*>(sX + (16 * n + li) * G::LD + 16 * (w * G::DT + a) + 4 * g) = pack4(X[a][n]);
}

template <int DIM>
__device__ __forceinline__ void init_x(f32x4_t (&X)[Geo<DIM>::DT][Geo<DIM>::NTL], const float* __restrict__ src,
                                       int w, int g, int li) {
  using G = Geo<DIM>;
#pragma unroll
  for (int a = 0; a < G::DT; ++a)
#pragma unroll
    for (int n = 0; n < G::NTL; ++n)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        X[a][n][u] = src ? src[(16 * n + li) * DIM + 16 * (w * G::DT + a) + 4 * g + u] : 0.f;
}

// Own-row tile writes (row i of the chunk, features 8g + 32s + e), scaled.
template <int DIM>
__device__ __forceinline__ void put_row(uint16_t* lds, const i32x4 (&raw)[Geo<DIM>::KS], int i, int g, float sc) {
#pragma unroll
  for (int s = 0; s < Geo<DIM>::KS; ++s)
    *reinterpret_cast<i16x8*>(lds + i * Geo<DIM>::LD + 8 * g + 32 * s) =
        sc == 1.f ? __builtin_bit_cast(i16x8, raw[s]) : pack8(unpack8(__builtin_bit_cast(i16x8, raw[s])) * sc);
}

// ---------------------------------------------------------------------------
// Forward sweep: dq, p_i per token (into qdq), the segment's suffix
// aggregate dR = sum_i exp(B_i) q_i dy_i^T (B_i: log decay from the segment
// start through token i) with Lambda in the record's first Z slot, and at
// each inner anchor the state entering it (anch_s, null when the segments
// have no inner anchor).
// ---------------------------------------------------------------------------
template <int DIM>
__global__ __launch_bounds__(NT, DIM == 64 ? 2 : 1) void k_ret_dq(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                 const bf16_t* __restrict__ v, const float* __restrict__ lg,
                                                 const bf16_t* __restrict__ dy, const float* __restrict__ carry,
                                                 bf16_t* __restrict__ dq, float* __restrict__ qdq,
                                                 float* __restrict__ r_agg, float* __restrict__ anch_s, int64_t N,
                                                 int P, int seg_len) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sK = smem;
  uint16_t* sKs = sK + T * LD;
  uint16_t* sV = sKs + T * LD;
  uint16_t* sQ = sV + T * LD;
  uint16_t* sQs = sQ + T * LD;
  uint16_t* sG = sQs + T * LD;
  uint16_t* sS = sG + T * LD;  // bf16 S, row-major [d][m]
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query (key) row tile of this wave; odd workgroups take the tiles in
  // reverse so that two workgroups on a CU give each SIMD the same
  // triangular intra-chunk work
  const int rw = (blockIdx.x & 1) ? 3 - w : w;
  uint16_t* sOut = sS + DIM * LD + w * 16 * LD;  // this wave's output staging tile
  float* sB = reinterpret_cast<float*>(sS + DIM * LD + 4 * 16 * LD) + 64 * w;  // this wave's copy of b
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  const float* cs = carry ? carry + (bh * P + seg) * E : nullptr;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               rg = make_rsrc(dy + hoff, hbytes), rdq = make_rsrc(dq + hoff, hbytes),
               rl = make_rsrc(lg + bh * N, N * 4);
  float* qdqh = qdq + bh * N;
  const int i = 16 * rw + li;
  const int cc = 4 * (li % 4);

  f32x4_t Sacc[DT][NTL], Racc[DT][NTL];
  init_s<DIM>(Sacc, cs, w, g, li);
  init_x<DIM>(Racc, nullptr, w, g, li);
  // bf16 S row-major for the S dy product: element (d, m) from the S layout
  // Sacc[dt][n] = S[16(w DT + dt) + 4g + u][16n + li]
  auto write_s = [&]() {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int n = 0; n < NTL; ++n)
          sS[(16 * (w * DT + dt) + 4 * g + u) * LD + 16 * n + li] = static_cast<uint16_t>(bf(Sacc[dt][n][u]));
  };
  write_s();

  i32x4 kraw[PC], vraw[PC], qraw[KS], graw[KS];
  float lgv;
  auto fetch = [&](int64_t cc0) {
    const int soff = static_cast<int>(cc0 * DIM * 2);
    bload_tile<DIM>(kraw, rk, soff);
    bload_tile<DIM>(vraw, rv, soff);
    bload_q<DIM>(qraw, rq, soff, i, g);
    bload_q<DIM>(graw, rg, soff, i, g);
    lgv = gate(rl, l, cc0);
  };
  fetch(r0);
  float Bc = 0.f;  // log2 decay from the segment start to before this chunk
  const int na = ret_anchors(seg_len);
  for (int64_t c0 = r0; c0 < r1; c0 += T) {
    // at an inner anchor, the state entering this chunk (S[d][m] row-major)
    // for the dk/dv sweep's <S, R> there
    if (anch_s && c0 > r0 && (c0 - r0) % kRetAnchor == 0) {
      float* dst = anch_s + ((bh * P + seg) * na + (c0 - r0) / kRetAnchor - 1) * (DIM * DIM);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int n = 0; n < NTL; ++n) dst[(16 * (w * DT + dt) + 4 * g + u) * DIM + 16 * n + li] = Sacc[dt][n][u];
    }
    const float b = wave_incl_scan(lgv * kLog2e);
    const float bT = last_lane(b);
    const float bi = __shfl(b, i, 64);
    sB[l] = b;
    store_tile_v<DIM>(sK, kraw);
    store_tile_scaled<DIM>(sKs, kraw, b, bT);
    store_tile_v<DIM>(sV, vraw);
    put_row<DIM>(sQ, qraw, i, g, 1.f);
    put_row<DIM>(sQs, qraw, i, g, ex2(Bc + bi));
    put_row<DIM>(sG, graw, i, g, 1.f);
    i16x8 gq[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) gq[s] = __builtin_bit_cast(i16x8, graw[s]);
    __syncthreads();
    const int soff = static_cast<int>(c0 * DIM * 2);
    const int64_t nrow = min(static_cast<int64_t>(T), r1 - c0);
    if (c0 + T < r1) fetch(c0 + T);

    // dQ^T[d][i] = 2^(b_i) (S dy_i)[d] + sum_j K^T B^T
    f32x4_t o[NTL];
    const float di = ex2(bi);
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
      o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) o[n] = mfma(lds8(sS + (16 * n + li) * LD + 8 * g + 32 * s), gq[s], o[n]);
      o[n] *= di;
    }
    // p_i = q_i . 2^(b_i) S dy_i (fp32)
    float qd = 0.f;
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
      const f32x4_t qv = unpack4(*reinterpret_cast<const i16x4*>(sQ + i * LD + 16 * n + 4 * g));
#pragma unroll
      for (int u = 0; u < 4; ++u) qd += qv[u] * o[n][u];
    }
    qd = shfl_sum_groups(qd);
    // B^T[j][i] = (v_j . dy_i) 2^(b_i - b_j), j <= i (as in the forward)
    i16x4 bt[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      if (t <= rw) {
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma(lds8(sV + (16 * t + li) * LD + 8 * g + 32 * s), gq[s], acc);
        const f32x4_t bj = *reinterpret_cast<const f32x4_t*>(sB + 16 * t + 4 * g);
        if (t < rw) {
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] *= ex2(bi - bj[u]);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] = 4 * g + u <= li ? acc[u] * ex2(bi - bj[u]) : 0.f;
        }
      }
      bt[t] = pack4(acc);
    }
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        if (2 * tp <= rw) {
          const int jr = 32 * tp + 4 * g + li / 4;
          const i16x8 a = cat(lds_tr(sK + jr * LD + 16 * n + cc), lds_tr(sK + (jr + 16) * LD + 16 * n + cc));
          o[n] = mfma(a, cat(bt[2 * tp], bt[2 * tp + 1]), o[n]);
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NTL; ++n) stage_piece<DIM>(sOut, pack4(o[n]), li, g, n);
    store_staged<DIM, DIM>(sOut, rdq, 16 * rw, 0, soff);
    if (g == 0 && i < nrow) qdqh[c0 + i] = qd;
    // state and suffix aggregate
    decay_update<DIM>(Sacc, bT, sKs, sV, w, g, li);
    outer_xt<DIM>(Racc, sG, sQs, w, g, li);
    Bc += bT;
    __syncthreads();
    write_s();
  }
  if (r_agg) {
    float* rec = r_agg + (bh * P + seg) * E;
#pragma unroll
    for (int a = 0; a < DT; ++a)
#pragma unroll
      for (int n = 0; n < NTL; ++n)
#pragma unroll
        for (int u = 0; u < 4; ++u) rec[(16 * n + li) * DIM + 16 * (w * DT + a) + 4 * g + u] = Racc[a][n][u];
    if (tid == 0) rec[DIM * DIM] = Bc * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Reverse sweep: dk, dv; completes a_j = p_j + rowsum_j - colsum_j - r_j in
// place in qdq, and forms Y = <S, R> at each inner anchor (anch_y) from the
// states the forward sweep kept there (anch_s).
// carry_r: the suffix state decayed to the segment's last token (or null).
// ---------------------------------------------------------------------------
template <int DIM>
__global__ __launch_bounds__(NT, DIM == 64 ? 2 : 1) void k_ret_dkdv(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                   const bf16_t* __restrict__ v, const float* __restrict__ lg,
                                                   const bf16_t* __restrict__ dy, const float* __restrict__ carry_r,
                                                   bf16_t* __restrict__ dk, bf16_t* __restrict__ dv,
                                                   float* __restrict__ qdq, const float* __restrict__ anch_s,
                                                   float* __restrict__ anch_y, int64_t N, int P, int seg_len) {
  using G = Geo<DIM>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sK = smem;
  uint16_t* sV = sK + T * LD;
  uint16_t* sQ = sV + T * LD;
  uint16_t* sQs = sQ + T * LD;
  uint16_t* sG = sQs + T * LD;
  uint16_t* sR = sG + T * LD;  // bf16 R, row-major [d][m]
  float* sRow = reinterpret_cast<float*>(sR + DIM * LD);  // [wave][row] partial row sums of w
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query (key) row tile of this wave; odd workgroups take the tiles in
  // reverse so that two workgroups on a CU give each SIMD the same
  // triangular intra-chunk work
  const int rw = (blockIdx.x & 1) ? 3 - w : w;
  uint16_t* sDV = reinterpret_cast<uint16_t*>(sRow + 4 * T) + w * 2 * 16 * LD;  // this wave's dv, dk staging
  uint16_t* sDK = sDV + 16 * LD;
  float* sB0 = reinterpret_cast<float*>(reinterpret_cast<uint16_t*>(sRow + 4 * T) + 4 * 2 * 16 * LD);
  float* sB = sB0 + 64 * w;  // this wave's copy of b
  float* sY = sB0 + 4 * 64;  // per-wave parts of <S, R> at an inner anchor
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  const float* cr = carry_r ? carry_r + (bh * P + seg) * E : nullptr;
  const int64_t hoff = bh * N * DIM;
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rq = make_rsrc(q + hoff, hbytes), rk = make_rsrc(k + hoff, hbytes), rv = make_rsrc(v + hoff, hbytes),
               rg = make_rsrc(dy + hoff, hbytes), rdk = make_rsrc(dk + hoff, hbytes),
               rdv = make_rsrc(dv + hoff, hbytes), rl = make_rsrc(lg + bh * N, N * 4);
  float* qdqh = qdq + bh * N;
  const int j = 16 * rw + li;  // this lane's key row
  const int cc = 4 * (li % 4);

  f32x4_t Racc[DT][NTL];
  init_x<DIM>(Racc, cr, w, g, li);
  write_x<DIM>(sR, Racc, w, g, li);

  const int64_t nch = (r1 - r0 + T - 1) / T;
  i32x4 kraw[PC], vraw[PC], qraw[PC], graw[PC];
  float lgv;
  // p_j from the forward sweep, loaded with the chunk's tiles so that the
  // update of a_j at the end of the chunk waits on no load
  float pj = 0.f;
  auto fetch = [&](int64_t cc0) {
    const int soff = static_cast<int>(cc0 * DIM * 2);
    bload_tile<DIM>(kraw, rk, soff);
    bload_tile<DIM>(vraw, rv, soff);
    bload_tile<DIM>(qraw, rq, soff);
    bload_tile<DIM>(graw, rg, soff);
    lgv = gate(rl, l, cc0);
    if (g == 0 && cc0 + j < r1) pj = qdqh[cc0 + j];
  };
  fetch(r0 + (nch - 1) * T);
  const int na = ret_anchors(seg_len);
  for (int64_t ci = nch - 1; ci >= 0; --ci) {
    const int64_t c0 = r0 + ci * T;
    // an inner anchor at the end of this chunk: <S, R> there, with R the
    // suffix state decayed to the chunk's last token (Racc before this
    // chunk) and S the state the dq sweep kept for the anchor
    int yk = -1;
    if (anch_s && c0 + T < r1 && (c0 + T - r0) % kRetAnchor == 0) {
      yk = static_cast<int>((c0 + T - r0) / kRetAnchor) - 1;
      const float* src = anch_s + ((bh * P + seg) * na + yk) * (DIM * DIM);
      float part = 0.f;
#pragma unroll
      for (int a = 0; a < DT; ++a)
#pragma unroll
        for (int n = 0; n < NTL; ++n) {
          const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(src + (16 * n + li) * DIM + 16 * (w * DT + a) + 4 * g);
#pragma unroll
          for (int u = 0; u < 4; ++u) part += Racc[a][n][u] * sv[u];
        }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) part += __shfl_xor(part, off, 64);
      part = shfl_sum_groups(part);
      if (l == 0) sY[w] = part;
    }
    const float b = wave_incl_scan(lgv * kLog2e);
    const float bT = last_lane(b);
    sB[l] = b;
    store_tile_v<DIM>(sK, kraw);
    store_tile_v<DIM>(sV, vraw);
    store_tile_v<DIM>(sQ, qraw);
    store_tile_decay<DIM>(sQs, qraw, b);  // row i times 2^(b_i)
    store_tile_v<DIM>(sG, graw);
    __syncthreads();
    if (yk >= 0 && tid == 0) anch_y[(bh * P + seg) * na + yk] = sY[0] + sY[1] + sY[2] + sY[3];
    const int soff = static_cast<int>(c0 * DIM * 2);
    const int64_t nrow = min(static_cast<int64_t>(T), r1 - c0);
    const float pcur = pj;
    if (ci > 0) fetch(c0 - T);
    // the chunk's compute at raised wave priority, back to 0 before its
    // stores (as in the linear-attention dq sweep; dk/dv 201 -> 195 us here)
    __builtin_amdgcn_s_setprio(2);

    const float bj = __shfl(b, j, 64);
    i16x8 kreg[KS], vreg[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kreg[s] = lds8(sK + j * LD + 8 * g + 32 * s);
      vreg[s] = lds8(sV + j * LD + 8 * g + 32 * s);
    }
    // A[i][j] = (q_i . k_j) 2^(b_i - b_j), Bm[i][j] = (dy_i . v_j) 2^(b_i - b_j),
    // query tiles t >= rw; above the diagonal tile every query follows the
    // key, on it queries i < j are selected away; wv: the pair terms w_ij in
    // fp32
    i16x4 am[4], bm[4];
    float wv[16];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      f32x4_t a = {0.f, 0.f, 0.f, 0.f}, bb = {0.f, 0.f, 0.f, 0.f};
      if (t >= rw) {
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          a = mfma(lds8(sQ + (16 * t + li) * LD + 8 * g + 32 * s), kreg[s], a);
          bb = mfma(lds8(sG + (16 * t + li) * LD + 8 * g + 32 * s), vreg[s], bb);
        }
        const f32x4_t bq = *reinterpret_cast<const f32x4_t*>(sB + 16 * t + 4 * g);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float dec = ex2(bq[u] - bj);
          if (t == rw) dec = 4 * g + u >= li ? dec : 0.f;
          a[u] *= dec;
          wv[4 * t + u] = a[u] * bb[u];
          bb[u] *= dec;
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) wv[4 * t + u] = 0.f;
      }
      am[t] = pack4(a);
      bm[t] = pack4(bb);
    }
    // column sum (key j): over this lane's 16 rows, then the four groups
    float colsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) colsum += wv[r];
    colsum = shfl_sum_groups(colsum);
    // row sums over this wave's 16 keys: halve the 16 values across the
    // lanes of the row in four DPP exchanges, each with a partner whose bit
    // 3, 2, 1, 0 differs (li ^ 8, ^ 7, ^ 2, ^ 1: every lane of the row is
    // counted once); lane li keeps row r = li, i.e. query
    // i = 16 (li / 4) + 4g + li % 4
    {
      float h8[8], h4[4], h2[2];
      const bool b3 = li & 8, b2 = li & 4, b1 = li & 2, b0 = li & 1;
#pragma unroll
      for (int x = 0; x < 8; ++x) h8[x] = (b3 ? wv[x + 8] : wv[x]) + dpp_row<kDppXor8>(b3 ? wv[x] : wv[x + 8]);
#pragma unroll
      for (int x = 0; x < 4; ++x) h4[x] = (b2 ? h8[x + 4] : h8[x]) + dpp_row<kDppXor7>(b2 ? h8[x] : h8[x + 4]);
#pragma unroll
      for (int x = 0; x < 2; ++x) h2[x] = (b1 ? h4[x + 2] : h4[x]) + dpp_row<kDppXor2>(b1 ? h4[x] : h4[x + 2]);
      const float h1 = (b0 ? h2[1] : h2[0]) + dpp_row<kDppXor1>(b0 ? h2[0] : h2[1]);
      sRow[w * T + 16 * (li >> 2) + 4 * g + (li & 3)] = h1;
    }
    const float dj = ex2(bT - bj);
    float kd = 0.f;
#pragma unroll
    for (int n = 0; n < NTL; ++n) {
      // dv^T[m][j] = 2^(b_T - b_j) R^T k_j + sum_i dy^T A
      f32x4_t ov = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int dr = 32 * s + 8 * g + li / 4;
        ov = mfma(cat(lds_tr(sR + dr * LD + 16 * n + cc), lds_tr(sR + (dr + 4) * LD + 16 * n + cc)), kreg[s], ov);
      }
      ov *= dj;
      // dk^T[d][j] = 2^(b_T - b_j) R v_j + sum_i q^T Bm
      f32x4_t ok = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) ok = mfma(lds8(sR + (16 * n + li) * LD + 8 * g + 32 * s), vreg[s], ok);
      ok *= dj;
      // r_j = k_j . 2^(b_T - b_j) R v_j (fp32)
      const f32x4_t kv = unpack4(*reinterpret_cast<const i16x4*>(sK + j * LD + 16 * n + 4 * g));
#pragma unroll
      for (int u = 0; u < 4; ++u) kd += kv[u] * ok[u];
#pragma unroll
      for (int tp = 0; tp < 2; ++tp) {
        if (2 * tp + 1 >= rw) {
          const int ir = 32 * tp + 4 * g + li / 4;
          ov = mfma(cat(lds_tr(sG + ir * LD + 16 * n + cc), lds_tr(sG + (ir + 16) * LD + 16 * n + cc)),
                    cat(am[2 * tp], am[2 * tp + 1]), ov);
          ok = mfma(cat(lds_tr(sQ + ir * LD + 16 * n + cc), lds_tr(sQ + (ir + 16) * LD + 16 * n + cc)),
                    cat(bm[2 * tp], bm[2 * tp + 1]), ok);
        }
      }
      stage_piece<DIM>(sDV, pack4(ov), li, g, n);
      stage_piece<DIM>(sDK, pack4(ok), li, g, n);
    }
    __builtin_amdgcn_s_setprio(0);
    store_staged<DIM, DIM>(sDV, rdv, 16 * rw, 0, soff);
    store_staged<DIM, DIM>(sDK, rdk, 16 * rw, 0, soff);
    kd = shfl_sum_groups(kd);
    // R for the previous chunk: 2^(b_T) R + sum_i 2^(b_i) q_i dy_i^T
    const float dT = ex2(bT);
#pragma unroll
    for (int a = 0; a < DT; ++a)
#pragma unroll
      for (int n = 0; n < NTL; ++n) Racc[a][n] *= dT;
    outer_xt<DIM>(Racc, sG, sQs, w, g, li);
    __syncthreads();
    write_x<DIM>(sR, Racc, w, g, li);
    if (g == 0 && j < nrow) {
      const float rowsum = sRow[j] + sRow[T + j] + sRow[2 * T + j] + sRow[3 * T + j];
      qdqh[c0 + j] = pcur + (rowsum - colsum - kd);
    }
  }
}

// Reverse decayed exclusive scan of the suffix aggregates: record p receives
// the suffix state decayed to segment p's last token,
// C_{P-1} = 0, C_{p-1} = dR_p + exp(Lambda_p) C_p; the total (dS0) goes to tot.
__global__ __launch_bounds__(NT) void k_ret_rscan(float* __restrict__ recs, int P, int64_t E, int64_t DM, int64_t nb,
                                                  float* tot) {
  const int64_t bh = blockIdx.x / nb;
  const int64_t e = (blockIdx.x % nb) * NT + threadIdx.x;
  if (e >= DM) return;
  float carry = 0.f;
  for (int p0 = P - 1; p0 >= 0; p0 -= kRetScanBatch) {
    float x[kRetScanBatch], lam[kRetScanBatch];
#pragma unroll
    for (int j = 0; j < kRetScanBatch; ++j) {
      const int p = p0 - j;
      x[j] = p >= 0 ? recs[(bh * P + p) * E + e] : 0.f;
      lam[j] = p >= 0 ? recs[(bh * P + p) * E + DM] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kRetScanBatch; ++j) {
      const int p = p0 - j;
      if (p >= 0) {
        recs[(bh * P + p) * E + e] = carry;
        carry = x[j] + __expf(lam[j]) * carry;
      }
    }
  }
  if (tot) tot[bh * DM + e] = carry;
}

// d log gamma_t over segment p = [r0, r1), one block per (head, segment),
// from its anchors: for t in [b_k, b_{k+1}) (b_0 = r0, b_k = r0 + k
// kRetAnchor the inner anchors, the last interval ending at r1)
//   d log gamma_t = Y(b_{k+1}) + sum_{t <= m < b_{k+1}} a_m,
// Y at an inner anchor from the dk/dv sweep (anch_y), Y at the segment's end
// = <S, R> there: S the state after its last token (the next segment's carry
// record), R the suffix state decayed to that token (its own reverse-scan
// record); zero for the last segment.
__global__ __launch_bounds__(NT) void k_ret_dlg(const float* __restrict__ a, const float* __restrict__ srecs,
                                                const float* __restrict__ rrecs, const float* __restrict__ anch_y,
                                                float* __restrict__ dlg, int64_t N, int P, int seg_len, int64_t E,
                                                int64_t DM) {
  __shared__ float wsum[4];
  const int64_t bh = blockIdx.x / P;
  const int p = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(p) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const float* ah = a + bh * N;
  float* oh = dlg + bh * N;
  const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;
  float y = 0.f;
  if (p + 1 < P) {
    const float* s = srecs + (bh * P + p + 1) * E;
    const float* r = rrecs + (bh * P + p) * E;
    // unrolled so that eight pairs of loads are in flight at once (the sum
    // keeps its order)
#pragma unroll 8
    for (int64_t e = tid; e < DM; e += NT) y += s[e] * r[e];
  }
  y += __shfl_xor(y, 1, 64);
  y += __shfl_xor(y, 2, 64);
  y += __shfl_xor(y, 4, 64);
  y += __shfl_xor(y, 8, 64);
  y += __shfl_xor(y, 16, 64);
  y += __shfl_xor(y, 32, 64);
  if (l == 0) wsum[w] = y;
  __syncthreads();
  float carry = wsum[0] + wsum[1] + wsum[2] + wsum[3];
  __syncthreads();
  // inner anchors of this segment: b_k < r1 for k = 1 .. K
  const int na = ret_anchors(seg_len);
  const int K = static_cast<int>((r1 - r0 - 1) / kRetAnchor);
  // Each interval is walked from its top in blocks of NT * kDlgPer tokens
  // (kRetAnchor = one block): thread tid holds the kDlgPer consecutive tokens
  // ending kDlgPer * tid below the block's top, so a block's suffix sums are
  // each thread's own suffix sums plus an exclusive scan of the thread
  // totals over the threads.
  constexpr int kDlgPer = 4;
  int64_t top = r1;
  for (int kk = K; kk >= 0; --kk) {
    const int64_t lo = r0 + static_cast<int64_t>(kk) * kRetAnchor;
    for (int64_t hi = top; hi > lo; hi -= NT * kDlgPer) {
      const int64_t t0 = hi - static_cast<int64_t>(kDlgPer) * (tid + 1);
      float x[kDlgPer];
#pragma unroll
      for (int u = 0; u < kDlgPer; ++u) x[u] = t0 + u >= lo ? ah[t0 + u] : 0.f;
#pragma unroll
      for (int u = kDlgPer - 2; u >= 0; --u) x[u] += x[u + 1];
      const float incl = wave_incl_scan(x[0]);
      if (l == 63) wsum[w] = incl;
      const float up = __shfl_up(incl, 1, 64);
      __syncthreads();
      float before = carry;
      for (int u = 0; u < w; ++u) before += wsum[u];
      if (l > 0) before += up;  // the totals of this wave's earlier lanes
#pragma unroll
      for (int u = 0; u < kDlgPer; ++u)
        if (t0 + u >= lo) oh[t0 + u] = before + x[u];
      const float total = wsum[0] + wsum[1] + wsum[2] + wsum[3];
      __syncthreads();
      carry += total;
    }
    if (kk > 0) carry = anch_y[(bh * P + p) * na + kk - 1];
    top = lo;
  }
}

// each also holds a 16-row output staging tile per wave (two in the dk / dv
// sweep) and each wave's 64-float copy of the chunk's b
size_t lds_ret_fwd(int dim) {
  return (3 * T * (dim + kLdsPad) + dim * (dim + kLdsPad) + 4 * 16 * (dim + kLdsPad)) * sizeof(uint16_t) +
         4 * T * sizeof(float);
}
size_t lds_ret_seg(int dim) { return 2 * T * (dim + kLdsPad) * sizeof(uint16_t); }
size_t lds_ret_seg_wave64() {
  const size_t tiles = 4 * 2 * T * (64 + kLdsPad) * sizeof(uint16_t);
  const size_t parts = 4 * 64 * (64 + 4) * sizeof(float);
  return (tiles > parts ? tiles : parts) + (kRetSegWaveChunks + 4 + 4 * 64) * sizeof(float);
}
size_t lds_ret_dq(int dim) {
  return (6 * T * (dim + kLdsPad) + dim * (dim + kLdsPad) + 4 * 16 * (dim + kLdsPad)) * sizeof(uint16_t) +
         4 * T * sizeof(float);
}
size_t lds_ret_dkdv(int dim) {
  return (5 * T * (dim + kLdsPad) + dim * (dim + kLdsPad) + 4 * 2 * 16 * (dim + kLdsPad)) * sizeof(uint16_t) +
         2 * 4 * T * sizeof(float) + 4 * sizeof(float);
}

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
  const int nseg = g.nseg > 0 ? g.nseg : g.P;
  const int64_t grid = g.BH * nseg;
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  if (g.D == 64 && (g.seg_len + T - 1) / T <= kRetSegWaveChunks)
    LA_RLAUNCH(k_ret_seg_wave64, grid, lds_ret_seg_wave64(), st, K, V, lg, recs, g.N, g.P, nseg, g.seg_len);
  if (g.D == 64) LA_RLAUNCH((k_ret_seg_state<64>), grid, lds_ret_seg(64), st, K, V, lg, recs, g.N, g.P, nseg, g.seg_len);
  if (g.D == 128)
    LA_RLAUNCH((k_ret_seg_state<128>), grid, lds_ret_seg(128), st, K, V, lg, recs, g.N, g.P, nseg, g.seg_len);
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

hipError_t launch_ret_bwd_dq(const SegGeom& g, const void* q, const void* k, const void* v, const float* lg,
                             const void* dy, const float* carry_s, float* r_agg, void* dq, float* a, float* anch_s,
                             hipStream_t st) {
  const int64_t grid = g.BH * g.P;
  const bf16_t* Q = static_cast<const bf16_t*>(q);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  const bf16_t* Gy = static_cast<const bf16_t*>(dy);
  bf16_t* dQ = static_cast<bf16_t*>(dq);
  if (g.D == 64)
    LA_RLAUNCH((k_ret_dq<64>), grid, lds_ret_dq(64), st, Q, K, V, lg, Gy, carry_s, dQ, a, r_agg, anch_s, g.N, g.P,
               g.seg_len);
  if (g.D == 128)
    LA_RLAUNCH((k_ret_dq<128>), grid, lds_ret_dq(128), st, Q, K, V, lg, Gy, carry_s, dQ, a, r_agg, anch_s, g.N,
               g.P, g.seg_len);
  return hipErrorNotSupported;
}

hipError_t launch_ret_rscan(const SegGeom& g, float* r_agg, float* dS0, hipStream_t st) {
  const int64_t DM = static_cast<int64_t>(g.D) * g.M;
  const int64_t nb = (DM + NT - 1) / NT;
  hipLaunchKernelGGL(k_ret_rscan, dim3(static_cast<unsigned>(g.BH * nb)), dim3(NT), 0, st, r_agg, g.P,
                     state_elems(g.D, g.M), DM, nb, dS0);
  return hipGetLastError();
}

hipError_t launch_ret_bwd_dkdv(const SegGeom& g, const void* q, const void* k, const void* v, const float* lg,
                               const void* dy, const float* r_agg, void* dk, void* dv, float* a, const float* anch_s,
                               float* anch_y, hipStream_t st) {
  const int64_t grid = g.BH * g.P;
  const bf16_t* Q = static_cast<const bf16_t*>(q);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  const bf16_t* Gy = static_cast<const bf16_t*>(dy);
  bf16_t* dK = static_cast<bf16_t*>(dk);
  bf16_t* dV = static_cast<bf16_t*>(dv);
  if (g.D == 64)
    LA_RLAUNCH((k_ret_dkdv<64>), grid, lds_ret_dkdv(64), st, Q, K, V, lg, Gy, r_agg, dK, dV, a, anch_s, anch_y, g.N,
               g.P, g.seg_len);
  if (g.D == 128)
    LA_RLAUNCH((k_ret_dkdv<128>), grid, lds_ret_dkdv(128), st, Q, K, V, lg, Gy, r_agg, dK, dV, a, anch_s, anch_y,
               g.N, g.P, g.seg_len);
  return hipErrorNotSupported;
}

hipError_t launch_ret_dlg(const SegGeom& g, const float* a, const float* carry_s, const float* r_agg,
                          const float* anch_y, float* dlg, hipStream_t st) {
  hipLaunchKernelGGL(k_ret_dlg, dim3(static_cast<unsigned>(g.BH * g.P)), dim3(NT), 0, st, a, carry_s, r_agg, anch_y, dlg, g.N,
                     g.P, g.seg_len, state_elems(g.D, g.M), static_cast<int64_t>(g.D) * g.M);
  return hipGetLastError();
}

}  // namespace la
