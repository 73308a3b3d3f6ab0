// bf16 MFMA kernels for the chunked causal / non-causal forward (gfx950).
//
// Method ("[Paper walkthrough] Transformers are RNNs", wkq9411.github.io):
// phi = elu + 1 (section 2); S_i = sum_{j<=i} phi(K_j) V_j^T,
// Z_i = sum_{j<=i} phi(K_j), out_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i
// (section 3, eq:mask and eq:output); non-causal phi(Q)(phi(K)^T V)
// (section 2, eq:linear).
//
// Layout of the work.  One workgroup (4 wave64s) walks one segment of one
// (b,h) sequence in chunks of T = 64 tokens.  For a chunk that starts after
// state (S, Z) the causal sums split exactly (the sums are associative):
//   num_i = phi(Q_i)^T S + sum_{j<=i in chunk} (phi(Q_i).phi(K_j)) V_j
//   den_i = phi(Q_i)^T Z + sum_{j<=i in chunk}  phi(Q_i).phi(K_j)
// Wave w owns rows i = 16w .. 16w+15 of the chunk.  It computes the scores
// transposed, A^T = phi(K) phi(Q)^T, one 16x16 tile per key tile j <= i; in
// the MFMA accumulator layout a lane then holds four consecutive keys of one
// query, so two key tiles, rounded to bf16, are directly the B operand of
// the next product O^T = V^T A^T (with the key index permuted the same way
// on the V side, read with LDS transpose loads).  Scores are split into a
// bf16 high part and a bf16 remainder so that the near-constant scores
// phi(Q).phi(K) ~ D keep their small spread through the bf16 operand.  The
// carried state enters as O^T += S^T phi(Q)^T with S^T kept in LDS as bf16;
// S itself stays fp32 in MFMA accumulators (each wave owns D/4 rows of it)
// and Z is fp32.
// Denominators use the same (hi + lo) scores and bf16 phi(Q) as the
// numerator, so each output row is a convex combination of the weights
// actually applied.
//
// Operands per chunk: phi(Q) rows go straight from HBM to registers (only
// their wave needs them); phi(K) and V are staged once per chunk in LDS,
// token-major.  The next chunk's Q, K, V are loaded into registers while the
// current chunk computes.
#include "la_internal.h"
#include "la_mfma_common.h"

namespace la {
namespace {

using namespace mf;

constexpr int NT = kNT;
constexpr int T = kT;

// Waves per workgroup: 4 at D = 64; 8 at D = 128, where the pairs of waves
// on one 16-row query tile split the output columns and every wave owns one
// 16-row slab of the state, so that a wave's registers stay within what
// two resident waves per SIMD allow.
template <int DIM>
constexpr int kFwdWaves = DIM == 128 ? 8 : 4;

// S (fp32 accumulators) -> S^T bf16 in LDS; Z -> LDS as a bf16 pair
// (hi at sZ[d], the rounding remainder lo at sZ[DIM + d]), the operand of the
// denominator's MFMA.
template <int DIM, int NW>
__device__ __forceinline__ void write_state(uint16_t* sST, uint16_t* sZ,
                                            const f32x4_t (&Sacc)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)],
                                            const f32x4_t (&zacc)[(Geo<DIM, NW>::DT)], int w, int g, int li) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    const int d0 = 16 * (w * G::DT + dt);
#pragma unroll
    for (int n = 0; n < G::NTL; ++n)
      *reinterpret_cast<i16x4*>(sST + (16 * n + li) * G::LD + d0 + 4 * g) = pack4(Sacc[dt][n]);
    if (li == 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const short hi = bf(zacc[dt][u]);
        sZ[d0 + 4 * g + u] = static_cast<uint16_t>(hi);
        sZ[DIM + d0 + 4 * g + u] = static_cast<uint16_t>(bf(zacc[dt][u] - fb(hi)));
      }
    }
  }
}

// S += phi(K_c)^T V_c and Z += colsum phi(K_c) for this wave's state rows
// (TT-token chunk tiles).
template <int DIM, int NW, int TT = T>
__device__ __forceinline__ void state_update(f32x4_t (&Sacc)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)],
                                             f32x4_t (&zacc)[(Geo<DIM, NW>::DT)], const uint16_t* sKf,
                                             const uint16_t* sV, int w, int g, int li) {
  using G = Geo<DIM, NW>;
  const short one = 0x3f80;  // bf16 1.0
  const i16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    const int d0 = 16 * (w * G::DT + dt);
#pragma unroll
    for (int s = 0; s < TT / 32; ++s) {
      const int jr = 32 * s + 8 * g + li / 4;
      const int cc = 4 * (li % 4);
      const i16x8 a = cat(lds_tr(sKf + jr * G::LD + d0 + cc), lds_tr(sKf + (jr + 4) * G::LD + d0 + cc));
      zacc[dt] = mfma(a, ones, zacc[dt]);
#pragma unroll
      for (int n = 0; n < G::NTL; ++n) {
        const i16x8 b = cat(lds_tr(sV + jr * G::LD + 16 * n + cc), lds_tr(sV + (jr + 4) * G::LD + 16 * n + cc));
        Sacc[dt][n] = mfma(a, b, Sacc[dt][n]);
      }
    }
  }
}

template <int DIM, int NW>
__device__ __forceinline__ void init_state(f32x4_t (&Sacc)[(Geo<DIM, NW>::DT)][(Geo<DIM, NW>::NTL)],
                                           f32x4_t (&zacc)[(Geo<DIM, NW>::DT)], const float* __restrict__ cs, int w,
                                           int g, int li) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int dt = 0; dt < G::DT; ++dt) {
    const int d0 = 16 * (w * G::DT + dt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = d0 + 4 * g + u;
#pragma unroll
      for (int n = 0; n < G::NTL; ++n) Sacc[dt][n][u] = cs ? cs[d * DIM + 16 * n + li] : 0.f;
      zacc[dt][u] = cs ? cs[DIM * DIM + d] : 0.f;
    }
  }
}

// One chunk's outputs for this wave: query tile rt (phi(Q) rows in qf),
// output column tiles nb .. nb + NTW - 1.  Intra-chunk scores (masked, as a
// bf16 hi + lo pair), the denominator, the inter-chunk product S^T phi(Q)^T
// and the intra-chunk V^T A^T; returns den for query row li.
template <int DIM, int NW, bool CAUSAL, int NTW>
__device__ __forceinline__ float chunk_outputs(f32x4_t (&o)[NTW], const i16x8 (&qf)[(Geo<DIM, NW>::KS)],
                                               const uint16_t* sKf, const uint16_t* sV, const uint16_t* sST,
                                               const uint16_t* sZ, int rt, int nb, int g, int li) {
  using G = Geo<DIM, NW>;
  constexpr int LD = G::LD, KS = G::KS;
  const short one = 0x3f80;  // bf16 1.0
  const i16x8 ones = {one, one, one, one, one, one, one, one};
  // Intra-chunk scores A^T (key tiles t <= rt), masked.  With phi ~ 1 + x
  // the scores sit near D with a small spread, so one bf16 rounding would
  // lose most of that spread; each score is carried as hi + lo, two bf16
  // values whose sum keeps ~16 significant bits, and both enter the MFMA.
  i16x4 ahi[4], alo[4];
  if (CAUSAL) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      ahi[t] = i16x4{0, 0, 0, 0};
      alo[t] = i16x4{0, 0, 0, 0};
      if (t <= rt) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) acc = mfma(lds8(sKf + (16 * t + li) * LD + 8 * g + 32 * s), qf[s], acc);
        if (t == rt) {
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (4 * g + u > li) acc[u] = 0.f;
        }
        ahi[t] = pack4(acc);
        alo[t] = pack4(acc - unpack4(ahi[t]));
      }
    }
  }
  // The denominator on the MFMA: the inter-chunk part phi(Q_i)^T Z with
  // every row of the A operand equal to Z (as its bf16 hi and lo parts, ~16
  // significant bits), and below the intra-chunk part, the sum of the same
  // hi + lo scores the numerator uses, against a ones operand.  Every row
  // of dz ends up holding den for query li.
  f32x4_t dz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    dz = mfma(lds8(sZ + 8 * g + 32 * s), qf[s], dz);
    dz = mfma(lds8(sZ + DIM + 8 * g + 32 * s), qf[s], dz);
  }

  // O^T = S^T phi(Q)^T (+ V^T A^T), this wave's output tiles
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) o[n] = mfma(lds8(sST + (16 * (nb + n) + li) * LD + 8 * g + 32 * s), qf[s], o[n]);
  }
  if (CAUSAL) {
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
      if (2 * tp <= rt) {
        const i16x8 bhi = cat(ahi[2 * tp], ahi[2 * tp + 1]);
        const i16x8 blo = cat(alo[2 * tp], alo[2 * tp + 1]);
        dz = mfma(ones, bhi, dz);
        dz = mfma(ones, blo, dz);
        const int jr = 32 * tp + 4 * g + li / 4;
        const int cc = 4 * (li % 4);
#pragma unroll
        for (int n = 0; n < NTW; ++n) {
          const int m0 = 16 * (nb + n) + cc;
          const i16x8 a = cat(lds_tr(sV + jr * LD + m0), lds_tr(sV + (jr + 16) * LD + m0));
          o[n] = mfma(a, bhi, o[n]);
          o[n] = mfma(a, blo, o[n]);
        }
      }
    }
  }
  return dz[0];
}

// ---------------------------------------------------------------------------
template <int DIM, bool CAUSAL>
__global__ __launch_bounds__(64 * kFwdWaves<DIM>, 2) void k_fwd_mfma(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                 const bf16_t* __restrict__ v, bf16_t* __restrict__ out,
                                                 float* __restrict__ den_out, const float* __restrict__ carry,
                                                 int64_t N, int P, int seg_len) {
  constexpr int NW = kFwdWaves<DIM>;
  using G = Geo<DIM, NW>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  constexpr int NCG = NW / 4;       // column groups per query tile
  constexpr int NTW = NTL / NCG;    // output tiles per wave
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sKf = smem;
  uint16_t* sV = sKf + T * LD;
  uint16_t* sST = sV + T * LD;
  uint16_t* sZ = sST + DIM * LD;  // Z as bf16 hi [DIM], lo [DIM]
  // With two waves per query tile, phi(Q) is staged once in LDS rather than
  // computed by both waves of a pair from their own loads.
  constexpr bool kQInLds = NCG > 1;
  uint16_t* sQf = sZ + 2 * DIM;
  // per-wave output staging: 16 rows x NTW * 16 columns
  constexpr int OC = NTW * 16;
  uint16_t* sOut = sQf + (kQInLds ? T * LD : 0);

  // w is made wave-uniform (an SGPR) so that branches on it are scalar: an
  // MFMA under an EXEC-masked branch still writes every lane.
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query row tile; the triangular intra-chunk work grows with it, so odd
  // workgroups take the tiles in reverse and two workgroups sharing a CU
  // give every SIMD the same total
  const int rt = (blockIdx.x & 1) ? 3 - (w & 3) : (w & 3);
  const int nb = NCG == 1 ? 0 : (w >> 2) * NTW;  // first output tile of this wave
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  const float* cs = carry ? (CAUSAL ? carry + (bh * P + seg) * E : carry + bh * E) : nullptr;
  // Buffer loads and stores over the head's rows (past its end: zero / dropped),
  // so that no load or store sits under a branch: every chunk issues the same
  // memory operations, and the wait for the prefetched tiles at the top of
  // the loop need not also wait for the previous chunk's stores.
  const rsrc_t rq = make_rsrc(q + bh * N * DIM, N * DIM * 2);
  const rsrc_t rk = make_rsrc(k + bh * N * DIM, N * DIM * 2);
  const rsrc_t rv = make_rsrc(v + bh * N * DIM, N * DIM * 2);
  const rsrc_t ro = make_rsrc(out ? out + bh * N * DIM : nullptr, out ? N * DIM * 2 : 0);
  const rsrc_t rd = make_rsrc(den_out ? den_out + bh * N : nullptr, den_out ? N * 4 : 0);
  const int i = 16 * rt + li;  // this lane's query row within the chunk
  // den is stored by the 16 lanes of group 0 of the waves holding column
  // tile 0; the other lanes aim past the range
  const int den_voff = (g == 0 && nb == 0) ? 4 * i : static_cast<int>(4 * N);
  uint16_t* sO = sOut + w * 16 * (OC + kLdsPad);

  f32x4_t Sacc[DT][NTL];
  f32x4_t zacc[DT];
  init_state<DIM, NW>(Sacc, zacc, cs, w, g, li);
  write_state<DIM, NW>(sST, sZ, Sacc, zacc, w, g, li);

  int64_t c0 = r0;
  int nrow = static_cast<int>(min(static_cast<int64_t>(T), r1 - c0));
  constexpr int QN = kQInLds ? PC : KS;  // q pieces held per lane
  i32x4 kraw[PC], vraw[PC], qraw[QN];
  // Rows of a chunk past the segment's end lie past the head's end (segments
  // are whole chunks), so the buffer range check zeroes them.  The loads
  // keep one order (K, V, Q: the scheduler may not move them), and the first
  // chunk runs as a copy of the loop body ahead of the loop, so that every
  // path into the loop's top has the same memory operations after the
  // prefetch: the wait for the tiles then counts the previous chunk's
  // stores as still in flight instead of waiting for them too.
  auto fetch = [&](int64_t cc0) {
    const int soff = static_cast<int>(cc0 * DIM * 2);
    __builtin_amdgcn_sched_barrier(0);
    if (CAUSAL) {
      bload_tile<DIM, NW>(kraw, rk, soff);
      __builtin_amdgcn_sched_barrier(0);
      bload_tile<DIM, NW>(vraw, rv, soff);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kQInLds)
      bload_tile<DIM, NW>(qraw, rq, soff);
    else
      bload_q<DIM>(qraw, rq, soff, i, g);
    __builtin_amdgcn_sched_barrier(0);
  };
  fetch(c0);

  auto chunk_step = [&]() __attribute__((always_inline)) {
    if (CAUSAL) {
      store_tile<DIM, true, NW>(sKf, kraw, nrow);
      store_tile<DIM, false, NW>(sV, vraw, nrow);
    }
    i16x8 qf[KS];
    if constexpr (kQInLds) {
      store_tile<DIM, true, NW>(sQf, qraw, nrow);
      __syncthreads();
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = lds8(sQf + i * LD + 8 * g + 32 * s);
    } else {
#pragma unroll
      for (int s = 0; s < KS; ++s) qf[s] = i < nrow ? phi8(qraw[s]) : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
      __syncthreads();
    }

    // prefetch the next chunk while this one computes
    const int64_t c1 = c0 + T;
    const int nrow1 = c1 < r1 ? static_cast<int>(min(static_cast<int64_t>(T), r1 - c1)) : 0;
    if (nrow1 > 0) fetch(c1);

    f32x4_t o[NTW];
    const float den = chunk_outputs<DIM, NW, CAUSAL, NTW>(o, qf, sKf, sV, sST, sZ, rt, nb, g, li);
    // rows past the head's end (den may be 0 there) are dropped by the
    // stores' range check
    const float inv = 1.f / den;
#pragma unroll
    for (int n = 0; n < NTW; ++n) stage_piece<OC>(sO, pack4(o[n] * inv), li, g, n);
    store_staged<OC, DIM>(sO, ro, 16 * rt, 16 * nb, static_cast<int>(c0 * DIM * 2));
    bstore4(rd, den, den_voff, static_cast<int>(c0 * 4));

    if (CAUSAL) state_update<DIM, NW>(Sacc, zacc, sKf, sV, w, g, li);
    __syncthreads();
    if (CAUSAL) write_state<DIM, NW>(sST, sZ, Sacc, zacc, w, g, li);
    c0 = c1;
    nrow = nrow1;
  };
  chunk_step();  // segments are never empty
  while (c0 < r1) chunk_step();
}

// ---------------------------------------------------------------------------
// The causal D = 128 forward with double-buffered chunk tiles.  Same
// arithmetic and work split as k_fwd_mfma<128, true> (eight waves, a pair of
// waves per 16-row query tile splitting the output columns, every wave one
// 16-row slab of the fp32 state), but the next chunk's phi(K), V and phi(Q)
// go into the other half of a double buffer at the end of the current
// chunk's work instead of after a barrier.  A chunk then has one long phase
// (outputs, state update, the next chunk's tiles) and a short one (S^T and Z
// written back), so the waves' VALU work (phi, the hi / lo splits) overlaps
// other waves' matrix and LDS work instead of running while the matrix
// cores idle.  One workgroup per CU (155 KB of LDS).
__global__ __launch_bounds__(512, 1) void k_fwd_mfma_db(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                       const bf16_t* __restrict__ v, bf16_t* __restrict__ out,
                                                       float* __restrict__ den_out, const float* __restrict__ carry,
                                                       int64_t N, int P, int seg_len) {
  constexpr int DIM = 128, NW = 8;
  using G = Geo<DIM, NW>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS, PC = G::PC, DT = G::DT;
  constexpr int NTW = NTL / 2;  // output tiles per wave
  constexpr int OC = NTW * 16;
  constexpr int TILE = T * LD;
  extern __shared__ __align__(16) uint16_t smem[];
  // [phi(K) 0, V 0, phi(Q) 0][phi(K) 1, V 1, phi(Q) 1][S^T][Z hi, lo][output staging]
  uint16_t* sST = smem + 6 * TILE;
  uint16_t* sZ = sST + DIM * LD;
  uint16_t* sOut = sZ + 2 * DIM;

  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // query row tile: waves w and w + 4 share a SIMD, so the second four take
  // the tiles in reverse and every SIMD gets one short and one long triangle
  const int rt = w < 4 ? w : 3 - (w & 3);
  const int nb = (w >> 2) * NTW;  // first output tile of this wave
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  const float* cs = carry ? carry + (bh * P + seg) * E : nullptr;
  const rsrc_t rq = make_rsrc(q + bh * N * DIM, N * DIM * 2);
  const rsrc_t rk = make_rsrc(k + bh * N * DIM, N * DIM * 2);
  const rsrc_t rv = make_rsrc(v + bh * N * DIM, N * DIM * 2);
  const rsrc_t ro = make_rsrc(out ? out + bh * N * DIM : nullptr, out ? N * DIM * 2 : 0);
  const rsrc_t rd = make_rsrc(den_out ? den_out + bh * N : nullptr, den_out ? N * 4 : 0);
  const int i = 16 * rt + li;
  const int den_voff = (g == 0 && nb == 0) ? 4 * i : static_cast<int>(4 * N);
  uint16_t* sO = sOut + w * 16 * (OC + kLdsPad);

  f32x4_t Sacc[DT][NTL];
  f32x4_t zacc[DT];
  init_state<DIM, NW>(Sacc, zacc, cs, w, g, li);
  write_state<DIM, NW>(sST, sZ, Sacc, zacc, w, g, li);

  // Rows of a chunk past the segment's end lie past the head's end
  // (segments are whole chunks): the buffer range check zeroes them, and
  // store_tile zeroes phi(K) and phi(Q) there.  Two chunks are in flight:
  // while chunk c computes, one register set holds chunk c + 1 (staged into
  // the other LDS half at the end of chunk c, then refilled with chunk
  // c + 3) and the other is receiving chunk c + 2.  A load for a chunk past
  // the segment's end is still issued, at an offset past the head's range
  // (zeros, no memory traffic), so that every trip issues the same memory
  // operations and the waits for one set leave the other's loads in flight.
  struct Raw {
    i32x4 k[PC], v[PC], q[PC];
  };
  Raw ra, rb;
  const int hbytes = static_cast<int>(N * DIM * 2);
  auto fetch = [&](Raw& x, int64_t cc0) {
    const int soff = cc0 < r1 ? static_cast<int>(cc0 * DIM * 2) : hbytes;
    bload_tile<DIM, NW>(x.k, rk, soff);
    bload_tile<DIM, NW>(x.v, rv, soff);
    bload_tile<DIM, NW>(x.q, rq, soff);
  };
  auto put = [&](uint16_t* tiles, const Raw& x, int nr) {
    store_tile<DIM, true, NW>(tiles, x.k, nr);
    store_tile<DIM, false, NW>(tiles + TILE, x.v, nr);
    store_tile<DIM, true, NW>(tiles + 2 * TILE, x.q, nr);
  };
  auto rows_of = [&](int64_t cc0) { return cc0 < r1 ? static_cast<int>(min(static_cast<int64_t>(T), r1 - cc0)) : 0; };

  int64_t c0 = r0;
  fetch(ra, c0);
  put(smem, ra, rows_of(c0));
  fetch(ra, c0 + T);
  fetch(rb, c0 + 2 * T);
  __syncthreads();
  int buf = 0;
  // one chunk; `nx` holds chunk c0 + T on entry and chunk c0 + 3T on exit
  auto step = [&](Raw& nx) __attribute__((always_inline)) {
    const uint16_t* sKf = smem + buf * 3 * TILE;
    const uint16_t* sV = sKf + TILE;
    const uint16_t* sQf = sKf + 2 * TILE;
    const int nrow1 = rows_of(c0 + T);

    i16x8 qf[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = lds8(sQf + i * LD + 8 * g + 32 * s);
    f32x4_t o[NTW];
    const float den = chunk_outputs<DIM, NW, true, NTW>(o, qf, sKf, sV, sST, sZ, rt, nb, g, li);
    const float inv = 1.f / den;
#pragma unroll
    for (int n = 0; n < NTW; ++n) stage_piece<OC>(sO, pack4(o[n] * inv), li, g, n);
    store_staged<OC, DIM>(sO, ro, 16 * rt, 16 * nb, static_cast<int>(c0 * DIM * 2));
    bstore4(rd, den, den_voff, static_cast<int>(c0 * 4));

    // The state update, then the next chunk's tiles into the other half
    // (last read in the previous chunk, before its barriers).  A whole next
    // chunk (wave-uniform test) takes a copy without row guards, so that the
    // phi arithmetic and the update's MFMAs share one basic block and the
    // scheduler can interleave them.
    uint16_t* nxt = smem + (buf ^ 1) * 3 * TILE;
    if (nrow1 == T) {
      state_update<DIM, NW>(Sacc, zacc, sKf, sV, w, g, li);
      store_tile_full<DIM, true, NW>(nxt, nx.k);
      store_tile_full<DIM, false, NW>(nxt + TILE, nx.v);
      store_tile_full<DIM, true, NW>(nxt + 2 * TILE, nx.q);
    } else {
      state_update<DIM, NW>(Sacc, zacc, sKf, sV, w, g, li);
      if (nrow1 > 0) put(nxt, nx, nrow1);
    }
    fetch(nx, c0 + 3 * T);
    __syncthreads();  // every read of S^T, Z and this half done
    write_state<DIM, NW>(sST, sZ, Sacc, zacc, w, g, li);
    __syncthreads();  // S^T, Z and the next half written
    c0 += T;
    buf ^= 1;
  };
  while (c0 < r1) {
    step(ra);
    if (c0 >= r1) break;
    step(rb);
  }
}

// ---------------------------------------------------------------------------
// The D = 64 forward with 128-token chunks (plan chunk 128).  Same
// arithmetic as k_fwd_mfma (hi + lo scores, S^T in LDS as bf16, fp32 state in
// MFMA accumulators), over chunks twice as long: the inter-chunk product and
// the state read-out run once per 128 tokens instead of per 64, and the
// masked triangle doubles.  Four waves; wave w takes query row tiles w and
// 7 - w of each chunk, so every wave does the same triangular work (9 key
// tiles), and owns state rows 16w .. 16w + 15.  Segments are whole numbers
// of 128-token chunks (the host cuts them so), so the only partial chunk is
// a sequence's last, whose rows past the end the stores' range check drops.
// ---------------------------------------------------------------------------
constexpr int T2 = 128;

template <bool CAUSAL>
__global__ __launch_bounds__(256, 2) void k_fwd_mfma_t128(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ v, bf16_t* __restrict__ out,
                                                          float* __restrict__ den_out, const float* __restrict__ carry,
                                                          int64_t N, int P, int seg_len) {
  constexpr int DIM = 64, NW = 4;
  using G = Geo<DIM, NW>;
  constexpr int LD = G::LD, NTL = G::NTL, KS = G::KS;
  constexpr int PC2 = T2 * DIM / 8 / 256;  // 16-byte pieces per thread per 128 x 64 tile
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sKf = smem;
  uint16_t* sV = sKf + T2 * LD;
  uint16_t* sST = sV + T2 * LD;
  uint16_t* sZ = sST + DIM * LD;  // Z as bf16 hi [DIM], lo [DIM]
  uint16_t* sOut = sZ + 2 * DIM;  // per-wave output staging, 16 x DIM
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / P;
  const int seg = blockIdx.x % P;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  constexpr int64_t E = static_cast<int64_t>(DIM) * DIM + DIM;
  const float* cs = carry ? (CAUSAL ? carry + (bh * P + seg) * E : carry + bh * E) : nullptr;
  const bf16_t* qh = q + bh * N * DIM;
  const bf16_t* kh = k + bh * N * DIM;
  const bf16_t* vh = v + bh * N * DIM;
  const rsrc_t ro = make_rsrc(out ? out + bh * N * DIM : nullptr, out ? N * DIM * 2 : 0);
  float* dh = den_out ? den_out + bh * N : nullptr;
  const short one = 0x3f80;  // bf16 1.0
  const i16x8 ones = {one, one, one, one, one, one, one, one};
  uint16_t* sO = sOut + w * 16 * (DIM + kLdsPad);
  const int rts[2] = {w, 7 - w};  // wave-uniform query row tiles

  f32x4_t Sacc[G::DT][NTL];
  f32x4_t zacc[G::DT];
  init_state<DIM, NW>(Sacc, zacc, cs, w, g, li);
  write_state<DIM, NW>(sST, sZ, Sacc, zacc, w, g, li);

  auto load_kv = [&](i32x4 (&raw)[PC2], const bf16_t* src, int64_t cc0, int nr) {
#pragma unroll
    for (int r = 0; r < PC2; ++r) {
      const int p = tid + 256 * r;
      const int j = p / G::ROW8, c8 = p % G::ROW8;
      raw[r] = j < nr ? gload16(src + (cc0 + j) * DIM + c8 * 8) : i32x4{0, 0, 0, 0};
    }
  };
  auto store_kv = [&](uint16_t* lds, const i32x4 (&raw)[PC2], int nr, bool apply_phi) {
#pragma unroll
    for (int r = 0; r < PC2; ++r) {
      const int p = tid + 256 * r;
      const int j = p / G::ROW8, c8 = p % G::ROW8;
      i16x8 val = {0, 0, 0, 0, 0, 0, 0, 0};
      if (j < nr) val = apply_phi ? phi8(raw[r]) : __builtin_bit_cast(i16x8, raw[r]);
      *reinterpret_cast<i16x8*>(lds + j * LD + c8 * 8) = val;
    }
  };

  int64_t c0 = r0;
  int nrow = static_cast<int>(min(static_cast<int64_t>(T2), r1 - c0));
  i32x4 kraw[PC2], vraw[PC2], qraw[2][KS];
  if (CAUSAL) {
    load_kv(kraw, kh, c0, nrow);
    load_kv(vraw, vh, c0, nrow);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) load_q<DIM>(qraw[x], qh, c0, nrow, 16 * rts[x] + li, g);

  while (c0 < r1) {
    if (CAUSAL) {
      store_kv(sKf, kraw, nrow, true);
      store_kv(sV, vraw, nrow, false);
    }
    i16x8 qf[2][KS];
#pragma unroll
    for (int x = 0; x < 2; ++x)
#pragma unroll
      for (int s = 0; s < KS; ++s)
        qf[x][s] = 16 * rts[x] + li < nrow ? phi8(qraw[x][s]) : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
    __syncthreads();

    // prefetch the next chunk while this one computes
    const int64_t c1 = c0 + T2;
    const int nrow1 = c1 < r1 ? static_cast<int>(min(static_cast<int64_t>(T2), r1 - c1)) : 0;
    if (nrow1 > 0) {
      if (CAUSAL) {
        load_kv(kraw, kh, c1, nrow1);
        load_kv(vraw, vh, c1, nrow1);
      }
#pragma unroll
      for (int x = 0; x < 2; ++x) load_q<DIM>(qraw[x], qh, c1, nrow1, 16 * rts[x] + li, g);
    }

#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int rt = rts[x];
      const int i = 16 * rt + li;
      // intra-chunk scores A^T for key tiles t <= rt, masked, as hi + lo
      i16x4 ahi[T2 / 16], alo[T2 / 16];
      if (CAUSAL) {
#pragma unroll
        for (int t = 0; t < T2 / 16; ++t) {
          ahi[t] = i16x4{0, 0, 0, 0};
          alo[t] = i16x4{0, 0, 0, 0};
          if (t <= rt) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = mfma(lds8(sKf + (16 * t + li) * LD + 8 * g + 32 * s), qf[x][s], acc);
            if (t == rt) {
#pragma unroll
              for (int u = 0; u < 4; ++u)
                if (4 * g + u > li) acc[u] = 0.f;
            }
            ahi[t] = pack4(acc);
            alo[t] = pack4(acc - unpack4(ahi[t]));
          }
        }
      }
      // denominator: phi(Q_i)^T Z (Z as hi + lo) and the intra-chunk scores
      f32x4_t dz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        dz = mfma(lds8(sZ + 8 * g + 32 * s), qf[x][s], dz);
        dz = mfma(lds8(sZ + DIM + 8 * g + 32 * s), qf[x][s], dz);
      }
      // O^T = S^T phi(Q)^T (+ V^T A^T)
      f32x4_t o[NTL];
#pragma unroll
      for (int n = 0; n < NTL; ++n) {
        o[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) o[n] = mfma(lds8(sST + (16 * n + li) * LD + 8 * g + 32 * s), qf[x][s], o[n]);
      }
      if (CAUSAL) {
#pragma unroll
        for (int tp = 0; tp < T2 / 32; ++tp) {
          if (2 * tp <= rt) {
            const i16x8 bhi = cat(ahi[2 * tp], ahi[2 * tp + 1]);
            const i16x8 blo = cat(alo[2 * tp], alo[2 * tp + 1]);
            dz = mfma(ones, bhi, dz);
            dz = mfma(ones, blo, dz);
            const int jr = 32 * tp + 4 * g + li / 4;
            const int cc = 4 * (li % 4);
#pragma unroll
            for (int n = 0; n < NTL; ++n) {
              const i16x8 a = cat(lds_tr(sV + jr * LD + 16 * n + cc), lds_tr(sV + (jr + 16) * LD + 16 * n + cc));
              o[n] = mfma(a, bhi, o[n]);
              o[n] = mfma(a, blo, o[n]);
            }
          }
        }
      }
      const float den = dz[0];
      if (out) {
        const float inv = 1.f / den;
#pragma unroll
        for (int n = 0; n < NTL; ++n) stage_piece<DIM>(sO, pack4(o[n] * inv), li, g, n);
        store_staged<DIM, DIM>(sO, ro, 16 * rt, 0, static_cast<int>(c0 * DIM * 2));
      }
      if (i < nrow && dh && g == 0) dh[c0 + i] = den;
    }

    if (CAUSAL) state_update<DIM, NW, T2>(Sacc, zacc, sKf, sV, w, g, li);
    __syncthreads();
    if (CAUSAL) write_state<DIM, NW>(sST, sZ, Sacc, zacc, w, g, li);
    c0 = c1;
    nrow = nrow1;
  }
}

// Segment aggregates dS = phi(K)^T V, dZ = colsum phi(K) over one segment.
// phi(K) = mu + E(K) is split (mu in {0, 1} per feature, from the segment's
// first chunk: decide_mu) so that the records are as exact as fp32 allows:
// the MFMAs sum E(K)^T V and colsum E(K) with E carried as bf16 (elu where
// phi ~ 1, a rounding relative to E rather than to 1; phi itself where
// phi << 1), and the mu part enters in fp32 as dS = mu (colsum V)^T + E^T V,
// dZ = mu count + colsum E.  The backward splits the carried states again
// and relies on that precision.
template <int DIM>
__global__ __launch_bounds__(64 * kFwdWaves<DIM>, 2) void k_seg_state_mfma(const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
                                                       float* __restrict__ s_out, int64_t s_stride,
                                                       float* __restrict__ z_out, int64_t z_stride, int64_t N,
                                                       int P, int nseg, int seg_len) {
  constexpr int NW = kFwdWaves<DIM>;
  using G = Geo<DIM, NW>;
  constexpr int LD = G::LD, NTL = G::NTL, PC = G::PC, DT = G::DT;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* sKe = smem;
  uint16_t* sV = sKe + T * LD;
  float* sMuF = reinterpret_cast<float*>(sV + T * LD);
  uint16_t* sMuB = reinterpret_cast<uint16_t*>(sMuF + DIM);
  // w is made wave-uniform (an SGPR) so that branches on it are scalar: an
  // MFMA under an EXEC-masked branch still writes every lane.
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t bh = blockIdx.x / nseg;
  const int seg = blockIdx.x % nseg;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rk = make_rsrc(k + bh * N * DIM, hbytes), rv = make_rsrc(v + bh * N * DIM, hbytes);
  static_assert(NTL == NW, "one column tile of U per wave");
  f32x4_t Sacc[DT][NTL];
  f32x4_t zacc[DT];
  // column sums of V, this wave's tile: lane holds U[16w + li] (the waves
  // share the tiles through LDS at the end)
  f32x4_t uacc = {0.f, 0.f, 0.f, 0.f};
  init_state<DIM, NW>(Sacc, zacc, nullptr, w, g, li);
  const short one = 0x3f80;  // bf16 1.0
  const i16x8 ones = {one, one, one, one, one, one, one, one};
  i32x4 kraw[PC], vraw[PC];
  // rows past the head's end load as zero (V = 0; E is zeroed past nrow)
  bload_tile<DIM, NW>(kraw, rk, static_cast<int>(r0 * DIM * 2));
  bload_tile<DIM, NW>(vraw, rv, static_cast<int>(r0 * DIM * 2));
  store_tile_e<DIM, NW>(sKe, kraw);
  __syncthreads();
  decide_mu<DIM, LD>(sKe, static_cast<int>(min(static_cast<int64_t>(T), r1 - r0)), sMuF, sMuB);
  __syncthreads();
  const MuOff moff = mu_offsets<DIM, NW>(sMuF);
  for (int64_t c0 = r0; c0 < r1; c0 += T) {
    store_tile_emu<DIM, NW>(sKe, kraw, static_cast<int>(min(static_cast<int64_t>(T), r1 - c0)), moff);
    store_tile_v<DIM, NW>(sV, vraw);
    __syncthreads();
    if (c0 + T < r1) {
      bload_tile<DIM, NW>(kraw, rk, static_cast<int>((c0 + T) * DIM * 2));
      bload_tile<DIM, NW>(vraw, rv, static_cast<int>((c0 + T) * DIM * 2));
    }
    state_update<DIM, NW>(Sacc, zacc, sKe, sV, w, g, li);
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      const int jr = 32 * s + 8 * g + li / 4;
      const int cc = 4 * (li % 4);
      uacc = mfma(ones, cat(lds_tr(sV + jr * LD + 16 * w + cc), lds_tr(sV + (jr + 4) * LD + 16 * w + cc)), uacc);
    }
    __syncthreads();
  }
  // every wave's U tile to LDS (over the K tile, free after the last barrier)
  float* sU = reinterpret_cast<float*>(sKe);
  if (g == 0) sU[16 * w + li] = uacc[0];
  __syncthreads();
  const int64_t rec = bh * P + seg;
  const float count = static_cast<float>(r1 - r0);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d0 = 16 * (w * DT + dt);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int d = d0 + 4 * g + u;
      const float mu = sMuF[d];
#pragma unroll
      for (int n = 0; n < NTL; ++n)
        s_out[rec * s_stride + d * DIM + 16 * n + li] = Sacc[dt][n][u] + mu * sU[16 * n + li];
      if (li == 0) z_out[rec * z_stride + d] = zacc[dt][u] + mu * count;
    }
  }
}

// The same aggregates at D = 64 with wave-private chunks: wave w of the
// workgroup sums chunks w, w + 4, w + 8, ... of the segment into a full
// 64 x 64 partial of its own (16 fp32 accumulator tiles), staging each chunk
// in a private LDS tile, so the chunk loop has no workgroup barrier and
// every staged element is read from LDS once (the A and B operands of all
// sixteen tiles are held in registers).  The four partials are added in
// wave order at the end.  Same split as above: dS = mu U^T + E^T V,
// dZ = mu count + colsum E, with mu chosen from the segment's first chunk.
__global__ __launch_bounds__(256, 2) void k_seg_state_wave64(const bf16_t* __restrict__ k,
                                                             const bf16_t* __restrict__ v, float* __restrict__ s_out,
                                                             int64_t s_stride, float* __restrict__ z_out,
                                                             int64_t z_stride, int64_t N, int P, int nseg,
                                                             int seg_len) {
  constexpr int DIM = 64, LD = DIM + kLdsPad;
  constexpr int PW = T * DIM / 8 / 64;  // 16-byte pieces per lane per chunk tile
  constexpr int RP = DIM + 4;           // fp32 row stride of the partials in LDS
  extern __shared__ __align__(16) uint16_t smem[];
  const int tid = threadIdx.x, l = tid & 63, g = l >> 4, li = l & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint16_t* sK = smem + w * 2 * T * LD;
  uint16_t* sV = sK + T * LD;
  const int64_t bh = blockIdx.x / nseg;
  const int seg = blockIdx.x % nseg;
  const int64_t r0 = static_cast<int64_t>(seg) * seg_len;
  const int64_t r1 = min(N, r0 + seg_len);
  const int64_t hbytes = N * DIM * 2;
  const rsrc_t rk = make_rsrc(k + bh * N * DIM, hbytes), rv = make_rsrc(v + bh * N * DIM, hbytes);
  const int nch = static_cast<int>((r1 - r0 + T - 1) / T);
  const short one = 0x3f80;  // bf16 1.0
  const i16x8 ones = {one, one, one, one, one, one, one, one};
  f32x4_t S[4][4], zacc[4], uacc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    zacc[a] = uacc[a] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < 4; ++b) S[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // piece p of lane l: row (64 p + l) / 8, features 8 ((64 p + l) % 8) ..
  i32x4 kr[PW], vr[PW];
  auto fetch = [&](int c) {
    const int soff = static_cast<int>((r0 + static_cast<int64_t>(c) * T) * DIM * 2);
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      kr[p] = bload16(rk, (64 * p + l) * 16, soff);
      vr[p] = bload16(rv, (64 * p + l) * 16, soff);
    }
  };
  if (w < nch) fetch(w);
  // the split constant mu: wave 0 stages the segment's first chunk as elu
  // (rows past the head's end load as zero, elu(0) = 0) for decide_mu
  float* sMuF = reinterpret_cast<float*>(smem + 4 * 2 * T * LD);
  uint16_t* sMuB = reinterpret_cast<uint16_t*>(sMuF + DIM);
  if (w == 0) {
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const int e = 64 * p + l;
      f32x8_t x = unpack8(__builtin_bit_cast(i16x8, kr[p]));
#pragma unroll
      for (int q = 0; q < 8; ++q) x[q] = elu_fast(x[q]);
      *reinterpret_cast<i16x8*>(sK + (e >> 3) * LD + (e & 7) * 8) = pack8(x);
    }
  }
  __syncthreads();
  decide_mu<DIM, LD>(smem, static_cast<int>(min(static_cast<int64_t>(T), r1 - r0)), sMuF, sMuB);
  __syncthreads();
  const MuOff moff = mu_offsets<DIM>(sMuF);
  for (int c = w; c < nch; c += 4) {
    // rows past the head's end: V loaded as zero, E stored as zero
    const int nr = static_cast<int>(min(static_cast<int64_t>(T), r1 - r0 - static_cast<int64_t>(c) * T));
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const int e = 64 * p + l;
      const i16x8 ke = emu8(kr[p], moff);
      *reinterpret_cast<i16x8*>(sK + (e >> 3) * LD + (e & 7) * 8) =
          (e >> 3) < nr ? ke : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
      *reinterpret_cast<i16x8*>(sV + (e >> 3) * LD + (e & 7) * 8) = __builtin_bit_cast(i16x8, vr[p]);
    }
    if (c + 4 < nch) fetch(c + 4);
    // the tiles are private to this wave: its LDS operations complete in
    // order, so only the compiler has to be kept from reordering them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int s = 0; s < T / 32; ++s) {
      const int jr = 32 * s + 8 * g + li / 4;
      const int cc = 4 * (li % 4);
      i16x8 a[4], b[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        a[n] = cat(lds_tr(sK + jr * LD + 16 * n + cc), lds_tr(sK + (jr + 4) * LD + 16 * n + cc));
        b[n] = cat(lds_tr(sV + jr * LD + 16 * n + cc), lds_tr(sV + (jr + 4) * LD + 16 * n + cc));
      }
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        zacc[n] = mfma(a[n], ones, zacc[n]);
        uacc[n] = mfma(ones, b[n], uacc[n]);
      }
#pragma unroll
      for (int dn = 0; dn < 4; ++dn)
#pragma unroll
        for (int mn = 0; mn < 4; ++mn) S[dn][mn] = mfma(a[dn], b[mn], S[dn][mn]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // partials to LDS: Sp[w][d][m] (rows padded to RP floats), Zp[w][d], Up[w][m]
  __syncthreads();
  float* Sp = reinterpret_cast<float*>(smem);
  float* Zp = Sp + 4 * DIM * RP;
  float* Up = Zp + 4 * DIM;
#pragma unroll
  for (int dn = 0; dn < 4; ++dn)
#pragma unroll
    for (int mn = 0; mn < 4; ++mn)
#pragma unroll
      for (int u = 0; u < 4; ++u) Sp[(w * DIM + 16 * dn + 4 * g + u) * RP + 16 * mn + li] = S[dn][mn][u];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    if (li == 0)
#pragma unroll
      for (int u = 0; u < 4; ++u) Zp[w * DIM + 16 * n + 4 * g + u] = zacc[n][u];
    if (g == 0) Up[w * DIM + 16 * n + li] = uacc[n][0];
  }
  __syncthreads();
  const int64_t rec = bh * P + seg;
  const float count = static_cast<float>(r1 - r0);
  const int m = tid & 63;
  const float um = ((Up[m] + Up[DIM + m]) + Up[2 * DIM + m]) + Up[3 * DIM + m];
  for (int d = tid >> 6; d < DIM; d += 4) {
    const float sum = ((Sp[d * RP + m] + Sp[(DIM + d) * RP + m]) + Sp[(2 * DIM + d) * RP + m]) +
                      Sp[(3 * DIM + d) * RP + m];
    s_out[rec * s_stride + d * DIM + m] = sum + sMuF[d] * um;
  }
  if (tid < DIM)
    z_out[rec * z_stride + tid] =
        (((Zp[tid] + Zp[DIM + tid]) + Zp[2 * DIM + tid]) + Zp[3 * DIM + tid]) + sMuF[tid] * count;
}

size_t lds_fwd(int dim) {
  const int tiles = dim == 128 ? 3 : 2;  // K, V (and phi(Q) with two waves per query tile)
  const int waves = dim == 128 ? 8 : 4;  // each with a 16 x 64 output staging tile
  return (tiles * T * (dim + kLdsPad) + dim * (dim + kLdsPad) + waves * 16 * (64 + kLdsPad)) * sizeof(uint16_t) +
         dim * sizeof(float);
}
size_t lds_fwd_db() {
  return (6 * T * (128 + kLdsPad) + 128 * (128 + kLdsPad) + 2 * 128 + 8 * 16 * (64 + kLdsPad)) * sizeof(uint16_t);
}
size_t lds_fwd_t128() {
  return (2 * T2 * (64 + kLdsPad) + 64 * (64 + kLdsPad) + 2 * 64 + 4 * 16 * (64 + kLdsPad)) * sizeof(uint16_t);
}
// (each + the split constant mu as fp32 and bf16)
size_t lds_seg(int dim) { return 2 * T * (dim + kLdsPad) * sizeof(uint16_t) + dim * (sizeof(float) + sizeof(uint16_t)); }
// four wave-private K / V tile pairs (the partials reuse the space at the
// end), then mu
size_t lds_seg_wave64() {
  const size_t tiles = 4 * 2 * T * (64 + kLdsPad) * sizeof(uint16_t);
  const size_t parts = (4 * 64 * (64 + 4) + 2 * 4 * 64) * sizeof(float);
  static_assert((4 * 64 * (64 + 4) + 2 * 4 * 64) * sizeof(float) <= 4 * 2 * T * (64 + kLdsPad) * sizeof(uint16_t),
                "the partials fit below mu");
  return (tiles > parts ? tiles : parts) + 64 * (sizeof(float) + sizeof(uint16_t));
}

#define LA_MLAUNCH(kernel, nthreads, grid, lds, st, ...)                                                \
  do {                                                                                                  \
    hipError_t e_ = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),                          \
                                        hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds)); \
    if (e_ != hipSuccess) return e_;                                                                    \
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(nthreads), lds, st, __VA_ARGS__); \
    return hipGetLastError();                                                                           \
  } while (0)

}  // namespace

int mfma_supported(int op, int64_t D, int64_t M, int dtype) {
  if (D != M) return 0;
  // fp32 (v_mfma_f32_16x16x4_f32): forward at D = M = 64, prefix state at 64 and 128
  if (dtype == 0) return (D == 64 && op == 0 /* forward */) || ((D == 64 || D == 128) && op == 2 /* prefix state */);
  if (dtype != 1 || (D != 64 && D != 128)) return 0;
  return op == 0 /* forward */ || op == 1 /* backward */ || op == 2 /* prefix state */;
}

hipError_t launch_forward_mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                               void* out, float* den_out, const float* carry, hipStream_t st) {
  const int64_t grid = g.BH * g.P;
  const bf16_t* Q = static_cast<const bf16_t*>(q);
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  bf16_t* O = static_cast<bf16_t*>(out);
  if (g.D == 64 && g.chunk == T2) {
    if (causal) LA_MLAUNCH((k_fwd_mfma_t128<true>), 256, grid, lds_fwd_t128(), st, Q, K, V, O, den_out, carry, g.N, g.P, g.seg_len);
    LA_MLAUNCH((k_fwd_mfma_t128<false>), 256, grid, lds_fwd_t128(), st, Q, K, V, O, den_out, carry, g.N, g.P, g.seg_len);
  }
  if (g.D == 64) {
    if (causal) LA_MLAUNCH((k_fwd_mfma<64, true>), 64 * kFwdWaves<64>, grid, lds_fwd(64), st, Q, K, V, O, den_out, carry, g.N, g.P, g.seg_len);
    LA_MLAUNCH((k_fwd_mfma<64, false>), 64 * kFwdWaves<64>, grid, lds_fwd(64), st, Q, K, V, O, den_out, carry, g.N, g.P, g.seg_len);
  }
  if (g.D == 128) {
    if (causal) LA_MLAUNCH(k_fwd_mfma_db, 512, grid, lds_fwd_db(), st, Q, K, V, O, den_out, carry, g.N, g.P, g.seg_len);
    LA_MLAUNCH((k_fwd_mfma<128, false>), 64 * kFwdWaves<128>, grid, lds_fwd(128), st, Q, K, V, O, den_out, carry, g.N, g.P, g.seg_len);
  }
  return hipErrorNotSupported;
}

hipError_t launch_seg_state_mfma(const SegGeom& g, const void* k, const void* v, float* s_out, int64_t s_stride,
                                 float* z_out, int64_t z_stride, hipStream_t st) {
  const int nseg = g.nseg > 0 ? g.nseg : g.P;
  const int64_t grid = g.BH * nseg;
  const bf16_t* K = static_cast<const bf16_t*>(k);
  const bf16_t* V = static_cast<const bf16_t*>(v);
  if (g.D == 64)
    LA_MLAUNCH(k_seg_state_wave64, 256, grid, lds_seg_wave64(), st, K, V, s_out, s_stride, z_out, z_stride, g.N, g.P,
               nseg, g.seg_len);
  if (g.D == 128)
    LA_MLAUNCH((k_seg_state_mfma<128>), 64 * kFwdWaves<128>, grid, lds_seg(128), st, K, V, s_out, s_stride, z_out, z_stride, g.N,
               g.P, nseg, g.seg_len);
  return hipErrorNotSupported;
}

}  // namespace la
