// Shared pieces of the bf16 MFMA kernels (gfx950, wave64).
//
// MFMA used: v_mfma_f32_16x16x32_bf16 (D = A(16x32) * B(32x16) + C, fp32
// accumulate).  Lane layouts (l = lane, g = l / 16, li = l % 16):
//   A operand: A[li][8g + e], e = 0..7        (8 bf16 per lane)
//   B operand: B[8g + e][li]                   (8 bf16 per lane)
//   C / D    : C[4g + u][li], u = 0..3         (4 fp32 per lane)
// ds_read_tr16_b64 (LDS transpose read) within each 16-lane group returns to
// lane i the elements  out[i][u] = in[lane 4u + i/4][i % 4]  where in[L] is
// the 4 x 16-bit block lane L addresses.  With it, a token-major LDS tile
// X[j][c] gives an operand whose k index runs along tokens j: lane li of
// group g points at row (j0 + li / 4), column (c0 + 4 (li % 4)) and receives
// X[j0 + u][c0 + li] for u = 0..3.
#pragma once

#include "la_device.h"

namespace la {
namespace mf {

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ __forceinline__ f32x4_t mfma(i16x8 a, i16x8 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// 16-byte LDS read of 8 consecutive bf16.
__device__ __forceinline__ i16x8 lds8(const uint16_t* p) { return *reinterpret_cast<const i16x8*>(p); }

// Transposing 8-byte LDS read (see the header comment).
__device__ __forceinline__ i16x4 lds_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ i16x8 cat(i16x4 a, i16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));

// fp32 -> bf16 conversions use the hardware round-to-nearest-even packed
// convert (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ short bf(float x) {
  const f32x2_t v = {x, 0.f};
  return __builtin_bit_cast(short, __builtin_convertvector(v, bf16x2_t)[0]);
}
__device__ __forceinline__ float fb(short h) { return bf16_to_f32(static_cast<uint16_t>(h)); }

// Two fp32 -> one packed pair of bf16 (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ int pack2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(int, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ i16x4 pack4(f32x4_t v) {
  const i32x2 r = {pack2(v[0], v[1]), pack2(v[2], v[3])};
  return __builtin_bit_cast(i16x4, r);
}

__device__ __forceinline__ i16x8 pack8(f32x8_t v) {
  const i32x4 r = {pack2(v[0], v[1]), pack2(v[2], v[3]), pack2(v[4], v[5]), pack2(v[6], v[7])};
  return __builtin_bit_cast(i16x8, r);
}

__device__ __forceinline__ f32x8_t unpack8(i16x8 h) {
  return __builtin_convertvector(__builtin_bit_cast(bf16x8_t, h), f32x8_t);
}

__device__ __forceinline__ f32x4_t unpack4(i16x4 h) {
  return __builtin_convertvector(__builtin_bit_cast(bf16x4_t, h), f32x4_t);
}

// phi for the bf16 kernels: e^x through the hardware exp2 (its error is far
// below the bf16 rounding that follows).
__device__ __forceinline__ float phi_fast(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// elu(x) = phi(x) - 1 (alpha = 1), for kernels that carry phi = 1 + elu with
// the ones part in fp32 and only the small elu part as a bf16 operand.
__device__ __forceinline__ float elu_fast(float x) { return x > 0.f ? x : __expf(x) - 1.f; }

// phi applied to 8 bf16 values (raw 16-byte vector), result rounded to bf16.
__device__ __forceinline__ i16x8 phi8(i32x4 raw) {
  f32x8_t x = unpack8(__builtin_bit_cast(i16x8, raw));
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = phi_fast(x[e]);
  return pack8(x);
}

// Sum over the four 16-lane groups (lanes li, li+16, li+32, li+48), every
// lane receiving it, with the gfx950 lane swaps instead of LDS permutes.
// v_permlane16_swap(a, b) exchanges the odd 16-lane rows of a with the even
// rows of b, v_permlane32_swap(a, b) the upper 32 lanes of a with the lower
// 32 of b (checked on the hardware); with a = b = x, a + b is x plus its
// lane ^ 16 (then lane ^ 32) partner, the pairs and order of two xor
// shuffles, so the sums are the same bits.  The s_nop covers the wait a
// permlane needs after a VALU write of its operands.
__device__ __forceinline__ float shfl_sum_groups(float x) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  x = a + b;
  a = x;
  b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return a + b;
}

// x from another lane of the same 16-lane row by a DPP control whose every
// lane has a source (row_ror, row_half_mirror, quad_perm).
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor8 = 0x128;         // row_ror:8 = lane ^ 8 within a row
constexpr int kDppXor7 = 0x141;         // row_half_mirror = lane ^ 7
constexpr int kDppXor2 = 0x4e;          // quad_perm [2, 3, 0, 1]
constexpr int kDppXor1 = 0xb1;          // quad_perm [1, 0, 3, 2]

__device__ __forceinline__ i32x4 gload16(const bf16_t* p) { return *reinterpret_cast<const i32x4*>(p); }

// Raw buffer access (stride 0) over one head's rows: loads past the range
// return zero and stores past it are dropped, so a partial last chunk needs
// no row guards, and addresses are 32-bit offsets (a per-lane constant plus a
// wave-uniform chunk offset) instead of 64-bit pointers.  The host keeps every
// head under 2^31 bytes.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 buffer descriptor word 3 (32-bit data format)
constexpr int kStoreNT = 2;              // buffer cache-policy bits: non-temporal

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           kRsrcWord3);
}
__device__ __forceinline__ i32x4 bload16(rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
// A 16-byte store with the whole offset in the VGPR and a zero SGPR offset.
// The compiler keeps the next instructions from overwriting the data VGPRs
// of a store wider than 8 bytes (it inserts wait states) only when the store
// takes no SGPR offset; with one it assumes the data are read in time.  On
// gfx950 they were not always: with an SGPR offset and a VALU write of the
// data VGPRs as the next instruction, half of the lanes intermittently stored
// the new value.  A zero SGPR offset keeps the guard.  (The range check
// covers the sum of the offsets either way.)
__device__ __forceinline__ void bstore16(rsrc_t r, i16x8 v, int voff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, kStoreNT);
}
__device__ __forceinline__ void bstore8(rsrc_t r, i16x4 v, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff, 0);
}
__device__ __forceinline__ void bstore4(rsrc_t r, float v, int voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, v), r, voff, soff, 0);
}

constexpr int kNT = 256;  // threads per workgroup (4 wave64s)
constexpr int kT = 64;    // tokens per chunk
// LDS row padding (elements): a row of a T x DIM tile starts 16 bytes after
// a multiple of 128, so the 16-byte row reads of eight consecutive rows hit
// distinct banks.
constexpr int kLdsPad = 8;

// NW wave64s per workgroup (4, or 8 for the D = 128 forward kernels).
template <int DIM, int NW = 4>
struct Geo {
  static constexpr int NT = 64 * NW;            // threads per workgroup
  static constexpr int LD = DIM + kLdsPad;      // padded LDS row stride (elements)
  static constexpr int NTL = DIM / 16;          // 16-wide tiles along D (= M)
  static constexpr int KS = DIM / 32;           // 32-deep k-steps along D (= M)
  static constexpr int PC = kT * DIM / 8 / NT;  // 16-byte pieces per thread per T x DIM tile
  static constexpr int DT = NTL / NW;           // state row tiles owned by each wave
  static constexpr int ROW8 = DIM / 8;          // 16-byte pieces per row
};

// Global -> registers: thread's pieces of a T x DIM token-major tile.
template <int DIM, int NW = 4>
__device__ __forceinline__ void load_tile(i32x4 (&raw)[(Geo<DIM, NW>::PC)], const bf16_t* __restrict__ src,
                                          int64_t c0, int nrow) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + G::NT * r;
    const int j = p / G::ROW8, c8 = p % G::ROW8;
    raw[r] = j < nrow ? gload16(src + (c0 + j) * DIM + c8 * 8) : i32x4{0, 0, 0, 0};
  }
}

// Registers -> LDS (phi applied when asked); rows past nrow are zero.
template <int DIM, bool PHI, int NW = 4>
__device__ __forceinline__ void store_tile(uint16_t* lds, const i32x4 (&raw)[(Geo<DIM, NW>::PC)], int nrow) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + G::NT * r;
    const int j = p / G::ROW8, c8 = p % G::ROW8;
    i16x8 val = {0, 0, 0, 0, 0, 0, 0, 0};
    if (j < nrow) val = PHI ? phi8(raw[r]) : __builtin_bit_cast(i16x8, raw[r]);
    *reinterpret_cast<i16x8*>(lds + j * G::LD + c8 * 8) = val;
  }
}

// store_tile for a whole chunk (every row in range): no row guard, so the
// caller's code around it stays one basic block.
template <int DIM, bool PHI, int NW = 4>
__device__ __forceinline__ void store_tile_full(uint16_t* lds, const i32x4 (&raw)[(Geo<DIM, NW>::PC)]) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + G::NT * r;
    const int j = p / G::ROW8, c8 = p % G::ROW8;
    *reinterpret_cast<i16x8*>(lds + j * G::LD + c8 * 8) = PHI ? phi8(raw[r]) : __builtin_bit_cast(i16x8, raw[r]);
  }
}

// Registers -> LDS as bf16 elu(x), and each row's sum of the rounded values
// (fp32) into rowsum[j]; rows past nrow are zero.  The ROW8 pieces of a row
// sit in ROW8 consecutive lanes, so the row sum is a butterfly over them.
template <int DIM>
__device__ __forceinline__ void store_tile_elu(uint16_t* lds, const i32x4 (&raw)[Geo<DIM>::PC], int nrow,
                                               float* rowsum) {
  using G = Geo<DIM>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + kNT * r;
    const int j = p / G::ROW8, c8 = p % G::ROW8;
    i16x8 val = {0, 0, 0, 0, 0, 0, 0, 0};
    float sum = 0.f;
    if (j < nrow) {
      f32x8_t x = unpack8(__builtin_bit_cast(i16x8, raw[r]));
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = elu_fast(x[e]);
      val = pack8(x);
      const f32x8_t xr = unpack8(val);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += xr[e];
    }
    *reinterpret_cast<i16x8*>(lds + j * G::LD + c8 * 8) = val;
#pragma unroll
    for (int off = 1; off < G::ROW8; off <<= 1) sum += __shfl_xor(sum, off, 64);
    if (c8 == 0) rowsum[j] = sum;
  }
}

// Coalesced output rows.  An MFMA accumulator tile gives lane (li, g) four
// consecutive columns of row li, so storing straight from it writes 16 rows
// in 8-byte pieces per instruction, which the memory system takes well
// below its streaming rate.  Instead each wave puts its pieces into a
// private LDS tile of 16 rows x COLS bf16 (row stride COLS + kLdsPad) and
// reads it back in 16-byte pieces, so every store instruction writes whole
// runs of consecutive row bytes.
__device__ __forceinline__ void wave_lds_sync() {
  // a wave's LDS operations complete in order: only the compiler has to be
  // kept from moving them across this point
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
template <int COLS>
__device__ __forceinline__ void stage_piece(uint16_t* stage, i16x4 v, int li, int g, int n) {
  *reinterpret_cast<i16x4*>(stage + li * (COLS + kLdsPad) + 16 * n + 4 * g) = v;
}
// Rows row0 .. row0 + 15 of a row-major [*, ROWLEN] bf16 tensor, columns
// col0 .. col0 + COLS - 1, from the staged tile; `soff` is the chunk's byte
// offset.  Rows past the buffer's range are dropped by the hardware check.
// The stores are non-temporal: outputs are not read again by the kernel
// that writes them, and the hint keeps them from lingering dirty in the
// caches into the next kernel (the pass that follows the dk / dv sweep ran
// 17 us faster with it).
template <int COLS, int ROWLEN>
__device__ __forceinline__ void store_staged(const uint16_t* stage, rsrc_t dst, int row0, int col0, int soff) {
  constexpr int PR = COLS / 8;  // 16-byte pieces per row
  const int l = threadIdx.x & 63;
  wave_lds_sync();
#pragma unroll
  for (int k = 0; k < 16 * PR / 64; ++k) {
    const int p = 64 * k + l, r = p / PR, c8 = p % PR;
    const i16x8 v = *reinterpret_cast<const i16x8*>(stage + r * (COLS + kLdsPad) + 8 * c8);
    bstore16(dst, v, ((row0 + r) * ROWLEN + col0 + 8 * c8) * 2 + soff);
  }
  wave_lds_sync();
}

// Buffer versions of load_tile / load_q: `soff` is the chunk's first row in
// bytes; rows past the head's end read as zero.
template <int DIM, int NW = 4>
__device__ __forceinline__ void bload_tile(i32x4 (&raw)[(Geo<DIM, NW>::PC)], rsrc_t src, int soff) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + G::NT * r;
    raw[r] = bload16(src, ((p / G::ROW8) * DIM + (p % G::ROW8) * 8) * 2, soff);
  }
}
template <int DIM>
__device__ __forceinline__ void bload_q(i32x4 (&raw)[Geo<DIM>::KS], rsrc_t src, int soff, int i, int g) {
#pragma unroll
  for (int s = 0; s < Geo<DIM>::KS; ++s) raw[s] = bload16(src, (i * DIM + 8 * g + 32 * s) * 2, soff);
}

// Registers -> LDS as bf16 elu(x) for tiles whose rows past the end were
// loaded as zero (elu(0) = 0, so no row guard is needed).
template <int DIM, int NW = 4>
__device__ __forceinline__ void store_tile_e(uint16_t* lds, const i32x4 (&raw)[(Geo<DIM, NW>::PC)]) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + G::NT * r;
    f32x8_t x = unpack8(__builtin_bit_cast(i16x8, raw[r]));
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = elu_fast(x[e]);
    *reinterpret_cast<i16x8*>(lds + (p / G::ROW8) * G::LD + (p % G::ROW8) * 8) = pack8(x);
  }
}

// The split phi = mu + E that the backward's dq sweep and the segment
// aggregates carry, with one constant mu_f per feature f: the mu part is
// summed in fp32 and only E = phi - mu is rounded to bf16.  Where a sum over
// keys cancels along a direction in which phi is nearly constant (every
// key's phi close to mu), a bf16 rounding of phi itself would leave an error
// of 2^-9 phi that the cancellation amplifies; E = phi - mu keeps the
// rounding relative to the spread instead.  mu_rule takes mu_f = 1 where the
// mean phi m of feature f is within 1/8 of 1 (then E = elu, and a segment
// whose features all have mu = 1 runs the plain split), and m rounded to
// bf16 otherwise (so that mu is exact as an MFMA operand).
__device__ __forceinline__ float mu_rule(float m) {
  return fabsf(m - 1.f) <= 0.125f ? 1.f : fb(bf(m));
}

// decide_mu over a chunk: the mean phi of column f of the bf16 elu tile sE
// (rows < nrow), one thread per feature so the sum has a fixed order.  sMuF
// gets mu as fp32, sMuB as bf16 bits (the same value).
template <int DIM, int LD>
__device__ __forceinline__ void decide_mu(const uint16_t* sE, int nrow, float* sMuF, uint16_t* sMuB) {
  const int d = threadIdx.x;
  if (d < DIM) {
    float s = 0.f;
    for (int j = 0; j < nrow; ++j) s += fb(static_cast<short>(sE[j * LD + d]));
    const float mu = nrow > 0 ? mu_rule(1.f + s / static_cast<float>(nrow)) : 1.f;
    sMuF[d] = mu;
    sMuB[d] = static_cast<uint16_t>(bf(mu));
  }
}

// The thread's mu for the eight features of its tile pieces (feature
// 8 (p % ROW8) + e, the same for all of a thread's pieces since the
// workgroup size is a multiple of ROW8).
struct MuOff {
  float c[8];
};
template <int DIM, int NW = 4>
__device__ __forceinline__ MuOff mu_offsets(const float* sMuF) {
  const int c8 = threadIdx.x % Geo<DIM, NW>::ROW8;
  MuOff m;
#pragma unroll
  for (int e = 0; e < 8; ++e) m.c[e] = sMuF[8 * c8 + e];
  return m;
}

// E = phi(x) - mu for a raw bf16 piece, in fp32 and then rounded to bf16.
__device__ __forceinline__ i16x8 emu8(i32x4 raw, const MuOff& m) {
  f32x8_t x = unpack8(__builtin_bit_cast(i16x8, raw));
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = phi_fast(x[e]) - m.c[e];
  return pack8(x);
}

// Registers -> LDS as bf16 E = phi(x) - mu; rows j >= nrow are zero.
template <int DIM, int NW = 4>
__device__ __forceinline__ void store_tile_emu(uint16_t* lds, const i32x4 (&raw)[(Geo<DIM, NW>::PC)], int nrow,
                                               const MuOff& m) {
  using G = Geo<DIM, NW>;
  static_assert(G::NT % G::ROW8 == 0, "a thread's pieces share their features");
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + G::NT * r;
    const int j = p / G::ROW8;
    const i16x8 val = emu8(raw[r], m);
    *reinterpret_cast<i16x8*>(lds + j * G::LD + (p % G::ROW8) * 8) =
        j < nrow ? val : i16x8{0, 0, 0, 0, 0, 0, 0, 0};
  }
}

// Registers -> LDS unchanged (rows past the end already zero).
template <int DIM, int NW = 4>
__device__ __forceinline__ void store_tile_v(uint16_t* lds, const i32x4 (&raw)[(Geo<DIM, NW>::PC)]) {
  using G = Geo<DIM, NW>;
#pragma unroll
  for (int r = 0; r < G::PC; ++r) {
    const int p = threadIdx.x + G::NT * r;
    *reinterpret_cast<i16x8*>(lds + (p / G::ROW8) * G::LD + (p % G::ROW8) * 8) = __builtin_bit_cast(i16x8, raw[r]);
  }
}

// This wave's query rows (i = 16w + li), 8 features per k-step.
template <int DIM>
__device__ __forceinline__ void load_q(i32x4 (&raw)[Geo<DIM>::KS], const bf16_t* __restrict__ src, int64_t c0,
                                       int nrow, int i, int g) {
#pragma unroll
  for (int s = 0; s < Geo<DIM>::KS; ++s)
    raw[s] = i < nrow ? gload16(src + (c0 + i) * DIM + 8 * g + 32 * s) : i32x4{0, 0, 0, 0};
}

}  // namespace mf
}  // namespace la
