// Host-side launch interface between the C ABI (la_host.hip) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// Per-head state record in a workspace: D*M floats of S (row-major [D][M])
// followed by D floats of Z (or R, r for the backward's suffix records);
// E = D*M + D.
__host__ __device__ inline int64_t state_elems(int D, int M) { return static_cast<int64_t>(D) * M + D; }

// Retention backward: the gate gradients are anchored every kRetAnchor tokens
// inside a segment (as well as at its end).  Anchor k of a segment starting
// at r0 sits at token r0 + k kRetAnchor (k >= 1, strictly inside the
// segment); a segment of seg_len tokens has at most ret_anchors(seg_len).
constexpr int kRetAnchor = 1024;
__host__ __device__ inline int ret_anchors(int64_t seg_len) {
  return seg_len > 0 ? static_cast<int>((seg_len - 1) / kRetAnchor) : 0;
}

struct SegGeom {
  int64_t BH;   // B * H independent sequences
  int64_t N;    // tokens per sequence
  int D, M;     // feature widths
  int P;        // segments per sequence
  int seg_len;  // tokens per segment (a multiple of the chunk)
  int chunk;    // tokens per intra-chunk tile
  // segment-state passes: aggregates of segments 0 .. nseg - 1 only (0: all
  // P).  A causal forward that returns no final state never reads the last
  // segment's aggregate (the exclusive scan only hands it to the total).
  int nseg = 0;
};

// ---- generic kernels (any D, M with D*M <= 16384, fp32 or bf16 inputs) ----
// dtype: 0 = fp32, 1 = bf16 (raw 16-bit).

// Largest chunk (32 or 16) whose LDS footprint fits a CU for kernel `which`
// (0 forward, 1 segment state, 2 backward dq, 3 backward dk/dv); 0 if none.
int generic_chunk_for(int D, int M, int which);

// Segment aggregates dS = sum phi(K_j) V_j^T, dZ = sum phi(K_j) over each
// segment; written at s_out + (bh*P + s)*s_stride and z_out + (bh*P + s)*z_stride.
hipError_t launch_seg_state_generic(int dtype, const SegGeom& g, const void* k, const void* v, float* s_out,
                                    int64_t s_stride, float* z_out, int64_t z_stride, hipStream_t st);

// In-place exclusive scan of [BH][P][E] records over the segment axis
// (reverse = suffix sums), starting from init_s [BH][D*M], init_z [BH][D]
// when init_s is not null (a state carried in from earlier tokens) and from
// zero otherwise.  The inclusive total of each head goes to
// tot_s + bh*ts_stride (first D*M entries) and tot_z + bh*tz_stride (last D),
// when tot_s is not null; a total may overwrite its init in place.
hipError_t launch_seg_scan(float* agg, int64_t BH, int P, int D, int M, int reverse,
                           const float* init_s, const float* init_z, float* tot_s, int64_t ts_stride,
                           float* tot_z, int64_t tz_stride, hipStream_t st);

// Chunked forward.  carry: per-(bh, segment) exclusive prefix records
// (causal) or per-bh totals (non-causal), or null for a zero state (P == 1).
// out may be null (then only den_out is produced).
hipError_t launch_forward_generic(int dtype, int causal, const SegGeom& g, const void* q, const void* k,
                                  const void* v, void* out, float* den_out, const float* carry,
                                  hipStream_t st);

// Backward, forward sweep: dq, the per-row c and den [BH][N] (formed in fp32
// from the carried state; the stored out and den are not read) and, as a
// by-product, the per-segment suffix aggregates (R, r) written to r_agg
// [BH][P][E].
hipError_t launch_bwd_dq_generic(int dtype, int causal, const SegGeom& g, const void* q, const void* k,
                                 const void* v, const void* dout, const float* carry_s, void* dq, float* r_agg,
                                 float* c_out, float* den_out, hipStream_t st);

// Backward, reverse sweep: dk, dv from the suffix carry (exclusive suffix
// records for causal, per-bh totals for non-causal) and the forward sweep's
// den and c.
hipError_t launch_bwd_dkdv_generic(int dtype, int causal, const SegGeom& g, const void* q, const void* k,
                                   const void* v, const void* dout, const float* den, const float* c,
                                   const float* carry_r, void* dk, void* dv, hipStream_t st);

// ---- decode ----
hipError_t launch_poly_decode_step(int dtype, int64_t BH, int D, int M, float* S, float* Z, const void* q,
                                   const void* k, const void* v, void* out, hipStream_t st);
hipError_t launch_ret_decode_step(int dtype, int64_t BH, int D, int M, float* S, const void* q, const void* k,
                                  const void* v, const float* lg, void* y, hipStream_t st);
hipError_t launch_decode_step(int dtype, int64_t BH, int D, int M, float* S, float* Z, const void* q,
                              const void* k, const void* v, void* out, hipStream_t st);

}  // namespace la
