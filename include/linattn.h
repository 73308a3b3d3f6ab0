/*
 * linattn.h -- C ABI of the MI355X (gfx950) causal linear-attention library.
 *
 * The method (phi = elu + 1 feature map; prefix states S_i, Z_i; readout
 * phi(Q_i)^T S_i / phi(Q_i)^T Z_i) is defined on the page
 * "[Paper walkthrough] Transformers are RNNs" (wkq9411.github.io):
 *   section 2  -- phi(x) = elu(x) + 1 with alpha = 1, and the non-causal
 *                 form phi(Q)(phi(K)^T V) (eq:linear);
 *   section 3  -- the causal mask (eq:mask), S_i = sum_{j<=i} phi(K_j) V_j^T,
 *                 Z_i = sum_{j<=i} phi(K_j), readout eq:output;
 *   section 3.1 -- the cumulative-sum gradients eq:gq .. eq:gv;
 *   section 4  -- the RNN form s_i = s_{i-1} + phi(k_i) v_i^T,
 *                 z_i = z_{i-1} + phi(k_i), s_0 = z_0 = 0.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller.  The library
 *    allocates no device memory; scratch space comes from the caller's
 *    `workspace` (size from la_workspace_bytes).  It keeps no state between
 *    calls except a thread-local error string.
 *  - Tensors are contiguous row-major: q, k [B,H,N,D]; v, out, dout
 *    [B,H,N,M]; den [B,H,N]; decode state S [B,H,D,M], Z [B,H,D]; decode
 *    inputs q, k [B,H,D], v, out [B,H,M].
 *  - `dtype` (la_dtype) applies to q, k, v, out, dout, dq, dk, dv.  All
 *    accumulation is fp32; den, S and Z are always fp32.  bf16 results are
 *    rounded to nearest even.
 *  - Sizes: B, H, N >= 1; 1 <= D, M <= 256 (LA_ERR_UNSUPPORTED otherwise).
 *  - Alignment: every tensor pointer must be aligned to its element size
 *    (2 bytes bf16, 4 bytes fp32; LA_ERR_INVALID otherwise); workspace and
 *    saved records must be 16-byte aligned.  The MFMA kernels move tensors in
 *    16-byte vectors, so they run only when every q, k, v, out, dout, dq,
 *    dk, dv pointer of the call is 16-byte aligned (any pointer from
 *    hipMalloc or torch's allocator is).  A call on the automatic plan
 *    with a pointer that is only element-aligned runs the generic kernels
 *    instead, cut into the same segments (so the sizes la_workspace_bytes
 *    and la_saved_bytes report still suffice); a plan that asks for the
 *    MFMA kernels is then refused with LA_ERR_UNSUPPORTED.  The retention,
 *    polynomial and softmax calls, which have no generic kernels, return
 *    LA_ERR_UNSUPPORTED unless their tensor pointers are 16-byte aligned
 *    (state pointers S, Z, S0, dS0 and the fp32 outputs den_out, lse,
 *    dlog_gamma need 4 bytes).
 *  - Outputs must not overlap inputs (LA_ERR_INVALID), except the decode
 *    state S, Z, which is updated in place by design.
 *  - Validation runs before any HIP call: null pointers, sizes < 1, unknown
 *    dtype, overlapping buffers and a too-small workspace return at once
 *    with LA_ERR_INVALID (or LA_ERR_UNSUPPORTED) and set la_last_error().
 *  - Calls enqueue work on `stream` (NULL = the default stream) and return
 *    without synchronising.  A launch failure returns LA_ERR_DEVICE; a fault
 *    inside a kernel surfaces at the caller's next synchronisation.
 *  - No atomics are used in reductions: for a fixed plan the results are
 *    bitwise reproducible.
 */
#ifndef LINATTN_H
#define LINATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum la_status {
  LA_OK = 0,
  LA_ERR_INVALID = 1,     /* bad argument: null, size < 1, overlap, workspace */
  LA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. D or M > 256)   */
  LA_ERR_DEVICE = 3       /* a HIP call failed (launch, stream)              */
} la_status;

typedef enum la_dtype { LA_F32 = 0, LA_BF16 = 1 } la_dtype;

typedef enum la_op {
  LA_OP_FORWARD = 0,
  LA_OP_BACKWARD = 1,
  LA_OP_PREFIX_STATE = 2,
  LA_OP_DECODE = 3,
  LA_OP_FORWARD_STATE = 4,  /* la_forward_state  */
  LA_OP_BACKWARD_STATE = 5, /* la_backward_state */
  LA_OP_RETENTION_FORWARD = 6,  /* la_retention_forward  */
  LA_OP_RETENTION_BACKWARD = 7, /* la_retention_backward */
  LA_OP_POLY_BACKWARD = 8       /* la_poly_backward      */
} la_op;

/* Kernel family choice for the *_ex entry points (0 = automatic).
 * LA_KERNEL_MFMA_ONE_LAUNCH: the MFMA kernels, with the causal bf16
 * backward at D = M = 64 as one launch (see la_backward_ex); elsewhere the
 * same as LA_KERNEL_MFMA. */
typedef enum la_kernel {
  LA_KERNEL_AUTO = 0,
  LA_KERNEL_GENERIC = 1,
  LA_KERNEL_MFMA = 2,
  LA_KERNEL_MFMA_ONE_LAUNCH = 3
} la_kernel;

/* Tuning plan.  Every field 0 means "let the library choose".
 *   chunk    -- tokens per intra-chunk tile (generic: 16 or 32; MFMA: 64,
 *               or 128 for the bf16 forward at D = M = 64: segments are then
 *               whole 128-token chunks, and the other kernels of a call with
 *               this plan keep 64-token chunks over those segments)
 *   segments -- how many independent pieces each sequence is cut into along
 *               N; each piece's state is carried in by an exclusive scan of
 *               the pieces before it (the prefix sums split exactly by
 *               associativity).
 *   kernel   -- la_kernel. */
typedef struct la_plan {
  int32_t chunk;
  int32_t segments;
  int32_t kernel;
} la_plan;

/* Forward.  out_i = phi(Q_i)^T S_i / phi(Q_i)^T Z_i (causal != 0, the sums
 * run over j <= i: "Transformers are RNNs" walkthrough, section 3, eq:mask
 * and eq:output) or phi(Q_i)^T S_N / phi(Q_i)^T Z_N (causal == 0: section 2,
 * eq:linear).  No scale and no epsilon are applied.
 *   q, k: [B,H,N,D]; v: [B,H,N,M]  (inputs, dtype)
 *   out:  [B,H,N,M]                 (output, dtype)
 *   den_out: [B,H,N] fp32 row denominators phi(Q_i)^T Z_i, or NULL (the
 *            backward does not need it: it forms den itself in fp32). */
la_status la_forward(const void* q, const void* k, const void* v, void* out,
                     int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                     int causal, int dtype, float* den_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/* As la_forward, with a tuning plan (NULL = automatic) and, when `saved` is
 * not NULL, the prefix states it computes kept for la_backward_ex: fp32
 * records of D*M + D floats (S row-major, then Z), the state entering each
 * segment of the plan for causal != 0 ([B,H,segments], none when the plan
 * has one segment), or the totals S_N, Z_N for causal == 0 ([B,H]).
 * `saved_bytes` must be at least la_saved_bytes(); `saved` is 16-byte
 * aligned and must not overlap any other argument. */
la_status la_forward_ex(const void* q, const void* k, const void* v, void* out,
                        int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                        int causal, int dtype, float* den_out,
                        float* saved, size_t saved_bytes,
                        void* workspace, size_t workspace_bytes, hipStream_t stream,
                        const la_plan* plan);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): la_forward
 * with no workspace argument.  The segment records it needs live in a static
 * device array of the library, 64 MiB (67108864 bytes) per GPU, held from the
 * first call on that GPU until the process ends; the call allocates nothing
 * and calls no allocating routine.  Same arguments, plan, kernels and results
 * (bit for bit) as la_forward; the scratch it needs is la_workspace_bytes
 * (LA_OP_FORWARD, ...) bytes, and a call needing more than 64 MiB returns
 * LA_ERR_UNSUPPORTED before any HIP call (with the automatic plan a causal
 * call needs at most about 34 MB: 512 segment records of D*M + D floats).
 * Nothing in the scratch needs to start at zero.  All calls on one GPU share
 * its array and it keeps the last call's contents: calls that overlap on one
 * GPU (concurrent streams, or several host threads) race and must be
 * serialised by the caller.  `stream` must belong to the calling thread's
 * current device (LA_ERR_DEVICE otherwise); the array's address on a device
 * is looked up once, on that device's first call (a call that is being
 * captured into a graph should not be a device's first). */
la_status la_forward_noalloc(const void* q, const void* k, const void* v, void* out,
                             int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                             int causal, int dtype, float* den_out, hipStream_t stream);

/* Bytes of the `saved` record of la_forward_ex for these sizes and plan (0
 * when there is nothing to keep: causal with a single segment). */
size_t la_saved_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                      int causal, int dtype, const la_plan* plan);

/* Backward of L = sum(dout * out) with respect to the RAW q, k, v.
 * Numerator terms: "Transformers are RNNs" walkthrough, section 3.1,
 * eq:gq (prefix matrix) and the phi(K) / V equations up to eq:gv (suffix
 * matrix).  Normaliser terms (left there to autograd) by the chain rule:
 * g_i = dout_i / den_i, c_i = -(dout_i . out_i) / den_i,
 *   grad phi(Q_i) = S_i g_i + c_i Z_i,
 *   grad phi(K_i) = R_i V_i + r_i,   grad V_i = R_i^T phi(K_i),
 * with R_i = sum_{j>=i} phi(Q_j) g_j^T, r_i = sum_{j>=i} c_j phi(Q_j); then
 * dq = grad phi(Q) * phi'(q), dk = grad phi(K) * phi'(k), dv = grad V.
 *   q, k, v: forward inputs; out: the forward's output; dout: upstream grad
 *   den: [B,H,N] fp32 from la_forward, or NULL
 *   dq, dk: [B,H,N,D]; dv: [B,H,N,M] (outputs, dtype)
 * out and den are checked (size, alignment, no overlap with the outputs) but
 * not read: the first sweep forms num_i and den_i of every row in fp32 from
 * the prefix state, as the forward does, and takes c_i = -(dout_i . num_i) /
 * den_i^2 from them.  A c_i from the stored bf16 out would carry out's 2^-9
 * rounding, and for phi ~ 1 the two terms of grad phi(Q) cancel in the
 * all-ones direction several times over, so dq would lose about a decimal
 * digit.
 * Precision (bf16): the MFMA kernels feed bf16 operands to the matrix cores
 * with fp32 accumulation; where a sum would cancel along a direction in
 * which phi is nearly constant they split phi = mu + E per feature (mu the
 * mean phi of a segment's first chunk, rounded to bf16, or 1 where that mean
 * is within 1/8 of 1) and keep the mu part in fp32, so E's bf16 rounding is
 * relative to phi's spread rather than its size.  Against the fp64 result
 * the gradients' relative L2 error measures 2e-3 to 4e-3 for q, k ~ N(0,
 * 1/D) or N(0, 1), for q, k ~ N(-3, 1), with every other feature shifted to
 * -3, with only the keys shifted, and for q, k ~ N(s, 1/D) with s = -3, -1
 * or +2 (v ~ N(0, 1/D) or N(0, 1), dout ~ N(0, 1)); features below about
 * -12, where phi < 1e-5 is held to fp32's absolute rounding, are not covered.
 * fp32 inputs: ~1e-6. */
la_status la_backward(const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* den, void* dq, void* dk, void* dv,
                      int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                      int causal, int dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/* As la_backward, with a tuning plan (NULL = automatic) and `saved` (below).
 * With plan kernel LA_KERNEL_MFMA_ONE_LAUNCH the causal bf16 MFMA backward at
 * D = M = 64 runs as one launch when its grid fits on the device at once:
 * each workgroup sweeps its segment forwards (dq), hands its suffix
 * aggregate to the workgroups of the earlier segments through flags in the
 * workspace and sweeps the same segment backwards (dk, dv) from the later
 * segments' aggregates; results are those of the default two launches, bit
 * for bit (measured slower on MI355X: the default stays two launches).  A
 * hand-off that times out is reported by la_device_error.
 * `saved`: the record la_forward_ex left for the same q, k, v, sizes, causal, dtype and
 * plan, or NULL.  With it the prefix states S, Z are read instead of being
 * recomputed (a pass over k and v and a scan fewer).  LA_ERR_INVALID if
 * saved_bytes is short of la_saved_bytes() or the forward and backward
 * plans cut the sequence differently (e.g. different kernels requested). */
la_status la_backward_ex(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* den,
                         const float* saved, size_t saved_bytes,
                         void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                         int causal, int dtype,
                         void* workspace, size_t workspace_bytes, hipStream_t stream,
                         const la_plan* plan);

/* Causal forward that carries a state across calls: the N tokens continue
 * a sequence whose earlier tokens left the state (S0, Z0) (the RNN form of
 * the walkthrough's section 4 starts from s_0 = z_0 = 0; "The deep link
 * between Transformer and RNN" (xxqk.cn), section 4.2, keeps one state per
 * session and saves / restores it):
 *   out_i = phi(Q_i)^T (S0 + S_i) / phi(Q_i)^T (Z0 + Z_i),
 * and the state after the N tokens, S0 + S_N and Z0 + Z_N, is written to
 * S_out, Z_out.  A prefill, a multi-token decode step and the next block of
 * a long sequence are all this call; its state feeds la_decode_step.
 *   S0 [B,H,D,M], Z0 [B,H,D] fp32, or both NULL (zero state);
 *   S_out [B,H,D,M], Z_out [B,H,D] fp32, or both NULL; they may be S0, Z0
 *     themselves (updated in place) but must not overlap them otherwise;
 *   q, k, v, out, den_out as in la_forward (causal); workspace from
 *   la_workspace_bytes(LA_OP_FORWARD_STATE, ...). */
la_status la_forward_state(const void* q, const void* k, const void* v, void* out,
                           int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype,
                           const float* S0, const float* Z0, float* S_out, float* Z_out,
                           float* den_out, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Backward of la_forward_state (L = sum(dout * out)): dq, dk, dv as in
 * la_backward with the prefix sweep starting from (S0, Z0), and, since every
 * row reads the carried state, dL/dS0 = sum_i phi(Q_i) g_i^T and
 * dL/dZ0 = sum_i c_i phi(Q_i) (the full suffix sums R_1, r_1) into dS0
 * [B,H,D,M] and dZ0 [B,H,D] fp32 (both NULL to skip).  Workspace from
 * la_workspace_bytes(LA_OP_BACKWARD_STATE, ...). */
la_status la_backward_state(const void* q, const void* k, const void* v, const void* out,
                            const void* dout, const float* den, const float* S0, const float* Z0,
                            void* dq, void* dk, void* dv, float* dS0, float* dZ0,
                            int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decayed / gated linear attention ("retention"): "08 - Transformer and
 * Variants" (by-xin.github.io), section 1.3.4 -- RetNet's H_t = gamma
 * H_{t-1} + v_t k_t^T, y_t = H_t q_t, and gated retention with a per-token
 * gamma_t; no feature map and no normaliser, as printed.  The state is
 * stored as S = H^T [B,H,D,M] fp32 (S_t = gamma_t S_{t-1} + k_t v_t^T,
 * y_t = S_t^T q_t), so
 *   y_i = sum_{j<=i} exp(L_i - L_j) (q_i . k_j) v_j + exp(L_i) S0^T q_i,
 *   L_i = sum_{l<=i} log gamma_l.
 *   q, k: [B,H,N,D]; v, y: [B,H,N,M] (bf16, D = M in {64, 128}; other
 *     shapes and dtypes return LA_ERR_UNSUPPORTED)
 *   log_gamma: [B,H,N] fp32, log of the decay, <= 0 (RetNet: one value per
 *     head repeated; gamma = 1 gives the undecayed sum); values below -80
 *     are taken as -80 (gamma ~ 0, a full reset); NaN propagates
 *   S0: [B,H,D,M] fp32 state carried in, or NULL (zero);
 *   S_out: [B,H,D,M] fp32, the state after the N tokens, or NULL; may be S0
 *     itself (in place).
 * Workspace from la_workspace_bytes(LA_OP_RETENTION_FORWARD, ...). */
la_status la_retention_forward(const void* q, const void* k, const void* v, const float* log_gamma,
                               void* y, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                               int dtype, const float* S0, float* S_out, float* saved,
                               size_t saved_bytes, void* workspace, size_t workspace_bytes,
                               hipStream_t stream);

/* Bytes of la_retention_forward's `saved` record for these sizes: the state
 * entering each segment of its plan ([B,H,segments] records of D*M + D
 * floats: S row-major, then D floats the library uses internally), which
 * la_retention_backward reads instead of recomputing them.  `saved` is
 * 16-byte aligned, caller-owned, and must not overlap any other argument;
 * NULL keeps nothing.  0 for unsupported sizes. */
size_t la_retention_saved_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype);

/* Backward of la_retention_forward for L = sum(dy * y), by the chain rule
 * through the recurrence (the page gives no gradients):
 *   dq_i = S_i dy_i;  R_j = sum_{i>=j} exp(L_i - L_j) q_i dy_i^T;
 *   dk_j = R_j v_j;  dv_j = R_j^T k_j;  dS0 = gamma_1 R_1;
 *   dlog_gamma_t = sum_{m>=t} (q_m . dq_m - k_m . dk_m).
 *   dq, dk: [B,H,N,D], dv: [B,H,N,M] (dtype); dlog_gamma: [B,H,N] fp32;
 *   dS0: [B,H,D,M] fp32 or NULL; S0 as given to the forward (or NULL);
 *   saved: the record la_retention_forward kept for the same q, k, v,
 *     log_gamma, S0 and sizes, or NULL (then the states are recomputed);
 *     LA_ERR_INVALID when saved_bytes is short of la_retention_saved_bytes().
 * Workspace from la_workspace_bytes(LA_OP_RETENTION_BACKWARD, ...). */
la_status la_retention_backward(const void* q, const void* k, const void* v, const float* log_gamma,
                                const void* dy, const float* S0, const float* saved,
                                size_t saved_bytes, void* dq, void* dk, void* dv,
                                float* dlog_gamma, float* dS0, int64_t B, int64_t H, int64_t N,
                                int64_t D, int64_t M, int dtype, void* workspace,
                                size_t workspace_bytes, hipStream_t stream);

/* One decayed recurrent step per (b,h), in place ("08 - Transformer and
 * Variants", section 1.3.4, the recurrence itself):
 *   S <- gamma S + k v^T,  y = S^T q,  gamma = exp(log_gamma[b,h]).
 *   S: [B,H,D,M] fp32, read and written (owned by the caller; a state from
 *   la_retention_forward's S_out continues that sequence);
 *   q, k: [B,H,D], v, y: [B,H,M] (dtype, fp32 or bf16); log_gamma: [B,H]
 *   fp32 (below -80 taken as -80).  Any D, M <= 256.  Inputs must not
 *   overlap S or y; no workspace. */
la_status la_retention_decode_step(float* S, const void* q, const void* k, const void* v,
                                   const float* log_gamma, void* y, int64_t B, int64_t H, int64_t D,
                                   int64_t M, int dtype, hipStream_t stream);

/* Linear attention with the degree-2 polynomial kernel ("[Paper
 * walkthrough] Transformers are RNNs", section 2, "feature map and
 * computation cost", item (3): sim(q, k) = (q^T k)^2, C = D^2 features),
 * in eq:common form, causal per eq:mask when causal != 0:
 *   out_i = sum_{j<=i} (q_i . k_j)^2 v_j / den_i,  den_i = sum_{j<=i} (q_i . k_j)^2,
 * with out_i = 0 where den_i = 0 (no epsilon; every weight is then 0).
 *   q, k: [B,H,N,D], v, out: [B,H,N,M] (bf16, D = M in {64, 128});
 *   den_out: [B,H,N] fp32 or NULL (kept for la_poly_backward).
 * The weights enter the numerator rounded to bf16 and out is normalised by
 * their sum (an exact convex combination of the values); den_out is the sum
 * of the fp32 weights.
 * No workspace.  LA_ERR_UNSUPPORTED for other dtypes or sizes. */
la_status la_poly_forward(const void* q, const void* k, const void* v, void* out, float* den_out,
                          int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                          int dtype, hipStream_t stream);

/* Backward of la_poly_forward for L = sum(dout * out), by the chain rule
 * through the masked sum (the page gives no gradients); with
 * s_ij = q_i . k_j, g_i = dout_i / den_i, c_i = -(dout_i . out_i) / den_i:
 *   dS_ij = 2 s_ij (g_i . v_j + c_i) over the masked pairs,
 *   dq_i = sum_j dS_ij k_j,  dk_j = sum_i dS_ij q_i,  dv_j = sum_i s_ij^2 g_i,
 * and g_i = c_i = 0 where den_i = 0.
 *   out, den: la_poly_forward's outputs for the same q, k, v and causal
 *   (den required); dout: [B,H,N,M]; dq, dk: [B,H,N,D], dv: [B,H,N,M].
 * Workspace from la_workspace_bytes(LA_OP_POLY_BACKWARD, ...) (B*H*N
 * floats). */
la_status la_poly_backward(const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* den, void* dq, void* dk, void* dv,
                           int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                           int dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The polynomial map's linear-form state after N tokens ("[Paper
 * walkthrough] Transformers are RNNs", section 2, item (3), with eq:mask's
 * S, Z): S[c][m] = sum_t phi(k_t)_c v_t[m], Z[c] = sum_t phi(k_t)_c, with
 * phi(k)_{a D + b} = k_a k_b (C = D^2 rows).
 *   k: [B,H,N,D], v: [B,H,N,M] (bf16, D = M in {64, 128});
 *   S: [B,H,D*D,M] fp32, Z: [B,H,D*D] fp32 (outputs, overwritten).
 * The products enter the state rounded to bf16 once; Z sums them in fp32.
 * No workspace. */
la_status la_poly_prefix_state(const void* k, const void* v, float* S, float* Z, int64_t B,
                               int64_t H, int64_t N, int64_t D, int64_t M, int dtype,
                               hipStream_t stream);

/* One recurrent step of the polynomial map per (b,h), in place (the
 * section 4 loop with phi(x)_{a D + b} = x_a x_b):
 *   S <- S + phi(k) v^T,  Z <- Z + phi(k),  out = phi(q)^T S / phi(q)^T Z
 * (0 where the denominator is 0).
 *   S: [B,H,D*D,M], Z: [B,H,D*D] fp32 (read and written, caller-owned);
 *   q, k: [B,H,D], v, out: [B,H,M] (fp32 or bf16); D a power of two <= 128,
 *   M <= 256.  No workspace. */
la_status la_poly_decode_step(float* S, float* Z, const void* q, const void* k, const void* v,
                              void* out, int64_t B, int64_t H, int64_t D, int64_t M, int dtype,
                              hipStream_t stream);

/* Softmax attention, the comparison baseline ("[Paper walkthrough]
 * Transformers are RNNs", section 1, eq:softmax; causal per eq:mask),
 * computed blockwise with the running maximum / denominator / weighted sum
 * update of "Transformer study notes (4)", section "FlashAttention":
 *   out = softmax(Q K^T / sqrt(D)) V,  lse_i = log sum_j exp(q_i.k_j / sqrt(D)).
 *   q, k: [B,H,N,D], v, out: [B,H,N,M] (bf16, D = M in {64, 128});
 *   lse: [B,H,N] fp32 or NULL.  No workspace. */
la_status la_softmax_forward(const void* q, const void* k, const void* v, void* out, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                             int dtype, hipStream_t stream);

/* One KV-cache decode step per (b,h) ("The deep link between Transformer and
 * RNN", section 3): append (k, v) at position L of the caches, then
 *   out = softmax(q . K[0..L] / sqrt(D)) V[0..L].
 *   k_cache: [B,H,capacity,D], v_cache: [B,H,capacity,M] (dtype; caller-owned,
 *   positions 0 .. L-1 filled, position L written), 0 <= L < capacity;
 *   q, k: [B,H,D], v, out: [B,H,M]; fp32 or bf16, D = M in {64, 128}.
 *   The caller advances L.  No workspace. */
la_status la_softmax_decode_step(void* k_cache, void* v_cache, const void* q, const void* k,
                                 const void* v, void* out, int64_t B, int64_t H, int64_t L,
                                 int64_t capacity, int64_t D, int64_t M, int dtype,
                                 hipStream_t stream);

/* One RNN decode step per (b,h), in place ("Transformers are RNNs"
 * walkthrough, section 4; the state is updated first, then read):
 *   S <- S + phi(k) v^T;  Z <- Z + phi(k);  out = phi(q)^T S / phi(q)^T Z.
 *   S: [B,H,D,M] fp32, Z: [B,H,D] fp32 (in/out; caller-owned, so a saved
 *      copy of S, Z is a checkpoint of the session)
 *   q, k: [B,H,D]; v, out: [B,H,M] (dtype).  Needs no workspace. */
la_status la_decode_step(float* S, float* Z, const void* q, const void* k, const void* v,
                         void* out, int64_t B, int64_t H, int64_t D, int64_t M,
                         int dtype, hipStream_t stream);

/* State after a prefix (section 3's S_N, Z_N; overwrites S and Z):
 *   S = sum_j phi(K_j) V_j^T, Z = sum_j phi(K_j) over the N tokens.
 *   k: [B,H,N,D]; v: [B,H,N,M] (dtype); S: [B,H,D,M], Z: [B,H,D] fp32. */
la_status la_prefix_state(const void* k, const void* v, float* S, float* Z,
                          int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                          int dtype, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* Workspace bytes an entry point needs for these sizes (0 if none).
 * `op` is la_op; `plan` may be NULL (automatic plan, as the plain calls). */
size_t la_workspace_bytes(int op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                          int causal, int dtype);
size_t la_workspace_bytes_ex(int op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                             int causal, int dtype, const la_plan* plan);

/* Resolve the automatic plan for a call (what la_forward / la_backward use). */
la_status la_resolve_plan(int op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M,
                          int causal, int dtype, const la_plan* requested, la_plan* resolved);

/* Per-kernel timing (a tracing aid for benchmarks and profiling runs).
 * la_profile_enable(1) clears earlier records and starts bracketing every
 * kernel the library launches with a pair of HIP events recorded on that
 * launch's stream; la_profile_enable(0) stops.  la_profile_report waits for
 * the recorded events, writes one line per kernel name into buf,
 *   "<name> <launches> <total milliseconds>\n",
 * and clears the records.  LA_ERR_INVALID if buf is NULL or too small. */
la_status la_profile_enable(int on);
la_status la_profile_report(char* buf, size_t len);
/* Restrict the timing to the kernels named in `names` (comma-separated,
 * e.g. "mfma.bwd_dq"); NULL or "" times every kernel.  Each timed launch
 * adds two event records to its stream, so timing only the kernel of
 * interest keeps the rest of the stream undisturbed. */
la_status la_profile_select(const char* names);

const char* la_status_str(int status);
/* Detail of the last non-OK status returned on this thread ("" if none). */
const char* la_last_error(void);

/* Synchronises `stream` and reports (then clears) an error a kernel of this
 * library recorded on the stream's device: LA_ERR_DEVICE when a bounded wait
 * of one workgroup for another's result ran out.  The one kernel that waits
 * so, the one-launch causal backward (see la_backward), is launched only
 * when its whole grid fits on the device at once, and every workgroup only
 * waits for workgroups dispatched before it; should a wait still run out
 * (after 0.5 s), that workgroup writes NaN into its dk, dv rows, sets the
 * error and finishes normally. */
la_status la_device_error(hipStream_t stream);
/* Library version, major * 10000 + minor * 100 + patch. */
int la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LINATTN_H */
