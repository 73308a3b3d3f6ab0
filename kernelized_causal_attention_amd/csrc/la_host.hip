// C ABI of the library: argument validation (before any HIP call), plan
// choice, workspace carving and kernel dispatch.  See include/linattn.h.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <initializer_list>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "la_internal.h"
#include "linattn.h"

#define LA_API extern "C" __attribute__((visibility("default")))

namespace la {
int mfma_supported(int op, int64_t D, int64_t M, int dtype);
hipError_t launch_forward_mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                               void* out, float* den_out, const float* carry, hipStream_t st);
hipError_t launch_seg_state_mfma(const SegGeom& g, const void* k, const void* v, float* s_out,
                                 int64_t s_stride, float* z_out, int64_t z_stride, hipStream_t st);
int retention_supported(int64_t D, int64_t M, int dtype);
hipError_t launch_ret_seg_state(const SegGeom& g, const void* k, const void* v, const float* lg, float* recs,
                                hipStream_t st);
hipError_t launch_ret_scan(float* recs, int64_t BH, int P, int D, int M, const float* init, float* tot,
                           hipStream_t st);
hipError_t launch_ret_forward(const SegGeom& g, const void* q, const void* k, const void* v, const float* lg, void* y,
                              const float* carry, hipStream_t st);
int poly_supported(int64_t D, int64_t M, int dtype);
hipError_t launch_poly_forward(int64_t BH, int64_t N, int D, const void* q, const void* k, const void* v, void* out,
                               float* den, int causal, hipStream_t st);
int softmax_supported(int64_t D, int64_t M, int dtype);
hipError_t launch_softmax_forward(int64_t BH, int64_t N, int D, const void* q, const void* k, const void* v,
                                  void* out, float* lse, int causal, hipStream_t st);
hipError_t launch_softmax_decode(int dtype, int64_t BH, int D, void* kc, void* vc, const void* q, const void* k,
                                 const void* v, void* out, int64_t L, int64_t cap, hipStream_t st);
hipError_t launch_poly_state(int64_t BH, int64_t N, int D, const void* k, const void* v, float* S, float* Z,
                             hipStream_t st);
hipError_t launch_poly_bwd(int pass, int64_t BH, int64_t N, int D, const void* q, const void* k, const void* v,
                           const void* out, const void* dout, const float* den, void* dq, void* dk, void* dv,
                           float* cvec, int causal, hipStream_t st);
hipError_t launch_ret_bwd_dq(const SegGeom& g, const void* q, const void* k, const void* v, const float* lg,
                             const void* dy, const float* carry_s, float* r_agg, void* dq, float* a, float* anch_s,
                             hipStream_t st);
hipError_t launch_ret_rscan(const SegGeom& g, float* r_agg, float* dS0, hipStream_t st);
hipError_t launch_ret_bwd_dkdv(const SegGeom& g, const void* q, const void* k, const void* v, const float* lg,
                               const void* dy, const float* r_agg, void* dk, void* dv, float* a, const float* anch_s,
                               float* anch_y, hipStream_t st);
hipError_t launch_ret_dlg(const SegGeom& g, const float* a, const float* carry_s, const float* r_agg,
                          const float* anch_y, float* dlg, hipStream_t st);
// raw_carry: `carry` holds the segments' own aggregates (no scan ran); each
// segment sums those before it
hipError_t launch_forward_f32mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                                  void* out, float* den_out, const float* carry, hipStream_t st, int raw_carry = 0);
hipError_t launch_seg_state_f32mfma(const SegGeom& g, const void* k, const void* v, float* s_out,
                                    int64_t s_stride, float* z_out, int64_t z_stride, hipStream_t st);
hipError_t launch_bwd_dq_mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                              const void* dout, const float* carry_s, void* dq, float* r_agg, float* c_out,
                              float* den_out, hipStream_t st);
int bwd_fused_supported(int causal, int D);
int64_t bwd_fused_resident(int dim);
hipError_t launch_bwd_fused_mfma(const SegGeom& g, const void* q, const void* k, const void* v, const void* dout,
                                 const float* carry_s, void* dq, void* dk, void* dv, float* r_agg, float* c_ws,
                                 float* den_ws, unsigned* flags, unsigned* err, unsigned want, long long spin_ticks,
                                 hipStream_t st);
// carry_raw: carry_r holds the raw suffix aggregates (summed in the kernel)
// rather than their reverse exclusive scan.
hipError_t launch_bwd_dkdv_mfma(int causal, const SegGeom& g, const void* q, const void* k, const void* v,
                                const void* dout, const float* den, const float* c, const float* carry_r,
                                void* dk, void* dv, hipStream_t st, int carry_raw = 0);
}  // namespace la

namespace {

thread_local std::string g_err;

la_status fail(la_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

la_status ok() {
  g_err.clear();
  return LA_OK;
}

la_status dev(hipError_t e, const char* where) {
  if (e == hipSuccess) return ok();
  return fail(LA_ERR_DEVICE, "%s: %s", where, hipGetErrorString(e));
}

constexpr int64_t kMaxFeat = 256;
constexpr int64_t kMaxState = 16384;  // D*M floats of state per head
constexpr int64_t kMaxElems = int64_t(1) << 40;
constexpr size_t kAlign = 256;

size_t dtype_size(int dtype) { return dtype == LA_BF16 ? 2 : 4; }

struct Span {
  const char* name;
  uintptr_t lo, hi;
};

Span span(const char* name, const void* p, int64_t elems, size_t esz) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{name, lo, lo + static_cast<uintptr_t>(elems) * esz};
}

bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

la_status check_sizes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype) {
  if (B < 1 || H < 1 || N < 1 || D < 1 || M < 1)
    return fail(LA_ERR_INVALID, "sizes must be >= 1 (B=%lld H=%lld N=%lld D=%lld M=%lld)", (long long)B,
                (long long)H, (long long)N, (long long)D, (long long)M);
  if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_INVALID, "unknown dtype %d", dtype);
  if (D > kMaxFeat || M > kMaxFeat || D * M > kMaxState)
    return fail(LA_ERR_UNSUPPORTED, "D=%lld, M=%lld: need D, M <= 256 and D*M <= 16384", (long long)D,
                (long long)M);
  if (B * H > kMaxElems || B * H * N > kMaxElems || B * H * N * std::max(D, M) > kMaxElems)
    return fail(LA_ERR_UNSUPPORTED, "problem too large (B*H*N*max(D,M) > 2^40)");
  return LA_OK;
}

la_status check_ptr(const void* p, const char* name, int dtype) {
  if (!p) return fail(LA_ERR_INVALID, "%s is NULL", name);
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  const size_t need = dtype_size(dtype);
  if (a % need) return fail(LA_ERR_INVALID, "%s is not %zu-byte aligned", name, need);
  return LA_OK;
}

// The MFMA kernels move q, k, v, out, dout, dq, dk, dv (and, in the families
// that have no generic kernels, every other per-token tensor) in 16-byte
// vectors through buffer loads and stores; a tensor that is only
// dtype-aligned goes to the generic kernels (element accesses) or, where
// there are none, is refused.
bool vec16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p && (reinterpret_cast<uintptr_t>(p) & 15)) return false;
  return true;
}

la_status need_vec16(std::initializer_list<const void*> ptrs, const char* what) {
  if (vec16(ptrs)) return LA_OK;
  return fail(LA_ERR_UNSUPPORTED, "%s: every tensor pointer must be 16-byte aligned (these kernels have no "
              "element-wise fallback)", what);
}

la_status check_disjoint(const Span* outs, int nout, const Span* ins, int nin) {
  for (int i = 0; i < nout; ++i) {
    if (!outs[i].lo) continue;
    for (int j = 0; j < nin; ++j)
      if (ins[j].lo && overlap(outs[i], ins[j]))
        return fail(LA_ERR_INVALID, "output %s overlaps input %s", outs[i].name, ins[j].name);
    for (int j = i + 1; j < nout; ++j)
      if (outs[j].lo && overlap(outs[i], outs[j]))
        return fail(LA_ERR_INVALID, "outputs %s and %s overlap", outs[i].name, outs[j].name);
  }
  return LA_OK;
}

// ---------------------------------------------------------------- plans ----
struct Plan {
  int kernel;    // LA_KERNEL_GENERIC or LA_KERNEL_MFMA
  int P;         // segments
  int seg_len;   // tokens per segment
  int chunk;     // chunk used by the forward-type kernels (informational)
  bool one_launch = false;  // the causal MFMA backward as one launch where it can
};

// vec_ok: every tensor pointer of the call is 16-byte aligned (the sizing
// queries, which see no pointers, assume so).  When it is not, the automatic
// plan keeps the segmentation the MFMA kernels would use -- so workspace and
// saved-state sizes stay what la_workspace_bytes / la_saved_bytes report --
// but runs the generic kernels; a plan that asks for the MFMA kernels is
// refused.
la_status resolve(int op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype,
                  const la_plan* req, Plan* out, bool vec_ok = true) {
  (void)causal;
  int kernel = req ? req->kernel : LA_KERNEL_AUTO;
  if (kernel < LA_KERNEL_AUTO || kernel > LA_KERNEL_MFMA_ONE_LAUNCH)
    return fail(LA_ERR_INVALID, "plan.kernel=%d", kernel);
  const bool one_launch = kernel == LA_KERNEL_MFMA_ONE_LAUNCH;
  if (one_launch) kernel = LA_KERNEL_MFMA;
  // the state-carrying and retention calls use the forward / backward plans
  const int op_in = op;
  if (op == LA_OP_FORWARD_STATE || op == LA_OP_RETENTION_FORWARD) op = LA_OP_FORWARD;
  if (op == LA_OP_RETENTION_BACKWARD) op = LA_OP_BACKWARD;
  if (op == LA_OP_BACKWARD_STATE) op = LA_OP_BACKWARD;
  // the MFMA kernels address one head's rows with 32-bit buffer offsets
  const int mfma_ok = la::mfma_supported(op, D, M, dtype) && N * std::max(D, M) * 2 < (int64_t(1) << 31);
  if (kernel == LA_KERNEL_MFMA && !mfma_ok)
    return fail(LA_ERR_UNSUPPORTED, "no MFMA kernel for op %d, N=%lld, D=%lld, M=%lld, dtype %d", op, (long long)N,
                (long long)D, (long long)M, dtype);
  if (kernel == LA_KERNEL_MFMA && !vec_ok)
    return fail(LA_ERR_UNSUPPORTED, "the MFMA kernels need 16-byte aligned tensor pointers");
  if (kernel == LA_KERNEL_AUTO) kernel = mfma_ok ? LA_KERNEL_MFMA : LA_KERNEL_GENERIC;
  // a misaligned call on the automatic plan: MFMA segmentation, generic kernels
  const bool demoted = kernel == LA_KERNEL_MFMA && !vec_ok;
  int chunk = req ? req->chunk : 0;
  // chunk 128 (bf16, D = M = 64): the forward runs 128-token chunks and every
  // segment is a whole number of them; the other kernels keep 64-token
  // chunks over the same segments, so records stay interchangeable between
  // calls with this plan
  if (chunk == 128 && !(kernel == LA_KERNEL_MFMA && dtype == LA_BF16 && D == 64 && M == 64))
    return fail(LA_ERR_INVALID, "plan.chunk=128 is the bf16 MFMA forward at D = M = 64 only");
  // The backward cuts its segments as the forward of the same call does, so
  // that the forward's saved records fit it: where the automatic plan runs
  // the MFMA forward but has no MFMA backward (fp32 at D = M = 64), the
  // generic backward runs over the MFMA forward's segments.
  bool mfma_seg = kernel == LA_KERNEL_MFMA;
  if (op == LA_OP_BACKWARD && kernel == LA_KERNEL_GENERIC && (!req || req->kernel == LA_KERNEL_AUTO))
    mfma_seg = la::mfma_supported(LA_OP_FORWARD, D, M, dtype) && N * std::max(D, M) * 2 < (int64_t(1) << 31);
  const int unit = mfma_seg ? (chunk == 128 ? 128 : 64) : 32;  // segment granularity
  if (demoted) {
    kernel = LA_KERNEL_GENERIC;
    chunk = 0;
  }
  if (kernel == LA_KERNEL_GENERIC) {
    if (chunk != 0 && chunk != 16 && chunk != 32)
      return fail(LA_ERR_INVALID, "plan.chunk=%d (generic kernels take 16 or 32)", chunk);
    const int tc = la::generic_chunk_for((int)D, (int)M, op == LA_OP_BACKWARD ? 3 : 0);
    if (tc == 0) return fail(LA_ERR_UNSUPPORTED, "D=%lld, M=%lld do not fit in LDS", (long long)D, (long long)M);
    if (chunk == 0 || chunk > tc) chunk = tc;
  } else {
    if (chunk != 0 && chunk != 64 && chunk != 128)
      return fail(LA_ERR_INVALID, "plan.chunk=%d (MFMA kernels take 64, or 128 for the D = 64 bf16 forward)", chunk);
    if (chunk == 0) chunk = 64;
  }
  const int64_t nunits = (N + unit - 1) / unit;
  const int64_t BH = B * H;
  int64_t P = req && req->segments > 0 ? req->segments : 0;
  if (req && req->segments < 0) return fail(LA_ERR_INVALID, "plan.segments=%d", req->segments);
  if (P == 0) {
    // Generic kernels: about 1024 independent workgroups (four per CU on the
    // 256 CUs of an MI355X) so that several segments' loads are in flight per
    // CU.  MFMA kernels: about 512, one full round of the backward kernels at
    // two workgroups per CU (measured best on the B=8, H=16, N=8192, D=64
    // step: 512 beats 1024, 768 and 2048).  Segments keep at least 4 units;
    // more segments only add scan work.
    const int64_t target = (kernel == LA_KERNEL_MFMA || mfma_seg) ? 512 : 1024;
    const int64_t want = (target + BH - 1) / BH;
    P = std::min<int64_t>(want, std::max<int64_t>(1, nunits / 4));
    // (the retention backward anchors its gate gradients every kRetAnchor
    // tokens inside a segment as well as at its end, so its segments need no
    // cap of their own)
  }
  P = std::max<int64_t>(1, std::min<int64_t>(P, nunits));
  const int64_t seg_units = (nunits + P - 1) / P;
  const int64_t seg_len = seg_units * unit;
  P = (N + seg_len - 1) / seg_len;
  if (BH * P > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  if (seg_len > 0x7fffffffLL) return fail(LA_ERR_UNSUPPORTED, "segment too long");
  out->kernel = kernel;
  out->one_launch = one_launch;
  out->P = static_cast<int>(P);
  out->seg_len = static_cast<int>(seg_len);
  out->chunk = chunk;
  return LA_OK;
}

// Workspace carving: regions of floats, each 256-byte aligned.
struct Carve {
  size_t off = 0;
  size_t take(size_t floats) {
    const size_t at = off;
    off += (floats * sizeof(float) + kAlign - 1) / kAlign * kAlign;
    return at;
  }
};

struct WsLayout {
  size_t aggS = 0, totS = 0, aggR = 0, totR = 0, den = 0, cvec = 0;
  size_t flags = 0;             // MFMA backward: one hand-off flag per segment
  size_t anchS = 0, anchY = 0;  // retention backward: states and <S, R> at the inner anchors
  size_t bytes = 0;
};

WsLayout layout(int op, int64_t BH, int64_t N, int64_t D, int64_t M, int causal, const Plan& p) {
  WsLayout w;
  Carve c;
  const size_t E = static_cast<size_t>(la::state_elems(static_cast<int>(D), static_cast<int>(M)));
  const size_t recs = static_cast<size_t>(BH) * p.P * E;
  if (op == LA_OP_FORWARD_STATE || op == LA_OP_RETENTION_FORWARD) {
    w.aggS = c.take(recs);
  } else if (op == LA_OP_FORWARD) {
    if (causal) {
      if (p.P > 1) w.aggS = c.take(recs);
    } else {
      w.aggS = c.take(recs);
      w.totS = c.take(static_cast<size_t>(BH) * E);
    }
  } else if (op == LA_OP_RETENTION_BACKWARD) {
    w.aggS = c.take(recs);
    w.aggR = c.take(recs);
    w.den = c.take(static_cast<size_t>(BH) * N);  // per-token q.dq - k.dk
    const size_t na = static_cast<size_t>(la::ret_anchors(p.seg_len));
    if (na) {
      w.anchS = c.take(static_cast<size_t>(BH) * p.P * na * D * M);
      w.anchY = c.take(static_cast<size_t>(BH) * p.P * na);
    }
  } else if (op == LA_OP_BACKWARD || op == LA_OP_BACKWARD_STATE) {
    w.aggS = c.take(recs);
    w.totS = c.take(static_cast<size_t>(BH) * E);
    w.aggR = c.take(recs);
    w.totR = c.take(static_cast<size_t>(BH) * E);
    w.den = c.take(static_cast<size_t>(BH) * N);
    w.cvec = c.take(static_cast<size_t>(BH) * N);
    if (p.kernel == LA_KERNEL_MFMA) w.flags = c.take(static_cast<size_t>(BH) * p.P);
  } else if (op == LA_OP_PREFIX_STATE) {
    if (p.P > 1) w.aggS = c.take(recs);
  }
  w.bytes = c.off;
  return w;
}

float* at(void* ws, size_t off) { return reinterpret_cast<float*>(static_cast<char*>(ws) + off); }

// Prefix states a forward leaves for its backward: the state entering each
// segment (causal; none with one segment) or the totals (non-causal).
size_t saved_floats(int64_t BH, int64_t D, int64_t M, int causal, const Plan& p) {
  const size_t E = static_cast<size_t>(la::state_elems(static_cast<int>(D), static_cast<int>(M)));
  if (causal) return p.P > 1 ? static_cast<size_t>(BH) * p.P * E : 0;
  return static_cast<size_t>(BH) * E;
}

}  // namespace


// ============================================================ tracing ====
// Optional per-kernel timing: while enabled, every launch is bracketed by a
// pair of HIP events recorded on the launch stream.
namespace {

struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};

std::mutex g_prof_mu;
bool g_prof_on = false;
std::string g_prof_only;  // comma-separated kernel names to time ("" = all)

bool prof_wanted(const char* name) {
  if (g_prof_only.empty()) return true;
  const std::string key = std::string(",") + name + ",";
  return (std::string(",") + g_prof_only + ",").find(key) != std::string::npos;
}
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_get() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <typename F>
hipError_t timed(const char* name, hipStream_t st, F&& f) {
  if (!g_prof_on || !prof_wanted(name)) return f();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    a = pool_get();
    b = pool_get();
  }
  if (!a || !b) return f();
  hipEventRecord(a, st);
  const hipError_t e = f();
  hipEventRecord(b, st);
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof.push_back({name, a, b});
  return e;
}

const char* kname(int kernel, const char* generic_name, const char* mfma_name) {
  return kernel == LA_KERNEL_MFMA ? mfma_name : generic_name;
}

}  // namespace

// ======================================================= static scratch ====
// For callers that cannot allocate (graph capture, tight serving loops):
// la_forward_noalloc keeps its segment records in this file-scope device
// array instead of a caller workspace.  Every GPU the library runs on holds
// its own copy until the process ends; its address on each device is taken
// once, with that device current, and kept.  In host code `scratch` names a
// host-side stand-in, never the device memory: only the kept address is
// passed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
void* g_err_addr[kMaxDevices] = {};

}  // namespace

// Set by a kernel whose bounded cross-workgroup wait ran out (the fused
// backward's hand-off); read and cleared by la_device_error.  As with
// `scratch`, host code uses only the address taken on each device.
static __device__ __align__(16) unsigned int dev_err_word[4];

namespace {

// The device `stream` runs on, which must be the calling thread's current one.
hipError_t stream_device(hipStream_t stream, int* out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (stream) {
    hipDevice_t sd = 0;
    if ((e = hipStreamGetDevice(stream, &sd)) != hipSuccess) return e;
    if (sd != cur) return hipErrorInvalidDevice;
  }
  if (cur < 0 || cur >= kMaxDevices) return hipErrorInvalidDevice;
  *out = cur;
  return hipSuccess;
}

// The scratch address on the device `stream` runs on.
hipError_t scratch_for_stream(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = stream_device(stream, &cur);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[cur]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[cur] = p;
  }
  *out = g_scratch_addr[cur];
  return hipSuccess;
}

// The device error word's address on the device `stream` runs on.
hipError_t err_word_for_stream(hipStream_t stream, unsigned** out) {
  int cur = 0;
  hipError_t e = stream_device(stream, &cur);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_err_addr[cur]) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(dev_err_word))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_err_addr[cur] = p;
  }
  *out = static_cast<unsigned*>(g_err_addr[cur]);
  return hipSuccess;
}

// Bound of a cross-workgroup wait in the device's real-time counter ticks
// (0.5 s; the counter rate is queried once per device).  LA_HANDOFF_TEST=1
// in the environment makes the fused backward wait for a flag value that is
// never published, with a 20 us bound, so that tests can exercise the
// timeout path (every workgroup still runs to its end).
long long handoff_ticks(int dev, bool test_mode) {
  static int rate_khz[kMaxDevices] = {};
  int r = rate_khz[dev];
  if (r <= 0) {
    if (hipDeviceGetAttribute(&r, hipDeviceAttributeWallClockRate, dev) != hipSuccess || r <= 0) r = 100000;
    rate_khz[dev] = r;
  }
  return test_mode ? static_cast<long long>(r) / 50 : static_cast<long long>(r) * 500;
}

bool handoff_test_mode() {
  const char* v = getenv("LA_HANDOFF_TEST");
  return v && v[0] == '1';
}

}  // namespace

// ============================================================ dispatch ====
namespace {

la::SegGeom geom(int64_t BH, int64_t N, int64_t D, int64_t M, const Plan& p, int chunk) {
  la::SegGeom g;
  g.BH = BH;
  g.N = N;
  g.D = static_cast<int>(D);
  g.M = static_cast<int>(M);
  g.P = p.P;
  g.seg_len = p.seg_len;
  g.chunk = chunk;
  return g;
}

// The geometry for a segment-state pass whose scan produces no total: the
// last segment's aggregate would only feed that total, so it is skipped.
// With one segment there is nothing left to sum: callers skip the pass (the
// scan then writes the initial state into the record).
la::SegGeom without_last(const la::SegGeom& g) {
  la::SegGeom r = g;
  if (g.P > 1) r.nseg = g.P - 1;
  return r;
}

// Segment aggregates of (S, Z) into ws records [BH][P][E].
hipError_t seg_state(int dtype, const Plan& p, const la::SegGeom& gbase, const void* k, const void* v,
                     float* recs, hipStream_t st) {
  const int64_t E = la::state_elems(gbase.D, gbase.M);
  float* z = recs + static_cast<int64_t>(gbase.D) * gbase.M;
  if (p.kernel == LA_KERNEL_MFMA)
    return timed("mfma.seg_state", st, [&] {
      return dtype == LA_F32 ? la::launch_seg_state_f32mfma(gbase, k, v, recs, E, z, E, st)
                             : la::launch_seg_state_mfma(gbase, k, v, recs, E, z, E, st);
    });
  la::SegGeom g = gbase;
  g.chunk = la::generic_chunk_for(g.D, g.M, 1);
  return timed("generic.seg_state", st,
               [&] { return la::launch_seg_state_generic(dtype, g, k, v, recs, E, z, E, st); });
}

hipError_t fwd_pass(int dtype, int causal, const Plan& p, const la::SegGeom& gbase, const void* q,
                    const void* k, const void* v, void* out, float* den_out, const float* carry,
                    hipStream_t st, int raw_carry = 0) {
  const bool t128 = p.kernel == LA_KERNEL_MFMA && gbase.chunk == 128;
  const char* name = t128 ? (out ? "mfma.forward_t128" : "mfma.forward_t128_den")
                     : out ? kname(p.kernel, "generic.forward", "mfma.forward")
                           : kname(p.kernel, "generic.forward_den", "mfma.forward_den");
  if (p.kernel == LA_KERNEL_MFMA)
    return timed(name, st, [&] {
      return dtype == LA_F32 ? la::launch_forward_f32mfma(causal, gbase, q, k, v, out, den_out, carry, st, raw_carry)
                             : la::launch_forward_mfma(causal, gbase, q, k, v, out, den_out, carry, st);
    });
  la::SegGeom g = gbase;
  g.chunk = std::min(p.chunk, la::generic_chunk_for(g.D, g.M, 0));
  return timed(name, st,
               [&] { return la::launch_forward_generic(dtype, causal, g, q, k, v, out, den_out, carry, st); });
}

hipError_t scan(float* agg, int64_t BH, int P, int D, int M, int reverse, float* tot_s, int64_t ts_stride,
                float* tot_z, int64_t tz_stride, hipStream_t st, const float* init_s = nullptr,
                const float* init_z = nullptr) {
  return timed("seg_scan", st, [&] {
    return la::launch_seg_scan(agg, BH, P, D, M, reverse, init_s, init_z, tot_s, ts_stride, tot_z, tz_stride, st);
  });
}

// State-carrying calls (la_forward_state / la_backward_state).
struct StateArgs {
  bool on = false;               // the call carries a state (causal only)
  const float* S0 = nullptr;     // [BH][D][M] state carried in, or null (zero)
  const float* Z0 = nullptr;     // [BH][D]
  float* S_out = nullptr;        // forward: state after the N tokens; backward: dL/dS0
  float* Z_out = nullptr;        // forward: Z after the N tokens; backward: dL/dZ0
};

la_status check_state(const StateArgs& st, int64_t BH, int64_t D, int64_t M, Span* spans) {
  if (!st.on) return LA_OK;
  if ((st.S0 == nullptr) != (st.Z0 == nullptr)) return fail(LA_ERR_INVALID, "S0 and Z0 must both be given or both be NULL");
  if ((st.S_out == nullptr) != (st.Z_out == nullptr))
    return fail(LA_ERR_INVALID, "the two state outputs must both be given or both be NULL");
  for (const void* p : {static_cast<const void*>(st.S0), static_cast<const void*>(st.Z0),
                        static_cast<const void*>(st.S_out), static_cast<const void*>(st.Z_out)})
    if (p && (reinterpret_cast<uintptr_t>(p) & 3)) return fail(LA_ERR_INVALID, "state pointers must be 4-byte aligned");
  spans[0] = span("S0", st.S0, st.S0 ? BH * D * M : 0, 4);
  spans[1] = span("Z0", st.Z0, st.Z0 ? BH * D : 0, 4);
  return LA_OK;
}

la_status do_forward(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H, int64_t N,
                     int64_t D, int64_t M, int causal, int dtype, float* den_out, float* saved,
                     size_t saved_bytes, void* workspace, size_t workspace_bytes, hipStream_t stream,
                     const la_plan* plan, const StateArgs& st = StateArgs(), bool static_scratch = false) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  causal = causal ? 1 : 0;
  if ((s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(out, "out", dtype)))
    return s;
  if (den_out && (reinterpret_cast<uintptr_t>(den_out) & 3)) return fail(LA_ERR_INVALID, "den_out misaligned");
  if (saved && (reinterpret_cast<uintptr_t>(saved) & 15)) return fail(LA_ERR_INVALID, "saved must be 16-byte aligned");
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  Plan p;
  if ((s = resolve(LA_OP_FORWARD, B, H, N, D, M, causal, dtype, plan, &p, vec16({q, k, v, out})))) return s;
  const size_t nsaved = saved_floats(BH, D, M, causal, p);
  if (saved && saved_bytes < nsaved * sizeof(float))
    return fail(LA_ERR_INVALID, "saved too small: %zu bytes given, %zu needed", saved_bytes, nsaved * sizeof(float));
  float* sv = nsaved ? saved : nullptr;
  Span sspan[2] = {span("S0", nullptr, 0, 4), span("Z0", nullptr, 0, 4)};
  if ((s = check_state(st, BH, D, M, sspan))) return s;
  // the state outputs may update S0, Z0 in place (exactly the same memory)
  const Span ins[] = {span("q", q, BH * N * D, es), span("k", k, BH * N * D, es), span("v", v, BH * N * M, es),
                      span("workspace", workspace, workspace ? (int64_t)workspace_bytes : 0, 1),
                      st.S_out == st.S0 ? span("S0", nullptr, 0, 4) : sspan[0],
                      st.Z_out == st.Z0 ? span("Z0", nullptr, 0, 4) : sspan[1]};
  const Span outs[] = {span("out", out, BH * N * M, es), span("den_out", den_out, den_out ? BH * N : 0, 4),
                       span("saved", sv, sv ? static_cast<int64_t>(nsaved) : 0, 4),
                       span("S_out", st.S_out, st.S_out ? BH * D * M : 0, 4),
                       span("Z_out", st.Z_out, st.Z_out ? BH * D : 0, 4)};
  if ((s = check_disjoint(outs, 5, ins, 6))) return s;
  if (st.S_out == st.S0 && st.S0 && (s = check_disjoint(&outs[0], 3, &sspan[0], 2))) return s;
  const WsLayout w = layout(st.on ? LA_OP_FORWARD_STATE : LA_OP_FORWARD, BH, N, D, M, causal, p);
  if (static_scratch) {
    // the library's static device scratch stands in for the workspace
    if (w.bytes > kScratchBytes)
      return fail(LA_ERR_UNSUPPORTED,
                  "this call needs %zu bytes of scratch; the static scratch holds %zu (call la_forward with a "
                  "workspace instead)", w.bytes, kScratchBytes);
    if (w.bytes) {
      hipError_t e0 = scratch_for_stream(stream, &workspace);
      if (e0 != hipSuccess) return dev(e0, "static scratch");
      workspace_bytes = kScratchBytes;
    }
  }
  if (workspace_bytes < w.bytes)
    return fail(LA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, w.bytes);
  if (w.bytes && !workspace) return fail(LA_ERR_INVALID, "workspace is NULL (%zu bytes needed)", w.bytes);
  if (w.bytes && (reinterpret_cast<uintptr_t>(workspace) & 15))
    return fail(LA_ERR_INVALID, "workspace must be 16-byte aligned");

  const la::SegGeom g = geom(BH, N, D, M, p, p.chunk);
  hipError_t e;
  if (st.on) {
    // every segment's carry-in (starting from S0, Z0) and the final state
    // come from the segment aggregates and their scan, as exact as fp32
    float* agg = sv ? sv : at(workspace, w.aggS);
    // (with one segment and no final state the scan only writes S0, Z0 into
    // the first record: there is no aggregate to compute)
    if ((st.S_out || p.P > 1) &&
        (e = seg_state(dtype, p, st.S_out ? g : without_last(g), k, v, agg, stream)))
      return dev(e, "segment state");
    if ((e = scan(agg, BH, p.P, g.D, g.M, 0, st.S_out, D * M, st.Z_out, D, stream, st.S0, st.Z0)))
      return dev(e, "segment scan");
    return dev(fwd_pass(dtype, 1, p, g, q, k, v, out, den_out, agg, stream), "forward");
  }
  if (causal) {
    const float* carry = nullptr;
    if (p.P > 1) {
      // (summing the carry from the raw aggregates inside the forward kernel,
      // as the dk/dv sweep does, measured slower here: the forward must also
      // write the prefix records for the backward, and that prologue cost
      // more than the scan launch)
      // the last segment's aggregate would only feed the total, which is not
      // asked for: the segment-state pass skips that segment, and the scan
      // reads its (unset) record only into the discarded total
      float* agg = sv ? sv : at(workspace, w.aggS);
      if ((e = seg_state(dtype, p, without_last(g), k, v, agg, stream))) return dev(e, "segment state");
      // The fp32 MFMA forward sums its carry from the raw aggregates itself
      // (in the scan's order: the same bits) when no prefix records are to be
      // kept and there are few segments: one launch fewer, which at this
      // kernel's sizes is worth more than the repeated record reads (segment
      // s reads s records, P (P - 1) / 2 per head in all).
      if (dtype == LA_F32 && p.kernel == LA_KERNEL_MFMA && !sv && p.P <= 8)
        return dev(fwd_pass(dtype, 1, p, g, q, k, v, out, den_out, agg, stream, 1), "forward");
      if ((e = scan(agg, BH, p.P, g.D, g.M, 0, nullptr, 0, nullptr, 0, stream)))
        return dev(e, "segment scan");
      carry = agg;
    }
    return dev(fwd_pass(dtype, 1, p, g, q, k, v, out, den_out, carry, stream), "forward");
  }
  float* agg = at(workspace, w.aggS);
  float* tot = sv ? sv : at(workspace, w.totS);
  const int64_t E = la::state_elems(g.D, g.M);
  if ((e = seg_state(dtype, p, g, k, v, agg, stream))) return dev(e, "segment state");
  if ((e = scan(agg, BH, p.P, g.D, g.M, 0, tot, E, tot + D * M, E, stream)))
    return dev(e, "segment scan");
  return dev(fwd_pass(dtype, 0, p, g, q, k, v, out, den_out, tot, stream), "forward");
}

la_status do_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                      const float* den, const float* saved, size_t saved_bytes, void* dq, void* dk, void* dv,
                      int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype,
                      void* workspace, size_t workspace_bytes, hipStream_t stream, const la_plan* plan,
                      const StateArgs& st = StateArgs()) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  causal = causal ? 1 : 0;
  if ((s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(out, "out", dtype)) || (s = check_ptr(dout, "dout", dtype)) ||
      (s = check_ptr(dq, "dq", dtype)) || (s = check_ptr(dk, "dk", dtype)) || (s = check_ptr(dv, "dv", dtype)))
    return s;
  if (den && (reinterpret_cast<uintptr_t>(den) & 3)) return fail(LA_ERR_INVALID, "den misaligned");
  if (saved && (reinterpret_cast<uintptr_t>(saved) & 15)) return fail(LA_ERR_INVALID, "saved must be 16-byte aligned");
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  Plan p;
  if ((s = resolve(LA_OP_BACKWARD, B, H, N, D, M, causal, dtype, plan, &p,
                   vec16({q, k, v, out, dout, dq, dk, dv}))))
    return s;
  const size_t nsaved = saved_floats(BH, D, M, causal, p);
  if (saved) {
    // the saved states are per segment of the forward's plan
    Plan pf;
    if ((s = resolve(LA_OP_FORWARD, B, H, N, D, M, causal, dtype, plan, &pf))) return s;
    if (pf.P != p.P || pf.seg_len != p.seg_len)
      return fail(LA_ERR_INVALID, "saved states are cut into %d segments of %d tokens, the backward into %d of %d",
                  pf.P, pf.seg_len, p.P, p.seg_len);
    if (saved_bytes < nsaved * sizeof(float))
      return fail(LA_ERR_INVALID, "saved too small: %zu bytes given, %zu needed", saved_bytes,
                  nsaved * sizeof(float));
  }
  const float* sv = nsaved ? saved : nullptr;
  Span sspan[2] = {span("S0", nullptr, 0, 4), span("Z0", nullptr, 0, 4)};
  if ((s = check_state(st, BH, D, M, sspan))) return s;
  const Span ins[] = {span("q", q, BH * N * D, es),       span("k", k, BH * N * D, es),
                      span("v", v, BH * N * M, es),       span("out", out, BH * N * M, es),
                      span("dout", dout, BH * N * M, es), span("den", den, den ? BH * N : 0, 4),
                      span("saved", sv, sv ? static_cast<int64_t>(nsaved) : 0, 4),
                      span("workspace", workspace, workspace ? (int64_t)workspace_bytes : 0, 1),
                      sspan[0], sspan[1]};
  const Span outs[] = {span("dq", dq, BH * N * D, es), span("dk", dk, BH * N * D, es),
                       span("dv", dv, BH * N * M, es), span("dS0", st.S_out, st.S_out ? BH * D * M : 0, 4),
                       span("dZ0", st.Z_out, st.Z_out ? BH * D : 0, 4)};
  if ((s = check_disjoint(outs, 5, ins, 10))) return s;
  const WsLayout w = layout(st.on ? LA_OP_BACKWARD_STATE : LA_OP_BACKWARD, BH, N, D, M, causal, p);
  if (workspace_bytes < w.bytes)
    return fail(LA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, w.bytes);
  if (!workspace) return fail(LA_ERR_INVALID, "workspace is NULL (%zu bytes needed)", w.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return fail(LA_ERR_INVALID, "workspace must be 16-byte aligned");

  const la::SegGeom g = geom(BH, N, D, M, p, p.chunk);
  const int64_t E = la::state_elems(g.D, g.M);
  float* aggS = at(workspace, w.aggS);
  float* totS = at(workspace, w.totS);
  float* aggR = at(workspace, w.aggR);
  float* totR = at(workspace, w.totR);
  hipError_t e;
  const float* carry_s = nullptr;
  if (st.on) {
    // carry-in from S0, Z0 through the segment scan (any number of segments;
    // with one, the scan only writes S0, Z0 into its record)
    if (p.P > 1 && (e = seg_state(dtype, p, without_last(g), k, v, aggS, stream))) return dev(e, "segment state");
    if ((e = scan(aggS, BH, p.P, g.D, g.M, 0, nullptr, 0, nullptr, 0, stream, st.S0, st.Z0)))
      return dev(e, "segment scan");
    carry_s = aggS;
  } else if (saved) {
    carry_s = sv;  // the forward's scanned states (null: one causal segment)
  } else if (causal) {
    if (p.P > 1) {
      if ((e = seg_state(dtype, p, without_last(g), k, v, aggS, stream))) return dev(e, "segment state");
      if ((e = scan(aggS, BH, p.P, g.D, g.M, 0, nullptr, 0, nullptr, 0, stream)))
        return dev(e, "segment scan");
      carry_s = aggS;
    }
  } else {
    if ((e = seg_state(dtype, p, g, k, v, aggS, stream))) return dev(e, "segment state");
    if ((e = scan(aggS, BH, p.P, g.D, g.M, 0, totS, E, totS + D * M, E, stream)))
      return dev(e, "segment scan");
    carry_s = totS;
  }
  // the suffix aggregates are needed across segments, and for dL/dS0, dL/dZ0
  // (their totals) in a state-carrying call
  float* r_agg = (causal && p.P == 1 && !st.S_out) ? nullptr : aggR;
  // Both kernel families recompute num and den in fp32 inside the forward
  // sweep (neither reads out or den) and pass den and c to the reverse sweep
  // through the workspace.
  float* cw = at(workspace, w.cvec);
  float* dw = at(workspace, w.den);
  if (p.kernel == LA_KERNEL_MFMA && p.one_launch && causal && !st.on && dtype == LA_BF16 &&
      la::bwd_fused_supported(causal, D)) {
    // one launch: the forward sweep, the hand-off of the suffix aggregates
    // and the reverse sweep (bit for bit the two-launch result), when every
    // workgroup of the grid can be resident at once.  Not the default: on
    // the B=8 H=16 N=8192 D=64 step it measured 0.33-0.36 ms against
    // 0.30 ms for the two launches (the agent-scope fences of the hand-off
    // cost more than the reverse sweep saves by re-reading from the cache).
    const int64_t resident = la::bwd_fused_resident(static_cast<int>(D));
    if (resident >= BH * p.P) {
      int devno = 0;
      unsigned* errw = nullptr;
      if ((e = stream_device(stream, &devno)) || (e = err_word_for_stream(stream, &errw)))
        return dev(e, "backward hand-off set-up");
      const bool test = handoff_test_mode();
      return dev(timed("mfma.bwd_fused", stream,
                       [&] {
                         return la::launch_bwd_fused_mfma(g, q, k, v, dout, carry_s, dq, dk, dv, aggR, cw, dw,
                                                          reinterpret_cast<unsigned*>(at(workspace, w.flags)), errw,
                                                          test ? 2u : 1u, handoff_ticks(devno, test), stream);
                       }),
                 "backward (one launch)");
    }
  }
  if (p.kernel == LA_KERNEL_MFMA) {
    e = timed("mfma.bwd_dq", stream,
              [&] { return la::launch_bwd_dq_mfma(causal, g, q, k, v, dout, carry_s, dq, r_agg, cw, dw, stream); });
  } else {
    la::SegGeom gd = g;
    gd.chunk = std::min(p.chunk, la::generic_chunk_for(g.D, g.M, 2));
    e = timed("generic.bwd_dq", stream, [&] {
      return la::launch_bwd_dq_generic(dtype, causal, gd, q, k, v, dout, carry_s, dq, r_agg, cw, dw, stream);
    });
  }
  if (e) return dev(e, "backward dq");
  const float* carry_r = nullptr;
  int carry_raw = 0;
  if (causal) {
    if (p.kernel == LA_KERNEL_MFMA && p.P > 1 && !st.S_out) {
      // the MFMA dk/dv sweep sums its suffix carry from the raw aggregates
      carry_r = aggR;
      carry_raw = 1;
    } else if (p.P > 1 || st.S_out) {
      if ((e = scan(aggR, BH, p.P, g.D, g.M, 1, st.S_out, D * M, st.Z_out, D, stream)))
        return dev(e, "suffix scan");
      if (p.P > 1) carry_r = aggR;
    }
  } else {
    if ((e = scan(aggR, BH, p.P, g.D, g.M, 1, totR, E, totR + D * M, E, stream)))
      return dev(e, "suffix scan");
    carry_r = totR;
  }
  if (p.kernel == LA_KERNEL_MFMA) {
    e = timed("mfma.bwd_dkdv", stream,
              [&] {
                return la::launch_bwd_dkdv_mfma(causal, g, q, k, v, dout, dw, cw, carry_r, dk, dv, stream,
                                                carry_raw);
              });
  } else {
    la::SegGeom gk = g;
    gk.chunk = std::min(p.chunk, la::generic_chunk_for(g.D, g.M, 3));
    e = timed("generic.bwd_dkdv", stream, [&] {
      return la::launch_bwd_dkdv_generic(dtype, causal, gk, q, k, v, dout, dw, cw, carry_r, dk, dv, stream);
    });
  }
  return dev(e, "backward dk/dv");
}

}  // namespace

// ================================================================ ABI ====
LA_API la_status la_forward(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                            int64_t N, int64_t D, int64_t M, int causal, int dtype, float* den_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return do_forward(q, k, v, out, B, H, N, D, M, causal, dtype, den_out, nullptr, 0, workspace, workspace_bytes,
                    stream, nullptr);
}

LA_API la_status la_forward_ex(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                               int64_t N, int64_t D, int64_t M, int causal, int dtype, float* den_out,
                               float* saved, size_t saved_bytes, void* workspace, size_t workspace_bytes,
                               hipStream_t stream, const la_plan* plan) {
  return do_forward(q, k, v, out, B, H, N, D, M, causal, dtype, den_out, saved, saved_bytes, workspace,
                    workspace_bytes, stream, plan);
}

LA_API la_status la_forward_noalloc(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                                    int64_t N, int64_t D, int64_t M, int causal, int dtype, float* den_out,
                                    hipStream_t stream) {
  return do_forward(q, k, v, out, B, H, N, D, M, causal, dtype, den_out, nullptr, 0, nullptr, 0, stream, nullptr,
                    StateArgs(), true);
}

LA_API la_status la_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* den, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                             int64_t D, int64_t M, int causal, int dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  return do_backward(q, k, v, out, dout, den, nullptr, 0, dq, dk, dv, B, H, N, D, M, causal, dtype, workspace,
                     workspace_bytes, stream, nullptr);
}

LA_API la_status la_backward_ex(const void* q, const void* k, const void* v, const void* out,
                                const void* dout, const float* den, const float* saved, size_t saved_bytes,
                                void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N, int64_t D,
                                int64_t M, int causal, int dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream, const la_plan* plan) {
  return do_backward(q, k, v, out, dout, den, saved, saved_bytes, dq, dk, dv, B, H, N, D, M, causal, dtype,
                     workspace, workspace_bytes, stream, plan);
}

LA_API la_status la_forward_state(const void* q, const void* k, const void* v, void* out, int64_t B, int64_t H,
                                  int64_t N, int64_t D, int64_t M, int dtype, const float* S0, const float* Z0,
                                  float* S_out, float* Z_out, float* den_out, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  StateArgs st;
  st.on = true;
  st.S0 = S0;
  st.Z0 = Z0;
  st.S_out = S_out;
  st.Z_out = Z_out;
  return do_forward(q, k, v, out, B, H, N, D, M, 1, dtype, den_out, nullptr, 0, workspace, workspace_bytes, stream,
                    nullptr, st);
}

LA_API la_status la_backward_state(const void* q, const void* k, const void* v, const void* out,
                                   const void* dout, const float* den, const float* S0, const float* Z0, void* dq,
                                   void* dk, void* dv, float* dS0, float* dZ0, int64_t B, int64_t H, int64_t N,
                                   int64_t D, int64_t M, int dtype, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  StateArgs st;
  st.on = true;
  st.S0 = S0;
  st.Z0 = Z0;
  st.S_out = dS0;
  st.Z_out = dZ0;
  return do_backward(q, k, v, out, dout, den, nullptr, 0, dq, dk, dv, B, H, N, D, M, 1, dtype, workspace,
                     workspace_bytes, stream, nullptr, st);
}

LA_API size_t la_retention_saved_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype) {
  if (check_sizes(B, H, N, D, M, dtype) != LA_OK || !la::retention_supported(D, M, dtype)) return 0;
  Plan p;
  if (resolve(LA_OP_RETENTION_FORWARD, B, H, N, D, M, 1, dtype, nullptr, &p) != LA_OK) return 0;
  return static_cast<size_t>(B * H) * p.P * la::state_elems(static_cast<int>(D), static_cast<int>(M)) * sizeof(float);
}

LA_API la_status la_retention_forward(const void* q, const void* k, const void* v, const float* log_gamma,
                                      void* y, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int dtype,
                                      const float* S0, float* S_out, float* saved, size_t saved_bytes,
                                      void* workspace, size_t workspace_bytes, hipStream_t stream) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(y, "y", dtype)) || (s = check_ptr(log_gamma, "log_gamma", LA_F32)))
    return s;
  for (const void* p : {static_cast<const void*>(S0), static_cast<const void*>(S_out)})
    if (p && (reinterpret_cast<uintptr_t>(p) & 3)) return fail(LA_ERR_INVALID, "state pointers must be 4-byte aligned");
  if (!la::retention_supported(D, M, dtype))
    return fail(LA_ERR_UNSUPPORTED, "retention kernels take bf16 with D = M in {64, 128} (D=%lld, M=%lld, dtype %d)",
                (long long)D, (long long)M, dtype);
  if ((s = need_vec16({q, k, v, y, log_gamma}, "retention forward"))) return s;
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  Plan p;
  if ((s = resolve(LA_OP_RETENTION_FORWARD, B, H, N, D, M, 1, dtype, nullptr, &p))) return s;
  if (p.kernel != LA_KERNEL_MFMA) return fail(LA_ERR_UNSUPPORTED, "sequence too long for the retention kernels");
  const size_t nsaved = static_cast<size_t>(BH) * p.P * la::state_elems(static_cast<int>(D), static_cast<int>(M));
  if (saved && saved_bytes < nsaved * sizeof(float))
    return fail(LA_ERR_INVALID, "saved too small: %zu bytes given, %zu needed", saved_bytes, nsaved * sizeof(float));
  if (saved && (reinterpret_cast<uintptr_t>(saved) & 15)) return fail(LA_ERR_INVALID, "saved must be 16-byte aligned");
  const Span ins[] = {span("q", q, BH * N * D, es), span("k", k, BH * N * D, es), span("v", v, BH * N * M, es),
                      span("log_gamma", log_gamma, BH * N, 4),
                      span("workspace", workspace, workspace ? (int64_t)workspace_bytes : 0, 1),
                      S_out == S0 ? span("S0", nullptr, 0, 4) : span("S0", S0, S0 ? BH * D * M : 0, 4)};
  const Span outs[] = {span("y", y, BH * N * M, es), span("S_out", S_out, S_out ? BH * D * M : 0, 4),
                       span("saved", saved, saved ? static_cast<int64_t>(nsaved) : 0, 4)};
  if ((s = check_disjoint(outs, 3, ins, 6))) return s;
  if (S_out && S_out == S0) {
    const Span s0[] = {span("S0", S0, BH * D * M, 4)};
    if ((s = check_disjoint(outs, 1, s0, 1))) return s;
  }
  const WsLayout w = layout(LA_OP_RETENTION_FORWARD, BH, N, D, M, 1, p);
  if (workspace_bytes < w.bytes)
    return fail(LA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, w.bytes);
  if (!workspace) return fail(LA_ERR_INVALID, "workspace is NULL (%zu bytes needed)", w.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return fail(LA_ERR_INVALID, "workspace must be 16-byte aligned");
  const la::SegGeom g = geom(BH, N, D, M, p, p.chunk);
  const float* carry = nullptr;
  hipError_t e;
  if (p.P > 1 || S0 || S_out || saved) {
    // segment aggregates and their decayed scan from S0; the total is the
    // state after the N tokens; kept in `saved` when given
    float* recs = saved ? saved : at(workspace, w.aggS);
    // without S_out the last segment's aggregate would only feed the total
    const la::SegGeom gs = S_out ? g : without_last(g);
    // (with one segment and no S_out the scan only writes S0 into the record)
    if ((S_out || p.P > 1) &&
        (e = timed("ret.seg_state", stream, [&] { return la::launch_ret_seg_state(gs, k, v, log_gamma, recs, stream); })))
      return dev(e, "retention segment state");
    if ((e = timed("ret.scan", stream, [&] { return la::launch_ret_scan(recs, BH, p.P, g.D, g.M, S0, S_out, stream); })))
      return dev(e, "retention scan");
    carry = recs;
  }
  return dev(timed("ret.forward", stream,
                   [&] { return la::launch_ret_forward(g, q, k, v, log_gamma, y, carry, stream); }),
             "retention forward");
}

LA_API la_status la_retention_backward(const void* q, const void* k, const void* v, const float* log_gamma,
                                       const void* dy, const float* S0, const float* saved, size_t saved_bytes,
                                       void* dq, void* dk, void* dv, float* dlog_gamma, float* dS0, int64_t B,
                                       int64_t H, int64_t N, int64_t D, int64_t M, int dtype, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(dy, "dy", dtype)) || (s = check_ptr(log_gamma, "log_gamma", LA_F32)) ||
      (s = check_ptr(dq, "dq", dtype)) || (s = check_ptr(dk, "dk", dtype)) || (s = check_ptr(dv, "dv", dtype)) ||
      (s = check_ptr(dlog_gamma, "dlog_gamma", LA_F32)))
    return s;
  for (const void* p : {static_cast<const void*>(S0), static_cast<const void*>(dS0)})
    if (p && (reinterpret_cast<uintptr_t>(p) & 3)) return fail(LA_ERR_INVALID, "state pointers must be 4-byte aligned");
  if (!la::retention_supported(D, M, dtype))
    return fail(LA_ERR_UNSUPPORTED, "retention kernels take bf16 with D = M in {64, 128} (D=%lld, M=%lld, dtype %d)",
                (long long)D, (long long)M, dtype);
  if ((s = need_vec16({q, k, v, dy, log_gamma, dq, dk, dv}, "retention backward"))) return s;
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  Plan p;
  if ((s = resolve(LA_OP_RETENTION_BACKWARD, B, H, N, D, M, 1, dtype, nullptr, &p))) return s;
  if (p.kernel != LA_KERNEL_MFMA) return fail(LA_ERR_UNSUPPORTED, "sequence too long for the retention kernels");
  const size_t nsaved = static_cast<size_t>(BH) * p.P * la::state_elems(static_cast<int>(D), static_cast<int>(M));
  if (saved && saved_bytes < nsaved * sizeof(float))
    return fail(LA_ERR_INVALID, "saved too small: %zu bytes given, %zu needed", saved_bytes, nsaved * sizeof(float));
  if (saved && (reinterpret_cast<uintptr_t>(saved) & 15)) return fail(LA_ERR_INVALID, "saved must be 16-byte aligned");
  const Span ins[] = {span("q", q, BH * N * D, es), span("k", k, BH * N * D, es), span("v", v, BH * N * M, es),
                      span("log_gamma", log_gamma, BH * N, 4), span("dy", dy, BH * N * M, es),
                      span("S0", S0, S0 ? BH * D * M : 0, 4),
                      span("workspace", workspace, workspace ? (int64_t)workspace_bytes : 0, 1),
                      span("saved", saved, saved ? static_cast<int64_t>(nsaved) : 0, 4)};
  const Span outs[] = {span("dq", dq, BH * N * D, es), span("dk", dk, BH * N * D, es), span("dv", dv, BH * N * M, es),
                       span("dlog_gamma", dlog_gamma, BH * N, 4), span("dS0", dS0, dS0 ? BH * D * M : 0, 4)};
  if ((s = check_disjoint(outs, 5, ins, 8))) return s;
  const WsLayout w = layout(LA_OP_RETENTION_BACKWARD, BH, N, D, M, 1, p);
  if (workspace_bytes < w.bytes)
    return fail(LA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, w.bytes);
  if (!workspace) return fail(LA_ERR_INVALID, "workspace is NULL (%zu bytes needed)", w.bytes);
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return fail(LA_ERR_INVALID, "workspace must be 16-byte aligned");
  const la::SegGeom g = geom(BH, N, D, M, p, p.chunk);
  float* rrec = at(workspace, w.aggR);
  float* a = at(workspace, w.den);
  float* anch_s = w.anchS ? at(workspace, w.anchS) : nullptr;
  float* anch_y = w.anchY ? at(workspace, w.anchY) : nullptr;
  hipError_t e;
  // the states entering each segment: the forward's, or recomputed from S0
  const float* recs = saved;
  if (!saved) {
    float* r = at(workspace, w.aggS);
    const la::SegGeom gs = without_last(g);  // the scan below keeps no total
    if (p.P > 1 &&
        (e = timed("ret.seg_state", stream, [&] { return la::launch_ret_seg_state(gs, k, v, log_gamma, r, stream); })))
      return dev(e, "retention segment state");
    if ((e = timed("ret.scan", stream, [&] { return la::launch_ret_scan(r, BH, p.P, g.D, g.M, S0, nullptr, stream); })))
      return dev(e, "retention scan");
    recs = r;
  }
  // forward sweep (dq, p, suffix aggregates), reverse scan of the
  // aggregates (total = dS0), reverse sweep (dk, dv, a), gate gradients
  if ((e = timed("ret.bwd_dq", stream, [&] {
         return la::launch_ret_bwd_dq(g, q, k, v, log_gamma, dy, recs, rrec, dq, a, anch_s, stream);
       })))
    return dev(e, "retention backward (dq)");
  if ((e = timed("ret.rscan", stream, [&] { return la::launch_ret_rscan(g, rrec, dS0, stream); })))
    return dev(e, "retention backward (suffix scan)");
  if ((e = timed("ret.bwd_dkdv", stream, [&] {
         return la::launch_ret_bwd_dkdv(g, q, k, v, log_gamma, dy, rrec, dk, dv, a, anch_s, anch_y, stream);
       })))
    return dev(e, "retention backward (dk, dv)");
  return dev(timed("ret.dlg", stream,
                   [&] { return la::launch_ret_dlg(g, a, recs, rrec, anch_y, dlog_gamma, stream); }),
             "retention backward (d log gamma)");
}

LA_API la_status la_poly_forward(const void* q, const void* k, const void* v, void* out, float* den_out, int64_t B,
                                 int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype,
                                 hipStream_t stream) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(out, "out", dtype)))
    return s;
  if (den_out && (reinterpret_cast<uintptr_t>(den_out) & 3)) return fail(LA_ERR_INVALID, "den_out misaligned");
  if (!la::poly_supported(D, M, dtype))
    return fail(LA_ERR_UNSUPPORTED, "polynomial kernels take bf16 with D = M in {64, 128} (D=%lld, M=%lld, dtype %d)",
                (long long)D, (long long)M, dtype);
  if ((s = need_vec16({q, k, v, out}, "polynomial forward"))) return s;
  if (N * D * 2 >= (int64_t(1) << 31)) return fail(LA_ERR_UNSUPPORTED, "head too large for 32-bit offsets");
  const int64_t BH = B * H;
  if (BH * ((N + 127) / 128) > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("q", q, BH * N * D, es), span("k", k, BH * N * D, es), span("v", v, BH * N * M, es)};
  const Span outs[] = {span("out", out, BH * N * M, es), span("den_out", den_out, den_out ? BH * N : 0, 4)};
  if ((s = check_disjoint(outs, 2, ins, 3))) return s;
  return dev(timed("poly.forward", stream,
                   [&] { return la::launch_poly_forward(BH, N, (int)D, q, k, v, out, den_out, causal ? 1 : 0, stream); }),
             "polynomial forward");
}

LA_API la_status la_poly_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                  const float* den, void* dq, void* dk, void* dv, int64_t B, int64_t H, int64_t N,
                                  int64_t D, int64_t M, int causal, int dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(out, "out", dtype)) || (s = check_ptr(dout, "dout", dtype)) ||
      (s = check_ptr(den, "den", LA_F32)) || (s = check_ptr(dq, "dq", dtype)) || (s = check_ptr(dk, "dk", dtype)) ||
      (s = check_ptr(dv, "dv", dtype)))
    return s;
  if (!la::poly_supported(D, M, dtype))
    return fail(LA_ERR_UNSUPPORTED, "polynomial kernels take bf16 with D = M in {64, 128} (D=%lld, M=%lld, dtype %d)",
                (long long)D, (long long)M, dtype);
  if ((s = need_vec16({q, k, v, out, dout, den, dq, dk, dv}, "polynomial backward"))) return s;
  if (N * D * 2 >= (int64_t(1) << 31)) return fail(LA_ERR_UNSUPPORTED, "head too large for 32-bit offsets");
  const int64_t BH = B * H;
  if (BH * ((N + 63) / 64) > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  const size_t need = la_workspace_bytes(LA_OP_POLY_BACKWARD, B, H, N, D, M, causal, dtype);
  if (workspace_bytes < need)
    return fail(LA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);
  if (!workspace) return fail(LA_ERR_INVALID, "workspace is NULL (%zu bytes needed)", need);
  if (reinterpret_cast<uintptr_t>(workspace) & 15) return fail(LA_ERR_INVALID, "workspace must be 16-byte aligned");
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("q", q, BH * N * D, es), span("k", k, BH * N * D, es), span("v", v, BH * N * M, es),
                      span("out", out, BH * N * M, es), span("dout", dout, BH * N * M, es), span("den", den, BH * N, 4),
                      span("workspace", workspace, (int64_t)workspace_bytes, 1)};
  const Span outs[] = {span("dq", dq, BH * N * D, es), span("dk", dk, BH * N * D, es), span("dv", dv, BH * N * M, es)};
  if ((s = check_disjoint(outs, 3, ins, 7))) return s;
  float* cvec = static_cast<float*>(workspace);
  hipError_t e;
  if ((e = timed("poly.bwd_dq", stream, [&] {
         return la::launch_poly_bwd(0, BH, N, (int)D, q, k, v, out, dout, den, dq, dk, dv, cvec, causal ? 1 : 0,
                                    stream);
       })))
    return dev(e, "polynomial backward (dq)");
  return dev(timed("poly.bwd_dkdv", stream,
                   [&] {
                     return la::launch_poly_bwd(1, BH, N, (int)D, q, k, v, out, dout, den, dq, dk, dv, cvec,
                                                causal ? 1 : 0, stream);
                   }),
             "polynomial backward (dk, dv)");
}

LA_API la_status la_poly_prefix_state(const void* k, const void* v, float* S, float* Z, int64_t B, int64_t H,
                                      int64_t N, int64_t D, int64_t M, int dtype, hipStream_t stream) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) || (s = check_ptr(S, "S", LA_F32)) ||
      (s = check_ptr(Z, "Z", LA_F32)))
    return s;
  if (!la::poly_supported(D, M, dtype))
    return fail(LA_ERR_UNSUPPORTED, "polynomial kernels take bf16 with D = M in {64, 128} (D=%lld, M=%lld, dtype %d)",
                (long long)D, (long long)M, dtype);
  if ((s = need_vec16({k, v}, "polynomial prefix state"))) return s;
  if (N * D * 2 >= (int64_t(1) << 31)) return fail(LA_ERR_UNSUPPORTED, "head too large for 32-bit offsets");
  const int64_t BH = B * H;
  if (BH * D * (D / 64) > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("k", k, BH * N * D, es), span("v", v, BH * N * M, es)};
  const Span outs[] = {span("S", S, BH * D * D * M, 4), span("Z", Z, BH * D * D, 4)};
  if ((s = check_disjoint(outs, 2, ins, 2))) return s;
  return dev(timed("poly.state", stream, [&] { return la::launch_poly_state(BH, N, (int)D, k, v, S, Z, stream); }),
             "polynomial prefix state");
}

LA_API la_status la_poly_decode_step(float* S, float* Z, const void* q, const void* k, const void* v, void* out,
                                     int64_t B, int64_t H, int64_t D, int64_t M, int dtype, hipStream_t stream) {
  la_status s = check_sizes(B, H, 1, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(S, "S", LA_F32)) || (s = check_ptr(Z, "Z", LA_F32)) || (s = check_ptr(q, "q", dtype)) ||
      (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) || (s = check_ptr(out, "out", dtype)))
    return s;
  if (D > 128 || (D & (D - 1)))
    return fail(LA_ERR_UNSUPPORTED, "polynomial decode takes D a power of two <= 128 (D=%lld)", (long long)D);
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("q", q, BH * D, es), span("k", k, BH * D, es), span("v", v, BH * M, es)};
  const Span outs[] = {span("S", S, BH * D * D * M, 4), span("Z", Z, BH * D * D, 4), span("out", out, BH * M, es)};
  if ((s = check_disjoint(outs, 3, ins, 3))) return s;
  if (BH > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  return dev(timed("poly.decode", stream,
                   [&] { return la::launch_poly_decode_step(dtype, BH, (int)D, (int)M, S, Z, q, k, v, out, stream); }),
             "polynomial decode step");
}

LA_API la_status la_softmax_forward(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                                    int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype,
                                    hipStream_t stream) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(out, "out", dtype)))
    return s;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3)) return fail(LA_ERR_INVALID, "lse misaligned");
  if (!la::softmax_supported(D, M, dtype))
    return fail(LA_ERR_UNSUPPORTED, "softmax kernels take bf16 with D = M in {64, 128} (D=%lld, M=%lld, dtype %d)",
                (long long)D, (long long)M, dtype);
  if ((s = need_vec16({q, k, v, out}, "softmax forward"))) return s;
  if (N * D * 2 >= (int64_t(1) << 31)) return fail(LA_ERR_UNSUPPORTED, "head too large for 32-bit offsets");
  const int64_t BH = B * H;
  if (BH * ((N + 127) / 128) > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("q", q, BH * N * D, es), span("k", k, BH * N * D, es), span("v", v, BH * N * M, es)};
  const Span outs[] = {span("out", out, BH * N * M, es), span("lse", lse, lse ? BH * N : 0, 4)};
  if ((s = check_disjoint(outs, 2, ins, 3))) return s;
  return dev(timed("softmax.forward", stream,
                   [&] { return la::launch_softmax_forward(BH, N, (int)D, q, k, v, out, lse, causal ? 1 : 0, stream); }),
             "softmax forward");
}

LA_API la_status la_softmax_decode_step(void* k_cache, void* v_cache, const void* q, const void* k, const void* v,
                                        void* out, int64_t B, int64_t H, int64_t L, int64_t capacity, int64_t D,
                                        int64_t M, int dtype, hipStream_t stream) {
  la_status s = check_sizes(B, H, 1, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(k_cache, "k_cache", dtype)) || (s = check_ptr(v_cache, "v_cache", dtype)) ||
      (s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) ||
      (s = check_ptr(out, "out", dtype)))
    return s;
  if (D != M || (D != 64 && D != 128))
    return fail(LA_ERR_UNSUPPORTED, "the KV-cache step takes D = M in {64, 128} (D=%lld, M=%lld)", (long long)D,
                (long long)M);
  if (L < 0 || L >= capacity)
    return fail(LA_ERR_INVALID, "cache length %lld must be in [0, capacity %lld)", (long long)L, (long long)capacity);
  for (const void* p : {k_cache, v_cache})
    if (reinterpret_cast<uintptr_t>(p) & 15) return fail(LA_ERR_INVALID, "caches must be 16-byte aligned");
  const int64_t BH = B * H;
  if (BH > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("q", q, BH * D, es), span("k", k, BH * D, es), span("v", v, BH * M, es)};
  const Span outs[] = {span("k_cache", k_cache, BH * capacity * D, es), span("v_cache", v_cache, BH * capacity * M, es),
                       span("out", out, BH * M, es)};
  if ((s = check_disjoint(outs, 3, ins, 3))) return s;
  return dev(timed("softmax.decode", stream,
                   [&] {
                     return la::launch_softmax_decode(dtype, BH, (int)D, k_cache, v_cache, q, k, v, out, L, capacity,
                                                      stream);
                   }),
             "softmax KV-cache decode step");
}

LA_API la_status la_decode_step(float* S, float* Z, const void* q, const void* k, const void* v, void* out,
                                int64_t B, int64_t H, int64_t D, int64_t M, int dtype, hipStream_t stream) {
  la_status s = check_sizes(B, H, 1, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(S, "S", LA_F32)) || (s = check_ptr(Z, "Z", LA_F32)) || (s = check_ptr(q, "q", dtype)) ||
      (s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) || (s = check_ptr(out, "out", dtype)))
    return s;
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("q", q, BH * D, es), span("k", k, BH * D, es), span("v", v, BH * M, es)};
  const Span outs[] = {span("S", S, BH * D * M, 4), span("Z", Z, BH * D, 4), span("out", out, BH * M, es)};
  if ((s = check_disjoint(outs, 3, ins, 3))) return s;
  if (BH > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  return dev(timed("decode", stream,
                   [&] { return la::launch_decode_step(dtype, BH, (int)D, (int)M, S, Z, q, k, v, out, stream); }),
             "decode step");
}

LA_API la_status la_retention_decode_step(float* S, const void* q, const void* k, const void* v,
                                          const float* log_gamma, void* y, int64_t B, int64_t H, int64_t D,
                                          int64_t M, int dtype, hipStream_t stream) {
  la_status s = check_sizes(B, H, 1, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(S, "S", LA_F32)) || (s = check_ptr(q, "q", dtype)) || (s = check_ptr(k, "k", dtype)) ||
      (s = check_ptr(v, "v", dtype)) || (s = check_ptr(log_gamma, "log_gamma", LA_F32)) ||
      (s = check_ptr(y, "y", dtype)))
    return s;
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("q", q, BH * D, es), span("k", k, BH * D, es), span("v", v, BH * M, es),
                      span("log_gamma", log_gamma, BH, 4)};
  const Span outs[] = {span("S", S, BH * D * M, 4), span("y", y, BH * M, es)};
  if ((s = check_disjoint(outs, 2, ins, 4))) return s;
  if (BH > 0xffffffffLL) return fail(LA_ERR_UNSUPPORTED, "grid too large");
  return dev(timed("ret.decode", stream,
                   [&] {
                     return la::launch_ret_decode_step(dtype, BH, (int)D, (int)M, S, q, k, v, log_gamma, y, stream);
                   }),
             "retention decode step");
}

LA_API la_status la_prefix_state(const void* k, const void* v, float* S, float* Z, int64_t B, int64_t H,
                                 int64_t N, int64_t D, int64_t M, int dtype, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if ((s = check_ptr(k, "k", dtype)) || (s = check_ptr(v, "v", dtype)) || (s = check_ptr(S, "S", LA_F32)) ||
      (s = check_ptr(Z, "Z", LA_F32)))
    return s;
  const int64_t BH = B * H;
  const size_t es = dtype_size(dtype);
  const Span ins[] = {span("k", k, BH * N * D, es), span("v", v, BH * N * M, es),
                      span("workspace", workspace, workspace ? (int64_t)workspace_bytes : 0, 1)};
  const Span outs[] = {span("S", S, BH * D * M, 4), span("Z", Z, BH * D, 4)};
  if ((s = check_disjoint(outs, 2, ins, 3))) return s;
  Plan p;
  if ((s = resolve(LA_OP_PREFIX_STATE, B, H, N, D, M, 1, dtype, nullptr, &p, vec16({k, v})))) return s;
  const WsLayout w = layout(LA_OP_PREFIX_STATE, BH, N, D, M, 1, p);
  if (workspace_bytes < w.bytes)
    return fail(LA_ERR_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, w.bytes);
  if (w.bytes && !workspace) return fail(LA_ERR_INVALID, "workspace is NULL (%zu bytes needed)", w.bytes);
  const la::SegGeom g = geom(BH, N, D, M, p, p.chunk);
  hipError_t e;
  if (p.P == 1) {
    if (p.kernel == LA_KERNEL_MFMA)
      return dev(timed("mfma.seg_state", stream, [&] {
                   return dtype == LA_F32 ? la::launch_seg_state_f32mfma(g, k, v, S, D * M, Z, D, stream)
                                          : la::launch_seg_state_mfma(g, k, v, S, D * M, Z, D, stream);
                 }),
                 "prefix state");
    la::SegGeom gs = g;
    gs.chunk = la::generic_chunk_for(g.D, g.M, 1);
    return dev(timed("generic.seg_state", stream,
                     [&] { return la::launch_seg_state_generic(dtype, gs, k, v, S, D * M, Z, D, stream); }),
               "prefix state");
  }
  float* agg = at(workspace, w.aggS);
  if ((e = seg_state(dtype, p, g, k, v, agg, stream))) return dev(e, "prefix state");
  return dev(scan(agg, BH, p.P, g.D, g.M, 0, S, D * M, Z, D, stream), "prefix scan");
}

LA_API size_t la_workspace_bytes_ex(int op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                                    int dtype, const la_plan* plan) {
  if (op == LA_OP_DECODE) return 0;
  if (check_sizes(B, H, N, D, M, dtype) != LA_OK) return 0;
  if (op == LA_OP_POLY_BACKWARD)
    return la::poly_supported(D, M, dtype) ? (static_cast<size_t>(B * H * N) * sizeof(float) + kAlign - 1) / kAlign * kAlign
                                           : 0;
  Plan p;
  if (resolve(op, B, H, N, D, M, causal ? 1 : 0, dtype, op == LA_OP_PREFIX_STATE ? nullptr : plan, &p) != LA_OK)
    return 0;
  return layout(op, B * H, N, D, M, causal ? 1 : 0, p).bytes;
}

LA_API size_t la_saved_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal, int dtype,
                             const la_plan* plan) {
  if (check_sizes(B, H, N, D, M, dtype) != LA_OK) return 0;
  Plan p;
  if (resolve(LA_OP_FORWARD, B, H, N, D, M, causal ? 1 : 0, dtype, plan, &p) != LA_OK) return 0;
  return saved_floats(B * H, D, M, causal ? 1 : 0, p) * sizeof(float);
}

LA_API size_t la_workspace_bytes(int op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                                 int dtype) {
  return la_workspace_bytes_ex(op, B, H, N, D, M, causal, dtype, nullptr);
}

LA_API la_status la_resolve_plan(int op, int64_t B, int64_t H, int64_t N, int64_t D, int64_t M, int causal,
                                 int dtype, const la_plan* requested, la_plan* resolved) {
  la_status s = check_sizes(B, H, N, D, M, dtype);
  if (s != LA_OK) return s;
  if (!resolved) return fail(LA_ERR_INVALID, "resolved is NULL");
  Plan p;
  if ((s = resolve(op, B, H, N, D, M, causal ? 1 : 0, dtype, requested, &p))) return s;
  resolved->chunk = p.chunk;
  resolved->segments = p.P;
  resolved->kernel = p.kernel;
  return ok();
}

LA_API const char* la_status_str(int status) {
  switch (status) {
    case LA_OK: return "LA_OK";
    case LA_ERR_INVALID: return "LA_ERR_INVALID";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_DEVICE: return "LA_ERR_DEVICE";
    default: return "LA_UNKNOWN_STATUS";
  }
}

LA_API const char* la_last_error(void) { return g_err.c_str(); }

LA_API la_status la_device_error(hipStream_t stream) {
  unsigned* addr = nullptr;
  hipError_t e = err_word_for_stream(stream, &addr);
  if (e != hipSuccess) return dev(e, "device error word");
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return dev(e, "stream synchronize");
  unsigned word = 0;
  if ((e = hipMemcpy(&word, addr, sizeof word, hipMemcpyDeviceToHost)) != hipSuccess) return dev(e, "read error word");
  if (!word) return ok();
  const unsigned zero = 0;
  if ((e = hipMemcpy(addr, &zero, sizeof zero, hipMemcpyHostToDevice)) != hipSuccess) return dev(e, "clear error word");
  return fail(LA_ERR_DEVICE, "a workgroup's bounded wait for another workgroup's result ran out; the outputs "
              "of that call hold NaN where it gave up");
}

LA_API int la_version(void) { return 100; }

LA_API la_status la_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRec& r : g_prof) {
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_prof.clear();
  g_prof_on = on != 0;
  return ok();
}

LA_API la_status la_profile_select(const char* names) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_only = names ? names : "";
  return ok();
}

LA_API la_status la_profile_report(char* buf, size_t len) {
  if (!buf || len == 0) return fail(LA_ERR_INVALID, "buffer is NULL or empty");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::map<std::string, std::pair<long, double>> agg;
  hipError_t err = hipSuccess;
  for (const ProfRec& r : g_prof) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) err = e;
    auto& a = agg[r.name];
    a.first += 1;
    a.second += ms;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_prof.clear();
  std::string text;
  for (const auto& kv : agg) {
    char line[256];
    snprintf(line, sizeof line, "%s %ld %.6f\n", kv.first.c_str(), kv.second.first, kv.second.second);
    text += line;
  }
  if (text.size() + 1 > len) return fail(LA_ERR_INVALID, "buffer too small (%zu bytes needed)", text.size() + 1);
  memcpy(buf, text.c_str(), text.size() + 1);
  if (err != hipSuccess) return dev(err, "profile events");
  return ok();
}
