// Streaming HBM ceilings of the MI355X for the traffic mixes of the
// attention kernels: R tensors read and W tensors written, each 134 MB (the
// size of one [8,16,8192,64] bf16 tensor), 16-byte accesses, grid-stride.
// The rate a plain streaming kernel reaches for a given mix is the practical
// ceiling a kernel with that mix can be held against, next to the 8 TB/s
// specification.  Prints one JSON object per line.
//
// Mixes: r1, r2 (segment aggregates), r1w1 (decode step: read and write S),
// r3w1 (forward), r4w1 (dq sweep), r4w2 (dk/dv sweep); and r4w2 with the
// stores issued from an MFMA accumulator layout (8-byte pieces, 16 rows per
// instruction) to show what that store layout costs.
//
// Then the matrix-core ceilings: a register-only loop of independent
// v_mfma_f32_16x16x32_bf16 (and v_mfma_f32_16x16x4_f32) over the whole chip,
// the rate an MFMA-bound kernel can be held against next to the 2.5 PFLOP/s
// (157.3 TFLOP/s fp32) specification.  One JSON object per line as well,
// keyed "mfma".
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr long kBytes = 134217728L;  // 8 * 16 * 8192 * 64 * 2
constexpr int kU = 4;                // 16-byte vectors in flight per tensor per thread

#define CHECK(x)                                                                    \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));          \
      std::exit(1);                                                                 \
    }                                                                               \
  } while (0)

struct Ptrs {
  const i32x4* in[4];
  i32x4* out[2];
};

// Coalesced: every access is a 16-byte vector, consecutive lanes consecutive.
template <int R, int W>
__global__ __launch_bounds__(256) void k_stream(Ptrs p, long n16, int* sink) {
  const long stride = static_cast<long>(gridDim.x) * blockDim.x;
  i32x4 acc = {0, 0, 0, 0};
  for (long base = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x; base < n16; base += stride * kU) {
    i32x4 x[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) x[u] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (base + u * stride < n16) x[u] += p.in[r][base + u * stride];
#pragma unroll
    for (int w = 0; w < W; ++w)
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (base + u * stride < n16) p.out[w][base + u * stride] = x[u] + w;
#pragma unroll
    for (int u = 0; u < kU; ++u) acc += x[u];
  }
  // keeps the loads of the read-only mixes alive; never true for the data
  if (W == 0 && acc.x == 0x12345678 && acc.y == 0x9abcdef) sink[0] = acc.z;
}

// r4w2 with accumulator-layout stores: each wave owns 2 KB blocks (16 rows
// of 128 B); the reads are coalesced 16-byte vectors, the writes 8-byte
// pieces, lane (li, g) at row li, byte 32 n + 8 g, n = 0..3.
__global__ __launch_bounds__(256) void k_rowstore(Ptrs p, long nblk) {
  const int l = threadIdx.x & 63, li = l & 15, g = l >> 4;
  const long wave = (static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const long nwave = (static_cast<long>(gridDim.x) * blockDim.x) >> 6;
  for (long b = wave; b < nblk; b += nwave) {
    const long v0 = b * 128;  // first 16-byte vector of the block
    i32x4 x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x0 += p.in[r][v0 + l];
      x1 += p.in[r][v0 + 64 + l];
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      char* blk = reinterpret_cast<char*>(p.out[w] + v0);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const i32x4 s = (n & 1) ? x1 : x0;
        *reinterpret_cast<i32x2*>(blk + li * 128 + n * 32 + g * 8) = i32x2{s.x + n + w, s.y};
      }
    }
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// ACC chains of `iters` MFMAs per wave, operands from the thread index so
// nothing folds; the sum is stored (per lane) only when it takes a value it
// never takes, which keeps the loop alive.  A wave needs about 16
// independent 16x16 accumulators before the dependent-issue latency stops
// limiting it (bf16 at four waves per SIMD: 8 chains ~1.3 PFLOP/s, 16
// chains ~2.1), so the loops run 16 (16x16 shapes) or 4 (32x32).
template <int ACC>
__global__ __launch_bounds__(256) void k_mfma_bf16(int iters, float* sink) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.001f * static_cast<float>((threadIdx.x + e) & 63));
    b[e] = static_cast<__bf16>(0.5f - 0.001f * static_cast<float>((threadIdx.x * 3 + e) & 63));
  }
  f32x4_t c[ACC];
#pragma unroll
  for (int j = 0; j < ACC; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < ACC; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < ACC; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == -1.0f) sink[threadIdx.x] = s;
}

template <int ACC>
__global__ __launch_bounds__(256) void k_mfma_bf16_32(int iters, float* sink) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1.0f + 0.001f * static_cast<float>((threadIdx.x + e) & 63));
    b[e] = static_cast<__bf16>(0.5f - 0.001f * static_cast<float>((threadIdx.x * 3 + e) & 63));
  }
  f32x16_t c[ACC];
#pragma unroll
  for (int j = 0; j < ACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < ACC; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < ACC; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  if (s == -1.0f) sink[threadIdx.x] = s;
}

template <int ACC>
__global__ __launch_bounds__(256) void k_mfma_f32(int iters, float* sink) {
  const float a = 1.0f + 0.001f * static_cast<float>(threadIdx.x & 63);
  const float b = 0.5f - 0.001f * static_cast<float>((threadIdx.x * 3) & 63);
  f32x4_t c[ACC];
#pragma unroll
  for (int j = 0; j < ACC; ++j) c[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it)
#pragma unroll
    for (int j = 0; j < ACC; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c[j], 0, 0, 0);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < ACC; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (s == -1.0f) sink[threadIdx.x] = s;
}

template <typename F>
float best_us(F launch) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  for (int i = 0; i < 3; ++i) launch();
  CHECK(hipDeviceSynchronize());
  float best = 1e30f;
  for (int i = 0; i < 10; ++i) {
    CHECK(hipEventRecord(e0));
    launch();
    CHECK(hipEventRecord(e1));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (ms < best) best = ms;
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  return best * 1e3f;
}

template <int R, int W>
void mix(const char* name, const Ptrs& p, int* sink) {
  const long n16 = kBytes / 16;
  float best = 1e30f;
  int best_grid = 0;
  for (int grid : {1024, 2048, 4096}) {
    const float us = best_us([&] { hipLaunchKernelGGL((k_stream<R, W>), dim3(grid), dim3(256), 0, 0, p, n16, sink); });
    CHECK(hipGetLastError());
    if (us < best) best = us, best_grid = grid;
  }
  const double bytes = static_cast<double>(R + W) * kBytes;
  std::printf("{\"mix\": \"%s\", \"read_bytes\": %.0f, \"write_bytes\": %.0f, \"us\": %.1f, \"GBps\": %.0f, "
              "\"grid\": %d}\n", name, static_cast<double>(R) * kBytes, static_cast<double>(W) * kBytes, best,
              bytes / best / 1e3, best_grid);
}

}  // namespace

int main() {
  void* buf[6];
  for (auto& b : buf) {
    CHECK(hipMalloc(&b, kBytes));
    CHECK(hipMemset(b, 1, kBytes));
  }
  int* sink = nullptr;
  CHECK(hipMalloc(&sink, sizeof(int)));
  Ptrs p;
  for (int r = 0; r < 4; ++r) p.in[r] = static_cast<const i32x4*>(buf[r]);
  for (int w = 0; w < 2; ++w) p.out[w] = static_cast<i32x4*>(buf[4 + w]);
  // settle the clocks
  for (int i = 0; i < 200; ++i) hipLaunchKernelGGL((k_stream<1, 1>), dim3(2048), dim3(256), 0, 0, p, kBytes / 16, sink);
  CHECK(hipDeviceSynchronize());
  mix<1, 0>("r1", p, sink);
  mix<2, 0>("r2", p, sink);
  mix<1, 1>("r1w1", p, sink);
  mix<3, 1>("r3w1", p, sink);
  mix<4, 1>("r4w1", p, sink);
  mix<4, 2>("r4w2", p, sink);
  float best = 1e30f;
  for (int grid : {1024, 2048, 4096}) {
    const float us = best_us([&] { hipLaunchKernelGGL(k_rowstore, dim3(grid), dim3(256), 0, 0, p, kBytes / 2048); });
    CHECK(hipGetLastError());
    if (us < best) best = us;
  }
  std::printf("{\"mix\": \"r4w2_rowstore\", \"read_bytes\": %.0f, \"write_bytes\": %.0f, \"us\": %.1f, \"GBps\": %.0f}\n",
              4.0 * kBytes, 2.0 * kBytes, best, 6.0 * kBytes / best / 1e3);
  for (auto& b : buf) CHECK(hipFree(b));
  // matrix cores: 16 wave64s per CU (4 per SIMD), 256 CUs
  float* fsink = nullptr;
  CHECK(hipMalloc(&fsink, 256 * sizeof(float)));
  int dev = 0, ncu = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  const int grid = 4 * ncu;
  struct MfmaCase {
    const char* name;
    void (*kern)(int, float*);
    int iters;
    double flops_per_iter;  // per wave
  };
  const MfmaCase cases[] = {{"bf16_16x16x32", k_mfma_bf16<16>, 2048, 16 * (16.0 * 16 * 32 * 2)},
                            {"bf16_32x32x16", k_mfma_bf16_32<4>, 2048, 4 * (32.0 * 32 * 16 * 2)},
                            {"f32_16x16x4", k_mfma_f32<16>, 512, 16 * (16.0 * 16 * 4 * 2)}};
  for (const auto& c : cases) {
    const float us = best_us([&] { hipLaunchKernelGGL(c.kern, dim3(grid), dim3(256), 0, 0, c.iters, fsink); });
    CHECK(hipGetLastError());
    const double flops = static_cast<double>(grid) * 4 * c.iters * c.flops_per_iter;
    std::printf("{\"mfma\": \"%s\", \"flops\": %.0f, \"us\": %.1f, \"TFLOPs\": %.1f, \"grid\": %d}\n", c.name,
                flops, us, flops / us / 1e6, grid);
  }
  CHECK(hipFree(fsink));
  CHECK(hipFree(sink));
  return 0;
}
