// Device-side helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// bf16 is carried as its raw 16-bit pattern.
typedef uint16_t bf16_t;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ float ld(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
__device__ __forceinline__ void st(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void st(bf16_t* p, int64_t i, float x) { p[i] = f32_to_bf16(x); }

// phi(x) = elu(x) + 1 with alpha = 1: x + 1 above zero, e^x at or below
// ("Transformers are RNNs" walkthrough, section 2).
__device__ __forceinline__ float phi(float x) { return x > 0.f ? x + 1.f : expf(x); }

// phi'(x) = 1 above zero, e^x at or below; since e^x <= 1 there and
// x + 1 > 1 above, phi'(x) = min(phi(x), 1) exactly.
__device__ __forceinline__ float phi_prime_from_phi(float f) { return fminf(f, 1.f); }

}  // namespace la
