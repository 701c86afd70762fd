// Device-side helpers shared by the HIP kernels of libsage (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;  // every kernel runs 4 waves of 64 lanes

// bf16 bit pattern (low or high half of a 32-bit word) -> fp32, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_bits_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
// The same rounding, returned as the fp32 value of the bf16 result.
__device__ __forceinline__ float bf16_round_f32(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}

// Unpack 8 bf16 (one 16-byte load) to fp32.
__device__ __forceinline__ void unpack8(const uint4& v, float* x) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}

// Wave-wide (64 lanes) max of a non-negative float.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Symmetric INT8 code: clamp(rne(x), -127, 127).
__device__ __forceinline__ int i8_code(float x) {
  float r = __builtin_rintf(x);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

}  // namespace sage
