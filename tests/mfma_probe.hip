// Test helper (not part of libsage): one FP8 matrix-core instruction per wave,
// on operands the host chose, so that tests can compare the hardware result
// with an exact fp64 sum.  The attention's P.V and the row-wise FP8 GEMM both
// accumulate with v_mfma_f32_32x32x64_f8f6f4 (E4M3 A and B, fp32 C and D);
// their tolerances rest on how this instruction rounds a 64-term block, and on
// the operand layout written below.
//
// Layout per wave (lane l = 0..63), checked by the tests against fp64:
//   A (32 x 64): lane l holds A[l % 32][32 (l / 32) + j], byte j = 0..31
//   B (64 x 32): lane l holds B[32 (l / 32) + j][l % 32], byte j = 0..31
//   C, D (32 x 32): register i of lane l is element
//                   [8 (i / 4) + 4 (l / 32) + i % 4][l % 32]
#include <hip/hip_runtime.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// INT8 32x32x32: A (32 x 32) lane l holds A[l % 32][16 (l / 32) + j], B (32 x 32)
// lane l holds B[16 (l / 32) + j][l % 32], byte j = 0..15; C, D int32 as above.
// The chain variant adds a second product on top, as the attention's QK^T
// chains do.
__global__ __launch_bounds__(64) void mfma_i8_kernel(const v4i* a, const v4i* b, const v16i* c, v16i* d) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  d[i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[i], c[i], 0, 0, 0);
}

__global__ __launch_bounds__(64) void mfma_f8_kernel(const v8i* a, const v8i* b, const v16f* c, v16f* d) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  d[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[i], c[i], 0, 0, 0, 0, 0, 0);
}

extern "C" int probe_mfma_i8(const void* a, const void* b, const void* c, void* d, int nwaves,
                             void* stream) {
  if (nwaves <= 0) return 0;
  hipLaunchKernelGGL(mfma_i8_kernel, dim3(nwaves), dim3(64), 0, (hipStream_t)stream, (const v4i*)a,
                     (const v4i*)b, (const v16i*)c, (v16i*)d);
  return (int)hipGetLastError();
}

// a, b: nwaves * 64 * 32 bytes; c, d: nwaves * 64 * 16 floats.  Device
// pointers; returns a hipError_t.
extern "C" int probe_mfma_f8(const void* a, const void* b, const void* c, void* d, int nwaves,
                             void* stream) {
  if (nwaves <= 0) return 0;
  hipLaunchKernelGGL(mfma_f8_kernel, dim3(nwaves), dim3(64), 0, (hipStream_t)stream, (const v8i*)a,
                     (const v8i*)b, (const v16f*)c, (v16f*)d);
  return (int)hipGetLastError();
}
