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
// With block scales (E8M0, 127 = 1): lane l's scale_a byte scales row l % 32
// of A over k-block l / 32, and its scale_b byte scales column l % 32 of B
// over k-block l / 32.
#include <hip/hip_runtime.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(64) void mfma_f8_kernel(const v8i* a, const v8i* b, const v16f* c, v16f* d) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  d[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[i], c[i], 0, 0, 0, 0, 0, 0);
}

__global__ __launch_bounds__(64) void mfma_f8_scaled_kernel(const v8i* a, const v8i* b, const v16f* c,
                                                            const int* sa, const int* sb, v16f* d) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  d[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[i], c[i], 0, 0, 0, sa[i], 0, sb[i]);
}

// a, b: nwaves * 64 * 32 bytes; c, d: nwaves * 64 * 16 floats; sa, sb:
// nwaves * 64 ints (byte 0 is the E8M0 scale).  Device pointers; returns a
// hipError_t.
extern "C" int probe_mfma_f8(const void* a, const void* b, const void* c, void* d, int nwaves,
                             void* stream) {
  if (nwaves <= 0) return 0;
  hipLaunchKernelGGL(mfma_f8_kernel, dim3(nwaves), dim3(64), 0, (hipStream_t)stream, (const v8i*)a,
                     (const v8i*)b, (const v16f*)c, (v16f*)d);
  return (int)hipGetLastError();
}

extern "C" int probe_mfma_f8_scaled(const void* a, const void* b, const void* c, const void* sa,
                                    const void* sb, void* d, int nwaves, void* stream) {
  if (nwaves <= 0) return 0;
  hipLaunchKernelGGL(mfma_f8_scaled_kernel, dim3(nwaves), dim3(64), 0, (hipStream_t)stream,
                     (const v8i*)a, (const v8i*)b, (const v16f*)c, (const int*)sa, (const int*)sb,
                     (v16f*)d);
  return (int)hipGetLastError();
}
