// Test helper (not part of libsage): issue-rate probes for the instructions
// whose costs bound the attention kernel's key step.  Each wave runs `iters`
// iterations of independent dependency chains of one instruction and times
// its loop with the shader-clock counter (s_memtime).  A workgroup holds
// 4 * W waves, i.e. W per SIMD, and more than half of a CU's LDS, so no two
// workgroups share a CU.  The kernel reports each wave's loop cycles; the
// caller divides by the instructions the wave issued and multiplies by 1 / W
// to get cycles per wave64 instruction per SIMD.  Every chain's final value is
// written out, so no link of a chain is dead code.
//
//   op 0  v_fma_f32                         x = fma(x, a, b)
//   op 1  v_cvt_f32_i32                     v = bits(float(v))
//   op 2  v_exp_f32                         x = exp2(x)
//   op 3  v_cvt_pk_fp8_f32                  w = pk_fp8(x0, x1, w): the old word is an input
//   op 4  v_mfma_i32_32x32x32_i8            acc = A B + acc (kChains / 2 accumulators)
//   op 5  v_mfma_scale_f32_32x32x64_f8f6f4  acc = A B + acc (kChains / 2 accumulators)
//
// probe_pair: one SIMD's two waves keep to different units (see pair_kernel).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kChains = 8;

template <int OP>
__global__ void issue_kernel(int iters, const float* __restrict__ seed, uint64_t* __restrict__ cyc,
                             float* __restrict__ sink) {
  // 81 KiB of LDS per workgroup: at most one workgroup per CU
  __shared__ float s_pad[20736];
  const int lane = threadIdx.x & 63;
  const int wid = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const float a = seed[lane], b = seed[(lane + 1) & 63];
  s_pad[threadIdx.x] = a;
  float out = 0.0f;
  if constexpr (OP <= 3) {
    float x[kChains];
    int v[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      x[j] = seed[(lane + j) & 63];
      v[j] = __float_as_int(x[j]);
    }
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) {
        if constexpr (OP == 0) x[j] = __builtin_fmaf(x[j], a, b);
        if constexpr (OP == 1) v[j] = __float_as_int((float)v[j]);
        if constexpr (OP == 2) x[j] = __builtin_amdgcn_exp2f(x[j]);
        if constexpr (OP == 3) v[j] = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, v[j], false);
      }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (lane == 0) cyc[wid] = t1 - t0;
#pragma unroll
    for (int j = 0; j < kChains; ++j) out += x[j] + (float)v[j];
  } else {
    constexpr int NA = kChains / 2;  // accumulators (independent chains)
    const int s = __float_as_int(seed[lane]);
    if constexpr (OP == 4) {
      const v4i A = v4i{s, s ^ 1, s ^ 2, s ^ 3}, B = v4i{s ^ 4, s ^ 5, s ^ 6, s ^ 7};
      v16i acc[NA];
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = j + e;
      __syncthreads();
      const uint64_t t0 = __builtin_amdgcn_s_memtime();
      for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < NA; ++j) acc[j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A, B, acc[j], 0, 0, 0);
      }
      const uint64_t t1 = __builtin_amdgcn_s_memtime();
      if (lane == 0) cyc[wid] = t1 - t0;
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) out += (float)acc[j][e];
    } else {
      // E4M3 operand bytes 0x38 (1.0) and 0x30 (0.5): finite products
      const v8i A = v8i{0x38383838, 0x30303030, 0x38383838, 0x30303030, 0x38383838, 0x30303030,
                        0x38383838, 0x30303030};
      const v8i B = A;
      v16f acc[NA];
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = a;
      __syncthreads();
      const uint64_t t0 = __builtin_amdgcn_s_memtime();
      for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < NA; ++j)
          acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc[j], 0, 0, 0, 0, 0, 0);
      }
      const uint64_t t1 = __builtin_amdgcn_s_memtime();
      if (lane == 0) cyc[wid] = t1 - t0;
#pragma unroll
      for (int j = 0; j < NA; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) out += acc[j][e];
    }
  }
  __syncthreads();
  sink[(size_t)wid * 64 + lane] = out + s_pad[(threadIdx.x + 64) % blockDim.x];
}

// Waves 0-3 of an eight-wave workgroup (one per SIMD) run `iters_m`
// iterations of the FP8 MFMA chains of op 5 while waves 4-7, their SIMD
// partners, run `iters_v` iterations of the vector chains of op VOP (0-3):
// how much of the two units' work overlaps when each wave keeps to one of them.
template <int VOP>
__global__ void pair_kernel(int iters_m, int iters_v, const float* __restrict__ seed, uint64_t* __restrict__ cyc,
                            float* __restrict__ sink) {
  __shared__ float s_pad[20736];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wid = blockIdx.x * (blockDim.x >> 6) + wave;
  const float a = seed[lane];
  s_pad[threadIdx.x] = a;
  float out = 0.0f;
  if (wave < 4) {
    const v8i A = v8i{0x38383838, 0x30303030, 0x38383838, 0x30303030, 0x38383838, 0x30303030,
                      0x38383838, 0x30303030};
    v16f acc[kChains / 2];
#pragma unroll
    for (int j = 0; j < kChains / 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[j][e] = a;
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters_m; ++i) {
#pragma unroll
      for (int j = 0; j < kChains / 2; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, A, acc[j], 0, 0, 0, 0, 0, 0);
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (lane == 0) cyc[wid] = t1 - t0;
#pragma unroll
    for (int j = 0; j < kChains / 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) out += acc[j][e];
  } else {
    const float b = seed[(lane + 1) & 63];
    float x[kChains];
    int v[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) {
      x[j] = seed[(lane + j) & 63];
      v[j] = __float_as_int(x[j]);
    }
    __syncthreads();
    const uint64_t t0 = __builtin_amdgcn_s_memtime();
    for (int i = 0; i < iters_v; ++i) {
#pragma unroll
      for (int j = 0; j < kChains; ++j) {
        if constexpr (VOP == 0) x[j] = __builtin_fmaf(x[j], a, b);
        if constexpr (VOP == 1) v[j] = __float_as_int((float)v[j]);
        if constexpr (VOP == 2) x[j] = __builtin_amdgcn_exp2f(x[j]);
        if constexpr (VOP == 3) v[j] = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, v[j], false);
      }
    }
    const uint64_t t1 = __builtin_amdgcn_s_memtime();
    if (lane == 0) cyc[wid] = t1 - t0;
#pragma unroll
    for (int j = 0; j < kChains; ++j) out += x[j] + (float)v[j];
  }
  __syncthreads();
  sink[(size_t)wid * 64 + lane] = out + s_pad[(threadIdx.x + 64) % blockDim.x];
}

}  // namespace

// The pair kernel with vector op vop (0-3) on `blocks` eight-wave
// workgroups; cyc gets one loop-cycle count per wave (blocks * 8), sink one
// float per thread.  Returns a hipError_t.
extern "C" int probe_pair(int vop, int blocks, int iters_m, int iters_v, const float* seed, uint64_t* cyc,
                          float* sink) {
  if (vop < 0 || vop > 3 || blocks < 1 || iters_m < 1 || iters_v < 1) return -1;
  const dim3 grid(blocks), block(512);
  switch (vop) {
    case 0: hipLaunchKernelGGL(pair_kernel<0>, grid, block, 0, 0, iters_m, iters_v, seed, cyc, sink); break;
    case 1: hipLaunchKernelGGL(pair_kernel<1>, grid, block, 0, 0, iters_m, iters_v, seed, cyc, sink); break;
    case 2: hipLaunchKernelGGL(pair_kernel<2>, grid, block, 0, 0, iters_m, iters_v, seed, cyc, sink); break;
    default: hipLaunchKernelGGL(pair_kernel<3>, grid, block, 0, 0, iters_m, iters_v, seed, cyc, sink); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  return (int)hipDeviceSynchronize();
}

// Runs op on `blocks` workgroups of 4 * waves_per_simd waves each; cyc gets
// one loop-cycle count per wave (blocks * 4 * waves_per_simd entries), sink
// one float per thread.  seed holds 64 floats.  Returns a hipError_t.
extern "C" int probe_issue(int op, int blocks, int waves_per_simd, int iters, const float* seed, uint64_t* cyc,
                           float* sink) {
  if (op < 0 || op > 5 || blocks < 1 || waves_per_simd < 1 || waves_per_simd > 4 || iters < 1) return -1;
  const dim3 grid(blocks), block(256 * waves_per_simd);
  switch (op) {
    case 0: hipLaunchKernelGGL(issue_kernel<0>, grid, block, 0, 0, iters, seed, cyc, sink); break;
    case 1: hipLaunchKernelGGL(issue_kernel<1>, grid, block, 0, 0, iters, seed, cyc, sink); break;
    case 2: hipLaunchKernelGGL(issue_kernel<2>, grid, block, 0, 0, iters, seed, cyc, sink); break;
    case 3: hipLaunchKernelGGL(issue_kernel<3>, grid, block, 0, 0, iters, seed, cyc, sink); break;
    case 4: hipLaunchKernelGGL(issue_kernel<4>, grid, block, 0, 0, iters, seed, cyc, sink); break;
    default: hipLaunchKernelGGL(issue_kernel<5>, grid, block, 0, 0, iters, seed, cyc, sink); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  return (int)hipDeviceSynchronize();
}
