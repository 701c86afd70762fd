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

// 16 bytes per lane from base + voff + soff straight into LDS at lds + 16 lane
// (buffer_load_dwordx4 ... lds; lds wave-uniform).  The buffer resource spans
// `bytes` bytes from `base` (word 3: 32-bit data format, no swizzle; reads past
// the record count return zero), so the lane offset stays one 32-bit VGPR and
// the uniform offset an SGPR, with no per-load address arithmetic.  Kept out
// of kernel bodies: the host pass drops the launch stubs of a kernel whose body
// names the resource type.
__device__ __forceinline__ void lds_load16(const void* base, int bytes, void* lds, int voff, int soff) {
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, bytes, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

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

// Two fp32 -> bf16 bits, round to nearest even, packed (lo in bits 0..15):
// one v_cvt_pk_bf16_f32.  Bit-identical to bf16_bits_rne on every finite
// input (checked over all 2^32 patterns on gfx950).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
// The same rounding of a pair, returned in place as fp32 values.
__device__ __forceinline__ void bf16x2_round(float& lo, float& hi) {
  const uint32_t w = bf16x2_rne(lo, hi);
  lo = bf16_lo(w);
  hi = bf16_hi(w);
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

// The QK RMSNorm + RoPE producer on token rows spread over LPR consecutive
// lanes: lane lc of a row's group holds channels 8 lc .. 8 lc + 7, i.e.
// rotation pairs 4 lc .. 4 lc + 3.  The arithmetic is the eager composition
// with each bf16 rounding kept:
//   r = fp32(1 / sqrt(sum_d x_d^2 / D + eps)), in fp64;
//   u = bf16(bf16(x r) w);  y_2i = bf16(u_2i c - u_2i+1 s),
//   y_2i+1 = bf16(u_2i s + u_2i+1 c)  (fp32 products, then the sum).
// bf16 squares are exact in fp64, and so is their sum under the condition
// stated in sage.h, so the order of the additions below leaves every bit as
// it is.

// r of P rows (P <= LPR, both powers of two; x[p] is row p of this lane's
// group).  The P sums of squares are reduce-scattered over the group, so
// lane lc ends with the whole sum of row lc / (LPR / P) and takes the fp64
// square root and divide for that row only (returned in r_own); the P values
// are then broadcast back into r[].  Every lane of the group must call it.
template <int LPR, int P>
__device__ __forceinline__ void rows_rsqrt(const float (&x)[P][8], double eps, float (&r)[P],
                                           float& r_own) {
  static_assert(P >= 1 && P <= LPR && (P & (P - 1)) == 0 && (LPR & (LPR - 1)) == 0, "P, LPR");
  const int lane = __lane_id();
  const int lc = lane & (LPR - 1);
  double ss[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    ss[p] = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double v = (double)x[p][j];
      ss[p] = __builtin_fma(v, v, ss[p]);  // v*v is exact: one rounding, as mul + add
    }
  }
  // halving steps: at offset o the lane keeps the half of its live rows
  // selected by bit o of lc and adds the partner's copy of that half; rows
  // are split on bit LPR/2 first (row weight P/2), then LPR/4, ...
  int live = P;
#pragma unroll
  for (int o = LPR / 2; o > 0; o >>= 1) {
    if (live > 1) {
      const bool hi = (lc & o) != 0;
#pragma unroll
      for (int i = 0; i < P / 2; ++i) {
        if (i < live / 2) {
          const double keep = hi ? ss[i + live / 2] : ss[i];
          const double send = hi ? ss[i] : ss[i + live / 2];
          ss[i] = keep + __shfl_xor(send, o, 64);
        }
      }
      live /= 2;
    } else {
      ss[0] += __shfl_xor(ss[0], o, 64);
    }
  }
  r_own = (float)(1.0 / __builtin_sqrt(ss[0] * (1.0 / (8 * LPR)) + eps));
  constexpr int STRIDE = LPR / P;  // row p's r sits in lanes p*STRIDE .. of the group
#pragma unroll
  for (int p = 0; p < P; ++p) r[p] = __shfl(r_own, (lane & ~(LPR - 1)) + p * STRIDE, 64);
}

// The rest of the producer for P rows of this lane, given each row's r.
template <int P>
__device__ __forceinline__ void norm_rope_apply(float (&x)[P][8], const float (&w)[8],
                                                const float (&cs)[P][8], const float (&r)[P]) {
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float u0 = x[p][2 * i] * r[p], u1 = x[p][2 * i + 1] * r[p];
      bf16x2_round(u0, u1);
      u0 *= w[2 * i];
      u1 *= w[2 * i + 1];
      bf16x2_round(u0, u1);
      const float c = cs[p][2 * i], s = cs[p][2 * i + 1];
      const float a0 = u0 * c, a1 = u1 * s;
      const float b0 = u0 * s, b1 = u1 * c;
      float y0 = a0 - a1, y1 = b0 + b1;
      bf16x2_round(y0, y1);
      x[p][2 * i] = y0;
      x[p][2 * i + 1] = y1;
    }
}

// Both steps for P rows.
template <int LPR, int P>
__device__ __forceinline__ void norm_rope8_rows(float (&x)[P][8], const float (&w)[8],
                                                const float (&cs)[P][8], double eps) {
  float r[P], r_own;
  rows_rsqrt<LPR, P>(x, eps, r, r_own);
  norm_rope_apply<P>(x, w, cs, r);
}

// Loads of the producer's per-lane constants: 8 bf16 weights at channel
// 8 lc, and the (c, s) pairs 4 lc .. 4 lc + 3 of token n (table fp32
// [N][D/2][2], 16-byte aligned).
__device__ __forceinline__ void load_w8(const uint16_t* w, int lc, float (&out)[8]) {
  unpack8(*(const uint4*)(w + 8 * lc), out);
}
template <int D>
__device__ __forceinline__ void load_cs8(const float* rope, int64_t n, int lc, float (&cs)[8]) {
  const float4* p = (const float4*)(rope + (n * (D / 2) + 4 * lc) * 2);
  const float4 a = p[0], b = p[1];
  cs[0] = a.x; cs[1] = a.y; cs[2] = a.z; cs[3] = a.w;
  cs[4] = b.x; cs[5] = b.y; cs[6] = b.z; cs[7] = b.w;
}

// Symmetric INT8 code: clamp(rne(x), -127, 127).
__device__ __forceinline__ int i8_code(float x) {
  float r = __builtin_rintf(x);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

}  // namespace sage
