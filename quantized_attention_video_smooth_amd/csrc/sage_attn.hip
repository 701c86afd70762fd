// Fused non-causal attention on INT8 Q/K and FP8 V (gfx950).
//
// Method: "FLUX.3 Action RTX 5090 report", §02 stage 03 (INT8 QK, FP8 PV,
// FP32 accumulation, V smoothing kept) and "MiniMax H3 on DGX Spark", §01
// (QK INT8 / PV FP8).  The pages give no kernel design for this chip; this one
// is built around the CDNA4 32x32 MFMA tiles:
//
//   * a workgroup = 4 waves = 128 queries of one (b, h); a wave owns 32
//     queries, which is exactly one Q quantisation block, so q_scale is a
//     per-wave scalar;
//   * the key loop walks 64-key tiles (one K quantisation block, so k_scale is
//     a per-tile scalar), staged through LDS with double buffering;
//   * S^T = K Q^T with v_mfma_i32_32x32x32_i8 (exact int32).  In that layout
//     lane l holds 32 scores of query l%32, so the row max, the exponentials
//     and the row sum are lane-local except for one exchange between the two
//     32-lane halves;
//   * the probabilities are converted to E4M3 in registers (v_cvt_pk_fp8_f32)
//     and used directly as the B operand of O^T = V^T P^T with
//     v_mfma_f32_32x32x64_f8f6f4; V is stored with the slot permutation that
//     makes those bytes line up (sage_v_slot in sage.h);
//   * exp2 with log2(e) and the static P scale 448 folded into one FMA;
//     the rescale of the accumulator is skipped when no row max moved.
#include <hip/hip_runtime.h>

#include "sage_device.h"
#include "sage_internal.h"

namespace sage {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448)

template <int D>
struct AttnCfg {
  static constexpr int DC = D / 32;          // 32-wide d chunks
  static constexpr int KROW = D + 16;        // LDS bytes per K row (padded: conflict-free b128 reads)
  static constexpr int VROW = 64 + 16;       // LDS bytes per V^T row
  static constexpr int KBYTES = 64 * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KCH = 64 * D / 16;    // 16-byte chunks per K tile
  static constexpr int VCH = D * 4;          // 16-byte chunks per V tile (64 bytes per row)
  static constexpr int KPT = KCH / kThreads; // chunks per thread
  static constexpr int VPT = VCH / kThreads;
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const int8_t* __restrict__ q_i8, const float* __restrict__ q_scale,
    const int8_t* __restrict__ k_i8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v_fp8, const float* __restrict__ v_scale,
    const float* __restrict__ v_mean, int H, int N, int Np, int n_qtiles, int total_tiles,
    float cq0, uint16_t* __restrict__ out, int64_t o_sb, int64_t o_sn, int64_t o_sh) {
  using C = AttnCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * C::STAGE];

  // XCD-aware mapping: workgroup i runs on XCD i % 8; give each XCD a
  // contiguous run of (head, q-tile) work so a head's K/V stay in one L2.
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total_tiles) return;  // whole workgroup exits before any barrier
  const int bh = logical / n_qtiles, qt = logical - bh * n_qtiles;
  const int b = bh / H, h = bh - b * H;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = lane >> 5, l32 = lane & 31;
  const int q0 = qt * 128 + wave * 32;
  const int ntiles = Np / 64;

  // Q^T operand (B of the S^T MFMA): lane holds query q0+l32, d = 32*dc + 16*half .. +16.
  v4i qop[C::DC];
  float cq = 0.0f;
  if (q0 < Np) {
    const int8_t* qp = q_i8 + ((size_t)bh * Np + q0 + l32) * D + 16 * half;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) qop[dc] = *(const v4i*)(qp + 32 * dc);
    cq = q_scale[(size_t)bh * (Np / 32) + q0 / 32] * cq0;
  } else {
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) qop[dc] = v4i{0, 0, 0, 0};
  }

  const int8_t* kbase = k_i8 + (size_t)bh * Np * D;
  const uint8_t* vbase = v_fp8 + (size_t)bh * D * Np;
  const float* ksc = k_scale + (size_t)bh * ntiles;

  // Per-thread share of one K tile (KPT chunks) and one V^T tile (VPT chunks).
  uint4 kreg[C::KPT], vreg[C::VPT];
#define SAGE_GLOAD(t_)                                                                   \
  do {                                                                                   \
    _Pragma("unroll") for (int i_ = 0; i_ < C::KPT; ++i_) {                              \
      const int c_ = tid + kThreads * i_;                                                \
      kreg[i_] = *(const uint4*)(kbase + (size_t)(t_) * 64 * D + c_ * 16);               \
    }                                                                                    \
    _Pragma("unroll") for (int i_ = 0; i_ < C::VPT; ++i_) {                              \
      const int c_ = tid + kThreads * i_;                                                \
      vreg[i_] = *(const uint4*)(vbase + (size_t)(c_ >> 2) * Np + (t_) * 64 + (c_ & 3) * 16); \
    }                                                                                    \
  } while (0)
#define SAGE_SSTORE(buf_)                                                                \
  do {                                                                                   \
    uint8_t* ks_ = smem + (buf_) * C::STAGE;                                             \
    uint8_t* vs_ = ks_ + C::KBYTES;                                                      \
    _Pragma("unroll") for (int i_ = 0; i_ < C::KPT; ++i_) {                              \
      const int c_ = tid + kThreads * i_;                                                \
      *(uint4*)(ks_ + (c_ / (D / 16)) * C::KROW + (c_ % (D / 16)) * 16) = kreg[i_];      \
    }                                                                                    \
    _Pragma("unroll") for (int i_ = 0; i_ < C::VPT; ++i_) {                              \
      const int c_ = tid + kThreads * i_;                                                \
      *(uint4*)(vs_ + (c_ >> 2) * C::VROW + (c_ & 3) * 16) = vreg[i_];                   \
    }                                                                                    \
  } while (0)

  v16f acc[C::DC];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dc][i] = 0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  SAGE_GLOAD(0);
  SAGE_SSTORE(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    // prefetch the next tile (the last iteration re-reads its own tile; the
    // other buffer is free then, so the unconditional store below is harmless)
    SAGE_GLOAD(min(t + 1, ntiles - 1));
    const uint8_t* ks = smem + buf * C::STAGE;
    const uint8_t* vs = ks + C::KBYTES;

    // ---- S^T = K Q^T (two 32-key halves of the tile) ----
    v16i s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      const uint8_t* kr = ks + (32 * kb + l32) * C::KROW + 16 * half;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        const v4i a = *(const v4i*)(kr + 32 * dc);
        s[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qop[dc], s[kb], 0, 0, 0);
      }
    }
    // key index of s[kb][i] inside the tile: 32*kb + 8*(i/4) + 4*half + i%4
    const int nvalid = N - t * 64;  // keys at or beyond nvalid are padding
    if (nvalid < 64) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          if (key >= nvalid) s[kb][i] = INT32_MIN;
        }
    }
    int mxi = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mxi = max(mxi, s[kb][i]);
    mxi = max(mxi, __shfl_xor(mxi, 32, 64));

    const float c = cq * ksc[t];
    const float m_new = fmaxf(m_run, (float)mxi * c);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if (__any(m_new != m_run)) {
      l_run *= alpha;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dc][i] *= alpha;
    }
    m_run = m_new;
    const float bias = kLog2_448 - m_new;

    // ---- P = exp2(s*c - m) * 448, row sum, E4M3 pack (byte 16*kb + i) ----
    v8i pop;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * r + e;
          float x = __builtin_amdgcn_exp2f(__builtin_fmaf((float)s[kb][i], c, bias));
          if (nvalid < 64) {
            const int key = 32 * kb + 8 * r + 4 * half + e;
            if (key >= nvalid) x = 0.0f;
          }
          p[e] = x;
          lsum += x;
        }
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        pop[4 * kb + r] = w;
      }
    l_run += lsum;

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      const uint8_t* vr = vs + (32 * dc + l32) * C::VROW + 32 * half;
      const v4i lo = *(const v4i*)(vr);
      const v4i hi = *(const v4i*)(vr + 16);
      const v8i a = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      acc[dc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pop, acc[dc], 0, 0, 0, 0, 0, 0);
    }

    SAGE_SSTORE(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / (448 * l) * v_scale + v_mean, bf16 NHD ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv_l = 1.0f / l_tot;
  const int qi = q0 + l32;
  if (qi < N) {
    uint16_t* orow = out + (int64_t)b * o_sb + (int64_t)qi * o_sn + (int64_t)h * o_sh;
    const float* vsc = v_scale + (size_t)bh * D;
    const float* vmu = v_mean + (size_t)bh * D;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * dc + 8 * g + 4 * half;
        uint32_t bits[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float o = acc[dc][4 * g + e] * inv_l * vsc[d0 + e] + vmu[d0 + e];
          bits[e] = bf16_bits_rne(o);
        }
        *(uint2*)(orow + d0) = make_uint2(bits[0] | (bits[1] << 16), bits[2] | (bits[3] << 16));
      }
  }
#undef SAGE_GLOAD
#undef SAGE_SSTORE
}

template <int D>
hipError_t attn_impl(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                     const float* v_mean, int B, int N, int H, float sm_scale, uint16_t* out,
                     int64_t o_sb, int64_t o_sn, int64_t o_sh, hipStream_t stream) {
  const int Np = (int)padded_tokens(N);
  const int n_qtiles = (int)ceil_div(N, 128);
  const int total = B * H * n_qtiles;
  const int grid = (int)ceil_div(total, 8) * 8;
  const float cq0 = sm_scale * kLog2e;
  hipLaunchKernelGGL((attn_fwd_kernel<D>), dim3(grid), dim3(kThreads), 0, stream, q_i8, q_scale,
                     k_i8, k_scale, v_fp8, v_scale, v_mean, H, N, Np, n_qtiles, total, cq0, out,
                     o_sb, o_sn, o_sh);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                           const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                           const float* v_mean, int B, int N, int H, int D, float sm_scale,
                           uint16_t* out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
                           hipStream_t stream) {
  if (D == 128)
    return attn_impl<128>(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, B, N, H, sm_scale,
                          out, o_sb, o_sn, o_sh, stream);
  return attn_impl<64>(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, B, N, H, sm_scale, out,
                       o_sb, o_sn, o_sh, stream);
}

}  // namespace sage
