// Host-side internals of libsage: workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sage {

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t padded_tokens(int64_t N) { return ceil_div(N, 64) * 64; }

// Token chunks per (b, h) for the channel-statistics pass: about 1024
// workgroups (four per CU of a 256-CU part, the occupancy the pass runs at),
// but no chunk shorter than 384 tokens (or than N).  Same-box timings of 512,
// 1024, 2048 and 4096 target workgroups (sage_quant_qk / sage_quant_v per
// call): at the quant-only size (B1 H40 N32760: chunks of 1260 tokens at
// 1024) 1024 was best, 512 2-4% slower; at the FLUX joint size (B2 H24 N4608)
// 512 (chunks of 419 tokens) was best, 1024 (210 tokens) 7-9% slower and 2048
// 16-32% slower.  A workgroup's partials, its hand-over and the head's
// finalisation cost about as much as streaming ~400 tokens, so shorter chunks
// lose; fewer workgroups than ~4 per CU leave HBM latency exposed.
struct StatsSplit {
  int nchunk;
  int rows_per_chunk;
};
inline StatsSplit stats_split(int B, int N, int H) {
  int64_t bh = (int64_t)B * H;
  int64_t want = ceil_div(1024, bh);
  int64_t maxc = ceil_div(N, 384);
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  int rpc = (int)ceil_div(N, want);
  return StatsSplit{(int)ceil_div(N, rpc), rpc};
}

// Arrival counters at the start of every quantiser workspace: one int per
// (b, h) when a head is split into more than one statistics chunk, which
// happens only for fewer than 1024 heads (stats_split).  The region has a
// fixed size, so partials of one shape never land on the counters of another;
// it must be zero before a workspace's first use and every call leaves it zero.
constexpr size_t kCounterBytes = 2048 * sizeof(int);

// sage_quant_qk workspace: arrival counters (above), fp64 partial sums and
// partial sums of |x| [BH][nchunk][D], exactness witnesses [BH][nchunk][D]
// (uint32: smallest non-zero |x| bits - 1, 0xFFFF for none); with the QK
// RMSNorm + RoPE producer in front (nr), also each K row's fp32 r [BH][Np],
// written by the statistics pass and read by the quantisation pass.
struct QkWorkspace {
  size_t cnt_off, partial_off, abs_off, wit_off, rk_off, bytes;
};
inline QkWorkspace qk_workspace(int B, int N, int H, int D, bool nr = false) {
  StatsSplit s = stats_split(B, N, H);
  size_t bh = (size_t)B * H, n = bh * s.nchunk * D;
  QkWorkspace w;
  w.cnt_off = 0;
  w.partial_off = kCounterBytes;
  w.abs_off = w.partial_off + align256(n * sizeof(double));
  w.wit_off = w.abs_off + align256(n * sizeof(double));
  w.rk_off = w.wit_off + align256(n * sizeof(uint32_t));
  w.bytes = w.rk_off + (nr ? align256(bh * padded_tokens(N) * sizeof(float)) : 0);
  return w;
}

// sage_quant_v workspace: arrival counters [BH] (as above), fp64 partial sums
// and sums of |x|, fp32 partial min and max, exactness witnesses
// [BH][nchunk][D], per-channel 448/a [BH][D].
struct VWorkspace {
  size_t cnt_off, sum_off, abs_off, min_off, max_off, wit_off, inv_off, bytes;
};
inline VWorkspace v_workspace(int B, int N, int H, int D) {
  StatsSplit s = stats_split(B, N, H);
  size_t bh = (size_t)B * H, n = bh * s.nchunk * D;
  VWorkspace w;
  w.cnt_off = 0;
  w.sum_off = kCounterBytes;
  w.abs_off = w.sum_off + align256(n * sizeof(double));
  w.min_off = w.abs_off + align256(n * sizeof(double));
  w.max_off = w.min_off + align256(n * sizeof(float));
  w.wit_off = w.max_off + align256(n * sizeof(float));
  w.inv_off = w.wit_off + align256(n * sizeof(uint32_t));
  w.bytes = w.inv_off + align256(bh * D * sizeof(float));
  return w;
}

// Bytes at the start of a quantiser workspace that must be zero before its
// first use (the arrival counters).
inline size_t workspace_zero_bytes() { return kCounterBytes; }

// The QK RMSNorm + RoPE producer's constants: bf16 weights [D] of the Q and
// K norms, the (cos, sin) table fp32 [N][D/2][2], eps.
struct NormRope {
  const uint16_t* wq;
  const uint16_t* wk;
  const float* rope;
  double eps;
};

// nr == nullptr: Q and K are quantised as given; else they are the producer's
// inputs and are normalised and rotated on the fly.
hipError_t launch_quant_qk(const uint16_t* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                           const uint16_t* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                           int B, int N, int H, int D, int q_block, int k_block, const NormRope* nr,
                           int8_t* q_i8, float* q_scale,
                           int8_t* k_i8, float* k_scale, uint16_t* k_mean, void* workspace,
                           hipStream_t stream);

hipError_t launch_norm_rope(const uint16_t* x, int64_t sb, int64_t sn, int64_t sh, int B, int N,
                            int H, int D, const uint16_t* w, const float* rope, double eps,
                            uint16_t* y, int64_t y_sb, int64_t y_sn, int64_t y_sh,
                            hipStream_t stream);

// Q alone (the Q half of launch_quant_qk, no workspace).
hipError_t launch_quant_q(const uint16_t* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, int B, int N,
                          int H, int D, int q_block, int8_t* q_i8, float* q_scale,
                          hipStream_t stream);

hipError_t launch_quant_v(const uint16_t* v, int64_t v_sb, int64_t v_sn, int64_t v_sh, int B, int N,
                          int H, int D, uint8_t* v_fp8, float* v_scale, float* v_mean,
                          void* workspace, hipStream_t stream);

// Forced attention workgroup size (0 automatic, 4 or 8 waves), process-wide,
// for benchmark comparisons.
void set_attn_waves(int waves);
// Forced key-step schedule of the attention (0 default, 1 compiler order,
// 2 interleaved), process-wide, for benchmark comparisons.
void set_attn_schedule(int schedule);

// Waves per workgroup and grid size of the attention launch for these sizes
// (N: queries).
void attn_shape(int B, int N, int H, int D, int* waves, int* workgroups);

// Nq queries against Nk keys (Nq == Nk for self-attention over one sequence).
hipError_t launch_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                           const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                           const float* v_mean, int B, int Nq, int Nk, int H, int D, int q_block,
                           int k_block, float sm_scale, uint16_t* out, int64_t o_sb, int64_t o_sn,
                           int64_t o_sh, hipStream_t stream);

// Row-wise FP8 projections.
hipError_t launch_quant_rows_fp8(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* codes,
                                 float* scales, hipStream_t stream);
void gemm_fp8_shape(int M, int N, int* workgroups);
hipError_t launch_gemm_fp8_rowwise(const uint8_t* x8, const float* sx, int M, const uint8_t* w8,
                                   const float* sw, int N, int K, const uint16_t* bias,
                                   uint16_t* out, int64_t ldo, hipStream_t stream);

}  // namespace sage
