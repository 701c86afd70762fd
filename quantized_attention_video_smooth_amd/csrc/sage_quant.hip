// Quantisation kernels of libsage (gfx950): K smoothing + INT8 K, INT8 Q,
// V smoothing + FP8 E4M3 V with transpose, zero padding and token permutation.
//
// Method: "FLUX.3 Action RTX 5090 report", §02 stage 03 (per-block INT8 QK,
// FP8 PV, K and V smoothing) and card A (the K centring is done inside the
// quantiser, keeping the BF16 rounding of K - mean); card C (V is transposed,
// padded and permuted in one tiled pass; its mean, scale and quantisation are
// kept).  E4M3 layout per "Why can an A10 run FLUX.1", §1.1.
//
// All of this is HBM-bound streaming work.  Each tensor is read twice: once
// for the per-channel statistics (fp64 sums, and min / max for V) and once to
// quantise.  The statistics pass splits every (b, h) into token chunks and
// writes per-chunk partials; a small per-head kernel reduces them in a fixed
// order and writes the head's mean (and V's scale).  fp64 sums of bf16 values
// are exact under the condition stated in sage.h, so the mean bits do not
// depend on the summation order.
#include <hip/hip_runtime.h>

#include "sage_device.h"
#include "sage_internal.h"

namespace sage {

namespace {

// Storage slot of token t (0..63) inside a 64-token block of transposed V:
// slot bits (5..0) = token bits (2, 5, 4, 3, 1, 0).  With this order the 32
// probabilities one lane holds after the 32x32 INT8 S^T MFMAs (keys
// 8*(i/4) + 4*half + i%4 of each 32-key half-tile) line up with the 32 bytes
// that lane supplies to the FP8 PV MFMA.
__device__ __forceinline__ int v_slot(int t) {
  return (((t >> 2) & 1) << 5) | (((t >> 5) & 1) << 4) | (((t >> 3) & 3) << 2) | (t & 3);
}

// ---------------------------------------------------------------------------
// Channel statistics: grid (nchunk, B*H), 256 threads.  Each thread owns 8
// consecutive channels (one 16-byte load per token row); D/8 threads cover a
// row, so a pass reads 256/(D/8) rows.
// ---------------------------------------------------------------------------
// NR: the rows are first put through the QK RMSNorm + RoPE producer
// (weights nr_w, table rope), so the statistics are those of the producer's
// output; each row's r is stored in rk [BH][Np] for the quantisation pass.
template <int D, bool IS_V, bool NR = false>
__global__ __launch_bounds__(kThreads) void stats_kernel(
    const uint16_t* __restrict__ x, int64_t sb, int64_t sn, int64_t sh, int H, int N, int nchunk,
    int rows_per_chunk, double* __restrict__ psum, float* __restrict__ pmin,
    float* __restrict__ pmax, const uint16_t* __restrict__ nr_w, const float* __restrict__ rope,
    double eps, float* __restrict__ rk, int Np) {
  constexpr int LPR = D / 8;
  constexpr int RPP = kThreads / LPR;
  __shared__ double s_sum[RPP][D];
  __shared__ float s_min[IS_V ? RPP : 1][D];
  __shared__ float s_max[IS_V ? RPP : 1][D];

  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, lr = tid / LPR, lc = tid - lr * LPR;
  const uint16_t* base = x + (int64_t)b * sb + (int64_t)h * sh + lc * 8;
  const int r0 = c * rows_per_chunk;
  const int r1 = min(N, r0 + rows_per_chunk);

  double acc[8];
  float mn[8], mx[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] = 0.0;
    mn[j] = __builtin_inff();
    mx[j] = -__builtin_inff();
  }
  float w8[8];
  if constexpr (NR) load_w8(nr_w, lc, w8);
  // every lane of a token row takes the same path (the row index depends on
  // the row, not the lane), as the producer's cross-lane sum needs
  auto take = [&](const uint4& v, int row) {
    float f[8];
    unpack8(v, f);
    if constexpr (NR) {
      float f1[1][8], cs[1][8], r[1], r_own;
#pragma unroll
      for (int j = 0; j < 8; ++j) f1[0][j] = f[j];
      load_cs8<D>(rope, row, lc, cs[0]);
      rows_rsqrt<LPR, 1>(f1, eps, r, r_own);
      if (lc == 0) rk[(size_t)bh * Np + row] = r_own;
      norm_rope_apply<1>(f1, w8, cs, r);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = f1[0][j];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] += (double)f[j];
      if (IS_V) {
        mn[j] = fminf(mn[j], f[j]);
        mx[j] = fmaxf(mx[j], f[j]);
      }
    }
  };
  int r = r0 + lr;
  if constexpr (!NR) {
    for (; r + 7 * RPP < r1; r += 8 * RPP) {  // 8 independent 16-byte loads in flight
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = *(const uint4*)(base + (int64_t)(r + u * RPP) * sn);
#pragma unroll
      for (int u = 0; u < 8; ++u) take(v[u], r + u * RPP);
    }
  } else {
    // 2 rows per step, data and table loads issued together, the producer
    // run on both rows at once (2 rather than 4 rows: fewer live registers,
    // more waves per SIMD to overlap the producer's arithmetic with loads)
    for (; r + 1 * RPP < r1; r += 2 * RPP) {
      uint4 v[2];
      float f[2][8], cs[2][8];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        v[u] = *(const uint4*)(base + (int64_t)(r + u * RPP) * sn);
        load_cs8<D>(rope, r + u * RPP, lc, cs[u]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) unpack8(v[u], f[u]);
      float rr[2], r_own;
      rows_rsqrt<LPR, 2>(f, eps, rr, r_own);
      if ((lc & (LPR / 2 - 1)) == 0) rk[(size_t)bh * Np + r + (lc / (LPR / 2)) * RPP] = r_own;
      norm_rope_apply<2>(f, w8, cs, rr);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += (double)f[u][j];
    }
  }
  for (; r < r1; r += RPP) take(*(const uint4*)(base + (int64_t)r * sn), r);

#pragma unroll
  for (int j = 0; j < 8; ++j) {
    s_sum[lr][lc * 8 + j] = acc[j];
    if (IS_V) {
      s_min[lr][lc * 8 + j] = mn[j];
      s_max[lr][lc * 8 + j] = mx[j];
    }
  }
  __syncthreads();
  const size_t pbase = ((size_t)bh * nchunk + c) * D;
  if (tid < D) {
    double s = 0.0;
    float lo = __builtin_inff(), hi = -__builtin_inff();
    for (int i = 0; i < RPP; ++i) {
      s += s_sum[i][tid];
      if (IS_V) {
        lo = fminf(lo, s_min[i][tid]);
        hi = fmaxf(hi, s_max[i][tid]);
      }
    }
    psum[pbase + tid] = s;
    if (IS_V) {
      pmin[pbase + tid] = lo;
      pmax[pbase + tid] = hi;
    }
  }
}

// ---------------------------------------------------------------------------
// Per-head finalisation: grid (B*H), D threads.  Reduces the chunk partials in
// ascending chunk order; K: k_mean = bf16(fp32(sum / N)); V: v_mean, v_scale
// and 448/a (kept in the workspace for the quantisation pass).
// ---------------------------------------------------------------------------
template <int D, bool IS_V>
__global__ __launch_bounds__(D) void finalize_kernel(
    const double* __restrict__ psum, const float* __restrict__ pmin, const float* __restrict__ pmax,
    int N, int nchunk, uint16_t* __restrict__ k_mean, float* __restrict__ v_mean,
    float* __restrict__ v_scale, float* __restrict__ v_inv) {
  const int bh = blockIdx.x, d = threadIdx.x;
  double s = 0.0;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  const size_t base = (size_t)bh * nchunk * D + d;
  int c = 0;
  for (; c + 8 <= nchunk; c += 8) {  // 8 loads in flight, summed in ascending chunk order
    double ps[8];
    float pl[8], ph[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      ps[u] = psum[base + (size_t)(c + u) * D];
      if (IS_V) {
        pl[u] = pmin[base + (size_t)(c + u) * D];
        ph[u] = pmax[base + (size_t)(c + u) * D];
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      s += ps[u];
      if (IS_V) {
        lo = fminf(lo, pl[u]);
        hi = fmaxf(hi, ph[u]);
      }
    }
  }
  for (; c < nchunk; ++c) {
    s += psum[base + (size_t)c * D];
    if (IS_V) {
      lo = fminf(lo, pmin[base + (size_t)c * D]);
      hi = fmaxf(hi, pmax[base + (size_t)c * D]);
    }
  }
  const float mean = (float)(s / (double)N);
  if (!IS_V) {
    k_mean[(size_t)bh * D + d] = (uint16_t)bf16_bits_rne(mean);
  } else {
    const float a = fmaxf(fabsf(hi - mean), fabsf(lo - mean));
    const float inv = 448.0f / a;
    const bool zero = (a == 0.0f) || !__builtin_isfinite(inv);
    v_mean[(size_t)bh * D + d] = mean;
    v_scale[(size_t)bh * D + d] = zero ? 0.0f : a / 448.0f;
    v_inv[(size_t)bh * D + d] = zero ? 0.0f : inv;
  }
}

// ---------------------------------------------------------------------------
// Fused K centre + BF16 round + INT8 (z = 0) and Q INT8 (z = 1).
// grid (Np/64, B*H, 2), 256 threads; one 64-token x D tile per workgroup
// (one K block or four 16-token K blocks when k_block == 16; two 32-token Q
// blocks, or 64 per-token Q scales when q_block == 1).  Outputs are
// head-major [B,H,Np,D].
// ---------------------------------------------------------------------------
// NR: Q and K rows go through the QK RMSNorm + RoPE producer first (weights
// wq / wk, table rope), as the statistics pass did for K.
template <int D, bool NR = false>
__global__ __launch_bounds__(kThreads) void qk_quant_kernel(
    const uint16_t* __restrict__ q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
    const uint16_t* __restrict__ k, int64_t k_sb, int64_t k_sn, int64_t k_sh, int H, int N, int Np,
    const uint16_t* __restrict__ k_mean, int8_t* __restrict__ q_i8, float* __restrict__ q_scale,
    int8_t* __restrict__ k_i8, float* __restrict__ k_scale, int q_block, int k_block,
    const uint16_t* __restrict__ wq, const uint16_t* __restrict__ wk,
    const float* __restrict__ rope, double eps, const float* __restrict__ rk, int q_only) {
  constexpr int LPR = D / 8;
  constexpr int RPP = kThreads / LPR;
  constexpr int PASSES = 64 / RPP;
  __shared__ float s_red[2][kThreads / 64];

  // heads in reverse order: the statistics pass walked them forwards, so the
  // most recently read heads (most likely still in the memory-side cache)
  // are re-read first
  const int t = blockIdx.x, bh = gridDim.y - 1 - blockIdx.y;
  const bool is_q = (blockIdx.z | q_only) != 0;  // q_only: a grid of Q tiles alone
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, lr = tid / LPR, lc = tid - lr * LPR;
  const uint16_t* src = is_q ? q + (int64_t)b * q_sb + (int64_t)h * q_sh
                             : k + (int64_t)b * k_sb + (int64_t)h * k_sh;
  const int64_t sn = is_q ? q_sn : k_sn;
  src += lc * 8;

  float mean[8];
  if (!is_q) {
    const uint4 m = *(const uint4*)(k_mean + (size_t)bh * D + lc * 8);
    unpack8(m, mean);
  }
  float w8[8];
  if constexpr (NR) load_w8(is_q ? wq : wk, lc, w8);

  float x[PASSES][8];
  float mp[PASSES];                // this thread's absmax in each pass
  float a_lo = 0.0f, a_hi = 0.0f;  // absmax of rows 0..31 and 32..63 of the tile
  if constexpr (NR) {
    // every lane loads (rows beyond N read row N-1 and are zeroed below), so
    // the producer's cross-lane steps see whole groups; all loads first
    uint4 raw[PASSES];
    float cs[PASSES][8], rr[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int r = min(t * 64 + lr + p * RPP, N - 1);
      raw[p] = *(const uint4*)(src + (int64_t)r * sn);
      load_cs8<D>(rope, r, lc, cs[p]);
      if (!is_q) rr[p] = rk[(size_t)bh * Np + r];  // K: r from the statistics pass
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) unpack8(raw[p], x[p]);
    if (is_q) {
      float r_own;
      rows_rsqrt<LPR, PASSES>(x, eps, rr, r_own);
    }
    norm_rope_apply<PASSES>(x, w8, cs, rr);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int r = t * 64 + lr + p * RPP;
    if (r < N) {
      if constexpr (!NR) {
        const uint4 v = *(const uint4*)(src + (int64_t)r * sn);
        unpack8(v, x[p]);
      }
      if (!is_q) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[p][j] = bf16_round_f32(x[p][j] - mean[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x[p][j] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(x[p][j]));
    mp[p] = m;
    if (p < PASSES / 2) a_lo = fmaxf(a_lo, m); else a_hi = fmaxf(a_hi, m);
  }
  if (is_q && q_block == 1) {
    // one scale per token: the row's absmax over the LPR consecutive lanes
    // that hold it (a wave holds 64 / LPR whole rows)
    int8_t* dst = q_i8 + ((size_t)bh * Np + t * 64) * D + lc * 8;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(x[p][j]));
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) a = fmaxf(a, __shfl_xor(a, o, 64));
      const float iv = 127.0f / a;
      const bool zero = (a == 0.0f) || !__builtin_isfinite(iv);
      const float inv = zero ? 0.0f : iv;
      const int rr = lr + p * RPP;
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0 |= (uint32_t)(i8_code(x[p][j] * inv) & 0xFF) << (8 * j);
        w1 |= (uint32_t)(i8_code(x[p][j + 4] * inv) & 0xFF) << (8 * j);
      }
      *(uint2*)(dst + (size_t)rr * D) = make_uint2(w0, w1);
      if (lc == 0) q_scale[(size_t)bh * Np + t * 64 + rr] = zero ? 0.0f : a / 127.0f;
    }
    return;  // whole workgroup (is_q and q_block are uniform), before any barrier
  }
  if (!is_q && k_block == 16) {
    // four K scales per 64-token tile.  The rows one wave holds in one pass
    // (RPW consecutive rows) lie inside one 16-token block, so each block's
    // absmax is a max over (pass, wave) pairs of per-wave maxima.
    constexpr int RPW = 64 / LPR;
    static_assert(RPW <= 16 && 16 % RPW == 0, "a wave's rows of a pass must sit in one block");
    __shared__ float s16[PASSES][kThreads / 64];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const float w = wave_max(mp[p]);
      if ((tid & 63) == 0) s16[p][tid >> 6] = w;
    }
    __syncthreads();
    float inv16[4], sc16[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int p = 0; p < PASSES; ++p)
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w)
          if ((p * RPP + w * RPW) / 16 == j) a = fmaxf(a, s16[p][w]);
      const float iv = 127.0f / a;
      const bool zero = (a == 0.0f) || !__builtin_isfinite(iv);
      inv16[j] = zero ? 0.0f : iv;
      sc16[j] = zero ? 0.0f : a / 127.0f;
    }
    int8_t* dst = k_i8 + ((size_t)bh * Np + t * 64) * D + lc * 8;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int rr = lr + p * RPP, blk = rr >> 4;
      float iv = inv16[0];
#pragma unroll
      for (int j = 1; j < 4; ++j) iv = (blk == j) ? inv16[j] : iv;
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w0 |= (uint32_t)(i8_code(x[p][j] * iv) & 0xFF) << (8 * j);
        w1 |= (uint32_t)(i8_code(x[p][j + 4] * iv) & 0xFF) << (8 * j);
      }
      *(uint2*)(dst + (size_t)rr * D) = make_uint2(w0, w1);
    }
    if (tid == 0) {
#pragma unroll
      for (int j = 0; j < 4; ++j) k_scale[(size_t)bh * (Np / 16) + 4 * t + j] = sc16[j];
    }
    return;
  }
  a_lo = wave_max(a_lo);
  a_hi = wave_max(a_hi);
  if ((tid & 63) == 0) {
    s_red[0][tid >> 6] = a_lo;
    s_red[1][tid >> 6] = a_hi;
  }
  __syncthreads();
  a_lo = fmaxf(fmaxf(s_red[0][0], s_red[0][1]), fmaxf(s_red[0][2], s_red[0][3]));
  a_hi = fmaxf(fmaxf(s_red[1][0], s_red[1][1]), fmaxf(s_red[1][2], s_red[1][3]));
  if (!is_q) a_lo = a_hi = fmaxf(a_lo, a_hi);

  float inv[2], scale[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float a = s ? a_hi : a_lo;
    const float iv = 127.0f / a;
    const bool zero = (a == 0.0f) || !__builtin_isfinite(iv);
    inv[s] = zero ? 0.0f : iv;
    scale[s] = zero ? 0.0f : a / 127.0f;
  }

  int8_t* dst = (is_q ? q_i8 : k_i8) + ((size_t)bh * Np + t * 64) * D + lc * 8;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int rr = lr + p * RPP;
    const float iv = inv[p < PASSES / 2 ? 0 : 1];
    uint32_t w0 = 0, w1 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w0 |= (uint32_t)(i8_code(x[p][j] * iv) & 0xFF) << (8 * j);
      w1 |= (uint32_t)(i8_code(x[p][j + 4] * iv) & 0xFF) << (8 * j);
    }
    *(uint2*)(dst + (size_t)rr * D) = make_uint2(w0, w1);
  }
  if (tid == 0) {
    if (is_q) {
      q_scale[(size_t)bh * (Np / 32) + 2 * t] = scale[0];
      q_scale[(size_t)bh * (Np / 32) + 2 * t + 1] = scale[1];
    } else {
      k_scale[(size_t)bh * (Np / 64) + t] = scale[0];
    }
  }
}

// ---------------------------------------------------------------------------
// V centre + scale + E4M3, transposed to [B,H,D,Np] with the slot permutation.
// grid (ceil(Np/128), B*H), 256 threads; one 128-token x D tile per workgroup.
// Each thread converts 4 consecutive tokens x 8 channels (4 consecutive tokens
// land in 4 consecutive slots) and writes one 32-bit word per channel into an
// LDS tile [D][128]; the tile is then stored as 16-byte row chunks.  The LDS
// column chunk is XOR-swizzled by (row / 8) to spread banks.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void v_quant_kernel(
    const uint16_t* __restrict__ v, int64_t sb, int64_t sn, int64_t sh, int H, int N, int Np,
    const float* __restrict__ v_mean, const float* __restrict__ v_inv, uint8_t* __restrict__ v_fp8) {
  constexpr int CPR = D / 8;                     // 8-channel chunks per token row
  constexpr int MT = (32 * CPR) / kThreads;      // micro-tiles per thread
  constexpr int LROW = 128;                      // LDS bytes per channel row
  __shared__ __attribute__((aligned(16))) uint8_t tile[D * LROW];

  const int u = blockIdx.x, bh = gridDim.y - 1 - blockIdx.y;  // reverse head order (as above)
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x;
  const int tok0 = u * 128;
  const uint16_t* src = v + (int64_t)b * sb + (int64_t)h * sh;

#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int idx = tid + kThreads * m;
    const int cc = idx % CPR, g = idx / CPR;  // channel chunk, 4-token group (0..31)
    const int ch0 = cc * 8;
    float mu[8], iv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      mu[j] = v_mean[(size_t)bh * D + ch0 + j];
      iv[j] = v_inv[(size_t)bh * D + ch0 + j];
    }
    float x[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tok0 + 4 * g + r;
      if (tok < N) {
        unpack8(*(const uint4*)(src + (int64_t)tok * sn + ch0), x[r]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float y = (x[r][j] - mu[j]) * iv[j];
          y = fminf(fmaxf(y, -448.0f), 448.0f);
          x[r][j] = (iv[j] == 0.0f) ? 0.0f : y;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[r][j] = 0.0f;
      }
    }
    const int col = 64 * (g >> 4) + v_slot((4 * g) & 63);  // multiple of 4
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      int w = __builtin_amdgcn_cvt_pk_fp8_f32(x[0][j], x[1][j], 0, false);
      w = __builtin_amdgcn_cvt_pk_fp8_f32(x[2][j], x[3][j], w, true);
      const int row = ch0 + j;
      const int chunk = (col >> 4) ^ ((row >> 3) & 7);
      *(uint32_t*)(tile + row * LROW + chunk * 16 + (col & 15)) = (uint32_t)w;
    }
  }
  __syncthreads();
  constexpr int CHUNKS = D * (LROW / 16);
#pragma unroll
  for (int i = 0; i < CHUNKS / kThreads; ++i) {
    const int c = tid + kThreads * i;
    const int row = c >> 3, c16 = c & 7;
    const int colg = tok0 + c16 * 16;
    if (colg < Np) {
      const uint4 val = *(const uint4*)(tile + row * LROW + ((c16 ^ ((row >> 3) & 7)) * 16));
      *(uint4*)(v_fp8 + ((size_t)bh * D + row) * Np + colg) = val;
    }
  }
}

// ---------------------------------------------------------------------------
// The QK RMSNorm + RoPE producer on its own, storing BF16 NHD (report card B):
// grid (ceil(N*H / ROWS), B), 256 threads; a token row (n, h) per D/8 lanes,
// 4 rows per thread, all loads issued before the arithmetic.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void norm_rope_kernel(
    const uint16_t* __restrict__ x, int64_t sb, int64_t sn, int64_t sh, int N, int H,
    const uint16_t* __restrict__ w, const float* __restrict__ rope, double eps,
    uint16_t* __restrict__ y, int64_t y_sb, int64_t y_sn, int64_t y_sh) {
  constexpr int LPR = D / 8;
  constexpr int RPP = kThreads / LPR;
  constexpr int PASSES = 4;
  const int b = blockIdx.y;
  const int tid = threadIdx.x, lr = tid / LPR, lc = tid - lr * LPR;
  const int64_t rows = (int64_t)N * H;
  float w8[8];
  load_w8(w, lc, w8);
  // every lane loads (rows beyond the last read the last row and are not
  // stored), so the producer's cross-lane steps see whole groups
  uint4 v[PASSES];
  float f[PASSES][8], cs[PASSES][8];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t row = min((int64_t)blockIdx.x * (PASSES * RPP) + p * RPP + lr, rows - 1);
    const int64_t n = row / H, h = row - n * H;
    v[p] = *(const uint4*)(x + b * sb + n * sn + h * sh + 8 * lc);
    load_cs8<D>(rope, n, lc, cs[p]);
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) unpack8(v[p], f[p]);
  norm_rope8_rows<LPR, PASSES>(f, w8, cs, eps);
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t row = (int64_t)blockIdx.x * (PASSES * RPP) + p * RPP + lr;
    if (row < rows) {
      const int64_t n = row / H, h = row - n * H;
      uint32_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = bf16x2_rne(f[p][2 * j], f[p][2 * j + 1]);  // exact: bf16 values
      *(uint4*)(y + b * y_sb + n * y_sn + h * y_sh + 8 * lc) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <int D, bool NR>
hipError_t quant_qk_impl(const uint16_t* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                         const uint16_t* k, int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N,
                         int H, int q_block, int k_block, const NormRope& nr, int8_t* q_i8,
                         float* q_scale, int8_t* k_i8, float* k_scale, uint16_t* k_mean, void* ws,
                         hipStream_t stream) {
  const StatsSplit s = stats_split(B, N, H);
  const QkWorkspace w = qk_workspace(B, N, H, D, NR);
  char* wsb = (char*)ws;
  const int Np = (int)padded_tokens(N);
  float* rk = NR ? (float*)(wsb + w.rk_off) : nullptr;
  hipLaunchKernelGGL((stats_kernel<D, false, NR>), dim3(s.nchunk, B * H), dim3(kThreads), 0, stream,
                     k, k_sb, k_sn, k_sh, H, N, s.nchunk, s.rows_per_chunk,
                     (double*)(wsb + w.partial_off), (float*)nullptr, (float*)nullptr, nr.wk,
                     nr.rope, nr.eps, rk, Np);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((finalize_kernel<D, false>), dim3(B * H), dim3(D), 0, stream,
                     (const double*)(wsb + w.partial_off), (const float*)nullptr,
                     (const float*)nullptr, N, s.nchunk, k_mean, (float*)nullptr, (float*)nullptr,
                     (float*)nullptr);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((qk_quant_kernel<D, NR>), dim3(Np / 64, B * H, 2), dim3(kThreads), 0, stream,
                     q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, H, N, Np, (const uint16_t*)k_mean,
                     q_i8, q_scale, k_i8, k_scale, q_block, k_block, nr.wq, nr.wk, nr.rope, nr.eps,
                     (const float*)rk, 0);
  return hipGetLastError();
}

template <int D>
hipError_t quant_v_impl(const uint16_t* v, int64_t v_sb, int64_t v_sn, int64_t v_sh, int B, int N,
                        int H, uint8_t* v_fp8, float* v_scale, float* v_mean, void* ws,
                        hipStream_t stream) {
  const StatsSplit s = stats_split(B, N, H);
  const VWorkspace w = v_workspace(B, N, H, D);
  char* wsb = (char*)ws;
  const int Np = (int)padded_tokens(N);
  float* inv = (float*)(wsb + w.inv_off);
  hipLaunchKernelGGL((stats_kernel<D, true>), dim3(s.nchunk, B * H), dim3(kThreads), 0, stream, v,
                     v_sb, v_sn, v_sh, H, N, s.nchunk, s.rows_per_chunk,
                     (double*)(wsb + w.sum_off), (float*)(wsb + w.min_off),
                     (float*)(wsb + w.max_off), (const uint16_t*)nullptr, (const float*)nullptr, 0.0,
                     (float*)nullptr, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((finalize_kernel<D, true>), dim3(B * H), dim3(D), 0, stream,
                     (const double*)(wsb + w.sum_off), (const float*)(wsb + w.min_off),
                     (const float*)(wsb + w.max_off), N, s.nchunk, (uint16_t*)nullptr, v_mean,
                     v_scale, inv);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((v_quant_kernel<D>), dim3((Np + 127) / 128, B * H), dim3(kThreads), 0, stream,
                     v, v_sb, v_sn, v_sh, H, N, Np, (const float*)v_mean, (const float*)inv, v_fp8);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_qk(const uint16_t* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                           const uint16_t* k, int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N,
                           int H, int D, int q_block, int k_block, const NormRope* nr, int8_t* q_i8,
                           float* q_scale, int8_t* k_i8, float* k_scale, uint16_t* k_mean,
                           void* workspace, hipStream_t stream) {
  const NormRope none{nullptr, nullptr, nullptr, 0.0};
#define SAGE_QK_IMPL(DD, NRR)                                                                    \
  quant_qk_impl<DD, NRR>(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N, H, q_block, k_block,     \
                         nr ? *nr : none, q_i8, q_scale, k_i8, k_scale, k_mean, workspace, stream)
  if (D == 128) return nr ? SAGE_QK_IMPL(128, true) : SAGE_QK_IMPL(128, false);
  return nr ? SAGE_QK_IMPL(64, true) : SAGE_QK_IMPL(64, false);
#undef SAGE_QK_IMPL
}

hipError_t launch_quant_q(const uint16_t* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, int B, int N,
                          int H, int D, int q_block, int8_t* q_i8, float* q_scale,
                          hipStream_t stream) {
  const int Np = (int)padded_tokens(N);
#define SAGE_Q_ONLY(DD)                                                                          \
  hipLaunchKernelGGL((qk_quant_kernel<DD, false>), dim3(Np / 64, B * H, 1), dim3(kThreads), 0,     \
                     stream, q, q_sb, q_sn, q_sh, (const uint16_t*)nullptr, (int64_t)0, (int64_t)0,  \
                     (int64_t)0, H, N, Np, (const uint16_t*)nullptr, q_i8, q_scale, (int8_t*)nullptr, \
                     (float*)nullptr, q_block, 64, (const uint16_t*)nullptr,                         \
                     (const uint16_t*)nullptr, (const float*)nullptr, 0.0, (const float*)nullptr, 1)
  if (D == 128) SAGE_Q_ONLY(128);
  else SAGE_Q_ONLY(64);
#undef SAGE_Q_ONLY
  return hipGetLastError();
}

hipError_t launch_norm_rope(const uint16_t* x, int64_t sb, int64_t sn, int64_t sh, int B, int N,
                            int H, int D, const uint16_t* w, const float* rope, double eps,
                            uint16_t* y, int64_t y_sb, int64_t y_sn, int64_t y_sh,
                            hipStream_t stream) {
  const int64_t rows = (int64_t)N * H;
  if (D == 128) {
    constexpr int ROWS = 4 * (kThreads / 16);
    hipLaunchKernelGGL((norm_rope_kernel<128>), dim3((unsigned)ceil_div(rows, ROWS), B),
                       dim3(kThreads), 0, stream, x, sb, sn, sh, N, H, w, rope, eps, y, y_sb, y_sn,
                       y_sh);
  } else {
    constexpr int ROWS = 4 * (kThreads / 8);
    hipLaunchKernelGGL((norm_rope_kernel<64>), dim3((unsigned)ceil_div(rows, ROWS), B),
                       dim3(kThreads), 0, stream, x, sb, sn, sh, N, H, w, rope, eps, y, y_sb, y_sn,
                       y_sh);
  }
  return hipGetLastError();
}

hipError_t launch_quant_v(const uint16_t* v, int64_t v_sb, int64_t v_sn, int64_t v_sh, int B, int N,
                          int H, int D, uint8_t* v_fp8, float* v_scale, float* v_mean,
                          void* workspace, hipStream_t stream) {
  if (D == 128)
    return quant_v_impl<128>(v, v_sb, v_sn, v_sh, B, N, H, v_fp8, v_scale, v_mean, workspace, stream);
  return quant_v_impl<64>(v, v_sb, v_sn, v_sh, B, N, H, v_fp8, v_scale, v_mean, workspace, stream);
}

}  // namespace sage
