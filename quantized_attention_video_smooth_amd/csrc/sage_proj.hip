// Row-wise FP8 projections of libsage (gfx950): per-row E4M3 quantisation of
// activations (one scale per token) and weights (one scale per output row),
// and the scaled FP8 GEMM on them.
//
// Method: "FLUX.3 Action RTX 5090 report", §02 stage 02 (mixed-precision
// projections: Q/K projections stay BF16, the other selected projections run
// in row-wise FP8) and the "FLUX 3 Action" SGLang page's latency notes (E4M3
// weights with one scale per output row, per-token activation scales, a scaled
// FP8 GEMM with fp32 accumulation).  The rows are quantised with the rule of
// the V quantiser (E4M3 layout per "Why can an A10 run FLUX.1", §1.1).
//
// The GEMM computes out^T = W X^T with v_mfma_f32_32x32x64_f8f6f4: a W tile
// of 32 output rows is the A operand and an X tile of 32 tokens the B operand,
// so a lane's accumulators hold 4 consecutive outputs n of one token m per
// register group (8-byte bf16 stores in the epilogue).  A workgroup of 8
// waves computes a 256 (n) x 256 (m) block; each wave a 128 x 64 part of it
// (8 accumulator tiles).  K advances in 64-byte steps through a four-slot LDS
// ring, three stages ahead, filled by direct global->LDS loads, with the
// 16-byte chunks of each row XOR-swizzled so the operand reads are free of
// bank conflicts.  The bf16 output block is staged in the same LDS and
// written out in whole 512-byte rows.
#include <hip/hip_runtime.h>

#include "sage_device.h"
#include "sage_internal.h"

namespace sage {

namespace {

// ---------------------------------------------------------------------------
// Row quantisation: one wave per row, 4 rows per workgroup.  A lane holds up
// to P 8-element chunks of its row (chunk c = lane + 64 p) in registers, so
// the row is read once; a = max |x| over the row (wave reduction);
// code = E4M3(fp32(x) * (448 / a)) (round to nearest even, saturating);
// scale = a / 448; a == 0 or 448 / a not finite gives scale 0 and codes 0.
// ---------------------------------------------------------------------------
template <int P>
__global__ __launch_bounds__(kThreads) void rowq_kernel(const uint16_t* __restrict__ x, int64_t ldx,
                                                        int M, int K, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  const int lane = threadIdx.x & 63;
  const int m = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (m >= M) return;  // whole wave
  const uint16_t* row = x + (int64_t)m * ldx;
  const int nch = K / 8;
  uint4 raw[P];
  float a = 0.0f;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int c = lane + 64 * p;
    if (c < nch) {
      raw[p] = *(const uint4*)(row + 8 * c);
      float f[8];
      unpack8(raw[p], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[j]));
    }
  }
  a = wave_max(a);
  const float iv = 448.0f / a;
  const bool zero = (a == 0.0f) || !__builtin_isfinite(iv);
  const float inv = zero ? 0.0f : iv;
  uint8_t* out = codes + (int64_t)m * K;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int c = lane + 64 * p;
    if (c < nch) {
      float f[8];
      unpack8(raw[p], f);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = fminf(fmaxf(f[j] * inv, -448.0f), 448.0f);
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], w1, true);
      *(uint2*)(out + 8 * c) = make_uint2((uint32_t)w0, (uint32_t)w1);
    }
  }
  if (lane == 0) scales[m] = zero ? 0.0f : a / 448.0f;
}

// ---------------------------------------------------------------------------
// Scaled FP8 GEMM.
// ---------------------------------------------------------------------------
struct GemmCfg {
  static constexpr int NW = 8;           // waves
  static constexpr int NT = NW * 64;     // threads
  static constexpr int BN = 256;         // output rows n per workgroup (W rows)
  static constexpr int BM = 256;         // tokens m per workgroup (X rows)
  static constexpr int BK = 64;          // bytes of K per stage (one MFMA k-step)
  static constexpr int NBUF = 4;         // LDS ring depth (= stages in flight, see the loop)
  static constexpr int JN = BK / 16;     // 16-byte chunks per tile row
  static constexpr int ACH = BN * JN;    // chunks of the W tile
  static constexpr int BCH = BM * JN;    // chunks of the X tile
  static constexpr int STAGE = (ACH + BCH) * 16;
  static constexpr int CPT = (ACH + BCH) / NT;  // direct-load instructions per wave per stage
  static constexpr int WN = 128, WM = 64;       // wave tile
  static constexpr int TN = WN / 32, TM = WM / 32;
  static_assert(CPT * NT == ACH + BCH && ACH % NT == 0, "stage copy must split evenly");
};

// LDS chunk position of row r, chunk j: rows of JN = 4 chunks (64 bytes),
// chunk index XOR-swizzled by the row so that the 16 lanes of a ds_read_b128
// pass (16 consecutive rows, one logical chunk) hit 16 distinct 16-byte bank
// groups of the 256-byte bank row: 4 (r % 4) + (j ^ ((r / 4) % 4)) is
// distinct over any 16 consecutive rows.
__device__ __forceinline__ int gk_pos(int r, int j) { return 4 * r + (j ^ ((r >> 2) & 3)); }

__global__ __launch_bounds__(GemmCfg::NT, 1) void gemm_fp8_kernel(
    const uint8_t* __restrict__ x8, const float* __restrict__ sx, int M,
    const uint8_t* __restrict__ w8, const float* __restrict__ sw, int N, int K,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ out, int64_t ldo, int n_mblk,
    int total, int vec16) {
  using C = GemmCfg;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::NBUF * C::STAGE];

  // XCD-aware, grouped order.  Workgroup i runs on XCD i % 8: each XCD gets a
  // contiguous run of logical blocks, and within it the ~32 workgroups that run
  // at once (one per CU) form GN n-blocks x 32/GN m-blocks, walking through K
  // roughly together: each K slice they need comes from GN W blocks and 32/GN
  // X blocks (12 for GN = 8) rather than from 1 W and 32 X blocks, so most
  // requests hit the XCD's L2 instead of going to the memory-side cache.
  constexpr int GN = 8;
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total) return;  // whole workgroup, before any barrier
  const int n_nblk = total / n_mblk;
  const int grp = logical / (GN * n_mblk);
  const int first_nb = grp * GN;
  const int gsize = min(n_nblk - first_nb, GN);
  const int in_grp = logical - grp * GN * n_mblk;
  const int nb = first_nb + in_grp % gsize, mb = in_grp / gsize;
  const int n_base = nb * C::BN, m_base = mb * C::BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int wn = wave & 1, wm = wave >> 1;  // 2 x 4 waves
  const int n0 = wn * C::WN, m0 = wm * C::WM;

  // direct-load sources: instruction i of wave w fills chunk positions
  // g = (i * NW + w) * 64 + lane of the stage; the first ACH are the W tile,
  // the rest the X tile.  Rows beyond N or M read the last row (not stored).
  int64_t goff[C::CPT];
  bool is_x[C::CPT];
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int g = (i * C::NW + wave) * 64 + lane;
    const bool xb = g >= C::ACH;
    const int gg = xb ? g - C::ACH : g;
    const int r = gg / C::JN, jx = gg % C::JN;
    const int j = jx ^ ((r >> 2) & 3);
    if (!xb) goff[i] = (int64_t)min(n_base + r, N - 1) * K + 16 * j;
    else goff[i] = (int64_t)min(m_base + r, M - 1) * K + 16 * j;
    is_x[i] = xb;
  }
  auto load_stage = [&](int t) __attribute__((always_inline)) {
    uint8_t* slot = smem + (t % C::NBUF) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const uint8_t* src = (is_x[i] ? x8 : w8) + goff[i] + (int64_t)t * C::BK;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)src,
                                       (__attribute__((address_space(3))) void*)(slot + (i * C::NW + wave) * 1024),
                                       16, 0, 0);
    }
  };

  v16f acc[C::TN][C::TM];
#pragma unroll
  for (int a = 0; a < C::TN; ++a)
#pragma unroll
    for (int b = 0; b < C::TM; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.0f;

  // Software pipeline.  While the MFMAs of tile t run, the wave's LDS reads of
  // tile t+1 fill the other fragment buffer.  At stage t each wave waits for
  // its own direct loads of tile t+1 (vmcnt, leaving the two later tiles in
  // flight) and for its LDS reads of tile t (lgkmcnt 0), then a raw s_barrier
  // (compiler memory clobber) publishes tile t+1 and certifies that no wave
  // still reads tile t's slot, which the loads of tile t+NBUF then refill.
  // __syncthreads() would also wait for the loads still in flight.
  auto read_frags = [&](int t, v8i (&af)[C::TN], v8i (&bf)[C::TM]) __attribute__((always_inline)) {
    const uint8_t* wt = smem + (t % C::NBUF) * C::STAGE;
    const uint8_t* xt = wt + C::ACH * 16;
#pragma unroll
    for (int a = 0; a < C::TN; ++a) {
      const int r = n0 + 32 * a + l32;
      const v4i lo = *(const v4i*)(wt + 16 * gk_pos(r, 2 * half));
      const v4i hi = *(const v4i*)(wt + 16 * gk_pos(r, 2 * half + 1));
      af[a] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int b = 0; b < C::TM; ++b) {
      const int r = m0 + 32 * b + l32;
      const v4i lo = *(const v4i*)(xt + 16 * gk_pos(r, 2 * half));
      const v4i hi = *(const v4i*)(xt + 16 * gk_pos(r, 2 * half + 1));
      bf[b] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto mfmas = [&](const v8i (&af)[C::TN], const v8i (&bf)[C::TM]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < C::TN; ++a)
#pragma unroll
      for (int b = 0; b < C::TM; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[a], bf[b], acc[a][b], 0, 0, 0,
                                                                   0, 0, 0);
  };
  constexpr int WAIT2 = (2 * C::CPT & 15) | (7 << 4) | (0 << 8) | ((2 * C::CPT >> 4) << 14);
  constexpr int WAIT3 = (3 * C::CPT & 15) | (7 << 4) | (0 << 8) | ((3 * C::CPT >> 4) << 14);
  const int nk = K / C::BK;
#pragma unroll
  for (int i = 0; i < C::NBUF; ++i)
    if (i < nk) load_stage(i);
  if (nk >= C::NBUF) __builtin_amdgcn_s_waitcnt(WAIT3);
  else __builtin_amdgcn_s_waitcnt(0);
  __asm__ volatile("s_barrier" ::: "memory");
  v8i afA[C::TN], bfA[C::TM], afB[C::TN], bfB[C::TM];
  read_frags(0, afA, bfA);
  // one stage; cur holds tile t's fragments, nxt receives tile t+1's
  auto stage = [&](int t, const v8i (&af)[C::TN], const v8i (&bf)[C::TM], v8i (&an)[C::TN],
                   v8i (&bn)[C::TM]) __attribute__((always_inline)) {
    if (t + 1 < nk) {
      // loads issued so far: tiles <= t + NBUF - 1; tile t+1 must have landed
      if (t + 3 < nk) __builtin_amdgcn_s_waitcnt(WAIT2);
      else __builtin_amdgcn_s_waitcnt(0);
      __asm__ volatile("s_barrier" ::: "memory");
      if (t + C::NBUF < nk) load_stage(t + C::NBUF);
      read_frags(t + 1, an, bn);
    }
    mfmas(af, bf);
  };
  // The same stage for the steady state, with no conditions: tile t+1 and
  // tile t+NBUF exist.  Kept free of branches so the compiler's wait counting
  // sees that this stage's MFMAs need only the fragments read one stage ago
  // (the explicit wait at its start), not the reads of tile t+1 it has just
  // issued; with a branch merging in front of the MFMAs it waits for all LDS
  // reads there, which serialises the next tile's reads with this tile's MFMAs.
  auto stage_steady = [&](int t, const v8i (&af)[C::TN], const v8i (&bf)[C::TM], v8i (&an)[C::TN],
                          v8i (&bn)[C::TM]) __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(WAIT2);
    __asm__ volatile("s_barrier" ::: "memory");
    load_stage(t + C::NBUF);
    read_frags(t + 1, an, bn);
    __builtin_amdgcn_sched_barrier(0);  // keep the reads of tile t+1 ahead of tile t's MFMAs
    mfmas(af, bf);
    __builtin_amdgcn_sched_barrier(0);
  };
  int t = 0;
  for (; t + C::NBUF + 1 < nk; t += 2) {  // stages t and t+1 both load a tile NBUF ahead
    stage_steady(t, afA, bfA, afB, bfB);
    stage_steady(t + 1, afB, bfB, afA, bfA);
  }
  for (; t + 1 < nk; t += 2) {
    stage(t, afA, bfA, afB, bfB);
    stage(t + 1, afB, bfB, afA, bfA);
  }
  if (t < nk) stage(t, afA, bfA, afB, bfB);

  // ---- epilogue: out[m][n] = bf16((acc * sx[m]) * sw[n] + bias[n]) ----
  // accumulator register i of tile (a, b): n = n0 + 32 a + 8 (i / 4) + 4 half + i % 4,
  // m = m0 + 32 b + l32.  The bf16 block goes through LDS (the ring is free
  // once every wave's last operand reads are consumed): row m_loc, 16-byte
  // chunk c of its 512 bytes at chunk position c ^ (m_loc % 32), so the 32
  // rows one store instruction touches and the 32 chunks one read touches
  // spread over the banks.  It then leaves in whole rows: 32 lanes x 16 bytes
  // per row.
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ volatile("s_barrier" ::: "memory");
  constexpr int ROWB = C::BN * 2;  // bytes of one block row
  static_assert(C::BM * ROWB <= C::NBUF * C::STAGE, "output block must fit the LDS ring");
#pragma unroll
  for (int b = 0; b < C::TM; ++b) {
    const int m_loc = m0 + 32 * b + l32;
    const int m = m_base + m_loc;
    const float sxm = m < M ? sx[m] : 0.0f;
    uint8_t* lrow = smem + m_loc * ROWB;
#pragma unroll
    for (int a = 0; a < C::TN; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n_loc = n0 + 32 * a + 8 * g + 4 * half;
        const int n = n_base + n_loc;
        if (n >= N) continue;  // N % 4 == 0: a group is all in or all out; never stored
        const float4 s4 = *(const float4*)(sw + n);
        float y[4];
        y[0] = acc[a][b][4 * g + 0] * sxm * s4.x;
        y[1] = acc[a][b][4 * g + 1] * sxm * s4.y;
        y[2] = acc[a][b][4 * g + 2] * sxm * s4.z;
        y[3] = acc[a][b][4 * g + 3] * sxm * s4.w;
        if (bias) {
          const uint2 bb = *(const uint2*)(bias + n);
          y[0] += bf16_lo(bb.x);
          y[1] += bf16_hi(bb.x);
          y[2] += bf16_lo(bb.y);
          y[3] += bf16_hi(bb.y);
        }
        const int chunk = n_loc >> 3;
        *(uint2*)(lrow + 16 * (chunk ^ (m_loc & 31)) + 8 * half) =
            make_uint2(bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3]));
      }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __asm__ volatile("s_barrier" ::: "memory");
  constexpr int CPR = ROWB / 16;  // 16-byte chunks per block row
#pragma unroll 4
  for (int idx = tid; idx < C::BM * CPR; idx += C::NT) {
    const int r = idx / CPR, c = idx % CPR;
    const int m = m_base + r, n = n_base + 8 * c;
    if (m >= M || n >= N) continue;
    const uint4 v = *(const uint4*)(smem + r * ROWB + 16 * (c ^ (r & 31)));
    uint16_t* dst = out + (int64_t)m * ldo + n;
    if (vec16 && n + 8 <= N) {
      *(uint4*)dst = v;
    } else {
      *(uint2*)dst = make_uint2(v.x, v.y);
      if (n + 4 < N) *(uint2*)(dst + 4) = make_uint2(v.z, v.w);
    }
  }
}

}  // namespace

hipError_t launch_quant_rows_fp8(const uint16_t* x, int64_t ldx, int M, int K, uint8_t* codes,
                                 float* scales, hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div(M, kThreads / 64));
  const int per_lane = (int)ceil_div(K / 8, 64);
#define SAGE_ROWQ(PP)                                                                            \
  hipLaunchKernelGGL((rowq_kernel<PP>), grid, dim3(kThreads), 0, stream, x, ldx, M, K, codes, scales)
  if (per_lane <= 2) SAGE_ROWQ(2);
  else if (per_lane <= 4) SAGE_ROWQ(4);
  else if (per_lane <= 8) SAGE_ROWQ(8);
  else if (per_lane <= 16) SAGE_ROWQ(16);
  else SAGE_ROWQ(32);
#undef SAGE_ROWQ
  return hipGetLastError();
}

void gemm_fp8_shape(int M, int N, int* workgroups) {
  const int64_t tiles = ceil_div(M, GemmCfg::BM) * ceil_div(N, GemmCfg::BN);
  *workgroups = (int)(ceil_div(tiles, 8) * 8);
}

hipError_t launch_gemm_fp8_rowwise(const uint8_t* x8, const float* sx, int M, const uint8_t* w8,
                                   const float* sw, int N, int K, const uint16_t* bias,
                                   uint16_t* out, int64_t ldo, hipStream_t stream) {
  int grid;
  gemm_fp8_shape(M, N, &grid);
  const int n_mblk = (int)ceil_div(M, GemmCfg::BM);
  const int total = n_mblk * (int)ceil_div(N, GemmCfg::BN);
  hipLaunchKernelGGL(gemm_fp8_kernel, dim3(grid), dim3(GemmCfg::NT), 0, stream, x8, sx, M, w8, sw,
                     N, K, bias, out, ldo, n_mblk, total,
                     (int)(((uintptr_t)out % 16 == 0) && (ldo % 8 == 0)));
  return hipGetLastError();
}

}  // namespace sage
