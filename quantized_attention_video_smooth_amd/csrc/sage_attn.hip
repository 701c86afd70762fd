// Fused non-causal attention on INT8 Q/K and FP8 V (gfx950).
//
// Method: "FLUX.3 Action RTX 5090 report", §02 stage 03 (INT8 QK, FP8 PV,
// FP32 accumulation, V smoothing kept) and "MiniMax H3 on DGX Spark", §01
// (QK INT8 / PV FP8).  The pages give no kernel design for this chip; this one
// is built around the CDNA4 32x32 MFMA tiles and the measured cost of the
// softmax on the vector ALU (per 64-key tile a wave issues 512 cycles of MFMA
// but roughly twice that of VALU work):
//
//   * a workgroup = 8 waves (256 queries) or 4 waves (128 queries, two
//     workgroups per CU, chosen when the grid is shallow) of one (b, h); a
//     wave owns 32 queries, which is exactly one Q quantisation block (or,
//     with one Q scale per token, lane l's query has its own scale: free in
//     this layout, where each lane's scores belong to a single query);
//   * the key loop walks 64-key tiles (one K quantisation block, so k_scale is
//     a per-tile scalar; with 16-token K blocks, each 16-key block of a tile
//     lands in a fixed set of 8 accumulator registers per lane, so each set
//     gets its own scalar) through an LDS ring filled with direct global->LDS
//     loads (no VGPR staging) two or three tiles ahead, in an XOR-swizzled layout that
//     keeps the MFMA operand reads free of bank conflicts;
//   * S^T = K Q^T with v_mfma_i32_32x32x32_i8 (exact int32).  In that layout
//     lane l holds 32 scores of query l%32, so the row max, the exponentials
//     and the row sum are lane-local except for one exchange between the two
//     32-lane halves (v_permlane32_swap);
//   * the probabilities are converted to E4M3 in registers (v_cvt_pk_fp8_f32)
//     and used directly as the B operand of O^T = V^T P^T with
//     v_mfma_f32_32x32x64_f8f6f4; V is stored with the slot permutation that
//     makes those bytes line up (sage_v_slot in sage.h);
//   * software pipelining: S^T of tile t+1 is issued to the matrix cores before
//     the softmax of tile t runs on the vector ALU, so the two overlap within
//     a wave and across the two waves that share each SIMD; the P.V of tile t
//     is deferred to the next step and all 12 MFMAs of a step are spread
//     through its softmax instructions;
//   * exp2 with log2(e) and the static P scale 448 folded into one FMA; the
//     accumulator rescale is skipped when no row max moved.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "sage_device.h"
#include "sage_internal.h"

namespace sage {

// Workgroup size forced for benchmark comparisons (process-wide; 0 = chosen
// per launch by attn_waves).
static std::atomic<int> g_attn_waves{0};
void set_attn_waves(int waves) { g_attn_waves.store(waves, std::memory_order_relaxed); }
// Key-step schedule forced for benchmark comparisons (0 = the default).
static std::atomic<int> g_attn_sched{0};
void set_attn_schedule(int schedule) { g_attn_sched.store(schedule, std::memory_order_relaxed); }
// 0: the compiler's order, 1: interleaved (the default)
static int attn_schedule() { return g_attn_sched.load(std::memory_order_relaxed) == 1 ? 0 : 1; }

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// s_waitcnt immediates (gfx9 encoding: vmcnt[3:0] and [15:14], expcnt[6:4],
// lgkmcnt[11:8]; a field at its maximum does not wait).
constexpr int kWaitAll = 0;
template <int VM>
constexpr int kWaitLgkm0VmCpt = (VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14);
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448)

// NW waves per workgroup.  Eight waves (256 queries) share each K/V tile in
// LDS best on long grids; four waves (128 queries, two workgroups per CU)
// give finer load balance when the grid is only a few workgroups per CU deep.
template <int D, int NW_>
struct AttnCfg {
  static constexpr int NW = NW_;             // waves per workgroup
  static constexpr int NT = NW * 64;         // threads per workgroup
  static constexpr int QT = NW * 32;         // queries per workgroup
  static constexpr int DC = D / 32;          // 32-wide d chunks
  static constexpr int JN = D / 16;          // 16-byte chunks per K row
  static constexpr int KCH = 64 * JN;        // 16-byte chunks per K tile
  static constexpr int VCH = D * 4;          // 16-byte chunks per V^T tile (64 bytes per row)
  static constexpr int KBYTES = KCH * 16;
  static constexpr int STAGE = (KCH + VCH) * 16;
  // tiles loaded ahead of the one in softmax: two workgroups per CU keep
  // three in flight within the same LDS budget per CU
  static constexpr int AHEAD = NW == 8 ? 2 : 3;
  static constexpr int NBUF = 4;                 // LDS ring depth (>= AHEAD + 1; a power of two)
  static constexpr int CPT = (KCH + VCH) / NT;  // direct-load instructions per wave per tile
  static_assert(CPT * NT == KCH + VCH, "tile copy must split evenly");
};

// LDS chunk position (16-byte units) of K row r, chunk j, and of V^T row d,
// chunk c.  Unpadded rows with the chunk index XOR-swizzled by the row, so that
// the 16 lanes of each ds_read_b128 pass (16 consecutive rows, one chunk
// column) hit 16 distinct 16-byte bank groups.
template <int JN>
__device__ __forceinline__ int k_pos(int r, int j) { return JN * r + (j ^ ((r / (16 / JN)) % JN)); }
__device__ __forceinline__ int v_pos(int d, int c) { return 4 * d + (c ^ ((d >> 2) & 3)); }

// max / sum across the two 32-lane halves of a wave (lanes l and l^32).
__device__ __forceinline__ int xhalf_max(int v) {
  auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)r[0], (int)r[1]);
}
__device__ __forceinline__ float xhalf_maxf(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return fmaxf(__int_as_float(r[0]), __int_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// KB: K quantisation block (64: one scale per key tile; 16: four per tile).
// SCH: instruction schedule of a key step.  0: the compiler's own order;
// 1: in the steady main loop, O^T += V^T P^T of the previous tile is issued at
// the start of the step, and the step's 12 MFMAs are spread through the
// softmax's vector instructions (sched_group_barrier), so that one wave alone
// keeps the matrix cores busy in the shadow of its VALU work.  Schedule 1
// keeps the ring two tiles ahead, so the previous tile's slot is still intact
// during the step and its V^T operands are read there again instead of being
// held in registers.  Both schedules perform the same operations on the same
// values in the same order per accumulator, so their outputs are identical.
template <int D, int NW, int KB, int SCH>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attn_fwd_kernel(
    const int8_t* __restrict__ q_i8, const float* __restrict__ q_scale,
    const int8_t* __restrict__ k_i8, const float* __restrict__ k_scale,
    const uint8_t* __restrict__ v_fp8, const float* __restrict__ v_scale,
    const float* __restrict__ v_mean, int H, int Nq, int Npq, int Nk, int Npk, int n_qtiles,
    int total_tiles,
    int q_block, float cq0, uint16_t* __restrict__ out, int64_t o_sb, int64_t o_sn, int64_t o_sh) {
  using C = AttnCfg<D, NW>;
  // tiles loaded ahead of the one in softmax (schedule 1 reads the slot of the
  // previous tile during a step, so at most NBUF - 2 ahead)
  constexpr int AHEAD = SCH == 1 ? 2 : C::AHEAD;
  static_assert(SCH != 1 || AHEAD + 2 <= C::NBUF, "schedule 1 re-reads the previous tile's slot");
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::NBUF * C::STAGE];

  // XCD-aware mapping: workgroup i runs on XCD i % 8; give each XCD a
  // contiguous run of (head, q-tile) work so a head's K/V stay in one L2.
  const int per_xcd = gridDim.x / 8;
  const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (logical >= total_tiles) return;  // whole workgroup exits before any barrier
  const int bh = logical / n_qtiles, qt = logical - bh * n_qtiles;
  const int b = bh / H, h = bh - b * H;

  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform values kept in scalar registers (so the tile index, the
  // k_scale loads and the phase branches are scalar)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = lane >> 5, l32 = lane & 31;
  const int q0 = qt * C::QT + wave * 32;
  const int ntiles = Npk / 64;

  // Q^T operand (B of the S^T MFMA): lane holds query q0+l32, d = 32*dc + 16*half .. +16.
  v4i qop[C::DC];
  float cq = 0.0f;
  if (q0 < Npq) {
    const int8_t* qp = q_i8 + ((size_t)bh * Npq + q0 + l32) * D + 16 * half;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) qop[dc] = *(const v4i*)(qp + 32 * dc);
    // the scale of this lane's query: one per 32-query block (the whole
    // wave) or one per query (q_block == 1)
    cq = q_scale[(size_t)bh * (Npq / q_block) + (q0 + l32) / q_block] * cq0;
  } else {
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) qop[dc] = v4i{0, 0, 0, 0};
  }

  const int8_t* kbase = k_i8 + (size_t)bh * Npk * D;
  const uint8_t* vbase = v_fp8 + (size_t)bh * D * Npk;
  static_assert(KB == 64 || KB == 16, "K block is 64 or 16 tokens");
  constexpr int KPT = 64 / KB;  // K scales per key tile
  const float* ksc = k_scale + (size_t)bh * ntiles * KPT;

  // ---- global -> LDS staging: direct loads (global_load_lds_dwordx4) ----
  // Instruction i of wave w fills tile chunk positions g = (i*NW + w)*64 + lane
  // (K positions first, then V^T); every lane fetches the global chunk that
  // belongs at its LDS position, so the swizzled layout costs nothing here.
  // Whether a wave's instruction i copies V^T (else K) chunks depends on the
  // wave only (KCH is a multiple of 64), so it is a scalar condition.
  static_assert(C::KCH % 64 == 0, "K chunks must fill whole waves");
  auto is_v = [&](int i) __attribute__((always_inline)) { return (i * C::NW + wave) * 64 >= C::KCH; };
  int goff[C::CPT];  // per-lane global byte offset within a tile (tile term added per load)
#pragma unroll
  for (int i = 0; i < C::CPT; ++i) {
    const int g = (i * C::NW + wave) * 64 + lane;
    if (!is_v(i)) {
      const int r = g / C::JN, jx = g % C::JN;
      const int j = jx ^ ((r / (16 / C::JN)) % C::JN);
      goff[i] = r * D + j * 16;
    } else {
      const int p = g - C::KCH, d = p >> 2, cx = p & 3;
      const int c = cx ^ ((d >> 2) & 3);
      goff[i] = d * Npk + c * 16;
    }
  }
  // Loads address this head's K (Npk*D bytes) and V^T (D*Npk bytes) as buffers:
  // lane offset goff[i], tile offset t*64*D (K) or t*64 (V^T), both below the
  // record count for every t < ntiles.
  auto gload_lds = [&](int t, int sl) __attribute__((always_inline)) {
    uint8_t* slot = smem + sl * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int wbase = (i * C::NW + wave) * 64 * 16;  // this wave's LDS bytes in the slot
      void* dst = slot + wbase;
      if (is_v(i))
        lds_load16(vbase, D * Npk, dst, goff[i], t * 64);
      else
        lds_load16(kbase, Npk * D, dst, goff[i], t * 64 * D);
    }
  };

  v16f acc[C::DC];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[dc][i] = 0.0f;
  float m_run = -__builtin_inff();
  float l_run = 0.0f;
  v8i pop = v8i{0, 0, 0, 0, 0, 0, 0, 0};
  float ksc_cur[KPT];  // k_scale(s) of the tile whose softmax is next
#pragma unroll
  for (int j = 0; j < KPT; ++j) ksc_cur[j] = ksc[j];

  // S^T(t) = K(t) Q^T into sdst (operands read from LDS slot sl = t % NBUF).
  auto qk_mfma = [&](int sl, v16i (&sdst)[2]) __attribute__((always_inline)) {
    const uint8_t* ks = smem + sl * C::STAGE;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sdst[kb] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc) {
        const v4i a = *(const v4i*)(ks + 16 * k_pos<C::JN>(32 * kb + l32, 2 * dc + half));
        sdst[kb] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, qop[dc], sdst[kb], 0, 0, 0);
      }
    }
  };
  // V^T(t) operands from LDS, and O^T += V^T(t) P^T(t).
  auto load_v = [&](int sl, v8i (&vop)[C::DC]) __attribute__((always_inline)) {
    const uint8_t* vs = smem + sl * C::STAGE + C::KBYTES;
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc) {
      const v4i lo = *(const v4i*)(vs + 16 * v_pos(32 * dc + l32, 2 * half));
      const v4i hi = *(const v4i*)(vs + 16 * v_pos(32 * dc + l32, 2 * half + 1));
      vop[dc] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  auto pv_mfma = [&](const v8i (&vop)[C::DC]) __attribute__((always_inline)) {
#pragma unroll
    for (int dc = 0; dc < C::DC; ++dc)
      acc[dc] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop[dc], pop, acc[dc], 0, 0, 0, 0, 0, 0);
  };

  // Softmax of S^T(t) (in scur): row max, P = exp2(s*c - m) * 448 packed to
  // E4M3 (byte 16*kb + i of pop), row sum, accumulator rescale.
  auto softmax = [&](int t, v16i (&scur)[2], auto masked_tag, auto sched_tag) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    // c[j]: score multiplier of K block j of the tile; with KB = 16, block j
    // holds keys 16j..16j+15 = registers 8*(j%2)..+8 of scur[j/2]
    float c[KPT];
#pragma unroll
    for (int j = 0; j < KPT; ++j) c[j] = cq * ksc_cur[j];
    float ksc_next[KPT];  // used by the next tile
    const int tn = min(t + 1, ntiles - 1);
#pragma unroll
    for (int j = 0; j < KPT; ++j) ksc_next[j] = ksc[tn * KPT + j];
    // key index of scur[kb][i] inside the tile: 32*kb + 8*(i/4) + 4*half + i%4
    const int nvalid = Nk - t * 64;  // keys at or beyond nvalid are padding
    if constexpr (MASKED) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = 32 * kb + 8 * (i >> 2) + 4 * half + (i & 3);
          if (key >= nvalid) scur[kb][i] = INT32_MIN;
        }
    }
    float m_tile;
    if constexpr (KPT == 1) {
      int mxi = scur[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mxi = max(mxi, scur[kb][i]);
      m_tile = (float)xhalf_max(mxi) * c[0];
    } else {
      // integer max per 16-key block, then scaled (every multiplier >= 0);
      // a block wholly beyond Nk (scale 0) must not contribute its 0
      m_tile = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int mb = scur[j >> 1][8 * (j & 1)];
#pragma unroll
        for (int i = 1; i < 8; ++i) mb = max(mb, scur[j >> 1][8 * (j & 1) + i]);
        float v = (float)mb * c[j];
        if constexpr (MASKED) {
          if (16 * j >= nvalid) v = -__builtin_inff();
        }
        m_tile = fmaxf(m_tile, v);
      }
      m_tile = xhalf_maxf(m_tile);
    }
    const float m_new = fmaxf(m_run, m_tile);
    const float bias = kLog2_448 - m_new;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * r + e;
          float x = __builtin_amdgcn_exp2f(
              __builtin_fmaf((float)scur[kb][i], c[KPT == 1 ? 0 : 2 * kb + (r >> 1)], bias));
          if constexpr (MASKED) {
            const int key = 32 * kb + 8 * r + 4 * half + e;
            if (key >= nvalid) x = 0.0f;
          }
          p[e] = x;
          lsum += x;
        }
        // the high half is written next, so the old register serves as the
        // untouched half (no zeroing move)
        int w = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], pop[4 * kb + r], false);
        w = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w, true);
        pop[4 * kb + r] = w;
      }
    if constexpr (decltype(sched_tag)::value) {
      // this block holds (in program order) the previous tile's 8 V-operand
      // reads and 4 PV MFMAs, the 8 K-operand reads and 8 S^T MFMAs of the
      // next tile and the softmax up to the rescale branch
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // V operand reads (previous tile)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a PV MFMA (previous tile)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // two K operand reads
        // VALU instructions behind each PV MFMA (measured best: 8 with two
        // workgroups per CU, 12 with one)
        __builtin_amdgcn_sched_group_barrier(0x002, NW == 8 ? 12 : 8, 0);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // an S^T MFMA (next tile)
        if constexpr (NW == 8) {
          // four exp2 right behind it, then other vector instructions
          // (measured ~1% faster with one workgroup per CU, ~0.3% slower
          // with two)
          __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
        }
      }
    }
    // Keep the exponentials and packs in this basic block, ahead of the
    // rescale branch (the compiler would sink them past it): there they
    // share a block with the next tile's S^T MFMAs, and the register
    // allocation of the loop stays free of spills.
#pragma unroll
    for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(pop[i]));
    asm volatile("" : "+v"(lsum));
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if (__any(m_new != m_run)) {  // skip when no row max of this wave moved
      l_run *= alpha;
#pragma unroll
      for (int dc = 0; dc < C::DC; ++dc)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dc][i] *= alpha;
    }
    l_run += lsum;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < KPT; ++j) ksc_cur[j] = ksc_next[j];
  };

  // One tile: start the direct loads of tile t+AHEAD into the ring slot of
  // tile t+AHEAD-NBUF (t-1 or t-2, whose last reads were before the previous
  // barrier; a deferred PV reads the slot of t-1 during the step), issue
  // S^T(t+1) on the matrix cores, run the softmax of tile t on the vector ALU
  // meanwhile, then O^T += V^T(t) P^T(t).  The closing barrier needs this
  // wave's LDS reads drained (the slot of tile t is refilled next step) and the
  // loads of tile t+2 landed (read from the next step on); with AHEAD = 3 the
  // loads of tile t+3 stay in flight across it.  A raw s_barrier is used
  // because __syncthreads() would always wait for every load.
  // next_tag: std::true_type when tile t+1 exists (its S^T MFMAs are issued
  // here, in the same basic block as the softmax, so the two can interleave),
  // std::false_type for the last tile.
  // u: t % NBUF (a compile-time constant in the unrolled main loop)
  // steady_tag: std::true_type when tile t+AHEAD is known to exist, so the
  // refill and its wait need no run-time condition (no branch merging in
  // front of the next step's operand reads and their waits).
  auto step = [&](int t, int u, v16i (&scur)[2], v16i (&snext)[2], v8i (&vcur)[C::DC],
                  v8i (&vprev)[C::DC], auto masked_tag, auto next_tag,
                  auto steady_tag) __attribute__((always_inline)) {
    const bool issue = decltype(steady_tag)::value || t + AHEAD < ntiles;
    // schedule 1 defers the PV of a tile to the next step in the steady main
    // loop only; the steps after it multiply their own tile's PV (after one
    // flush), which keeps the register allocation of that code spill-free
    constexpr bool deferred = SCH == 1 && decltype(steady_tag)::value;
    if constexpr (deferred) {
      // the previous tile, from its slot (zero V^T before tile 0: adds nothing)
      load_v((u + C::NBUF - 1) % C::NBUF, vprev);
      pv_mfma(vprev);
    }
    if (issue) gload_lds(t + AHEAD, (u + AHEAD) % C::NBUF);
    if constexpr (decltype(next_tag)::value) qk_mfma((u + 1) % C::NBUF, snext);
    if constexpr (!deferred) load_v(u, vcur);
    constexpr bool sched = deferred && decltype(next_tag)::value && !decltype(masked_tag)::value;
    softmax(t, scur, masked_tag, std::integral_constant<bool, sched>{});
    if constexpr (!deferred) pv_mfma(vcur);
    if (issue && AHEAD > 2) __builtin_amdgcn_s_waitcnt(kWaitLgkm0VmCpt<C::CPT>);
    else __builtin_amdgcn_s_waitcnt(kWaitAll);
    __asm__ volatile("s_barrier" ::: "memory");
  };

  // ---- prologue: tiles 0 .. AHEAD-1 in LDS, S^T(0) issued ----
#pragma unroll
  for (int i = 0; i < AHEAD; ++i)
    if (i < ntiles) gload_lds(i, i);
  if constexpr (SCH == 1) {
    // V^T region of the last slot, read as "the previous tile" by tile 0
    uint4* z = (uint4*)(smem + (C::NBUF - 1) * C::STAGE + C::KBYTES);
    for (int i = tid; i < C::VCH; i += C::NT) z[i] = make_uint4(0, 0, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(kWaitAll);
  __syncthreads();
  v16i sA[2], sB[2];
  qk_mfma(0, sA);
  // V^T operand registers of the even / odd tiles (every read fills them
  // before its MFMAs)
  v8i vA[C::DC], vB[C::DC];
#pragma unroll
  for (int dc = 0; dc < C::DC; ++dc) vA[dc] = vB[dc] = v8i{0, 0, 0, 0, 0, 0, 0, 0};

  // ---- key loop ----
  // Main loop: groups of four tiles followed by at least one more tile (all
  // such tiles are full: only the last tile can hold padding), unrolled by the
  // ring depth so that every step's LDS slot is a constant (the slot base
  // becomes an instruction offset instead of a per-read address add) and the
  // S buffers alternate statically.  Then pairs, then one or two last tiles;
  // the last of them is padded when Nk % 64 != 0.
  const int nfull = Nk / 64;  // tiles without padding keys
  int t = 0;
  // unrolled by the ring depth: the slot of every step is a constant
  const std::false_type no{};
  const std::true_type yes{};
  for (; t + 3 + AHEAD < ntiles; t += 4) {  // every step of the group refills the ring
    step(t, 0, sA, sB, vA, vB, no, yes, yes);
    step(t + 1, 1, sB, sA, vB, vA, no, yes, yes);
    step(t + 2, 2, sA, sB, vA, vB, no, yes, yes);
    step(t + 3, 3, sB, sA, vB, vA, no, yes, yes);
  }
  if constexpr (SCH == 1) {
    if (t > 0) {  // the main loop ran: its last tile's PV is still pending
      load_v((t + C::NBUF - 1) % C::NBUF, vB);
      pv_mfma(vB);
    }
  }
  for (; t + 4 < ntiles; t += 4) {
    step(t, 0, sA, sB, vA, vB, no, yes, no);
    step(t + 1, 1, sB, sA, vB, vA, no, yes, no);
    step(t + 2, 2, sA, sB, vA, vB, no, yes, no);
    step(t + 3, 3, sB, sA, vB, vA, no, yes, no);
  }
  for (; t + 2 < ntiles; t += 2) {
    step(t, t % C::NBUF, sA, sB, vA, vB, no, yes, no);
    step(t + 1, (t + 1) % C::NBUF, sB, sA, vB, vA, no, yes, no);
  }
  auto last_step = [&](int t, v16i (&scur)[2], v16i (&snext)[2], v8i (&vcur)[C::DC],
                       v8i (&vprev)[C::DC]) __attribute__((always_inline)) {
    if (t < nfull) step(t, t % C::NBUF, scur, snext, vcur, vprev, no, no, no);
    else step(t, t % C::NBUF, scur, snext, vcur, vprev, yes, no, no);
  };
  // t is even here: S^T(t) is in sA, its V^T operands go to vA
  if (t + 1 < ntiles) {
    step(t, t % C::NBUF, sA, sB, vA, vB, no, yes, no);
    last_step(t + 1, sB, sA, vB, vA);
  } else {
    last_step(t, sA, sB, vA, vB);
  }

  // ---- epilogue: O = acc / (448 * l) * v_scale + v_mean, bf16 NHD ----
  const float l_tot = xhalf_sum(l_run);
  const float inv_l = 1.0f / l_tot;
  const int qi = q0 + l32;
  if (qi < Nq) {
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
}

template <int D, int NW, int KB, int SCH>
hipError_t attn_launch(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                       const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                       const float* v_mean, int B, int Nq, int Nk, int H, int q_block,
                       float sm_scale, uint16_t* out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
                       hipStream_t stream) {
  using C = AttnCfg<D, NW>;
  const int Npq = (int)padded_tokens(Nq), Npk = (int)padded_tokens(Nk);
  const int n_qtiles = (int)ceil_div(Nq, C::QT);
  const int total = B * H * n_qtiles;
  const int grid = (int)ceil_div(total, 8) * 8;
  const float cq0 = sm_scale * kLog2e;
  hipLaunchKernelGGL((attn_fwd_kernel<D, NW, KB, SCH>), dim3(grid), dim3(C::NT), 0, stream, q_i8, q_scale,
                     k_i8, k_scale, v_fp8, v_scale, v_mean, H, Nq, Npq, Nk, Npk, n_qtiles, total,
                     q_block, cq0,
                     out, o_sb, o_sn, o_sh);
  return hipGetLastError();
}

// Eight-wave workgroups when the grid is at least 8 of them per CU deep,
// else four-wave ones (measured on MI355X: FLUX-sized grids of ~3.4 per CU
// run ~20% faster with four waves, 20-deep grids ~1% slower).  N: queries.
int attn_waves(int B, int N, int H) {
  static std::atomic<int> ncu_cache{0};
  int ncu = ncu_cache.load(std::memory_order_relaxed);
  if (ncu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        ncu <= 0)
      ncu = 256;
    ncu_cache.store(ncu, std::memory_order_relaxed);
  }
  const int forced = g_attn_waves.load(std::memory_order_relaxed);
  if (forced == 4 || forced == 8) return forced;
  const int64_t wg8 = (int64_t)B * H * ceil_div(N, 256);
  return wg8 >= 8 * (int64_t)ncu ? 8 : 4;
}

template <int D, int KB>
hipError_t attn_impl(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                     const float* v_mean, int B, int Nq, int Nk, int H, int q_block,
                     float sm_scale, uint16_t* out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
                     hipStream_t stream) {
#define SAGE_ATTN_LAUNCH(NWW, SCHH)                                                               \
  attn_launch<D, NWW, KB, SCHH>(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, B, Nq, Nk, H, \
                                q_block, sm_scale, out, o_sb, o_sn, o_sh, stream)
  const bool interleaved = attn_schedule() == 1;
  if (attn_waves(B, Nq, H) == 8) return interleaved ? SAGE_ATTN_LAUNCH(8, 1) : SAGE_ATTN_LAUNCH(8, 0);
  return interleaved ? SAGE_ATTN_LAUNCH(4, 1) : SAGE_ATTN_LAUNCH(4, 0);
#undef SAGE_ATTN_LAUNCH
}

}  // namespace

void attn_shape(int B, int N, int H, int D, int* waves, int* workgroups) {
  (void)D;
  const int nw = attn_waves(B, N, H);
  *waves = nw;
  *workgroups = (int)(ceil_div((int64_t)B * H * ceil_div(N, 32 * nw), 8) * 8);
}

hipError_t launch_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                           const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                           const float* v_mean, int B, int Nq, int Nk, int H, int D, int q_block,
                           int k_block, float sm_scale, uint16_t* out, int64_t o_sb, int64_t o_sn,
                           int64_t o_sh, hipStream_t stream) {
#define SAGE_ATTN_IMPL(DD, KK)                                                                    \
  attn_impl<DD, KK>(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, B, Nq, Nk, H, q_block, \
                    sm_scale, out, o_sb, o_sn, o_sh, stream)
  if (D == 128) return k_block == 16 ? SAGE_ATTN_IMPL(128, 16) : SAGE_ATTN_IMPL(128, 64);
  return k_block == 16 ? SAGE_ATTN_IMPL(64, 16) : SAGE_ATTN_IMPL(64, 64);
#undef SAGE_ATTN_IMPL
}

}  // namespace sage
