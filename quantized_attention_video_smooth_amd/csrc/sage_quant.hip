// Quantisation kernels of libsage (gfx950): K smoothing + INT8 K, INT8 Q,
// V smoothing + FP8 E4M3 V with transpose, zero padding and token permutation.
//
// Method: "FLUX.3 Action RTX 5090 report", §02 stage 03 (INT8 QK with
// per-thread scales, read here as per block of 32 Q / 64 K tokens; FP8 PV; K
// and V smoothing) and card A (the K centring is done inside the
// quantiser, keeping the BF16 rounding of K - mean); card C (V is transposed,
// padded and permuted in one tiled pass; its mean, scale and quantisation are
// kept).  E4M3 layout per "Why can an A10 run FLUX.1", §1.1.
//
// All of this is HBM-bound streaming work.  Each tensor is read twice: once
// for the per-channel statistics (fp64 sums, and min / max for V) and once to
// quantise.  The statistics pass splits every (b, h) into token chunks and
// writes per-chunk partials; the last workgroup of each head to finish reduces
// them and writes the head's mean (and V's scale).  The mean is the exact
// channel sum rounded once to fp64, divided by N: fp64 sums of bf16 values
// are exact in any order unless a channel mixes tiny and large values, which
// the pass detects, and such a channel is summed again exactly.
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
// Exactness of the channel sums (reading R3).  The mean of a channel is
// fp64(exact sum) / N rounded to fp32: the exact sum rounded once to fp64.
// Plain fp64 accumulation (in any order) reaches that value whenever every
// partial sum is representable: all values are multiples of the smallest ulp
// u among the non-zero ones, and every partial sum is bounded by S = sum |x|,
// so this holds when S < 2^53 * u.  S itself is accumulated in fp64 next to
// the sum; a computed S below 2^52 * u proves the true S below 2^53 * u (a
// sum of non-negative terms loses less than a relative N * 2^-53 to rounding).
// The statistics pass records, per chunk and channel, S and the smallest
// non-zero |x| (as a bf16 bit pattern, two channels per word, 16-bit integer
// min); a channel that fails the test has its sum recomputed exactly
// (ExactSum) by the head's finalisation, with the whole workgroup.
// ---------------------------------------------------------------------------
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Witness of 2 bf16 (one 32-bit word) folded into wmin = min (|x| bits - 1),
// with 0 wrapping to 0xFFFF (no non-zero value).
__device__ __forceinline__ void witness2(uint32_t w, uint32_t& wmin) {
  const u16x2 am1 = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu) - (u16x2){1, 1};
  wmin = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, wmin), am1));
}

// True when plain fp64 accumulation of the channel is exact in any order,
// from its witness (min non-zero |x| bits - 1) and its computed sum of |x|.
__device__ __forceinline__ bool sum_is_exact(uint32_t mnb, double sum_abs) {
  if (mnb == 0xFFFFu) return true;  // every value is zero
  const uint32_t e = (mnb + 1) >> 7;  // biased exponent of the smallest non-zero |x|
  const int eu = (e == 0 ? 1 : (int)e) - 134;  // its ulp is 2^eu
  return sum_abs < __builtin_ldexp(1.0, 52 + eu);
}

// Exact sum of bf16 values: an integer in units of 2^-133 (the smallest bf16
// subnormal), positive and negative parts in 320-bit unsigned accumulators
// (|sum| < 2^31 * 2^8 * 2^253 < 2^320), rounded once to fp64 at the end.
struct ExactSum {
  uint64_t p[5], n[5];
  __device__ void init() {
#pragma unroll
    for (int i = 0; i < 5; ++i) p[i] = n[i] = 0;
  }
  __device__ static void add_at(uint64_t (&a)[5], uint64_t m, int sh) {
    const int li = sh >> 6, bo = sh & 63;
    const uint64_t lo = m << bo;
    const uint64_t hi = bo ? (m >> (64 - bo)) : 0;
    uint64_t c = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint64_t add = (i == li) ? lo : (i == li + 1) ? hi : 0;
      const uint64_t s1 = a[i] + add;
      const uint64_t c1 = s1 < add;
      const uint64_t s2 = s1 + c;
      const uint64_t c2 = s2 < c;
      a[i] = s2;
      c = c1 | c2;
    }
  }
  // x = (-1)^s * M * 2^(sh - 133): M = 128 + mantissa, sh = E - 1 for a
  // normal (biased exponent E), M = mantissa, sh = 0 for a subnormal.
  __device__ void add(uint32_t h) {
    const uint32_t e = (h >> 7) & 0xFF, m7 = h & 0x7F;
    if (e == 0xFF) return;  // Inf / NaN: unspecified results
    const uint64_t m = e ? (m7 | 0x80) : m7;
    if (m == 0) return;
    add_at((h & 0x8000) ? n : p, m, e ? (int)e - 1 : 0);
  }
  __device__ void merge(const ExactSum& o) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      add_at(p, o.p[i], 64 * i);  // exact limb-aligned adds (bo = 0)
      add_at(n, o.n[i], 64 * i);
    }
  }
  // (p - n) * 2^-133, rounded to nearest fp64, ties to even.
  __device__ double rounded() const {
    uint64_t d[5];
    uint64_t borrow = 0;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint64_t t = p[i] - n[i];
      const uint64_t b1 = p[i] < n[i];
      const uint64_t t2 = t - borrow;
      const uint64_t b2 = t < borrow;
      d[i] = t2;
      borrow = b1 | b2;
    }
    const bool neg = borrow != 0;
    if (neg) {  // two's complement negation
      uint64_t c = 1;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const uint64_t v = ~d[i] + c;
        c = (c && v == 0) ? 1 : 0;
        d[i] = v;
      }
    }
    int top = -1;
    for (int i = 4; i >= 0; --i)
      if (d[i]) {
        top = 64 * i + 63 - __builtin_clzll(d[i]);
        break;
      }
    if (top < 0) return 0.0;
    uint64_t mant;
    int lo = 0;
    if (top <= 52) {
      mant = d[0];
    } else {
      lo = top - 52;  // lowest kept bit
      const int li = lo >> 6, bo = lo & 63;
      mant = d[li] >> bo;
      if (bo && li + 1 < 5) mant |= d[li + 1] << (64 - bo);
      mant &= (((uint64_t)1) << 53) - 1;
      const int g = lo - 1;  // guard bit, then sticky below it
      const bool guard = (d[g >> 6] >> (g & 63)) & 1;
      bool sticky = false;
      for (int i = 0; i < (g >> 6); ++i) sticky |= d[i] != 0;
      if ((g & 63) && (d[g >> 6] & ((((uint64_t)1) << (g & 63)) - 1))) sticky = true;
      if (guard && (sticky || (mant & 1))) {
        ++mant;
        if (mant >> 53) {
          mant >>= 1;
          ++lo;
        }
      }
    }
    const double r = __builtin_ldexp((double)mant, lo - 133);
    return neg ? -r : r;
  }
};

// ---------------------------------------------------------------------------
// Hand-over of the per-chunk partials to the head's last workgroup.  The
// workgroups of a head run on different XCDs, each behind its own L2, which
// does not keep ordinary stores coherent with the other XCDs.  A device-scope
// fence makes them so by writing back and invalidating the whole L2, and one
// such fence per workgroup (~2000 per call) costs more than the statistics
// pass itself.  Instead, everything one workgroup writes for another goes out
// as a relaxed agent-scope atomic store (written through to the device's
// coherence point) and is read back as a relaxed agent-scope atomic load;
// waiting for the stores to complete (vmcnt) before the ticket is taken
// orders them before it, as the release half of a fence would, without the
// L2 write-back that only ordinary stores need.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void st_agent(double* p, double v) {
  __hip_atomic_store((uint64_t*)p, __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store((uint32_t*)p, __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ double ld_agent(const double* p) {
  return __builtin_bit_cast(double, __hip_atomic_load((uint64_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __builtin_bit_cast(float, __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load((uint32_t*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// All of this wave's memory operations complete; also a compiler barrier.
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stores of the INT8 / FP8 codes: non-temporal, so that the codes (read next by
// the attention, in a later launch) do not displace from the memory-side cache
// the K or V rows this call is about to read a second time.  Same-box timings
// at the quant-only size (B1 H40 N32760): sage_quant_qk 262 -> 242 us,
// sage_quant_v 167 -> 148 us; whole steps (quantisers + attention) at the FLUX
// joint, video-early and Long T2V sizes unchanged within 0.3%.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_codes(void* p, uint32_t w0, uint32_t w1) {
  __builtin_nontemporal_store(u32x2{w0, w1}, (u32x2*)p);
}
__device__ __forceinline__ void store_codes(void* p, const uint4& v) {
  __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, (u32x4*)p);
}

// Channel value of the QK RMSNorm + RoPE producer for token row x (bf16, unit
// channel stride) at channel d, given the row's r: the arithmetic of
// norm_rope_apply for the pair (d & ~1, d | 1), one channel returned.
template <int D>
__device__ __forceinline__ uint32_t nr_channel_bits(const uint16_t* xrow, int d, float r,
                                                    const uint16_t* w, const float* rope_row) {
  const int d0 = d & ~1;
  const uint32_t xw = *(const uint32_t*)(xrow + d0);
  const uint32_t ww = *(const uint32_t*)(w + d0);
  float u0 = bf16_lo(xw) * r, u1 = bf16_hi(xw) * r;
  bf16x2_round(u0, u1);
  u0 *= bf16_lo(ww);
  u1 *= bf16_hi(ww);
  bf16x2_round(u0, u1);
  const float c = rope_row[d0], s = rope_row[d0 + 1];
  const float a0 = u0 * c, a1 = u1 * s;
  const float b0 = u0 * s, b1 = u1 * c;
  float y0 = a0 - a1, y1 = b0 + b1;
  bf16x2_round(y0, y1);
  return __float_as_uint((d & 1) ? y1 : y0) >> 16;
}

// ---------------------------------------------------------------------------
// Channel statistics + per-head finalisation: grid (nchunk, B*H), 256
// threads.  Each thread owns 8 consecutive channels (one 16-byte load per
// token row); D/8 threads cover a row, so a pass reads 256/(D/8) rows.  A
// workgroup writes its chunk's partials (fp64 sums and sums of |x|, V's
// min / max, the exactness witnesses), then takes a ticket from the head's
// arrival counter; the last of the head's nchunk workgroups reduces the
// partials (in any order: the sums are exact whenever they are used) and
// writes the head's mean (K: k_mean = bf16(fp32(sum / N)); V: v_mean, v_scale
// and 448/a for the quantisation pass), recomputing the sum exactly for a
// channel whose witness fails, and leaves the counter zero.
// ---------------------------------------------------------------------------
// NR: the rows are first put through the QK RMSNorm + RoPE producer
// (weights nr_w, table rope), so the statistics are those of the producer's
// output; each row's r is stored in rk [BH][Np] for the quantisation pass.
template <int D, bool IS_V, bool NR = false>
__global__ __launch_bounds__(kThreads) void stats_kernel(
    const uint16_t* __restrict__ x, int64_t sb, int64_t sn, int64_t sh, int H, int N, int nchunk,
    int rows_per_chunk, double* __restrict__ psum, double* __restrict__ pabs,
    float* __restrict__ pmin, float* __restrict__ pmax, uint32_t* __restrict__ pwit,
    int* __restrict__ cnt, const uint16_t* __restrict__ nr_w, const float* __restrict__ rope,
    double eps, float* __restrict__ rk, int Np, uint16_t* __restrict__ k_mean,
    float* __restrict__ v_mean, float* __restrict__ v_scale, float* __restrict__ v_inv) {
  constexpr int LPR = D / 8;
  constexpr int RPP = kThreads / LPR;
  // s_sum holds the waves' partials, then the finalisation's, then the exact
  // sums' merge tree
  __shared__ __attribute__((aligned(16))) double s_sum[RPP][D];
  __shared__ float s_min[IS_V ? RPP : 1][D];
  __shared__ float s_max[IS_V ? RPP : 1][D];
  __shared__ double s_xsum[D];  // exact sums of the flagged channels
  __shared__ int s_list[D];     // the flagged channels
  __shared__ int s_last, s_nflag;
  static_assert(sizeof(uint64_t) * 10 * (kThreads / 2) <= sizeof(double) * RPP * D, "merge alias");
  uint64_t (*s_ex)[10] = (uint64_t(*)[10])(&s_sum[0][0]);

  const int c = blockIdx.x, bh = blockIdx.y;
  const int b = bh / H, h = bh - b * H;
  const int tid = threadIdx.x, lr = tid / LPR, lc = tid - lr * LPR;
  const uint16_t* head = x + (int64_t)b * sb + (int64_t)h * sh;
  const uint16_t* base = head + lc * 8;
  const int r0 = c * rows_per_chunk;
  const int r1 = min(N, r0 + rows_per_chunk);

  double acc[8], aacc[8];
  float mn[8], mx[8];
  uint32_t wmin[4];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    acc[j] = 0.0;
    aacc[j] = 0.0;
    mn[j] = __builtin_inff();
    mx[j] = -__builtin_inff();
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) wmin[j] = 0xFFFFFFFFu;
  float w8[8];
  if constexpr (NR) load_w8(nr_w, lc, w8);
  auto fold = [&](const float (&f)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const double d = (double)f[j];
      acc[j] += d;
      aacc[j] += __builtin_fabs(d);
      if (IS_V) {
        mn[j] = fminf(mn[j], f[j]);
        mx[j] = fmaxf(mx[j], f[j]);
      }
    }
  };
  // every lane of a token row takes the same path (the row index depends on
  // the row, not the lane), as the producer's cross-lane sum needs
  auto take = [&](const uint4& v, int row) {
    float f[8];
    unpack8(v, f);
    uint32_t wd[4] = {v.x, v.y, v.z, v.w};
    if constexpr (NR) {
      float f1[1][8], cs[1][8], r[1], r_own;
#pragma unroll
      for (int j = 0; j < 8; ++j) f1[0][j] = f[j];
      load_cs8<D>(rope, row, lc, cs[0]);
      rows_rsqrt<LPR, 1>(f1, eps, r, r_own);
      if (lc == 0) st_agent(rk + (size_t)bh * Np + row, r_own);
      norm_rope_apply<1>(f1, w8, cs, r);
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = f1[0][j];
#pragma unroll
      for (int j = 0; j < 4; ++j) wd[j] = bf16x2_rne(f[2 * j], f[2 * j + 1]);  // exact: bf16 values
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) witness2(wd[j], wmin[j]);
    fold(f);
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
    if (r < r1) {  // the leftover rows (fewer than 8 per thread) as one batch of loads
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        v[u] = r + u * RPP < r1 ? *(const uint4*)(base + (int64_t)(r + u * RPP) * sn) : uint4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (r + u * RPP < r1) take(v[u], r + u * RPP);
      r = r1;
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
      if ((lc & (LPR / 2 - 1)) == 0) st_agent(rk + (size_t)bh * Np + r + (lc / (LPR / 2)) * RPP, r_own);
      norm_rope_apply<2>(f, w8, cs, rr);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int j = 0; j < 4; ++j) witness2(bf16x2_rne(f[u][2 * j], f[u][2 * j + 1]), wmin[j]);
        fold(f[u]);
      }
    }
  }
  for (; r < r1; r += RPP) take(*(const uint4*)(base + (int64_t)r * sn), r);

  // ---- chunk partials: the row groups of a wave combined by lane
  // exchanges, then the waves' results in LDS (any order: the fp64 sums are
  // exact whenever they are used) ----
#pragma unroll
  for (int m = LPR; m < 64; m *= 2) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      acc[j] += __shfl_xor(acc[j], m);
      aacc[j] += __shfl_xor(aacc[j], m);
      if (IS_V) {
        mn[j] = fminf(mn[j], __shfl_xor(mn[j], m));
        mx[j] = fmaxf(mx[j], __shfl_xor(mx[j], m));
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u16x2 o = __builtin_bit_cast(u16x2, (uint32_t)__shfl_xor((int)wmin[j], m));
      wmin[j] = __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, wmin[j]), o));
    }
  }
  constexpr int NWV = kThreads / 64;
  double (*s_wsum)[D] = (double(*)[D])(&s_sum[0][0]);
  double (*s_wabs)[D] = s_wsum + NWV;
  uint32_t (*s_wwit)[D / 2] = (uint32_t(*)[D / 2])(s_wabs + NWV);
  static_assert((2 * sizeof(double) * D + sizeof(uint32_t) * D / 2) * NWV <= sizeof(double) * RPP * D,
                "wave partials alias");
  const int wv = tid >> 6;
  if ((tid & 63) < LPR) {  // the first row group of each wave holds the wave's values
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s_wsum[wv][lc * 8 + j] = acc[j];
      s_wabs[wv][lc * 8 + j] = aacc[j];
      if (IS_V) {
        s_min[wv][lc * 8 + j] = mn[j];
        s_max[wv][lc * 8 + j] = mx[j];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) s_wwit[wv][lc * 4 + j] = wmin[j];
  }
  __syncthreads();
  const size_t pbase = ((size_t)bh * nchunk + c) * D;
  if (tid < D) {
    double csum = 0.0, cabs = 0.0;
    float clo = __builtin_inff(), chi = -__builtin_inff();
    uint32_t wn = 0xFFFFu;
    const int sh16 = 16 * (tid & 1);
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
      csum += s_wsum[i][tid];
      cabs += s_wabs[i][tid];
      wn = min(wn, (s_wwit[i][tid >> 1] >> sh16) & 0xFFFFu);
      if (IS_V) {
        clo = fminf(clo, s_min[i][tid]);
        chi = fmaxf(chi, s_max[i][tid]);
      }
    }
    st_agent(psum + pbase + tid, csum);
    st_agent(pabs + pbase + tid, cabs);
    if (IS_V) {
      st_agent(pmin + pbase + tid, clo);
      st_agent(pmax + pbase + tid, chi);
    }
    st_agent(pwit + pbase + tid, wn);
  }

  // ---- arrival: the last workgroup of the head finalises it ----
  wait_vm();  // this workgroup's partials (and r values) complete before its ticket
  __syncthreads();
  // (one chunk per head: every workgroup finalises its own head, no counter)
  if (tid == 0)
    s_last = nchunk == 1 ||
             __hip_atomic_fetch_add(cnt + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nchunk - 1;
  __syncthreads();
  if (!s_last) return;  // whole workgroup; the partials below are read after the ticket

  // The head's partials: TPC threads per channel, each over every TPC-th
  // batch of 8 chunks (8 loads of each kind in flight, masked at the end),
  // their results combined in LDS.  Any order: the sums are exact whenever
  // they are used (else the channel is summed again below).
  constexpr int TPC = kThreads / D;
  double s_plain = 0.0, s_abs = 0.0;
  float lo = __builtin_inff(), hi = -__builtin_inff();
  bool flagged = false;
  {
    const int d = tid % D, part = tid / D;
    const size_t hb = (size_t)bh * nchunk * D + d;
    uint32_t wn = 0xFFFFu;
    for (int ch = 8 * part; ch < nchunk; ch += 8 * TPC) {
      double ps[8], pa[8];
      float pl[8], ph[8];
      uint32_t pw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        ps[u] = pa[u] = 0.0;
        pl[u] = __builtin_inff();
        ph[u] = -__builtin_inff();
        pw[u] = 0xFFFFu;
        if (ch + u < nchunk) {
          const size_t o = hb + (size_t)(ch + u) * D;
          ps[u] = ld_agent(psum + o);
          pa[u] = ld_agent(pabs + o);
          pw[u] = ld_agent(pwit + o);
          if (IS_V) {
            pl[u] = ld_agent(pmin + o);
            ph[u] = ld_agent(pmax + o);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        s_plain += ps[u];
        s_abs += pa[u];
        wn = min(wn, pw[u]);
        if (IS_V) {
          lo = fminf(lo, pl[u]);
          hi = fmaxf(hi, ph[u]);
        }
      }
    }
    double (*s_psum)[D] = (double(*)[D])(&s_sum[0][0]);
    double (*s_pabs)[D] = s_psum + TPC;
    uint32_t (*s_pwit)[D] = (uint32_t(*)[D])(s_pabs + TPC);
    static_assert((2 * sizeof(double) + sizeof(uint32_t)) * D * TPC <= sizeof(double) * RPP * D,
                  "finalisation partials alias");
    __syncthreads();  // the chunk partials' LDS is free again
    s_psum[part][d] = s_plain;
    s_pabs[part][d] = s_abs;
    s_pwit[part][d] = wn;
    if (IS_V) {
      s_min[part][d] = lo;
      s_max[part][d] = hi;
    }
    __syncthreads();
    if (tid < D) {
      s_plain = s_abs = 0.0;
      wn = 0xFFFFu;
      lo = __builtin_inff();
      hi = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < TPC; ++i) {
        s_plain += s_psum[i][tid];
        s_abs += s_pabs[i][tid];
        wn = min(wn, s_pwit[i][tid]);
        if (IS_V) {
          lo = fminf(lo, s_min[i][tid]);
          hi = fmaxf(hi, s_max[i][tid]);
        }
      }
      flagged = !sum_is_exact(wn, s_abs);
    }
  }
  // list of flagged channels (none for ordinary activations)
  if (tid == 0) s_nflag = 0;
  __syncthreads();
  if (tid < D && flagged) s_list[atomicAdd(&s_nflag, 1)] = tid;
  __syncthreads();
  const int nflag = s_nflag;
  // Exact sum of each flagged channel by the whole workgroup: token n goes to
  // thread n % 256, then the 256 partial sums are merged in a tree in LDS.
  for (int i = 0; i < nflag; ++i) {
    const int d = s_list[i];
    ExactSum ex;
    ex.init();
    auto bits_at = [&](int n) -> uint32_t {
      if constexpr (NR) {
        const float* rope_row = rope + (size_t)n * D;  // (cos, sin) pairs: D floats per token
        return nr_channel_bits<D>(head + (int64_t)n * sn, d, ld_agent(rk + (size_t)bh * Np + n), nr_w,
                                  rope_row);
      } else {
        return head[(int64_t)n * sn + d];
      }
    };
    int n = tid;
    for (; n + 3 * kThreads < N; n += 4 * kThreads) {  // 4 loads in flight
      uint32_t bv[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) bv[u] = bits_at(n + u * kThreads);
#pragma unroll
      for (int u = 0; u < 4; ++u) ex.add(bv[u]);
    }
    for (; n < N; n += kThreads) ex.add(bits_at(n));
    for (int w = kThreads / 2; w >= 1; w >>= 1) {
      if (tid >= w && tid < 2 * w) {
#pragma unroll
        for (int k = 0; k < 5; ++k) {
          s_ex[tid - w][k] = ex.p[k];
          s_ex[tid - w][5 + k] = ex.n[k];
        }
      }
      __syncthreads();
      if (tid < w) {
        ExactSum o;
#pragma unroll
        for (int k = 0; k < 5; ++k) {
          o.p[k] = s_ex[tid][k];
          o.n[k] = s_ex[tid][5 + k];
        }
        ex.merge(o);
      }
      __syncthreads();
    }
    if (tid == 0) s_xsum[d] = ex.rounded();
  }
  __syncthreads();
  if (tid < D) {
    const double s = flagged ? s_xsum[tid] : s_plain;
    const float mean = (float)(s / (double)N);
    if (!IS_V) {
      k_mean[(size_t)bh * D + tid] = (uint16_t)bf16_bits_rne(mean);
    } else {
      const float a = fmaxf(fabsf(hi - mean), fabsf(lo - mean));
      const float inv = 448.0f / a;
      const bool zero = (a == 0.0f) || !__builtin_isfinite(inv);
      v_mean[(size_t)bh * D + tid] = mean;
      v_scale[(size_t)bh * D + tid] = zero ? 0.0f : a / 448.0f;
      v_inv[(size_t)bh * D + tid] = zero ? 0.0f : inv;
    }
  }
  if (tid == 0 && nchunk > 1)  // ready for the next call
    __hip_atomic_store(cnt + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
      store_codes(dst + (size_t)rr * D, w0, w1);
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
      store_codes(dst + (size_t)rr * D, w0, w1);
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
    store_codes(dst + (size_t)rr * D, w0, w1);
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
      store_codes(v_fp8 + ((size_t)bh * D + row) * Np + colg, val);
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
                     (double*)(wsb + w.partial_off), (double*)(wsb + w.abs_off), (float*)nullptr,
                     (float*)nullptr,
                     (uint32_t*)(wsb + w.wit_off), (int*)(wsb + w.cnt_off), nr.wk, nr.rope, nr.eps, rk,
                     Np, k_mean, (float*)nullptr, (float*)nullptr, (float*)nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
                     (double*)(wsb + w.sum_off), (double*)(wsb + w.abs_off), (float*)(wsb + w.min_off),
                     (float*)(wsb + w.max_off), (uint32_t*)(wsb + w.wit_off),
                     (int*)(wsb + w.cnt_off), (const uint16_t*)nullptr, (const float*)nullptr, 0.0,
                     (float*)nullptr, 0, (uint16_t*)nullptr, v_mean, v_scale, inv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
