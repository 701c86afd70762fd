/*
 * CPU oracle for smoothed, quantised attention (SageAttention2-style).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests, the smoke check and the benchmark's CPU
 * baseline may load this library.  It shares no code, headers, tables or
 * constants with the HIP path; the only thing both sides consume is the seeded
 * input generator, which holds none of this arithmetic.
 *
 * Plain, slow and written to be checked by eye against the pages:
 *   [R]  "FLUX.3 Action RTX 5090 report": §02 Engineering, stage 03
 *        "SageAttention2" (INT8 QK, FP8 PV, FP32 accumulation, K smooth and V
 *        smooth kept, NHD layout); stage 04 (fusions are bit exact against the
 *        unfused composition); card A "K centering x INT8 quant" (subtract K's
 *        mean inside the quant step, keep the BF16 rounding, Q quant / scale /
 *        INT8 rules unchanged); card C "V alias + tiled transpose" (transpose,
 *        padding and permutation of V; V mean / scale / quant kept).
 *   [M]  "MiniMax H3 on DGX Spark": §01 precision map (Sage2++ is QK INT8 / PV FP8).
 *   [F]  "Why can an A10 run FLUX.1" article, §1.1: E4M3 = 1 sign, 4 exponent,
 *        3 mantissa bits.
 *   [S]  "FLUX 3 Action" SGLang page: §1 (4-axis (t, h, w, l) RoPE in the joint
 *        blocks) and the latency notes (QK RMSNorm + RoPE as one fused kernel).
 * Where the pages leave a step open, the reading used is stated at the step.
 * All non-codec arithmetic is fp64 unless a step fixes fp32 (the quantiser
 * rules are fp32 operations, so both sides take the same integer decisions).
 *
 * Parity pins: every function here is checked by tests against library casts
 * (torch bf16 / float8_e4m3fn), brute force, closed forms and invariances.
 *
 * Build: gcc -O2 -fPIC -shared -fopenmp -ffp-contract=off (no fast-math).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Codecs                                                                    */
/* ------------------------------------------------------------------------- */

/* bf16 bit pattern -> value (the upper half of an IEEE binary32). */
float orc_bf16_value(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* binary32 -> bf16, round to nearest, ties to even.  The low 16 bits are the
 * fraction of a bf16 ulp that is dropped: above one half rounds up, exactly one
 * half rounds to the even neighbour.  NaN maps to a quiet NaN. */
uint16_t orc_bf16_round(float x) {
  uint32_t u;
  memcpy(&u, &x, 4);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  uint32_t keep = u >> 16, drop = u & 0xFFFFu;
  if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u))) keep += 1u;
  return (uint16_t)keep;
}

/* OCP FP8 E4M3FN decode: bias 7; exponent field 0 is subnormal (m/8 * 2^-6);
 * S.1111.111 is NaN; there are no infinities ([F] §1.1 gives the 1/4/3 split). */
double orc_e4m3_decode(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return s ? -mag : mag;
}

/* Value -> E4M3FN, round to nearest even, saturating at +-448, sign kept
 * (so -0 and negatives that round to zero give 0x80).
 * Reading: the pages say "FP8" / E4M3 without a rounding rule; nearest-even
 * with saturation is the IEEE default restricted to the finite codes. */
uint8_t orc_e4m3_encode(double x) {
  const uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (isnan(x)) return 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  int e2;
  frexp(a, &e2);            /* a = f * 2^e2, f in [0.5, 1)  => floor(log2 a) = e2 - 1 */
  int ex = e2 - 1;          /* unbiased exponent of a (a > 0); a == 0 gives e2 = 0 */
  if (a == 0.0 || ex < -6) {
    /* subnormal range: grid step 2^-9; m in 0..8 (m == 8 is the smallest normal) */
    double m = nearbyint(ldexp(a, 9));
    return sign | (uint8_t)m;
  }
  double m = nearbyint(ldexp(a, 3 - ex)); /* in [8, 16] */
  if (m == 16.0) { m = 8.0; ex += 1; }
  return sign | (uint8_t)(((ex + 7) << 3) | ((int)m - 8));
}

/* INT8 code: round to nearest even, then clamp to the symmetric range. */
int orc_i8_code(float x) {
  double r = nearbyint((double)x);
  if (r > 127.0) r = 127.0;
  if (r < -127.0) r = -127.0;
  return (int)r;
}

/* Storage slot of token t (0..63) inside its 64-token block of transposed V.
 * Reading: the report's V tile does a "transpose, padding and permutation" but
 * never defines the permutation.  This build fixes it as the bit permutation
 *   slot bits (5..0) = token bits (2, 5, 4, 3, 1, 0)
 * i.e. slot = 32*t2 + 16*t5 + 8*t4 + 4*t3 + 2*t1 + t0. */
int orc_v_slot(int t) {
  const int b0 = t & 1, b1 = (t >> 1) & 1, b2 = (t >> 2) & 1;
  const int b3 = (t >> 3) & 1, b4 = (t >> 4) & 1, b5 = (t >> 5) & 1;
  return 32 * b2 + 16 * b5 + 8 * b4 + 4 * b3 + 2 * b1 + b0;
}

void orc_bf16_round_n(const float* x, uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_bf16_round(x[i]);
}
void orc_e4m3_encode_n(const double* x, uint8_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_e4m3_encode(x[i]);
}
void orc_e4m3_decode_n(const uint8_t* x, double* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_e4m3_decode(x[i]);
}

/* ------------------------------------------------------------------------- */
/* Channel statistics                                                        */
/* ------------------------------------------------------------------------- */

/* Smallest bf16 ulp among the non-zero values of a channel: 2^(e-7) for a
 * normal value with unbiased exponent e, 2^-133 for subnormals. */
static double bf16_ulp(uint16_t h) {
  int e = (h >> 7) & 0xFF;
  if (e == 0) return ldexp(1.0, -133);
  return ldexp(1.0, e - 127 - 7);
}

/* The correctly rounded (to nearest, ties to even) fp64 value of the exact sum
 * of x[0..n-1], by Shewchuk's exact-partials summation ("Adaptive Precision
 * Floating-Point Arithmetic and Fast Robust Geometric Predicates", 1997, as
 * used for Python's math.fsum): the running sum is kept as a list of
 * non-overlapping fp64 partials whose exact total is the exact sum so far;
 * at the end the partials are added from the largest down, with a correction
 * for a tie that the lower partials break.  Finite inputs. */
double orc_fsum(const double* x, int64_t n) {
  double stack[64];
  double* part = stack;
  int64_t np = 0, cap = 64;
  for (int64_t k = 0; k < n; ++k) {
    double v = x[k];
    int64_t i = 0;
    for (int64_t j = 0; j < np; ++j) {
      double y = part[j];
      if (fabs(v) < fabs(y)) {
        double t = v;
        v = y;
        y = t;
      }
      double hi = v + y;
      double lo = y - (hi - v); /* exact: hi + lo == v + y */
      if (lo != 0.0) part[i++] = lo;
      v = hi;
    }
    if (i == cap) {
      double* grown = (double*)malloc(sizeof(double) * (size_t)(2 * cap));
      memcpy(grown, part, sizeof(double) * (size_t)i);
      if (part != stack) free(part);
      part = grown;
      cap *= 2;
    }
    part[i] = v;
    np = i + 1;
  }
  double hi = 0.0;
  if (np > 0) {
    int64_t j = np - 1;
    double lo = 0.0;
    hi = part[j];
    while (j > 0) {
      double v = hi;
      double y = part[--j];
      hi = v + y;
      lo = y - (hi - v);
      if (lo != 0.0) break;
    }
    /* hi + lo is exact and lo is half an ulp of hi or less; if it is exactly
     * half and the next partial has the same sign, the true sum is beyond the
     * half-way point: round away from hi */
    if (j > 0 && ((lo < 0.0 && part[j - 1] < 0.0) || (lo > 0.0 && part[j - 1] > 0.0))) {
      double y = lo * 2.0;
      double v = hi + y;
      if (y == v - hi) hi = v;
    }
  }
  if (part != stack) free(part);
  return hi;
}

/* Sum of one channel (reading R3): the correctly rounded fp64 value of the
 * exact sum.  Returns 1 if plain fp64 accumulation is provably exact for this
 * channel in any order -- every value is a multiple of the smallest ulp u
 * among the non-zero values and sum|x| < u * 2^52, so every partial sum is
 * representable -- in which case the ascending fp64 sum is that value; else the
 * exact sum is rounded once (orc_fsum), and the return is 0.  (Reading: the
 * pages do not say how the mean is reduced; the exact sum makes it order-free
 * for every input.) */
static int channel_sum(const uint16_t* base, int64_t stride, int64_t n, double* sum_out) {
  double s = 0.0, sabs = 0.0, umin = INFINITY;
  for (int64_t j = 0; j < n; ++j) {
    uint16_t h = base[j * stride];
    double x = (double)orc_bf16_value(h);
    s += x;
    sabs += fabs(x);
    if (x != 0.0) {
      double u = bf16_ulp(h);
      if (u < umin) umin = u;
    }
  }
  const int exact = (umin == INFINITY) || (sabs < ldexp(umin, 52));
  if (!exact) {
    double* xs = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
    for (int64_t j = 0; j < n; ++j) xs[j] = (double)orc_bf16_value(base[j * stride]);
    s = orc_fsum(xs, n);
    free(xs);
  }
  *sum_out = s;
  return exact;
}

#define AT(p, b, n, h, sb, sn, sh) ((p)[(int64_t)(b) * (sb) + (int64_t)(n) * (sn) + (int64_t)(h) * (sh)])

/* Step 1 (card A, reading R1/R2/R3): K mean per (b, h, d) over all N tokens,
 * fp64 sum, fp64 / N, rounded to fp32 then to bf16 (the unfused path holds the
 * mean as a BF16 tensor).  Output k_mean[B][H][D].  Returns the number of
 * channels whose plain fp64 sum is not provably exact (their sum is the
 * rounded exact sum, see channel_sum). */
int orc_k_mean(const uint16_t* k, int64_t sb, int64_t sn, int64_t sh, int B, int N, int H, int D,
               uint16_t* k_mean) {
  int bad = 0;
#pragma omp parallel for collapse(2) reduction(+ : bad) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) {
        double s;
        bad += !channel_sum(&AT(k, b, 0, h, sb, sn, sh) + d, sn, N, &s);
        k_mean[((int64_t)b * H + h) * D + d] = orc_bf16_round((float)(s / (double)N));
      }
  return bad;
}

/* Step 2 (card A): kc = bf16(K - k_mean), an fp32 subtraction of two bf16
 * values followed by the explicit BF16 rounding.  Output kc[B][N][H][D]. */
void orc_k_center(const uint16_t* k, int64_t sb, int64_t sn, int64_t sh, int B, int N, int H, int D,
                  const uint16_t* k_mean, uint16_t* kc) {
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < N; ++n)
      for (int h = 0; h < H; ++h)
        for (int d = 0; d < D; ++d) {
          float x = orc_bf16_value((&AT(k, b, n, h, sb, sn, sh))[d]);
          float m = orc_bf16_value(k_mean[((int64_t)b * H + h) * D + d]);
          float diff = x - m;
          kc[(((int64_t)b * N + n) * H + h) * D + d] = orc_bf16_round(diff);
        }
}

/* INT8 rule for one block (card A: "INT8 rules unchanged"; reading R6):
 * a = absmax (exact), scale = a / 127, inv = 127 / a (fp32, correctly rounded),
 * code = clamp(rne(x * inv), -127, 127).  A zero block, or one whose inv is not
 * finite, gets scale 0 and all-zero codes. */
static float i8_block_params(float a, float* inv_out) {
  float inv = 127.0f / a;
  if (a == 0.0f || !isfinite(inv)) {
    *inv_out = 0.0f;
    return 0.0f;
  }
  *inv_out = inv;
  return a / 127.0f;
}

/* Per-block INT8 quantisation of a bf16 tensor x[B][N][H][D] (strided) with
 * `blk` tokens per block (the last block may be partial: absmax over its valid
 * tokens only).  codes[B][H][N][D], scales[B][H][ceil(N/blk)]. */
void orc_quant_i8_blocks(const uint16_t* x, int64_t sb, int64_t sn, int64_t sh, int B, int N, int H,
                         int D, int blk, int8_t* codes, float* scales) {
  const int nblk = (N + blk - 1) / blk;
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int t = 0; t < nblk; ++t) {
        const int j0 = t * blk, j1 = (j0 + blk < N) ? j0 + blk : N;
        float a = 0.0f;
        for (int j = j0; j < j1; ++j)
          for (int d = 0; d < D; ++d) {
            float v = fabsf(orc_bf16_value((&AT(x, b, j, h, sb, sn, sh))[d]));
            if (v > a) a = v;
          }
        float inv;
        float scale = i8_block_params(a, &inv);
        scales[((int64_t)b * H + h) * nblk + t] = scale;
        for (int j = j0; j < j1; ++j)
          for (int d = 0; d < D; ++d) {
            float v = orc_bf16_value((&AT(x, b, j, h, sb, sn, sh))[d]);
            int c = (scale == 0.0f) ? 0 : orc_i8_code(v * inv);
            codes[(((int64_t)b * H + h) * N + j) * D + d] = (int8_t)c;
          }
      }
}

/* ------------------------------------------------------------------------- */
/* Producer of Q and K: QK RMSNorm + RoPE                                     */
/* ------------------------------------------------------------------------- */

/* The fused QK RMSNorm + RoPE of the "FLUX 3 Action" SGLang page (§1: a 4-axis
 * (t, h, w, l) RoPE; latency notes: the fused kernel sits at bf16 rounding
 * level) whose BF16 NHD result feeds the quantiser (report card B).  Reading:
 * the eager composition with each bf16 rounding kept.  For token row x of a
 * head (D channels), with per-channel weights w (bf16) and the rotation table
 * rope[token][pair] = (c, s) (fp32):
 *   ms    = (sum_d x_d^2) / D           fp64
 *   r     = fp32(1 / sqrt(ms + eps))    fp64 add, sqrt and divide, then fp32
 *   n_d   = bf16(x_d * r)               fp32 product
 *   u_d   = bf16(n_d * w_d)             fp32 product of two bf16 values (exact)
 *   y_2i  = bf16(u_2i * c - u_2i+1 * s) fp32: both products rounded, then the
 *   y_2i+1= bf16(u_2i * s + u_2i+1 * c) difference / sum rounded
 * The fp64 sum of squares is exact when every x_d^2 is a multiple of u^2 (u
 * the smallest bf16 ulp among the row's non-zero values, always true) and
 * sum x_d^2 < u^2 2^53; it then does not depend on summation order.
 * x strided [B][N][H][D]; y contiguous [B][N][H][D] (bf16 bits).
 * Returns the number of rows whose sum is not provably exact. */
int orc_norm_rope(const uint16_t* x, int64_t sb, int64_t sn, int64_t sh, int B, int N, int H, int D,
                  const uint16_t* w, float eps, const float* rope, uint16_t* y) {
  int bad = 0;
#pragma omp parallel for collapse(2) reduction(+ : bad) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int n = 0; n < N; ++n)
      for (int h = 0; h < H; ++h) {
        const uint16_t* row = &AT(x, b, n, h, sb, sn, sh);
        uint16_t* out = y + (((int64_t)b * N + n) * H + h) * D;
        double ss = 0.0, umin = INFINITY;
        for (int d = 0; d < D; ++d) {
          double v = (double)orc_bf16_value(row[d]);
          ss += v * v;
          if (v != 0.0) {
            double u = bf16_ulp(row[d]);
            if (u < umin) umin = u;
          }
        }
        if (umin != INFINITY && !(ss < ldexp(umin * umin, 53))) bad += 1;
        const double ms = ss / (double)D;
        const float r = (float)(1.0 / sqrt(ms + (double)eps));
        for (int i = 0; i < D / 2; ++i) {
          float u0 = orc_bf16_value(orc_bf16_round(orc_bf16_value(row[2 * i]) * r));
          float u1 = orc_bf16_value(orc_bf16_round(orc_bf16_value(row[2 * i + 1]) * r));
          u0 = orc_bf16_value(orc_bf16_round(u0 * orc_bf16_value(w[2 * i])));
          u1 = orc_bf16_value(orc_bf16_round(u1 * orc_bf16_value(w[2 * i + 1])));
          const float c = rope[((int64_t)n * (D / 2) + i) * 2], s = rope[((int64_t)n * (D / 2) + i) * 2 + 1];
          const float a0 = u0 * c, a1 = u1 * s, b0 = u0 * s, b1 = u1 * c;
          out[2 * i] = orc_bf16_round(a0 - a1);
          out[2 * i + 1] = orc_bf16_round(b0 + b1);
        }
      }
  return bad;
}

/* Steps 1-4 as ONE routine (the fused form the report describes in card A:
 * center + BF16 round + quant with no K intermediate).  Q uses blocks of
 * q_block tokens on raw Q (reading R5/R7: no smoothing and no softmax scale
 * folded in): 32 for the block granularity of the path, 1 for one scale per
 * token (the finer "per-thread" granularity of §02 stage 03).  K uses blocks of
 * k_block tokens on the centred values: 64, the key tile (reading R4), or 16,
 * a finer variant in the same direction.
 * Outputs: q_i8/k_i8 [B][H][N][D], q_scale [B][H][ceil(N/q_block)],
 * k_scale [B][H][ceil(N/k_block)], k_mean [B][H][D] (bf16).
 * Returns the number of K channels whose fp64 sum is not provably exact. */
int orc_quant_qk(const uint16_t* q, int64_t qsb, int64_t qsn, int64_t qsh,
                 const uint16_t* k, int64_t ksb, int64_t ksn, int64_t ksh,
                 int B, int N, int H, int D, int q_block, int k_block,
                 int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, uint16_t* k_mean) {
  const int BQ = q_block, BK = k_block;
  const int nq = (N + BQ - 1) / BQ, nk = (N + BK - 1) / BK;
  int bad = 0;
#pragma omp parallel for collapse(2) reduction(+ : bad) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int64_t bh = (int64_t)b * H + h;
      float* mean = (float*)malloc(sizeof(float) * D);
      float* kc = (float*)malloc(sizeof(float) * (size_t)BK * D);
      /* K mean (step 1) */
      for (int d = 0; d < D; ++d) {
        double s;
        bad += !channel_sum(&AT(k, b, 0, h, ksb, ksn, ksh) + d, ksn, N, &s);
        uint16_t m16 = orc_bf16_round((float)(s / (double)N));
        k_mean[bh * D + d] = m16;
        mean[d] = orc_bf16_value(m16);
      }
      /* K center + round + INT8 per k_block-token block (steps 2-3) */
      for (int t = 0; t < nk; ++t) {
        const int j0 = t * BK, j1 = (j0 + BK < N) ? j0 + BK : N;
        float a = 0.0f;
        for (int j = j0; j < j1; ++j)
          for (int d = 0; d < D; ++d) {
            float x = orc_bf16_value((&AT(k, b, j, h, ksb, ksn, ksh))[d]);
            float c = orc_bf16_value(orc_bf16_round(x - mean[d]));
            kc[(size_t)(j - j0) * D + d] = c;
            if (fabsf(c) > a) a = fabsf(c);
          }
        float inv;
        float scale = i8_block_params(a, &inv);
        k_scale[bh * nk + t] = scale;
        for (int j = j0; j < j1; ++j)
          for (int d = 0; d < D; ++d) {
            float c = kc[(size_t)(j - j0) * D + d];
            k_i8[(bh * N + j) * D + d] = (int8_t)((scale == 0.0f) ? 0 : orc_i8_code(c * inv));
          }
      }
      /* Q INT8 per q_block-token block (step 4) */
      for (int t = 0; t < nq; ++t) {
        const int j0 = t * BQ, j1 = (j0 + BQ < N) ? j0 + BQ : N;
        float a = 0.0f;
        for (int j = j0; j < j1; ++j)
          for (int d = 0; d < D; ++d) {
            float x = fabsf(orc_bf16_value((&AT(q, b, j, h, qsb, qsn, qsh))[d]));
            if (x > a) a = x;
          }
        float inv;
        float scale = i8_block_params(a, &inv);
        q_scale[bh * nq + t] = scale;
        for (int j = j0; j < j1; ++j)
          for (int d = 0; d < D; ++d) {
            float x = orc_bf16_value((&AT(q, b, j, h, qsb, qsn, qsh))[d]);
            q_i8[(bh * N + j) * D + d] = (int8_t)((scale == 0.0f) ? 0 : orc_i8_code(x * inv));
          }
      }
      free(mean);
      free(kc);
    }
  return bad;
}

/* Steps 5-6 (card C; readings R8-R12): per (b, h, d) over all tokens,
 * mu = fp32(fp64 sum / N); a = max(|max - mu|, |min - mu|) in fp32 (equal to
 * the brute-force absmax of V - mu, asserted here); v_scale = a / 448,
 * inv = 448 / a; code = E4M3(fp32(V - mu) * inv).  Codes are stored transposed,
 * v_fp8[B][H][D][Np] (Np = N rounded up to 64), token t of block g at column
 * 64 g + slot(t mod 64); padding columns hold 0x00.
 * Returns (#channels whose plain fp64 sum is not provably exact) +
 * 2^20 * (#channels where the min/max identity failed). */
int orc_quant_v(const uint16_t* v, int64_t sb, int64_t sn, int64_t sh, int B, int N, int H, int D,
                uint8_t* v_fp8, float* v_scale, float* v_mean) {
  const int64_t Np = ((int64_t)N + 63) / 64 * 64;
  int inexact = 0, idbad = 0;
#pragma omp parallel for collapse(2) reduction(+ : inexact, idbad) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int d = 0; d < D; ++d) {
        const int64_t ch = ((int64_t)b * H + h) * D + d;
        const uint16_t* col = &AT(v, b, 0, h, sb, sn, sh) + d;
        double s;
        inexact += !channel_sum(col, sn, N, &s);
        float mu = (float)(s / (double)N);
        float mx = -INFINITY, mn = INFINITY;
        for (int j = 0; j < N; ++j) {
          float x = orc_bf16_value(col[(int64_t)j * sn]);
          if (x > mx) mx = x;
          if (x < mn) mn = x;
        }
        float hi = mx - mu, lo = mn - mu;
        float a = fmaxf(fabsf(hi), fabsf(lo));
        float brute = 0.0f;
        for (int j = 0; j < N; ++j) {
          float c = orc_bf16_value(col[(int64_t)j * sn]) - mu;
          if (fabsf(c) > brute) brute = fabsf(c);
        }
        idbad += (brute != a);
        float inv = 448.0f / a;
        float scale = a / 448.0f;
        int zero = (a == 0.0f) || !isfinite(inv);
        if (zero) scale = 0.0f;
        v_scale[ch] = scale;
        v_mean[ch] = mu;
        uint8_t* row = v_fp8 + ch * Np;
        for (int64_t j = 0; j < Np; ++j) row[j] = 0x00;
        for (int j = 0; j < N; ++j) {
          float c = orc_bf16_value(col[(int64_t)j * sn]) - mu;
          float y = c * inv;
          row[(j / 64) * 64 + orc_v_slot(j % 64)] = zero ? 0x00 : orc_e4m3_encode((double)y);
        }
      }
  return inexact + (idbad << 20);
}

/* ------------------------------------------------------------------------- */
/* Row-wise FP8 projections                                                  */
/* ------------------------------------------------------------------------- */

/* Stage 02 of the report's §02 keeps the Q/K projections in BF16 and runs
 * the other selected projections in row-wise FP8; the SGLang page's latency
 * notes fix the form: E4M3 weights with one scale per output row, per-token
 * activation scales, a scaled FP8 GEMM.  Reading: a row (a token of the
 * activation, an output row of the weight) is quantised with the V rule:
 * a = max_k |x[k]|, scale = a / 448, code = E4M3(fp32(x) * fp32(448 / a))
 * (round to nearest even, saturating at +-448); a == 0 or 448/a not finite
 * gives scale 0 and codes 0.  x is bf16 [M] rows of K values, row stride ld;
 * codes [M][K], scales [M]. */
void orc_quant_rows_e4m3(const uint16_t* x, int64_t ld, int M, int K, uint8_t* codes,
                         float* scales) {
#pragma omp parallel for schedule(static)
  for (int m = 0; m < M; ++m) {
    const uint16_t* row = x + (int64_t)m * ld;
    float a = 0.0f;
    for (int k = 0; k < K; ++k) {
      float v = fabsf(orc_bf16_value(row[k]));
      if (v > a) a = v;
    }
    const float inv = 448.0f / a;
    const int zero = (a == 0.0f) || !isfinite(inv);
    scales[m] = zero ? 0.0f : a / 448.0f;
    for (int k = 0; k < K; ++k)
      codes[(int64_t)m * K + k] = zero ? 0x00 : orc_e4m3_encode((double)(orc_bf16_value(row[k]) * inv));
  }
}

/* The scaled FP8 GEMM on such codes, for the output entries (rows[i], cols[j]):
 *   out = (sum_k dec(a[m][k]) dec(b[n][k])) * sa[m] * sb[n] + bias[n]
 * in fp64 (bias bf16 [N], or NULL for none).  Two magnitudes for the tests'
 * error bounds (not part of the result):
 *   absum = sa[m] sb[n] sum_k |p_k| + |bias[n]|,  p_k = dec(a[m][k]) dec(b[n][k]);
 *   blk   = sa[m] sb[n] sum over 64-term blocks of k (ascending) of
 *           (|exact sum of the earlier blocks| + max |p_k| in the block),
 * the magnitude that bounds a blocked accumulator which adds 64 products at a
 * time to its running value with a fixed number of bits below the larger of
 * the two.  a [M][K], b [N][K] (both K-contiguous); out, absum, blk [nr][nc]. */
void orc_gemm_fp8_rowwise(const uint8_t* a, const float* sa, int M, const uint8_t* b, const float* sb,
                          int N, int K, const uint16_t* bias, const int32_t* rows, int nr,
                          const int32_t* cols, int nc, double* out, double* absum, double* blk) {
  (void)M;
  (void)N;
  double lut[256];
  for (int c = 0; c < 256; ++c) lut[c] = orc_e4m3_decode((uint8_t)c);
#pragma omp parallel for collapse(2) schedule(static)
  for (int i = 0; i < nr; ++i)
    for (int j = 0; j < nc; ++j) {
      const int m = rows[i], n = cols[j];
      const uint8_t* ar = a + (int64_t)m * K;
      const uint8_t* br = b + (int64_t)n * K;
      double acc = 0.0, aacc = 0.0, bacc = 0.0, bmax = 0.0, before = 0.0;
      for (int k = 0; k < K; ++k) {
        if (k % 64 == 0) before = fabs(acc);
        const double t = lut[ar[k]] * lut[br[k]];
        acc += t;
        aacc += fabs(t);
        if (fabs(t) > bmax) bmax = fabs(t);
        if (k % 64 == 63 || k == K - 1) {
          bacc += before + bmax;
          bmax = 0.0;
        }
      }
      const double s = (double)sa[m] * (double)sb[n];
      const double bb = bias ? (double)orc_bf16_value(bias[n]) : 0.0;
      out[(int64_t)i * nc + j] = acc * s + bb;
      absum[(int64_t)i * nc + j] = aacc * s + fabs(bb);
      blk[(int64_t)i * nc + j] = bacc * s;
    }
}

/* ------------------------------------------------------------------------- */
/* Attention                                                                 */
/* ------------------------------------------------------------------------- */

/* Online softmax-weighted sum over keys in tiles of `bc` (ascending), for one
 * query row: s[0..n) scores, vals[n][dv] values.  Returns out[d] = acc[d] / l.
 * Reading R13-R17: the reference point for every tile is the running max
 * INCLUDING that tile; alpha = exp(m_old - m_new) rescales acc and l; the row
 * sum l accumulates the unquantised p.  With quant_p, the weight in acc is the
 * FP8 value E4M3(448 p) / 448 (a static scale, since p <= 1) -- the "FP8 PV" of
 * stage 03; without it the weight is p (plain flash attention). */
void orc_online_softmax_pv(const double* s, const double* vals, int n, int dv, int bc, int quant_p,
                           double* out) {
  double m = -INFINITY, l = 0.0;
  for (int d = 0; d < dv; ++d) out[d] = 0.0;
  for (int j0 = 0; j0 < n; j0 += bc) {
    const int j1 = (j0 + bc < n) ? j0 + bc : n;
    double mt = -INFINITY;
    for (int j = j0; j < j1; ++j)
      if (s[j] > mt) mt = s[j];
    const double m_new = (mt > m) ? mt : m;
    const double alpha = (m == -INFINITY) ? 0.0 : exp(m - m_new);
    l *= alpha;
    for (int d = 0; d < dv; ++d) out[d] *= alpha;
    for (int j = j0; j < j1; ++j) {
      const double p = exp(s[j] - m_new);
      l += p;
      const double w = quant_p ? orc_e4m3_decode(orc_e4m3_encode(448.0 * p)) / 448.0 : p;
      for (int d = 0; d < dv; ++d) out[d] += w * vals[(int64_t)j * dv + d];
    }
    m = m_new;
  }
  for (int d = 0; d < dv; ++d) out[d] /= l;
}

/* Step 7: the quantised path in fp64 with the kernel's granularity.
 * For query i of head (b, h):  s_j = (sum_d q_i8[i,d] k_i8[j,d]) * q_scale[i/q_block]
 * * sm_scale * k_scale[j/k_block]  (exact integer dot product, then fp64);
 * 64-key tiles, online softmax as above with FP8 P;
 * O[i,d] = (acc/l)[d] * v_scale[d] + v_mean[d]  (the V mean added back).
 * Inputs in the layouts produced by orc_quant_qk / orc_quant_v.
 * rows[0..nrows) are the query indices computed for every (b, h);
 * out[B][H][nrows][D] in fp64. */
void orc_attn_tiled(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                    const uint8_t* v_fp8, const float* v_scale, const float* v_mean,
                    int B, int N, int H, int D, double sm_scale, int bc, int q_block, int k_block,
                    const int32_t* rows, int nrows, double* out) {
  const int nq = (N + q_block - 1) / q_block, nk = (N + k_block - 1) / k_block;
  const int64_t Np = ((int64_t)N + 63) / 64 * 64;
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int64_t bh = (int64_t)b * H + h;
      /* dequantised V codes in token order: vals[j][d] = decode(v_fp8[d][slot]) */
      double* vals = (double*)malloc(sizeof(double) * (size_t)N * D);
      for (int j = 0; j < N; ++j)
        for (int d = 0; d < D; ++d)
          vals[(int64_t)j * D + d] =
              orc_e4m3_decode(v_fp8[(bh * D + d) * Np + (j / 64) * 64 + orc_v_slot(j % 64)]);
#pragma omp parallel for schedule(dynamic)
      for (int r = 0; r < nrows; ++r) {
        const int i = rows[r];
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* o = out + (bh * nrows + r) * D;
        const int8_t* qi = q_i8 + (bh * N + i) * D;
        const double cq = (double)q_scale[bh * nq + i / q_block] * sm_scale;
        for (int j = 0; j < N; ++j) {
          const int8_t* kj = k_i8 + (bh * N + j) * D;
          int64_t dot = 0;
          for (int d = 0; d < D; ++d) dot += (int64_t)qi[d] * (int64_t)kj[d];
          s[j] = (double)dot * cq * (double)k_scale[bh * nk + j / k_block];
        }
        orc_online_softmax_pv(s, vals, N, D, bc, 1, o);
        for (int d = 0; d < D; ++d) o[d] = o[d] * (double)v_scale[bh * D + d] + (double)v_mean[bh * D + d];
        free(s);
      }
      free(vals);
    }
}

/* Step 8: exact softmax attention in fp64 from the original bf16 Q, K, V
 * (no smoothing, no quantisation): O_i = sum_j softmax_j(q_i . k_j * sm_scale) v_j.
 * Inputs strided [B][N][H][D]; rows / out as in orc_attn_tiled. */
void orc_attn_exact(const uint16_t* q, int64_t qsb, int64_t qsn, int64_t qsh,
                    const uint16_t* k, int64_t ksb, int64_t ksn, int64_t ksh,
                    const uint16_t* v, int64_t vsb, int64_t vsn, int64_t vsh,
                    int B, int N, int H, int D, double sm_scale,
                    const int32_t* rows, int nrows, double* out) {
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      const int64_t bh = (int64_t)b * H + h;
      double* kd = (double*)malloc(sizeof(double) * (size_t)N * D);
      double* vd = (double*)malloc(sizeof(double) * (size_t)N * D);
      for (int j = 0; j < N; ++j)
        for (int d = 0; d < D; ++d) {
          kd[(int64_t)j * D + d] = orc_bf16_value((&AT(k, b, j, h, ksb, ksn, ksh))[d]);
          vd[(int64_t)j * D + d] = orc_bf16_value((&AT(v, b, j, h, vsb, vsn, vsh))[d]);
        }
#pragma omp parallel for schedule(dynamic)
      for (int r = 0; r < nrows; ++r) {
        const int i = rows[r];
        double* s = (double*)malloc(sizeof(double) * (size_t)N);
        double* o = out + (bh * nrows + r) * D;
        double m = -INFINITY;
        for (int j = 0; j < N; ++j) {
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += (double)orc_bf16_value((&AT(q, b, i, h, qsb, qsn, qsh))[d]) * kd[(int64_t)j * D + d];
          s[j] = dot * sm_scale;
          if (s[j] > m) m = s[j];
        }
        double l = 0.0;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int j = 0; j < N; ++j) {
          double p = exp(s[j] - m);
          l += p;
          for (int d = 0; d < D; ++d) o[d] += p * vd[(int64_t)j * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= l;
        free(s);
      }
      free(kd);
      free(vd);
    }
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Thread count of the OpenMP loops above (timing only; no result depends on it). */
void orc_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
