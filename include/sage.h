/*
 * sage.h -- C ABI of libsage.so: smoothed, quantised attention for MI355X
 * (gfx950), in the manner of SageAttention2 as used in the FLUX.3 Action and
 * MiniMax-H3 DiT blocks.
 *
 * Source pages (cited by title and section):
 *   "FLUX.3 Action RTX 5090 report", §02 Engineering: stage 03 "SageAttention2"
 *     (INT8 QK with per-thread scales, FP8 PV, FP32 accumulation, K smooth and
 *     V smooth kept, NHD layout; the scales here are per block of 32 Q / 64 K
 *     tokens, a reading of "per-thread" for the MFMA tiles of this chip); stage 04 (fusions bit-exact against the unfused path);
 *     card A (K centring fused into the INT8 quantiser, BF16 rounding kept);
 *     card B (producers write BF16 NHD directly); card C (V read as a slice of
 *     the V+MLP projection; tiled transpose, padding and permutation).
 *   "MiniMax H3 on DGX Spark", §01 precision map (QK INT8 / PV FP8).
 *   "Why can an A10 run FLUX.1", §1.1 (E4M3: 4 exponent, 3 mantissa bits).
 *   "FLUX 3 Action" SGLang page: §1 (4-axis (t, h, w, l) RoPE in the joint
 *     blocks) and the latency notes (QK RMSNorm + RoPE as one fused kernel;
 *     row-wise FP8 projections: E4M3 weights, one scale per output row,
 *     per-token activation scales, a scaled FP8 GEMM).
 *   "FLUX.3 Action RTX 5090 report", §02 stage 02 (mixed-precision
 *     projections: Q/K projections BF16, other selected projections row-wise FP8).
 *
 * Conventions shared by every entry point
 *   - Tensors named "[B,N,H,D]" are bf16 (uint16 bit patterns) in token-major
 *     NHD order with element strides (sb, sn, sh) and unit stride over d.
 *     Strides may describe a view into a wider buffer (e.g. V as a column slice
 *     of a fused projection output).
 *   - Np = N rounded up to a multiple of 64 (sage_padded_tokens).
 *   - Pointers marked "device" are HIP device pointers; `stream` is a
 *     hipStream_t passed as void* (NULL = the null stream).
 *   - The caller owns every buffer; the library allocates no device memory
 *     and keeps no per-call state.  Calls are asynchronous: they enqueue work on
 *     `stream` and return; buffers must stay valid until the stream reaches it.
 *   - Validation runs first; on failure a negative status is returned and
 *     nothing is enqueued.  Nothing throws or aborts across the ABI.  A launch
 *     failure returns SAGE_ERR_HIP.  NaN / Inf inputs give unspecified values.
 *   - Supported: D in {64, 128}; B, N, H >= 1; B*H*Np*D < 2^31; all base
 *     pointers and input strides 16-byte aligned (strides multiple of 8).
 *   - Inputs and outputs must not overlap (checked by address range).
 *   - The library is reentrant.  Quantised outputs are bit-deterministic;
 *     the attention output is bit-deterministic for a given build.
 */
#ifndef SAGE_H
#define SAGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum sage_status {
  SAGE_OK = 0,
  SAGE_ERR_NULL = -1,        /* a required pointer is NULL                       */
  SAGE_ERR_SHAPE = -2,       /* B, N or H < 1, or the problem is too large       */
  SAGE_ERR_UNSUPPORTED = -3, /* D not in {64, 128}                               */
  SAGE_ERR_STRIDE = -4,      /* a stride is not positive                         */
  SAGE_ERR_ALIGN = -5,       /* a pointer or stride breaks 16-byte alignment     */
  SAGE_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required       */
  SAGE_ERR_OVERLAP = -7,     /* an output overlaps an input or another output    */
  SAGE_ERR_HIP = -8,         /* a HIP launch or runtime call failed              */
  SAGE_ERR_VALUE = -9        /* a scalar argument is out of range (e.g. eps)     */
};

#define SAGE_BQ 32          /* Q quantisation block, tokens (one MFMA column tile) */
#define SAGE_BK 64          /* K quantisation block = attention key tile, tokens   */
#define SAGE_NPAD 64        /* token padding of the quantised layouts              */
#define SAGE_PERM_VERSION 1 /* version of the V slot map below                     */

/* Q scale granularity (q_block of the _ex entry points): one scale per 32-token
 * block (SAGE_Q_BLOCK, what sage_quant_qk / sage_attn_fwd use) or one per token
 * (SAGE_Q_TOKEN: the finer "per-thread" granularity of the report's §02 stage 03). */
#define SAGE_Q_BLOCK 32
#define SAGE_Q_TOKEN 1
/* K scale granularity (k_block of the _ex entry points): one scale per 64-token
 * block, the attention key tile (SAGE_K_BLOCK, what sage_quant_qk / sage_attn_fwd
 * use), or per 16-token block (SAGE_K_FINE: four scales per key tile). */
#define SAGE_K_BLOCK 64
#define SAGE_K_FINE 16

typedef struct {
  int32_t bq;             /* SAGE_BQ */
  int32_t bk;             /* SAGE_BK */
  int32_t n_pad_multiple; /* SAGE_NPAD */
  int32_t perm_version;   /* SAGE_PERM_VERSION */
} sage_layout;

/* Fills *out (host pointer) with the layout constants.  Returns SAGE_OK or
 * SAGE_ERR_NULL. */
int sage_get_layout(sage_layout* out);

/* N rounded up to a multiple of 64 (N >= 0). */
int64_t sage_padded_tokens(int64_t N);

/* Storage slot of token t (0..63) inside a 64-token block of the transposed V
 * (card C's "permutation"; the page does not define it).  Version 1:
 *     slot bits (5..0) = token bits (2, 5, 4, 3, 1, 0)
 * i.e. slot = 32*t2 + 16*t5 + 8*t4 + 4*t3 + 2*t1 + t0.  With this order the
 * 32 probabilities that one lane of the attention kernel holds after the INT8
 * QK^T MFMA are exactly the 32 V bytes that lane feeds to the FP8 PV MFMA.
 * Returns -1 for t outside 0..63. */
int sage_v_slot(int t);

/* Workspace (device memory, bytes) needed by sage_quant_qk / sage_quant_v:
 * per-head arrival counters, then per-chunk channel partials (and, for V, the
 * per-channel 448/a).  The first sage_workspace_zero_bytes() bytes hold
 * the counters: they must be zero before the first call that uses the
 * workspace (e.g. a zero-filled allocation), and every call leaves them zero;
 * the rest may hold anything and is clobbered.  One workspace must not be
 * shared by calls that may run concurrently.  Returns 0 for unsupported
 * shapes. */
size_t sage_quant_qk_workspace_size(int B, int N, int H, int D);
/* Workspace bytes of sage_norm_rope_quant_qk: those of sage_quant_qk plus one
 * fp32 per K token row (B*H*Np*4, rounded up to 256); 0 for unsupported sizes. */
size_t sage_norm_rope_quant_qk_workspace_size(int B, int N, int H, int D);
size_t sage_quant_v_workspace_size(int B, int N, int H, int D);
/* Bytes at the start of every quantiser workspace that must be zero before
 * its first use (the arrival counters; a fixed 8192). */
size_t sage_workspace_zero_bytes(void);

/*
 * sage_quant_qk -- K smoothing + INT8 K, and INT8 Q (report §02 stage 03;
 * card A "K centering x INT8 quant").
 *
 *   k_mean[b,h,d] = bf16( fp32( fp64(sum over all N tokens of K[b,n,h,d]) / N ) )
 *                   (the exact sum rounded once to fp64, then an fp64 divide)
 *   kc            = bf16( fp32(K) - fp32(k_mean) )          (BF16 rounding kept)
 *   per (b, h, 64-token block t):  a = max |kc|,  k_scale = a / 127,
 *       k_i8 = clamp(rne(kc * (127 / a)), -127, 127)        (fp32 ops, RNE)
 *   per (b, h, 32-token block s) of raw Q (no smoothing, no softmax scale):
 *       q_scale = max|Q| / 127,  q_i8 = clamp(rne(Q * (127 / max|Q|)), -127, 127)
 *   A block whose absmax is 0 (or whose 127/a overflows) gets scale 0, codes 0.
 *   The last block of a sequence takes its absmax over valid tokens only.
 *
 * Inputs (device): q, k bf16 [B,N,H,D] with element strides (sb, sn, sh).
 * Outputs (device, contiguous, written in full including padding):
 *   q_i8    int8  [B,H,Np,D]   head-major; rows N..Np-1 are 0
 *   q_scale fp32  [B,H,Np/32]  blocks past the end of the sequence are 0
 *   k_i8    int8  [B,H,Np,D]   rows N..Np-1 are 0
 *   k_scale fp32  [B,H,Np/64]
 *   k_mean  bf16  [B,H,D]
 * workspace: device, >= sage_quant_qk_workspace_size(B,N,H,D) bytes, counters
 * zero (see above).
 * The channel sum is the exact sum of the bf16 values rounded once to fp64, for
 * every input, so the mean bits never depend on a summation order.  Plain fp64
 * accumulation is that sum when the channel's sum of |x| (accumulated in fp64
 * alongside) is below u * 2^52, u being the ulp of its smallest non-zero bf16
 * value (true for ordinary activations); a channel that fails this check (a
 * tiny value among large ones) is summed again exactly by a slower path (the
 * head's last statistics workgroup re-reads that channel: ~N / 256 dependent
 * integer additions per thread).
 */
int sage_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                  const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                  int B, int N, int H, int D,
                  int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, uint16_t* k_mean,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_quant_qk_ex -- sage_quant_qk with the scale granularities as arguments
 * (finer steps toward the per-thread scales of the report's §02 stage 03).
 * q_block = SAGE_Q_BLOCK (32) or SAGE_Q_TOKEN (1): q_scale is fp32
 * [B,H,Np/q_block]; with 1, one scale per token,
 *     q_scale = max_d |Q[t,d]| / 127,  q_i8 = clamp(rne(Q * (127 / max_d |Q[t,d]|)), -127, 127).
 * k_block = SAGE_K_BLOCK (64) or SAGE_K_FINE (16): k_scale is fp32
 * [B,H,Np/k_block], the same absmax rule over k_block centred tokens.
 * The zero rule is unchanged (entries for blocks wholly beyond N are 0); the
 * Q outputs do not depend on k_block nor the K outputs on q_block, and
 * (SAGE_Q_BLOCK, SAGE_K_BLOCK) is sage_quant_qk bit for bit.  Other values
 * return SAGE_ERR_UNSUPPORTED.
 */
int sage_quant_qk_ex(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                     const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                     int B, int N, int H, int D,
                     int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, uint16_t* k_mean,
                     void* workspace, size_t workspace_bytes, int q_block, int k_block,
                     void* stream);

/*
 * sage_quant_qk_static -- sage_quant_qk for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * outputs bit for bit.  The workspace is a static device array of
 * SAGE_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; the call allocates nothing (its first call on a device also
 * zero-fills that device's array with a small kernel on `stream`).
 * Call with the stream's device current.  Problems whose workspace
 * (sage_quant_qk_workspace_size) exceeds SAGE_STATIC_SCRATCH_BYTES return
 * SAGE_ERR_WORKSPACE without enqueuing anything; other errors as sage_quant_qk.
 * Every call on a GPU uses that GPU's one array: calls that may overlap on one
 * GPU (other streams, other threads) race and must not be issued.
 */
#define SAGE_STATIC_SCRATCH_BYTES (16u << 20)
int sage_quant_qk_static(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                         const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                         int B, int N, int H, int D,
                         int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                         uint16_t* k_mean, void* stream);

/*
 * sage_quant_q -- the Q half of sage_quant_qk_ex alone.  Q's codes and scales
 * depend only on Q's own blocks (no statistics over the sequence), so under
 * sequence parallelism (the "FLUX 3 Action" SGLang page, §3.1 Multi-GPU: the
 * joint sequence is split and K/V are gathered) each rank quantises its own
 * token shard of Q with this call and feeds it to sage_attn_fwd_shard.
 * Inputs (device): q bf16 [B,N,H,D] with element strides (q_sb, q_sn, q_sh).
 * Outputs (device, contiguous, written in full including padding):
 *   q_i8 int8 [B,H,Np,D], q_scale fp32 [B,H,Np/q_block], q_block = SAGE_Q_BLOCK
 *   or SAGE_Q_TOKEN; bit-identical to the Q outputs of sage_quant_qk_ex for the
 *   same Q.  No workspace.  Errors as sage_quant_qk_ex.
 */
int sage_quant_q(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                 int B, int N, int H, int D, int8_t* q_i8, float* q_scale, int q_block,
                 void* stream);

/*
 * sage_norm_rope -- the QK RMSNorm + RoPE producer of Q or K ("FLUX 3 Action"
 * SGLang page: a fused QK RMSNorm + RoPE, 4-axis RoPE), storing BF16 NHD
 * directly (report card B).  Per token row x of a head, with weights w and
 * (c, s) = rope[token][pair] for channel pair (2i, 2i+1):
 *   r      = fp32( 1 / sqrt(sum_d x_d^2 / D + eps) )   fp64 sum, add, sqrt, divide
 *   u_d    = bf16( bf16(x_d * r) * w_d )                fp32 products
 *   y_2i   = bf16( u_2i * c - u_2i+1 * s )              fp32: products, then sum
 *   y_2i+1 = bf16( u_2i * s + u_2i+1 * c )
 * i.e. the eager composition with each of its bf16 roundings kept.  The fp64
 * sum of squares is exact, and so independent of reduction order, when
 * sum_d x_d^2 < u^2 * 2^53 for u the smallest bf16 ulp among the row's
 * non-zero values (a row of O(1) values holding a value below ~2^-20 of
 * them can break it; the result then still differs from the exact one only
 * through the fp64 rounding of that sum).
 * Inputs (device): x bf16 [B,N,H,D] (strided); w bf16 [D]; rope fp32
 * [N][D/2][2] = (cos, sin), the same for every batch entry and head; eps
 * finite and >= 0 (else SAGE_ERR_VALUE).  w and rope 16-byte aligned.
 * Output (device): y bf16 [B,N,H,D] with element strides (y_sb, y_sn, y_sh),
 * unit d-stride; it must not overlap x, w or rope.
 */
int sage_norm_rope(const void* x, int64_t x_sb, int64_t x_sn, int64_t x_sh,
                   int B, int N, int H, int D,
                   const uint16_t* w, const float* rope, float eps,
                   void* y, int64_t y_sb, int64_t y_sn, int64_t y_sh, void* stream);

/*
 * sage_norm_rope_quant_qk -- the producer fused into the quantiser: takes the
 * pre-norm Q and K, applies sage_norm_rope to each (weights wq and wk, the
 * same rope table and eps) while loading, and writes what sage_quant_qk_ex
 * writes for the producer's BF16 outputs, bit for bit, without storing them.
 * K is read twice (its mean needs the whole head), Q once.
 * Arguments: those of sage_quant_qk_ex plus wq, wk, rope and eps, checked as
 * for sage_norm_rope; the workspace is sage_norm_rope_quant_qk_workspace_size
 * bytes (it also carries each K row's r from the first K pass to the second).
 */
int sage_norm_rope_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                            const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                            int B, int N, int H, int D,
                            const uint16_t* wq, const uint16_t* wk, const float* rope, float eps,
                            int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                            uint16_t* k_mean, void* workspace, size_t workspace_bytes,
                            int q_block, int k_block, void* stream);

/*
 * sage_quant_v -- V smoothing + FP8 E4M3 V, transposed, padded and permuted
 * (report card C "V alias + tiled transpose"; E4M3 per the A10 FLUX.1 page §1.1).
 *
 *   v_mean[b,h,d]  = fp32( fp64(sum over N tokens of V) / N )   (exact sum,
 *                    rounded once to fp64, as for k_mean)
 *   a              = max(|max_n V - v_mean|, |min_n V - v_mean|)   (fp32)
 *   v_scale[b,h,d] = a / 448
 *   code           = E4M3FN( fp32(V - v_mean) * (448 / a) )  RNE, saturating,
 *                    sign kept; a == 0 (or 448/a overflowing) gives scale 0 and
 *                    codes 0x00.
 *
 * Input (device): v bf16 [B,N,H,D] with element strides; may alias a column
 * slice of a wider projection output.
 * Outputs (device, contiguous):
 *   v_fp8   uint8 [B,H,D,Np]  token t of 64-block g at column 64*g + sage_v_slot(t % 64);
 *                             padding columns hold 0x00
 *   v_scale fp32  [B,H,D]
 *   v_mean  fp32  [B,H,D]
 * workspace: as for sage_quant_qk (counters zero before first use), sized by
 * sage_quant_v_workspace_size.
 */
int sage_quant_v(const void* v, int64_t v_sb, int64_t v_sn, int64_t v_sh,
                 int B, int N, int H, int D,
                 uint8_t* v_fp8, float* v_scale, float* v_mean,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_attn_fwd -- fused non-causal attention on the quantised operands
 * (report §02 stage 03: INT8 QK, FP8 PV, FP32 accumulation, V smooth).
 *
 * For query i of head (b, h), over 64-key tiles in ascending order:
 *   s_j = (sum_d q_i8[i,d] k_i8[j,d]) * q_scale[i/32] * k_scale[j/64] * sm_scale
 *   m   = running row max including the current tile; alpha = exp(m_old - m)
 *   p_j = exp(s_j - m);  l = alpha*l + sum p_j  (fp32, unquantised p)
 *   acc = alpha*acc + sum_j E4M3(448 p_j) * E4M3 V_j   (FP8 MFMA, fp32 accum)
 *   out[b,i,h,d] = bf16( acc[d] / (448 l) * v_scale[d] + v_mean[d] )   (RNE)
 * Keys at or beyond N are masked out (excluded from max and sums).
 *
 * Inputs (device): the outputs of sage_quant_qk and sage_quant_v for the same
 * B, N, H, D.  sm_scale <= 0 selects 1/sqrt(D).
 * Output (device): out bf16 [B,N,H,D] with element strides (o_sb, o_sn, o_sh),
 * unit stride over d (e.g. a contiguous NHD tensor).
 */
int sage_attn_fwd(const int8_t* q_i8, const float* q_scale,
                  const int8_t* k_i8, const float* k_scale,
                  const uint8_t* v_fp8, const float* v_scale, const float* v_mean,
                  int B, int N, int H, int D, float sm_scale,
                  void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh, void* stream);

/* sage_attn_fwd on the outputs of sage_quant_qk_ex with the same q_block and
 * k_block: s_j uses q_scale[i / q_block] * k_scale[j / k_block].  The running
 * max is still taken per 64-key tile.  (SAGE_Q_BLOCK, SAGE_K_BLOCK) is
 * sage_attn_fwd; values other than those of sage_quant_qk_ex return
 * SAGE_ERR_UNSUPPORTED. */
int sage_attn_fwd_ex(const int8_t* q_i8, const float* q_scale,
                     const int8_t* k_i8, const float* k_scale,
                     const uint8_t* v_fp8, const float* v_scale, const float* v_mean,
                     int B, int N, int H, int D, float sm_scale,
                     void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh, int q_block, int k_block,
                     void* stream);

/*
 * sage_attn_fwd_shard -- sage_attn_fwd_ex for Nq queries against Nk keys: the
 * attention of one rank under sequence parallelism (the "FLUX 3 Action"
 * SGLang page, §3.1 Multi-GPU: the joint sequence is split and K/V are
 * gathered), i.e. its own query shard against the whole gathered sequence.
 * Inputs (device):
 *   q_i8 int8 [B,H,Npq,D], q_scale fp32 [B,H,Npq/q_block]  (Npq = padded Nq),
 *     e.g. from sage_quant_q on the rank's Q shard;
 *   k_i8 int8 [B,H,Npk,D], k_scale fp32 [B,H,Npk/k_block], v_fp8 uint8
 *     [B,H,D,Npk], v_scale / v_mean fp32 [B,H,D]  (Npk = padded Nk): the
 *     quantised K and V of the whole sequence.
 * Output (device): out bf16 [B,Nq,H,D] with element strides (o_sb, o_sn, o_sh).
 * Query row i of the shard is computed exactly as row i0 + i of sage_attn_fwd_ex
 * over the whole sequence when the shard starts at token i0 (a multiple of
 * q_block) and its Q codes and scales are that sequence's: the key loop, its
 * tile order and every rounding are the same.  Nq == Nk is sage_attn_fwd_ex.
 * Errors as sage_attn_fwd_ex, with both Nq and Nk checked.
 */
int sage_attn_fwd_shard(const int8_t* q_i8, const float* q_scale, int Nq,
                        const int8_t* k_i8, const float* k_scale,
                        const uint8_t* v_fp8, const float* v_scale, const float* v_mean, int Nk,
                        int B, int H, int D, float sm_scale,
                        void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh, int q_block,
                        int k_block, void* stream);

/*
 * sage_quant_rows_fp8 -- row-wise E4M3 quantisation of a bf16 matrix (report
 * §02 stage 02; SGLang page: per-token activation scales, one scale per
 * weight output row).  For each row m of x (K values):
 *   a = max_k |x[m,k]|,  scales[m] = a / 448,
 *   codes[m,k] = E4M3FN( fp32(x[m,k]) * fp32(448 / a) )   RNE, saturating;
 * a == 0 (or 448 / a overflowing) gives scale 0 and codes 0x00.  The rule is
 * that of sage_quant_v.
 * Input (device): x bf16 [M, ldx] row-major (ldx >= K, multiple of 8),
 * 16-byte aligned.  Outputs (device): codes uint8 [M, K] contiguous (16-byte
 * aligned), scales fp32 [M].  Supported: 1 <= M, 8 <= K <= 16384, K % 8 == 0.
 */
int sage_quant_rows_fp8(const void* x, int64_t ldx, int M, int K, uint8_t* codes, float* scales,
                        void* stream);

/*
 * sage_gemm_fp8_rowwise -- the scaled FP8 GEMM of a row-wise FP8 projection:
 *   out[m,n] = bf16( (sum_k x8[m,k] w8[n,k]) * x_scale[m] * w_scale[n] + bias[n] )
 * with E4M3 codes from sage_quant_rows_fp8, the sum accumulated in fp32 on the
 * matrix cores, the scales applied in fp32 in that order, bias bf16 [N] (or
 * NULL), RNE to bf16.  out may be a column slice of a wider buffer (e.g. the
 * V + MLP projection whose V part sage_quant_v then reads in place).
 * Inputs (device): x8 uint8 [M, K], w8 uint8 [N, K] (row-major, 16-byte
 * aligned), x_scale fp32 [M], w_scale fp32 [N] (16-byte aligned), bias
 * (8-byte aligned).  Output (device): out bf16 [M, ldo] row-major, ldo >= N,
 * ldo % 4 == 0, 8-byte aligned; it must not overlap an input.
 * Supported: M >= 1, N >= 4 with N % 4 == 0, K >= 128 with K % 128 == 0,
 * M, N <= 2^24 (else SAGE_ERR_UNSUPPORTED / SAGE_ERR_SHAPE).
 */
int sage_gemm_fp8_rowwise(const uint8_t* x8, const float* x_scale, int M, const uint8_t* w8,
                          const float* w_scale, int N, int K, const void* bias, void* out,
                          int64_t ldo, void* stream);

/* Launch shape that sage_attn_fwd uses for these sizes on the current device:
 * waves per workgroup (32 queries each) and workgroups launched.  Eight waves
 * (256 queries per workgroup, one per CU) when the grid is at least eight such
 * workgroups per CU deep, else four (128 queries, two per CU: finer load
 * balance for shallow grids).  Without a device a 256-CU part is assumed.
 * The shape depends on the queries only: for sage_attn_fwd_shard pass N = Nq.
 * Returns SAGE_OK, SAGE_ERR_NULL, or the shape status of sage_attn_fwd. */
int sage_attn_launch_shape(int B, int N, int H, int D, int* waves_per_workgroup,
                           int* workgroups);

/* Benchmark hook (process-wide, not meant for concurrent callers): forces the
 * workgroup size of later sage_attn_fwd* launches (0: chosen per launch as
 * sage_attn_launch_shape describes, 4 or 8 waves).  The output does not depend
 * on it.  Returns SAGE_OK or SAGE_ERR_VALUE. */
int sage_attn_tuning(int waves_per_workgroup);

/* Benchmark hook (process-wide, like sage_attn_tuning): forces the
 * instruction schedule of later sage_attn_fwd* launches: 0 the library's
 * default (2), 1 the compiler's own order of each key step, 2 each step's
 * MFMAs spread through its softmax instructions (the previous tile's P.V
 * first).  The output does not depend on it (the same operations on the same
 * values).
 * Returns SAGE_OK or SAGE_ERR_VALUE. */
int sage_attn_schedule(int schedule);

/* Host-only argument checks of the three entry points: same arguments (less
 * the stream), same status codes, no HIP calls; usable without a GPU. */
int sage_validate_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                           const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                           int B, int N, int H, int D,
                           const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                           const float* k_scale, const uint16_t* k_mean,
                           const void* workspace, size_t workspace_bytes);
int sage_validate_quant_v(const void* v, int64_t v_sb, int64_t v_sn, int64_t v_sh,
                          int B, int N, int H, int D,
                          const uint8_t* v_fp8, const float* v_scale, const float* v_mean,
                          const void* workspace, size_t workspace_bytes);
int sage_validate_attn_fwd(const int8_t* q_i8, const float* q_scale,
                           const int8_t* k_i8, const float* k_scale,
                           const uint8_t* v_fp8, const float* v_scale, const float* v_mean,
                           int B, int N, int H, int D,
                           const void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh);
/* The same checks for the _ex entry points (q_block and k_block last). */
int sage_validate_quant_qk_ex(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                              const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                              int B, int N, int H, int D,
                              const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                              const float* k_scale, const uint16_t* k_mean,
                              const void* workspace, size_t workspace_bytes, int q_block,
                              int k_block);
int sage_validate_attn_fwd_ex(const int8_t* q_i8, const float* q_scale,
                              const int8_t* k_i8, const float* k_scale,
                              const uint8_t* v_fp8, const float* v_scale, const float* v_mean,
                              int B, int N, int H, int D,
                              const void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
                              int q_block, int k_block);

int sage_validate_quant_q(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                          int B, int N, int H, int D, const int8_t* q_i8, const float* q_scale,
                          int q_block);
int sage_validate_attn_fwd_shard(const int8_t* q_i8, const float* q_scale, int Nq,
                                 const int8_t* k_i8, const float* k_scale,
                                 const uint8_t* v_fp8, const float* v_scale, const float* v_mean,
                                 int Nk, int B, int H, int D,
                                 const void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
                                 int q_block, int k_block);

int sage_validate_norm_rope(const void* x, int64_t x_sb, int64_t x_sn, int64_t x_sh,
                            int B, int N, int H, int D,
                            const uint16_t* w, const float* rope, float eps,
                            const void* y, int64_t y_sb, int64_t y_sn, int64_t y_sh);
int sage_validate_norm_rope_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                                     const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                                     int B, int N, int H, int D,
                                     const uint16_t* wq, const uint16_t* wk, const float* rope,
                                     float eps, const int8_t* q_i8, const float* q_scale,
                                     const int8_t* k_i8, const float* k_scale,
                                     const uint16_t* k_mean, const void* workspace,
                                     size_t workspace_bytes, int q_block, int k_block);

int sage_validate_quant_rows_fp8(const void* x, int64_t ldx, int M, int K, const uint8_t* codes,
                                 const float* scales);
int sage_validate_gemm_fp8_rowwise(const uint8_t* x8, const float* x_scale, int M,
                                   const uint8_t* w8, const float* w_scale, int N, int K,
                                   const void* bias, const void* out, int64_t ldo);

/* Static, never-NULL description of a status code. */
const char* sage_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* SAGE_H */
