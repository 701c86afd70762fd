// C ABI of libsage: argument validation and dispatch to the HIP launchers.
// The contract of every function is documented in include/sage.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "../../include/sage.h"
#include "sage_internal.h"

namespace {

using sage::ceil_div;
using sage::padded_tokens;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, size_t bytes) {
  uintptr_t a = (uintptr_t)p;
  return Range{a, a + bytes};
}
bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(int B, int N, int H, int D) {
  if (B < 1 || N < 1 || H < 1) return SAGE_ERR_SHAPE;
  if (D != 64 && D != 128) return SAGE_ERR_UNSUPPORTED;
  const int64_t elems = (int64_t)B * H * padded_tokens(N) * D;
  if (elems >= ((int64_t)1 << 31)) return SAGE_ERR_SHAPE;
  return SAGE_OK;
}

// Strides of size-1 dimensions are never used; the others must be positive
// and keep 16-byte alignment of every 8-element (16-byte) row chunk.
int check_strides(int B, int N, int H, int64_t sb, int64_t sn, int64_t sh) {
  const int64_t s[3] = {B > 1 ? sb : 0, N > 1 ? sn : 0, H > 1 ? sh : 0};
  const int sz[3] = {B, N, H};
  for (int i = 0; i < 3; ++i) {
    if (sz[i] > 1 && s[i] <= 0) return SAGE_ERR_STRIDE;
    if (s[i] % 8 != 0) return SAGE_ERR_ALIGN;
  }
  return SAGE_OK;
}

// Bytes spanned by a bf16 [B,N,H,D] view.
size_t view_bytes(int B, int N, int H, int D, int64_t sb, int64_t sn, int64_t sh) {
  const int64_t last = (B > 1 ? (int64_t)(B - 1) * sb : 0) + (N > 1 ? (int64_t)(N - 1) * sn : 0) +
                       (H > 1 ? (int64_t)(H - 1) * sh : 0) + D;
  return (size_t)last * 2;
}

bool any_overlap(const Range* outs, int n_out, const Range* ins, int n_in) {
  for (int i = 0; i < n_out; ++i) {
    for (int j = i + 1; j < n_out; ++j)
      if (overlaps(outs[i], outs[j])) return true;
    for (int j = 0; j < n_in; ++j)
      if (overlaps(outs[i], ins[j])) return true;
  }
  return false;
}

int status_of(hipError_t e) { return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP; }

// Checks shared by sage_quant_qk_ex, sage_norm_rope_quant_qk (nr: the
// workspace requirement differs) and sage_quant_qk_static (with_ws false: the
// workspace is the library's static scratch, not a caller buffer).
int validate_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
                int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N, int H, int D,
                const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                const uint16_t* k_mean, const void* workspace, size_t workspace_bytes, int q_block,
                int k_block, bool nr, bool with_ws = true) {
  if (!q || !k || !q_i8 || !q_scale || !k_i8 || !k_scale || !k_mean || (with_ws && !workspace))
    return SAGE_ERR_NULL;
  int st = check_shape(B, N, H, D);
  if (st != SAGE_OK) return st;
  if (q_block != SAGE_Q_BLOCK && q_block != SAGE_Q_TOKEN) return SAGE_ERR_UNSUPPORTED;
  if (k_block != SAGE_K_BLOCK && k_block != SAGE_K_FINE) return SAGE_ERR_UNSUPPORTED;
  if ((st = check_strides(B, N, H, q_sb, q_sn, q_sh)) != SAGE_OK) return st;
  if ((st = check_strides(B, N, H, k_sb, k_sn, k_sh)) != SAGE_OK) return st;
  if (!aligned16(q) || !aligned16(k) || !aligned16(q_i8) || !aligned16(k_i8) ||
      !aligned16(k_mean) || (with_ws && !aligned16(workspace)) || ((uintptr_t)q_scale & 3u) ||
      ((uintptr_t)k_scale & 3u))
    return SAGE_ERR_ALIGN;
  const size_t need = sage::qk_workspace(B, N, H, D, nr).bytes;
  if (with_ws && workspace_bytes < need) return SAGE_ERR_WORKSPACE;
  const int64_t Np = padded_tokens(N), bh = (int64_t)B * H;
  const Range outs[6] = {range_of(q_i8, bh * Np * D), range_of(q_scale, bh * (Np / q_block) * 4),
                         range_of(k_i8, bh * Np * D), range_of(k_scale, bh * (Np / k_block) * 4),
                         range_of(k_mean, bh * D * 2), range_of(workspace, with_ws ? need : 0)};
  const Range ins[2] = {range_of(q, view_bytes(B, N, H, D, q_sb, q_sn, q_sh)),
                        range_of(k, view_bytes(B, N, H, D, k_sb, k_sn, k_sh))};
  if (any_overlap(outs, 6, ins, 2)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

// ---- sage_quant_qk_static: the quantiser workspace as a static device array ----
// One copy per GPU the library runs on, held until the process ends.  In host
// code this name is a stand-in, not a device address: kernels get the
// per-device address that hipGetSymbolAddress returns (kept in g_scratch).
static __device__ __align__(256) uint8_t scratch[SAGE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

__global__ void zero_words(uint32_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// The current device's scratch address.  On the first call for a device (with
// that device current) it is looked up and the whole array is zeroed on
// `stream`, which orders the fill before the caller's kernels.  nullptr on a
// HIP error.
void* scratch_for_current_device(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev]) return g_scratch[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, stream, (uint32_t*)ptr,
                     (size_t)SAGE_STATIC_SCRATCH_BYTES / 4);
  if (hipGetLastError() != hipSuccess) return nullptr;
  g_scratch[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" {

int sage_get_layout(sage_layout* out) {
  if (!out) return SAGE_ERR_NULL;
  out->bq = SAGE_BQ;
  out->bk = SAGE_BK;
  out->n_pad_multiple = SAGE_NPAD;
  out->perm_version = SAGE_PERM_VERSION;
  return SAGE_OK;
}

int64_t sage_padded_tokens(int64_t N) { return N <= 0 ? 0 : padded_tokens(N); }

int sage_v_slot(int t) {
  if (t < 0 || t > 63) return -1;
  return (((t >> 2) & 1) << 5) | (((t >> 5) & 1) << 4) | (((t >> 3) & 3) << 2) | (t & 3);
}

size_t sage_quant_qk_workspace_size(int B, int N, int H, int D) {
  if (check_shape(B, N, H, D) != SAGE_OK) return 0;
  return sage::qk_workspace(B, N, H, D).bytes;
}

size_t sage_norm_rope_quant_qk_workspace_size(int B, int N, int H, int D) {
  if (check_shape(B, N, H, D) != SAGE_OK) return 0;
  return sage::qk_workspace(B, N, H, D, true).bytes;
}

size_t sage_quant_v_workspace_size(int B, int N, int H, int D) {
  if (check_shape(B, N, H, D) != SAGE_OK) return 0;
  return sage::v_workspace(B, N, H, D).bytes;
}

size_t sage_workspace_zero_bytes(void) { return sage::workspace_zero_bytes(); }


int sage_validate_quant_qk_ex(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                              const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N,
                              int H, int D, const int8_t* q_i8, const float* q_scale,
                              const int8_t* k_i8, const float* k_scale, const uint16_t* k_mean,
                              const void* workspace, size_t workspace_bytes, int q_block,
                              int k_block) {
  return validate_qk(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N, H, D, q_i8, q_scale, k_i8,
                     k_scale, k_mean, workspace, workspace_bytes, q_block, k_block, false);
}

int sage_validate_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
                           int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N, int H, int D,
                           const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                           const float* k_scale, const uint16_t* k_mean, const void* workspace,
                           size_t workspace_bytes) {
  return sage_validate_quant_qk_ex(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N, H, D, q_i8,
                                   q_scale, k_i8, k_scale, k_mean, workspace, workspace_bytes,
                                   SAGE_Q_BLOCK, SAGE_K_BLOCK);
}

int sage_validate_quant_v(const void* v, int64_t v_sb, int64_t v_sn, int64_t v_sh, int B, int N,
                          int H, int D, const uint8_t* v_fp8, const float* v_scale,
                          const float* v_mean, const void* workspace, size_t workspace_bytes) {
  if (!v || !v_fp8 || !v_scale || !v_mean || !workspace) return SAGE_ERR_NULL;
  int st = check_shape(B, N, H, D);
  if (st != SAGE_OK) return st;
  if ((st = check_strides(B, N, H, v_sb, v_sn, v_sh)) != SAGE_OK) return st;
  if (!aligned16(v) || !aligned16(v_fp8) || !aligned16(workspace) || ((uintptr_t)v_scale & 3u) ||
      ((uintptr_t)v_mean & 3u))
    return SAGE_ERR_ALIGN;
  const size_t need = sage::v_workspace(B, N, H, D).bytes;
  if (workspace_bytes < need) return SAGE_ERR_WORKSPACE;
  const int64_t Np = padded_tokens(N), bh = (int64_t)B * H;
  const Range outs[4] = {range_of(v_fp8, bh * D * Np), range_of(v_scale, bh * D * 4),
                         range_of(v_mean, bh * D * 4), range_of(workspace, need)};
  const Range ins[1] = {range_of(v, view_bytes(B, N, H, D, v_sb, v_sn, v_sh))};
  if (any_overlap(outs, 4, ins, 1)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

int sage_validate_attn_fwd_shard(const int8_t* q_i8, const float* q_scale, int Nq,
                                 const int8_t* k_i8, const float* k_scale, const uint8_t* v_fp8,
                                 const float* v_scale, const float* v_mean, int Nk, int B, int H,
                                 int D, const void* out, int64_t o_sb, int64_t o_sn, int64_t o_sh,
                                 int q_block, int k_block) {
  if (!q_i8 || !q_scale || !k_i8 || !k_scale || !v_fp8 || !v_scale || !v_mean || !out)
    return SAGE_ERR_NULL;
  int st = check_shape(B, Nq, H, D);
  if (st != SAGE_OK) return st;
  if ((st = check_shape(B, Nk, H, D)) != SAGE_OK) return st;
  if (q_block != SAGE_Q_BLOCK && q_block != SAGE_Q_TOKEN) return SAGE_ERR_UNSUPPORTED;
  if (k_block != SAGE_K_BLOCK && k_block != SAGE_K_FINE) return SAGE_ERR_UNSUPPORTED;
  if ((st = check_strides(B, Nq, H, o_sb, o_sn, o_sh)) != SAGE_OK) return st;
  if (!aligned16(q_i8) || !aligned16(k_i8) || !aligned16(v_fp8) || !aligned16(out) ||
      ((uintptr_t)q_scale & 3u) || ((uintptr_t)k_scale & 3u) || ((uintptr_t)v_scale & 3u) ||
      ((uintptr_t)v_mean & 3u))
    return SAGE_ERR_ALIGN;
  const int64_t Npq = padded_tokens(Nq), Npk = padded_tokens(Nk), bh = (int64_t)B * H;
  const Range outs[1] = {range_of(out, view_bytes(B, Nq, H, D, o_sb, o_sn, o_sh))};
  const Range ins[7] = {range_of(q_i8, bh * Npq * D),     range_of(q_scale, bh * (Npq / q_block) * 4),
                        range_of(k_i8, bh * Npk * D),     range_of(k_scale, bh * (Npk / k_block) * 4),
                        range_of(v_fp8, bh * D * Npk),    range_of(v_scale, bh * D * 4),
                        range_of(v_mean, bh * D * 4)};
  if (any_overlap(outs, 1, ins, 7)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

int sage_validate_attn_fwd_ex(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                              const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                              const float* v_mean, int B, int N, int H, int D, const void* out,
                              int64_t o_sb, int64_t o_sn, int64_t o_sh, int q_block, int k_block) {
  return sage_validate_attn_fwd_shard(q_i8, q_scale, N, k_i8, k_scale, v_fp8, v_scale, v_mean, N, B,
                                      H, D, out, o_sb, o_sn, o_sh, q_block, k_block);
}

int sage_validate_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                           const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                           const float* v_mean, int B, int N, int H, int D, const void* out,
                           int64_t o_sb, int64_t o_sn, int64_t o_sh) {
  return sage_validate_attn_fwd_ex(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, B, N, H, D,
                                   out, o_sb, o_sn, o_sh, SAGE_Q_BLOCK, SAGE_K_BLOCK);
}

int sage_quant_qk_ex(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
                     int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N, int H, int D,
                     int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, uint16_t* k_mean,
                     void* workspace, size_t workspace_bytes, int q_block, int k_block,
                     void* stream) {
  const int st = sage_validate_quant_qk_ex(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N, H, D,
                                           q_i8, q_scale, k_i8, k_scale, k_mean, workspace,
                                           workspace_bytes, q_block, k_block);
  if (st != SAGE_OK) return st;
  return status_of(sage::launch_quant_qk((const uint16_t*)q, B > 1 ? q_sb : 0, q_sn, H > 1 ? q_sh : 0,
                                         (const uint16_t*)k, B > 1 ? k_sb : 0, k_sn,
                                         H > 1 ? k_sh : 0, B, N, H, D, q_block, k_block, nullptr, q_i8,
                                         q_scale, k_i8,
                                         k_scale, k_mean, workspace, (hipStream_t)stream));
}

int sage_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
                  int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N, int H, int D,
                  int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, uint16_t* k_mean,
                  void* workspace, size_t workspace_bytes, void* stream) {
  return sage_quant_qk_ex(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N, H, D, q_i8, q_scale, k_i8,
                          k_scale, k_mean, workspace, workspace_bytes, SAGE_Q_BLOCK, SAGE_K_BLOCK,
                          stream);
}

int sage_quant_qk_static(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
                         int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N, int H, int D,
                         int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                         uint16_t* k_mean, void* stream) {
  int st = validate_qk(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N, H, D, q_i8, q_scale, k_i8,
                       k_scale, k_mean, nullptr, 0, SAGE_Q_BLOCK, SAGE_K_BLOCK, false, false);
  if (st != SAGE_OK) return st;
  if (sage::qk_workspace(B, N, H, D).bytes > (size_t)SAGE_STATIC_SCRATCH_BYTES) return SAGE_ERR_WORKSPACE;
  void* ws = scratch_for_current_device((hipStream_t)stream);
  if (!ws) return SAGE_ERR_HIP;
  return status_of(sage::launch_quant_qk((const uint16_t*)q, B > 1 ? q_sb : 0, q_sn, H > 1 ? q_sh : 0,
                                         (const uint16_t*)k, B > 1 ? k_sb : 0, k_sn,
                                         H > 1 ? k_sh : 0, B, N, H, D, SAGE_Q_BLOCK, SAGE_K_BLOCK,
                                         nullptr, q_i8, q_scale, k_i8, k_scale, k_mean, ws,
                                         (hipStream_t)stream));
}

int sage_validate_quant_q(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, int B, int N,
                          int H, int D, const int8_t* q_i8, const float* q_scale, int q_block) {
  if (!q || !q_i8 || !q_scale) return SAGE_ERR_NULL;
  int st = check_shape(B, N, H, D);
  if (st != SAGE_OK) return st;
  if (q_block != SAGE_Q_BLOCK && q_block != SAGE_Q_TOKEN) return SAGE_ERR_UNSUPPORTED;
  if ((st = check_strides(B, N, H, q_sb, q_sn, q_sh)) != SAGE_OK) return st;
  if (!aligned16(q) || !aligned16(q_i8) || ((uintptr_t)q_scale & 3u)) return SAGE_ERR_ALIGN;
  const int64_t Np = padded_tokens(N), bh = (int64_t)B * H;
  const Range outs[2] = {range_of(q_i8, bh * Np * D), range_of(q_scale, bh * (Np / q_block) * 4)};
  const Range ins[1] = {range_of(q, view_bytes(B, N, H, D, q_sb, q_sn, q_sh))};
  if (any_overlap(outs, 2, ins, 1)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

int sage_quant_q(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, int B, int N, int H, int D,
                 int8_t* q_i8, float* q_scale, int q_block, void* stream) {
  const int st = sage_validate_quant_q(q, q_sb, q_sn, q_sh, B, N, H, D, q_i8, q_scale, q_block);
  if (st != SAGE_OK) return st;
  return status_of(sage::launch_quant_q((const uint16_t*)q, B > 1 ? q_sb : 0, q_sn, H > 1 ? q_sh : 0,
                                        B, N, H, D, q_block, q_i8, q_scale, (hipStream_t)stream));
}

int sage_quant_v(const void* v, int64_t v_sb, int64_t v_sn, int64_t v_sh, int B, int N, int H, int D,
                 uint8_t* v_fp8, float* v_scale, float* v_mean, void* workspace,
                 size_t workspace_bytes, void* stream) {
  const int st = sage_validate_quant_v(v, v_sb, v_sn, v_sh, B, N, H, D, v_fp8, v_scale, v_mean,
                                       workspace, workspace_bytes);
  if (st != SAGE_OK) return st;
  return status_of(sage::launch_quant_v((const uint16_t*)v, B > 1 ? v_sb : 0, v_sn, H > 1 ? v_sh : 0,
                                        B, N, H, D, v_fp8, v_scale, v_mean, workspace,
                                        (hipStream_t)stream));
}

int sage_attn_fwd_shard(const int8_t* q_i8, const float* q_scale, int Nq, const int8_t* k_i8,
                        const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                        const float* v_mean, int Nk, int B, int H, int D, float sm_scale, void* out,
                        int64_t o_sb, int64_t o_sn, int64_t o_sh, int q_block, int k_block,
                        void* stream) {
  const int st = sage_validate_attn_fwd_shard(q_i8, q_scale, Nq, k_i8, k_scale, v_fp8, v_scale,
                                              v_mean, Nk, B, H, D, out, o_sb, o_sn, o_sh, q_block,
                                              k_block);
  if (st != SAGE_OK) return st;
  if (!(sm_scale > 0.0f)) sm_scale = 1.0f / __builtin_sqrtf((float)D);
  return status_of(sage::launch_attn_fwd(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, B, Nq,
                                         Nk, H, D, q_block, k_block, sm_scale, (uint16_t*)out,
                                         B > 1 ? o_sb : 0, o_sn, H > 1 ? o_sh : 0,
                                         (hipStream_t)stream));
}

int sage_attn_fwd_ex(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                     const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                     const float* v_mean, int B, int N, int H, int D, float sm_scale, void* out,
                     int64_t o_sb, int64_t o_sn, int64_t o_sh, int q_block, int k_block,
                     void* stream) {
  return sage_attn_fwd_shard(q_i8, q_scale, N, k_i8, k_scale, v_fp8, v_scale, v_mean, N, B, H, D,
                             sm_scale, out, o_sb, o_sn, o_sh, q_block, k_block, stream);
}

int sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                  const float* k_scale, const uint8_t* v_fp8, const float* v_scale,
                  const float* v_mean, int B, int N, int H, int D, float sm_scale, void* out,
                  int64_t o_sb, int64_t o_sn, int64_t o_sh, void* stream) {
  return sage_attn_fwd_ex(q_i8, q_scale, k_i8, k_scale, v_fp8, v_scale, v_mean, B, N, H, D, sm_scale,
                          out, o_sb, o_sn, o_sh, SAGE_Q_BLOCK, SAGE_K_BLOCK, stream);
}

int sage_validate_norm_rope(const void* x, int64_t x_sb, int64_t x_sn, int64_t x_sh, int B, int N,
                            int H, int D, const uint16_t* w, const float* rope, float eps,
                            const void* y, int64_t y_sb, int64_t y_sn, int64_t y_sh) {
  if (!x || !w || !rope || !y) return SAGE_ERR_NULL;
  int st = check_shape(B, N, H, D);
  if (st != SAGE_OK) return st;
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps)) return SAGE_ERR_VALUE;
  if ((st = check_strides(B, N, H, x_sb, x_sn, x_sh)) != SAGE_OK) return st;
  if ((st = check_strides(B, N, H, y_sb, y_sn, y_sh)) != SAGE_OK) return st;
  if (!aligned16(x) || !aligned16(y) || !aligned16(w) || !aligned16(rope)) return SAGE_ERR_ALIGN;
  const Range outs[1] = {range_of(y, view_bytes(B, N, H, D, y_sb, y_sn, y_sh))};
  const Range ins[3] = {range_of(x, view_bytes(B, N, H, D, x_sb, x_sn, x_sh)),
                        range_of(w, (size_t)D * 2), range_of(rope, (size_t)N * D * 4)};
  if (any_overlap(outs, 1, ins, 3)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

int sage_norm_rope(const void* x, int64_t x_sb, int64_t x_sn, int64_t x_sh, int B, int N, int H,
                   int D, const uint16_t* w, const float* rope, float eps, void* y, int64_t y_sb,
                   int64_t y_sn, int64_t y_sh, void* stream) {
  const int st = sage_validate_norm_rope(x, x_sb, x_sn, x_sh, B, N, H, D, w, rope, eps, y, y_sb,
                                         y_sn, y_sh);
  if (st != SAGE_OK) return st;
  return status_of(sage::launch_norm_rope((const uint16_t*)x, B > 1 ? x_sb : 0, N > 1 ? x_sn : 0,
                                          H > 1 ? x_sh : 0, B, N, H, D, w, rope, (double)eps,
                                          (uint16_t*)y, B > 1 ? y_sb : 0, N > 1 ? y_sn : 0,
                                          H > 1 ? y_sh : 0, (hipStream_t)stream));
}

int sage_validate_norm_rope_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh,
                                     const void* k, int64_t k_sb, int64_t k_sn, int64_t k_sh,
                                     int B, int N, int H, int D, const uint16_t* wq,
                                     const uint16_t* wk, const float* rope, float eps,
                                     const int8_t* q_i8, const float* q_scale, const int8_t* k_i8,
                                     const float* k_scale, const uint16_t* k_mean,
                                     const void* workspace, size_t workspace_bytes, int q_block,
                                     int k_block) {
  int st = validate_qk(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N, H, D, q_i8, q_scale, k_i8,
                       k_scale, k_mean, workspace, workspace_bytes, q_block, k_block, true);
  if (st != SAGE_OK) return st;
  if (!wq || !wk || !rope) return SAGE_ERR_NULL;
  if (!(eps >= 0.0f) || !__builtin_isfinite(eps)) return SAGE_ERR_VALUE;
  if (!aligned16(wq) || !aligned16(wk) || !aligned16(rope)) return SAGE_ERR_ALIGN;
  const int64_t Np = padded_tokens(N), bh = (int64_t)B * H;
  const Range outs[6] = {range_of(q_i8, bh * Np * D), range_of(q_scale, bh * (Np / q_block) * 4),
                         range_of(k_i8, bh * Np * D), range_of(k_scale, bh * (Np / k_block) * 4),
                         range_of(k_mean, bh * D * 2),
                         range_of(workspace, sage::qk_workspace(B, N, H, D, true).bytes)};
  const Range ins[3] = {range_of(wq, (size_t)D * 2), range_of(wk, (size_t)D * 2),
                        range_of(rope, (size_t)N * D * 4)};
  if (any_overlap(outs, 6, ins, 3)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

int sage_norm_rope_quant_qk(const void* q, int64_t q_sb, int64_t q_sn, int64_t q_sh, const void* k,
                            int64_t k_sb, int64_t k_sn, int64_t k_sh, int B, int N, int H, int D,
                            const uint16_t* wq, const uint16_t* wk, const float* rope, float eps,
                            int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                            uint16_t* k_mean, void* workspace, size_t workspace_bytes, int q_block,
                            int k_block, void* stream) {
  const int st = sage_validate_norm_rope_quant_qk(q, q_sb, q_sn, q_sh, k, k_sb, k_sn, k_sh, B, N,
                                                  H, D, wq, wk, rope, eps, q_i8, q_scale, k_i8,
                                                  k_scale, k_mean, workspace, workspace_bytes,
                                                  q_block, k_block);
  if (st != SAGE_OK) return st;
  const sage::NormRope nr{wq, wk, rope, (double)eps};
  return status_of(sage::launch_quant_qk((const uint16_t*)q, B > 1 ? q_sb : 0, q_sn, H > 1 ? q_sh : 0,
                                         (const uint16_t*)k, B > 1 ? k_sb : 0, k_sn,
                                         H > 1 ? k_sh : 0, B, N, H, D, q_block, k_block, &nr, q_i8,
                                         q_scale, k_i8, k_scale, k_mean, workspace,
                                         (hipStream_t)stream));
}

int sage_validate_quant_rows_fp8(const void* x, int64_t ldx, int M, int K, const uint8_t* codes,
                                 const float* scales) {
  if (!x || !codes || !scales) return SAGE_ERR_NULL;
  if (M < 1 || K < 8 || (int64_t)M * K >= ((int64_t)1 << 40)) return SAGE_ERR_SHAPE;
  if (K % 8 != 0 || K > 16384) return SAGE_ERR_UNSUPPORTED;
  if (ldx < K) return SAGE_ERR_STRIDE;
  if (ldx % 8 != 0 || !aligned16(x) || !aligned16(codes) || ((uintptr_t)scales & 3u))
    return SAGE_ERR_ALIGN;
  const Range outs[2] = {range_of(codes, (size_t)M * K), range_of(scales, (size_t)M * 4)};
  const Range ins[1] = {range_of(x, ((size_t)(M - 1) * ldx + K) * 2)};
  if (any_overlap(outs, 2, ins, 1)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

int sage_quant_rows_fp8(const void* x, int64_t ldx, int M, int K, uint8_t* codes, float* scales,
                        void* stream) {
  const int st = sage_validate_quant_rows_fp8(x, ldx, M, K, codes, scales);
  if (st != SAGE_OK) return st;
  return status_of(sage::launch_quant_rows_fp8((const uint16_t*)x, ldx, M, K, codes, scales,
                                               (hipStream_t)stream));
}

int sage_validate_gemm_fp8_rowwise(const uint8_t* x8, const float* x_scale, int M,
                                   const uint8_t* w8, const float* w_scale, int N, int K,
                                   const void* bias, const void* out, int64_t ldo) {
  if (!x8 || !x_scale || !w8 || !w_scale || !out) return SAGE_ERR_NULL;
  if (M < 1 || N < 1 || K < 1 || M > (1 << 24) || N > (1 << 24)) return SAGE_ERR_SHAPE;
  if (K % 128 != 0 || N % 4 != 0) return SAGE_ERR_UNSUPPORTED;
  if (ldo < N) return SAGE_ERR_STRIDE;
  if (ldo % 4 != 0 || !aligned16(x8) || !aligned16(w8) || !aligned16(w_scale) ||
      ((uintptr_t)x_scale & 3u) || ((uintptr_t)bias & 7u) || ((uintptr_t)out & 7u))
    return SAGE_ERR_ALIGN;
  const Range outs[1] = {range_of(out, ((size_t)(M - 1) * ldo + N) * 2)};
  const Range ins[5] = {range_of(x8, (size_t)M * K), range_of(x_scale, (size_t)M * 4),
                        range_of(w8, (size_t)N * K), range_of(w_scale, (size_t)N * 4),
                        range_of(bias, bias ? (size_t)N * 2 : 0)};
  if (any_overlap(outs, 1, ins, 5)) return SAGE_ERR_OVERLAP;
  return SAGE_OK;
}

int sage_gemm_fp8_rowwise(const uint8_t* x8, const float* x_scale, int M, const uint8_t* w8,
                          const float* w_scale, int N, int K, const void* bias, void* out,
                          int64_t ldo, void* stream) {
  const int st = sage_validate_gemm_fp8_rowwise(x8, x_scale, M, w8, w_scale, N, K, bias, out, ldo);
  if (st != SAGE_OK) return st;
  return status_of(sage::launch_gemm_fp8_rowwise(x8, x_scale, M, w8, w_scale, N, K,
                                                 (const uint16_t*)bias, (uint16_t*)out, ldo,
                                                 (hipStream_t)stream));
}

int sage_attn_launch_shape(int B, int N, int H, int D, int* waves_per_workgroup,
                           int* workgroups) {
  if (!waves_per_workgroup || !workgroups) return SAGE_ERR_NULL;
  const int st = check_shape(B, N, H, D);
  if (st != SAGE_OK) return st;
  sage::attn_shape(B, N, H, D, waves_per_workgroup, workgroups);
  return SAGE_OK;
}

int sage_attn_schedule(int schedule) {
  if (schedule < 0 || schedule > 2) return SAGE_ERR_VALUE;
  sage::set_attn_schedule(schedule);
  return SAGE_OK;
}

int sage_attn_tuning(int waves_per_workgroup) {
  if (waves_per_workgroup != 0 && waves_per_workgroup != 4 && waves_per_workgroup != 8)
    return SAGE_ERR_VALUE;
  sage::set_attn_waves(waves_per_workgroup);
  return SAGE_OK;
}

const char* sage_status_string(int status) {
  switch (status) {
    case SAGE_OK: return "ok";
    case SAGE_ERR_NULL: return "a required pointer is NULL";
    case SAGE_ERR_SHAPE: return "B, N or H < 1, or B*H*Np*D >= 2^31";
    case SAGE_ERR_UNSUPPORTED: return "unsupported head dimension (D must be 64 or 128)";
    case SAGE_ERR_STRIDE: return "a stride of a dimension longer than 1 is not positive";
    case SAGE_ERR_ALIGN: return "a pointer or stride breaks 16-byte alignment";
    case SAGE_ERR_WORKSPACE: return "workspace missing or smaller than required";
    case SAGE_ERR_OVERLAP: return "an output overlaps an input or another output";
    case SAGE_ERR_HIP: return "a HIP launch or runtime call failed";
    case SAGE_ERR_VALUE: return "a scalar argument is out of range (eps must be finite and >= 0)";
    default: return "unknown status";
  }
}

}  // extern "C"
