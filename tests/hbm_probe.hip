// Test helper (not part of libsage): plain read kernels that measure what HBM
// delivers to the quantisers' access pattern, against which their measured
// traffic rates are judged.  Each kernel XOR-folds the 16-byte words it reads
// and writes one word per thread, so no read can be optimised away.
//
//   rows: grid (nchunk, H), 256 threads; one head's D = 128 bf16 channels of
//         token n sit at x + (n*H + h)*256 bytes (the NHD layout the
//         quantisers read), 16 lanes per 256-byte row slice, 8 rows in flight
//         per thread: the statistics pass's loads without its arithmetic.
//   flat: a contiguous read of the same bytes, 8 x 16 B in flight per thread.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

__global__ __launch_bounds__(256) void read_rows(const uint4* __restrict__ x, int N, int H, int rpc,
                                                 uint32_t* __restrict__ out) {
  const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x, lr = tid / 16, lc = tid % 16;
  const int r0 = c * rpc, r1 = min(N, r0 + rpc);
  uint32_t acc = 0;
  int r = r0 + lr;
  for (; r + 7 * 16 < r1; r += 8 * 16) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = x[((size_t)(r + u * 16) * H + h) * 16 + lc];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; r < r1; r += 16) {
    const uint4 v = x[((size_t)r * H + h) * 16 + lc];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[((size_t)h * gridDim.x + c) * 256 + tid] = acc;
}

__global__ __launch_bounds__(256) void read_flat(const uint4* __restrict__ x, size_t n16, size_t per_wg,
                                                 uint32_t* __restrict__ out) {
  const size_t b0 = blockIdx.x * per_wg, b1 = min(n16, b0 + per_wg);
  uint32_t acc = 0;
  size_t i = b0 + threadIdx.x;
  for (; i + 7 * 256 < b1; i += 8 * 256) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = x[i + u * 256];
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < b1; i += 256) {
    const uint4 v = x[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// x: N*H*128 bf16 (device); out: >= nchunk*H*256 words.  Returns a hipError_t.
extern "C" int probe_read_rows(const void* x, int N, int H, int nchunk, void* out, void* stream) {
  if (N <= 0 || H <= 0 || nchunk <= 0) return (int)hipErrorInvalidValue;
  const int rpc = (N + nchunk - 1) / nchunk;
  hipLaunchKernelGGL(read_rows, dim3(nchunk, H), dim3(256), 0, (hipStream_t)stream, (const uint4*)x, N, H,
                     rpc, (uint32_t*)out);
  return (int)hipGetLastError();
}

// x: bytes (a multiple of 16, device); out: >= wgs*256 words.
extern "C" int probe_read_flat(const void* x, size_t bytes, int wgs, void* out, void* stream) {
  if (bytes % 16 || wgs <= 0) return (int)hipErrorInvalidValue;
  const size_t n16 = bytes / 16, per = (n16 + wgs - 1) / wgs;
  hipLaunchKernelGGL(read_flat, dim3(wgs), dim3(256), 0, (hipStream_t)stream, (const uint4*)x, n16, per,
                     (uint32_t*)out);
  return (int)hipGetLastError();
}
