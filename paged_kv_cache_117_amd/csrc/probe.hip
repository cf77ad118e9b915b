// pa_probe_read: a read-only bandwidth probe, the measured ceiling that the
// decode kernels' HBM figures are read against.  Not part of the paged
// attention method: it reads memory and keeps a digest, nothing else.
//
// Two access patterns:
//  * sequential: a grid-stride sweep of 16-byte non-temporal loads, four per
//    thread in flight -- the best a plain stream of reads reaches;
//  * 4 KiB gather: each wavefront reads whole 4 KiB chunks (64 lanes x 16
//    bytes x 4) in a caller-given order, four chunks in flight -- the shape of
//    the decode gather, where a 16-slot tile of one KV head (16 x 128 dims x 2
//    bytes) is one contiguous 4 KiB run for K and one for V, at block
//    positions the block tables scatter over the pool.
// Each thread XORs what it reads and stores one 32-bit word, so the loads
// cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChunk16 = 256;  // 16-byte vectors per 4 KiB chunk
constexpr int kInflight = 4;   // chunks in flight per wavefront

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }

__global__ __launch_bounds__(kThreads) void probe_sequential(const u32x4* __restrict__ a, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 x0 = load_nt(a + i), x1 = load_nt(a + i + stride);
    const u32x4 x2 = load_nt(a + i + 2 * stride), x3 = load_nt(a + i + 3 * stride);
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  for (; i < n16; i += stride) acc ^= load_nt(a + i);
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Wavefront w of W takes positions w, w + W, ... of `order`; entries outside
// [0, nbuf) (chunks in the buffer) count as nothing: their loads read chunk
// 0 instead (so every load is unconditional and all four chunks stay in
// flight) and the values are dropped.
__global__ __launch_bounds__(kThreads) void probe_gather(const u32x4* __restrict__ a, const int32_t* __restrict__ order,
                                                         int n, int nbuf, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int W = gridDim.x * (kThreads / 64);
  const int w = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  u32x4 acc = {0u, 0u, 0u, 0u};
  int c = w;
  for (; c + (kInflight - 1) * W < n; c += kInflight * W) {
    u32x4 x[kInflight][4];
    bool ok[kInflight];
#pragma unroll
    for (int k = 0; k < kInflight; ++k) {
      const int id = order[c + k * W];
      ok[k] = id >= 0 && id < nbuf;
      const u32x4* p = a + (size_t)(ok[k] ? id : 0) * kChunk16;
#pragma unroll
      for (int j = 0; j < 4; ++j) x[k][j] = load_nt(p + 64 * j + lane);
    }
#pragma unroll
    for (int k = 0; k < kInflight; ++k)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (ok[k]) acc ^= x[k][j];
  }
  for (; c < n; c += W) {
    const int id = order[c];
    if (id < 0 || id >= nbuf) continue;
    const u32x4* p = a + (size_t)id * kChunk16;
#pragma unroll
    for (int j = 0; j < 4; ++j) acc ^= load_nt(p + 64 * j + lane);
  }
  sink[(size_t)blockIdx.x * kThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace
}  // namespace pa

using namespace pa;

extern "C" pa_status_t pa_probe_read(const void* buf, size_t bytes, const int32_t* chunk_order, int num_chunks,
                                     int mode, int workgroups, uint32_t* sink, void* stream) {
  clear_error();
  if (mode != 0 && mode != 1) return fail(PA_ERR_UNSUPPORTED, "pa_probe_read: mode %d (0 sequential, 1 gather)", mode);
  if (workgroups <= 0 || workgroups > (1 << 20))
    return fail(PA_ERR_SHAPE, "pa_probe_read: workgroups=%d", workgroups);
  if (bytes == 0 || bytes % 4096 != 0) return fail(PA_ERR_SHAPE, "pa_probe_read: bytes=%zu (a multiple of 4096)", bytes);
  if (bytes / 4096 > (size_t)INT32_MAX) return fail(PA_ERR_SHAPE, "pa_probe_read: bytes=%zu too large", bytes);
  if (mode == 1 && num_chunks < 0) return fail(PA_ERR_SHAPE, "pa_probe_read: num_chunks=%d", num_chunks);
  if (!buf || !sink || (mode == 1 && num_chunks > 0 && !chunk_order))
    return fail(PA_ERR_NULL, "pa_probe_read: NULL pointer");
  if (((uintptr_t)buf & 15) != 0) return fail(PA_ERR_SHAPE, "pa_probe_read: buffer must be 16-byte aligned");
  const u32x4* a = static_cast<const u32x4*>(buf);
  if (mode == 0)
    hipLaunchKernelGGL(probe_sequential, dim3(workgroups), dim3(kThreads), 0, (hipStream_t)stream, a, bytes / 16,
                       sink);
  else
    hipLaunchKernelGGL(probe_gather, dim3(workgroups), dim3(kThreads), 0, (hipStream_t)stream, a, chunk_order,
                       num_chunks, (int)(bytes / 4096), sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "pa_probe_read: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
