// pa_write_kv and pa_copy_blocks: byte-exact moves of K/V rows and blocks.
//
// Write (reshape-and-cache): every new token's K and V rows go to the slot
// the block manager assigned, one launch for the whole step (PagedAttention
// (tensortonic), "5. Reading the Cache During Attention"; PagedAttention and
// vLLM: Paging the KV Cache Like an OS, "Step 5", the fused write kernel).
// Copy: whole K and V blocks for copy-on-write, all pairs of a step in one
// launch (same page, "Step 4" and the batched copy kernel of "Step 5").
//
// Swap: whole blocks between the device pool and a pool in pinned host memory
// (either direction), all pairs in one launch, for preemption by swapping
// (PagedAttention: Virtual Memory for the KV Cache, "Scheduling and
// preemption": evicted blocks are copied to CPU memory and brought back
// later; Batching and PagedAttention, FAQ on running out of blocks).
//
// All are pure data movement: 16-byte vector loads/stores, one token (write)
// or one block slice (copy, swap) per workgroup, so each workgroup moves
// contiguous rows.  Out-of-range slots / block ids are skipped, never
// dereferenced.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_kernels.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void write_kv_kernel(char* __restrict__ kp, char* __restrict__ vp,
                                                            const char* __restrict__ kn,
                                                            const char* __restrict__ vn,
                                                            const int64_t* __restrict__ slots, int num_kv_heads,
                                                            int row_bytes, int block_size, int64_t num_slots) {
  const int i = blockIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / block_size;
  const int off = (int)(slot % block_size);
  const int per_row = row_bytes >> 4;  // 16-byte vectors per (token, head) row
  const int n = num_kv_heads * per_row;
  for (int v = threadIdx.x; v < n; v += kThreads) {
    const int h = v / per_row;
    const int c = v - h * per_row;
    const size_t dst = (((size_t)blk * num_kv_heads + h) * block_size + off) * (size_t)row_bytes + (size_t)c * 16;
    const size_t src = ((size_t)i * num_kv_heads + h) * (size_t)row_bytes + (size_t)c * 16;
    const uint4 kx = *reinterpret_cast<const uint4*>(kn + src);
    const uint4 vx = *reinterpret_cast<const uint4*>(vn + src);
    *reinterpret_cast<uint4*>(kp + dst) = kx;
    *reinterpret_cast<uint4*>(vp + dst) = vx;
  }
}

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(char* __restrict__ kp, char* __restrict__ vp,
                                                               const int32_t* __restrict__ pairs,
                                                               size_t block_bytes, int num_blocks) {
  const int p = blockIdx.x;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  char* pool = blockIdx.z ? vp : kp;
  const uint4* s = reinterpret_cast<const uint4*>(pool + (size_t)src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(pool + (size_t)dst * block_bytes);
  const size_t n = block_bytes >> 4;
  for (size_t v = (size_t)blockIdx.y * kThreads + threadIdx.x; v < n; v += (size_t)gridDim.y * kThreads) d[v] = s[v];
}

// The fused step's write when its decode does not run the stream kernel:
// each sequence's new K and V rows (k_new[s], v_new[s]) go to its last
// position L-1, found through its block table (one workgroup per
// sequence).  Sequences with L outside [1, max_ctx] or an out-of-range block
// id write nothing.
__global__ __launch_bounds__(kThreads) void write_last_kernel(char* __restrict__ kp, char* __restrict__ vp,
                                                              const char* __restrict__ kn,
                                                              const char* __restrict__ vn,
                                                              const int32_t* __restrict__ bt,
                                                              const int32_t* __restrict__ cl, int maxb, int max_ctx,
                                                              int num_kv_heads, int row_bytes, int lbs,
                                                              int num_blocks) {
  const int s = blockIdx.x;
  const int L = cl[s];
  if (L < 1 || L > max_ctx) return;
  const int pos = L - 1;
  const int blk = bt[(size_t)s * maxb + (pos >> lbs)];
  if (blk < 0 || blk >= num_blocks) return;
  const int off = pos & ((1 << lbs) - 1);
  const int per_row = row_bytes >> 4;
  const int n = num_kv_heads * per_row;
  for (int v = threadIdx.x; v < n; v += kThreads) {
    const int h = v / per_row;
    const int c = v - h * per_row;
    const size_t dst = ((((size_t)blk * num_kv_heads + h) << lbs) + off) * (size_t)row_bytes + (size_t)c * 16;
    const size_t src = ((size_t)s * num_kv_heads + h) * (size_t)row_bytes + (size_t)c * 16;
    *reinterpret_cast<uint4*>(kp + dst) = *reinterpret_cast<const uint4*>(kn + src);
    *reinterpret_cast<uint4*>(vp + dst) = *reinterpret_cast<const uint4*>(vn + src);
  }
}

// Whole-block copies between two pools (device or pinned host memory, same
// block shape): dst[pair.dst] = src[pair.src] for K (blockIdx.z = 0) and V.
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(char* __restrict__ dk, char* __restrict__ dv,
                                                               const char* __restrict__ sk,
                                                               const char* __restrict__ sv,
                                                               const int32_t* __restrict__ pairs,
                                                               size_t block_bytes, int num_src, int num_dst) {
  const int p = blockIdx.x;
  const int32_t src = pairs[2 * p];
  const int32_t dst = pairs[2 * p + 1];
  if (src < 0 || src >= num_src || dst < 0 || dst >= num_dst) return;
  const uint4* s = reinterpret_cast<const uint4*>((blockIdx.z ? sv : sk) + (size_t)src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>((blockIdx.z ? dv : dk) + (size_t)dst * block_bytes);
  const size_t n = block_bytes >> 4;
  for (size_t v = (size_t)blockIdx.y * kThreads + threadIdx.x; v < n; v += (size_t)gridDim.y * kThreads) d[v] = s[v];
}

// The device address through which a kernel reaches `p`: device memory as
// is, pinned (page-locked, device-mapped) host memory through its mapping.
// Anything else -- pageable host memory in particular -- is refused, since a
// kernel touching it would fault.
const char* device_view(const void* p, const char* what, pa_status_t* st) {
  hipPointerAttribute_t at{};
  const hipError_t e = hipPointerGetAttributes(&at, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky query error
    *st = fail(PA_ERR_SHAPE, "pa_swap_blocks: %s is neither device memory nor pinned host memory", what);
    return nullptr;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged || at.type == hipMemoryTypeUnified)
    return static_cast<const char*>(p);
  if (at.type == hipMemoryTypeHost && at.devicePointer && at.hostPointer)
    return static_cast<const char*>(at.devicePointer) +
           (static_cast<const char*>(p) - static_cast<const char*>(at.hostPointer));
  *st = fail(PA_ERR_SHAPE, "pa_swap_blocks: %s is not device-accessible (memory type %d)", what, (int)at.type);
  return nullptr;
}

bool pow2_block(int bs) { return bs >= 1 && bs <= 128 && (bs & (bs - 1)) == 0; }

int elem_bytes(pa_dtype_t dt) { return dt == PA_FP32 ? 4 : (dt == PA_FP16 || dt == PA_BF16) ? 2 : 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

void launch_write_last(void* k_pool, void* v_pool, const void* k_new, const void* v_new, const int32_t* bt,
                       const int32_t* cl, int num_seqs, int maxb, int max_ctx, int num_kv_heads, int head_dim,
                       int elem_bytes, int lbs, int num_blocks, hipStream_t st) {
  hipLaunchKernelGGL(write_last_kernel, dim3(num_seqs), dim3(kThreads), 0, st, (char*)k_pool, (char*)v_pool,
                     (const char*)k_new, (const char*)v_new, bt, cl, maxb, max_ctx, num_kv_heads,
                     head_dim * elem_bytes, lbs, num_blocks);
}

}  // namespace pa

extern "C" pa_status_t pa_write_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                   const int64_t* slot_mapping, int num_tokens, int num_kv_heads, int head_dim,
                                   int block_size, int num_blocks, pa_dtype_t dtype, void* stream) {
  using namespace pa;
  clear_error();
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: unknown dtype %d", (int)dtype);
  if (!pow2_block(block_size)) return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: block_size %d (a power of two up to 128)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_write_kv: head_dim %d", head_dim);
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "pa_write_kv: num_tokens=%d num_kv_heads=%d num_blocks=%d", num_tokens, num_kv_heads,
                num_blocks);
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return fail(PA_ERR_NULL, "pa_write_kv: NULL pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_SHAPE, "pa_write_kv: tensors must be 16-byte aligned");
  const int row_bytes = head_dim * eb;
  hipLaunchKernelGGL(write_kv_kernel, dim3(num_tokens), dim3(kThreads), 0, (hipStream_t)stream, (char*)k_pool,
                     (char*)v_pool, (const char*)k_new, (const char*)v_new, slot_mapping, num_kv_heads, row_bytes,
                     block_size, (int64_t)num_blocks * block_size);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "pa_write_kv: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" pa_status_t pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs, int num_pairs,
                                      int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                      pa_dtype_t dtype, void* stream) {
  using namespace pa;
  clear_error();
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: unknown dtype %d", (int)dtype);
  if (!pow2_block(block_size)) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: block_size %d (a power of two up to 128)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_copy_blocks: head_dim %d", head_dim);
  if (num_pairs < 0 || num_kv_heads <= 0 || num_blocks < 0)
    return fail(PA_ERR_SHAPE, "pa_copy_blocks: num_pairs=%d num_kv_heads=%d num_blocks=%d", num_pairs, num_kv_heads,
                num_blocks);
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !block_pairs) return fail(PA_ERR_NULL, "pa_copy_blocks: NULL pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool)) return fail(PA_ERR_SHAPE, "pa_copy_blocks: pools must be 16-byte aligned");
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * eb;
  const size_t vecs = block_bytes / 16;
  unsigned ychunks = (unsigned)((vecs + kThreads - 1) / kThreads);
  if (ychunks > 64) ychunks = 64;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, ychunks, 2), dim3(kThreads), 0, (hipStream_t)stream,
                     (char*)k_pool, (char*)v_pool, block_pairs, block_bytes, num_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "pa_copy_blocks: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}

extern "C" pa_status_t pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                                      const int32_t* block_pairs, int num_pairs, int num_kv_heads, int head_dim,
                                      int block_size, int num_src_blocks, int num_dst_blocks, pa_dtype_t dtype,
                                      void* stream) {
  using namespace pa;
  clear_error();
  const int eb = elem_bytes(dtype);
  if (eb == 0) return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: unknown dtype %d", (int)dtype);
  if (!pow2_block(block_size)) return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: block_size %d (a power of two up to 128)", block_size);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_swap_blocks: head_dim %d", head_dim);
  if (num_pairs < 0 || num_kv_heads <= 0 || num_src_blocks < 0 || num_dst_blocks < 0)
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: num_pairs=%d num_kv_heads=%d num_src_blocks=%d num_dst_blocks=%d",
                num_pairs, num_kv_heads, num_src_blocks, num_dst_blocks);
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs) return fail(PA_ERR_NULL, "pa_swap_blocks: NULL pointer");
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v))
    return fail(PA_ERR_SHAPE, "pa_swap_blocks: pools must be 16-byte aligned");
  pa_status_t st = PA_OK;
  const char* dk = device_view(dst_k, "dst_k", &st);
  if (!dk) return st;
  const char* dv = device_view(dst_v, "dst_v", &st);
  if (!dv) return st;
  const char* sk = device_view(src_k, "src_k", &st);
  if (!sk) return st;
  const char* sv = device_view(src_v, "src_v", &st);
  if (!sv) return st;
  const char* pp = device_view(block_pairs, "block_pairs", &st);
  if (!pp) return st;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * eb;
  const size_t vecs = block_bytes / 16;
  unsigned ychunks = (unsigned)((vecs + kThreads - 1) / kThreads);
  if (ychunks > 64) ychunks = 64;
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(num_pairs, ychunks, 2), dim3(kThreads), 0, (hipStream_t)stream,
                     const_cast<char*>(dk), const_cast<char*>(dv), sk, sv, reinterpret_cast<const int32_t*>(pp),
                     block_bytes, num_src_blocks, num_dst_blocks);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "pa_swap_blocks: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
