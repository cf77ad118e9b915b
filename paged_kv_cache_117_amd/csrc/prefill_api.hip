// pa_prefill: argument checks and launch of the prefill kernel
// (prefill.hip).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "pa_internal.h"
#include "prefill_kernels.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

extern "C" pa_status_t pa_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start, int num_seqs, int num_tokens, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, int max_query_len, float scale, pa_dtype_t dtype,
                                  void* stream) {
  using namespace pa;
  clear_error();
  if (dtype != PA_FP32 && dtype != PA_FP16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: unknown dtype %d", (int)dtype);
  if (dtype == PA_FP32) return fail(PA_ERR_UNSUPPORTED, "pa_prefill: fp32 KV is not supported (fp16 or bf16)");
  int lbs = -1;
  for (int k = 3; k <= 7; ++k)
    if (block_size == 1 << k) lbs = k;
  if (lbs < 0) return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size %d (8, 16, 32, 64 or 128)", block_size);
  if (head_dim != 64 && head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: head_dim %d (64 or 128)", head_dim);
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: negative num_seqs %d, num_tokens %d or max_query_len %d", num_seqs,
                num_tokens, max_query_len);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: num_q_heads %d must be a positive multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "pa_prefill: num_blocks %d, max_blocks_per_seq %d", num_blocks, max_blocks_per_seq);
  if (max_query_len > num_tokens)
    return fail(PA_ERR_SHAPE, "pa_prefill: max_query_len %d exceeds num_tokens %d", max_query_len, num_tokens);
  if ((int64_t)max_blocks_per_seq * block_size > 0x7fffffffLL)
    return fail(PA_ERR_SHAPE, "pa_prefill: max_blocks_per_seq %d too large", max_blocks_per_seq);
  if ((int64_t)num_tokens * num_q_heads * head_dim > 0x7fffffffffffLL)
    return fail(PA_ERR_SHAPE, "pa_prefill: %d tokens of %d heads is too large", num_tokens, num_q_heads);
  if (!isfinite(scale)) return fail(PA_ERR_SHAPE, "pa_prefill: scale is not finite");
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_NULL, "pa_prefill: NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PA_ERR_SHAPE, "pa_prefill: out, q and the pools must be 16-byte aligned");

  PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.kp = static_cast<const char*>(k_pool);
  a.vp = static_cast<const char*>(v_pool);
  a.bt = block_tables;
  a.cl = context_lens;
  a.qs = query_start;
  a.B = num_seqs;
  a.N = num_tokens;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.g = num_q_heads / num_kv_heads;
  a.D = head_dim;
  a.num_blocks = num_blocks;
  a.maxb = max_blocks_per_seq;
  a.max_q = max_query_len;
  a.lbs = lbs;
  a.neg_scale = scale < 0.f;
  a.qscale = fabsf(scale) * 1.4426950408889634f;
  a.dtype = dtype;
  // Grid: 8 XCDs x ceil(items / 8) work items x row tiles (the kernel maps
  // each workgroup to an item and tile; see prefill.hip).
  const int64_t tiles = ((int64_t)max_query_len * a.g + kPrefillRows - 1) / kPrefillRows;
  const int64_t items = (int64_t)num_kv_heads * num_seqs;
  const int64_t grid = 8 * ((items + 7) / 8) * tiles;
  if (grid > 0x7fffffffLL)
    return fail(PA_ERR_SHAPE, "pa_prefill: launch of %lld workgroups is too large", (long long)grid);
  a.tiles = (int)tiles;
  a.grid = (int)grid;
  launch_prefill_mfma(a, static_cast<hipStream_t>(stream));
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "pa_prefill: launch failed: %s", hipGetErrorString(e));
  return PA_OK;
}
