// pa_prefill / pa_prefill_workspace_bytes: argument checks, the split
// decision, workspace carving and the launches (kernels in prefill.hip).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "decode_kernels.h"
#include "pa_internal.h"
#include "prefill_kernels.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Automatic split: a launch of fewer than kFewGroups workgroups (row tiles
// x KV heads x sequences) over contexts longer than kSplitMin positions is
// cut into position partitions until it has about kTargetGroups workgroups
// -- one round of two resident workgroups on each of the 256 compute units;
// a second round measured slower (64 new tokens after 24k-32k cached ones:
// 666 TFLOP/s at 8 partitions, 543 at 16) -- each walking at least kSplitMin
// positions.  Only sizes enter the choice (no device query), so the
// workspace size is known ahead of the call.
constexpr int64_t kFewGroups = 512, kTargetGroups = 512, kSplitMin = 512;

struct Split {
  int P = 1, psteps = 0;
};

Split choose_split(int num_seqs, int num_q_heads, int num_kv_heads, int max_query_len, int max_context_len,
                   int partition_size) {
  Split sp;
  if (num_seqs <= 0 || num_kv_heads <= 0 || num_q_heads <= 0 || max_query_len <= 0 || max_context_len <= 0)
    return sp;
  const int64_t g = num_q_heads / num_kv_heads;
  const int64_t tiles = ((int64_t)max_query_len * g + pa::kPrefillRows - 1) / pa::kPrefillRows;
  const int64_t groups = tiles * num_kv_heads * num_seqs;
  const int64_t S = pa::kPrefillStep;
  int64_t psize;
  if (partition_size > 0) {
    psize = (partition_size + S - 1) / S * S;
  } else {
    if (groups >= kFewGroups || max_context_len <= kSplitMin) return sp;
    int64_t P = (kTargetGroups + groups - 1) / groups;
    const int64_t pmax = (max_context_len + kSplitMin - 1) / kSplitMin;
    if (P > pmax) P = pmax;
    psize = ((max_context_len + P - 1) / P + S - 1) / S * S;
  }
  const int64_t P = (max_context_len + psize - 1) / psize;
  if (P <= 1) return sp;
  sp.P = (int)P;
  sp.psteps = (int)(psize / S);
  return sp;
}

}  // namespace

extern "C" size_t pa_prefill_workspace_bytes(int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads,
                                             int head_dim, int max_query_len, int max_context_len,
                                             int partition_size) {
  if (num_seqs <= 0 || num_tokens <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads != 0 || head_dim <= 0 || max_query_len <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  const Split sp =
      choose_split(num_seqs, num_q_heads, num_kv_heads, max_query_len, max_context_len, partition_size);
  return pa::prefill_workspace(num_tokens, num_q_heads, head_dim, sp.P).total;
}

namespace {

// The matrix-core launch (main kernel, then the merge of a split launch)
// once the arguments are checked and the split and workspace are settled.
// query_start NULL: one query row per sequence (row s of q and out), the
// decode layout.
pa_status_t launch_rows(const char* who, void* out, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens, const int32_t* query_start,
                        int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads, int head_dim, int lbs,
                        int num_blocks, int max_blocks_per_seq, int max_query_len, int max_context_len, float scale,
                        pa_dtype_t dtype, const Split& sp, const pa::PrefillWorkspace& wl, void* workspace,
                        void* stream) {
  using namespace pa;
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
  a.max_ctx = max_context_len;
  a.lbs = lbs;
  a.neg_scale = scale < 0.f;
  a.qscale = fabsf(scale) * 1.4426950408889634f;
  a.dtype = dtype;
  a.P = sp.P;
  a.psteps = sp.psteps;
  if (wl.total) {
    char* ws = static_cast<char*>(workspace);
    a.ws_o = reinterpret_cast<float*>(ws + wl.o_off);
    a.ws_m = reinterpret_cast<float*>(ws + wl.m_off);
    a.ws_l = reinterpret_cast<float*>(ws + wl.l_off);
  }
  // Kernel variant.  Both default kernels load K/V straight into LDS; the
  // 8-wavefront one shares each step's K/V between 256 rows and is 2-10%
  // faster when sequences bring that many rows per KV head, while a step
  // of mostly short chunks (decode-like single tokens) keeps 128-row
  // workgroups, two per compute unit (the wide kernel measured 16% slower
  // there).  Only sizes the caller passes enter the choice: average query
  // rows per (sequence, KV head) = num_tokens * g / num_seqs.
  // PA_PREFILL_KERNEL=regs | dma | w8 forces one (read at each call, for
  // comparisons).
  a.kind = (int64_t)num_tokens * a.g >= (int64_t)kWideRows * num_seqs ? kPrefillWide : kPrefillDirect;
  {
    const char* k = getenv("PA_PREFILL_KERNEL");
    if (k && strcmp(k, "regs") == 0) a.kind = kPrefillRegs;
    if (k && strcmp(k, "dma") == 0) a.kind = kPrefillDirect;
    if (k && strcmp(k, "w8") == 0) a.kind = kPrefillWide;
  }
  if (!query_start) a.kind = kPrefillDirect;  // the decode layout has one instance
  // Grid: 8 XCDs x ranks per XCD.  In the tile order (split launches, or
  // more than 64 * kLptPerLane items per XCD) rank r names an item, a row
  // tile and a partition: ceil(items / 8) x row tiles of max_query_len x
  // partitions.  In the longest-first order rank k is the XCD's k-th longest
  // walk and ranks past the XCD's last walk exit at once, so the grid need
  // only cover the walks that can exist.  Since query_start is non-decreasing
  // from 0 to num_tokens, the sequences' chunks hold num_tokens tokens in
  // all, one XCD holds at most m = ceil(Hkv / 8) KV heads of a sequence, and
  // each of its items rounds up to whole row tiles once: at most
  // ceil(m * num_tokens * g / R) + ceil(items / 8) walks per XCD.  A step
  // of mostly single-token sequences beside a few long chunks then launches
  // about as many workgroups as it has walks instead of max_query_len's
  // tiles for every sequence.
  const int64_t rows_per_wg = a.kind == kPrefillWide ? kWideRows : kPrefillRows;
  const int64_t tiles = ((int64_t)max_query_len * a.g + rows_per_wg - 1) / rows_per_wg;
  const int64_t items = (int64_t)num_kv_heads * num_seqs;
  const int64_t per_xcd = (items + 7) / 8;
  int64_t ranks = per_xcd * tiles * sp.P;
  if (sp.P == 1 && per_xcd <= 64 * kLptPerLane) {
    const int64_t m = (num_kv_heads + 7) / 8;
    const int64_t walks = (m * num_tokens * a.g + rows_per_wg - 1) / rows_per_wg + per_xcd;
    if (walks < ranks) ranks = walks;
  }
  const int64_t grid = 8 * ranks;
  if (grid > 0x7fffffffLL)
    return fail(PA_ERR_SHAPE, "%s: launch of %lld workgroups is too large", who, (long long)grid);
  a.tiles = (int)tiles;
  a.grid = (int)grid;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  take_main_kernel_events(&a.ev_start, &a.ev_stop);
  launch_prefill_mfma(a, st);
  launch_prefill_reduce(a, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" pa_status_t pa_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* query_start, int num_seqs, int num_tokens, int num_q_heads,
                                  int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                  int max_blocks_per_seq, int max_query_len, int max_context_len,
                                  int partition_size, float scale, pa_dtype_t dtype, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  using namespace pa;
  clear_error();
  if (dtype != PA_FP32 && dtype != PA_FP16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: unknown dtype %d", (int)dtype);
  int lbs = -1;
  for (int k = 3; k <= 7; ++k)
    if (block_size == 1 << k) lbs = k;
  if (lbs < 0) return fail(PA_ERR_UNSUPPORTED, "pa_prefill: block_size %d (8, 16, 32, 64 or 128)", block_size);
  if (dtype == PA_FP32 && lbs < 4)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill: fp32 KV takes block_size 16, 32, 64 or 128 (got %d)", block_size);
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
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_SHAPE, "pa_prefill: max_context_len %d outside [0, max_blocks_per_seq*block_size = %lld]",
                max_context_len, (long long)max_blocks_per_seq * block_size);
  if (partition_size < 0) return fail(PA_ERR_SHAPE, "pa_prefill: partition_size %d < 0", partition_size);
  // (the kernels address a slot as block id * block bytes + a 32-bit offset)
  if ((int64_t)num_kv_heads * head_dim * block_size * 4 > 0xffffffffLL)
    return fail(PA_ERR_SHAPE, "pa_prefill: a block of %d KV heads x %d slots x %d dims is too large", num_kv_heads,
                block_size, head_dim);
  if ((int64_t)num_tokens * num_q_heads * head_dim > 0x7fffffffffffLL)
    return fail(PA_ERR_SHAPE, "pa_prefill: %d tokens of %d heads is too large", num_tokens, num_q_heads);
  if (!isfinite(scale)) return fail(PA_ERR_SHAPE, "pa_prefill: scale is not finite");
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || !query_start)
    return fail(PA_ERR_NULL, "pa_prefill: NULL pointer");
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16))
    return fail(PA_ERR_SHAPE, "pa_prefill: out, q and the pools must be 16-byte aligned");

  const Split sp =
      choose_split(num_seqs, num_q_heads, num_kv_heads, max_query_len, max_context_len, partition_size);
  const PrefillWorkspace wl = prefill_workspace(num_tokens, num_q_heads, head_dim, sp.P);
  if (wl.total > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "pa_prefill: needs %zu bytes of workspace, got NULL", wl.total);
    if (workspace_bytes < wl.total)
      return fail(PA_ERR_WORKSPACE, "pa_prefill: needs %zu bytes of workspace, got %zu", wl.total, workspace_bytes);
    if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "pa_prefill: workspace must be 256-byte aligned");
  }

  if (dtype == PA_FP32) {
    // fp32 KV: the VALU attention kernel with one query token per work item
    // (a token at position p is a single-query attention over p + 1
    // positions of its sequence), no split.
    DecodeArgs d{};
    d.out = out;
    d.q = q;
    d.kp = static_cast<const char*>(k_pool);
    d.vp = static_cast<const char*>(v_pool);
    d.bt = block_tables;
    d.cl = context_lens;
    d.B = num_tokens;
    d.Hq = num_q_heads;
    d.Hkv = num_kv_heads;
    d.g = num_q_heads / num_kv_heads;
    d.gmax = d.g >= 8 ? 8 : d.g > 2 ? 4 : d.g;
    d.nsub = (d.g + d.gmax - 1) / d.gmax;
    d.D = head_dim;
    d.num_blocks = num_blocks;
    d.maxb = max_blocks_per_seq;
    d.max_ctx = 0x7fffffff;
    d.psize = 1 << 28;  // one partition: the whole walk
    d.P = 1;
    d.qscale = scale * 1.4426950408889634f;
    d.dtype = dtype;
    d.lm = lbs - 4;
    d.qst = query_start;
    d.nseq = num_seqs;
    d.max_q = max_query_len;
    if ((int64_t)num_tokens * num_kv_heads * d.nsub > 0x7fffffffLL)
      return fail(PA_ERR_SHAPE, "pa_prefill: launch of %lld workgroups is too large",
                  (long long)num_tokens * num_kv_heads * d.nsub);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    take_main_kernel_events(&d.ev_start, &d.ev_stop);
    launch_decode_valu(d, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "pa_prefill: launch failed: %s", hipGetErrorString(e));
    return PA_OK;
  }

  return launch_rows("pa_prefill", out, q, k_pool, v_pool, block_tables, context_lens, query_start, num_seqs,
                     num_tokens, num_q_heads, num_kv_heads, head_dim, lbs, num_blocks, max_blocks_per_seq,
                     max_query_len, max_context_len, scale, dtype, sp, wl, workspace, stream);
}

namespace pa {

size_t decode_rows_workspace(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_context_len,
                             int partition_size) {
  const Split sp = choose_split(num_seqs, num_q_heads, num_kv_heads, 1, max_context_len, partition_size);
  return prefill_workspace(num_seqs, num_q_heads, head_dim, sp.P).total;
}

pa_status_t decode_rows(const char* who, void* out, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int lbs, int num_blocks, int max_blocks_per_seq,
                        int max_context_len, int partition_size, float scale, pa_dtype_t dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const Split sp = choose_split(num_seqs, num_q_heads, num_kv_heads, 1, max_context_len, partition_size);
  const PrefillWorkspace wl = prefill_workspace(num_seqs, num_q_heads, head_dim, sp.P);
  if (wl.total > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got NULL", who, wl.total);
    if (workspace_bytes < wl.total)
      return fail(PA_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got %zu", who, wl.total, workspace_bytes);
    if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
  }
  return launch_rows(who, out, q, k_pool, v_pool, block_tables, context_lens, nullptr, num_seqs, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, lbs, num_blocks, max_blocks_per_seq, 1, max_context_len,
                     scale, dtype, sp, wl, workspace, stream);
}

}  // namespace pa
