// pa_decode / pa_decode_workspace_bytes: argument checks, workspace carving
// and kernel selection.  The kernels themselves live in decode*.hip.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "decode_kernels.h"
#include "pa_internal.h"
#include "prefill_kernels.h"

namespace {

constexpr int kDefaultPartition = 512;
// pa_write_kv_decode fuses the write into the stream kernel up to this many
// KV bytes per launch (bounded by num_seqs * max_context_len).
constexpr uint64_t kFuseMaxKvBytes = 2ull << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// PA_DECODE_KERNEL=valu selects the VALU partition kernel for 16-bit KV too,
// PA_DECODE_KERNEL=partition the MFMA partition kernels instead of the
// balanced split (read at each call, so a process can compare them).
const char* kernel_override() {
  const char* v = getenv("PA_DECODE_KERNEL");
  return v ? v : "";
}
bool force_valu() { return strcmp(kernel_override(), "valu") == 0; }
bool force_partition() { return strcmp(kernel_override(), "partition") == 0; }

// Compute units of the current device (cached per device); 256 if the
// query fails.
int cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load();
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev].store(n);
  }
  return n;
}

int parts_for(int max_ctx, int psize) { return max_ctx <= 0 ? 1 : (max_ctx + psize - 1) / psize; }

// Upper bound of the balanced split's units (every sequence at max_ctx).
int64_t stream_units_bound(int B, int Hq, int Hkv, int max_ctx, int unit) {
  const int g = Hq / Hkv, gmax = pa::mfma_gmax(g), nsub = (g + gmax - 1) / gmax;
  const int64_t per_seg = ((int64_t)(max_ctx + 15) / 16 + unit - 1) / unit;
  return (int64_t)B * Hkv * nsub * per_seg;
}

}  // namespace

extern "C" size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                            int max_context_len, int partition_size) {
  const int psize = partition_size == 0 ? kDefaultPartition : partition_size;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0 || head_dim <= 0 ||
      max_context_len < 0 || psize <= 0)
    return 0;
  size_t need = pa::workspace_layout(num_seqs, num_q_heads, head_dim, parts_for(max_context_len, psize)).total;
  if (num_seqs <= pa::kStreamMaxSeqs) {
    const size_t st = pa::stream_layout(num_seqs, num_q_heads, num_kv_heads, head_dim).total;
    if (st > need) need = st;
  }
  // (blocks of 8 slots: the prefill kernel's split; never more than the above)
  const size_t rows8 =
      pa::decode_rows_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size);
  if (rows8 > need) need = rows8;
  return need;
}

namespace {

// ---------------------------------------------------------------------------
// Scratch of pa_decode_noalloc: a file-scope device array (one copy per GPU,
// held until the process ends).  Host code never passes the array's name to
// a kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device with hipGetSymbolAddress, with that
// device current, and the looked-up pointer is what the kernels receive.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
__device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first call there), or NULL with the failing status in *st.
void* scratch_ptr(pa_status_t* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    *st = pa::fail(PA_ERR_LAUNCH, "pa_decode_noalloc: no current device (or device id %d >= %d)", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      *st = pa::fail(PA_ERR_LAUNCH, "pa_decode_noalloc: hipGetSymbolAddress(scratch) failed on device %d: %s", dev,
                     hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// pa_decode's body.  `workspace` NULL with `use_scratch`: the partials go to
// the device's scratch array, laid out for the wavefronts this launch uses.
pa_status_t decode_impl(const char* who, void* out, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                        int max_context_len, float scale, pa_dtype_t dtype, int partition_size, void* workspace,
                        size_t workspace_bytes, void* stream, bool use_scratch, const void* k_new = nullptr,
                        const void* v_new = nullptr) {
  using namespace pa;
  clear_error();
  if (dtype != PA_FP32 && dtype != PA_FP16 && dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "%s: unknown dtype %d", who, (int)dtype);
  // The kernels walk 16-slot tiles (one MFMA operand); a block holds 2^lm of
  // them.  Blocks of 8 slots go through the prefill kernel, which walks
  // token rows (16-bit KV).
  int lm = -1;
  for (int k = 0; k <= 3; ++k)
    if (block_size == 16 << k) lm = k;
  const bool rows8 = block_size == 8;
  if (lm < 0 && !rows8)
    return fail(PA_ERR_UNSUPPORTED, "%s: block_size %d (8, 16, 32, 64 or 128)", who, block_size);
  if (rows8 && dtype == PA_FP32)
    return fail(PA_ERR_UNSUPPORTED, "%s: fp32 KV takes block_size 16, 32, 64 or 128 (got 8)", who);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d (64 or 128)", who, head_dim);
  if (num_seqs < 0 || num_seqs > 65535)
    return fail(PA_ERR_SHAPE, "%s: num_seqs %d outside [0, 65535]", who, num_seqs);
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_SHAPE, "%s: num_q_heads %d must be a positive multiple of num_kv_heads %d", who, num_q_heads,
                num_kv_heads);
  if (num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "%s: num_blocks %d, max_blocks_per_seq %d", who, num_blocks, max_blocks_per_seq);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PA_ERR_SHAPE, "%s: max_context_len %d outside [0, max_blocks_per_seq*block_size = %lld]",
                who, max_context_len, (long long)max_blocks_per_seq * block_size);
  const int psize = partition_size == 0 ? kDefaultPartition : partition_size;
  if (psize <= 0 || psize % 16 != 0)
    return fail(PA_ERR_SHAPE, "%s: partition_size %d must be a positive multiple of 16", who, partition_size);
  if (!isfinite(scale)) return fail(PA_ERR_SHAPE, "%s: scale is not finite", who);
  if (rows8 ? (int64_t)num_kv_heads * head_dim * block_size * 4 > 0xffffffffLL
            : ((int64_t)num_blocks * num_kv_heads << lm) > 0x7fffffffLL)
    return fail(PA_ERR_SHAPE, "%s: %d blocks of %d KV heads is too large", who, num_blocks, num_kv_heads);
  if (num_seqs == 0) return PA_OK;
  const bool fused = k_new != nullptr || v_new != nullptr;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens || (fused && (!k_new || !v_new)))
    return fail(PA_ERR_NULL, "%s: NULL pointer", who);
  if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      (fused && (!aligned(k_new, 16) || !aligned(v_new, 16))))
    return fail(PA_ERR_SHAPE, "%s: out, q, the pools and the new rows must be 16-byte aligned", who);

  if (rows8) {
    // workspace first (nothing is launched when it is refused), then the
    // write of a fused step, then the attention
    const size_t need =
        decode_rows_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, partition_size);
    if (use_scratch && need > 0) {
      if (need > kScratchBytes)
        return fail(PA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch, more than its %zu", who, need,
                    kScratchBytes);
      pa_status_t sst = PA_OK;
      workspace = scratch_ptr(&sst);
      if (!workspace) return sst;
      workspace_bytes = kScratchBytes;
    }
    if (need > 0) {
      if (!workspace) return fail(PA_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got NULL", who, need);
      if (workspace_bytes < need)
        return fail(PA_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got %zu", who, need, workspace_bytes);
      if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
    }
    if (fused)
      launch_write_last(const_cast<void*>(k_pool), const_cast<void*>(v_pool), k_new, v_new, block_tables,
                        context_lens, num_seqs, max_blocks_per_seq, max_context_len, num_kv_heads, head_dim, 2, 3,
                        num_blocks, static_cast<hipStream_t>(stream));
    return decode_rows(who, out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads, num_kv_heads,
                       head_dim, 3, num_blocks, max_blocks_per_seq, max_context_len, partition_size, scale, dtype,
                       workspace, workspace_bytes, stream);
  }

  const int P = parts_for(max_context_len, psize);
  const int g = num_q_heads / num_kv_heads;
  // Balanced split: 16-bit KV, batches whose lengths fit its LDS table.
  // Units are single blocks unless a partition size is given.
  const bool half = dtype != PA_FP32 && !force_valu();
  const int unit = partition_size == 0 ? 1 : psize / 16;
  // (its tile descriptors hold the tile row ((block * num_kv_heads + head) << lm) + tile in 27 bits)
  const bool use_stream = half && num_seqs <= kStreamMaxSeqs && !force_partition() &&
                          stream_units_bound(num_seqs, num_q_heads, num_kv_heads, max_context_len, unit) < (1 << 30) &&
                          ((int64_t)num_blocks * num_kv_heads << lm) < (1 << 27);
  // MFMA partition kernels: 16-bit KV, partitions of at most 4096 positions
  // (a wave holds at most 64 block ids).  Everything else: the VALU kernel.
  const bool mfma = half && (use_stream || psize <= 4096);
  // Balanced split: one workgroup of 4 independent wavefronts per CU (4
  // wavefronts with two tiles in flight each keep a CU's share of HBM busy),
  // and never more wavefronts than units.
  int grid = 1;
  if (use_stream) {
    const int64_t units = stream_units_bound(num_seqs, num_q_heads, num_kv_heads, max_context_len, unit);
    int64_t gr = cu_count();
    if (gr > kStreamMaxWaves / 4) gr = kStreamMaxWaves / 4;
    if (gr > (units + 3) / 4) gr = (units + 3) / 4;
    grid = gr < 1 ? 1 : (int)gr;
  }
  const WorkspaceLayout wl = workspace_layout(num_seqs, num_q_heads, head_dim, P);
  // The caller's workspace is sized without knowing the device (slots for
  // kStreamMaxWaves wavefronts); the scratch array only for this launch's.
  const StreamLayout sl =
      stream_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, use_scratch ? (size_t)grid * 4 : kStreamMaxWaves);
  const size_t need = use_stream ? sl.total : wl.total;
  if (use_scratch && need > 0) {
    if (need > kScratchBytes)
      return fail(PA_ERR_WORKSPACE, "%s: these sizes need %zu bytes of scratch, more than its %zu", who, need,
                  kScratchBytes);
    pa_status_t sst = PA_OK;
    workspace = scratch_ptr(&sst);
    if (!workspace) return sst;
    workspace_bytes = kScratchBytes;
  }
  if (need > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got NULL", who, need);
    if (workspace_bytes < need)
      return fail(PA_ERR_WORKSPACE, "%s: needs %zu bytes of workspace, got %zu", who, need, workspace_bytes);
    if (!aligned(workspace, 256)) return fail(PA_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", who);
  }

  DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.kp = static_cast<const char*>(k_pool);
  a.vp = static_cast<const char*>(v_pool);
  a.bt = block_tables;
  a.cl = context_lens;
  char* ws = static_cast<char*>(workspace);
  if (use_stream) {
    a.ws_o = reinterpret_cast<float*>(ws + sl.o_off);
    a.ws_m = reinterpret_cast<float*>(ws + sl.m_off);
    a.ws_l = reinterpret_cast<float*>(ws + sl.l_off);
    a.info = reinterpret_cast<int2*>(ws + sl.info_off);
  } else if (wl.total) {
    a.ws_o = reinterpret_cast<float*>(ws + wl.o_off);
    a.ws_m = reinterpret_cast<float*>(ws + wl.m_off);
    a.ws_l = reinterpret_cast<float*>(ws + wl.l_off);
  }
  a.B = num_seqs;
  a.Hq = num_q_heads;
  a.Hkv = num_kv_heads;
  a.g = g;
  // Query heads per work item: the MFMA kernels take up to 16 (one matrix
  // column each; 4, 8 or 16 sizes their buffers), the VALU kernel 1, 2, 4
  // or 8 (one accumulator set each).
  a.gmax = mfma ? mfma_gmax(g) : g >= 8 ? 8 : g > 2 ? 4 : g;
  a.nsub = (a.g + a.gmax - 1) / a.gmax;
  a.D = head_dim;
  a.num_blocks = num_blocks;
  a.maxb = max_blocks_per_seq;
  a.max_ctx = max_context_len;
  a.psize = psize;
  a.P = P;
  a.qscale = scale * 1.4426950408889634f;
  a.dtype = dtype;
  a.lm = lm;
  a.stream = use_stream;
  if (use_stream) {
    a.unit = unit;
    a.grid = grid;
    a.entries = 1;
  } else {
    // Partitions of up to 64 blocks: one wavefront each, and the
    // workgroup's four partitions merged into one workspace entry.
    a.wave_part = mfma && psize / 16 <= 64;
    a.per_entry = a.wave_part ? 4 : 1;
    a.entries = (P + a.per_entry - 1) / a.per_entry;
    if ((int64_t)a.entries * num_kv_heads * a.nsub * num_seqs > 0x7fffffffLL)
      return fail(PA_ERR_SHAPE, "%s: launch of %lld workgroups is too large",
                  who, (long long)a.entries * num_kv_heads * a.nsub * num_seqs);
  }

  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (fused) {
    // The stream kernel's fused form costs a little on every tile (address
    // selects for the one tile per sequence that holds its new token); the
    // separate write launch costs a fixed ~4 us.  Measured on MI355X, fusing
    // pays up to about 2 GiB of KV per launch (the Llama-3.1-8B layer at 64
    // sequences: +2% per step) and not beyond (the Qwen2.5-72B layer at 128
    // sequences of 4k-8k: -0.3%); the bound uses max_context_len.  Both forms
    // give identical bits.  (The kernel also addresses the new rows with
    // 32-bit byte offsets.)
    const int eb = dtype == PA_FP32 ? 4 : 2;
    const uint64_t kv_bound = (uint64_t)num_seqs * max_context_len * num_kv_heads * head_dim * eb * 2;
    if (use_stream && kv_bound <= kFuseMaxKvBytes && (uint64_t)num_seqs * num_kv_heads * head_dim * eb < (1ull << 32)) {
      // the stream kernel writes each sequence's new rows and attends to them
      a.kn = static_cast<const char*>(k_new);
      a.vn = static_cast<const char*>(v_new);
    } else {
      launch_write_last(const_cast<void*>(k_pool), const_cast<void*>(v_pool), k_new, v_new, block_tables,
                        context_lens, num_seqs, max_blocks_per_seq, max_context_len, num_kv_heads, head_dim, eb,
                        4 + lm, num_blocks, st);
    }
  }
  take_main_kernel_events(&a.ev_start, &a.ev_stop);
  if (mfma)
    launch_decode_mfma(a, st);
  else
    launch_decode_valu(a, st);
  if (a.stream)
    launch_decode_stream_reduce(a, st);
  else if (a.entries > 1)
    launch_decode_reduce(a, st);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_LAUNCH, "%s: launch failed: %s", who, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace

extern "C" pa_status_t pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                 int num_q_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                                 int max_blocks_per_seq, int max_context_len, float scale, pa_dtype_t dtype,
                                 int partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl("pa_decode", out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_size, workspace, workspace_bytes, stream, false);
}

extern "C" pa_status_t pa_write_kv_decode(void* out, const void* q, void* k_pool, void* v_pool, const void* k_new,
                                          const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                                          int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int num_blocks, int max_blocks_per_seq,
                                          int max_context_len, float scale, pa_dtype_t dtype, int partition_size,
                                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!k_new || !v_new) {
    pa::clear_error();
    return pa::fail(PA_ERR_NULL, "pa_write_kv_decode: NULL pointer");
  }
  return decode_impl("pa_write_kv_decode", out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_size, workspace, workspace_bytes, stream, false, k_new, v_new);
}

extern "C" pa_status_t pa_decode_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                                         const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                                         int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                                         int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                                         pa_dtype_t dtype, int partition_size, void* stream) {
  return decode_impl("pa_decode_noalloc", out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_q_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_context_len, scale, dtype,
                     partition_size, nullptr, 0, stream, true);
}
