/*
 * pa.h -- C ABI of libpa: paged KV cache decode path for AMD MI355X (gfx950).
 *
 * The KV cache is a pool of fixed-size blocks; each sequence reaches its
 * blocks through a block table that maps logical block j (positions
 * bs*j..bs*j+bs-1, bs = block_size, 16 by default) to a physical block id
 * (PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 3: blocks
 * and block tables"; PagedAttention (tensortonic), "4. Finding Tokens with a
 * Block Table").
 *
 * Layouts (all row-major, C order):
 *   K pool, V pool : [num_blocks][num_kv_heads][block_size][head_dim]  (two tensors)
 *   q, out         : [num_seqs][num_q_heads][head_dim]
 *   k_new, v_new   : [num_tokens][num_kv_heads][head_dim]
 *   block_tables   : int32 [num_seqs][max_blocks_per_seq]
 *   context_lens   : int32 [num_seqs]
 *   slot_mapping   : int64 [num_tokens], slot = block * block_size + offset
 *   block_pairs    : int32 [num_pairs][2] = (src, dst)
 * q, out, pools and new K/V share one element type (pa_dtype_t).  Query head
 * h reads KV head h / (num_q_heads / num_kv_heads).
 *
 * Conventions for every device entry point:
 *   - Pointers marked "device" are device addresses the caller allocated;
 *     the library never allocates or frees them and keeps none after return.
 *     Tensor base pointers must be 16-byte aligned.
 *   - Work is enqueued on `stream` (a hipStream_t, NULL = the default
 *     stream) and runs asynchronously.  The return code covers host-side
 *     argument checks and the launch itself; faults surface at the caller's
 *     next synchronisation.
 *   - The contents of index arrays are the caller's contract (the block
 *     manager below produces them).  The kernels still never access memory
 *     outside the pools: an out-of-range slot or block pair is skipped, and
 *     a sequence with an out-of-range length or block id gets NaN outputs.
 *   - No exception crosses the ABI.  On a non-OK status, pa_last_error()
 *     returns a message (thread-local, valid until the next call on that
 *     thread).
 *   - Arithmetic is float32 for every storage type.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_FP32 = 0, PA_FP16 = 1, PA_BF16 = 2 } pa_dtype_t;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,        /* a required pointer is NULL */
  PA_ERR_SHAPE = 2,       /* sizes inconsistent or out of range, misaligned pointer */
  PA_ERR_UNSUPPORTED = 3, /* block_size, head_dim (64/128) or dtype the call does not take */
  PA_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  PA_ERR_LAUNCH = 5,      /* the HIP runtime refused the launch */
  PA_ERR_NO_BLOCKS = 6,   /* block manager: the free list cannot cover the request */
  PA_ERR_NOT_FOUND = 7,   /* block manager: unknown sequence id */
  PA_ERR_EXISTS = 8       /* block manager: sequence id already in use */
} pa_status_t;

/*
 * pa_decode -- single-query decode attention through block tables.
 *
 * For each sequence s with L = context_lens[s] and each query head h
 * (KV head j = h / g, g = num_q_heads / num_kv_heads):
 *   x_t   = scale * q[s][h] . K_j(t)           for positions t = 0..L-1,
 *   out   = sum_t softmax(x)_t * V_j(t),
 * where position t lives in physical block block_tables[s][t / bs] at slot
 * t % bs (bs = block_size).  This is ordinary attention over the sequence's valid positions,
 * the final block truncated at L; only addresses differ (PagedAttention and
 * vLLM: Paging the KV Cache Like an OS, "Step 5: attention over scattered
 * blocks"; PagedAttention (tensortonic), "5. Reading the Cache During
 * Attention"; PagedAttention: Virtual Memory for the KV Cache, "PagedAttention:
 * attention over non-contiguous blocks").  A decode step writes the step's
 * own token first (pa_write_kv), so L counts it.
 *
 * The context is processed in pieces with an online (running max / sum)
 * softmax (PagedAttention (tensortonic), "10. How PagedAttention Fits with
 * FlashAttention"); a sequence split over several pieces is merged by a
 * log-sum-exp weighted reduce, because softmax must normalise over all valid
 * positions at once (same page, section 5).  With partition_size > 0 the
 * pieces are whole partitions of that many positions (several consecutive
 * partitions of one sequence may be merged on the fly by the same rule).
 * With partition_size 0, 16-bit KV and up to 4096 sequences, the batch's
 * blocks are split evenly over the GPU's wavefronts, cutting sequences at
 * block boundaries wherever the even split falls; otherwise partitions of
 * 512 positions are used.  Every choice computes the same attention; results
 * differ only by fp32 rounding order.
 *
 *   out              device, [num_seqs][num_q_heads][head_dim], dtype; written
 *   q                device, [num_seqs][num_q_heads][head_dim], dtype
 *   k_pool, v_pool   device, [num_blocks][num_kv_heads][block_size][head_dim], dtype
 *   block_tables     device, int32 [num_seqs][max_blocks_per_seq]; entries at
 *                    index >= ceil(L/block_size) are never read
 *   context_lens     device, int32 [num_seqs]; 0 <= L <= max_context_len
 *                    (L = 0 writes a zero row)
 *   max_context_len  host hint >= every context_lens[s]; sizes the launch;
 *                    must be <= max_blocks_per_seq * block_size
 *   scale            softmax scale (typically 1/sqrt(head_dim)), finite
 *   partition_size   positions per partition, a positive multiple of
 *                    16; 0 = automatic (see above)
 *   workspace        device scratch of at least pa_decode_workspace_bytes(...)
 *                    bytes (may be NULL when that is 0); 256-byte aligned;
 *                    contents need no initialisation and are clobbered
 *   stream           hipStream_t or NULL
 * Supported: block_size 16, 32, 64 or 128 (the kernels walk 16-slot tiles,
 * 2^k of them per block) and, for fp16/bf16 KV, 8: blocks of 8 slots run
 * through pa_prefill's kernel with one query row per sequence (its
 * workspace then fits in pa_decode_workspace_bytes; fp32 KV with 8 returns
 * PA_ERR_UNSUPPORTED); head_dim 64 or 128,
 * any num_q_heads that is a multiple of num_kv_heads.  `out` must not alias
 * any input or the workspace.
 *
 * Kernel selection can be overridden for measurements through the
 * environment variable PA_DECODE_KERNEL, read at each call: "valu" runs
 * 16-bit KV through the vector-ALU partition kernel (the fp32 kernel, no
 * matrix cores), "partition" runs the matrix-core partition kernels instead
 * of the even split.  Unset or any other value: the choice described above.
 * Every choice computes the same attention within the stated tolerances.
 */
pa_status_t pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, pa_dtype_t dtype, int partition_size,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_write_kv_decode -- one decode step in one launch: each sequence's new
 * token is written into the pool and attended to, as pa_write_kv followed
 * by pa_decode would do, with the write fused into the attention kernel
 * (PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 5": the
 * write kernels are fused to cut launch overhead; PagedAttention
 * (tensortonic), "5. Reading the Cache During Attention": the new key and
 * value go to their block and offset, then the query attends to every valid
 * position including the new one).
 *
 * For each sequence s with 1 <= L = context_lens[s] <= max_context_len, the
 * new token is position L-1: its K and V rows k_new[s][h][:], v_new[s][h][:]
 * are stored at block block_tables[s][(L-1) / block_size], slot
 * (L-1) % block_size, for every KV head h, and out[s] is pa_decode's
 * attention over positions 0..L-1 of the pool after that store.  The result
 * is bit-identical to pa_write_kv with slot_mapping[s] = that slot followed
 * by pa_decode with the same partition_size.  Sequences with L = 0, an
 * out-of-range L or an out-of-range block id at position L-1 write nothing
 * (their outputs are as in pa_decode: zero or NaN).
 *
 *   k_pool, v_pool   device, written at the new tokens' slots, read elsewhere
 *   k_new, v_new     device, [num_seqs][num_kv_heads][head_dim], dtype; read
 * All other arguments, the workspace (pa_decode_workspace_bytes) and the
 * errors are pa_decode's.  The new tokens' slots must be distinct (each
 * sequence owns its last block, which the block manager guarantees by
 * copy-on-write).  With 16-bit KV, up to 4096 sequences and at most 2 GiB of
 * K and V in num_seqs * max_context_len positions, the write is done by the
 * attention kernel itself; otherwise (where the fused kernel's small cost
 * per tile outweighs one launch) by a separate launch before it.
 */
pa_status_t pa_write_kv_decode(void* out, const void* q, void* k_pool, void* v_pool,
                               const void* k_new, const void* v_new,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                               int block_size, int num_blocks, int max_blocks_per_seq,
                               int max_context_len, float scale, pa_dtype_t dtype, int partition_size,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc -- pa_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, results and errors as pa_decode minus
 * the workspace: the partials of split sequences go to a scratch array the
 * library holds in device memory, PA_DECODE_NOALLOC_SCRATCH_BYTES per GPU,
 * reserved when the library's device code is loaded on that GPU and kept
 * until the process ends.  The call allocates nothing (no hipMalloc, no
 * allocating library routine).  Sizes whose partials do not fit the scratch
 * return PA_ERR_WORKSPACE before any launch; with 16-bit KV and up to 4096
 * sequences (the even split) the need is two slots of up to 16 query rows
 * per wavefront of the launch plus 8 bytes per (sequence, head group),
 * e.g. 4 MiB for the Llama-3.1-8B layer at 64 sequences.
 * Every call on one GPU shares that GPU's scratch, which keeps the last
 * call's contents (nothing in it needs clearing between calls): calls that
 * overlap in time on one GPU -- on different streams, or from different
 * threads -- race and their results are undefined.  Serialise them (one
 * stream, or events between streams).
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
pa_status_t pa_decode_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, int max_blocks_per_seq,
                              int max_context_len, float scale, pa_dtype_t dtype, int partition_size,
                              void* stream);

/* Bytes of workspace pa_decode needs for these sizes and any dtype: partials
 * of the partitions (none when every sequence fits one partition) and, for
 * batches of up to 4096 sequences, the pieces of the even split (a fixed
 * number of slots of num_q_heads / num_kv_heads rows, at most 16).  The
 * value does not depend on the device.  Returns 0 for invalid sizes as well;
 * pa_decode reports those. */
size_t pa_decode_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                 int max_context_len, int partition_size);

/*
 * pa_prefill -- paged attention for several new tokens per sequence: a
 * chunk of a long prompt fed over several steps, or the rest of a prompt
 * after its first blocks were found in the prefix cache (Batching and
 * PagedAttention, continuous batching and its chunked-prefill FAQ; vLLM's
 * PagedAttention: How Memory Management Supports Large Model Inference,
 * "2.5": each step computes the next run of a request's tokens).
 *
 * Sequence s has L = context_lens[s] cached positions; the last
 * T = query_start[s+1] - query_start[s] of them are this step's tokens,
 * whose K/V the caller has already written (pa_write_kv).  For the i-th new
 * token (query row query_start[s] + i, position p = L - T + i) and each query
 * head h (KV head j = h / g):
 *   x_t = scale * q[row][h] . K_j(t)            for t = 0..p   (causal),
 *   out[row][h] = sum_t softmax(x)_t * V_j(t),
 * with position t read from block block_tables[s][t / bs], slot t % bs.
 * Where a position lives changes neither its place in the sequence nor the
 * causal mask (PagedAttention (tensortonic), "5. Reading the Cache During
 * Attention").  With T = 1 this is pa_decode's attention.
 *
 *   out              device, [num_tokens][num_q_heads][head_dim], dtype; rows of
 *                    every sequence with T > 0 are written, nothing else
 *   q                device, [num_tokens][num_q_heads][head_dim], dtype
 *   k_pool, v_pool   device, [num_blocks][num_kv_heads][block_size][head_dim], dtype
 *   block_tables     device, int32 [num_seqs][max_blocks_per_seq]; entries at
 *                    index >= ceil(L/block_size) are never read
 *   context_lens     device, int32 [num_seqs]
 *   query_start      device, int32 [num_seqs + 1]: query_start[0] = 0,
 *                    non-decreasing, query_start[num_seqs] = num_tokens;
 *                    T = 0 is allowed (no rows)
 *   max_query_len    host, >= every T (sizes the launch), <= num_tokens
 *   max_context_len  host, >= every L when the launch is split (below);
 *                    <= max_blocks_per_seq * block_size
 *   partition_size   0: automatic -- a launch of fewer than 512 workgroups
 *                    (row tiles of 128 query rows x KV heads x sequences)
 *                    over contexts longer than 512 positions is cut into
 *                    position partitions (at least 512 positions each) until
 *                    it has about 512; > 0: always cut at that many
 *                    positions (rounded up to a multiple of 64).  Each
 *                    partition's rows carry an online-softmax partial and a
 *                    second kernel merges them with log-sum-exp weights, the
 *                    same rule as pa_decode's reduce.
 *   scale            softmax scale (typically 1/sqrt(head_dim)), finite
 *   workspace        device scratch of at least pa_prefill_workspace_bytes(...)
 *                    bytes (NULL allowed when that is 0); 256-byte aligned;
 *                    contents need no initialisation and are clobbered
 *   stream           hipStream_t or NULL
 * Supported: fp16 and bf16 with block_size 8, 16, 32, 64 or 128 (matrix
 * cores); fp32 with block_size 16, 32, 64 or 128 (VALU, one query token per
 * work item, never split); head_dim 64 or 128; any num_q_heads that is a
 * multiple of num_kv_heads.
 * The library picks the workgroup width from the sizes passed: 8
 * wavefronts over 256 query rows when the batch averages at least 256 rows
 * per (sequence, KV head), num_tokens * (num_q_heads / num_kv_heads) >=
 * 256 * num_seqs, else 4 wavefronts over 128 rows; both give the same bits.
 * The environment variable PA_PREFILL_KERNEL (read at each call) forces a
 * kernel, for measurements: "dma" (4 wavefronts), "w8" (8 wavefronts) or
 * "regs" (K and V staged through registers instead of loaded straight into
 * LDS; same results within the tolerances).
 * Device-side contract violations are never dereferenced: a sequence with
 * T > L, L > max_blocks_per_seq * block_size, T > max_query_len, L >
 * max_context_len in a split launch, or a row range outside [0, num_tokens)
 * gets NaN rows (those inside [0, num_tokens)); a block id outside
 * [0, num_blocks) makes the rows that would read it NaN.  The launch is
 * sized from the sizes passed assuming query_start keeps its rules (the
 * chunks together hold at most num_tokens tokens); for a query_start that
 * decreases somewhere, which rows are written is unspecified (nothing
 * outside the given buffers is read or written).  `out` must not alias any
 * input or the workspace.
 */
pa_status_t pa_prefill(void* out, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, int num_seqs, int num_tokens,
                       int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                       int num_blocks, int max_blocks_per_seq, int max_query_len,
                       int max_context_len, int partition_size, float scale, pa_dtype_t dtype,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_time_next_main_kernel -- timing hook (instrumentation, not part of the
 * pages' method).  The next pa_decode or pa_prefill call that launches
 * kernels hands the two events to the launch of its main kernel
 * (hipExtLaunchKernel), so they take that kernel's start and end and not
 * those of any merge kernel after it, and then drops the request;
 * hipEventElapsedTime of the pair is the main kernel's duration.
 *   start_event, stop_event  hipEvent_t handles created by the caller (not
 *                            owned by the library); both NULL cancels a
 *                            pending request; exactly one NULL returns
 *                            PA_ERR_NULL
 * One pending request per process (the last call wins); a call that fails
 * its argument checks leaves the request pending.
 */
pa_status_t pa_time_next_main_kernel(void* start_event, void* stop_event);

/*
 * pa_probe_read -- read-bandwidth probe (instrumentation, not part of the
 * pages' method): the measured ceiling that the decode kernels' HBM rates are
 * read against.  Reads device memory with 16-byte non-temporal loads and
 * stores one 32-bit digest per thread so the reads cannot be dropped.
 *   buf          device, `bytes` bytes (a multiple of 4096), 16-byte aligned;
 *                read only
 *   mode 0       sequential: a grid-stride sweep over the whole buffer
 *   mode 1       4 KiB gather: wavefront w of W reads whole 4 KiB chunks
 *                chunk_order[w], chunk_order[w + W], ... (four chunks in
 *                flight), the access shape of gathering one KV head's
 *                16-slot tiles (16 x 128 dims x 2 bytes) from scattered
 *                blocks; entries outside [0, bytes / 4096) are skipped
 *   chunk_order  device, int32 [num_chunks] (mode 1 only; may be NULL for
 *                mode 0)
 *   workgroups   launch size (256 threads each), 1 .. 2^20
 *   sink         device, uint32 [workgroups * 256], written
 * Returns PA_ERR_UNSUPPORTED for another mode, PA_ERR_SHAPE / PA_ERR_NULL for
 * bad sizes or pointers, PA_ERR_LAUNCH if the launch fails; nothing is
 * allocated.
 */
pa_status_t pa_probe_read(const void* buf, size_t bytes, const int32_t* chunk_order, int num_chunks,
                          int mode, int workgroups, uint32_t* sink, void* stream);

/* Bytes of workspace pa_prefill needs for these sizes (0 when the launch is
 * not split); depends on sizes only, not on the device or the dtype.
 * Returns 0 for invalid sizes as well; pa_prefill reports those. */
size_t pa_prefill_workspace_bytes(int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads,
                                  int head_dim, int max_query_len, int max_context_len,
                                  int partition_size);

/*
 * pa_write_kv -- store the new tokens' K and V rows in their slots
 * (reshape-and-cache).  For each token i whose slot = slot_mapping[i]
 * satisfies 0 <= slot < num_blocks * block_size:
 *   k_pool[slot / block_size][h][slot % block_size][:] = k_new[i][h][:]
 *   v_pool[slot / block_size][h][slot % block_size][:] = v_new[i][h][:]
 * for every KV head h.  The new key and value go to the block and offset the
 * block manager assigned before the query attends to them (PagedAttention
 * (tensortonic), "5. Reading the Cache During Attention"); every token of the
 * step is written by one launch (PagedAttention and vLLM: Paging the KV Cache
 * Like an OS, "Step 5", where the write kernels are fused to save launches).
 *
 *   k_pool, v_pool   device, [num_blocks][num_kv_heads][block_size][head_dim],
 *                    dtype; only the addressed rows are written, no other
 *                    byte is touched
 *   k_new, v_new     device, [num_tokens][num_kv_heads][head_dim], dtype; read
 *   slot_mapping     device, int64 [num_tokens]; slot = block * block_size +
 *                    offset.  A negative slot skips its token (padding); a
 *                    slot >= num_blocks * block_size is a caller error and is
 *                    skipped too, never written
 *   num_tokens       >= 0 (0 launches nothing)
 *   stream           hipStream_t or NULL
 * The non-negative slots of one call must be distinct: two tokens naming one
 * slot race and the row holds either token's bytes.  Supported: fp32, fp16
 * and bf16, head_dim 64 or 128, any block_size that is a power of two up to
 * 128 (pa_copy_blocks and pa_swap_blocks take the same block sizes).
 * Returns PA_ERR_NULL, PA_ERR_SHAPE (negative sizes, tensors not 16-byte
 * aligned), PA_ERR_UNSUPPORTED or PA_ERR_LAUNCH before or at the launch;
 * the copy itself cannot fail.
 */
pa_status_t pa_write_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                        const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                        int head_dim, int block_size, int num_blocks, pa_dtype_t dtype,
                        void* stream);

/*
 * pa_copy_blocks -- batched copy-on-write block copies.  For each pair
 * (src, dst): the whole K block k_pool[dst] = k_pool[src] (every KV head,
 * every slot) and the same for V, in one launch (PagedAttention and vLLM:
 * Paging the KV Cache Like an OS, "Step 4" copy-on-write and "Step 5" the
 * batched copy kernel).  Destinations must be distinct from one another and
 * from every source (the block manager guarantees this); pairs with an id
 * outside [0, num_blocks) are skipped.
 *
 *   block_pairs      device, int32 [num_pairs][2]
 */
pa_status_t pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* block_pairs,
                           int num_pairs, int num_kv_heads, int head_dim, int block_size,
                           int num_blocks, pa_dtype_t dtype, void* stream);

/*
 * pa_swap_blocks -- batched whole-block copies between two pools of the same
 * block shape, for preemption by swapping: evicted blocks go from the device
 * pool to a pool in host memory and come back later, possibly to other block
 * ids (PagedAttention: Virtual Memory for the KV Cache, "Scheduling and
 * preemption"; Batching and PagedAttention, FAQ on running out of blocks).
 * For each pair (src, dst):
 *   dst_k[dst] = src_k[src] and dst_v[dst] = src_v[src]  (every KV head, every slot).
 * Swap-out: dst = host pool, src = device pool; swap-in the reverse; both
 * device pools also work.  One launch; the GPU reads or writes the host pool
 * directly over the host link.
 *
 *   dst_k, dst_v     [num_dst_blocks][num_kv_heads][block_size][head_dim], dtype
 *   src_k, src_v     [num_src_blocks][num_kv_heads][block_size][head_dim], dtype
 *   block_pairs      int32 [num_pairs][2] = (src id, dst id)
 * Every pointer must be device memory or pinned, device-mapped host memory
 * (hipHostMalloc, or a torch tensor made with pin_memory=True); anything else
 * (pageable memory) returns PA_ERR_SHAPE before any launch.  Pairs with an id
 * outside its pool are skipped.  Destinations must be distinct and must not
 * overlap a source block of the same call.
 */
pa_status_t pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                           const int32_t* block_pairs, int num_pairs, int num_kv_heads, int head_dim,
                           int block_size, int num_src_blocks, int num_dst_blocks, pa_dtype_t dtype,
                           void* stream);

/* Message for the last non-OK status on this thread ("" if none). */
const char* pa_last_error(void);

/* ABI version of this header (bumped on incompatible changes). */
int pa_abi_version(void);

/*
 * Host block manager (CPU only; no GPU calls).  A FIFO free list of physical
 * block ids, a reference count per block and one block table per sequence
 * (PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 3" and
 * "Step 4"; vLLM's PagedAttention: How Memory Management Supports Large Model
 * Inference, "2.2", "2.3" and "7").
 *   - A block is taken from the front of the free list only when a sequence's
 *     last block is full (on-demand allocation).
 *   - fork copies the parent's table and increments each block's count.
 *   - Appending into a partly filled last block whose count is > 1 first
 *     copies it (copy-on-write): a fresh block is taken, (src, dst) is queued
 *     for pa_copy_blocks, the table is repointed and src's count drops.  A
 *     writer that finds the count at 1 writes in place.  Full blocks are never
 *     copied.
 *   - Freeing a sequence decrements its blocks' counts; blocks reaching 0
 *     return, in table order, to the back of the free list -- except blocks
 *     named by a queued copy, which are held until pa_bm_take_copies.
 *   - Appends are all-or-nothing: PA_ERR_NO_BLOCKS leaves every table, count
 *     and the free list unchanged.
 * A pa_bm_t is not thread-safe; use one per thread or lock around it.
 */
typedef struct pa_bm pa_bm_t;

/* initial_free_order: NULL (0..num_blocks-1) or a permutation of 0..num_blocks-1.
 * Returns NULL on invalid arguments (message in pa_last_error). */
pa_bm_t* pa_bm_create(int num_blocks, int block_size, const int32_t* initial_free_order);
void pa_bm_destroy(pa_bm_t* bm);
pa_status_t pa_bm_add_seq(pa_bm_t* bm, int64_t seq_id);
/* Reserve slots for n_tokens more tokens; slots_out (nullable) receives
 * n_tokens int64 slots. */
pa_status_t pa_bm_append(pa_bm_t* bm, int64_t seq_id, int n_tokens, int64_t* slots_out);
/* One token for each of n sequences (distinct ids), all or nothing over the
 * batch; slots_out receives n slots in order. */
pa_status_t pa_bm_append_batch(pa_bm_t* bm, const int64_t* seq_ids, int n, int64_t* slots_out);
pa_status_t pa_bm_fork(pa_bm_t* bm, int64_t parent, int64_t child);
pa_status_t pa_bm_free_seq(pa_bm_t* bm, int64_t seq_id);
/* Writes up to cap entries of the table; returns its length (-1: unknown id). */
int pa_bm_table(const pa_bm_t* bm, int64_t seq_id, int32_t* out, int cap);
/* Fills out[n][max_blocks] with the tables of seq_ids, padding with pad.
 * PA_ERR_SHAPE if a table is longer than max_blocks. */
pa_status_t pa_bm_tables(const pa_bm_t* bm, const int64_t* seq_ids, int n, int32_t* out,
                         int max_blocks, int32_t pad);
/* Token count of a sequence (-1: unknown id). */
int pa_bm_num_tokens(const pa_bm_t* bm, int64_t seq_id);
/* Number of queued copy-on-write pairs. */
int pa_bm_num_pending_copies(const pa_bm_t* bm);
/* Drains the queued (src, dst) pairs into pairs_out[cap][2] and releases held
 * blocks.  Returns the number of pairs, or -1 (nothing drained) if cap is
 * smaller than pa_bm_num_pending_copies. */
int pa_bm_take_copies(pa_bm_t* bm, int32_t* pairs_out, int cap);
int pa_bm_num_free(const pa_bm_t* bm);
/* Reference count of a block (-1: out of range). */
int pa_bm_refcount(const pa_bm_t* bm, int32_t block);

/*
 * Swapping (PagedAttention: Virtual Memory for the KV Cache, "Scheduling and
 * preemption": a group -- e.g. the beams of one request -- is evicted whole,
 * its blocks copied to CPU memory and brought back later).  The host pool
 * has its own FIFO free list of host block ids 0..num_host_blocks-1 and its
 * own counts.
 *   - swap_out(group): every distinct block of the group's tables goes to a
 *     host block popped from the host free list, in order of first
 *     appearance (sequence order, then table order); pairs_out receives
 *     (device block, host block) for pa_swap_blocks; the device blocks return
 *     to the back of the free list; tables now hold host ids.  Refused
 *     (nothing changes) if a block is shared with a sequence outside the
 *     group (PA_ERR_SHAPE), copy-on-write pairs are pending (PA_ERR_SHAPE:
 *     take and run them first), or the host pool is short (PA_ERR_NO_BLOCKS).
 *   - swap_in(group): the reverse, into device blocks popped from the free
 *     list; pairs_out receives (host block, device block).
 *   - A swapped-out sequence cannot be appended to, forked or exported with
 *     pa_bm_tables; pa_bm_free_seq releases its host blocks.
 * pairs_out must hold cap >= the number of distinct blocks (at most the sum
 * of the group's table lengths) pairs of int32.
 */
pa_status_t pa_bm_set_host_blocks(pa_bm_t* bm, int num_host_blocks);
pa_status_t pa_bm_swap_out(pa_bm_t* bm, const int64_t* seq_ids, int n, int32_t* pairs_out, int cap,
                           int* num_pairs_out);
pa_status_t pa_bm_swap_in(pa_bm_t* bm, const int64_t* seq_ids, int n, int32_t* pairs_out, int cap,
                          int* num_pairs_out);
/* 1 swapped out, 0 on the device, -1 unknown id. */
int pa_bm_is_swapped(const pa_bm_t* bm, int64_t seq_id);
int pa_bm_num_host_free(const pa_bm_t* bm);
/* Count of a host block (-1: out of range). */
int pa_bm_host_refcount(const pa_bm_t* bm, int32_t host_block);

/*
 * Prefix cache (vLLM's PagedAttention: How Memory Management Supports Large
 * Model Inference, "2.4" and "7"; PagedAttention (tensortonic), "8. Reusing
 * Work Across Separate Requests").  A manager made by pa_bm_create_cached
 * keys every full block by a chained hash
 *   h_j = SHA-256(h_{j-1} || tokens of block j as int32 little-endian || extra_key),
 * h_{-1} = 32 zero bytes, and keeps a map from hash to block.
 *   - pa_bm_add_seq_cached starts a sequence from its prompt: it walks the
 *     prompt's full blocks and takes each matching cached block (count + 1)
 *     until the first miss.  *num_cached_out = the tokens whose K/V are
 *     already in those blocks, except that a prompt found whole still
 *     computes its last token (n_tokens - 1).  The caller then appends the
 *     rest with pa_bm_append_tokens.
 *   - pa_bm_append_tokens appends like pa_bm_append and enters each block
 *     that fills into the map (the first block with a given hash keeps the
 *     entry).  pa_bm_append / pa_bm_append_batch also work but leave the
 *     sequence's later blocks unhashed (no token ids).
 *   - Freed blocks keep their entries and go to the back of the free list,
 *     a sequence's last blocks first; a block taken from the front loses its
 *     entry.  The free list is thus the eviction order (least recently freed
 *     first), and a block in use is never evicted.
 * pa_bm_add_seq_cached / pa_bm_append_tokens return PA_ERR_UNSUPPORTED on a
 * manager made by pa_bm_create.
 */
pa_bm_t* pa_bm_create_cached(int num_blocks, int block_size, const int32_t* initial_free_order);
pa_status_t pa_bm_add_seq_cached(pa_bm_t* bm, int64_t seq_id, const int32_t* tokens, int n_tokens,
                                 const void* extra_key, int extra_len, int* num_cached_out);
pa_status_t pa_bm_append_tokens(pa_bm_t* bm, int64_t seq_id, const int32_t* tokens, int n_tokens,
                                int64_t* slots_out);
/* Entries in the hash map. */
int pa_bm_num_cached_blocks(const pa_bm_t* bm);
/* The chained hash of a sequence's j-th full block into out32 (0), or -1. */
int pa_bm_block_hash(const pa_bm_t* bm, int64_t seq_id, int j, uint8_t* out32);
/* The block the map holds for a 32-byte hash, or -1. */
int pa_bm_cached_block(const pa_bm_t* bm, const uint8_t* hash32);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
