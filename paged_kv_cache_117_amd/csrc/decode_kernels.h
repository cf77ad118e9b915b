// Internal interface between the pa_decode entry point and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

struct DecodeArgs {
  void* out;
  const void* q;
  const char* kp;
  const char* vp;
  const int32_t* bt;
  const int32_t* cl;
  float* ws_o;  // [B][Hq][entries][D] partition (group) outputs, normalised
  float* ws_m;  // [B][Hq][entries] running max, base-2 domain
  float* ws_l;  // [B][Hq][entries] running sum
  int2* info;     // balanced split: [B][Hkv * nsub] (first piece slot, piece count) per segment
  int stream;     // balanced-split kernel (ws_o / ws_m / ws_l hold its pieces)
  int unit;       // balanced split: blocks per unit of work
  int grid;       // balanced split: workgroups
  int wave_part;  // MFMA kernels: one wavefront per partition (partitions of <= 64 blocks)
  int entries;    // partial entries per (sequence, query head) row of the workspace actually used
  int per_entry;  // partitions merged into one entry: ceil(nparts / per_entry) entries per sequence
  int B, Hq, Hkv, g, gmax, nsub, D;
  int num_blocks, maxb, max_ctx, psize, P;
  float qscale;  // scale * log2(e)
  pa_dtype_t dtype;
  int lm;        // log2(block_size / 16): the kernels walk 16-slot tiles, 2^lm per block
  // VALU kernel only: several query tokens per sequence (pa_prefill on fp32
  // KV).  B is then the number of query tokens, qst the [nseq + 1] row starts.
  const int32_t* qst;
  int nseq, max_q;
  // Fused write (stream kernel): the step's new K/V rows [B][Hkv][D], read
  // for each sequence's last position and stored into its pool slot; NULL
  // for plain decode.
  const char* kn;
  const char* vn;
  // Caller's timing events for the main kernel (hipEvent_t, or NULL): passed
  // to its launch, so they take the kernel's own start and end.
  void* ev_start;
  void* ev_stop;
};

// Workspace: the partition partials, when some sequence spans more than one
// partition (sized for P entries per row, the most any kernel uses).
struct WorkspaceLayout {
  size_t o_off, m_off, l_off, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline WorkspaceLayout workspace_layout(size_t B, size_t Hq, size_t D, size_t P) {
  WorkspaceLayout w{};
  if (P <= 1) return w;
  const size_t rows = B * Hq * P;
  w.o_off = 0;
  w.m_off = align256(rows * D * sizeof(float));
  w.l_off = w.m_off + align256(rows * sizeof(float));
  w.total = w.l_off + align256(rows * sizeof(float));
  return w;
}

// Balanced split: batches up to this many sequences (their lengths are
// staged in LDS), at most this many wavefronts (two piece slots each).
constexpr int kStreamMaxSeqs = 4096;
constexpr int kStreamMaxWaves = 4096;

// Query heads per work item of the MFMA kernels (one matrix column each).
inline int mfma_gmax(int g) { return g <= 4 ? 4 : g <= 8 ? 8 : 16; }

// Workspace of the balanced split: pieces (o [slot][gmax][D], m and l
// [slot][gmax]) for two slots per wavefront (2 * kStreamMaxWaves when the
// device is not known), then the segment records.
struct StreamLayout {
  size_t o_off, m_off, l_off, info_off, total;
};

inline StreamLayout stream_layout(size_t B, size_t Hq, size_t Hkv, size_t D, size_t max_waves = kStreamMaxWaves) {
  const size_t g = Hq / Hkv, gmax = (size_t)mfma_gmax((int)g), nsub = (g + gmax - 1) / gmax;
  const size_t slots = 2 * max_waves;
  StreamLayout w{};
  w.o_off = 0;
  w.m_off = align256(slots * gmax * D * sizeof(float));
  w.l_off = w.m_off + align256(slots * gmax * sizeof(float));
  w.info_off = w.l_off + align256(slots * gmax * sizeof(float));
  w.total = w.info_off + align256(B * Hkv * nsub * 2 * sizeof(int));
  return w;
}

// Partition kernels (the reduce is launched separately when P > 1).
void launch_decode_valu(const DecodeArgs& a, hipStream_t st);   // any dtype
void launch_decode_mfma(const DecodeArgs& a, hipStream_t st);   // fp16 / bf16, main kernel only
void launch_decode_reduce(const DecodeArgs& a, hipStream_t st);
void launch_decode_stream_reduce(const DecodeArgs& a, hipStream_t st);  // the balanced split's merge

// Each sequence's new K/V rows to its last position through its block table
// (the fused write and decode, when the decode runs another kernel than the
// even split).  Launched on `st`.
void launch_write_last(void* k_pool, void* v_pool, const void* k_new, const void* v_new, const int32_t* bt,
                       const int32_t* cl, int num_seqs, int maxb, int max_ctx, int num_kv_heads, int head_dim,
                       int elem_bytes, int lbs, int num_blocks, hipStream_t st);

}  // namespace pa
