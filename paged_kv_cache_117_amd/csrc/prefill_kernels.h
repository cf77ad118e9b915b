// Internal interface between the pa_prefill entry point and its kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

// Matrix column groups (16 query rows each) per wavefront of the prefill
// kernel; a workgroup of 4 wavefronts takes 64 * kPrefillNC rows.
constexpr int kPrefillNC = 2;
constexpr int kPrefillRows = 64 * kPrefillNC;
// Kernel variants of the 16-bit path: K/V staged through registers into
// LDS; loaded straight into LDS by 4-wavefront workgroups of kPrefillRows
// rows; the same with 8-wavefront workgroups of kWideRows rows (one per
// compute unit, two wavefronts per SIMD, each step's K/V shared by twice the
// rows).
constexpr int kPrefillRegs = 0, kPrefillDirect = 1, kPrefillWide = 2;
constexpr int kWideWaves = 8;
constexpr int kWideRows = 64 * kPrefillNC * 2;

struct PrefillArgs {
  void* out;
  const void* q;
  const char* kp;
  const char* vp;
  const int32_t* bt;
  const int32_t* cl;
  const int32_t* qs;  // query_start [B + 1], or NULL: row s is sequence s's one query row
  int B, N, Hq, Hkv, g, D;
  int num_blocks, maxb, max_q;
  int tiles;      // row tiles per (sequence, KV head) in the launch
  int P;          // position partitions per row tile (1: no split, rows written directly)
  int psteps;     // steps (64 positions each) per partition when P > 1
  int max_ctx;    // every context length must be <= this when P > 1
  float* ws_o;    // P > 1: [N * Hq][P][D] normalised partial rows
  float* ws_m;    // P > 1: [N * Hq][P] reference max, base-2 domain
  float* ws_l;    // P > 1: [N * Hq][P] sum of weights
  int grid;       // workgroups launched: 8 x ranks per XCD (see prefill_grid_ranks)
  int neg_scale;  // scale < 0: the kernel flips the query's sign
  int lbs;        // log2(block_size)
  float qscale;   // |scale| * log2(e)
  pa_dtype_t dtype;
  int kind;        // kPrefillRegs, kPrefillDirect or kPrefillWide
  void* ev_start;  // caller's timing events for prefill_mfma (hipEvent_t, or NULL)
  void* ev_stop;
};

// Positions per step of the prefill kernel (partitions are whole steps).
constexpr int kPrefillStep = 64;

// Work items (sequence, KV head) per lane of the kernel's longest-walk-first
// pick: unsplit launches with up to 64 * kLptPerLane items per XCD use it.
constexpr int kLptPerLane = 4;

// Workspace of a split launch: partial rows, then maxima, then sums.
struct PrefillWorkspace {
  size_t o_off, m_off, l_off, total;
};

inline PrefillWorkspace prefill_workspace(size_t N, size_t Hq, size_t D, size_t P) {
  PrefillWorkspace w{};
  if (P <= 1) return w;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rows = N * Hq * P;
  w.m_off = al(rows * D * sizeof(float));
  w.l_off = w.m_off + al(rows * sizeof(float));
  w.total = w.l_off + al(rows * sizeof(float));
  return w;
}

void launch_prefill_mfma(const PrefillArgs& a, hipStream_t st);    // fp16 / bf16, main kernel only

// Decode attention (one query row per sequence) through the prefill kernel:
// pa_decode's route for blocks of 8 slots, which its 16-slot tiles cannot
// walk.  Arguments checked by the caller except the workspace.
size_t decode_rows_workspace(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int max_context_len,
                             int partition_size);
pa_status_t decode_rows(const char* who, void* out, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int num_q_heads,
                        int num_kv_heads, int head_dim, int lbs, int num_blocks, int max_blocks_per_seq,
                        int max_context_len, int partition_size, float scale, pa_dtype_t dtype, void* workspace,
                        size_t workspace_bytes, void* stream);
void launch_prefill_reduce(const PrefillArgs& a, hipStream_t st);  // the merge (nothing when P == 1)

}  // namespace pa
