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

struct PrefillArgs {
  void* out;
  const void* q;
  const char* kp;
  const char* vp;
  const int32_t* bt;
  const int32_t* cl;
  const int32_t* qs;  // query_start [B + 1]
  int B, N, Hq, Hkv, g, D;
  int num_blocks, maxb, max_ctx, max_q;
  int tiles;      // row tiles per (sequence, KV head) in the launch
  int grid;       // workgroups launched: 8 * ceil(B * Hkv / 8) * tiles
  int neg_scale;  // scale < 0: the kernel flips the query's sign
  int lbs;        // log2(block_size)
  float qscale;   // |scale| * log2(e)
  pa_dtype_t dtype;
};

void launch_prefill_mfma(const PrefillArgs& a, hipStream_t st);  // fp16 / bf16

}  // namespace pa
