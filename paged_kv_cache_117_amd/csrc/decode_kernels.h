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
  float* ws_o;  // [B][Hq][P][D] partition outputs (normalised)
  float* ws_m;  // [B][Hq][P] running max, base-2 domain
  float* ws_l;  // [B][Hq][P] running sum
  uint32_t* ctr;  // work-queue counters (ticket, done); zero between calls
  int persist_grid;  // > 0: persistent MFMA kernel with this many workgroups
  int B, Hq, Hkv, g, gmax, nsub, D;
  int num_blocks, maxb, max_ctx, psize, P;
  float qscale;  // scale * log2(e)
  pa_dtype_t dtype;
};

// Workspace: 256 bytes of work-queue counters (must be zero before the
// first call; every call leaves them zero), then, when some sequence spans
// more than one partition, the partition partials.
struct WorkspaceLayout {
  size_t ctr_off, o_off, m_off, l_off, total;
};

constexpr size_t kCounterBytes = 256;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline WorkspaceLayout workspace_layout(size_t B, size_t Hq, size_t D, size_t P) {
  WorkspaceLayout w{};
  w.ctr_off = 0;
  w.total = kCounterBytes;
  if (P <= 1) return w;
  const size_t rows = B * Hq * P;
  w.o_off = kCounterBytes;
  w.m_off = w.o_off + align256(rows * D * sizeof(float));
  w.l_off = w.m_off + align256(rows * sizeof(float));
  w.total = w.l_off + align256(rows * sizeof(float));
  return w;
}

// The persistent MFMA kernel keeps every sequence's length and item counts in
// LDS: it serves batches up to this size.
constexpr int kPersistMaxSeqs = 1024;
// Threads per persistent workgroup: 8 compute waves, a merge wave and a fill
// wave.
constexpr int kPersistThreads = 640;

// Partition kernels (the reduce is launched separately when P > 1).
void launch_decode_valu(const DecodeArgs& a, hipStream_t st);   // any dtype
void launch_decode_mfma(const DecodeArgs& a, hipStream_t st);   // fp16 / bf16; launches the reduce itself
void launch_decode_reduce(const DecodeArgs& a, hipStream_t st);
// The persistent kernel for (dtype, head_dim, gmax), or NULL when there is
// none (gmax other than 4 or 8); for occupancy queries.
const void* decode_persist_kernel(pa_dtype_t dtype, int head_dim, int gmax);

}  // namespace pa
