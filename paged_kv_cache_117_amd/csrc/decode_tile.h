// Tile machinery of the 16-bit decode path on gfx950, shared by the decode
// kernels (decode_mfma.hip) and the decode-shaped rows of the prefill kernel
// (prefill.hip): one wavefront computes attention of up to 16 query rows
// against 16-slot tiles of one KV head with both products on the matrix
// cores, K and V loaded straight into the operand registers.
//
// Per tile (16 consecutive slots of one block -- a block of 16 << lm slots
// holds 2^lm tiles -- and one KV head):
//  * Scores S = K q^T are one chain of v_mfma_f32_16x16x32_{bf16,f16}: the K
//    tile is the A operand (lane (G, c) loads 16 bytes of token c at dims
//    32k+8G, exactly the operand layout, so K goes from HBM to the matrix
//    core with no shuffles), the query rows padded to 16 with zeros are the
//    B operand.  Lane (G, c) receives S[token 4G+j][row c], j = 0..3.
//  * PV is computed transposed, O^T = V^T P, with v_mfma_f32_16x16x16: lane
//    (G, c) loads tokens 4G..4G+3 at dims [c*DPL, +DPL) of the V tile, so the
//    A operand (rows = dims, k = those four tokens) needs only an in-register
//    v_perm_b32 interleave, and the B operand (k = tokens, n = rows) is the
//    lane's own four weights from the score layout.  The output has the row
//    in the lane's column, so the online-softmax rescale multiplies by the
//    lane's own factor: no cross-lane traffic in PV.
//  * Rescaling by 2^(m_old - m_new) is unconditional (branch-free); it is
//    exactly 1 when the running max did not grow.
//  * KV tiles are loaded non-temporally: each is read once per step.
// Everything here lives in an anonymous namespace: each kernel source gets
// its own copy.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_device.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

// 16 tokens x 32 dims (A) times 32 dims x 16 heads (B), fp32 accumulate.
template <int DT>
__device__ __forceinline__ f32x4 mfma_qk(const uint4& a, const uint4& b, const f32x4& c) {
  if constexpr (DT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}

// 16 dims x 4k tokens (A: a0 = k 0,1; a1 = k 2,3 of this lane's k-group)
// times 4k tokens x 16 heads (B, same packing), fp32 accumulate.
template <int DT>
__device__ __forceinline__ f32x4 mfma_pv(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, const f32x4& c) {
  const uint2 a = make_uint2(a0, a1);
  const uint2 b = make_uint2(b0, b1);
  if constexpr (DT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, a), __builtin_bit_cast(bf16x4, b), c,
                                                     0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                                 0);
  }
}

// Two fp32 weights rounded (nearest even) to the KV type, `a` in the low half.
template <int DT>
__device__ __forceinline__ uint32_t pack_pair(float a, float b) {
  if constexpr (DT == PA_BF16) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    const f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// The value of lane l combined (`op`) with the value of lane l^16 (resp.
// l^32), i.e. the other token groups of the MFMA output layout, through the
// LDS crossbar (ds_bpermute; `addr` is the partner lane times 4).  gfx950's
// v_permlane16/32_swap would stay on the VALU, but this compiler folds the
// two results of the swap intrinsic into one when they are combined.
template <typename Op>
__device__ __forceinline__ float xchg(float x, int addr, Op op) {
  return op(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(addr, __builtin_bit_cast(int, x))));
}
struct MaxOp {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct AddOp {
  __device__ float operator()(float a, float b) const { return a + b; }
};

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Workgroup barrier that orders LDS only: the waves exchange nothing else,
// and __syncthreads() would also make a wave with global stores in flight
// wait for them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-lane tile machinery of one wavefront.
template <int DT, int D>
struct Tile {
  static constexpr int ROWB = D * 2;  // bytes of one token row of one head
  static constexpr int KS = D / 32;   // QK MFMA k-steps over the head dim
  static constexpr int DPL = D / 16;  // V dims per lane = PV MFMAs per tile
  static constexpr int NW = DPL / 2;  // 32-bit words per V row in this lane
  static constexpr int QROW = D + 8;  // LDS row stride (elements) of the query tile: conflict-free operand reads
  static constexpr int QCH = D / 8;   // 16-byte chunks per query row
  using VVec = typename std::conditional<DPL == 8, uint4, uint2>::type;

  // Thread `tid`'s 16-byte chunk of the query group (16 rows, rows >= nh
  // zero; `qrow0` is the group's first row), for store_q.
  __device__ static __forceinline__ uint4 load_q(const char* qrow0, int nh, int tid) {
    const int h = tid / QCH, c = tid - h * QCH;
    return h < nh ? *reinterpret_cast<const uint4*>(qrow0 + (size_t)h * ROWB + c * 16) : make_uint4(0, 0, 0, 0);
  }
  __device__ static __forceinline__ void store_q(uint16_t (*sq)[QROW], const uint4& v, int tid) {
    const int h = tid / QCH, c = tid - h * QCH;
    if (h < 16) *reinterpret_cast<uint4*>(&sq[h][c * 8]) = v;
  }

  // One (block, head) tile at `kb` / `vb`, non-temporal loads.  Offsets are
  // unsigned 32-bit so the loads take the scalar tile base plus a 32-bit
  // vector offset.  K and V rows past `rmax` (the block's last filled slot)
  // re-read that row (same cache lines, no extra memory traffic): their
  // scores are masked, their weights exactly 0, and the values are finite.
  __device__ static __forceinline__ void load(const char* kb, const char* vb, int grp, int col, int rmax,
                                              uint4 (&kr)[KS], VVec (&vr)[4]) {
    const uint32_t k_lane = min(col, rmax) * ROWB + grp * 16;
    const uint32_t v_col = col * DPL * 2;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + (k_lane + k * 64)));
      kr[k] = make_uint4(t.x, t.y, t.z, t.w);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* pv = vb + ((uint32_t)min(grp * 4 + i, rmax) * ROWB + v_col);
      if constexpr (DPL == 8) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pv));
        vr[i] = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pv));
        vr[i] = make_uint2(t.x, t.y);
      }
    }
  }

  // The same tile for the fused write and decode: when `is_new` (the tile
  // holds its sequence's last position, slot `rmax`, whose K and V rows are
  // still at `knew` / `vnew`), rows at and past `rmax` come from there
  // instead of the pool, so the tile computes exactly what it computes once
  // the rows are in the pool.  Branch-free (per-lane address selects, the
  // same load instructions for every tile): a branch here would define the
  // tile registers on two paths and the copies at the join would make every
  // tile wait for all loads in flight.
  __device__ static __forceinline__ void load_sel(const char* kb, const char* vb, const char* knew, const char* vnew,
                                                  bool is_new, int grp, int col, int rmax, uint4 (&kr)[KS],
                                                  VVec (&vr)[4]) {
    const char* kl = ((is_new && col >= rmax) ? knew : kb + (uint32_t)min(col, rmax) * ROWB) + grp * 16;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kl + k * 64));
      kr[k] = make_uint4(t.x, t.y, t.z, t.w);
    }
    const uint32_t v_col = col * DPL * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = min(grp * 4 + i, rmax);
      const char* pv = ((is_new && r == rmax) ? vnew : vb + (uint32_t)r * ROWB) + v_col;
      if constexpr (DPL == 8) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(pv));
        vr[i] = make_uint4(t.x, t.y, t.z, t.w);
      } else {
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(pv));
        vr[i] = make_uint2(t.x, t.y);
      }
    }
  }

  // The new token's K and V rows of a tile loaded by load_sel, from the
  // lanes that hold them, to slot `rmax` of the tile at `kb` / `vb`: lanes
  // with col = rmax hold its K row (16 bytes per k-step and lane group),
  // lanes of group rmax / 4 its V row (this lane's dims).
  __device__ static __forceinline__ void store_new(char* kb, char* vb, int grp, int col, int rmax,
                                                   const uint4 (&kr)[KS], const VVec (&vr)[4]) {
    if (col == rmax) {
#pragma unroll
      for (int k = 0; k < KS; ++k) *reinterpret_cast<uint4*>(kb + (uint32_t)rmax * ROWB + grp * 16 + k * 64) = kr[k];
    }
    // (one predicated store per row slot, each with a static index: a
    // selected vr[rmax & 3] would become a dynamic index, and the compiler
    // would then keep the V tile in LDS)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (grp * 4 + i == rmax) *reinterpret_cast<VVec*>(vb + (uint32_t)rmax * ROWB + col * DPL * 2) = vr[i];
  }

  // Scores (MFMA), online-softmax update, PV (MFMA) for one tile whose first
  // slot in this lane's group is token `tok0`; tokens at or past `lim` get
  // score -inf.  The QK B operand is read from the LDS query tile (`qsrc`:
  // this lane's row and k-group) one 32-dim step at a time, next to its
  // MFMA (4 live VGPRs instead of 16), and the scheduling barriers keep each
  // pair of PV permutes next to its MFMA (computed all at once they would
  // hold 4*NW more).  Straight-line code: branches here make the compiler
  // duplicate the accumulator.
  __device__ static __forceinline__ void consume(const uint4 (&kr)[KS], const VVec (&vr)[4], const uint16_t* qsrc,
                                                 int tok0, int lim, float qscale, int x16, int x32, float& m_run,
                                                 float& l_run, f32x4 (&acc)[DPL]) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      const uint4 qk = *reinterpret_cast<const uint4*>(qsrc + k * 32);
      sacc = mfma_qk<DT>(kr[k], qk, sacc);
      __builtin_amdgcn_sched_barrier(0);
    }
    float sv[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) sv[jj] = tok0 + jj < lim ? sacc[jj] * qscale : kNegInf;
    float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
    bm = xchg(bm, x16, MaxOp());
    bm = xchg(bm, x32, MaxOp());
    const float mn = fmaxf(m_run, bm);
    const float alpha = fast_exp2(m_run - mn);
    m_run = mn;
    l_run *= alpha;
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[u] *= alpha;
    float pv[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) pv[jj] = fast_exp2(sv[jj] - m_run);
    l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
    // B operand: P[token 4G+e][head col], e = 0..3, rounded to the KV type.
    const uint32_t pb0 = pack_pair<DT>(pv[0], pv[1]);
    const uint32_t pb1 = pack_pair<DT>(pv[2], pv[3]);
    // A operand for output dims DPL*m + u: V[token 4G+e][dim DPL*col + u];
    // v_perm_b32 gathers the same dim of two token rows into one word.
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t r0 = (&vr[0].x)[w], r1 = (&vr[1].x)[w], r2 = (&vr[2].x)[w], r3 = (&vr[3].x)[w];
      acc[2 * w] = mfma_pv<DT>(__builtin_amdgcn_perm(r1, r0, 0x05040100u), __builtin_amdgcn_perm(r3, r2, 0x05040100u),
                               pb0, pb1, acc[2 * w]);
      __builtin_amdgcn_sched_barrier(0);
      acc[2 * w + 1] = mfma_pv<DT>(__builtin_amdgcn_perm(r1, r0, 0x07060302u),
                                   __builtin_amdgcn_perm(r3, r2, 0x07060302u), pb0, pb1, acc[2 * w + 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // This wave's result into LDS: l summed over the four token groups, then
  // (m, l) of head `col` (l = 0 for a wave without tokens) and, when the
  // wave saw any token, the normalised rows o = acc / l (acc[u][j] holds dim
  // DPL*(4*grp + j) + u).
  __device__ static __forceinline__ void stage(float m_run, float l_run, const f32x4 (&acc)[DPL], bool any, int grp,
                                               int col, int nh, int x16, int x32, float* sm, float* sl, float* srow) {
    l_run = xchg(xchg(l_run, x16, AddOp()), x32, AddOp());
    if (grp == 0) {
      sm[col] = m_run;
      sl[col] = any ? l_run : 0.f;
    }
    if (any && col < nh) {
      const float inv = 1.f / l_run;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float* dst = srow + col * D + DPL * (4 * grp + jj);
#pragma unroll
        for (int u = 0; u < DPL; u += 4)
          *reinterpret_cast<float4*>(dst + u) =
              make_float4(acc[u][jj] * inv, acc[u + 1][jj] * inv, acc[u + 2][jj] * inv, acc[u + 3][jj] * inv);
      }
    }
  }
};

// The two-tile pipeline of one wave over its tiles k = 0..cnt-1 (cnt >= 1):
// issue(k, K, V) loads tile k, consume(k, K, V, valid) computes it.  Inside
// the loop every issue is unconditional and names an existing tile, so the
// loads stay in a fixed order and each consume waits only for its own tile;
// the last one to three tiles are consumed after the loop on straight-line
// paths of their own (exact wait counts on each), with no load past the last
// tile (a load the wave never consumes still delays the wave's end by a
// memory round trip).  With cnt = 1 the prologue loads tile 0 into both
// buffers.  The scheduling barriers keep each tile's work and its prefetch
// in program order (left alone, the scheduler hoists the next tile's MFMAs
// above this tile's PV, so a consume waits for both buffers), and the
// compiler memory barriers keep the prologue's A before B as in the loop
// (else the wait counts, merged over both paths, make A wait for half of B).
// The pool pointers behind `issue` must not be __restrict__: loads through
// restrict pointers may move across those barriers.  `preloaded`: the caller
// has already issued tiles 0 and min(1, cnt-1) into A and B.
// kExactTail = false keeps one loop for the whole walk instead (the last
// iterations re-read the last tile, consuming it as empty): half the code
// and fewer live registers, which the partition kernels need to keep four
// waves per SIMD.
template <bool kExactTail = true, typename KBuf, typename VBuf, typename Issue, typename Consume>
__device__ __forceinline__ void pipeline(int cnt, KBuf& kA, VBuf& vA, KBuf& kB, VBuf& vB, Issue&& issue,
                                         Consume&& consume, bool preloaded = false) {
  const int last = cnt - 1;
  __builtin_amdgcn_sched_barrier(0);
  if (!preloaded) {
    issue(0, kA, vA);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(min(1, last), kB, vB);
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!kExactTail) {
    for (int k = 0; k < cnt; k += 2) {
      consume(k, kA, vA, true);
      __builtin_amdgcn_sched_barrier(0);
      issue(min(k + 2, last), kA, vA);
      __builtin_amdgcn_sched_barrier(0);
      consume(k + 1, kB, vB, k + 1 < cnt);
      __builtin_amdgcn_sched_barrier(0);
      issue(min(k + 3, last), kB, vB);
      __builtin_amdgcn_sched_barrier(0);
    }
    return;
  }
  int k = 0;
  for (; k + 3 < cnt; k += 2) {  // tiles k+2 and k+3 exist
    consume(k, kA, vA, true);
    __builtin_amdgcn_sched_barrier(0);
    issue(k + 2, kA, vA);
    __builtin_amdgcn_sched_barrier(0);
    consume(k + 1, kB, vB, true);
    __builtin_amdgcn_sched_barrier(0);
    issue(k + 3, kB, vB);
    __builtin_amdgcn_sched_barrier(0);
  }
  // cnt - k tiles remain (1, 2 or 3): A holds tile k, B tile k + 1 (or a
  // copy of tile k when cnt = 1)
  const int r = cnt - k;
  consume(k, kA, vA, true);
  __builtin_amdgcn_sched_barrier(0);
  if (r == 3) {
    issue(k + 2, kA, vA);
    __builtin_amdgcn_sched_barrier(0);
    consume(k + 1, kB, vB, true);
    __builtin_amdgcn_sched_barrier(0);
    consume(k + 2, kA, vA, true);
  } else if (r == 2) {
    consume(k + 1, kB, vB, true);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Lane k's tile row for logical 16-slot tile bidx(k), k < cnt (0 elsewhere):
// the tile is slots [16 (t mod 2^lm), +16) of table entry t >> lm, i.e. row
// ((id * Hkv + kvh) << lm) + t mod 2^lm of 16 * ROWB bytes.  Ids outside
// [0, num_blocks) become 0, never dereferenced, and set `bad` (in every lane).
template <typename F>
__device__ __forceinline__ int load_ids(const int32_t* btrow, int cnt, int num_blocks, F bidx, bool& bad, int Hkv,
                                        int kvh, int lm) {
  const int lane = threadIdx.x & 63;
  int id = 0, t = 0;
  if (lane < cnt) {
    t = bidx(lane);
    id = btrow[t >> lm];
  }
  const bool ok = id >= 0 && id < num_blocks;
  bad = !__all(lane >= cnt || ok);
  return ok ? ((id * Hkv + kvh) << lm) | (t & ((1 << lm) - 1)) : 0;
}

}  // namespace
}  // namespace pa
