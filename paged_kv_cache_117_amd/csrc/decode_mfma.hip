// pa_decode partition kernels for 16-bit KV (fp16 / bf16) on gfx950.
//
// Same computation as the VALU kernel in decode.hip (online softmax over a
// partition's blocks in logical order, base-2 exponentials, log-sum-exp
// partials), organised for bandwidth with both products on the matrix cores.
//
// Per tile (16 slots of one block, one KV head), in one wavefront:
//  * Scores S = K q^T are one chain of v_mfma_f32_16x16x32_{bf16,f16}: the K
//    tile is the A operand (lane (G, c) loads 16 bytes of token c at dims
//    32k+8G, exactly the operand layout, so K goes from HBM to the matrix
//    core with no shuffles), the query group padded to 16 heads with zeros is
//    the B operand.  Lane (G, c) receives S[token 4G+j][head c], j = 0..3.
//  * PV is computed transposed, O^T = V^T P, with v_mfma_f32_16x16x16: lane
//    (G, c) loads tokens 4G..4G+3 at dims [c*DPL, +DPL) of the V tile, so the
//    A operand (rows = dims, k = those four tokens) needs only an in-register
//    v_perm_b32 interleave, and the B operand (k = tokens, n = heads) is the
//    lane's own four weights from the score layout.  The output has the head
//    in the lane's column, so the online-softmax rescale multiplies by the
//    lane's own factor: no cross-lane traffic in PV.
//  * Rescaling by 2^(m_old - m_new) is unconditional (branch-free); it is
//    exactly 1 when the running max did not grow.
//  * KV tiles are loaded non-temporally: each is read once per step, and
//    streaming them past the caches raises the gather bandwidth measurably
//    (and leaves the caches to what is reused: tables, queries, partials).
//
// Unfilled slots of a final block get score -inf (weight exactly 0) and
// their V rows are replaced by the last filled row of the block (finite), so
// NaN/Inf garbage there never reaches the result.  Block ids outside
// [0, num_blocks) are never dereferenced: the result is NaN instead.
//
// Two kernels share this tile code:
//  * decode_part_wave (partitions of up to 64 blocks): one wavefront per
//    partition, four consecutive partitions per workgroup, merged in LDS into
//    one entry (the final row, or a partial for the reduce) per workgroup.
//  * decode_part_mfma (partitions of 65..256 blocks): the four wavefronts of
//    a workgroup share one partition, blocks dealt round-robin.
// Both stage each wave's (m, l) and normalised rows in LDS and write the
// workgroup's entry with the same log-sum-exp merge as the reduce kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "decode_kernels.h"
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

constexpr int kWaves = 4;
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
  // vector offset.  V rows past `rmax` (the block's last filled slot)
  // re-read that row: their weights are exactly 0 and the values are finite.
  __device__ static __forceinline__ void load(const char* kb, const char* vb, int grp, int col, int rmax,
                                              uint4 (&kr)[KS], VVec (&vr)[4]) {
    const uint32_t k_lane = col * ROWB + grp * 16;
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

// The four waves' staged results (m_w, l_w per head, normalised rows o_w;
// l_w = 0 for a wave without tokens) merged with weights l_w 2^(m_w - M), as
// the reduce kernel merges partitions, and written with 16-byte stores
// (consecutive threads on consecutive bytes): the final rows when the
// sequence has a single entry, else the entry's (o, m, l) at index `e` of `E`
// per row.  `bad` makes the entry NaN.
template <int DT, int D, int GMAX>
__device__ __forceinline__ void merge_write(const float (*sm)[16], const float (*sl)[16], const float* srow, bool bad,
                                            int nentries, int e, size_t row0, int nh, int E, void* out, float* ws_o,
                                            float* ws_m, float* ws_l) {
  const float nan = __builtin_nanf("");
  auto merged = [&](int h, int d, float* M_out, float* den_out) {
    float M = sm[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm[w][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = sl[w][h] * fast_exp2(sm[w][h] - M);  // 0 for a wave without tokens
      den += wt;
      num = fmaf(wt, sl[w][h] > 0.f ? srow[(w * GMAX + h) * D + d] : 0.f, num);
    }
    *M_out = M;
    *den_out = den;
    return num / den;
  };
  if (nentries == 1) {
    constexpr int EPC = 16 / Elem<DT>::kBytes;
    for (int c = threadIdx.x; c < nh * (D / EPC); c += 256) {
      const int h = c / (D / EPC);
      const int dd = (c - h * (D / EPC)) * EPC;
      float f[EPC];
#pragma unroll
      for (int i = 0; i < EPC; ++i) {
        float M, den;
        f[i] = bad ? nan : merged(h, dd + i, &M, &den);
      }
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(out) + ((row0 + h) * D + dd) * Elem<DT>::kBytes) =
          pack16<DT>(f);
    }
  } else {
    for (int c = threadIdx.x; c < nh * (D / 4); c += 256) {
      const int h = c / (D / 4);
      const int dd = (c - h * (D / 4)) * 4;
      float M = 0.f, den = 0.f, v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = bad ? nan : merged(h, dd + i, &M, &den);
      *reinterpret_cast<float4*>(&ws_o[((row0 + h) * E + e) * D + dd]) = make_float4(v[0], v[1], v[2], v[3]);
      if (dd == 0) {
        ws_m[(row0 + h) * E + e] = bad ? nan : M;
        ws_l[(row0 + h) * E + e] = bad ? nan : den;
      }
    }
  }
}

// The rows of a sequence with L = 0: zero (NaN for an invalid length).
template <int DT, int D>
__device__ __forceinline__ void fill_rows(void* out, size_t row0, int nh, bool bad_len) {
  const float fill = bad_len ? __builtin_nanf("") : 0.f;
  for (int i = threadIdx.x; i < nh * D; i += 256) store_elem<DT>(out, row0 * D + i, fill);
}

// The two-tile pipeline of one wave over its tiles k = 0..cnt-1 (cnt >= 1):
// issue(k, K, V) loads tile k, consume(k, K, V, valid) computes it.  Every
// issue is unconditional (indices past the end re-read the last tile, an L2
// hit), so the loads stay in a fixed order and each consume waits only for
// its own tile.  The scheduling barriers keep each tile's work and its
// prefetch in program order (left alone, the scheduler hoists the next
// tile's MFMAs above this tile's PV, so a consume waits for both buffers),
// and the compiler memory barriers keep the prologue's A before B as in the
// loop (else the wait counts, merged over both paths, make A wait for half
// of B).  The pool pointers behind `issue` must not be __restrict__: loads
// through restrict pointers may move across those barriers.
template <typename KBuf, typename VBuf, typename Issue, typename Consume>
__device__ __forceinline__ void pipeline(int cnt, KBuf& kA, VBuf& vA, KBuf& kB, VBuf& vB, Issue&& issue,
                                         Consume&& consume) {
  const int last = cnt - 1;
  __builtin_amdgcn_sched_barrier(0);
  issue(0, kA, vA);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  issue(min(1, last), kB, vB);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
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
}

// What both kernels share once a workgroup knows its (sequence, head group):
// the query tile in LDS, one wave's tile stream over `cnt` blocks (the k-th
// at logical block first + k * step, its physical id in lane k of `myid`),
// staging and the merged write of entry `e` of `nentries`.
template <int DT, int D, int GMAX>
struct Body {
  using T = Tile<DT, D>;
  static constexpr int KS = T::KS, DPL = T::DPL, ROWB = T::ROWB;
  using VVec = typename T::VVec;
  struct Shared {
    __attribute__((aligned(16))) uint16_t q[16][T::QROW];
    __attribute__((aligned(16))) float row[kWaves * GMAX * D];  // the waves' normalised rows
    float m[kWaves][16];
    float l[kWaves][16];
    int bad[kWaves];
  };

  __device__ static __forceinline__ void run(Shared& sh, const char* kp, const char* vp, int myid, bool bad, int cnt,
                                             int first, int step, int L, int kvh, int Hkv, int nh, float qscale,
                                             int nentries, int e, size_t row0, int E, void* out, float* ws_o,
                                             float* ws_m, float* ws_l) {
    const int lane = threadIdx.x & 63;
    const int wave = uni(threadIdx.x >> 6);
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int x16 = (lane ^ 16) << 2;  // ds_bpermute addresses of the partner lanes
    const int x32 = (lane ^ 32) << 2;
    const size_t blk_stride = (size_t)Hkv * 16 * ROWB;
    const size_t head_off = (size_t)kvh * 16 * ROWB;
    const uint16_t* qsrc = &sh.q[col][grp * 8];
    float m_run = kNegInf;  // running max of head `col`, base 2
    float l_run = 0.f;      // running sum over this lane's tokens
    f32x4 acc[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (cnt > 0) {
      uint4 kA[KS], kB[KS];
      VVec vA[4], vB[4];
      pipeline(
          cnt, kA, vA, kB, vB,
          [&](int k, uint4(&kr)[KS], VVec(&vr)[4]) {
            const size_t off = (size_t)__builtin_amdgcn_readlane(myid, k) * blk_stride + head_off;
            T::load(kp + off, vp + off, grp, col, min(15, L - 1 - (first + k * step) * 16), kr, vr);
          },
          [&](int k, const uint4(&kr)[KS], const VVec(&vr)[4], bool valid) {
            // a compiler memory barrier keeps the query reads here (hoisted,
            // they would hold 16 VGPRs)
            asm volatile("" ::: "memory");
            T::consume(kr, vr, qsrc, (first + k * step) * 16 + grp * 4, valid ? L : 0, qscale, x16, x32, m_run,
                       l_run, acc);
          });
    }
    T::stage(m_run, l_run, acc, cnt > 0, grp, col, nh, x16, x32, sh.m[wave], sh.l[wave], sh.row + wave * GMAX * D);
    if (lane == 0) sh.bad[wave] = bad;
    lds_barrier();
    merge_write<DT, D, GMAX>(sh.m, sh.l, sh.row, sh.bad[0] | sh.bad[1] | sh.bad[2] | sh.bad[3], nentries, e, row0, nh,
                             E, out, ws_o, ws_m, ws_l);
  }
};

// Lane k's physical id of logical block bidx(k) for k < cnt (0 elsewhere);
// ids outside [0, num_blocks) become 0, never dereferenced, and set `bad`
// (in every lane).
template <typename F>
__device__ __forceinline__ int load_ids(const int32_t* btrow, int cnt, int num_blocks, F bidx, bool& bad) {
  const int lane = threadIdx.x & 63;
  int id = 0;
  if (lane < cnt) id = btrow[bidx(lane)];
  const bool ok = id >= 0 && id < num_blocks;
  bad = !__all(lane >= cnt || ok);
  return ok ? id : 0;
}

// Where a workgroup of either kernel sits in the 1-D grid: KV head (and
// query sub-group) fastest, then sequence, then the entry rank counted from
// the end of the sequence.  Workgroups are dealt round-robin to the 8 XCDs
// by linear id, so every XCD gets an equal share of heads of every sequence;
// ranking from the end dispatches the entries far from the end first (absent
// for short sequences: those workgroups leave at once) and every sequence's
// last, shortest entry last.
struct Place {
  int s, rank, kvh, nh;
  size_t row0;
  __device__ Place(int B, int Hq, int Hkv, int g, int nsub, int E, int gmax) {
    const int hs = Hkv * nsub;
    const int idx = blockIdx.x;
    const int hsub = idx % hs;
    s = (idx / hs) % B;
    rank = E - 1 - idx / (hs * B);
    kvh = hsub / nsub;
    const int sub = hsub - kvh * nsub;
    nh = min(gmax, g - sub * gmax);
    row0 = (size_t)s * Hq + kvh * g + sub * gmax;
  }
};

// ---------------------------------------------------------------------------
// One wavefront per partition (partitions of up to 64 blocks).
//
// Entry r of a sequence holds partitions nparts-1-4r-w, w = 0..3 (counted
// from the end), one per wave.  Each wave streams its partition with its own
// running (m, l, acc); the only barriers are after the query load and at the
// end, where the four partitions are merged into the entry: the final row
// when the sequence has at most 4 partitions, else a partial that the reduce
// merges with the other entries.  One partial per 4 partitions: partial
// writes interleaved with the KV read stream cost HBM efficiency far beyond
// their size.
// ---------------------------------------------------------------------------
template <int DT, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_part_wave(void* __restrict__ out, const void* __restrict__ q,
                                                       const char* kp, const char* vp,
                                                       const int32_t* __restrict__ bt, const int32_t* __restrict__ cl,
                                                       float* __restrict__ ws_o, float* __restrict__ ws_m,
                                                       float* __restrict__ ws_l, int B, int Hq, int Hkv, int g,
                                                       int nsub, int num_blocks, int maxb, int max_ctx, float qscale,
                                                       int psize, int E) {
  using Bd = Body<DT, D, GMAX>;
  static_assert(GMAX <= 16, "one MFMA column per query head");
  __shared__ typename Bd::Shared sh;
  const Place pl(B, Hq, Hkv, g, nsub, E, GMAX);
  // The query group does not depend on the context length: its load goes
  // out first.
  const uint4 qv = Bd::T::load_q(reinterpret_cast<const char*>(q) + pl.row0 * Bd::ROWB, pl.nh, threadIdx.x);

  int L = cl[pl.s];
  const bool bad_len = L < 0 || L > max_ctx;
  if (bad_len) L = 0;
  const int nparts = (L + psize - 1) / psize;
  const int nent = (nparts + 3) / 4;
  if (L == 0) {
    if (pl.rank == 0) fill_rows<DT, D>(out, pl.row0, pl.nh, bad_len);
    return;
  }
  if (pl.rank >= nent) return;  // the whole workgroup: no partition here
  Bd::T::store_q(sh.q, qv, threadIdx.x);
  lds_barrier();  // the query tile is in LDS (every wave of the workgroup gets here)

  const int wave = uni(threadIdx.x >> 6);
  const int p = nparts - 1 - 4 * pl.rank - wave;  // < 0: this wave has no partition
  const int pblk = psize / 16;
  const int b0 = max(p, 0) * pblk;
  const int cnt = p < 0 ? 0 : min(pblk, (L + 15) / 16 - b0);
  bool bad;
  const int myid = load_ids(bt + (size_t)pl.s * maxb, cnt, num_blocks, [&](int k) { return b0 + k; }, bad);
  Bd::run(sh, kp, vp, myid, bad, cnt, b0, 1, L, pl.kvh, Hkv, pl.nh, qscale, nent, pl.rank, pl.row0, E, out, ws_o,
          ws_m, ws_l);
}

// ---------------------------------------------------------------------------
// One workgroup per partition (partitions of 65..256 blocks).
//
// The four waves share the partition, blocks dealt round-robin (wave w takes
// blocks w, w+4, ...), and merge like the waves of decode_part_wave.  Entries
// are partitions; rank 0 is the sequence's last.
// ---------------------------------------------------------------------------
template <int DT, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_part_mfma(void* __restrict__ out, const void* __restrict__ q,
                                                       const char* kp, const char* vp,
                                                       const int32_t* __restrict__ bt, const int32_t* __restrict__ cl,
                                                       float* __restrict__ ws_o, float* __restrict__ ws_m,
                                                       float* __restrict__ ws_l, int B, int Hq, int Hkv, int g,
                                                       int nsub, int num_blocks, int maxb, int max_ctx, float qscale,
                                                       int psize, int E) {
  using Bd = Body<DT, D, GMAX>;
  static_assert(GMAX <= 16, "one MFMA column per query head");
  __shared__ typename Bd::Shared sh;
  const Place pl(B, Hq, Hkv, g, nsub, E, GMAX);
  const uint4 qv = Bd::T::load_q(reinterpret_cast<const char*>(q) + pl.row0 * Bd::ROWB, pl.nh, threadIdx.x);

  int L = cl[pl.s];
  const bool bad_len = L < 0 || L > max_ctx;
  if (bad_len) L = 0;
  const int nparts = (L + psize - 1) / psize;
  if (L == 0) {
    if (pl.rank == 0) fill_rows<DT, D>(out, pl.row0, pl.nh, bad_len);
    return;
  }
  if (pl.rank >= nparts) return;
  Bd::T::store_q(sh.q, qv, threadIdx.x);
  lds_barrier();

  const int wave = uni(threadIdx.x >> 6);
  const int p = nparts - 1 - pl.rank;
  const int b0 = p * (psize / 16);
  const int nb = min(psize / 16, (L + 15) / 16 - b0);                  // blocks of the partition
  const int cnt = nb > wave ? (nb - wave + kWaves - 1) / kWaves : 0;  // this wave's (<= 64)
  bool bad;
  const int myid =
      load_ids(bt + (size_t)pl.s * maxb, cnt, num_blocks, [&](int k) { return b0 + wave + k * kWaves; }, bad);
  Bd::run(sh, kp, vp, myid, bad, cnt, b0 + wave, kWaves, L, pl.kvh, Hkv, pl.nh, qscale, nparts, p, pl.row0, E, out,
          ws_o, ws_m, ws_l);
}

template <int DT, int D, int GMAX>
void launch(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.entries * a.Hkv * a.nsub * a.B;
  if (a.wave_part)
    hipLaunchKernelGGL((decode_part_wave<DT, D, GMAX>), dim3(grid), dim3(256), 0, st, a.out, a.q, a.kp, a.vp, a.bt,
                       a.cl, a.ws_o, a.ws_m, a.ws_l, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb, a.max_ctx,
                       a.qscale, a.psize, a.entries);
  else
    hipLaunchKernelGGL((decode_part_mfma<DT, D, GMAX>), dim3(grid), dim3(256), 0, st, a.out, a.q, a.kp, a.vp, a.bt,
                       a.cl, a.ws_o, a.ws_m, a.ws_l, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb, a.max_ctx,
                       a.qscale, a.psize, a.entries);
}

template <int DT, int D>
void launch_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.gmax) {
    case 4: launch<DT, D, 4>(a, st); break;
    case 8: launch<DT, D, 8>(a, st); break;
    default: launch<DT, D, 16>(a, st); break;
  }
}

template <int DT>
void launch_d(const DecodeArgs& a, hipStream_t st) {
  if (a.D == 64)
    launch_g<DT, 64>(a, st);
  else
    launch_g<DT, 128>(a, st);
}

}  // namespace

void launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == PA_FP16)
    launch_d<PA_FP16>(a, st);
  else
    launch_d<PA_BF16>(a, st);
}

}  // namespace pa
