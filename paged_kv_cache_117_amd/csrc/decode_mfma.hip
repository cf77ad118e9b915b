// pa_decode partition kernels for 16-bit KV (fp16 / bf16) on gfx950.
//
// Same computation as the VALU kernel in decode.hip (online softmax over a
// partition's blocks in logical order, base-2 exponentials, log-sum-exp
// partials), organised for bandwidth with both products on the matrix cores.
//
// Work item = (sequence, KV head, query sub-group of up to GMAX heads,
// partition).  A workgroup of 4 wavefronts takes one item at a time: wave w
// walks the partition's blocks w, w+4, ... with two tiles (K and V of one
// block) in flight, and the four waves' (m, l, acc) are merged through LDS.
//
// Per tile (16 slots of one block, one KV head):
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
//
// Unfilled slots of a final block get score -inf (weight exactly 0) and
// their V rows are replaced by the last filled row of the block (finite), so
// NaN/Inf garbage there never reaches the result.  Block ids outside
// [0, num_blocks) are never dereferenced: the item produces NaN instead.
//
// Two kernels share this tile code:
//  * decode_persist: one workgroup per resident slot (CUs x occupancy).
//    Workgroups draw items from an atomic ticket counter in the workspace,
//    full partitions first and every sequence's shorter last partition at the
//    end (longest work first), and look two tickets ahead: while a workgroup
//    computes one item its waves already hold the next item's block ids and
//    query, and the tile pipeline runs straight into the next item's first
//    tiles.  A slot therefore never waits for a launch, a length, a table or
//    its first tiles except at the very start.  The last workgroup to find
//    the queue empty resets the counters, so they are zero between calls.
//  * decode_part_mfma: one workgroup per item in a 1-D grid (many sequences
//    or query groups larger than 8).
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

// Workgroup barrier that orders LDS only.  __syncthreads() also orders
// global memory, so a wave with stores or atomics in flight waits for them
// to complete before it can arrive; the persistent kernel exchanges
// everything through LDS and never reads its own global writes.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}


// Per-lane tile machinery of one wavefront.
template <int DT, int D, bool kPinPerms = false>
struct Tile {
  static constexpr int ROWB = D * 2;  // bytes of one token row of one head
  static constexpr int KS = D / 32;   // QK MFMA k-steps over the head dim
  static constexpr int DPL = D / 16;  // V dims per lane = PV MFMAs per tile
  static constexpr int NW = DPL / 2;  // 32-bit words per V row in this lane
  using VVec = typename std::conditional<DPL == 8, uint4, uint2>::type;

  // QK B operand: lane (G, c) holds q[head c][dims 32k + 8G .. +8]; heads
  // >= nh are zero.  `qrow0` is the first head of the group.
  __device__ static __forceinline__ void load_q(const char* qrow0, int nh, int grp, int col, uint4 (&qop)[KS]) {
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qop[k] = col < nh ? *reinterpret_cast<const uint4*>(qrow0 + (size_t)col * ROWB + grp * 16 + k * 64)
                        : make_uint4(0, 0, 0, 0);
  }

  // One (block, head) tile at `kb` / `vb`.  Offsets are unsigned 32-bit so
  // the loads take the scalar tile base plus a 32-bit vector offset.  V rows
  // past `rmax` (the block's last filled slot) re-read that row: their
  // weights are exactly 0 and the values are finite.
  __device__ static __forceinline__ void load(const char* kb, const char* vb, int grp, int col, int rmax,
                                              uint4 (&kr)[KS], VVec (&vr)[4]) {
    const uint32_t k_lane = col * ROWB + grp * 16;
    const uint32_t v_col = col * DPL * 2;
#pragma unroll
    for (int k = 0; k < KS; ++k) kr[k] = *reinterpret_cast<const uint4*>(kb + (k_lane + k * 64));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vr[i] = *reinterpret_cast<const VVec*>(vb + ((uint32_t)min(grp * 4 + i, rmax) * ROWB + v_col));
  }

  // Scores (MFMA), online-softmax update, PV (MFMA) for one tile whose first
  // slot in this lane's group is token `tok0`.  Tokens at or past `lim` get
  // score -inf.  Straight-line code: branches here make the compiler
  // duplicate the accumulator.
  __device__ static __forceinline__ void consume(const uint4 (&kr)[KS], const VVec (&vr)[4], const uint4 (&qop)[KS],
                                                 int tok0, int lim, float qscale, int x16, int x32, float& m_run,
                                                 float& l_run, f32x4 (&acc)[DPL]) {
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KS; ++k) sacc = mfma_qk<DT>(kr[k], qop[k], sacc);
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
    // v_perm_b32 gathers the same dim of two token rows into one word.  Each
    // pair of permutes stays next to its MFMA (scheduling barriers): computed
    // all at once they would hold 4*NW extra VGPRs.
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t r0 = (&vr[0].x)[w], r1 = (&vr[1].x)[w], r2 = (&vr[2].x)[w], r3 = (&vr[3].x)[w];
      acc[2 * w] = mfma_pv<DT>(__builtin_amdgcn_perm(r1, r0, 0x05040100u), __builtin_amdgcn_perm(r3, r2, 0x05040100u),
                               pb0, pb1, acc[2 * w]);
      if constexpr (kPinPerms) __builtin_amdgcn_sched_barrier(0);
      acc[2 * w + 1] = mfma_pv<DT>(__builtin_amdgcn_perm(r1, r0, 0x07060302u),
                                   __builtin_amdgcn_perm(r3, r2, 0x07060302u), pb0, pb1, acc[2 * w + 1]);
      if constexpr (kPinPerms) __builtin_amdgcn_sched_barrier(0);
    }
  }

  // This wave's share of the workgroup merge: the sum over the four token
  // groups of l, then (m, l) per head and acc[u][j] = O[head col][dim
  // DPL*(4*grp + j) + u] (unnormalised) into LDS.
  template <int SROW>
  __device__ static __forceinline__ void stage(float m_run, float l_run, const f32x4 (&acc)[DPL], int grp, int col,
                                               int nh, int x16, int x32, float* sm, float* sl, float* sacc) {
    l_run = xchg(xchg(l_run, x16, AddOp()), x32, AddOp());
    if (grp == 0) {
      sm[col] = m_run;
      sl[col] = l_run;
    }
    if (col < nh) {
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        float* dst = sacc + col * SROW + DPL * (4 * grp + jj);
#pragma unroll
        for (int u = 0; u < DPL; u += 4)
          *reinterpret_cast<float4*>(dst + u) = make_float4(acc[u][jj], acc[u + 1][jj], acc[u + 2][jj], acc[u + 3][jj]);
      }
    }
  }
};

// The workgroup merge of NWV waves' staged (m, l, acc) (weights
// 2^(m_w - M); waves without blocks have m_w = -inf) and the item's output:
// the final row when the sequence has one partition, else the partition's
// (o, m, l) partials.  L = 0 writes `fill` (0, or NaN for an invalid length).
template <int DT, int D, int GMAX, int SROW, int NWV = kWaves>
__device__ __forceinline__ void merge_store(const float (*sm)[16], const float (*sl)[16], const float* sacc,
                                            bool anybad, int L, bool bad_len, int nparts, int s, int p, int hbase,
                                            int nh, int Hq, int P, void* out, float* ws_o, float* ws_m, float* ws_l,
                                            int first, int stride) {
  const float nan = __builtin_nanf("");
  for (int idx = first; idx < nh * D; idx += stride) {
    const int h = idx / D;
    const int d = idx - h * D;
    const size_t row = (size_t)s * Hq + hbase + h;
    if (L == 0) {
      store_elem<DT>(out, row * D + d, bad_len ? nan : 0.f);
      continue;
    }
    float M = sm[0][h];
#pragma unroll
    for (int w = 1; w < NWV; ++w) M = fmaxf(M, sm[w][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float e = fast_exp2(sm[w][h] - M);
      den = fmaf(e, sl[w][h], den);
      num = fmaf(e, sacc[(w * GMAX + h) * SROW + d], num);
    }
    if (nparts == 1) {
      store_elem<DT>(out, row * D + d, anybad ? nan : num / den);
    } else {
      ws_o[(row * P + p) * D + d] = anybad ? nan : num / den;
      if (d == 0) {
        ws_m[row * P + p] = anybad ? nan : M;
        ws_l[row * P + p] = anybad ? nan : den;
      }
    }
  }
}

// Physical ids of this wave's blocks of an item, lane i holding the i-th (at
// most 64: the host sends partitions longer than 4096 positions to the VALU
// kernel).  Ids outside [0, num_blocks) become 0 and set `bad`.
__device__ __forceinline__ int load_ids(const int32_t* btrow, int b0, int wave, int cnt, int lane, int num_blocks,
                                        bool& bad) {
  int id = 0;
  if (lane < cnt) id = btrow[b0 + wave + lane * kWaves];
  const bool ok = lane >= cnt || (id >= 0 && id < num_blocks);
  bad = !__all(ok);
  return (id >= 0 && id < num_blocks) ? id : 0;
}

// ---------------------------------------------------------------------------
// One workgroup per item.
// ---------------------------------------------------------------------------
template <int DT, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_part_mfma(void* __restrict__ out, const void* __restrict__ q,
                                                       const char* __restrict__ kp, const char* __restrict__ vp,
                                                       const int32_t* __restrict__ bt, const int32_t* __restrict__ cl,
                                                       float* __restrict__ ws_o, float* __restrict__ ws_m,
                                                       float* __restrict__ ws_l, int B, int Hq, int Hkv, int g,
                                                       int nsub, int num_blocks, int maxb, int max_ctx, float qscale,
                                                       int psize, int P) {
  using T = Tile<DT, D>;
  constexpr int KS = T::KS, DPL = T::DPL, ROWB = T::ROWB;
  constexpr int SROW = D + 4;  // LDS row stride (floats) of the merge buffer
  using VVec = typename T::VVec;
  static_assert(GMAX <= 16, "one MFMA column per query head");

  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ __attribute__((aligned(16))) float s_acc[kWaves * GMAX * SROW];
  __shared__ int s_bad[kWaves];

  const int tid = threadIdx.x;
  // wave-uniform: keep it (and everything derived from it) in SGPRs
  const int wave = uni(tid >> 6);
  const int lane = tid & 63;
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int x16 = (lane ^ 16) << 2;  // ds_bpermute addresses of the partner lanes
  const int x32 = (lane ^ 32) << 2;
  // 1-D grid: KV head (and query sub-group) fastest, then sequence, then
  // partition rank counted from the end of the sequence.  Workgroups are
  // dealt round-robin to the 8 XCDs by linear id, so every XCD gets an equal
  // share of heads of every sequence; ranking partitions from the end puts
  // every sequence's partial last partition (the short work items) at the
  // end of the dispatch order and the empty ranks at the start.
  const int hs = Hkv * nsub;
  const int idx = blockIdx.x;
  const int hsub = idx % hs;
  const int s = (idx / hs) % B;
  const int rank = P - 1 - idx / (hs * B);  // 0 = the sequence's last partition
  const int kvh = hsub / nsub;
  const int sub = hsub - kvh * nsub;
  const int hbase = kvh * g + sub * GMAX;
  const int nh = min(GMAX, g - sub * GMAX);

  // The q operand does not depend on the context length: its loads go out
  // before the length arrives.
  uint4 qop[KS];
  T::load_q(reinterpret_cast<const char*>(q) + ((size_t)s * Hq + hbase) * ROWB, nh, grp, col, qop);

  int L = cl[s];
  const bool bad_len = L < 0 || L > max_ctx;
  if (bad_len) L = 0;
  const int nparts = (L + psize - 1) / psize;
  if (L == 0 ? rank != 0 : rank >= nparts) return;
  const int p = L == 0 ? 0 : nparts - 1 - rank;

  const int nblk = (L + 15) / 16;
  const int b0 = p * (psize / 16);
  const int b1 = min(b0 + psize / 16, nblk);
  const int cnt = b1 - b0 > wave ? (b1 - b0 - wave + kWaves - 1) / kWaves : 0;
  const size_t blk_stride = (size_t)Hkv * 16 * ROWB;
  const size_t head_off = (size_t)kvh * 16 * ROWB;

  float m_run = kNegInf;  // running max of head `col`, base 2
  float l_run = 0.f;      // running sum over this lane's tokens
  f32x4 acc[DPL];
#pragma unroll
  for (int u = 0; u < DPL; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  if (cnt > 0) {
    const int myid = load_ids(bt + (size_t)s * maxb, b0, wave, cnt, lane, num_blocks, bad);
    uint4 kA[KS], kB[KS];
    VVec vA[4], vB[4];
    auto issue = [&](int j, uint4(&kr)[KS], VVec(&vr)[4]) {
      const int phys = __builtin_amdgcn_readlane(myid, j);
      const int rmax = min(15, L - 1 - (b0 + wave + j * kWaves) * 16);
      T::load(kp + (size_t)phys * blk_stride + head_off, vp + (size_t)phys * blk_stride + head_off, grp, col, rmax,
              kr, vr);
    };
    auto consume = [&](int j, const uint4(&kr)[KS], const VVec(&vr)[4], bool valid) {
      T::consume(kr, vr, qop, (b0 + wave + j * kWaves) * 16 + grp * 4, valid ? L : 0, qscale, x16, x32, m_run,
                 l_run, acc);
    };
    // Two tiles in flight per wave.  Every issue is unconditional (indices
    // past the end re-read the last tile, an L2 hit) so the loads stay in a
    // fixed order and each consume waits only for its own tile.  The
    // scheduling barriers keep each tile's work and its prefetch in program
    // order: left alone, the scheduler hoists the next tile's MFMAs above
    // this tile's PV (so a consume waits for both buffers) and moves loads
    // across the PV step (longer live ranges, fewer waves per SIMD).
    const int last = cnt - 1;
    __builtin_amdgcn_sched_barrier(0);
    issue(0, kA, vA);
    __builtin_amdgcn_sched_barrier(0);
    issue(min(1, last), kB, vB);
    __builtin_amdgcn_sched_barrier(0);
    for (int j = 0; j < cnt; j += 2) {
      consume(j, kA, vA, true);
      __builtin_amdgcn_sched_barrier(0);
      issue(min(j + 2, last), kA, vA);
      __builtin_amdgcn_sched_barrier(0);
      consume(j + 1, kB, vB, j + 1 < cnt);
      __builtin_amdgcn_sched_barrier(0);
      issue(min(j + 3, last), kB, vB);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  T::template stage<SROW>(m_run, l_run, acc, grp, col, nh, x16, x32, s_m[wave], s_l[wave],
                          s_acc + wave * GMAX * SROW);
  if (lane == 0) s_bad[wave] = bad;
  __syncthreads();
  const bool anybad = s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3];
  merge_store<DT, D, GMAX, SROW>(s_m, s_l, s_acc, anybad, L, bad_len, nparts, s, p, hbase, nh, Hq, P, out, ws_o, ws_m,
                                 ws_l, tid, 256);
}

// ---------------------------------------------------------------------------
// Persistent workgroups drawing items from a ticket counter.
//
// One workgroup per CU: 8 compute waves, a store wave and a fill wave.  The
// compute waves issue no vector memory operation but the tile loads, so each
// wait on a tile is an exact count and two tiles stay in flight per wave
// across item boundaries.  The fill wave draws tickets, decodes them and
// loads each item's block ids and query group into a ring of 4 LDS slots,
// three items ahead; the compute waves merge their (m, l, acc) through LDS
// into an output buffer that the store wave writes out.  Each helper waits
// only on its own memory operations.
//
// Barriers, in the order every wave passes them: S (setup), then for each
// item i: Y(i-1) (item i-1 written out: staging and output buffers free),
// X(i) (item i staged), Z(i) (item i merged).  Compute waves: tiles of i,
// Y(i-1), stage, X(i), merge, Z(i).  Store wave: X(i), Z(i), write item i,
// Y(i).  Fill wave: X(i), Z(i), fill slot i+3, Y(i).  Slot i+3 reuses the
// slot of item i-1, which nobody reads after Y(i-1).
// ---------------------------------------------------------------------------

constexpr int kSlots = 4;
constexpr int kMaxPartBlocks = 256;  // partitions of up to 4096 positions
constexpr int kPW = 8;               // compute waves of a persistent workgroup
constexpr int kStoreWave = kPW;
constexpr int kFillWave = kPW + 1;
static_assert(kPersistThreads == (kPW + 2) * 64, "8 compute waves + store wave + fill wave");

// LDS slot descriptor fields.
enum : int { kValid, kSeq, kPart, kKvh, kHbase, kNh, kLen, kBadLen, kNparts, kB0, kNblk, kBad, kDescInts };

template <int DT, int D, int GMAX>
__global__ __launch_bounds__(kPersistThreads) void decode_persist(
    void* __restrict__ out, const void* __restrict__ q, const char* __restrict__ kp, const char* __restrict__ vp,
    const int32_t* __restrict__ bt, const int32_t* __restrict__ cl, float* __restrict__ ws_o,
    float* __restrict__ ws_m, float* __restrict__ ws_l, uint32_t* __restrict__ ctr, int B, int Hq, int Hkv, int g,
    int nsub, int num_blocks, int maxb, int max_ctx, float qscale, int psize, int P) {
  using T = Tile<DT, D, true>;
  constexpr int KS = T::KS, DPL = T::DPL, ROWB = T::ROWB;
  constexpr int SROW = D + 4;  // LDS row stride (floats) of the staging buffer
  constexpr int QROW = D + 8;  // LDS row stride (elements) of a query tile: conflict-free operand reads
  using VVec = typename T::VVec;
  static_assert(GMAX <= 16, "one MFMA column per query head");

  __shared__ int s_len[kPersistMaxSeqs];       // lengths, -1 for an invalid one
  __shared__ int s_fcum[kPersistMaxSeqs + 1];  // full partitions of sequences < s
  __shared__ int s_pcum[kPersistMaxSeqs + 1];  // last partial (or empty) partitions of sequences < s
  __shared__ int s_desc[kSlots][kDescInts];
  __shared__ int s_ids[kSlots][kMaxPartBlocks];
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kSlots][16][QROW];
  __shared__ float s_m[kPW][16];
  __shared__ float s_l[kPW][16];
  __shared__ __attribute__((aligned(16))) float s_acc[kPW * GMAX * SROW];
  __shared__ __attribute__((aligned(16))) float s_out[GMAX][D];  // merged item: normalised rows
  __shared__ float s_outm[GMAX];    // its running max and sum per head
  __shared__ float s_outl[GMAX];

  const int tid = threadIdx.x;
  const int wave = uni(tid >> 6);
  const int lane = tid & 63;
  const int hs = Hkv * nsub;
  const int pblk = psize / 16;

  if (wave == kStoreWave) {
    // ======================= store wave =======================
    // 16-byte stores: a row of the output (EPC elements) or of the fp32
    // partials (4 floats) per lane and instruction.
    constexpr int EPC = 16 / Elem<DT>::kBytes;
    const float nan = __builtin_nanf("");
    lds_barrier();  // S
    lds_barrier();  // Y(-1)
    if (!uni(s_desc[0][kValid])) return;
    for (int it = 0;; ++it) {
      lds_barrier();  // X(it)
      lds_barrier();  // Z(it)
      const int* d = s_desc[it & 3];
      const int s = uni(d[kSeq]), p = uni(d[kPart]), hbase = uni(d[kHbase]), nh = uni(d[kNh]);
      const int L = uni(d[kLen]), nparts = uni(d[kNparts]);
      const bool bad_len = uni(d[kBadLen]) != 0, anybad = uni(d[kBad]) != 0;
      const size_t row0 = (size_t)s * Hq + hbase;
      if (L == 0 || nparts == 1) {
        const float fill = L == 0 ? (bad_len ? nan : 0.f) : nan;
        const bool use_fill = L == 0 || anybad;
        for (int c = lane; c < nh * (D / EPC); c += 64) {
          const int h = c / (D / EPC);
          const int dd = (c - h * (D / EPC)) * EPC;
          float f[EPC];
#pragma unroll
          for (int e = 0; e < EPC; ++e) f[e] = use_fill ? fill : s_out[h][dd + e];
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(out) + ((row0 + h) * D + dd) * Elem<DT>::kBytes) =
              pack16<DT>(f);
        }
      } else {
        for (int c = lane; c < nh * (D / 4); c += 64) {
          const int h = c / (D / 4);
          const int dd = (c - h * (D / 4)) * 4;
          float4 v = *reinterpret_cast<const float4*>(&s_out[h][dd]);
          if (anybad) v = make_float4(nan, nan, nan, nan);
          *reinterpret_cast<float4*>(&ws_o[((row0 + h) * P + p) * D + dd]) = v;
        }
        if (lane < nh) {
          ws_m[(row0 + lane) * P + p] = anybad ? nan : s_outm[lane];
          ws_l[(row0 + lane) * P + p] = anybad ? nan : s_outl[lane];
        }
      }
      const bool more = uni(s_desc[(it + 1) & 3][kValid]) != 0;
      lds_barrier();  // Y(it)
      if (!more) return;
    }
  }

  if (wave == kFillWave) {
    // ======================= fill wave =======================
    // Tickets: lane 0 draws; the k-th drawn ticket is this workgroup's item k.
    uint32_t tk[5] = {0, 0, 0, 0, 0};
    if (lane == 0)
      for (int k = 0; k < 5; ++k) tk[k] = atomicAdd(&ctr[0], 1u);

    // Lengths -> items per sequence -> exclusive prefix sums.  The queue
    // holds every full partition (sequence-major), then every sequence's
    // partial or empty last partition; ticket t is item t / hs, KV head and
    // query sub-group t % hs.  All lengths arrive in one round trip
    // (lane-strided), then each lane scans a contiguous chunk.
    constexpr int kLenPerLane = kPersistMaxSeqs / 64;
    int lens[kLenPerLane];
#pragma unroll
    for (int k = 0; k < kLenPerLane; ++k) lens[k] = lane + 64 * k < B ? cl[lane + 64 * k] : 0;
#pragma unroll
    for (int k = 0; k < kLenPerLane; ++k)
      if (lane + 64 * k < B) s_len[lane + 64 * k] = (lens[k] < 0 || lens[k] > max_ctx) ? -1 : lens[k];
    const int chunk = (B + 63) / 64;
    const int sbeg = min(lane * chunk, B), send = min(sbeg + chunk, B);
    int nf = 0, np = 0;
    for (int s = sbeg; s < send; ++s) {
      const int Lc = max(s_len[s], 0);
      nf += Lc / psize;
      np += (Lc % psize != 0 || Lc == 0) ? 1 : 0;
    }
    int xf = nf, xp = np;  // inclusive scan over the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int yf = __shfl_up(xf, off), yp = __shfl_up(xp, off);
      if (lane >= off) {
        xf += yf;
        xp += yp;
      }
    }
    {
      int cf = xf - nf, cp = xp - np;
      for (int s = sbeg; s < send; ++s) {
        s_fcum[s] = cf;
        s_pcum[s] = cp;
        const int Lc = max(s_len[s], 0);
        cf += Lc / psize;
        cp += (Lc % psize != 0 || Lc == 0) ? 1 : 0;
      }
    }
    const int F = __shfl(xf, 63), R = __shfl(xp, 63);
    const uint32_t ntk = (uint32_t)(F + R) * (uint32_t)hs;

    // Lane 0: a ticket past the end has been drawn.  Each workgroup draws
    // past the end once, then takes no more tickets; the last one to do so
    // (all others have stopped drawing) resets both counters.
    bool exhausted = false;
    auto take = [&](uint32_t t) -> int {  // lane 0: drawn ticket -> item ticket or -1
      if (t < ntk) return (int)t;
      if (!exhausted) {
        exhausted = true;
        if (atomicAdd(&ctr[1], 1u) == gridDim.x - 1) {
          atomicExch(&ctr[0], 0u);
          atomicExch(&ctr[1], 0u);
        }
      }
      return -1;
    };
    int item_tk[5] = {-1, -1, -1, -1, -1};
    if (lane == 0) {
      // all five values are in hand before any finish, so no draw of this
      // workgroup can land after a reset
      for (int k = 0; k < 5; ++k) item_tk[k] = tk[k] < ntk ? (int)tk[k] : -1;
      if (item_tk[4] < 0) take(ntk);
    }
    auto find = [&](const int* cum, int i) {
      int lo = 0, hi = B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (uni(cum[mid]) <= i)
          lo = mid;
        else
          hi = mid;
      }
      return lo;
    };

    // A slot is filled in two steps: prepare decodes the ticket and issues
    // the loads of the item's block ids and query group into registers;
    // commit (one round later, the data long arrived) sanitises the ids (an
    // id outside [0, num_blocks) becomes 0 and marks the item bad) and
    // writes descriptor, ids and query (heads >= nh zero) to the slot.
    constexpr int QCH = D / 8;                      // 16-byte chunks per query row
    constexpr int QPL = 16 * QCH / 64;              // query chunks per lane
    constexpr int IPL = kMaxPartBlocks / 64;        // block ids per lane
    struct Staged {
      int valid, s, p, kvh, hbase, nh, Lc, bad_len, b0, nb;
      int ids[IPL];
      uint4 qv[QPL];
    };
    auto prepare = [&](int t) {
      Staged st{};
      t = __shfl(t, 0);
      if (t < 0) return st;
      st.valid = 1;
      const int i = t / hs;
      const int hsub = t - i * hs;
      int L;
      if (i < F) {
        st.s = find(s_fcum, i);
        st.p = i - uni(s_fcum[st.s]);
        L = uni(s_len[st.s]);
      } else {
        st.s = find(s_pcum, i - F);
        L = uni(s_len[st.s]);
        st.p = max(L, 0) / psize;
      }
      st.Lc = max(L, 0);
      st.bad_len = L < 0;
      st.kvh = hsub / nsub;
      const int sub = hsub - st.kvh * nsub;
      st.hbase = st.kvh * g + sub * GMAX;
      st.nh = min(GMAX, g - sub * GMAX);
      const int nblk = (st.Lc + 15) / 16;
      st.b0 = st.p * pblk;
      st.nb = max(min(st.b0 + pblk, nblk) - st.b0, 0);
      const int32_t* row = bt + (size_t)st.s * maxb + st.b0;
#pragma unroll
      for (int k = 0; k < IPL; ++k) st.ids[k] = lane + 64 * k < st.nb ? row[lane + 64 * k] : 0;
      const char* qg = reinterpret_cast<const char*>(q) + ((size_t)st.s * Hq + st.hbase) * ROWB;
#pragma unroll
      for (int k = 0; k < QPL; ++k) {
        const int c = lane + 64 * k, h = c / QCH, ch = c - h * QCH;
        st.qv[k] = h < st.nh ? *reinterpret_cast<const uint4*>(qg + (size_t)h * ROWB + ch * 16) : make_uint4(0, 0, 0, 0);
      }
      return st;
    };
    auto commit = [&](int slot, const Staged& st) {
      int* d = s_desc[slot];
      if (!st.valid) {
        if (lane == 0) d[kValid] = 0;
        return;
      }
      bool bad = false;
#pragma unroll
      for (int k = 0; k < IPL; ++k) {
        if (lane + 64 * k < st.nb) {
          int id = st.ids[k];
          if (id < 0 || id >= num_blocks) {
            bad = true;
            id = 0;
          }
          s_ids[slot][lane + 64 * k] = id;
        }
      }
      const bool anybad = __any(bad);
#pragma unroll
      for (int k = 0; k < QPL; ++k) {
        const int c = lane + 64 * k, h = c / QCH, ch = c - h * QCH;
        *reinterpret_cast<uint4*>(&s_q[slot][h][ch * 8]) = st.qv[k];
      }
      if (lane == 0) {
        d[kValid] = 1;
        d[kSeq] = st.s;
        d[kPart] = st.p;
        d[kKvh] = st.kvh;
        d[kHbase] = st.hbase;
        d[kNh] = st.nh;
        d[kLen] = st.Lc;
        d[kBadLen] = st.bad_len;
        d[kNparts] = (st.Lc + psize - 1) / psize;
        d[kB0] = st.b0;
        d[kNblk] = st.nb;
        d[kBad] = anybad;
      }
    };

    commit(0, prepare(item_tk[0]));
    commit(1, prepare(item_tk[1]));
    lds_barrier();  // S
    commit(2, prepare(item_tk[2]));
    Staged staged = prepare(item_tk[3]);
    // Lane 0: t_next is the (checked) ticket of the next slot to prepare, -1
    // once the queue is exhausted; t_pend a draw not yet checked.  A slot
    // gets -1 only after exhaustion, when no draw is outstanding, and tickets
    // are used in draw order, so no drawn item is lost.
    int t_next = item_tk[4];
    uint32_t t_pend = 0;
    bool pend = false;
    if (lane == 0) {
      pend = !exhausted;
      if (pend) t_pend = atomicAdd(&ctr[0], 1u);
    }
    lds_barrier();  // Y(-1)
    if (!uni(s_desc[0][kValid])) return;
    for (int it = 0;; ++it) {
      lds_barrier();  // X(it)
      lds_barrier();  // Z(it)
      const bool more = uni(s_desc[(it + 1) & 3][kValid]) != 0;
      if (more) {
        commit((it + 3) & 3, staged);
        staged = prepare(t_next);
        if (lane == 0) {
          t_next = pend ? take(t_pend) : -1;
          pend = !exhausted;
          if (pend) t_pend = atomicAdd(&ctr[0], 1u);
        }
      }
      lds_barrier();  // Y(it)
      if (!more) return;
    }
  }

  // ======================= compute waves =======================
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int x16 = (lane ^ 16) << 2;
  const int x32 = (lane ^ 32) << 2;
  const size_t blk_stride = (size_t)Hkv * 16 * ROWB;

  lds_barrier();  // S
  struct Cur {
    int slot, valid, L, b0, kvh, cnt, cnt2;
  };
  auto read_item = [&](int slot) {
    const int* d = s_desc[slot];
    Cur c{};
    c.slot = slot;
    c.valid = uni(d[kValid]);
    if (!c.valid) return c;
    c.L = uni(d[kLen]);
    c.b0 = uni(d[kB0]);
    c.kvh = uni(d[kKvh]);
    const int nb = uni(d[kNblk]);
    c.cnt = nb > wave ? (nb - wave + kPW - 1) / kPW : 0;
    c.cnt2 = (c.cnt + 1) & ~1;
    return c;
  };
  // lane i: physical id of this wave's i-th block of the item in `slot`
  auto read_ids = [&](const Cur& c) { return lane < c.cnt ? s_ids[c.slot][wave + lane * kPW] : 0; };

  Cur cur = read_item(0);
  if (!cur.valid) {
    lds_barrier();  // Y(-1)
    return;
  }
  Cur nxt = read_item(1);
  int id_cur = read_ids(cur);
  int id_nxt = read_ids(nxt);

  uint4 kA[KS], kB[KS];
  VVec vA[4], vB[4];
  // Tile k of this wave's stream: tiles 0..cnt2-1 of the current item (the
  // padding tile of an odd count re-reads the last one), then the next
  // item's tiles.  When neither item has a tile there, block 0 of the pool
  // is read (in bounds, never consumed).
  auto issue = [&](int k, uint4(&kr)[KS], VVec(&vr)[4]) {
    const bool use_n = k >= cur.cnt2;
    const int cnt = use_n ? nxt.cnt : cur.cnt;
    const int j = min(use_n ? k - cur.cnt2 : k, max(cnt - 1, 0));
    const int phys = __builtin_amdgcn_readlane(use_n ? id_nxt : id_cur, j);
    const int L = use_n ? nxt.L : cur.L;
    const int b0 = use_n ? nxt.b0 : cur.b0;
    const size_t off = (size_t)phys * blk_stride + (size_t)(use_n ? nxt.kvh : cur.kvh) * 16 * ROWB;
    const int rmax = max(0, min(15, L - 1 - (b0 + wave + j * kPW) * 16));
    T::load(kp + off, vp + off, grp, col, rmax, kr, vr);
  };

  for (int it = 0;; ++it) {
    // QK B operand rows of this item's query group (LDS, read per tile)
    const uint16_t* qsrc = &s_q[cur.slot][col][grp * 8];
    float m_run = kNegInf, l_run = 0.f;
    f32x4 acc[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The first item's tiles, or (a wave with no block in this item) the
    // next item's first tiles: otherwise the previous item's tail issued them.
    if (it == 0 || cur.cnt2 == 0) {
      __builtin_amdgcn_sched_barrier(0);
      issue(0, kA, vA);
      __builtin_amdgcn_sched_barrier(0);
      issue(1, kB, vB);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int j = 0; j < cur.cnt2; j += 2) {
      const int tok = (cur.b0 + wave + j * kPW) * 16 + grp * 4;
      uint4 qop[KS];
#pragma unroll
      for (int k = 0; k < KS; ++k) qop[k] = *reinterpret_cast<const uint4*>(qsrc + k * 32);
      T::consume(kA, vA, qop, tok, cur.L, qscale, x16, x32, m_run, l_run, acc);
      __builtin_amdgcn_sched_barrier(0);
      issue(j + 2, kA, vA);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < KS; ++k) qop[k] = *reinterpret_cast<const uint4*>(qsrc + k * 32);
      T::consume(kB, vB, qop, tok + 16 * kPW, j + 1 < cur.cnt ? cur.L : 0, qscale, x16, x32, m_run, l_run, acc);
      __builtin_amdgcn_sched_barrier(0);
      issue(j + 3, kB, vB);
      __builtin_amdgcn_sched_barrier(0);
    }
    lds_barrier();  // Y(it-1): the previous item is written out
    T::template stage<SROW>(m_run, l_run, acc, grp, col, GMAX, x16, x32, s_m[wave], s_l[wave],
                            s_acc + wave * GMAX * SROW);
    lds_barrier();  // X(it)
    // Merge the 8 waves (weights 2^(m_w - M); waves without blocks have
    // m_w = -inf) into the output buffer, all compute threads in parallel.
    {
      const int nh = uni(s_desc[cur.slot][kNh]);
      for (int idx = tid; idx < nh * D; idx += kPW * 64) {
        const int h = idx / D;
        const int dd = idx - h * D;
        float M = s_m[0][h];
#pragma unroll
        for (int w = 1; w < kPW; ++w) M = fmaxf(M, s_m[w][h]);
        float den = 0.f, num = 0.f;
#pragma unroll
        for (int w = 0; w < kPW; ++w) {
          const float e = fast_exp2(s_m[w][h] - M);
          den = fmaf(e, s_l[w][h], den);
          num = fmaf(e, s_acc[(w * GMAX + h) * SROW + dd], num);
        }
        s_out[h][dd] = num / den;
        if (dd == 0) {
          s_outm[h] = M;
          s_outl[h] = den;
        }
      }
    }
    lds_barrier();  // Z(it)
    if (!nxt.valid) {
      lds_barrier();  // Y(it)
      return;
    }
    cur = nxt;
    id_cur = id_nxt;
    nxt = read_item((it + 2) & 3);
    id_nxt = read_ids(nxt);
  }
}

template <int DT, int D, int GMAX>
void launch(const DecodeArgs& a, hipStream_t st) {
  bool persist = false;
  if constexpr (GMAX <= 8) persist = a.persist_grid > 0;
  if (persist) {
    hipLaunchKernelGGL((decode_persist<DT, D, (GMAX <= 8 ? GMAX : 8)>), dim3(a.persist_grid), dim3(kPersistThreads), 0, st, a.out, a.q, a.kp, a.vp,
                       a.bt, a.cl, a.ws_o, a.ws_m, a.ws_l, a.ctr, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb,
                       a.max_ctx, a.qscale, a.psize, a.P);
  } else {
    const unsigned grid = (unsigned)a.P * a.Hkv * a.nsub * a.B;
    hipLaunchKernelGGL((decode_part_mfma<DT, D, GMAX>), dim3(grid), dim3(256), 0, st, a.out, a.q, a.kp, a.vp, a.bt,
                       a.cl, a.ws_o, a.ws_m, a.ws_l, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb, a.max_ctx,
                       a.qscale, a.psize, a.P);
  }
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

template <int DT, int D>
const void* persist_fn(int gmax) {
  if (gmax == 4) return reinterpret_cast<const void*>(&decode_persist<DT, D, 4>);
  return reinterpret_cast<const void*>(&decode_persist<DT, D, 8>);
}

}  // namespace

const void* decode_persist_kernel(pa_dtype_t dtype, int head_dim, int gmax) {
  if (gmax != 4 && gmax != 8) return nullptr;
  if (dtype == PA_FP16) return head_dim == 64 ? persist_fn<PA_FP16, 64>(gmax) : persist_fn<PA_FP16, 128>(gmax);
  return head_dim == 64 ? persist_fn<PA_BF16, 64>(gmax) : persist_fn<PA_BF16, 128>(gmax);
}

void launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == PA_FP16)
    launch_d<PA_FP16>(a, st);
  else
    launch_d<PA_BF16>(a, st);
  if (a.P > 1) launch_decode_reduce(a, st);
}

}  // namespace pa
