// pa_prefill kernels: paged attention for several new tokens per sequence
// (a prefill chunk, or the continuation after a prefix-cache hit), causal
// inside the paged context, for 16-bit KV on gfx950.
//
// Sequence s has L cached positions of which the last T are this step's
// tokens; new token i sits at position p = L - T + i and attends to
// positions 0..p.  Query rows are numbered token-major within a KV head's
// group, rho = i * g + h (h = query head within the group), so one pass over
// a K/V tile serves every query head that shares it.
//
// One workgroup of W wavefronts (4, or 8 when the batch brings at least 256
// query rows per (sequence, KV head)) takes one (sequence, KV head, tile of
// R = 32 W rows); each wave owns 32 rows as two matrix column groups of 16.
// The workgroup walks the positions 0..(largest p of its rows) in steps of
// 64, each computed as two passes of 32:
//  * K and V of the step go from the pool straight into one of two LDS
//    buffers (global->LDS 16-byte loads, 16-byte chunks XOR-swizzled on the
//    load side so the operand reads below are free of bank conflicts); the
//    next step's loads are in flight while the current one computes.
//  * Scores S^T = K Q^T with v_mfma_f32_16x16x32: the K rows (A operand,
//    lane (G, c) reads token c at dims 32k + 8G) come from LDS, the query
//    rows (B operand) sit in registers for the whole walk.  Lane (G, c) gets
//    S[token 4G + j][row c] for each 16-token half of the pass.
//  * Online softmax per row in base 2.  The running max is kept in raw score
//    units, so each weight is one fma and one exp2: p = 2^(s*qs - m*qs),
//    qs = |scale| * log2(e) (a negative scale flips the query's sign bits,
//    which is exact).  Only passes that cross a row's causal limit apply the
//    mask.
//  * PV transposed, O^T = V^T P^T, again with v_mfma_f32_16x16x32: lane
//    group G's eight k-slots are tokens 4G..4G+3 of the first half and of
//    the second half, which are exactly the eight weights the lane holds
//    from the score layout.  The V^T operand comes from the transposing LDS
//    read (two per output tile, shared by the wave's column groups), so
//    output tile u holds dims 16u..16u+15.  The output keeps the query row
//    in the lane's column, so the rescale by 2^(m_old - m_new) is
//    lane-local.
// A register-staged variant (K/V through registers, V staged transposed in
// LDS) is kept for comparison; it computes the same rows within rounding.
//
// Positions past L-1 inside the last step re-read position L-1 (finite;
// masked).  Block ids outside [0, num_blocks) are never dereferenced: the
// workgroup's rows become NaN.  A sequence whose (T, L) cannot be served
// (T > L, L past the table, T past max_query_len, bad row range) gets NaN
// rows instead of a computed result.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "decode_tile.h"
#include "pa_device.h"
#include "prefill_kernels.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;                 // wavefronts per workgroup (the 8-wavefront instance: kWideWaves)
constexpr int kPair = 32;                 // positions per compute pass: two 16-slot halves
constexpr int kPairs = 2;                 // passes per step (one barrier, one load batch)
constexpr int kStep = kPair * kPairs;     // positions per step
static_assert(kStep == kPrefillStep, "partitions are whole steps");

template <int DT>
__device__ __forceinline__ f32x4 mfma32(const uint4& a, const uint4& b, const f32x4& c) {
  if constexpr (DT == PA_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 weights rounded (nearest even) to the KV type, `a` in the low half.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (DT == PA_BF16) {
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    const f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
}

// Max of x over lanes l, l ^ 16, l ^ 32 and l ^ 48: the four token groups
// of the MFMA output layout.
__device__ __forceinline__ float max_groups(float x, int x16, int x32) {
  x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x16, __builtin_bit_cast(int, x))));
  return fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(x32, __builtin_bit_cast(int, x))));
}

// Longest walk first within each XCD.  Every workgroup of one (sequence,
// KV head) item runs on the same XCD (shared L2), but the workgroups of an
// item walk very different numbers of positions (row tile t of a chunk
// after `base` cached positions walks up to base + its last token), and
// an order by tile index alone leaves a long tail on the XCDs whose last
// workgroups are long ones.  So, for unsplit launches, workgroup rank k of
// an XCD (its k-th workgroup in dispatch order) takes the k-th longest walk
// of that XCD's items (ties: item, then tile, ascending).  A workgroup's
// walk length is its step count (base + last row's token) / kStep + 1, and
// within an item it does not decrease with the tile, so the number of an
// item's tiles with at least v steps has a closed form; one wavefront
// finds the k-th longest by a binary search over v on the sums of those
// counts (every wavefront of the workgroup computes the same pick).
// Unservable items take one workgroup each, ranked last, at the tile that
// writes their NaN rows.
// (kLptPerLane items per lane: the in-kernel order covers up to 256 items per XCD)

// Sequence s's query rows [q0, q1): query_start's entries, or (kRows, the
// decode layout, no query_start) one row per sequence, row s.  A template
// argument, so that the prefill instances compile exactly as without it.
template <bool kRows>
__device__ __forceinline__ void seq_range(const PrefillArgs& a, int s, int& q0, int& q1) {
  if constexpr (kRows) {
    q0 = s;
    q1 = s + 1;
  } else {
    q0 = a.qs[s];
    q1 = a.qs[s + 1];
  }
}

struct LptItem {
  int ntiles = 0;  // row tiles of a servable item
  int base = 0;    // cached positions before the chunk
  int rows = 0;    // chunk tokens x heads per KV head
  int tmax = 0;    // last chunk token, (rows - 1) / g
  int q0 = 0, q1 = 0, L = 0;  // the sequence's query range and length, as read
  bool used = false;
  bool ok = false;  // servable
};

// Inclusive scans over the wavefront's 64 lanes with DPP (row shifts by 1,
// 2, 4, 8 inside each row of 16 lanes, lanes before the row start taking 0,
// then row 0's last lane into row 1 and row 2's into row 3, then row 1's
// last lane into rows 2 and 3): six VALU steps, where each step of a lane
// shuffle is a round trip through the LDS crossbar.  The pick below runs
// about ten wave-wide sums per workgroup before any of its loads can go
// out, so their latency is part of every workgroup's start.  Max takes
// values >= 0 (0 stands for the missing lanes).
__device__ __forceinline__ int wave_scan_add(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}
__device__ __forceinline__ int wave_scan_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false));
  return x;
}
__device__ __forceinline__ int wave_sum(int x) { return __builtin_amdgcn_readlane(wave_scan_add(x), 63); }

// Tiles of the item walking at least v >= 1 steps (v at most one past the
// item's longest walk, so (v - 1) * kStep stays within the context length
// plus a step).  need = (v - 1) kStep - base is the chunk token the walk
// must reach: none of the item's tiles when need > tmax, else those whose
// last row (t + 1) R - 1 reaches row need * g (all when need <= 0).  An
// unservable item (base = tmax = ntiles = 0) counts one tile at v = 1.
// Straight-line selects (the clamp keeps need * g <= rows - 1): the search
// evaluates this for four items per lane about ten times per workgroup.
__device__ __forceinline__ int lpt_count(const LptItem& it, int v, int R, int g) {
  const int need = (v - 1) * kStep - it.base;
  const int tiles = it.ntiles - min(max(need, 0), it.tmax) * g / R;
  return !it.used || need > it.tmax ? 0 : (it.ok ? tiles : 1);
}

// Rank k of XCD xcd -> (item, tile) and the item's sequence's query_start
// entries and length as read here; false past the XCD's last workgroup.
__device__ bool lpt_pick(const PrefillArgs& a, int xcd, int k, int per_xcd, int R, bool rows, int& item_out,
                         int& tile_out, int& q0_out, int& q1_out, int& L_out) {
  const int lane = (int)threadIdx.x & 63;
  const int items = a.B * a.Hkv;
  const int c = (per_xcd + 63) >> 6;  // items per lane, lane-major
  LptItem it[kLptPerLane];
  int vmax = 0;
#pragma unroll
  for (int e = 0; e < kLptPerLane; ++e) {
    const int j = lane * c + e;
    if (e >= c || j >= per_xcd) continue;
    const int item = j * 8 + xcd;
    if (item >= items) continue;
    const int s = item / a.Hkv;
    const int q0 = rows ? s : a.qs[s], q1 = rows ? s + 1 : a.qs[s + 1], L = a.cl[s];
    const int T = q1 - q0;
    it[e].q0 = q0;
    it[e].q1 = q1;
    it[e].L = L;
    it[e].used = true;
    it[e].ok = !(q0 < 0 || q1 < q0 || q1 > a.N || T > L || (int64_t)L > ((int64_t)a.maxb << a.lbs) || T > a.max_q);
    if (it[e].ok) {
      it[e].rows = T * a.g;
      it[e].tmax = (it[e].rows - 1) / a.g;
      it[e].base = L - T;
      it[e].ntiles = (it[e].rows + R - 1) / R;
      if (it[e].ntiles > 0) vmax = max(vmax, (L - 1) / kStep + 1);
    } else {
      vmax = max(vmax, 1);
    }
  }
  vmax = __builtin_amdgcn_readlane(wave_scan_max(vmax), 63);
  auto count = [&](int v) {
    int n = 0;
#pragma unroll
    for (int e = 0; e < kLptPerLane; ++e) n += lpt_count(it[e], v, R, a.g);
    return wave_sum(n);
  };
  if (vmax < 1 || k >= count(1)) return false;
  int lo = 1, hi = vmax;  // count(lo) > k >= count(hi + 1)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (count(mid) > k)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int r = k - count(lo + 1);  // rank among the walks of exactly lo steps
  int cnt[kLptPerLane], mine = 0;
#pragma unroll
  for (int e = 0; e < kLptPerLane; ++e) {
    cnt[e] = lpt_count(it[e], lo, R, a.g) - lpt_count(it[e], lo + 1, R, a.g);
    mine += cnt[e];
  }
  const int incl = wave_scan_add(mine);
  const int excl = incl - mine;
  const bool here = excl <= r && r < incl;
  const int src = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(here));
  int pick_item = 0, pick_tile = 0, pq0 = 0, pq1 = 0, pL = 0;
  if (here) {
    int rr = r - excl;
#pragma unroll
    for (int e = 0; e < kLptPerLane; ++e) {
      if (rr >= 0 && rr < cnt[e]) {
        pick_item = (lane * c + e) * 8 + xcd;
        pick_tile = it[e].ok ? it[e].ntiles - lpt_count(it[e], lo, R, a.g) + rr : a.tiles - 1;
        pq0 = it[e].q0;
        pq1 = it[e].q1;
        pL = it[e].L;
      }
      rr -= cnt[e];
    }
  }
  item_out = __builtin_amdgcn_readlane(pick_item, src);
  tile_out = __builtin_amdgcn_readlane(pick_tile, src);
  q0_out = __builtin_amdgcn_readlane(pq0, src);
  q1_out = __builtin_amdgcn_readlane(pq1, src);
  L_out = __builtin_amdgcn_readlane(pL, src);
  return true;
}

// NaN (kZero: zero) into every element of query heads [h0, h0 + nh) of rows [r0, r1).
template <int DT, bool kZero = false>
__device__ void nan_rows(void* out, int r0, int r1, int Hq, int h0, int nh, int D) {
  const float nan = kZero ? 0.f : __builtin_nanf("");
  const int per_row = nh * D;
  for (long i = threadIdx.x; i < (long)(r1 - r0) * per_row; i += blockDim.x) {
    const int r = r0 + (int)(i / per_row);
    const int e = (int)(i % per_row);
    store_elem<DT>(out, ((size_t)r * Hq + h0) * D + e, nan);
  }
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// gfx950 transposing LDS read: within each group of 16 lanes, lane l receives
// element l % 4 of the 8-byte reads of lanes 4k + l / 4, k = 0..3 (lane
// layout measured on MI355X).  The four lanes 4k..4k+3 reading dims 4q..4q+3
// of token k therefore give lane l dim l of tokens 0..3.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4s*)(__attribute__((address_space(3))) const void*)p);
  return __builtin_bit_cast(uint2, r);
}

// One 16-byte global->LDS load per lane: lane i's 16 bytes at base + off_i
// (`base` wave-uniform, in scalar registers; off_i a per-lane byte offset
// below 2^31) go to LDS byte lds + 16 i (`lds` wave-uniform).  Issued as
// inline assembly on purpose: the compiler's wait-count pass treats a
// pending global->LDS load as a possible write to any LDS byte and makes
// every later LDS read wait for it, which would serialise the next step's
// loads with this step's reads of the other buffer; here the caller waits
// for the loads itself (s_waitcnt vmcnt(0) before the barrier that ends the
// step).  M0 is a reserved register, hence the compiler's warning about
// clobbering it; these kernels use M0 for nothing else (their assembly holds
// no other M0 write or read), and the statement sets it before its one use.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop

// Decode-shaped items: a (sequence, KV head) whose rows fit one matrix
// column group (T * g <= 16 -- single tokens of a mixed step, or a few) on
// blocks of at least 16 slots.  Through the 64-position LDS steps such an
// item keeps one step of K/V in flight per workgroup and computes 16 rows
// per pass for its few real ones; here it runs like the decode kernels
// instead: the first four wavefronts deal the partition's 16-slot tiles
// round-robin (wave w takes tiles w, w + 4, ...), each loading K and V
// straight into its matrix operands with two tiles in flight (the Tile
// machinery of the decode path): 64 KiB of K/V in flight per workgroup
// (4 wavefronts x 2 tiles x 8 KiB at D = 128) against the LDS path's one
// 32 KiB step.  Row rho = i g + h (token i, query head h) is the matrix column
// of lane c = rho; each lane masks past its own row's causal limit.  The
// running maxima start at -FLT_MAX (finite): a wave whose first tiles lie
// wholly past a row's limit then keeps that row's weights at exactly 0
// instead of forming -inf - -inf.  The waves' (m, l, normalised rows) are
// merged in LDS with weights l 2^(m - M) and written as the rows (one
// partition) or as the partition's partials, in the main path's format.
//   sq    LDS, 16 x (D + 8) 16-bit: the query tile, followed by the waves'
//         m and l and their invalid-block flags
//   srow  LDS, 4 x 16 x D floats: the waves' normalised rows
template <int DT, int D, int W>
__device__ __forceinline__ void short_rows(const PrefillArgs& a, int s, int kvh, int q0, int T, int L, int rows,
                                           int step0, int nsteps, int part, char* sq_bytes, float* srow) {
  using Tl = Tile<DT, D>;
  constexpr int KS = Tl::KS, QROW = Tl::QROW, QCH = Tl::QCH, ROWB = Tl::ROWB;
  using VVec = typename Tl::VVec;
  constexpr int NW = W < 4 ? W : 4;  // wavefronts that take tiles
  uint16_t(*sq)[QROW] = reinterpret_cast<uint16_t(*)[QROW]>(sq_bytes);
  float(*sm)[16] = reinterpret_cast<float(*)[16]>(sq_bytes + 16 * QROW * 2);
  float(*sl)[16] = sm + NW;
  int* sbad = reinterpret_cast<int*>(sl + NW);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int grp = lane >> 4, col = lane & 15;
  const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;
  const int g = a.g;
  const int base = L - T;

  // Query rows 0..rows-1 (row rho: token rho / g, head kvh g + rho % g),
  // zero past them.
  for (int idx = tid; idx < 16 * QCH; idx += 64 * W) {
    const int r = idx / QCH, ch = idx - r * QCH;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r < rows)
      v = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(a.q) +
                                          ((size_t)(q0 + r / g) * a.Hq + kvh * g + r % g) * ROWB + ch * 16);
    *reinterpret_cast<uint4*>(&sq[r][ch * 8]) = v;
  }
  lds_barrier();

  // This partition's positions [t_lo, t_hi): 16-slot tiles tb_lo .. tb_lo + ntile - 1.
  const int lm = a.lbs - 4;
  const int t_lo = step0 * kStep, t_hi = min(nsteps * kStep, L);
  const int tb_lo = t_lo >> 4, ntile = ((t_hi + 15) >> 4) - tb_lo;
  const int cnt = wave < NW && ntile > wave ? (ntile - wave + NW - 1) / NW : 0;
  // Positions at or past lim are masked in this lane's column (its row's
  // position + 1; padding columns copy the last row so they stay finite).
  const int lim = base + min(col, rows - 1) / g + 1;
  const float qsg = a.neg_scale ? -a.qscale : a.qscale;  // scale * log2(e)
  const uint16_t* qsrc = &sq[col][grp * 8];
  const int32_t* btrow = a.bt + (size_t)s * a.maxb;
  float m_run = -__FLT_MAX__, l_run = 0.f;
  f32x4 acc[Tl::DPL];
#pragma unroll
  for (int u = 0; u < Tl::DPL; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  bool bad = false;
  uint4 kA[KS], kB[KS];
  VVec vA[4], vB[4];
  for (int k0 = 0; k0 < cnt; k0 += 64) {  // table entries 64 tiles at a time
    const int c = min(64, cnt - k0);
    const int first = tb_lo + wave + k0 * NW;  // logical tile of this group's k = 0
    bool badg;
    const int myid = load_ids(btrow, c, a.num_blocks, [&](int k) { return first + k * NW; }, badg, a.Hkv, kvh, lm);
    bad |= badg;
    pipeline(
        c, kA, vA, kB, vB,
        [&](int k, uint4(&kr)[KS], VVec(&vr)[4]) {
          const size_t off = (size_t)(unsigned)__builtin_amdgcn_readlane(myid, k) * (16 * ROWB);
          Tl::load(a.kp + off, a.vp + off, grp, col, min(15, L - 1 - (first + k * NW) * 16), kr, vr);
        },
        [&](int k, const uint4(&kr)[KS], const VVec(&vr)[4], bool valid) {
          asm volatile("" ::: "memory");
          Tl::consume(kr, vr, qsrc, (first + k * NW) * 16 + grp * 4, valid ? lim : 0, qsg, x16, x32, m_run, l_run,
                      acc);
        });
  }
  // (each wave stages into its own slots, past the query tile: no barrier
  // before, one before the merge reads them)
  if (wave < NW) {
    Tl::stage(m_run, l_run, acc, cnt > 0, grp, col, rows, x16, x32, sm[wave], sl[wave], srow + wave * 16 * D);
    if (lane == 0) sbad[wave] = bad;
  }
  lds_barrier();
  bool any_bad = false;
#pragma unroll
  for (int w = 0; w < NW; ++w) any_bad |= sbad[w] != 0;
  const float nan = __builtin_nanf("");
  // One thread per (row, 4 dims): the merged row, then its store.
  for (int idx = tid; idx < rows * (D / 4); idx += 64 * W) {
    const int r = idx / (D / 4), d = (idx - r * (D / 4)) * 4;
    float M = sm[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm[w][r]);
    float den = 0.f, num[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = sl[w][r] * fast_exp2(sm[w][r] - M);  // 0 for a wave without positions of this row
      den += wt;
      if (sl[w][r] > 0.f) {
        const float4 o = *reinterpret_cast<const float4*>(srow + (w * 16 + r) * D + d);
        num[0] = fmaf(wt, o.x, num[0]);
        num[1] = fmaf(wt, o.y, num[1]);
        num[2] = fmaf(wt, o.z, num[2]);
        num[3] = fmaf(wt, o.w, num[3]);
      }
    }
    if (a.P > 1 && base + r / g < t_lo) continue;  // the row does not reach this partition
    const float inv = any_bad ? nan : 1.f / den;
    const size_t row = (size_t)(q0 + r / g) * a.Hq + kvh * g + r % g;
    if (a.P == 1) {
      float f[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) f[i] = num[i] * inv;
#pragma unroll
      for (int i = 4; i < 8; ++i) f[i] = 0.f;
      const uint4 v = pack16<DT>(f);
      *reinterpret_cast<uint2*>(reinterpret_cast<char*>(a.out) + (row * D + d) * 2) = make_uint2(v.x, v.y);
    } else {
      const size_t e = row * a.P + part;
      *reinterpret_cast<float4*>(a.ws_o + e * D + d) = make_float4(num[0] * inv, num[1] * inv, num[2] * inv,
                                                                   num[3] * inv);
      if (d == 0) {
        a.ws_m[e] = any_bad ? nan : M;
        a.ws_l[e] = den;
      }
    }
  }
}

// kDma = false: K and V go through registers into LDS (V transposed into the
// PV operand's k-slot order by the threads).  kDma = true: both go straight
// from global memory into LDS in token-row order (global->LDS 16-byte loads,
// lane i of an instruction filling bytes 16 i of its 1 KiB), and the PV
// operand is read with the transposing LDS read; no staging registers, no
// staging ALU work.
template <int DT, int D, int NC, bool kDma, int W, bool kRows>
__global__ __launch_bounds__(64 * W) void prefill_mfma(PrefillArgs a) {
  constexpr int ROW = D;                     // LDS row of K, elements (16-byte chunks XOR-swizzled)
  constexpr int KS = D / 32;                 // QK k-steps over the head dim
  constexpr int DPL = D / 16;                // output dims per lane per row = PV MFMAs per column group
  constexpr int CH = D / 8;                  // 16-byte chunks per token row
  constexpr int LOADS = kStep * CH / 256;    // chunks of K (and of V) per thread per step
  constexpr int PAIRS = LOADS / 2;           // (token pair, chunk) items per thread per step
  constexpr int VROW = kPair + 8;            // LDS row of V^T: one pass's 32 slots + 16 bytes of padding
  constexpr int R = W * 16 * NC;             // rows per workgroup
  static_assert(W == kWaves || (kDma && W == kWideWaves), "register staging assumes 4 wavefronts");
  static_assert(PAIRS >= 1 && kStep * CH % 512 == 0, "token pairs must split evenly over the threads");
  static_assert(8 % DPL == 0, "a 16-byte chunk's dims map to whole V^T rows");
  static_assert(D == 64 || D == 128, "the swizzle keys were measured for these row lengths");
  auto kkey = [](int r) { return r & (D / 8 - 1); };

  // LDS layout of K: the score reads have lane (G, c) read 16-byte chunk
  // G + 4k of row c (mod 16).  A 16-byte read takes 4 LDS cycles per
  // wavefront when its lanes do not conflict.  Chosen by measuring the
  // bank-conflict counter for these exact lane patterns on gfx950: rows
  // padded to 272 bytes measured 8 cycles (two-way conflicts); unpadded
  // rows with chunk j of row r stored at chunk j ^ kkey(r),
  // kkey(r) = r mod (D / 8), measured 4, and so do the stash writes of the
  // register-staged variant (lane = chunk of one token row).
  __shared__ __align__(16) uint16_t sK[2][kStep][ROW];
  // Register-staged variant: V transposed for the PV A operand: row
  // (pass, u * 16 + c) holds head dim DPL * c + u of the pass's 32
  // positions in k-slot order (slot 8G + e is token 16 (e / 4) + 4G + e % 4),
  // so lane (G, c) reads its operand for output tile u as one 16-byte chunk.
  // Rows are 80 bytes: the stash's 4-byte writes (16 lanes, 16 consecutive
  // rows, one column) then hit 16 distinct banks; the 16-byte reads measure
  // two-way conflicts, which costs less here than a 64-byte swizzled row
  // whose writes conflict.
  __shared__ __align__(16) uint16_t sV[kDma ? 1 : 2][kDma ? 1 : kPairs * D][kDma ? 8 : VROW];
  // kDma: V in token-row order, 16-byte chunk j of row r stored at chunk
  // j ^ vkey(r), so the transposing reads of one instruction (16 rows, the
  // same two chunks of each) spread over the banks.
  __shared__ __align__(16) uint16_t sVn[kDma ? 2 : 1][kDma ? kStep : 1][kDma ? ROW : 8];
  auto vkey = [](int r) { return 2 * (r & (D / 16 - 1)); };
  __shared__ int s_bad;

  // XCD-aware numbering.  The hardware deals workgroups round-robin over the
  // 8 XCDs (workgroup b runs on XCD b % 8).  Work item (sequence, KV head)
  // number i goes to XCD i % 8, so all row tiles of one item share that
  // XCD's L2 while the items -- and with 8 KV heads, one head of every
  // sequence -- are spread evenly over the XCDs.  Within an XCD an unsplit
  // launch runs its workgroups longest walk first (lpt_pick; the plain tile
  // order below beyond 256 items per XCD).  With P > 1 each row tile is cut
  // into P partitions of positions, latest tile first, its partitions in
  // order.
  const int items = a.B * a.Hkv;
  const int per_xcd = (items + 7) >> 3;  // items per XCD (upper bound)
  const int xcd = (int)(blockIdx.x & 7), local = (int)(blockIdx.x >> 3);
  int item, tile, part = 0;
  int q0 = 0, q1 = 0, L = 0;
  const bool picked = a.P == 1 && per_xcd <= 64 * kLptPerLane;
  if (picked) {
    if (!lpt_pick(a, xcd, local, per_xcd, R, kRows, item, tile, q0, q1, L)) return;
  } else {
    item = (local % per_xcd) * 8 + xcd;
    const int tp = local / per_xcd;
    tile = a.tiles - 1 - tp / a.P;
    part = tp % a.P;
  }
  if (item >= items) return;
  const int kvh = item % a.Hkv;
  const int s = item / a.Hkv;
  if (s >= a.B) return;

  if (!picked) {  // (the pick read these already)
    seq_range<kRows>(a, s, q0, q1);
    L = a.cl[s];
  }
  const int T = q1 - q0;
  const int g = a.g;
  if (q0 < 0 || q1 < q0 || q1 > a.N || T > L || (int64_t)L > ((int64_t)a.maxb << a.lbs) || T > a.max_q ||
      ((a.P > 1 || kRows) && L > a.max_ctx)) {
    // Unservable sequence: NaN over whatever part of its row range exists
    // (in the decode layout an empty context gives a zero row instead).
    if (tile == a.tiles - 1 && part == 0) {
      const int r0 = min(max(q0, 0), a.N), r1 = min(max(q1, r0), a.N);
      if (kRows && L == 0)
        nan_rows<DT, true>(a.out, r0, r1, a.Hq, kvh * g, g, D);
      else
        nan_rows<DT>(a.out, r0, r1, a.Hq, kvh * g, g, D);
    }
    return;
  }
  const int rows = T * g;
  if (tile * R >= rows) return;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int G = lane >> 4, c = lane & 15;
  const int x16 = (lane ^ 16) << 2, x32 = (lane ^ 32) << 2;
  const int base = L - T;  // position of new token 0

  // WG and wave row ranges; positions the workgroup must walk.
  const int rho_wg_last = min(tile * R + R, rows) - 1;
  const int nsteps_all = (base + rho_wg_last / g) / kStep + 1;
  const int step0 = part * a.psteps;  // this partition's steps [step0, nsteps)
  const int nsteps = a.P > 1 ? min(nsteps_all, step0 + a.psteps) : nsteps_all;
  if (step0 >= nsteps) return;  // no row of the tile reaches this partition
  if constexpr (kDma) {
    if (rows <= 16 && a.lbs >= 4) {  // (whole-workgroup branch)
      short_rows<DT, D, W>(a, s, kvh, q0, T, L, rows, step0, nsteps, part, reinterpret_cast<char*>(&sK[0][0][0]),
                           reinterpret_cast<float*>(&sVn[0][0][0]));
      return;
    }
  }
  const int rho_w0 = tile * R + wave * 16 * NC;
  const bool wave_on = rho_w0 < rows;
  const int lim_w_lo = base + min(rho_w0, rows - 1) / g;
  const int lim_w_hi = base + (min(rho_w0 + 16 * NC, rows) - 1) / g;

  // This lane's rows (one per column group) and their causal limits.
  const bool neg = a.neg_scale != 0;
  const float qs = a.qscale;  // |scale| * log2(e)
  int lim[NC];
  uint4 qr[NC][KS];
  const uint16_t* qp = reinterpret_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    const int rho = min(rho_w0 + 16 * n + c, rows - 1);
    const int i = rho / g, h = rho - i * g;
    lim[n] = base + i;
    const uint16_t* src = qp + ((size_t)(q0 + i) * a.Hq + kvh * g + h) * D + 8 * G;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      uint4 v = *reinterpret_cast<const uint4*>(src + 32 * k);
      if (neg) v = make_uint4(v.x ^ 0x80008000u, v.y ^ 0x80008000u, v.z ^ 0x80008000u, v.w ^ 0x80008000u);
      qr[n][k] = v;
    }
  }

  // Cooperative load of one step's K and V chunks into registers.
  const int32_t* btrow = a.bt + (size_t)s * a.maxb;
  const int bmask = (1 << a.lbs) - 1;  // slots per block - 1
  // Byte offsets: a block is Hkv * bs * D * 2 bytes (< 2^32, checked on the
  // host), so a slot's address is one 32 x 32 -> 64-bit multiply-add of the
  // block id plus a 32-bit offset inside the block.
  const uint32_t head_off = ((uint32_t)kvh * D * 2) << a.lbs;
  const uint32_t blk_bytes = ((uint32_t)a.Hkv * D * 2) << a.lbs;
  const char* kp = a.kp;
  const char* vp = a.vp;
  bool bad = false;
  // (plain vector types: HIP's uint4 is copied by memcpy, which keeps these
  // arrays in scratch memory)
  u32x4 kreg[LOADS], vreg[LOADS];
  // Thread item m (of PAIRS per step): token pair tp = it / CH (positions
  // 2 tp and 2 tp + 1 of the step) at 16-byte chunk ch = it % CH, it = tid +
  // 256 m; both tokens sit in one block (blocks hold >= 8 slots).  The block
  // id behind each item is fetched one step ahead of the K/V loads that use
  // it, as a per-lane vector load on purpose: a scalar load would share its
  // wait counter with the LDS operand reads, and since scalar loads complete
  // out of order the first operand wait of every step would then also wait
  // for the table lookup.  Positions past L-1 read position L-1.
  auto load_ids = [&](int step, int (&ids)[PAIRS]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
      const int tp = (tid + 256 * m) / CH;
      ids[m] = btrow[min(step * kStep + 2 * tp, L - 1) >> a.lbs];
    }
  };
  auto issue = [&](int step, const int (&ids)[PAIRS]) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
      const int it = tid + 256 * m;
      const int tp = it / CH, ch = it - tp * CH;
      uint32_t id = (uint32_t)ids[m];
      if (id >= (uint32_t)a.num_blocks) {
        bad = true;
        id = 0;
      }
      const uint32_t in_blk = head_off + ch * 16;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int pos = min(step * kStep + 2 * tp + j, L - 1);
        const uint64_t off = (uint64_t)id * blk_bytes + (in_blk + (uint32_t)(pos & bmask) * (D * 2));
        kreg[2 * m + j] = *reinterpret_cast<const u32x4*>(kp + off);
        vreg[2 * m + j] = *reinterpret_cast<const u32x4*>(vp + off);
      }
    }
  };
  auto stash = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < PAIRS; ++m) {
      const int it = tid + 256 * m;
      const int tp = it / CH, ch = it - tp * CH;
      *reinterpret_cast<u32x4*>(&sK[buf][2 * tp][(ch ^ kkey(2 * tp)) * 8]) = kreg[2 * m];
      *reinterpret_cast<u32x4*>(&sK[buf][2 * tp + 1][(ch ^ kkey(2 * tp + 1)) * 8]) = kreg[2 * m + 1];
      // V^T: the pair's values of each of the chunk's 8 dims, packed into
      // one word (token 2 tp in the low half) at k-slot sg, sg + 1.  Dim
      // dd = 8 ch + i goes to row pp D + (dd % DPL) 16 + dd / DPL, which
      // (DPL dividing 8) is the lane's row pp D + (8 / DPL) ch plus a
      // constant per i: one address per item, the rest immediate offsets.
      const int pp = (2 * tp) / kPair, t = (2 * tp) % kPair;
      const int sg = 8 * ((t >> 2) & 3) + 4 * (t >> 4) + (t & 3);
      uint16_t* vrow = &sV[buf][pp * D + (8 / DPL) * ch][sg];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t lo = vreg[2 * m][i >> 1], hi = vreg[2 * m + 1][i >> 1];
        *reinterpret_cast<uint32_t*>(vrow + ((i % DPL) * 16 + i / DPL) * VROW) =
            __builtin_amdgcn_perm(hi, lo, (i & 1) ? 0x07060302u : 0x05040100u);
      }
    }
  };

  // kDma: one step's K and V rows straight into LDS.  Wavefront w fills rows
  // [RW w, RW w + RW) of the step (RW = 64 / W) with NI instructions for K
  // and NI for V, each filling RPI consecutive rows (1 KiB); lane i fills
  // chunk i % CH of row i / CH and so loads the source chunk that belongs
  // there (the swizzles are applied on the load side).  Every 8-row half of
  // a wave's rows lies in one block (blocks hold a power of two >= 8 of
  // slots), so an instruction's addresses are a wave-uniform base -- its
  // half's first row in the block, in scalar registers -- plus a per-lane
  // offset that is the same at every step.  Only a step whose rows pass
  // L - 1 takes per-lane rows, clamped to L - 1 (V past the context must be
  // finite: its weights are zero, and 0 * NaN would poison the row).
  constexpr int RPI = 1024 / (D * 2);  // token rows per instruction
  constexpr int RW = kStep / W;        // rows of a step per wavefront
  constexpr int NH = RW / 8;           // 8-row halves per wavefront
  constexpr int NI2 = 8 / RPI;         // instructions per half
  constexpr int NI = NH * NI2;         // instructions per wave, K (and V)
  static_assert(kStep % (8 * W) == 0 && NH >= 1 && NI2 >= 1, "whole 8-row halves per wavefront");
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint32_t koff[NI], voff[NI];  // instruction m: offset of this lane's chunk from its half's first row
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const int h = m / NI2;
    const int r = (m % NI2) * RPI + lane / CH;  // row within the half
    const int rs = RW * wv + 8 * h + r;         // row within the step (swizzle key)
    const int ch = lane % CH;
    koff[m] = (uint32_t)(r * (D * 2) + (ch ^ kkey(rs)) * 16);
    voff[m] = (uint32_t)(r * (D * 2) + (ch ^ vkey(rs)) * 16);
  }
  const uint32_t ldsK = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)&sK[0][0][0]);
  const uint32_t ldsV = (uint32_t)__builtin_amdgcn_readfirstlane(
      (int)(uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)&sVn[0][0][0]);
  constexpr uint32_t kBufBytes = kStep * ROW * 2;
  // Table entries of the step's halves: lane l reads the entry of row l % 8
  // of each half, clamped to L - 1 -- one block per half whichever row.
  auto load_ids_dma = [&](int step, int (&ids)[NH]) __attribute__((always_inline)) {
    const int p = step * kStep + RW * wv + (lane & 7);
#pragma unroll
    for (int h = 0; h < NH; ++h) ids[h] = btrow[min(p + 8 * h, L - 1) >> a.lbs];
  };
  // Instruction m (K and V; rows of half m / NI2) of step `step` into buffer buf.
  auto dma_inst = [&](int step, int buf, const int (&ids)[NH], int m) __attribute__((always_inline)) {
    const int h = m / NI2, mm = m % NI2;
    const int p0 = step * kStep + RW * wv;
    const bool whole = p0 + RW - 1 < L;  // no row of the wave past L - 1
    uint32_t id = (uint32_t)__builtin_amdgcn_readfirstlane(ids[h]);
    if (id >= (uint32_t)a.num_blocks) {
      bad = true;
      id = 0;
    }
    const int ph = p0 + 8 * h;
    const uint32_t rb = whole ? (uint32_t)(ph & bmask) * (D * 2) : 0u;
    const uint64_t off = (uint64_t)id * blk_bytes + head_off + rb;
    uint32_t ko = koff[m], vo = voff[m];
    if (!whole) {  // the lane's row, clamped, replaces its row in the half
      const int r = mm * RPI + lane / CH;
      const uint32_t dr = (uint32_t)(min(ph + r, L - 1) & bmask) * (D * 2) - (uint32_t)(r * (D * 2));
      ko += dr;
      vo += dr;
    }
    const uint32_t lrow = (uint32_t)(RW * wv + 8 * h + mm * RPI) * (ROW * 2) + (uint32_t)buf * kBufBytes;
    dma16(kp + off, ko, ldsK + lrow);
    dma16(vp + off, vo, ldsV + lrow);
  };

  float m_run[NC];
  float moff[NC];   // -m_run * qs: the weights' exponent offset
  f32x4 l_acc[NC];  // row sums of the rounded weights, from the matrix core (all four entries equal)
  f32x4 acc[NC][DPL];
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    m_run[n] = -__FLT_MAX__;  // finite, so a zero scale gives 2^0, not NaN
    moff[n] = -m_run[n] * qs;  // (+inf for scales above 1: the first weights overflow and set the reference)
    l_acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[n][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Passes of 32 positions starting at t0 (LDS rows r0..r0+31 of a step).
  // Lazy rescaling: the weights use a reference max m_run that is raised
  // only when some weight of the wave comes out above 2^kSlack (then every
  // row moves to its true running max and its weights are recomputed);
  // otherwise the weights may exceed 1, by at most 2^kSlack, and the
  // accumulators keep their scale.  l and acc always share the reference,
  // so o = acc / l is exact.
  constexpr uint32_t kSlackBits = 0x43800000u;  // 2^kSlack = 256.0f, kSlack = 8
  constexpr uint32_t kOne2 = DT == PA_BF16 ? 0x3F803F80u : 0x3C003C00u;  // two 1.0s of the KV type
  const uint4 ones = make_uint4(kOne2, kOne2, kOne2, kOne2);
  // One pass in four parts (the direct-load kernel also runs two passes
  // with their parts interleaved): scores, V operands, weights, products.
  // Wave priority: a wavefront's matrix phases (score and PV products) run
  // at priority 1, its softmax at 0, so that where the two wavefronts of a
  // SIMD compete for issue the one feeding the matrix core wins (measured
  // +2-3% on the prefill workloads; without it the older wavefront wins every
  // tie).
  auto qk_scores = [&](int buf, int r0, f32x4 (&sc)[NC][2]) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int n = 0; n < NC; ++n) sc[n][0] = sc[n][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&sK[buf][r0 + 16 * half + c][((4 * k + G) ^ kkey(c)) * 8]);
#pragma unroll
        for (int n = 0; n < NC; ++n) sc[n][half] = mfma32<DT>(ka, qr[n][k], sc[n][half]);
      }
    }
  };
  // kDma: the pass's V operands (two transposing reads per output tile;
  // lane 4k + q of group G reads dims 16u + 4q.. of token 16 h + 4G + k,
  // h = 0, 1, so the lane receives dim 16u + c of the eight tokens of its
  // k-slots), read before the softmax, whose ALU work then covers their LDS
  // latency.
  constexpr int VN = kDma ? DPL : 1;  // V operands held per pass
  auto read_vops = [&](int buf, int r0, uint4 (&vops)[VN]) __attribute__((always_inline)) {
    if constexpr (kDma) {
      const int q = c & 3, kt = c >> 2;
      const int R0 = r0 + 4 * G + kt, R1 = R0 + 16;
      const char* row0 = reinterpret_cast<const char*>(&sVn[buf][R0][0]) + 8 * (q & 1);
      const char* row1 = reinterpret_cast<const char*>(&sVn[buf][R1][0]) + 8 * (q & 1);
#pragma unroll
      for (int u = 0; u < DPL; ++u) {
        const int cc = 2 * u + (q >> 1);  // 16-byte chunk of dims 16u + 4q
        const uint2 lo = lds_read_tr16(row0 + (cc ^ vkey(R0)) * 16);
        const uint2 hi = lds_read_tr16(row1 + (cc ^ vkey(R1)) * 16);
        vops[u] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    }
  };
  // Scores of the lane's eight k-slots (k-slot e of lane group G is token
  // 16*(e/4) + 4G + e%4 of the pass), masked past each row's limit, and
  // their weights 2^(x qs - m qs) against the rows' reference m.  Weights
  // are >= 0, so their bit patterns order like unsigned integers: one
  // integer max tells whether some weight of the lane passed 2^kSlack.
  // Only then (rarely) are the rows' maxima gathered across the four lane
  // groups, the accumulators rescaled and the weights recomputed.
  auto weights = [&](auto masked, const f32x4 (&sc)[NC][2], int t0, uint4 (&pb)[NC]) __attribute__((always_inline)) {
    constexpr bool kMasked = decltype(masked)::value;
    __builtin_amdgcn_s_setprio(0);
    float x[NC][8], p[NC][8];
    uint32_t pbits = 0;
#pragma unroll
    for (int n = 0; n < NC; ++n) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[n][e] = sc[n][e >> 2][e & 3];
        if constexpr (kMasked)
          if (t0 + 16 * (e >> 2) + 4 * G + (e & 3) > lim[n]) x[n][e] = -__builtin_huge_valf();
        // a masked score is -inf: 2^-inf = 0 (with a zero scale 0 * -inf
        // would be NaN, hence the select)
        p[n][e] = fast_exp2(fmaf(x[n][e], qs, moff[n]));
        if constexpr (kMasked) p[n][e] = x[n][e] == -__builtin_huge_valf() ? 0.f : p[n][e];
        pbits = max(pbits, __float_as_uint(p[n][e]));
      }
    }
    if (__builtin_amdgcn_ballot_w64(pbits > kSlackBits) != 0) {
#pragma unroll
      for (int n = 0; n < NC; ++n) {
        const float lm = fmaxf(fmaxf(fmaxf(x[n][0], x[n][1]), fmaxf(x[n][2], x[n][3])),
                               fmaxf(fmaxf(x[n][4], x[n][5]), fmaxf(x[n][6], x[n][7])));
        const float mn = fmaxf(m_run[n], max_groups(lm, x16, x32));
        const float alpha = fast_exp2((m_run[n] - mn) * qs);
        m_run[n] = mn;
        moff[n] = -mn * qs;
        l_acc[n] *= alpha;
#pragma unroll
        for (int u = 0; u < DPL; ++u) acc[n][u] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[n][e] = fast_exp2(fmaf(x[n][e], qs, moff[n]));
          if constexpr (kMasked) p[n][e] = x[n][e] == -__builtin_huge_valf() ? 0.f : p[n][e];
        }
      }
    }
#pragma unroll
    for (int n = 0; n < NC; ++n)
      pb[n] = make_uint4(pack2<DT>(p[n][0], p[n][1]), pack2<DT>(p[n][2], p[n][3]), pack2<DT>(p[n][4], p[n][5]),
                         pack2<DT>(p[n][6], p[n][7]));
  };
  // Row sums of the rounded weights (an all-ones A operand) and the PV
  // products; the V^T operand of output tile u is one 16-byte LDS read
  // (kDma: the operands read before the softmax).
  auto products = [&](int buf, int r0, const uint4 (&pb)[NC], const uint4 (&vops)[VN]) __attribute__((always_inline)) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int n = 0; n < NC; ++n) l_acc[n] = mfma32<DT>(ones, pb[n], l_acc[n]);
#pragma unroll
    for (int u = 0; u < DPL; ++u) {
      uint4 va;
      if constexpr (kDma) {
        va = vops[u];
      } else {
        va = *reinterpret_cast<const uint4*>(&sV[buf][(r0 / kPair) * D + u * 16 + c][8 * G]);
      }
#pragma unroll
      for (int n = 0; n < NC; ++n) acc[n][u] = mfma32<DT>(va, pb[n], acc[n][u]);
    }
  };
  // One pass over 32 positions starting at t0 (LDS rows r0..r0+31).
  auto pass = [&](auto masked, int buf, int r0, int t0) __attribute__((always_inline)) {
    f32x4 sc[NC][2];
    uint4 vops[VN], pb[NC];
    qk_scores(buf, r0, sc);
    read_vops(buf, r0, vops);
    weights(masked, sc, t0, pb);
    products(buf, r0, pb, vops);
  };

  if (tid == 0) s_bad = 0;
  auto passes = [&](int step, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int pp = 0; pp < kPairs; ++pp) {
      const int t0 = step * kStep + pp * kPair;
      if (!(wave_on && t0 <= lim_w_hi)) continue;
      // Only passes that reach past a row's causal limit need the mask.
      if (t0 + kPair - 1 > lim_w_lo)
        pass(std::true_type{}, buf, pp * kPair, t0);
      else
        pass(std::false_type{}, buf, pp * kPair, t0);
    }
  };
  if constexpr (kDma) {
    // The barrier after each step waits for this wave's loads into the other
    // buffer (the compiler's fence before s_barrier) and for every wave to
    // finish reading this one.
    int ids[NH];
    auto retire_ids = [&] {
#pragma unroll
      for (int h = 0; h < NH; ++h) asm volatile("" ::"v"(ids[h]));
    };
    load_ids_dma(step0, ids);
#pragma unroll
    for (int m = 0; m < NI; ++m) dma_inst(step0, 0, ids, m);
    load_ids_dma(step0 + 1, ids);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    retire_ids();
    // The next step's loads are issued half before each pass: a wavefront's
    // loads all at once would hold its instruction issue until the compute
    // unit's load path has taken them (measured: 2-6% slower than halves;
    // splitting each half again around the score products was slower
    // still).
    static_assert(kPairs == 2, "half of the next step's loads before each pass");
    constexpr int kFirst = NI >= 2 ? NI / 2 : NI;  // instructions issued before pass 0
    for (int step = step0; step < nsteps; ++step) {
      const int buf = (step - step0) & 1;
      const bool more = step + 1 < nsteps;
      auto issue_next = [&](int pp) __attribute__((always_inline)) {
        if (more) {
#pragma unroll
          for (int m = pp == 0 ? 0 : kFirst; m < (pp == 0 ? kFirst : NI); ++m) dma_inst(step + 1, buf ^ 1, ids, m);
        }
        if (pp == kPairs - 1 && step + 2 < nsteps) load_ids_dma(step + 2, ids);
      };
      const int ts = step * kStep;
#pragma unroll
      for (int pp = 0; pp < kPairs; ++pp) {
        issue_next(pp);
        const int t0 = ts + pp * kPair;
        if (!(wave_on && t0 <= lim_w_hi)) continue;
        if (t0 + kPair - 1 > lim_w_lo)
          pass(std::true_type{}, buf, pp * kPair, t0);
        else
          pass(std::false_type{}, buf, pp * kPair, t0);
      }
      __builtin_amdgcn_s_setprio(0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads into the other buffer
      __syncthreads();
      // (the next step's table entries arrived with that wait; using them
      // here lets the compiler retire their loads now, where nothing is
      // outstanding, instead of waiting between the next step's asm loads,
      // whose counts it cannot see)
      retire_ids();
    }
  } else {
    int ids[PAIRS];
    load_ids(step0, ids);
    issue(step0, ids);
    stash(0);
    load_ids(step0 + 1, ids);  // ids of the next step are always one step ahead of its loads
    __syncthreads();

    for (int step = step0; step < nsteps; ++step) {
      const int buf = (step - step0) & 1;
      const bool more = step + 1 < nsteps;
      if (more) issue(step + 1, ids);
      if (step + 2 < nsteps) load_ids(step + 2, ids);
      passes(step, buf);
      if (more) stash(buf ^ 1);
      __syncthreads();
    }
  }
  if (bad) s_bad = 1;
  __syncthreads();
  const bool wg_bad = s_bad != 0;

  // Epilogue: lane (G, c) holds dims [4*DPL*G, 4*DPL*G + 4*DPL) of row c of
  // each column group (acc[n][u][j] is dim DPL*(4G + j) + u).
  // With P > 1: the normalised partial row, its reference max (base 2) and
  // its sum go to the workspace for prefill_reduce -- only for rows that
  // reach this partition (the merge reads partitions 0..lim / psize).
  if (!wave_on) return;
#pragma unroll
  for (int n = 0; n < NC; ++n) {
    const float lt = l_acc[n][0];
    const int rho = rho_w0 + 16 * n + c;
    if (rho >= rows) continue;
    const int i = rho / g, h = rho - i * g;
    if (a.P > 1 && base + i < step0 * kStep) continue;
    const float inv = wg_bad ? __builtin_nanf("") : 1.f / lt;
    float f[4 * DPL];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int u = 0; u < DPL; ++u) f[j * DPL + u] = acc[n][u][j] * inv;
    const size_t row = (size_t)(q0 + i) * a.Hq + kvh * g + h;
    if constexpr (kDma) {
      // (the transposing reads give output tile u the contiguous dims
      // 16u..16u+15: acc[n][u][j] is dim 16u + 4G + j)
      if (a.P > 1) {
        const size_t e = row * a.P + part;
        float* dst = a.ws_o + e * D + 4 * G;
#pragma unroll
        for (int u = 0; u < DPL; ++u)
          *reinterpret_cast<float4*>(dst + 16 * u) =
              make_float4(acc[n][u][0] * inv, acc[n][u][1] * inv, acc[n][u][2] * inv, acc[n][u][3] * inv);
        if (G == 0) {
          a.ws_m[e] = wg_bad ? __builtin_nanf("") : m_run[n] * qs;
          a.ws_l[e] = lt;
        }
      } else {
        char* dst = reinterpret_cast<char*>(a.out) + (row * D + 4 * G) * 2;
#pragma unroll
        for (int u = 0; u < DPL; ++u) {
          const float f8[8] = {acc[n][u][0] * inv, acc[n][u][1] * inv, acc[n][u][2] * inv, acc[n][u][3] * inv,
                               0.f, 0.f, 0.f, 0.f};
          const uint4 v = pack16<DT>(f8);
          *reinterpret_cast<uint2*>(dst + 32 * u) = make_uint2(v.x, v.y);
        }
      }
      continue;
    }
    if (a.P > 1) {
      const size_t e = row * a.P + part;
      float* dst = a.ws_o + e * D + 4 * DPL * G;
#pragma unroll
      for (int v = 0; v < DPL; ++v) *reinterpret_cast<float4*>(dst + 4 * v) = make_float4(f[4 * v], f[4 * v + 1], f[4 * v + 2], f[4 * v + 3]);
      if (G == 0) {
        a.ws_m[e] = wg_bad ? __builtin_nanf("") : m_run[n] * qs;
        a.ws_l[e] = lt;
      }
    } else {
      char* dst = reinterpret_cast<char*>(a.out) + (row * D + 4 * DPL * G) * 2;
#pragma unroll
      for (int v = 0; v < DPL / 2; ++v) *reinterpret_cast<uint4*>(dst + 16 * v) = pack16<DT>(f + 8 * v);
    }
  }
}

// Merge of the partitions of a split launch: workgroup (token n, head
// group y), one thread per (head, 4 dims).  Row (token n, head h) of
// sequence s at position p took partitions 0..p / psize; each gives (o, m, l)
// and the row is sum_p w_p o_p / sum_p w_p with w_p = l_p 2^(m_p - M),
// M = max_p m_p (PagedAttention (tensortonic), "5. Reading the Cache During
// Attention": softmax normalises over all positions at once).  Partitions
// are read 8 at a time with all their loads in flight, the running maximum
// rescaling what came before.  Sequences the main kernel wrote as NaN are
// left alone.
constexpr int kMergeBatch = 8;

template <int DT, int D, bool kRows>
__global__ __launch_bounds__(256) void prefill_reduce(PrefillArgs a) {
  constexpr int HPB = 256 / (D / 4);  // heads per workgroup
  const int n = blockIdx.x;
  // the token's sequence: the last s with query_start[s] <= n (row n's own
  // sequence in the decode layout)
  int lo = kRows ? n : 0, hi = kRows ? n : a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qs[mid] <= n)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int s = lo;
  int q0, q1;
  seq_range<kRows>(a, s, q0, q1);
  const int L = a.cl[s];
  const int T = q1 - q0;
  if (n < q0 || n >= q1 || q0 < 0 || q1 > a.N || T > L || (int64_t)L > ((int64_t)a.maxb << a.lbs) ||
      T > a.max_q || L > a.max_ctx)
    return;
  const int h = blockIdx.y * HPB + (int)threadIdx.x / (D / 4);
  if (h >= a.Hq) return;
  const int d = ((int)threadIdx.x % (D / 4)) * 4;
  const int pos = L - T + (n - q0);
  const int np = pos / (a.psteps * kStep) + 1;
  const size_t row = (size_t)n * a.Hq + h;
  const float* pm = a.ws_m + row * a.P;
  const float* pl = a.ws_l + row * a.P;
  const float* po = a.ws_o + row * a.P * D + d;
  float M = -__builtin_huge_valf(), den = 0.f;
  float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = 0; p0 < np; p0 += kMergeBatch) {
    float mv[kMergeBatch], lv[kMergeBatch];
    float4 ov[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      mv[j] = -__builtin_huge_valf();
      lv[j] = 0.f;
      ov[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p0 + j < np) {
        mv[j] = pm[p0 + j];
        lv[j] = pl[p0 + j];
        ov[j] = *reinterpret_cast<const float4*>(po + (size_t)(p0 + j) * D);
      }
    }
    float Mn = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) Mn = fmaxf(Mn, mv[j]);
    const float r = fast_exp2(M - Mn);  // 0 on the first batch (M = -inf)
    den *= r;
    num = make_float4(num.x * r, num.y * r, num.z * r, num.w * r);
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const float w = lv[j] * fast_exp2(mv[j] - Mn);  // 0 past the last partition
      den += w;
      num = make_float4(fmaf(w, ov[j].x, num.x), fmaf(w, ov[j].y, num.y), fmaf(w, ov[j].z, num.z),
                        fmaf(w, ov[j].w, num.w));
    }
    M = Mn;
  }
  const float inv = 1.f / den;
  float f[8] = {num.x * inv, num.y * inv, num.z * inv, num.w * inv, 0.f, 0.f, 0.f, 0.f};
  const uint4 v = pack16<DT>(f);
  *reinterpret_cast<uint2*>(reinterpret_cast<char*>(a.out) + (row * D + d) * 2) = make_uint2(v.x, v.y);
}

template <int DT, int D, bool kMerge>
void launch_nc(const PrefillArgs& a, hipStream_t st) {
  constexpr int HPB = 256 / (D / 4);
  // (no query_start: the decode layout, on the 4-wavefront direct-load kernel only)
  const bool rows = a.qs == nullptr;
  if (!kMerge && rows)
    hipExtLaunchKernelGGL((prefill_mfma<DT, D, kPrefillNC, true, kWaves, true>), dim3(a.grid), dim3(64 * kWaves), 0,
                          st, static_cast<hipEvent_t>(a.ev_start), static_cast<hipEvent_t>(a.ev_stop), 0, a);
  else if (!kMerge && a.kind == kPrefillWide)
    hipExtLaunchKernelGGL((prefill_mfma<DT, D, kPrefillNC, true, kWideWaves, false>), dim3(a.grid),
                          dim3(64 * kWideWaves), 0, st, static_cast<hipEvent_t>(a.ev_start),
                          static_cast<hipEvent_t>(a.ev_stop), 0, a);
  else if (!kMerge && a.kind == kPrefillDirect)
    hipExtLaunchKernelGGL((prefill_mfma<DT, D, kPrefillNC, true, kWaves, false>), dim3(a.grid), dim3(64 * kWaves), 0,
                          st, static_cast<hipEvent_t>(a.ev_start), static_cast<hipEvent_t>(a.ev_stop), 0, a);
  else if (!kMerge)
    hipExtLaunchKernelGGL((prefill_mfma<DT, D, kPrefillNC, false, kWaves, false>), dim3(a.grid), dim3(64 * kWaves), 0,
                          st, static_cast<hipEvent_t>(a.ev_start), static_cast<hipEvent_t>(a.ev_stop), 0, a);
  else if (a.P > 1 && rows)
    hipLaunchKernelGGL((prefill_reduce<DT, D, true>), dim3(a.N, (a.Hq + HPB - 1) / HPB), dim3(256), 0, st, a);
  else if (a.P > 1)
    hipLaunchKernelGGL((prefill_reduce<DT, D, false>), dim3(a.N, (a.Hq + HPB - 1) / HPB), dim3(256), 0, st, a);
}

template <int DT, bool kMerge>
void launch_d(const PrefillArgs& a, hipStream_t st) {
  if (a.D == 64)
    launch_nc<DT, 64, kMerge>(a, st);
  else
    launch_nc<DT, 128, kMerge>(a, st);
}

}  // namespace

void launch_prefill_mfma(const PrefillArgs& a, hipStream_t st) {
  if (a.dtype == PA_FP16)
    launch_d<PA_FP16, false>(a, st);
  else
    launch_d<PA_BF16, false>(a, st);
}

void launch_prefill_reduce(const PrefillArgs& a, hipStream_t st) {
  if (a.dtype == PA_FP16)
    launch_d<PA_FP16, true>(a, st);
  else
    launch_d<PA_BF16, true>(a, st);
}

}  // namespace pa
