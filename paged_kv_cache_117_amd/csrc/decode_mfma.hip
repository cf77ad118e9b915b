// pa_decode partition kernels for 16-bit KV (fp16 / bf16) on gfx950.
//
// Same computation as the VALU kernel in decode.hip (online softmax over a
// partition's blocks in logical order, base-2 exponentials, log-sum-exp
// partials), organised for bandwidth with both products on the matrix cores.
//
// Per tile (16 consecutive slots of one block and one KV head) one
// wavefront computes scores and PV on the matrix cores with K and V loaded
// straight into the operand registers (Tile in decode_tile.h).  KV tiles are
// loaded non-temporally: each is read once per step, and streaming them past
// the caches raises the gather bandwidth measurably (and leaves the caches
// to what is reused: tables, queries, partials).
//
// Unfilled slots of a final block get score -inf (weight exactly 0) and
// their V rows are replaced by the last filled row of the block (finite), so
// NaN/Inf garbage there never reaches the result.  Block ids outside
// [0, num_blocks) are never dereferenced: the result is NaN instead.
//
// Three kernels share this tile code:
//  * decode_stream (batches of up to 4096 sequences): a persistent grid whose
//    wavefronts each stream an equal share of the batch's blocks, cutting
//    sequences wherever the even split falls; decode_stream_reduce merges
//    the cut ones.
//  * decode_part_wave (larger batches, partitions of up to 64 blocks): one
//    wavefront per partition, four consecutive partitions per workgroup,
//    merged in LDS into one entry (the final row, or a partial for the
//    reduce) per workgroup.
//  * decode_part_mfma (larger batches, partitions of 65..256 blocks): the
//    four wavefronts of a workgroup share one partition, blocks dealt
//    round-robin.
// The partition kernels stage each wave's (m, l) and normalised rows in LDS
// and write the workgroup's entry with the same log-sum-exp merge as the
// reduce kernel.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "decode_kernels.h"
#include "decode_tile.h"
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kWaves = 4;

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

// N consecutive output elements (8 or 4 of a 16-bit type: 16 or 8 bytes)
// from fp32, rounded to nearest even.
template <int DT, int N>
__device__ __forceinline__ void store_row(void* out, size_t idx, const float* f) {
  static_assert(N == 8 || N == 4, "16 or 8 bytes");
  if constexpr (N == 8) {
    *reinterpret_cast<uint4*>(reinterpret_cast<char*>(out) + idx * 2) = pack16<DT>(f);
  } else {
    const float g8[8] = {f[0], f[1], f[2], f[3], 0.f, 0.f, 0.f, 0.f};
    const uint4 v = pack16<DT>(g8);
    *reinterpret_cast<uint2*>(reinterpret_cast<char*>(out) + idx * 2) = make_uint2(v.x, v.y);
  }
}

// The rows of a sequence with L = 0: zero (NaN for an invalid length).
template <int DT, int D>
__device__ __forceinline__ void fill_rows(void* out, size_t row0, int nh, bool bad_len) {
  const float fill = bad_len ? __builtin_nanf("") : 0.f;
  for (int i = threadIdx.x; i < nh * D; i += 256) store_elem<DT>(out, row0 * D + i, fill);
}

// What both kernels share once a workgroup knows its (sequence, head group):
// the query tile in LDS, one wave's tile stream over `cnt` 16-slot tiles (the
// k-th at logical tile first + k * step, its tile row -- see load_ids -- in
// lane k of `myid`), staging and the merged write of entry `e` of `nentries`.
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
                                             int first, int step, int L, int nh, float qscale,
                                             int nentries, int e, size_t row0, int E, void* out, float* ws_o,
                                             float* ws_m, float* ws_l) {
    const int lane = threadIdx.x & 63;
    const int wave = uni(threadIdx.x >> 6);
    const int grp = lane >> 4;
    const int col = lane & 15;
    const int x16 = (lane ^ 16) << 2;  // ds_bpermute addresses of the partner lanes
    const int x32 = (lane ^ 32) << 2;
    const uint16_t* qsrc = &sh.q[col][grp * 8];
    float m_run = kNegInf;  // running max of head `col`, base 2
    float l_run = 0.f;      // running sum over this lane's tokens
    f32x4 acc[DPL];
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (cnt > 0) {
      uint4 kA[KS], kB[KS];
      VVec vA[4], vB[4];
      pipeline<false>(
          cnt, kA, vA, kB, vB,
          [&](int k, uint4(&kr)[KS], VVec(&vr)[4]) {
            const size_t off = (size_t)(unsigned)__builtin_amdgcn_readlane(myid, k) * (16 * ROWB);
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
                                                       int psize, int E, int lm) {
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
  const int myid =
      load_ids(bt + (size_t)pl.s * maxb, cnt, num_blocks, [&](int k) { return b0 + k; }, bad, Hkv, pl.kvh, lm);
  Bd::run(sh, kp, vp, myid, bad, cnt, b0, 1, L, pl.nh, qscale, nent, pl.rank, pl.row0, E, out, ws_o, ws_m, ws_l);
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
                                                       int psize, int E, int lm) {
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
      load_ids(bt + (size_t)pl.s * maxb, cnt, num_blocks, [&](int k) { return b0 + wave + k * kWaves; }, bad, Hkv,
               pl.kvh, lm);
  Bd::run(sh, kp, vp, myid, bad, cnt, b0 + wave, kWaves, L, pl.nh, qscale, nparts, p, pl.row0, E, out, ws_o, ws_m,
          ws_l);
}

// ---------------------------------------------------------------------------
// Balanced split: every wavefront of a persistent grid streams the same
// amount of KV.
//
// HBM throughput of this gather is set by the whole chip (every CU with a
// few tiles in flight saturates it), so a launch takes as long as its most
// loaded CU: with one workgroup per partition, ragged batches leave a long
// tail of a few busy CUs.  Here the work is cut into units (one block, or
// one partition when a partition size is given) in (sequence, head group,
// block) order, and wave w of W takes units [w Q / W, (w+1) Q / W) of the Q
// in the batch.  A wave's range can start and end inside a (sequence, head
// group) segment and cross whole segments in between: a segment it covers
// whole is written as final rows, a cut one as a piece (normalised o, m, l)
// in slot 2w (the wave's first segment) or 2w+1 (its last), and the reduce
// merges a cut segment's pieces with the same log-sum-exp weights as the
// partition reduce.  The wave holding a segment's first unit records where
// its pieces are.
//
// A wave works in chunks of up to kChunkTiles tiles: it first stages the
// chunk's pieces (portions of segments), one descriptor per tile (physical
// row of the tile's block and head, last filled slot) and the pieces' query
// rows in its part of LDS, with all loads in flight at once; then one tile
// pipeline runs through the whole chunk, across piece boundaries, writing
// each finished piece from registers.  Workgroups are dealt round-robin to
// the 8 XCDs: workgroup i takes the (i mod 8)-th eighth of the stream, so
// each XCD's L2 sees a contiguous run of sequences (shared prefix blocks of
// neighbouring sequences hit there).
// ---------------------------------------------------------------------------
constexpr int kChunkTiles = 1024;  // tile descriptors per wave and chunk
constexpr int kChunkPieces = 64;   // pieces per wave and chunk (one lane each while planning)
constexpr int kChunkQRows = 48;    // query rows per wave and chunk

// Inclusive prefix sum over the wavefront's 64 lanes with DPP: shifts by
// 1, 2, 4, 8 within each row of 16 lanes (lanes before the row start add
// 0), then row 0's total into row 1 and row 2's into row 3 (row_bcast:15),
// then rows 0-1's total into rows 2-3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sums over the wavefront of three values at once.
__device__ __forceinline__ int3 wave_excl_scan3(int a, int b, int c) {
  return make_int3(wave_incl_scan(a) - a, wave_incl_scan(b) - b, wave_incl_scan(c) - c);
}

struct Piece {
  int nt;     // tiles in this chunk
  int qrow;   // first query row in the wave's LDS rows
  int nh;     // query heads
  int row0;   // first output row
  int seg;    // s * hs + hsub
  int np;     // pieces of the segment (valid with kFirstUnit)
  int flags;  // kWhole | kEnds | kFirstUnit | kLastSlot | kStarts
  int bad;    // an invalid block id in this portion
  int bto;    // chunk tile kk is the sequence's 16-slot tile bto + kk
  int srow;   // first block-table entry of the sequence (s * maxb)
  int kvh;    // KV head
  int rb;     // last filled slot of chunk tile kk: min(15, rb - 16 kk)
  int kb;     // first chunk tile
  int nrow;   // row of the sequence's new token for this KV head in k_new / v_new (s * Hkv + kvh)
};
constexpr int kWhole = 1, kEnds = 2, kFirstUnit = 4, kLastSlot = 8, kStarts = 16, kWriter = 32;

// Tile descriptor in LDS: (tile row << 5) | (new-token tile << 4) | last filled slot.
constexpr int kDescNew = 16;

// One workgroup of four wavefronts per CU, one wavefront per SIMD: the
// register file is the wave's alone (the compiler may use up to 512 VGPRs).
template <int DT, int D, int GMAX, bool kFuse>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void decode_stream(
    void* __restrict__ out, const void* __restrict__ q,
                                                    const char* kp, const char* vp, const int32_t* __restrict__ bt,
                                                    const int32_t* __restrict__ cl, float* __restrict__ pc_o,
                                                    float* __restrict__ pc_m, float* __restrict__ pc_l,
                                                    int2* __restrict__ info, int B, int Hq, int Hkv, int g, int nsub,
                                                    int num_blocks, int maxb, int max_ctx, float qscale, int unit,
                                                    int lm, const char* kn, const char* vn) {
  using T = Tile<DT, D>;
  constexpr int KS = T::KS, DPL = T::DPL, ROWB = T::ROWB, QROW = T::QROW, QCH = T::QCH;
  using VVec = typename T::VVec;
  static_assert(GMAX <= 16, "one MFMA column per query head");
  __shared__ int s_len[kStreamMaxSeqs];  // context length, -1 when out of range
  __shared__ unsigned s_desc[kWaves][kChunkTiles];
  // fused write: byte offset of each chunk tile's new-token row in k_new / v_new
  __shared__ unsigned s_nrow[kFuse ? kWaves : 1][kFuse ? kChunkTiles : 1];
  __shared__ Piece s_pc[kWaves][kChunkPieces];
  __shared__ unsigned char s_own[kWaves][kChunkTiles];   // piece of each chunk tile
  __shared__ unsigned char s_qown[kWaves][kChunkQRows];  // piece of each query row
  __shared__ __attribute__((aligned(16))) uint16_t s_q[kWaves][kChunkQRows + 1][QROW];  // last row: zeros

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = uni(tid >> 6);
  const int grp = lane >> 4;
  const int col = lane & 15;
  const int x16 = (lane ^ 16) << 2;
  const int x32 = (lane ^ 32) << 2;
  const int hs = Hkv * nsub;  // segments per sequence

  for (int i = tid; i < B; i += 256) {
    const int L = cl[i];
    s_len[i] = (L < 0 || L > max_ctx) ? -1 : L;
  }
  for (int i = lane; i < QROW / 8; i += 64) *reinterpret_cast<uint4*>(&s_q[wave][kChunkQRows][i * 8]) = make_uint4(0, 0, 0, 0);
  lds_barrier();
  // Rows of sequences without positions: zero (NaN for an invalid length),
  // dealt round-robin to the workgroups.
  for (int s = blockIdx.x; s < B; s += gridDim.x) {
    const int L = uni(s_len[s]);
    if (L > 0) continue;
    const float fill = L < 0 ? __builtin_nanf("") : 0.f;
    for (int i = tid; i < Hq * D; i += 256) store_elem<DT>(out, (size_t)s * Hq * D + i, fill);
    for (int h = tid; h < hs; h += 256) info[(size_t)s * hs + h] = make_int2(0, 0);  // nothing to merge
  }
  auto seg_units = [&](int L) { return L <= 0 ? 0 : ((L + 15) / 16 + unit - 1) / unit; };

  // Q, then this wave's range (waves past the first Q have none).  Virtual
  // workgroup v: the XCD's share of the stream, in order.
  int qt = 0;
  for (int i = lane; i < B; i += 64) qt += seg_units(s_len[i]);
  qt = __builtin_amdgcn_readlane(wave_incl_scan(qt), 63) * hs;
  const int G = gridDim.x;
  const int xcd = blockIdx.x & 7, n8 = G >> 3, r8 = G & 7;
  const int v = xcd * n8 + min(xcd, r8) + (blockIdx.x >> 3);
  const int W = min(G * kWaves, qt);
  const int w = v * kWaves + wave;
  if (w >= W) return;
  const int u_lo = (int)((long long)w * qt / W);
  const int u_hi = (int)((long long)(w + 1) * qt / W);

  // The sequence holding unit u_lo: prefix sums of units per sequence, 64
  // sequences at a time.
  int s = 0, pre = 0;
  for (int c0 = 0, base = 0; c0 < B; c0 += 64) {
    const int i = c0 + lane;
    const int us = i < B ? seg_units(s_len[i]) * hs : 0;
    const int incl = wave_incl_scan(us);
    const int excl = base + incl - us;
    const unsigned long long hit = __ballot(us > 0 && excl <= u_lo && u_lo < excl + us);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      s = c0 + l;
      pre = __shfl(excl, l);
      break;
    }
    base += __builtin_amdgcn_readlane(incl, 63);
  }
  s = uni(s);
  const int off0 = u_lo - uni(pre);  // units of s before u_lo
  const int us0 = seg_units(uni(s_len[s]));
  if (us0 <= 0) return;  // (cannot happen: s holds unit u_lo)
  int hsub = off0 / us0;        // walker: segment within the sequence,
  int uin = off0 - hsub * us0;  // unit within the segment where the current piece starts,
  int u = u_lo;                 // its unit in the stream,
  int tdone = 0;                // and its tiles staged by earlier chunks
  bool first = true;            // the wave's first piece (slot 2w)

  // The wave's first two tiles are known already: tiles tb0 and tb0 + 1 of
  // segment (s, hsub).  Their table entries are loaded now, the first chunk
  // is planned while they travel, and the two tile loads go out before the
  // chunk's staging loads (they then overlap the staging round trip instead
  // of following it).  Lane 0 holds tile tb0's entry, lane 1 the next one
  // (clamped to the sequence's tiles; used only when that tile is in the
  // wave's first piece).
  const int s0 = s;  // (the planning walker moves s on)
  const int L0 = uni(s_len[s]);
  const int tb0 = uin * unit;
  const int kvh0 = nsub == 1 ? hsub : hsub / nsub;
  const int nt0_seq = (L0 + 15) >> 4;  // 16-slot tiles of s; the last holds its new token
  const int pre_id = bt[(size_t)s * maxb + (min(tb0 + (lane & 1), ((L0 + 15) >> 4) - 1) >> lm)];
  bool first_chunk = true;

  Piece* pcs = s_pc[wave];
  unsigned* desc = s_desc[wave];
  uint16_t (*sq)[QROW] = s_q[wave];
  uint4 kA[KS], kB[KS];
  VVec vA[4], vB[4];
  float m_run = kNegInf, l_run = 0.f;
  f32x4 acc[DPL];
  bool bad = false;
  auto reset = [&]() {
    m_run = kNegInf;
    l_run = 0.f;
#pragma unroll
    for (int uu = 0; uu < DPL; ++uu) acc[uu] = f32x4{0.f, 0.f, 0.f, 0.f};
    bad = false;
  };

  while (u < u_hi) {
    // ---- Plan the chunk, one candidate piece per lane: lane j takes the
    // j-th segment from the walker's position (empty for sequences without
    // positions); exclusive sums over the lanes give every candidate's
    // units, tiles and query rows.  The chunk takes candidates in order
    // until tiles, query rows or pieces run out; a piece cut by the tile
    // limit continues in the next chunk.
    int npc, ntc, nqr;
    {
      const int cseg = hsub + lane;
      const int dq = cseg / hs;
      const int sj = s + dq;  // the candidate's sequence and segment
      const int hj = cseg - dq * hs;
      const int Lj = sj < B ? max(s_len[sj], 0) : 0;
      const int nj = (Lj + 15) >> 4;
      const int usj = seg_units(Lj);
      const int uinj = lane == 0 ? uin : 0;
      const int tdj = lane == 0 ? tdone : 0;
      const int avj = max(usj - uinj, 0);
      const int kvhj = nsub == 1 ? hj : hj / nsub;
      const int subj = hj - kvhj * nsub;
      const int Uj = wave_excl_scan3(avj, 0, 0).x;  // units before the candidate
      const int kj = max(0, min(avj, u_hi - u - Uj));
      const int t1j = min((uinj + kj) * unit, nj);
      const int tbj = uinj * unit + tdj;
      const int cntj = kj > 0 ? t1j - tbj : 0;
      const int nhj = cntj > 0 ? min(GMAX, g - subj * GMAX) : 0;
      const unsigned long long ne = __ballot(cntj > 0);
      const int pidx = __builtin_popcountll(ne & ((1ull << lane) - 1));
      const int3 ex = wave_excl_scan3(cntj, nhj, 0);
      const int KBj = ex.x, QRj = ex.y;
      const bool fit = KBj < kChunkTiles && QRj + nhj <= kChunkQRows && pidx < kChunkPieces;
      const unsigned long long nofit = __ballot(cntj > 0 && !fit);
      const int lim = nofit ? __builtin_ctzll(nofit) : 64;
      const bool take = cntj > 0 && lane < lim;
      const int ctk = take ? min(cntj, kChunkTiles - KBj) : 0;
      const unsigned long long tk = __ballot(take);
      npc = __builtin_popcountll(tk);
      if (take) {
        const bool whole = uinj == 0 && kj == usj;
        const bool firstj = first && pidx == 0;
        int flags = (whole ? kWhole : 0) | (tbj + ctk == t1j ? kEnds : 0) | (firstj ? 0 : kLastSlot) |
                    (tdj == 0 ? kStarts : 0) | (subj == 0 ? kWriter : 0);
        int np = 1;
        if (uinj == 0) {
          flags |= kFirstUnit;
          if (!whole) {
            // the wave holding the segment's last unit
            const int w_last = (int)(((long long)(u + Uj + usj) * W - 1) / qt);
            np = w_last - w + 1;
          }
        }
        Piece& pc = pcs[pidx];
        pc.nt = ctk;
        pc.qrow = QRj;
        pc.nh = nhj;
        pc.row0 = sj * Hq + kvhj * g + subj * GMAX;
        pc.seg = sj * hs + hj;
        pc.np = np;
        pc.flags = flags;
        pc.bad = 0;
        pc.bto = tbj - KBj;  // chunk tile kk is the sequence's 16-slot tile bto + kk
        pc.srow = sj * maxb;
        pc.kvh = kvhj;
        pc.rb = Lj - 1 - (tbj - KBj) * 16;
        pc.kb = KBj;
        pc.nrow = sj * Hkv + kvhj;
        for (int r = 0; r < nhj; ++r) s_qown[wave][QRj + r] = (unsigned char)pidx;
      }
      // Advance the walker: into the piece cut by the tile limit, else to
      // the first candidate not taken (or past all 64).
      const int lt = tk ? 63 - __builtin_clzll(tk) : -1;  // last taken
      const bool cut = lt >= 0 && __builtin_amdgcn_readlane(ctk, lt) < __builtin_amdgcn_readlane(cntj, lt);
      if (npc == 0 && lim == 0) break;  // (cannot happen: a first non-empty candidate always fits)
      if (lt >= 0) {
        ntc = __builtin_amdgcn_readlane(KBj + ctk, lt);
        nqr = __builtin_amdgcn_readlane(QRj + nhj, lt);
      } else {
        ntc = nqr = 0;
      }
      const int c = cut ? lt : lim;
      const int Uc = c < 64 ? __builtin_amdgcn_readlane(Uj, c) : __builtin_amdgcn_readlane(Uj + avj, 63);
      if (cut) {
        tdone = __builtin_amdgcn_readlane(tdj + ctk, lt);
        uin = __builtin_amdgcn_readlane(uinj, lt);
        first = first && __builtin_amdgcn_readlane(pidx, lt) == 0;
      } else {
        tdone = 0;
        uin = c == 0 ? uin : 0;
        first = first && npc == 0;
      }
      const int cs = hsub + c;
      s = uni(s + cs / hs);
      hsub = uni(cs - (cs / hs) * hs);
      uin = uni(uin);
      tdone = uni(tdone);
      u = uni(u + Uc);
      npc = uni(npc);
      ntc = uni(ntc);
      nqr = uni(nqr);
    }
    if (npc == 0) {
      if (s >= B) break;  // (cannot happen: units remain, so sequences do)
      continue;           // 64 candidates without positions
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // The piece of every chunk tile, written piece by piece by the whole
    // wave (the pieces' first tiles are in the lanes that planned them).
    for (int p = 0; p < npc; ++p) {
      const int kb0 = uni(pcs[p].kb), n0 = uni(pcs[p].nt);
      for (int t = lane; t < n0; t += 64) s_own[wave][kb0 + t] = (unsigned char)p;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- The first chunk's first two tiles, from the entries loaded before
    // planning: the chunk's tile 0 is tb0, its tile 1 is tb0 + 1 when the
    // first piece has two tiles (tile 0 again when the chunk has one tile);
    // otherwise the pipeline's prologue issues them as usual.  Descriptors
    // are the ones staging computes below (an invalid id reads block 0,
    // never dereferenced past the pool; staging marks the piece bad).
    bool preloaded = false;
    if (first_chunk) {
      first_chunk = false;
      const int nt0 = uni(pcs[0].nt);
      if (nt0 >= 2 || ntc == 1) {
        const int tb1 = ntc == 1 ? tb0 : tb0 + 1;
        int idA = __builtin_amdgcn_readlane(pre_id, 0);
        int idB = __builtin_amdgcn_readlane(pre_id, ntc == 1 ? 0 : 1);
        const bool okA = idA >= 0 && idA < num_blocks, okB = idB >= 0 && idB < num_blocks;
        const bool newA = kFuse && okA && tb0 == nt0_seq - 1, newB = kFuse && okB && tb1 == nt0_seq - 1;
        idA = okA ? idA : 0;
        idB = okB ? idB : 0;
        const unsigned mask = (1u << lm) - 1u;
        const unsigned rowA = ((unsigned)(idA * Hkv + kvh0) << lm) | ((unsigned)tb0 & mask);
        const unsigned rowB = ((unsigned)(idB * Hkv + kvh0) << lm) | ((unsigned)tb1 & mask);
        const size_t nrow0 = ((size_t)s0 * Hkv + kvh0) * ROWB;
        const int rmA = min(15, L0 - 1 - 16 * tb0), rmB = min(15, L0 - 1 - 16 * tb1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kFuse)
          T::load_sel(kp + (size_t)rowA * (16 * ROWB), vp + (size_t)rowA * (16 * ROWB), kn + nrow0, vn + nrow0, newA,
                      grp, col, rmA, kA, vA);
        else
          T::load(kp + (size_t)rowA * (16 * ROWB), vp + (size_t)rowA * (16 * ROWB), grp, col, rmA, kA, vA);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kFuse)
          T::load_sel(kp + (size_t)rowB * (16 * ROWB), vp + (size_t)rowB * (16 * ROWB), kn + nrow0, vn + nrow0, newB,
                      grp, col, rmB, kB, vB);
        else
          T::load(kp + (size_t)rowB * (16 * ROWB), vp + (size_t)rowB * (16 * ROWB), grp, col, rmB, kB, vB);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        preloaded = true;
      }
    }

    // ---- Stage: block ids and query rows, all loads in flight together.
    constexpr int ND = kChunkTiles / 64;
    constexpr int NQ = (kChunkQRows * QCH + 63) / 64;
    int ids[ND], dpc[ND];
    uint4 qv[NQ];
    int qrw[NQ];
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int kk = lane + 64 * i;
      dpc[i] = 0;
      ids[i] = 0;
      if (kk < ntc) {
        const int p = s_own[wave][kk];
        dpc[i] = p;
        // (kk is inside piece p by construction; the check keeps a planning
        // error from reading outside the sequence's table row)
        if (kk - pcs[p].kb < pcs[p].nt) ids[i] = bt[pcs[p].srow + ((pcs[p].bto + kk) >> lm)];
        else ids[i] = -1;
      }
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int c = lane + 64 * i;
      const int r = c / QCH, cc = c - r * QCH;
      qv[i] = make_uint4(0, 0, 0, 0);
      qrw[i] = -1;
      if (r < nqr) {
        const int p = s_qown[wave][r];
        qrw[i] = r;
        if (r - pcs[p].qrow < pcs[p].nh)
          qv[i] = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(q) +
                                                  (size_t)(pcs[p].row0 + r - pcs[p].qrow) * ROWB + cc * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < ND; ++i) {
      const int kk = lane + 64 * i;
      if (kk < ntc) {
        const Piece& pc = pcs[dpc[i]];
        int id = ids[i];
        const bool ok = id >= 0 && id < num_blocks;
        if (!ok) {
          id = 0;
          atomicOr(&s_pc[wave][dpc[i]].bad, 1);
        }
        const unsigned row = ((unsigned)(id * Hkv + pc.kvh) << lm) | (unsigned)((pc.bto + kk) & ((1 << lm) - 1));
        // the tile holding the sequence's last position (its new token, when fused)
        const bool is_new = kFuse && ok && pc.rb - 16 * kk <= 15;
        desc[kk] = (row << 5) | (is_new ? (unsigned)kDescNew : 0u) | (unsigned)min(15, pc.rb - 16 * kk);
        if constexpr (kFuse) s_nrow[wave][kk] = (unsigned)pc.nrow * ROWB;
      }
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int c = lane + 64 * i;
      if (qrw[i] >= 0) *reinterpret_cast<uint4*>(&sq[qrw[i]][(c - qrw[i] * QCH) * 8]) = qv[i];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- One pipeline through the chunk.
    int cp = 0;                    // piece being consumed
    int cp_end = uni(pcs[0].nt);   // its end (chunk tile index)
    int cp_nh = uni(pcs[0].nh);
    int cp_qrow = uni(pcs[0].qrow);
    if (uni(pcs[0].flags) & kStarts) reset();
    bad |= uni(pcs[0].bad) != 0;
    const uint16_t* qsrc = &sq[col < cp_nh ? cp_qrow + col : kChunkQRows][grp * 8];
    pipeline(
        ntc, kA, vA, kB, vB,
        [&](int kk, uint4(&kr)[KS], VVec(&vr)[4]) {
          const unsigned d = (unsigned)uni((int)desc[kk]);
          const size_t off = (size_t)(d >> 5) * (16 * ROWB);
          if constexpr (kFuse) {
            const size_t noff = (unsigned)uni((int)s_nrow[wave][kk]);
            T::load_sel(kp + off, vp + off, kn + noff, vn + noff, (d & kDescNew) != 0, grp, col, (int)(d & 15), kr,
                        vr);
          } else {
            T::load(kp + off, vp + off, grp, col, (int)(d & 15), kr, vr);
          }
        },
        [&](int kk, const uint4(&kr)[KS], const VVec(&vr)[4], bool valid) {
          asm volatile("" ::: "memory");
          const unsigned dk = (unsigned)uni((int)desc[kk]);
          const int lim = valid ? (int)((dk & 15) + 1) : 0;
          T::consume(kr, vr, qsrc, 4 * grp, lim, qscale, x16, x32, m_run, l_run, acc);
          if (kFuse && (dk & kDescNew) && (uni(pcs[cp].flags) & kWriter)) {
            // the fused write: the new token's rows into their pool slot
            // (one KV head's segment of query sub-group 0 writes them)
            const size_t off = (size_t)(dk >> 5) * (16 * ROWB);
            T::store_new(const_cast<char*>(kp) + off, const_cast<char*>(vp) + off, grp, col, (int)(dk & 15), kr, vr);
          }
          if (valid && kk + 1 == cp_end) {
            const int flags = uni(pcs[cp].flags);
            if (flags & kEnds) {
              // The piece is complete: final rows, or this wave's piece.
              const int nh = cp_nh;
              const size_t row0 = (size_t)uni(pcs[cp].row0);
              const float l_tot = xchg(xchg(l_run, x16, AddOp()), x32, AddOp());
              const float inv = bad ? __builtin_nanf("") : 1.f / l_tot;
              const int slot = 2 * w + ((flags & kLastSlot) ? 1 : 0);
              if (col < nh) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                  const int d0 = DPL * (4 * grp + jj);
                  float f[DPL];
#pragma unroll
                  for (int uu = 0; uu < DPL; ++uu) f[uu] = acc[uu][jj] * inv;
                  if (flags & kWhole) {
                    store_row<DT, DPL>(out, (row0 + col) * D + d0, f);
                  } else {
                    float* po = pc_o + ((size_t)slot * GMAX + col) * D + d0;
#pragma unroll
                    for (int uu = 0; uu < DPL; uu += 4)
                      *reinterpret_cast<float4*>(po + uu) = make_float4(f[uu], f[uu + 1], f[uu + 2], f[uu + 3]);
                  }
                }
                if (!(flags & kWhole) && grp == 0) {
                  pc_m[(size_t)slot * GMAX + col] = bad ? __builtin_nanf("") : m_run;
                  pc_l[(size_t)slot * GMAX + col] = bad ? __builtin_nanf("") : l_tot;
                }
              }
              if ((flags & kFirstUnit) && lane == 0) info[uni(pcs[cp].seg)] = make_int2(slot, uni(pcs[cp].np));
              reset();
            }
            if (++cp < npc) {
              cp_end += uni(pcs[cp].nt);
              cp_nh = uni(pcs[cp].nh);
              cp_qrow = uni(pcs[cp].qrow);
              bad |= uni(pcs[cp].bad) != 0;
              qsrc = &sq[col < cp_nh ? cp_qrow + col : kChunkQRows][grp * 8];
            }
          }
        },
        preloaded);
  }
}

// Merge of a cut segment's pieces (one workgroup per segment; segments
// written whole, and sequences without positions, are already final).
template <int DT, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_stream_reduce(void* __restrict__ out, const float* __restrict__ pc_o,
                                                           const float* __restrict__ pc_m,
                                                           const float* __restrict__ pc_l,
                                                           const int2* __restrict__ info, int Hq, int g, int nsub) {
  const int hsub = blockIdx.x;
  const int s = blockIdx.y;
  // every segment's record is written by the stream kernel (count 0 for
  // sequences without positions, 1 for segments it wrote whole)
  const int2 inf = info[(size_t)s * gridDim.x + hsub];
  const int np = inf.y;
  if (np <= 1) return;
  const int w0 = inf.x >> 1;
  const int kvh = hsub / nsub;
  const int sub = hsub - kvh * nsub;
  const int nh = min(GMAX, g - sub * GMAX);
  const size_t row0 = (size_t)s * Hq + kvh * g + sub * GMAX;
  for (int c = threadIdx.x; c < nh * (D / 4); c += 256) {
    const int h = c / (D / 4);
    const int d = (c - h * (D / 4)) * 4;
    float M = kNegInf, den = 0.f;
    float4 num = make_float4(0.f, 0.f, 0.f, 0.f);
    // pieces in batches of 8: all loads of a batch in flight together
    for (int i0 = 0; i0 < np; i0 += 8) {
      float mv[8], lv[8];
      float4 ov[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        mv[j] = kNegInf;
        lv[j] = 0.f;
        ov[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (i0 + j < np) {
          const size_t slot = i0 + j == 0 ? (size_t)inf.x : 2 * (size_t)(w0 + i0 + j);
          mv[j] = pc_m[slot * GMAX + h];
          lv[j] = pc_l[slot * GMAX + h];
          ov[j] = *reinterpret_cast<const float4*>(pc_o + (slot * GMAX + h) * D + d);
        }
      }
      float Mn = M;
#pragma unroll
      for (int j = 0; j < 8; ++j) Mn = fmaxf(Mn, mv[j]);
      const float a = fast_exp2(M - Mn);  // 0 on the first batch (M = -inf)
      den *= a;
      num = make_float4(num.x * a, num.y * a, num.z * a, num.w * a);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float b = lv[j] * fast_exp2(mv[j] - Mn);  // 0 past the last piece
        den += b;
        num = make_float4(num.x + b * ov[j].x, num.y + b * ov[j].y, num.z + b * ov[j].z, num.w + b * ov[j].w);
      }
      M = Mn;
    }
    const float inv = 1.f / den;
    const float f[4] = {num.x * inv, num.y * inv, num.z * inv, num.w * inv};
    store_row<DT, 4>(out, (row0 + h) * D + d, f);
  }
}

// The main kernel's launch carries the caller's timing events (if any).
#define EV(a) static_cast<hipEvent_t>((a).ev_start), static_cast<hipEvent_t>((a).ev_stop)

template <int DT, int D, int GMAX>
void launch(const DecodeArgs& a, hipStream_t st) {
  if (a.stream) {
    if (a.kn)
      hipExtLaunchKernelGGL((decode_stream<DT, D, GMAX, true>), dim3(a.grid), dim3(256), 0, st, EV(a), 0, a.out, a.q, a.kp,
                         a.vp, a.bt, a.cl, a.ws_o, a.ws_m, a.ws_l, a.info, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks,
                         a.maxb, a.max_ctx, a.qscale, a.unit, a.lm, a.kn, a.vn);
    else
      hipExtLaunchKernelGGL((decode_stream<DT, D, GMAX, false>), dim3(a.grid), dim3(256), 0, st, EV(a), 0, a.out, a.q, a.kp,
                         a.vp, a.bt, a.cl, a.ws_o, a.ws_m, a.ws_l, a.info, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks,
                         a.maxb, a.max_ctx, a.qscale, a.unit, a.lm, a.kn, a.vn);
    return;
  }
  const unsigned grid = (unsigned)a.entries * a.Hkv * a.nsub * a.B;
  if (a.wave_part)
    hipExtLaunchKernelGGL((decode_part_wave<DT, D, GMAX>), dim3(grid), dim3(256), 0, st, EV(a), 0, a.out, a.q, a.kp, a.vp, a.bt,
                       a.cl, a.ws_o, a.ws_m, a.ws_l, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb, a.max_ctx,
                       a.qscale, a.psize, a.entries, a.lm);
  else
    hipExtLaunchKernelGGL((decode_part_mfma<DT, D, GMAX>), dim3(grid), dim3(256), 0, st, EV(a), 0, a.out, a.q, a.kp, a.vp, a.bt,
                       a.cl, a.ws_o, a.ws_m, a.ws_l, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb, a.max_ctx,
                       a.qscale, a.psize, a.entries, a.lm);
}

template <int DT, int D, int GMAX>
void launch_merge(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_stream_reduce<DT, D, GMAX>), dim3(a.Hkv * a.nsub, a.B), dim3(256), 0, st, a.out, a.ws_o,
                     a.ws_m, a.ws_l, a.info, a.Hq, a.g, a.nsub);
}

template <int DT, int D, bool kMerge>
void launch_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.gmax) {
    case 4: kMerge ? launch_merge<DT, D, 4>(a, st) : launch<DT, D, 4>(a, st); break;
    case 8: kMerge ? launch_merge<DT, D, 8>(a, st) : launch<DT, D, 8>(a, st); break;
    default: kMerge ? launch_merge<DT, D, 16>(a, st) : launch<DT, D, 16>(a, st); break;
  }
}

template <int DT, bool kMerge>
void launch_d(const DecodeArgs& a, hipStream_t st) {
  if (a.D == 64)
    launch_g<DT, 64, kMerge>(a, st);
  else
    launch_g<DT, 128, kMerge>(a, st);
}

}  // namespace

void launch_decode_mfma(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == PA_FP16)
    launch_d<PA_FP16, false>(a, st);
  else
    launch_d<PA_BF16, false>(a, st);
}

void launch_decode_stream_reduce(const DecodeArgs& a, hipStream_t st) {
  if (a.dtype == PA_FP16)
    launch_d<PA_FP16, true>(a, st);
  else
    launch_d<PA_BF16, true>(a, st);
}

}  // namespace pa
