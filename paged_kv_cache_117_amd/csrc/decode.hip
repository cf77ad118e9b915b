// pa_decode: single-query paged decode attention + log-sum-exp merge.
//
// What is computed: for each sequence s (length L) and query head h, ordinary
// softmax attention of q[s][h] over the L valid K/V rows of KV head h/g,
// where position t is found through the block table at block t/bs, slot t%bs
// (bs = 16 << lm; the kernels walk 16-slot tiles, 2^lm of them per block)
// (PagedAttention and vLLM: Paging the KV Cache Like an OS, "Step 5";
// PagedAttention (tensortonic), "5. Reading the Cache During Attention").
//
// Work decomposition: one work item = (sequence, KV head, query sub-group,
// partition of `psize` positions).  A work item walks its blocks in logical
// order keeping a running max m, running sum l and an accumulator (online
// softmax; PagedAttention (tensortonic), "10. How PagedAttention Fits with
// FlashAttention").  Scores are kept in the base-2 domain (q prescaled by
// scale*log2(e)), so every exponential is one v_exp_f32.  A sequence that
// fits one partition writes `out` directly; otherwise each partition writes
// (m_p, l_p, o_p = acc_p / l_p) to the workspace and the reduce kernel forms
//   M = max_p m_p,  w_p = l_p 2^(m_p - M),  out = sum_p w_p o_p / sum_p w_p,
// the weighting that makes per-partition results add up to the softmax over
// all positions (same page, section 5: per-page normalise-and-add is wrong).
//
// The arithmetic order depends only on logical positions (block j of the
// sequence, slot within the block), never on physical block ids, so any
// placement of the same logical cache gives bit-identical results.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_kernels.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// VALU partition kernel: one wavefront per work item.
//
// Tile mapping: a K or V tile (16 slots x D elements, 4 KiB for 16-bit D=128)
// is read with 16-byte loads; a token row of ROWB bytes is covered by
// LPR = ROWB/16 consecutive lanes, so lane (r, c) = (lane / LPR, lane % LPR)
// holds dims [c*EPL, c*EPL+EPL) of token row r of each RPI-row slice.  The
// NI loads of a tile together read it exactly once, contiguously.
// ---------------------------------------------------------------------------
template <int DT, int D, int GMAX>
__global__ __launch_bounds__(64) void decode_part_valu(void* __restrict__ out, const void* __restrict__ q,
                                                      const char* __restrict__ kp, const char* __restrict__ vp,
                                                      const int32_t* __restrict__ bt, const int32_t* __restrict__ cl,
                                                      float* __restrict__ ws_o, float* __restrict__ ws_m,
                                                      float* __restrict__ ws_l, int B, int Hq, int Hkv, int g,
                                                      int nsub, int num_blocks, int maxb, int max_ctx, float qscale,
                                                      int psize, int P, int lm, const int32_t* __restrict__ qst,
                                                      int nseq, int max_q) {
  constexpr int ES = Elem<DT>::kBytes;
  constexpr int ROWB = D * ES;
  constexpr int LPR = ROWB / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int NI = 16 / RPI;
  constexpr int EPL = 16 / ES;
  const int lane = threadIdx.x;
  const int r = lane / LPR;
  const int c = lane % LPR;
  // 1-D grid: KV head / sub-group fastest, then sequence, then partition, so
  // the round-robin deal of workgroups to the 8 XCDs balances the work.
  // With `qst` (several query tokens per sequence, pa_prefill): s is a
  // query token, row s of q and out, of the sequence `seq` whose rows
  // qst[seq] .. qst[seq+1]-1 hold it; at position L_seq - T + (s - qst[seq])
  // it sees that many positions plus one, through its sequence's table.
  const int hs = Hkv * nsub;
  const int idx = blockIdx.x;
  const int hsub = idx % hs;
  const int s = (idx / hs) % B;
  const int p = idx / (hs * B);
  const int kvh = hsub / nsub;
  const int sub = hsub - kvh * nsub;
  int seq = s, L;
  bool bad_len;
  if (qst) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (qst[mid] <= s)
        lo = mid;
      else
        hi = mid - 1;
    }
    seq = lo;
    const int q0 = qst[seq], q1 = qst[seq + 1], Ls = cl[seq], T = q1 - q0;
    bad_len = s < q0 || s >= q1 || q0 < 0 || q1 > B || T > Ls || (int64_t)Ls > ((int64_t)maxb << (lm + 4)) ||
              T > max_q;
    L = bad_len ? 0 : Ls - T + (s - q0) + 1;
  } else {
    L = cl[s];
    bad_len = L < 0 || L > max_ctx;
    if (bad_len) L = 0;
  }
  const int hbase = kvh * g + sub * GMAX;
  const int nh = min(GMAX, g - sub * GMAX);
  if (L == 0) {
    if (p == 0) {
      const float fill = bad_len ? __builtin_nanf("") : 0.f;
      for (int i = lane; i < nh * D; i += 64) store_elem<DT>(out, ((size_t)s * Hq + hbase) * D + i, fill);
    }
    return;
  }
  const int nparts = (L + psize - 1) / psize;
  if (p >= nparts) return;

  float qf[GMAX][EPL];
  const char* qrow = reinterpret_cast<const char*>(q) + ((size_t)s * Hq + hbase) * ROWB + c * 16;
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h < nh) {
      unpack16<DT>(*reinterpret_cast<const uint4*>(qrow + h * ROWB), qf[h]);
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] *= qscale;
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qf[h][e] = 0.f;
    }
  }

  float m[GMAX], lsum[GMAX], acc[GMAX][EPL];
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    m[h] = kNegInf;
    lsum[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }

  const int nblk = (L + 15) / 16;
  const int b0 = p * (psize / 16);
  const int b1 = min(b0 + psize / 16, nblk);
  const int32_t* btrow = bt + (size_t)seq * maxb;
  const size_t lane_off = (size_t)r * ROWB + c * 16;
  bool bad = false;

  // `blk` counts 16-slot tiles; a block of 16 << lm slots holds 1 << lm of
  // them, so tile blk is slots [16 (blk mod 2^lm), +16) of table entry blk >> lm.
  for (int blk = b0; blk < b1; ++blk) {
    const int phys = btrow[blk >> lm];
    if (phys < 0 || phys >= num_blocks) {
      bad = true;
      break;
    }
    const size_t row = ((((size_t)phys * Hkv + kvh) << lm) | (size_t)(blk & ((1 << lm) - 1)));
    const char* kb = kp + row * (16 * ROWB) + lane_off;
    const char* vb = vp + row * (16 * ROWB) + lane_off;
    uint4 kr[NI], vr[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) kr[i] = *reinterpret_cast<const uint4*>(kb + i * RPI * ROWB);
#pragma unroll
    for (int i = 0; i < NI; ++i) vr[i] = *reinterpret_cast<const uint4*>(vb + i * RPI * ROWB);

    float sc[NI][GMAX];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPL];
      unpack16<DT>(kr[i], kf);
#pragma unroll
      for (int h = 0; h < GMAX; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(qf[h][e], kf[e], a);
        sc[i][h] = a;
      }
    }
    // sum the partial dot products of one token row (lanes sharing r)
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int h = 0; h < GMAX; ++h) sc[i][h] += __shfl_xor(sc[i][h], off);

    const bool full = (blk + 1) * 16 <= L;
    if (!full) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (blk * 16 + i * RPI + r >= L) {
#pragma unroll
          for (int h = 0; h < GMAX; ++h) sc[i][h] = kNegInf;
        }
      }
    }

    float pr[NI][GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      float bm = sc[0][h];
#pragma unroll
      for (int i = 1; i < NI; ++i) bm = fmaxf(bm, sc[i][h]);
#pragma unroll
      for (int off = LPR; off < 64; off <<= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
      const float mn = fmaxf(m[h], bm);
      const float alpha = fast_exp2(m[h] - mn);
      m[h] = mn;
      float ls = lsum[h] * alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        pr[i][h] = fast_exp2(sc[i][h] - mn);
        ls += pr[i][h];
      }
      lsum[h] = ls;
    }

#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      unpack16<DT>(vr[i], vf);
      if (!full && blk * 16 + i * RPI + r >= L) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) vf[e] = 0.f;  // unfilled slots may hold NaN
      }
#pragma unroll
      for (int h = 0; h < GMAX; ++h)
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pr[i][h], vf[e], acc[h][e]);
    }
  }

  // combine the RPI token rows (same dims, different tokens)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
      lsum[h] += __shfl_xor(lsum[h], off);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += __shfl_xor(acc[h][e], off);
    }
  }
  if (r != 0) return;
  const float nan = __builtin_nanf("");
#pragma unroll
  for (int h = 0; h < GMAX; ++h) {
    if (h >= nh) break;
    const float inv = 1.f / lsum[h];
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = bad ? nan : acc[h][e] * inv;
    const size_t row = (size_t)s * Hq + hbase + h;
    if (nparts == 1) {
      *reinterpret_cast<uint4*>(reinterpret_cast<char*>(out) + row * ROWB + c * 16) = pack16<DT>(o);
    } else {
      float* wo = ws_o + (row * P + p) * D + c * EPL;
#pragma unroll
      for (int e = 0; e < EPL; e += 4) *reinterpret_cast<float4*>(wo + e) = make_float4(o[e], o[e + 1], o[e + 2], o[e + 3]);
      if (c == 0) {
        ws_m[row * P + p] = bad ? nan : m[h];
        ws_l[row * P + p] = bad ? nan : lsum[h];
      }
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Reduce: one workgroup per (query head, sequence), one thread per dim.  A
// row holds E entries; entry e is the merge of partitions per*e ..
// per*(e+1)-1 (per = 1: one partition each).
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(D) void decode_reduce(void* __restrict__ out, const int32_t* __restrict__ cl,
                                                   const float* __restrict__ ws_o, const float* __restrict__ ws_m,
                                                   const float* __restrict__ ws_l, int Hq, int max_ctx, int psize,
                                                   int E, int per) {
  const int h = blockIdx.x;
  const int s = blockIdx.y;
  const int d = threadIdx.x;
  const int L = cl[s];
  if (L < 0 || L > max_ctx) return;
  const int nent = ((L + psize - 1) / psize + per - 1) / per;  // this sequence's entries
  if (nent <= 1) return;  // written by the partition kernel
  const size_t base = ((size_t)s * Hq + h) * E;
  float M = kNegInf;
  for (int p = 0; p < nent; ++p) M = fmaxf(M, ws_m[base + p]);
  float num = 0.f, den = 0.f;
  for (int p = 0; p < nent; ++p) {
    const float w = ws_l[base + p] * fast_exp2(ws_m[base + p] - M);
    den += w;
    num = fmaf(w, ws_o[(base + p) * D + d], num);
  }
  store_elem<DT>(out, ((size_t)s * Hq + h) * D + d, num / den);
}

namespace {

template <int DT, int D, int GMAX>
void launch_valu(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.P * a.Hkv * a.nsub * a.B;
  hipExtLaunchKernelGGL((decode_part_valu<DT, D, GMAX>), dim3(grid), dim3(64), 0, st,
                        static_cast<hipEvent_t>(a.ev_start), static_cast<hipEvent_t>(a.ev_stop), 0, a.out, a.q, a.kp, a.vp, a.bt,
                     a.cl, a.ws_o, a.ws_m, a.ws_l, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb, a.max_ctx,
                     a.qscale, a.psize, a.P, a.lm, a.qst, a.nseq, a.max_q);
}

template <int DT, int D>
void launch_valu_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.gmax) {
    case 1: launch_valu<DT, D, 1>(a, st); break;
    case 2: launch_valu<DT, D, 2>(a, st); break;
    case 4: launch_valu<DT, D, 4>(a, st); break;
    default: launch_valu<DT, D, 8>(a, st); break;
  }
}

template <int DT, int D>
void launch_reduce(const DecodeArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((decode_reduce<DT, D>), dim3(a.Hq, a.B), dim3(D), 0, st, a.out, a.cl, a.ws_o, a.ws_m, a.ws_l,
                     a.Hq, a.max_ctx, a.psize, a.entries, a.per_entry);
}

template <int DT>
void launch_valu_d(const DecodeArgs& a, hipStream_t st) {
  if (a.D == 64)
    launch_valu_g<DT, 64>(a, st);
  else
    launch_valu_g<DT, 128>(a, st);
}

template <int DT>
void launch_reduce_d(const DecodeArgs& a, hipStream_t st) {
  if (a.D == 64)
    launch_reduce<DT, 64>(a, st);
  else
    launch_reduce<DT, 128>(a, st);
}

}  // namespace

void launch_decode_valu(const DecodeArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case PA_FP32: launch_valu_d<PA_FP32>(a, st); break;
    case PA_FP16: launch_valu_d<PA_FP16>(a, st); break;
    default: launch_valu_d<PA_BF16>(a, st); break;
  }
}

void launch_decode_reduce(const DecodeArgs& a, hipStream_t st) {
  switch (a.dtype) {
    case PA_FP32: launch_reduce_d<PA_FP32>(a, st); break;
    case PA_FP16: launch_reduce_d<PA_FP16>(a, st); break;
    default: launch_reduce_d<PA_BF16>(a, st); break;
  }
}

}  // namespace pa
