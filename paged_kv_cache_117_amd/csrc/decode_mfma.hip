// pa_decode partition kernel for 16-bit KV (fp16 / bf16) on gfx950.
//
// Same computation as the VALU kernel in decode.hip (online softmax over the
// partition's blocks in logical order, base-2 exponentials, log-sum-exp
// partials), organised for bandwidth:
//
//  * One workgroup of 4 wavefronts per work item (sequence, KV head, query
//    sub-group, partition).  Wave w takes the partition's blocks w, w+4, ...;
//    each wave double-buffers: the K and V tiles of its next block are in
//    flight while it computes the current one.  The four waves' (m, l, acc)
//    are merged through LDS at the end.
//  * Scores for the GQA query group x the 16-slot key tile are one MFMA
//    chain: v_mfma_f32_16x16x32_{bf16,f16} with the K tile as the A operand
//    (lane (G, c) loads 16 bytes of token c at dims 32k+8G, exactly the
//    operand layout, so K goes from HBM to the matrix core with no shuffles)
//    and the query group, padded to 16 heads with zeros, as the B operand.
//    Lane (G, c) receives S[token 4G+j][head c], j = 0..3.
//  * PV stays on the VALU: lane (G, c) loads dims [c*D/16, +D/16) of tokens
//    4G..4G+3 of the V tile and needs the weights of those tokens for every
//    head of the group; they sit in the same 16-lane row (lane h holds head
//    h).  Weights are packed in pairs of tokens to the KV type and delivered
//    by one DPP row_newbcast per (token pair, head); v_dot2_f32 multiplies a
//    pair of tokens' V values (interleaved by v_perm_b32) and accumulates in
//    fp32 -- half the VALU instructions of per-token FMAs.
//  * The accumulator is rescaled only when some head's running max grows
//    (a wave-uniform branch); exponentials of unchanged maxima are exactly 1.
//
// Unfilled slots of a final block are masked to -inf before the max and
// their V values are replaced by zero, so NaN/Inf garbage there never
// reaches the result.  Block ids outside [0, num_blocks) are never
// dereferenced: the work item produces NaN instead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "decode_kernels.h"
#include "pa_device.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr float kNegInf = -__builtin_inff();

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

// Lane N of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x150 + N, 0xF, 0xF, false));
}
template <int N>
__device__ __forceinline__ uint32_t row_bcast_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x150 + N, 0xF, 0xF, false);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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

// c + v.lo * p.lo + v.hi * p.hi in fp32 (v_dot2_f32_bf16 / v_dot2_f32_f16).
template <int DT>
__device__ __forceinline__ float dot2(uint32_t v, uint32_t p, float c) {
  if constexpr (DT == PA_BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v), __builtin_bit_cast(bf16x2, p), c, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, v), __builtin_bit_cast(f16x2, p), c, false);
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

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

template <int DT, int DPL>
__device__ __forceinline__ void unpack_v(const typename std::conditional<DPL == 8, uint4, uint2>::type& v,
                                         float* f) {
  if constexpr (DPL == 8) {
    unpack16<DT>(v, f);
  } else {
    const uint32_t w[2] = {v.x, v.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (DT == PA_BF16) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
      } else {
        f[2 * i] = fp16_lo(w[i]);
        f[2 * i + 1] = fp16_hi(w[i]);
      }
    }
  }
}

template <int DT, int D, int GMAX>
__global__ __launch_bounds__(256) void decode_part_mfma(void* __restrict__ out, const void* __restrict__ q,
                                                       const char* __restrict__ kp, const char* __restrict__ vp,
                                                       const int32_t* __restrict__ bt, const int32_t* __restrict__ cl,
                                                       float* __restrict__ ws_o, float* __restrict__ ws_m,
                                                       float* __restrict__ ws_l, int B, int Hq, int Hkv, int g,
                                                       int nsub, int num_blocks, int maxb, int max_ctx, float qscale,
                                                       int psize, int P) {
  constexpr int ROWB = D * 2;  // bytes of one token row of one head
  constexpr int KS = D / 32;   // MFMA k-steps over the head dim
  constexpr int DPL = D / 16;  // dims per lane in the PV step
  using VVec = typename std::conditional<DPL == 8, uint4, uint2>::type;

  __shared__ float s_m[kWaves][16];
  __shared__ float s_l[kWaves][16];
  __shared__ float s_acc[kWaves][GMAX][D];
  __shared__ int s_bad[kWaves];

  const int tid = threadIdx.x;
  // wave-uniform: keep it (and everything derived from it) in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int32_t* btrow = bt + (size_t)s * maxb;

  // The q operand does not depend on the context length: its loads go out
  // before the length arrives.  B operand: lane (G, c) holds
  // q[head c][dims 32k + 8G .. +8]; heads >= nh are zero.
  uint4 qop[KS];
  {
    const char* qrow = reinterpret_cast<const char*>(q) + ((size_t)s * Hq + hbase) * ROWB + grp * 16;
#pragma unroll
    for (int k = 0; k < KS; ++k)
      qop[k] = col < nh ? *reinterpret_cast<const uint4*>(qrow + (size_t)col * ROWB + k * 64) : make_uint4(0, 0, 0, 0);
  }

  int L = cl[s];
  const bool bad_len = L < 0 || L > max_ctx;
  if (bad_len) L = 0;
  const int nparts = (L + psize - 1) / psize;
  if (L == 0) {
    if (rank == 0) {
      const float fill = bad_len ? __builtin_nanf("") : 0.f;
      for (int i = tid; i < nh * D; i += 256) store_elem<DT>(out, ((size_t)s * Hq + hbase) * D + i, fill);
    }
    return;
  }
  if (rank >= nparts) return;
  const int p = nparts - 1 - rank;

  const int nblk = (L + 15) / 16;
  const int b0 = p * (psize / 16);
  const int b1 = min(b0 + psize / 16, nblk);
  const int nmine = b1 - b0 > wave ? (b1 - b0 - wave + kWaves - 1) / kWaves : 0;
  const size_t blk_stride = (size_t)Hkv * 16 * ROWB;
  const size_t head_off = (size_t)kvh * 16 * ROWB;
  const int k_lane = col * ROWB + grp * 16;          // + k * 64
  const int v_lane = grp * 4 * ROWB + col * DPL * 2;  // + i * ROWB

  float m_run = kNegInf;  // running max of head `col`, base 2
  float l_run = 0.f;      // running sum over this lane's tokens
  float acc[GMAX][DPL];
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = 0.f;
  bool bad = false;

  // Lane i holds the physical id of this wave's i-th block (at most 64: the
  // host sends partitions longer than 4096 positions to the VALU kernel).
  if (nmine > 0) {
    const int cnt = nmine;
    constexpr int chunk = 0;
    int myid = 0;
    if (lane < cnt) myid = btrow[b0 + wave + lane * kWaves];
    const bool ok = lane >= cnt || (myid >= 0 && myid < num_blocks);
    if (!__all(ok)) bad = true;
    if (!(myid >= 0 && myid < num_blocks)) myid = 0;  // never dereference a bad id

    uint4 kA[KS], kB[KS];
    VVec vA[4], vB[4];

    auto issue = [&](int j, uint4(&kr)[KS], VVec(&vr)[4]) {
      const int phys = __builtin_amdgcn_readlane(myid, j);
      const char* kb = kp + (size_t)phys * blk_stride + head_off;
      const char* vb = vp + (size_t)phys * blk_stride + head_off;
#pragma unroll
      for (int k = 0; k < KS; ++k) kr[k] = *reinterpret_cast<const uint4*>(kb + k_lane + k * 64);
#pragma unroll
      for (int i = 0; i < 4; ++i) vr[i] = *reinterpret_cast<const VVec*>(vb + v_lane + i * ROWB);
    };

    // One tile: scores (MFMA), online-softmax update, PV (VALU).  Straight-
    // line code (branches here make the compiler duplicate the accumulator):
    // slots at or past `lim` (the unfilled end of a final block, or every
    // slot of a padding step of the pipeline, `valid` false) get score -inf
    // and their packed V words are zeroed, so garbage there cannot leak.
    auto consume = [&](int j, const uint4(&kr)[KS], const VVec(&vr)[4], bool valid) {
      const int blk = b0 + wave + (chunk + j) * kWaves;
      const int lim = valid ? L : 0;
      const int tok0 = blk * 16 + grp * 4;  // first token of this lane's group
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KS; ++k) sacc = mfma_qk<DT>(kr[k], qop[k], sacc);
      float sv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) sv[jj] = tok0 + jj < lim ? sacc[jj] * qscale : kNegInf;
      float bm = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      bm = xchg(bm, x16, MaxOp());
      bm = xchg(bm, x32, MaxOp());
      // Rescale by 2^(m_old - m_new): exactly 1 when the max did not grow.
      const float mn = fmaxf(m_run, bm);
      const float alpha = fast_exp2(m_run - mn);
      m_run = mn;
      l_run *= alpha;
      static_for<GMAX>([&](auto hc) {
        constexpr int h = decltype(hc)::value;
        const float a = row_bcast<h>(alpha);
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[h][e] *= a;
      });
      float pv[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) pv[jj] = fast_exp2(sv[jj] - m_run);
      l_run += (pv[0] + pv[1]) + (pv[2] + pv[3]);
      // PV on packed pairs: tokens (4G, 4G+1) and (4G+2, 4G+3).  Lane h of
      // the row packs its two weights into one 16-bit pair; v_perm_b32 puts
      // the same dim of the two tokens side by side; v_dot2 accumulates the
      // pair in fp32.  Masked tokens have their V words zeroed.
      constexpr int NW = DPL / 2;  // 32-bit words per token row in this lane
      uint32_t vw[4][NW];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t keep = tok0 + i < lim ? 0xffffffffu : 0u;
        vw[i][0] = vr[i].x & keep;
        vw[i][1] = vr[i].y & keep;
        if constexpr (NW == 4) {
          vw[i][2] = vr[i].z & keep;
          vw[i][3] = vr[i].w & keep;
        }
      }
      const uint32_t pk[2] = {pack_pair<DT>(pv[0], pv[1]), pack_pair<DT>(pv[2], pv[3])};
#pragma unroll
      for (int j2 = 0; j2 < 2; ++j2) {
        uint32_t lo[NW], hi[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          lo[w] = __builtin_amdgcn_perm(vw[2 * j2 + 1][w], vw[2 * j2][w], 0x05040100u);
          hi[w] = __builtin_amdgcn_perm(vw[2 * j2 + 1][w], vw[2 * j2][w], 0x07060302u);
        }
        static_for<GMAX>([&](auto hc) {
          constexpr int h = decltype(hc)::value;
          const uint32_t ph = row_bcast_u<h>(pk[j2]);
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            acc[h][2 * w] = dot2<DT>(lo[w], ph, acc[h][2 * w]);
            acc[h][2 * w + 1] = dot2<DT>(hi[w], ph, acc[h][2 * w + 1]);
          }
        });
      }
    };

    // Two tiles in flight per wave.  Every issue is unconditional (indices
    // past the end re-read the last tile, an L2 hit) so the loads stay in a
    // fixed order and each consume waits only for its own tile.
    const int last = cnt - 1;
    issue(0, kA, vA);
    issue(min(1, last), kB, vB);
    for (int j = 0; j < cnt; j += 2) {
      consume(j, kA, vA, true);
      issue(min(j + 2, last), kA, vA);
      consume(j + 1, kB, vB, j + 1 < cnt);
      issue(min(j + 3, last), kB, vB);
    }
  }

  // Sum the four token groups of the wave (same head / dims, other tokens).
  l_run = xchg(xchg(l_run, x16, AddOp()), x32, AddOp());
#pragma unroll
  for (int h = 0; h < GMAX; ++h)
#pragma unroll
    for (int e = 0; e < DPL; ++e) acc[h][e] = xchg(xchg(acc[h][e], x16, AddOp()), x32, AddOp());
  if (grp == 0) {
    s_m[wave][col] = m_run;
    s_l[wave][col] = l_run;
#pragma unroll
    for (int h = 0; h < GMAX; ++h)
#pragma unroll
      for (int e = 0; e < DPL; ++e) s_acc[wave][h][col * DPL + e] = acc[h][e];
  }
  if (lane == 0) s_bad[wave] = bad;
  __syncthreads();

  // Merge the four waves: weights 2^(m_w - M); waves without blocks have m_w = -inf.
  const bool anybad = s_bad[0] | s_bad[1] | s_bad[2] | s_bad[3];
  const float nan = __builtin_nanf("");
  for (int idx = tid; idx < nh * D; idx += 256) {
    const int h = idx / D;
    const int d = idx - h * D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float den = 0.f, num = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float e = fast_exp2(s_m[w][h] - M);
      den = fmaf(e, s_l[w][h], den);
      num = fmaf(e, s_acc[w][h][d], num);
    }
    const size_t row = (size_t)s * Hq + hbase + h;
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

template <int DT, int D, int GMAX>
void launch(const DecodeArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.P * a.Hkv * a.nsub * a.B;
  hipLaunchKernelGGL((decode_part_mfma<DT, D, GMAX>), dim3(grid), dim3(256), 0, st, a.out, a.q, a.kp, a.vp, a.bt,
                     a.cl, a.ws_o, a.ws_m, a.ws_l, a.B, a.Hq, a.Hkv, a.g, a.nsub, a.num_blocks, a.maxb, a.max_ctx,
                     a.qscale, a.psize, a.P);
}

template <int DT, int D>
void launch_g(const DecodeArgs& a, hipStream_t st) {
  switch (a.gmax) {
    case 1: launch<DT, D, 1>(a, st); break;
    case 2: launch<DT, D, 2>(a, st); break;
    case 4: launch<DT, D, 4>(a, st); break;
    default: launch<DT, D, 8>(a, st); break;
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
  if (a.P > 1) launch_decode_reduce(a, st);
}

}  // namespace pa
