// dQ of the bfloat16 causal attention backward on gfx950 MFMA: the
// query-stationary pass (a wave owns 32 queries; K, V stream through LDS).
// The per-row values it reads, -delta_i and -lse_i / scale, come from the
// backward's prep kernel (attn_bwd_bf16.hip), which also documents the
// gradient formulas (pages: "Show HN: automatic deduction of FlashAttention
// kernel from 25 lines of SQL", the GRADIENT statement).
#include "common.h"
#include "launch.h"
#include "mfma_bf16.h"

namespace attn {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = 1;                   // 32-query MFMA columns per wave
constexpr int kRowsW = 32 * kQT;         // queries per wave
constexpr int kBlk = kRowsW * kWaves;    // queries per workgroup
constexpr int kT = 64;                   // keys per tile
constexpr int kT2 = 2 * kT;              // keys per LDS stage (two tiles: one barrier per 48 MFMAs)

// ---- dQ, query-stationary ---------------------------------------------------
//
// One key tile of the dQ pass for one wave (32 queries x 64 keys), as two
// halves of 32 keys: the second half's S^T / dP^T MFMAs are issued before the
// first half's exp / VALU work, and the first half's dQ MFMAs before the
// second half's, so each wave always has independent MFMA and VALU work in
// flight.  The score accumulators start from -lse/scale and -delta of their
// query (one per lane), as in the dK/dV pass.  MASKED: the tile holds absent
// pairs (past the wave's diagonal or a window's start, or past the end of the
// sequence), which get weight 0 (a select, not a branch).
// SEG: segment ids apply (segk: the tile's 64 key ids in LDS, sq: the lane's
// query id); a pair of different ids is absent.
template <bool MASKED, bool SEG>
__device__ __forceinline__ void dq_half_softmax(const floatx16 (&s)[kQT], const floatx16 (&dp)[kQT],
                                                uint32_t (&dsp)[kQT][8], int kt, int k0, int qw,
                                                int N, int i32, int h, float c_scale, int causal,
                                                int band, const int32_t* segk, int32_t sq) {
  int32_t sk[16];  // ids of the lane's 16 keys of this half
  if (MASKED && SEG) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int4 w = *(const int4*)(segk + 32 * kt + 8 * g + 4 * h);
      sk[4 * g + 0] = w.x; sk[4 * g + 1] = w.y; sk[4 * g + 2] = w.z; sk[4 * g + 3] = w.w;
    }
  }
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qw + 32 * qt + i32;
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      float dsv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * pr + e;
        float p = __builtin_amdgcn_exp2f(s[qt][r] * c_scale);
        if (MASKED) {
          const int key = k0 + 32 * kt + acc_row(r, h);
          p = (key >= N || (causal && key > qi) || (band && qi - key >= band) ||
               (SEG && sk[r] != sq)) ? 0.f : p;
        }
        dsv[e] = p * dp[qt][r];
      }
      dsp[qt][pr] = pack_bf16(dsv[0], dsv[1]);
    }
  }
}

// dq_half_softmax of a masked tile in the window and segment kernels, with
// the predicate tested as a range of each register's key offset: register r
// holds key kb + acc_row(r, 0), present when that offset lies strictly
// between lo and hi (fewer instructions per tile; the causal and full
// kernels keep the form above, which compiled to their faster loops).
template <bool SEG>
__device__ __forceinline__ void dq_half_softmax_range(const floatx16 (&s)[kQT],
                                                      const floatx16 (&dp)[kQT],
                                                      uint32_t (&dsp)[kQT][8], int kt, int k0,
                                                      int qw, int N, int i32, int h,
                                                      float c_scale, int causal, int band,
                                                      const int32_t* segk, int32_t sq) {
  int32_t sk[16];  // ids of the lane's 16 keys of this half
  if (SEG) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int4 w = *(const int4*)(segk + 32 * kt + 8 * g + 4 * h);
      sk[4 * g + 0] = w.x; sk[4 * g + 1] = w.y; sk[4 * g + 2] = w.z; sk[4 * g + 3] = w.w;
    }
  }
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qw + 32 * qt + i32;
    const int kb = k0 + 32 * kt + 4 * h;
    const int hi = causal ? min(N, qi + 1) - kb : N - kb;
    const int lo = band ? qi - band - kb : INT32_MIN;
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      float dsv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * pr + e;
        const int off = acc_row(r, 0);
        const float p = __builtin_amdgcn_exp2f(s[qt][r] * c_scale);
        dsv[e] = (!(off < hi && off > lo) || (SEG && sk[r] != sq) ? 0.f : p) * dp[qt][r];
      }
      dsp[qt][pr] = pack_bf16(dsv[0], dsv[1]);
    }
  }
}

__device__ __forceinline__ void dq_half_scores(const __bf16* ks, const __bf16* vs, int kt,
                                               int i32, int h, const bf16x8_t (&qop)[kQT][4],
                                               const bf16x8_t (&oop)[kQT][4],
                                               const float (&nls)[kQT], const float (&ndl)[kQT],
                                               floatx16 (&s)[kQT], floatx16 (&dp)[kQT]) {
  bf16x8_t ka[4], va[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    ka[kk] = read_row8(ks, 32 * kt + i32, 16 * kk + 8 * h);
    va[kk] = read_row8(vs, 32 * kt + i32, 16 * kk + 8 * h);
  }
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    floatx16 a, b;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      a[r] = nls[qt];
      b[r] = ndl[qt];
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      a = mma(ka[kk], qop[qt][kk], a);
      b = mma(va[kk], oop[qt][kk], b);
    }
    s[qt] = a;
    dp[qt] = b;
  }
}

template <bool MASKED, bool SEG, bool RANGE = false>
__device__ __forceinline__ void dq_tile(const __bf16* ks, const __bf16* vs, int lane, int k0,
                                        int qw, int N, float c_scale,
                                        const bf16x8_t (&qop)[kQT][4], const bf16x8_t (&oop)[kQT][4],
                                        const float (&nls)[kQT], const float (&ndl)[kQT],
                                        floatx16 (&dqacc)[2][kQT], int causal, int band,
                                        const int32_t* segk, int32_t sq) {
  const int i32 = lane & 31, h = lane >> 5;
  floatx16 s0[kQT], dp0[kQT], s1[kQT], dp1[kQT];
  uint32_t dsp0[kQT][8], dsp1[kQT][8];
  bf16x8_t ktr0[2][2], ktr1[2][2];
  dq_half_scores(ks, vs, 0, i32, h, qop, oop, nls, ndl, s0, dp0);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) ktr0[half][dt] = read_tr(ks, lane, half, 32 * dt);
  dq_half_scores(ks, vs, 1, i32, h, qop, oop, nls, ndl, s1, dp1);
  if constexpr (MASKED && RANGE)
    dq_half_softmax_range<SEG>(s0, dp0, dsp0, 0, k0, qw, N, i32, h, c_scale, causal, band, segk,
                               sq);
  else
    dq_half_softmax<MASKED, SEG>(s0, dp0, dsp0, 0, k0, qw, N, i32, h, c_scale, causal, band,
                                 segk, sq);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) ktr1[half][dt] = read_tr(ks, lane, 2 + half, 32 * dt);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
        dqacc[dt][qt] = mma(ktr0[half][dt], chunk_op(dsp0[qt], half), dqacc[dt][qt]);
  if constexpr (MASKED && RANGE)
    dq_half_softmax_range<SEG>(s1, dp1, dsp1, 1, k0, qw, N, i32, h, c_scale, causal, band, segk,
                               sq);
  else
    dq_half_softmax<MASKED, SEG>(s1, dp1, dsp1, 1, k0, qw, N, i32, h, c_scale, causal, band,
                                 segk, sq);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt)
        dqacc[dt][qt] = mma(ktr1[half][dt], chunk_op(dsp1[qt], half), dqacc[dt][qt]);
}

struct alignas(16) KVStage {
  __bf16 k[kT2 * kD];
  __bf16 v[kT2 * kD];
};

// CAUSAL: the causal predicate applies; BANDED: a window of band_arg keys does;
// SEG: only pairs of equal segment ids (seg, [B][N], batch = head / hpb) exist.
template <bool CAUSAL, bool BANDED, bool SEG>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ nlseg,
    const float* __restrict__ ndeltag, __bf16* __restrict__ dq, int heads, int N, int nqb,
    float c_scale, float scale, int band_arg, const int32_t* __restrict__ seg, int hpb) {
  constexpr int causal = CAUSAL;
  const int band = BANDED ? band_arg : 0;
  __shared__ KVStage st0, st1;
  __shared__ __attribute__((aligned(16))) int32_t sg[2][SEG ? kT2 : 4];  // the stages' key ids
  static_assert(kQT == 1 && kT2 == 2 * kT, "one query column per wave, two tiles per stage");
  int head, qb;
  if (!map_block(blockIdx.x, heads, nqb, true, 4, head, qb)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const int qw = qb * kBlk + wave * kRowsW;
  const int wq_last = min(qw + kRowsW, N) - 1;

  // stationary B operands of S^T = K Q^T and dP^T = V dO^T; per-lane -lse/scale, -delta
  bf16x8_t qop[kQT][4], oop[kQT][4];
  float nls[kQT], ndl[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qw + 32 * qt + i32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 a = make_uint4(0, 0, 0, 0), b = a;
      if (qi < N) {
        a = ldg16(q + base + (size_t)qi * kD + 16 * kk + 8 * h);
        b = ldg16(dout + base + (size_t)qi * kD + 16 * kk + 8 * h);
      }
      qop[qt][kk] = __builtin_bit_cast(bf16x8_t, a);
      oop[qt][kk] = __builtin_bit_cast(bf16x8_t, b);
    }
    nls[qt] = qi < N ? nlseg[(size_t)head * N + qi] : 0.f;
    ndl[qt] = qi < N ? ndeltag[(size_t)head * N + qi] : 0.f;
  }
  // segment ids: the lane's query id and the range of the wave's valid ids
  const int32_t* segrow = SEG ? seg + (size_t)(head / hpb) * N : nullptr;
  int32_t sq = 0, sqlo = 0, sqhi = 0;
  if (SEG) {
    const int qi = qw + i32;
    sq = qi < N ? segrow[qi] : 0;
    sqlo = qi < N ? sq : INT32_MAX;
    sqhi = qi < N ? sq : INT32_MIN;
#pragma unroll
    for (int o2 = 16; o2 >= 1; o2 >>= 1) {
      sqlo = min(sqlo, __shfl_xor(sqlo, o2));
      sqhi = max(sqhi, __shfl_xor(sqhi, o2));
    }
    sqlo = __builtin_amdgcn_readfirstlane(sqlo);
    sqhi = __builtin_amdgcn_readfirstlane(sqhi);
  }
  floatx16 dqacc[2][kQT];  // [dt][qt]: (feature x query), lane holds a query column
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < kQT; ++b) dqacc[a][b] = floatx16{};

  // keys of the workgroup's queries: stages t0 .. ntiles-1 of kT2 keys
  int t0 = band ? max(0, qb * kBlk - band + 1) / kT2 : 0;
  const int kend = causal ? min(N, qb * kBlk + kBlk) : N;
  int ntiles = (kend + kT2 - 1) / kT2;
  if (SEG) {
    // only the key tiles within the span of keys whose ids fall in the
    // block's query-id range (never empty: each query is also a key)
    __shared__ int32_t red[2][kWaves][4];
    const SegSpan sp = seg_span<kThreads>(segrow, N, qb * kBlk, kBlk, t0 * kT2, kend, threadIdx.x, red);
    t0 = __builtin_amdgcn_readfirstlane(sp.first / kT2);
    ntiles = __builtin_amdgcn_readfirstlane((sp.last + kT2 - 1) / kT2);
  }
  const int wlo = band ? qw - band + 1 : 0, whi = causal ? wq_last : N - 1;  // keys of this wave
  const uint32_t tbytes = (uint32_t)N * kD * 2;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + base, tbytes), rv = head_rsrc(v + base, tbytes);
  __amdgpu_buffer_rsrc_t rs = rk;
  if (SEG) rs = head_rsrc(segrow, (uint32_t)N * 4);
  // wave 0 also copies the stage's key ids (two more loads per stage)
  auto issue = [&](KVStage& s, int32_t* sgs, int t) {
    tile_async<kT2, kWaves>(rk, s.k, t * kT2, wave, lane);
    tile_async<kT2, kWaves>(rv, s.v, t * kT2, wave, lane);
    if (SEG && wave == 0) {
      rows_async(rs, (float*)sgs, t * kT2, lane);
      rows_async(rs, (float*)sgs + kT, t * kT2 + kT, lane);
    }
  };
  // one 64-key tile of a stage (keys k0 .. k0 + 63, at ks / vs / sgc in LDS)
  auto tile = [&](const __bf16* ks, const __bf16* vs, const int32_t* sgc,
                  int k0) __attribute__((always_inline)) {
    if (k0 <= whi && k0 + kT - 1 >= wlo) {
      // segments: no key id in the wave's id range -> no pair; all ids one and
      // the same -> the ids mask nothing
      bool seg_some = true, seg_one = true;
      if (SEG) {
        const int32_t skey = sgc[lane];
        const bool kin = k0 + lane < N;
        seg_some = __any(kin && skey >= sqlo && skey <= sqhi);
        seg_one = sqlo == sqhi && __all(!kin || skey == sqlo);
      }
      if (seg_some) {
        // masked: some pair of the tile is absent for some query of the wave
        if ((causal && k0 + kT - 1 > qw) || (k0 + kT > N) || (band && k0 < qw + kRowsW - band) ||
            !seg_one)
          dq_tile<true, SEG, SEG || BANDED>(ks, vs, lane, k0, qw, N, c_scale, qop, oop, nls, ndl,
                                            dqacc, causal, band, sgc, sq);
        else
          dq_tile<false, SEG>(ks, vs, lane, k0, qw, N, c_scale, qop, oop, nls, ndl, dqacc, causal,
                              band, sgc, sq);
      }
    }
  };
  // a two-stage ring: stage t + 1 is issued into the buffer that stage t - 1
  // left (every wave passed the barrier after it) and has all of stage t's
  // two tiles to land
  auto step = [&](KVStage& cur, int32_t* sgc, KVStage& ahead, int32_t* sga, int t) {
    if (t + 1 < ntiles) issue(ahead, sga, t + 1);
    tile(cur.k, cur.v, sgc, t * kT2);
    tile(cur.k + kT * kD, cur.v + kT * kD, sgc + kT, t * kT2 + kT);
    wait_vm_barrier<0>();  // stage t + 1 has landed; every wave is done with stage t
  };

  issue(st0, sg[0], t0);
  wait_vm_barrier<0>();
  for (int t = t0; t < ntiles; t += 2) {
    step(st0, sg[0], st1, sg[1], t);
    if (t + 1 < ntiles) step(st1, sg[1], st0, sg[0], t + 1);
  }

#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qw + 32 * qt + i32;
    if (qi >= N) continue;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        uint2 w;
        w.x = pack_bf16(dqacc[dt][qt][4 * g + 0] * scale, dqacc[dt][qt][4 * g + 1] * scale);
        w.y = pack_bf16(dqacc[dt][qt][4 * g + 2] * scale, dqacc[dt][qt][4 * g + 3] * scale);
        *(uint2*)(dq + base + (size_t)qi * kD + d) = w;
      }
  }
}

}  // namespace

hipError_t launch_bwd_dq_bf16(const __bf16* q, const __bf16* k, const __bf16* v,
                              const __bf16* dout, const float* nlse, const float* ndelta,
                              __bf16* dq, int64_t heads, int64_t N, double scale,
                              const Mask& mk, hipStream_t stream, const Timers& tm) {
  const float c = (float)(scale * 1.4426950408889634);
  const int nb = (int)((N + kBlk - 1) / kBlk);
  const unsigned grid = (unsigned)(8 * ((heads + 7) / 8) * nb);
  if (hipError_t e = mark(tm.start[kTimerBwdDq], stream)) return e;
  auto kern = mk.seg ? (mk.band > 0 ? bwd_dq_bf16<true, true, true>
                        : mk.causal ? bwd_dq_bf16<true, false, true>
                                    : bwd_dq_bf16<false, false, true>)
                     : (mk.band > 0 ? bwd_dq_bf16<true, true, false>
                        : mk.causal ? bwd_dq_bf16<true, false, false>
                                    : bwd_dq_bf16<false, false, false>);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, q, k, v, dout, nlse, ndelta, dq,
                     (int)heads, (int)N, nb, c, (float)scale, mk.band, mk.seg, mk.hpb);
  if (hipError_t e = mark(tm.stop[kTimerBwdDq], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
