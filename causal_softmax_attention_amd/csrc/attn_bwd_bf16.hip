// Causal attention backward for bfloat16 on gfx950 MFMA (float32 accumulation).
//
// Gradient of a loss with upstream gradient dO (pages: "Show HN: automatic
// deduction of FlashAttention kernel from 25 lines of SQL", the GRADIENT
// statement: grad(loss, q.x), grad(loss, k.x), grad(loss, v.x) of
// loss = SUM(x * x) / 2, so dO = O there).  With P_ij = exp(s_ij - lse_i) over
// the pairs j <= i, s_ij = scale q_i . k_j:
//   delta_i = sum_d dO_id O_id            (= sum_j P_ij dP_ij)
//   dP_ij   = dO_i . v_j,   dS_ij = P_ij (dP_ij - delta_i)
//   dV_j = sum_{i>=j} P_ij dO_i,  dK_j = scale sum_{i>=j} dS_ij q_i,
//   dQ_i = scale sum_{j<=i} dS_ij k_j.
// Scores are recomputed from q, k and the forward's saved lse; nothing N x N is
// stored.
//
// Three launches, no atomics (float atomics in L2 run at about one 4-byte add
// per channel-clock on this part, far too slow for a dQ accumulated across key
// blocks):
//   1. prep: delta_i and lse_i log2(e) per row (one pass over O and dO),
//   2. dK/dV, key-stationary: a wave owns 64 keys whose K and V stay in
//      registers as MFMA B operands; query tiles of 64 (Q, dO, lse, delta)
//      stream through a 3-stage LDS ring filled by asynchronous buffer loads
//      issued two tiles ahead.  S = Q K^T and dP = dO V^T are
//      formed as query x key accumulators, so after rounding to bf16 they are
//      the B operands of dV^T = dO^T P and dK^T = Q^T dS, whose A operands
//      come from transposing LDS reads of the same Q / dO tiles.
//   3. dQ, query-stationary: a wave owns 64 queries (Q, dO in registers, its
//      lse and delta per lane); key tiles (K, V) stream through LDS.  S^T and
//      dP^T are key x query accumulators, so dS^T is the B operand of
//      dQ^T = K^T dS^T.
// Each wave holds one SIMD (up to 512 registers) and issues its MFMAs among
// the independent exp / VALU work of the same tile.
#include "common.h"
#include "launch.h"
#include "mfma_bf16.h"

namespace attn {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsW = 64;               // stationary rows per wave
constexpr int kBlk = kRowsW * kWaves;    // stationary rows per workgroup
constexpr int kT = 64;                   // streamed rows per tile
constexpr int kT2 = 2 * kT;              // streamed rows per LDS stage (two tiles per barrier)
constexpr float kLog2e = 1.4426950408889634f;

// Per row: delta_i = sum_d dO_id O_id and lse2_i = lse_i log2(e) (the base-2
// exponent offset of P).  Eight lanes per row, 16 bytes each.
__global__ __launch_bounds__(256) void bwd_prep_bf16(const __bf16* __restrict__ o,
                                                     const __bf16* __restrict__ dout,
                                                     const float* __restrict__ lse,
                                                     float* __restrict__ delta,
                                                     float* __restrict__ lse2, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
  const int part = threadIdx.x & 7;
  float s = 0.f;
  if (r < rows) {
    const uint4 a = ldg16(o + r * kD + part * 8), b = ldg16(dout + r * kD + part * 8);
    const __bf16* x = (const __bf16*)&a;
    const __bf16* y = (const __bf16*)&b;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)x[e], (float)y[e], s);
  }
  s += __shfl_xor(s, 1);
  s += __shfl_xor(s, 2);
  s += __shfl_xor(s, 4);
  if (r < rows && part == 0) {
    delta[r] = s;
    lse2[r] = lse[r] * kLog2e;
  }
}

// One query tile of the dK/dV pass for one wave (64 keys x 64 queries).
// MASKED: the tile crosses the wave's diagonal or the end of the sequence, so
// absent pairs get weight 0 (a select).  Two sequential halves of 32 queries,
// fenced so that one half's operands and score tiles are live at a time.
template <bool MASKED>
__device__ __forceinline__ void dkdv_tile(const __bf16* qs, const __bf16* os, const float* lse2,
                                          const float* dl, int lane, int q0, int kw, int N,
                                          float c_scale, const bf16x8_t (&kop)[2][4],
                                          const bf16x8_t (&vop)[2][4], floatx16 (&dkacc)[2][2],
                                          floatx16 (&dvacc)[2][2]) {
  const int i32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    bf16x8_t qa[4], oa[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      qa[kk] = read_row8(qs, 32 * qt + i32, 16 * kk + 8 * h);
      oa[kk] = read_row8(os, 32 * qt + i32, 16 * kk + 8 * h);
    }
    // S = Q K^T and dP = dO V^T for 32 queries: lane holds a key column, query rows
    floatx16 s[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      floatx16 a = floatx16{}, b = floatx16{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        a = mma(qa[kk], kop[kt][kk], a);
        b = mma(oa[kk], vop[kt][kk], b);
      }
      s[kt] = a;
      dp[kt] = b;
    }
    // transposed operands of this half's two 16-query chunks, issued early
    bf16x8_t otr[2][2], qtr[2][2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        otr[half][dt] = read_tr(os, lane, 2 * qt + half, 32 * dt);
        qtr[half][dt] = read_tr(qs, lane, 2 * qt + half, 32 * dt);
      }
    float4 l4[4], d4[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      l4[g] = *(const float4*)(lse2 + 32 * qt + 8 * g + 4 * h);
      d4[g] = *(const float4*)(dl + 32 * qt + 8 * g + 4 * h);
    }
    uint32_t pp[2][8], dsp[2][8];  // [kt][pair]
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int key = kw + 32 * kt + i32;
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) {
        float pv[2], dsv[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * pr + e, g = r >> 2, w = r & 3;
          const float lr = w == 0 ? l4[g].x : w == 1 ? l4[g].y : w == 2 ? l4[g].z : l4[g].w;
          const float dr = w == 0 ? d4[g].x : w == 1 ? d4[g].y : w == 2 ? d4[g].z : d4[g].w;
          float p = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c_scale, -lr));
          if (MASKED) {
            const int qi = q0 + 32 * qt + acc_row(r, h);
            p = (key > qi || qi >= N) ? 0.f : p;
          }
          pv[e] = p;
          dsv[e] = p * (dp[kt][r] - dr);
        }
        pp[kt][pr] = pack_bf16(pv[0], pv[1]);
        dsp[kt][pr] = pack_bf16(dsv[0], dsv[1]);
      }
    }
    // dV^T += dO^T P and dK^T += Q^T dS over this half's two 16-query chunks
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          dvacc[dt][kt] = mma(otr[half][dt], chunk_op(pp[kt], half), dvacc[dt][kt]);
          dkacc[dt][kt] = mma(qtr[half][dt], chunk_op(dsp[kt], half), dkacc[dt][kt]);
        }
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct QStage {
  __bf16 q[kT2 * kD];
  __bf16 dout[kT2 * kD];
  float lse2[kT2];
  float delta[kT2];
};

__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2g,
    const float* __restrict__ deltag, __bf16* __restrict__ dk, __bf16* __restrict__ dv, int heads,
    int N, int nkb, float c_scale, float scale) {
  __shared__ QStage st0, st1, st2;
  int head, kb;
  if (!map_block(blockIdx.x, heads, nkb, false, head, kb)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const size_t rbase = (size_t)head * N;
  const int kw = kb * kBlk + wave * kRowsW;  // first key of this wave

  // stationary B operands: lane holds X[key kw + 32 kt + i32][16 kk + 8 h .. +7]
  bf16x8_t kop[2][4], vop[2][4];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = kw + 32 * kt + i32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 a = make_uint4(0, 0, 0, 0), b = a;
      if (key < N) {
        a = ldg16(k + base + (size_t)key * kD + 16 * kk + 8 * h);
        b = ldg16(v + base + (size_t)key * kD + 16 * kk + 8 * h);
      }
      kop[kt][kk] = __builtin_bit_cast(bf16x8_t, a);
      vop[kt][kk] = __builtin_bit_cast(bf16x8_t, b);
    }
  }
  floatx16 dkacc[2][2], dvacc[2][2];  // [dt][kt]: (feature x key) tiles, lane holds a key column
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      dkacc[a][b] = floatx16{};
      dvacc[a][b] = floatx16{};
    }

  const int qstart = kb * kBlk;  // queries before it see none of these keys
  const int ntiles = (N - qstart + kT2 - 1) / kT2;  // stages of 128 queries
  const uint32_t tbytes = (uint32_t)N * kD * 2, rbytes = (uint32_t)N * 4;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(q + base, tbytes), ro = head_rsrc(dout + base, tbytes);
  const __amdgpu_buffer_rsrc_t rl = head_rsrc(lse2g + rbase, rbytes), rd = head_rsrc(deltag + rbase, rbytes);
  auto issue = [&](QStage& s, int t) {
    const int r0 = qstart + t * kT2;
    // one 64-row half of lse2 / delta per wave, then the Q and dO rows
    if (wave < 2) rows_async(rl, s.lse2 + 64 * wave, r0 + 64 * wave, lane);
    else rows_async(rd, s.delta + 64 * (wave - 2), r0 + 64 * (wave - 2), lane);
    tile_async<kT2>(rq, s.q, r0, wave, lane);
    tile_async<kT2>(ro, s.dout, r0, wave, lane);
  };
  auto step = [&](QStage& cur, QStage& ahead, int t) {
    const bool pre = t + 2 < ntiles;
    if (pre) issue(ahead, t + 2);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int q0 = qstart + t * kT2 + sub * kT;
      const __bf16* qs = cur.q + sub * kT * kD;
      const __bf16* os = cur.dout + sub * kT * kD;
      if (kw < N && q0 + kT - 1 >= kw) {
        if ((q0 < kw + kRowsW - 1) || (q0 + kT > N))
          dkdv_tile<true>(qs, os, cur.lse2 + sub * kT, cur.delta + sub * kT, lane, q0, kw, N,
                          c_scale, kop, vop, dkacc, dvacc);
        else
          dkdv_tile<false>(qs, os, cur.lse2 + sub * kT, cur.delta + sub * kT, lane, q0, kw, N,
                           c_scale, kop, vop, dkacc, dvacc);
      }
    }
    if (pre) wait_vm_barrier<8>();
    else wait_vm_barrier<0>();
  };

  issue(st0, 0);
  if (ntiles > 1) issue(st1, 1);
  wait_vm_barrier<0>();
  for (int t = 0; t < ntiles; t += 3) {
    step(st0, st2, t);
    if (t + 1 < ntiles) step(st1, st0, t + 1);
    if (t + 2 < ntiles) step(st2, st1, t + 2);
  }

  // epilogue: lane holds key column kw + 32 kt + i32, feature rows 32 dt + acc_row(r, h)
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = kw + 32 * kt + i32;
    if (key >= N) continue;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        uint2 wk, wv;
        wk.x = pack_bf16(dkacc[dt][kt][4 * g + 0] * scale, dkacc[dt][kt][4 * g + 1] * scale);
        wk.y = pack_bf16(dkacc[dt][kt][4 * g + 2] * scale, dkacc[dt][kt][4 * g + 3] * scale);
        wv.x = pack_bf16(dvacc[dt][kt][4 * g + 0], dvacc[dt][kt][4 * g + 1]);
        wv.y = pack_bf16(dvacc[dt][kt][4 * g + 2], dvacc[dt][kt][4 * g + 3]);
        *(uint2*)(dk + base + (size_t)key * kD + d) = wk;
        *(uint2*)(dv + base + (size_t)key * kD + d) = wv;
      }
  }
}

// One key tile of the dQ pass for one wave (64 queries x 64 keys), as two
// halves of 32 keys: the second half's S^T / dP^T MFMAs are issued before the
// first half's exp / VALU work, and the first half's dQ MFMAs before the
// second half's, so each wave always has independent MFMA and VALU work in
// flight.  MASKED: the tile crosses the wave's diagonal or the end of the
// sequence, so absent pairs get weight 0 (a select, not a branch).
template <bool MASKED>
__device__ __forceinline__ void dq_half_softmax(const floatx16 (&s)[2], const floatx16 (&dp)[2],
                                                uint32_t (&dsp)[2][8], int kt, int k0, int qw,
                                                int N, int i32, int h, float c_scale,
                                                const float (&lse2)[2], const float (&dl)[2]) {
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = qw + 32 * qt + i32;
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      float dsv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * pr + e;
        float p = __builtin_amdgcn_exp2f(fmaf(s[qt][r], c_scale, -lse2[qt]));
        if (MASKED) {
          const int key = k0 + 32 * kt + acc_row(r, h);
          p = (key > qi || key >= N) ? 0.f : p;
        }
        dsv[e] = p * (dp[qt][r] - dl[qt]);
      }
      dsp[qt][pr] = pack_bf16(dsv[0], dsv[1]);
    }
  }
}

__device__ __forceinline__ void dq_half_scores(const __bf16* ks, const __bf16* vs, int kt,
                                               int i32, int h, const bf16x8_t (&qop)[2][4],
                                               const bf16x8_t (&oop)[2][4], floatx16 (&s)[2],
                                               floatx16 (&dp)[2]) {
  bf16x8_t ka[4], va[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    ka[kk] = read_row8(ks, 32 * kt + i32, 16 * kk + 8 * h);
    va[kk] = read_row8(vs, 32 * kt + i32, 16 * kk + 8 * h);
  }
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    floatx16 a = floatx16{}, b = floatx16{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      a = mma(ka[kk], qop[qt][kk], a);
      b = mma(va[kk], oop[qt][kk], b);
    }
    s[qt] = a;
    dp[qt] = b;
  }
}

template <bool MASKED>
__device__ __forceinline__ void dq_tile(const __bf16* ks, const __bf16* vs, int lane, int k0,
                                        int qw, int N, float c_scale,
                                        const bf16x8_t (&qop)[2][4], const bf16x8_t (&oop)[2][4],
                                        const float (&lse2)[2], const float (&dl)[2],
                                        floatx16 (&dqacc)[2][2]) {
  const int i32 = lane & 31, h = lane >> 5;
  floatx16 s0[2], dp0[2], s1[2], dp1[2];
  uint32_t dsp0[2][8], dsp1[2][8];
  bf16x8_t ktr0[2][2], ktr1[2][2];
  dq_half_scores(ks, vs, 0, i32, h, qop, oop, s0, dp0);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) ktr0[half][dt] = read_tr(ks, lane, half, 32 * dt);
  dq_half_scores(ks, vs, 1, i32, h, qop, oop, s1, dp1);
  dq_half_softmax<MASKED>(s0, dp0, dsp0, 0, k0, qw, N, i32, h, c_scale, lse2, dl);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) ktr1[half][dt] = read_tr(ks, lane, 2 + half, 32 * dt);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        dqacc[dt][qt] = mma(ktr0[half][dt], chunk_op(dsp0[qt], half), dqacc[dt][qt]);
  dq_half_softmax<MASKED>(s1, dp1, dsp1, 1, k0, qw, N, i32, h, c_scale, lse2, dl);
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int qt = 0; qt < 2; ++qt)
        dqacc[dt][qt] = mma(ktr1[half][dt], chunk_op(dsp1[qt], half), dqacc[dt][qt]);
}

struct KVStage {
  __bf16 k[kT2 * kD];
  __bf16 v[kT2 * kD];
};

__global__ __launch_bounds__(kThreads, 1) void bwd_dq_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse2g,
    const float* __restrict__ deltag, __bf16* __restrict__ dq, int heads, int N, int nqb,
    float c_scale, float scale) {
  __shared__ KVStage st0, st1, st2;
  int head, qb;
  if (!map_block(blockIdx.x, heads, nqb, true, head, qb)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const int qw = qb * kBlk + wave * kRowsW;
  const int wq_last = min(qw + kRowsW, N) - 1;

  // stationary B operands of S^T = K Q^T and dP^T = V dO^T; per-lane lse2, delta
  bf16x8_t qop[2][4], oop[2][4];
  float lse2[2], dl[2];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
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
    lse2[qt] = qi < N ? lse2g[(size_t)head * N + qi] : 0.f;
    dl[qt] = qi < N ? deltag[(size_t)head * N + qi] : 0.f;
  }
  floatx16 dqacc[2][2];  // [dt][qt]: (feature x query), lane holds a query column
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) dqacc[a][b] = floatx16{};

  const int kend = min(N, qb * kBlk + kBlk);
  const int ntiles = (kend + kT2 - 1) / kT2;
  const uint32_t tbytes = (uint32_t)N * kD * 2;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + base, tbytes), rv = head_rsrc(v + base, tbytes);
  auto issue = [&](KVStage& s, int t) {
    tile_async<kT2>(rk, s.k, t * kT2, wave, lane);
    tile_async<kT2>(rv, s.v, t * kT2, wave, lane);
  };
  auto step = [&](KVStage& cur, KVStage& ahead, int t) {
    const bool pre = t + 2 < ntiles;
    if (pre) issue(ahead, t + 2);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int k0 = t * kT2 + sub * kT;
      if (k0 <= wq_last) {
        if ((k0 + kT - 1 > qw) || (k0 + kT > N))
          dq_tile<true>(cur.k + sub * kT * kD, cur.v + sub * kT * kD, lane, k0, qw, N, c_scale, qop, oop, lse2, dl, dqacc);
        else
          dq_tile<false>(cur.k + sub * kT * kD, cur.v + sub * kT * kD, lane, k0, qw, N, c_scale, qop, oop, lse2, dl, dqacc);
      }
    }
    if (pre) wait_vm_barrier<8>();
    else wait_vm_barrier<0>();
  };

  issue(st0, 0);
  if (ntiles > 1) issue(st1, 1);
  wait_vm_barrier<0>();
  for (int t = 0; t < ntiles; t += 3) {
    step(st0, st2, t);
    if (t + 1 < ntiles) step(st1, st0, t + 1);
    if (t + 2 < ntiles) step(st2, st1, t + 2);
  }

#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
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

size_t bwd_workspace_bytes_bf16(int64_t heads, int64_t N) {
  return (size_t)heads * N * 2 * sizeof(float);  // delta, then lse * log2(e)
}

hipError_t launch_bwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* o,
                           const __bf16* dout, const float* lse, __bf16* dq, __bf16* dk,
                           __bf16* dv, void* workspace, int64_t heads, int64_t N, double scale,
                           hipStream_t stream, const Timers& tm) {
  const int64_t rows = heads * N;
  float* delta = (float*)workspace;
  float* lse2 = delta + rows;
  const float c = (float)(scale * 1.4426950408889634);
  const int nb = (int)((N + kBlk - 1) / kBlk);
  const unsigned grid = (unsigned)(8 * ((heads + 7) / 8) * nb);
  if (hipError_t e = mark(tm.start[kTimerBwdPre], stream)) return e;
  hipLaunchKernelGGL(bwd_prep_bf16, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, stream, o,
                     dout, lse, delta, lse2, rows);
  if (hipError_t e = mark(tm.stop[kTimerBwdPre], stream)) return e;
  if (hipError_t e = mark(tm.start[kTimerBwdDkdv], stream)) return e;
  hipLaunchKernelGGL(bwd_dkdv_bf16, dim3(grid), dim3(kThreads), 0, stream, q, k, v, dout, lse2,
                     delta, dk, dv, (int)heads, (int)N, nb, c, (float)scale);
  if (hipError_t e = mark(tm.stop[kTimerBwdDkdv], stream)) return e;
  if (hipError_t e = mark(tm.start[kTimerBwdDq], stream)) return e;
  hipLaunchKernelGGL(bwd_dq_bf16, dim3(grid), dim3(kThreads), 0, stream, q, k, v, dout, lse2,
                     delta, dq, (int)heads, (int)N, nb, c, (float)scale);
  if (hipError_t e = mark(tm.stop[kTimerBwdDq], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
