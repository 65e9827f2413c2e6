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
//   1. delta (one pass over O and dO),
//   2. dK/dV, key-stationary: a wave owns 64 keys whose K and V stay in
//      registers as MFMA B operands; query tiles of 64 (Q, dO, lse, delta)
//      stream through a 3-stage LDS ring.  S = Q K^T and dP = dO V^T are
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
constexpr int kStages = 3;
constexpr float kLog2e = 1.4426950408889634f;

// delta_i = sum_d dO_id O_id: eight lanes per row, 16 bytes each.
__global__ __launch_bounds__(256) void bwd_delta_bf16(const __bf16* __restrict__ o,
                                                      const __bf16* __restrict__ dout,
                                                      float* __restrict__ delta, int64_t rows) {
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
  if (r < rows && part == 0) delta[r] = s;
}

struct SmemKV {
  __bf16 q[kStages][kT * kD];
  __bf16 dout[kStages][kT * kD];
  float lse2[kStages][kT];
  float delta[kStages][kT];
};

__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, __bf16* __restrict__ dk, __bf16* __restrict__ dv, int heads,
    int N, int nkb, float c_scale, float scale) {
  __shared__ SmemKV sm;
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

  const int qstart = kb * kBlk;                 // queries before it see none of these keys
  const int ntiles = (N - qstart + kT - 1) / kT;
  uint4 qreg[2], oreg[2];
  float4 sreg;
  auto load_tile = [&](int t) {
    const int q0 = qstart + t * kT;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * kThreads, row = e >> 3, col = (e & 7) * 8, i = q0 + row;
      qreg[u] = make_uint4(0, 0, 0, 0);
      oreg[u] = make_uint4(0, 0, 0, 0);
      if (i < N) {
        qreg[u] = ldg16(q + base + (size_t)i * kD + col);
        oreg[u] = ldg16(dout + base + (size_t)i * kD + col);
      }
    }
    if (tid < 32) {
      const int j = tid & 15, i0 = q0 + 4 * j;
      const float* src = tid < 16 ? lse : delta;
      const float mul = tid < 16 ? kLog2e : 1.0f;
      float x[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = (i0 + e < N) ? src[rbase + i0 + e] * mul : 0.f;
      sreg = make_float4(x[0], x[1], x[2], x[3]);
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * kThreads, off = lds_at(e >> 3, (e & 7) * 8);
      *(uint4*)(&sm.q[st][off]) = qreg[u];
      *(uint4*)(&sm.dout[st][off]) = oreg[u];
    }
    if (tid < 16) *(float4*)(&sm.lse2[st][4 * tid]) = sreg;
    else if (tid < 32) *(float4*)(&sm.delta[st][4 * (tid - 16)]) = sreg;
  };

  load_tile(0);
  store_tile(0);
  if (ntiles > 1) {
    load_tile(1);
    store_tile(1);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int st = t % kStages;
    const bool pre = t + 2 < ntiles;
    if (pre) load_tile(t + 2);
    const int q0 = qstart + t * kT;
    if (kw < N && q0 + kT - 1 >= kw) {
      const __bf16* qs = sm.q[st];
      const __bf16* os = sm.dout[st];
      // S = Q K^T and dP = dO V^T as [qt][kt] tiles: lane holds key column, query rows
      floatx16 s[2][2], dp[2][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        bf16x8_t qa[4], oa[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          qa[kk] = read_row8(qs, 32 * qt + i32, 16 * kk + 8 * h);
          oa[kk] = read_row8(os, 32 * qt + i32, 16 * kk + 8 * h);
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          floatx16 a = floatx16{}, b = floatx16{};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            a = mma(qa[kk], kop[kt][kk], a);
            b = mma(oa[kk], vop[kt][kk], b);
          }
          s[qt][kt] = a;
          dp[qt][kt] = b;
        }
      }
      const bool masked = (q0 < kw + kRowsW - 1) || (q0 + kT > N);
      uint32_t pp[2][2][8], dsp[2][2][8];  // [qt][kt][pair] bf16 pairs
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float4 l4[4], d4[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          l4[g] = *(const float4*)(&sm.lse2[st][32 * qt + 8 * g + 4 * h]);
          d4[g] = *(const float4*)(&sm.delta[st][32 * qt + 8 * g + 4 * h]);
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int key = kw + 32 * kt + i32;
#pragma unroll
          for (int pr = 0; pr < 8; ++pr) {
            float pv[2], dv_[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 2 * pr + e, g = r >> 2, w = r & 3;
              const float lr = w == 0 ? l4[g].x : w == 1 ? l4[g].y : w == 2 ? l4[g].z : l4[g].w;
              const float dr = w == 0 ? d4[g].x : w == 1 ? d4[g].y : w == 2 ? d4[g].z : d4[g].w;
              float p = __builtin_amdgcn_exp2f(fmaf(s[qt][kt][r], c_scale, -lr));
              if (masked) {
                const int qi = q0 + 32 * qt + acc_row(r, h);
                if (key > qi || qi >= N) p = 0.f;
              }
              pv[e] = p;
              dv_[e] = p * (dp[qt][kt][r] - dr);
            }
            pp[qt][kt][pr] = pack_bf16(pv[0], pv[1]);
            dsp[qt][kt][pr] = pack_bf16(dv_[0], dv_[1]);
          }
        }
      }
      // dV^T += dO^T P and dK^T += Q^T dS over 4 chunks of 16 queries
#pragma unroll
      for (int c = 0; c < 4; ++c) {
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const bf16x8_t oa = read_tr(os, lane, c, 32 * dt);
          const bf16x8_t qa = read_tr(qs, lane, c, 32 * dt);
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) {
            dvacc[dt][kt] = mma(oa, chunk_op(pp[c >> 1][kt], c & 1), dvacc[dt][kt]);
            dkacc[dt][kt] = mma(qa, chunk_op(dsp[c >> 1][kt], c & 1), dkacc[dt][kt]);
          }
        }
      }
    }
    if (pre) store_tile((t + 2) % kStages);
    __syncthreads();
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

struct SmemQ {
  __bf16 k[kStages][kT * kD];
  __bf16 v[kStages][kT * kD];
};

__global__ __launch_bounds__(kThreads, 1) void bwd_dq_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, __bf16* __restrict__ dq, int heads, int N, int nqb,
    float c_scale, float scale) {
  __shared__ SmemQ sm;
  int head, qb;
  if (!map_block(blockIdx.x, heads, nqb, true, head, qb)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const int qw = qb * kBlk + wave * kRowsW;
  const int wq_last = min(qw + kRowsW, N) - 1;

  // stationary B operands of S^T = K Q^T and dP^T = V dO^T; per-lane lse, delta
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
    lse2[qt] = qi < N ? lse[(size_t)head * N + qi] * kLog2e : 0.f;
    dl[qt] = qi < N ? delta[(size_t)head * N + qi] : 0.f;
  }
  floatx16 dqacc[2][2];  // [dt][qt]: (feature x query), lane holds a query column
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) dqacc[a][b] = floatx16{};

  const int kend = min(N, qb * kBlk + kBlk);
  const int ntiles = (kend + kT - 1) / kT;
  uint4 kreg[2], vreg[2];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * kThreads, row = e >> 3, col = (e & 7) * 8, j = t * kT + row;
      kreg[u] = make_uint4(0, 0, 0, 0);
      vreg[u] = make_uint4(0, 0, 0, 0);
      if (j < N) {
        kreg[u] = ldg16(k + base + (size_t)j * kD + col);
        vreg[u] = ldg16(v + base + (size_t)j * kD + col);
      }
    }
  };
  auto store_tile = [&](int st) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * kThreads, off = lds_at(e >> 3, (e & 7) * 8);
      *(uint4*)(&sm.k[st][off]) = kreg[u];
      *(uint4*)(&sm.v[st][off]) = vreg[u];
    }
  };

  load_tile(0);
  store_tile(0);
  if (ntiles > 1) {
    load_tile(1);
    store_tile(1);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int st = t % kStages;
    const bool pre = t + 2 < ntiles;
    if (pre) load_tile(t + 2);
    const int k0 = t * kT;
    if (k0 <= wq_last) {
      const __bf16* ks = sm.k[st];
      const __bf16* vs = sm.v[st];
      floatx16 s[2][2], dp[2][2];  // [kt][qt]: lane holds query column, key rows
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
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
          s[kt][qt] = a;
          dp[kt][qt] = b;
        }
      }
      const bool masked = (k0 + kT - 1 > qw) || (k0 + kT > N);
      uint32_t dsp[2][2][8];  // [qt][kt][pair]
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int qi = qw + 32 * qt + i32;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int pr = 0; pr < 8; ++pr) {
            float dsv[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 2 * pr + e;
              float p = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][r], c_scale, -lse2[qt]));
              if (masked) {
                const int key = k0 + 32 * kt + acc_row(r, h);
                if (key > qi || key >= N) p = 0.f;
              }
              dsv[e] = p * (dp[kt][qt][r] - dl[qt]);
            }
            dsp[qt][kt][pr] = pack_bf16(dsv[0], dsv[1]);
          }
      }
      // dQ^T += K^T dS^T over 4 chunks of 16 keys
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const bf16x8_t ka = read_tr(ks, lane, c, 32 * dt);
#pragma unroll
          for (int qt = 0; qt < 2; ++qt)
            dqacc[dt][qt] = mma(ka, chunk_op(dsp[qt][c >> 1], c & 1), dqacc[dt][qt]);
        }
    }
    if (pre) store_tile((t + 2) % kStages);
    __syncthreads();
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

hipError_t launch_bwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* o,
                           const __bf16* dout, const float* lse, __bf16* dq, __bf16* dk,
                           __bf16* dv, void* workspace, int64_t heads, int64_t N, double scale,
                           hipStream_t stream, const Timers& tm) {
  float* delta = (float*)workspace;
  const int64_t rows = heads * N;
  const float c = (float)(scale * 1.4426950408889634);
  const int nb = (int)((N + kBlk - 1) / kBlk);
  const unsigned grid = (unsigned)(8 * ((heads + 7) / 8) * nb);
  if (hipError_t e = mark(tm.start[kTimerBwdPre], stream)) return e;
  hipLaunchKernelGGL(bwd_delta_bf16, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, stream, o,
                     dout, delta, rows);
  if (hipError_t e = mark(tm.stop[kTimerBwdPre], stream)) return e;
  if (hipError_t e = mark(tm.start[kTimerBwdDkdv], stream)) return e;
  hipLaunchKernelGGL(bwd_dkdv_bf16, dim3(grid), dim3(kThreads), 0, stream, q, k, v, dout, lse,
                     delta, dk, dv, (int)heads, (int)N, nb, c, (float)scale);
  if (hipError_t e = mark(tm.stop[kTimerBwdDkdv], stream)) return e;
  if (hipError_t e = mark(tm.start[kTimerBwdDq], stream)) return e;
  hipLaunchKernelGGL(bwd_dq_bf16, dim3(grid), dim3(kThreads), 0, stream, q, k, v, dout, lse, delta,
                     dq, (int)heads, (int)N, nb, c, (float)scale);
  if (hipError_t e = mark(tm.stop[kTimerBwdDq], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
