// Causal attention forward in float32 on gfx950 MFMA (v_mfma_f32_32x32x2f32).
//
// The method is the same as the bfloat16 forward (pages: "Show HN: automatic
// deduction of FlashAttention kernel from 25 lines of SQL", the view
// `attention` and the FlashAttention plan), computed entirely in float32: the
// MFMA multiplies float32 operands exactly and accumulates in float32.
//
// v_mfma_f32_32x32x2f32: with lane l = 32 h + i, A holds A[m = i][k = h],
// B holds B[k = h][n = i], C holds C[8(r/4) + 4h + r%4][n = i], r = 0..15.
//   * S^T = K Q^T: the contraction slot (step kk, half h) is feature 32 h + kk,
//     so a lane reads 32 consecutive floats of one K row (LDS) and keeps 32 of
//     its query row in registers.  Each lane owns one query column: the
//     softmax state is per lane, as in the bfloat16 kernel.
//   * O^T = V^T P^T: accumulator register r of a key tile is the B operand of
//     one MFMA whose two contraction slots are keys 8(r/4) + r%4 (h = 0) and
//     8(r/4) + 4 + r%4 (h = 1).  V is staged transposed in LDS ([feature][key]),
//     so the matching A operands for registers 4g..4g+3 are one 16-byte read.
// Float32 MFMAs dominate the time (128 per 32 x 64 tile per wave against about
// 100 VALU instructions), so each wave takes one 32-query column, two waves
// share a SIMD, and staging is plain double-buffered register copies.  Causal
// block skipping, the lazy max (exact max only when a lane's tile sum of
// weights exceeds 2^8) and the select path for masked tiles whose V holds
// inf/NaN follow the bfloat16 kernel.
#include "common.h"
#include "launch.h"
#include "mfma_bf16.h"

namespace attn {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;                 // queries per wave (one MFMA column)
constexpr int kBr = kQW * kWaves;       // queries per workgroup
constexpr int kBc = 64;                 // keys per tile
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 256.0f;
constexpr float kRefInit = -1e30f;  // initial reference exponent (see the kernel)

__device__ __forceinline__ floatx16 mma32(float a, float b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// float32 tiles: 64 rows of 64 floats padded to a 68-float stride, so the
// 16-byte reads of sixteen consecutive rows hit sixteen distinct bank groups and
// every read of a lane is its row base plus an immediate offset.
constexpr int kLd = 68;
__device__ __forceinline__ int at32(int row, int col) { return row * kLd + col; }

struct alignas(16) Smem {
  float k[2][kBc * kLd];       // [key][feature]
  float vt[2][kD * kLd];       // [feature][key]
  float p[kWaves][kQW * kBc];  // select path: the wave's weights as [query][key]
  int32_t seg[2][kBc];         // segment ids of the tile's keys (when they apply)
};

__device__ __forceinline__ bool finite4(float4 x) {
  return __builtin_isfinite(x.x) && __builtin_isfinite(x.y) && __builtin_isfinite(x.z) &&
         __builtin_isfinite(x.w);
}

// A pair (query i, key j) is absent when j >= N, or j > i under the causal
// predicate, or i - j >= band under a window of band keys.
__device__ __forceinline__ bool absent(int i, int j, int N, int causal, int band) {
  return j >= N || (causal && j > i) || (band && i - j >= band);
}

// SEG: segment ids apply (segk: the tile's key ids, sq: the lane's query id).
template <bool MASKED, bool SEG>
__device__ __forceinline__ void fwd_tile_f32(const float* ks, const float* vt, float* pscr,
                                             int lane, int k0, int qw, int N, float c_scale,
                                             int causal, int band, bool vnonfinite,
                                             const float (&qreg)[32], floatx16 (&oacc)[2],
                                             float& mref, float& lsum, const int32_t* segk,
                                             int32_t sq) {
  const int i32 = lane & 31, h = lane >> 5;
  const int qi = qw + i32;
  floatx16 s[2];  // [kt]: scores, then (in place) weights
  auto scores = [&]() {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      floatx16 acc = floatx16{};
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 x = *(const float4*)(ks + at32(32 * kt + i32, 32 * h + 4 * c));
        acc = mma32(x.x, qreg[4 * c + 0], acc);
        acc = mma32(x.y, qreg[4 * c + 1], acc);
        acc = mma32(x.z, qreg[4 * c + 2], acc);
        acc = mma32(x.w, qreg[4 * c + 3], acc);
      }
      s[kt] = acc;
    }
    if (MASKED) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        int32_t sk[16];  // ids of the lane's 16 keys of this half
        if (SEG) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int4 w = *(const int4*)(segk + 32 * kt + 8 * g + 4 * h);
            sk[4 * g + 0] = w.x; sk[4 * g + 1] = w.y; sk[4 * g + 2] = w.z; sk[4 * g + 3] = w.w;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int j = k0 + 32 * kt + acc_row(r, h);
          const bool gone = absent(qi, j, N, causal, band) || (SEG && sk[r] != sq);
          s[kt][r] = gone ? -__builtin_inff() : s[kt][r];
        }
      }
    }
  };
  float part = 0.f;
  auto weights = [&]() {
    const float nm = -mref;
    float acc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[kt][r] = __builtin_amdgcn_exp2f(fmaf(s[kt][r], c_scale, nm));
        acc += s[kt][r];
      }
    part = acc;
  };
  scores();
  weights();
  if (__any(!(part <= kTau))) {
    // rare exact path: scores again, raise the reference to the tile max, rescale
    scores();
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mref, mx * c_scale);
    if (mnew != mref) {
      const float alpha = __builtin_amdgcn_exp2f(mref - mnew);  // 0 from the initial reference
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      mref = mnew;
    }
    weights();
  }
  lsum += part;

  if (!(MASKED && vnonfinite)) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 va = *(const float4*)(vt + at32(32 * dt + i32, 32 * kt + 8 * g + 4 * h));
          oacc[dt] = mma32(va.x, s[kt][4 * g + 0], oacc[dt]);
          oacc[dt] = mma32(va.y, s[kt][4 * g + 1], oacc[dt]);
          oacc[dt] = mma32(va.z, s[kt][4 * g + 2], oacc[dt]);
          oacc[dt] = mma32(va.w, s[kt][4 * g + 3], oacc[dt]);
        }
  } else {
    // select path: a masked pair never multiplies (V holds inf/NaN)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) pscr[i32 * kBc + 32 * kt + acc_row(r, h)] = s[kt][r];
    __builtin_amdgcn_wave_barrier();
    for (int jj = 0; jj < kBc; ++jj) {
      const int j = k0 + jj;
      const float pj = pscr[i32 * kBc + jj];
      if (absent(qi, j, N, causal, band) || (SEG && segk[jj] != sq)) continue;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r2 = 0; r2 < 16; ++r2)
          oacc[dt][r2] += pj * vt[at32(32 * dt + acc_row(r2, h), jj)];
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// CAUSAL: the causal predicate applies; BANDED: a window of band_arg keys does;
// SEG: only pairs of equal segment ids (seg, [B][N], batch = head / hpb) exist.
template <bool CAUSAL, bool BANDED, bool SEG>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int heads, int N, int nqb, float c_scale,
    int band_arg, float* __restrict__ delta, const int32_t* __restrict__ seg, int hpb) {
  constexpr int causal = CAUSAL;
  const int band = BANDED ? band_arg : 0;
  __shared__ Smem sm;
  int head, qb;
  if (!mfma::map_block(blockIdx.x, heads, nqb, true, 4, head, qb)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const int qw = qb * kBr + wave * kQW;
  const int wq_last = min(qw + kQW, N) - 1;
  // segment ids: the lane's query id and the range of the wave's valid ids
  const int32_t* segrow = SEG ? seg + (size_t)(head / hpb) * N : nullptr;
  int32_t sq = 0, sqlo = 0, sqhi = 0, sreg = 0;
  if (SEG) {
    const int qi0 = qw + i32;
    sq = qi0 < N ? segrow[qi0] : 0;
    sqlo = qi0 < N ? sq : INT32_MAX;
    sqhi = qi0 < N ? sq : INT32_MIN;
#pragma unroll
    for (int o2 = 16; o2 >= 1; o2 >>= 1) {
      sqlo = min(sqlo, __shfl_xor(sqlo, o2));
      sqhi = max(sqhi, __shfl_xor(sqhi, o2));
    }
  }
  // keys of the workgroup's queries: from its first query's window start to
  // its last query (causal) or the end (full)
  int t0 = band ? max(0, qb * kBr - band + 1) / kBc : 0;
  const int kend = causal ? min(N, qb * kBr + kBr) : N;
  int ntiles = (kend + kBc - 1) / kBc;
  if (SEG) {
    // only the key tiles within the span of keys whose ids fall in the
    // block's query-id range (never empty: each query is also a key)
    __shared__ int32_t red[2][kWaves][4];
    const SegSpan sp = seg_span<kThreads>(segrow, N, qb * kBr, kBr, t0 * kBc, kend, threadIdx.x, red);
    t0 = __builtin_amdgcn_readfirstlane(sp.first / kBc);
    ntiles = __builtin_amdgcn_readfirstlane((sp.last + kBc - 1) / kBc);
  }
  const int wlo = band ? qw - band + 1 : 0, whi = causal ? wq_last : N - 1;  // keys of this wave
  const int qi = qw + i32;
  const bool active = qw < N;  // a wave past the end only joins the barriers

  float qreg[32];  // lane holds q[qi][32 h + kk]
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (qi < N) x = *(const float4*)(q + base + (size_t)qi * kD + 32 * h + 4 * c);
    qreg[4 * c] = x.x;
    qreg[4 * c + 1] = x.y;
    qreg[4 * c + 2] = x.z;
    qreg[4 * c + 3] = x.w;
  }
  floatx16 oacc[2] = {floatx16{}, floatx16{}};  // [dt]: O^T tile, lane holds the query column
  // reference exponent: finite, so a first tile whose pairs are all absent for
  // this lane gives weights exp2(-inf) = 0 (not -inf - -inf), and the first
  // tile with a present pair takes the exact path (its weights overflow)
  float mref = kRefInit, lsum = 0.f;

  // staging: a 64-key tile is 1024 16-byte chunks of K and of V, two per
  // thread.  K chunks go row-major (coalesced loads, contiguous stores); V
  // chunks go key-per-lane, so the transposed scalar stores of a wave land on
  // 64 consecutive keys of one feature row.
  float4 kreg[2], vreg[2];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + u * kThreads;
      const int jk = t * kBc + (c >> 4), jv = t * kBc + (c & 63);
      kreg[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      vreg[u] = kreg[u];
      if (jk < N) kreg[u] = *(const float4*)(k + base + (size_t)jk * kD + 4 * (c & 15));
      if (jv < N) vreg[u] = *(const float4*)(v + base + (size_t)jv * kD + 4 * (c >> 6));
    }
    if (SEG && tid < kBc) sreg = t * kBc + tid < N ? segrow[t * kBc + tid] : 0;
  };
  auto store_tile = [&](int buf) {
    bool fin = true;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = tid + u * kThreads, key = c & 63, d = 4 * (c >> 6);
      *(float4*)(&sm.k[buf][at32(c >> 4, 4 * (c & 15))]) = kreg[u];
      sm.vt[buf][at32(d + 0, key)] = vreg[u].x;
      sm.vt[buf][at32(d + 1, key)] = vreg[u].y;
      sm.vt[buf][at32(d + 2, key)] = vreg[u].z;
      sm.vt[buf][at32(d + 3, key)] = vreg[u].w;
      fin &= finite4(vreg[u]);
    }
    if (SEG && tid < kBc) sm.seg[buf][tid] = sreg;
    return fin;
  };

  load_tile(t0);
  // the barrier also ORs "this V tile holds a non-finite value" over the workgroup
  int vnonfinite = __syncthreads_or(!store_tile(0));
  for (int t = t0; t < ntiles; ++t) {
    const int buf = (t - t0) & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);
    const int k0 = t * kBc;
    if (active && k0 <= whi && k0 + kBc - 1 >= wlo) {
      // segments: no key id in the wave's id range -> no pair; all ids one and
      // the same -> the ids mask nothing (keys past N are masked anyway)
      bool seg_some = true, seg_one = true;
      if (SEG) {
        const int32_t skey = sm.seg[buf][lane];
        const bool kin = k0 + lane < N;
        seg_some = __any(kin && skey >= sqlo && skey <= sqhi);
        seg_one = sqlo == sqhi && __all(!kin || skey == sqlo);
      }
      // masked: some pair of the tile is absent for some query of the wave
      if (!seg_some) {
      } else if ((causal && k0 + kBc - 1 > qw) || (k0 + kBc > N) ||
                 (band && k0 < qw + kQW - band) || !seg_one) {
        fwd_tile_f32<true, SEG>(sm.k[buf], sm.vt[buf], sm.p[wave], lane, k0, qw, N, c_scale,
                                causal, band, vnonfinite != 0, qreg, oacc, mref, lsum,
                                sm.seg[buf], sq);
      } else {
        fwd_tile_f32<false, SEG>(sm.k[buf], sm.vt[buf], sm.p[wave], lane, k0, qw, N, c_scale,
                                 causal, band, false, qreg, oacc, mref, lsum, sm.seg[buf], sq);
      }
    }
    const bool fin = more ? store_tile(buf ^ 1) : true;
    vnonfinite = __syncthreads_or(!fin);
  }

  // epilogue; with delta given (the loss sum(o^2)/2, so dO = O) also the
  // backward's per-row delta_i = |o_i|^2
  const float l = lsum + __shfl_xor(lsum, 32);
  const float inv = 1.0f / l;
  if (qi < N) {
    float sq = 0.f;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        const float4 x = make_float4(oacc[dt][4 * g] * inv, oacc[dt][4 * g + 1] * inv,
                                     oacc[dt][4 * g + 2] * inv, oacc[dt][4 * g + 3] * inv);
        *(float4*)(o + base + (size_t)qi * kD + d) = x;
        sq = fmaf(x.x, x.x, fmaf(x.y, x.y, fmaf(x.z, x.z, fmaf(x.w, x.w, sq))));
      }
    if (h == 0) lse[(size_t)head * N + qi] = (mref + __log2f(l)) * kLn2;
    if (delta) {
      sq += __shfl_xor(sq, 32);  // the partner lane holds the row's other 32 features
      if (h == 0) delta[(size_t)head * N + qi] = sq;
    }
  }
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int64_t heads, int64_t N, double scale, const Mask& mk, void* bwd_ws,
                          hipStream_t stream, const Timers& tm) {
  const int nqb = (int)((N + kBr - 1) / kBr);
  const unsigned grid = (unsigned)(8 * ((heads + 7) / 8) * nqb);
  const float c = (float)(scale * 1.4426950408889634);
  auto kern = mk.seg ? (mk.band > 0 ? attn_fwd_f32_kernel<true, true, true>
                        : mk.causal ? attn_fwd_f32_kernel<true, false, true>
                                    : attn_fwd_f32_kernel<false, false, true>)
                     : (mk.band > 0 ? attn_fwd_f32_kernel<true, true, false>
                        : mk.causal ? attn_fwd_f32_kernel<true, false, false>
                                    : attn_fwd_f32_kernel<false, false, false>);
  if (hipError_t e = mark(tm.start[kTimerFwd], stream)) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse, (int)heads,
                     (int)N, nqb, c, mk.band, (float*)bwd_ws, mk.seg, mk.hpb);
  if (hipError_t e = mark(tm.stop[kTimerFwd], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
