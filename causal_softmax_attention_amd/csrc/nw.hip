// Nadaraya-Watson Gaussian-kernel average (pages: "Show HN: automatic deduction
// of FlashAttention kernel from 25 lines of SQL", the NADARAYA_WATSON query and
// check_nadaraya_watson): out_p = sum_q w_pq v_q / sum_q w_pq over every source,
// w_pq = exp(-((tx_p - sx_q)^2 + (ty_p - sy_q)^2) / denom).
//
// A workgroup takes 64 targets (one per lane) and its four waves split the
// sources into four contiguous ranges, so every SIMD runs four waves that
// hide one another's exp and load latency.  All lanes of a wave walk the same
// source, so the source columns are read with wave-uniform (scalar) loads and
// each pair costs only VALU work: 2 sub, mul, 2 fma, exp2, add, fma.  The
// distance is formed directly, (dx^2 + dy^2), not expanded into
// |t|^2 + |s|^2 - 2 t.s, which would cancel catastrophically at coordinates ~10.
//
// Running max, lazily: weights are exp2(e - m) in base 2, where m is a
// reference exponent that only ever equals the exact max of some source tile
// already seen, so sum_q w >= 1 holds over a wave's range and nothing
// underflows to 0/0.  A tile whose weights exceed 2^64 (including inf) is
// recomputed after m is raised to that tile's exact max and the running sums
// are rescaled; 2^64 times the number of sources stays far below float32's
// range.  The four ranges' (m, l, acc) are merged at the end against their
// largest m.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kSrcTile = 64;

__device__ __forceinline__ float tile_min_d2(float x, float y, const float* __restrict__ sx,
                                             const float* __restrict__ sy, int j0, int jn) {
  float dmin = __builtin_inff();
  for (int jj = 0; jj < jn; ++jj) {
    const float dx = x - sx[j0 + jj], dy = y - sy[j0 + jj];
    dmin = fminf(dmin, fmaf(dy, dy, dx * dx));
  }
  return dmin;
}

// Weights of sources [j0, j0 + jn) against reference exponent m: returns their
// sum in lt and sum of w v in at.  Two partial sums each, to shorten the
// dependent add chains.
template <int JN>
__device__ __forceinline__ void tile_sums(float x, float y, const float* __restrict__ sx,
                                          const float* __restrict__ sy,
                                          const float* __restrict__ sv, int j0, int jn,
                                          float kexp, float m, float& lt, float& at) {
  const float nm = -m;
  float l0 = 0.f, l1 = 0.f, a0 = 0.f, a1 = 0.f;
  const int n = JN > 0 ? JN : jn;
#pragma unroll 16
  for (int jj = 0; jj < n; ++jj) {
    const float dx = x - sx[j0 + jj], dy = y - sy[j0 + jj];
    const float d2 = fmaf(dy, dy, dx * dx);
    const float w = __builtin_amdgcn_exp2f(fmaf(d2, -kexp, nm));
    if (jj & 1) {
      l1 += w;
      a1 = fmaf(w, sv[j0 + jj], a1);
    } else {
      l0 += w;
      a0 = fmaf(w, sv[j0 + jj], a0);
    }
  }
  lt = l0 + l1;
  at = a0 + a1;
}

__global__ __launch_bounds__(kThreads) void nw_kernel(int nt, const float* __restrict__ tx,
                                                      const float* __restrict__ ty, int ns,
                                                      const float* __restrict__ sx,
                                                      const float* __restrict__ sy,
                                                      const float* __restrict__ sv, float kexp,
                                                      int chunk, float* __restrict__ out) {
  __shared__ float part[3][kWaves - 1][64];  // (m, l, acc) of waves 1..3
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int p = blockIdx.x * 64 + lane;
  const bool valid = p < nt;
  const float x = valid ? tx[p] : 0.f, y = valid ? ty[p] : 0.f;
  const int js = min(ns, wave * chunk), je = min(ns, js + chunk);  // this wave's sources

  // m: reference exponent (base 2) = -kexp * (smallest d^2 in the range's first
  // tile); -inf for an empty range, whose l and acc stay 0.
  float m = -kexp * tile_min_d2(x, y, sx, sy, js, min(kSrcTile, je - js));
  float l = 0.f, acc = 0.f;
  for (int j0 = js; j0 < je; j0 += kSrcTile) {
    const int jn = min(kSrcTile, je - j0);
    float lt, at;
    if (jn == kSrcTile) tile_sums<kSrcTile>(x, y, sx, sy, sv, j0, jn, kexp, m, lt, at);
    else tile_sums<0>(x, y, sx, sy, sv, j0, jn, kexp, m, lt, at);
    if (!(lt <= 0x1p64f)) {  // this tile holds a much larger weight: raise m, redo it
      const float mn = -kexp * tile_min_d2(x, y, sx, sy, j0, jn);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      acc *= alpha;
      m = mn;
      tile_sums<0>(x, y, sx, sy, sv, j0, jn, kexp, m, lt, at);
    }
    l += lt;
    acc += at;
  }
  if (wave > 0) {
    part[0][wave - 1][lane] = m;
    part[1][wave - 1][lane] = l;
    part[2][wave - 1][lane] = acc;
  }
  __syncthreads();
  if (wave == 0 && valid) {
    float mm = m;
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) mm = fmaxf(mm, part[0][w][lane]);
    float L = l * __builtin_amdgcn_exp2f(m - mm), A = acc * __builtin_amdgcn_exp2f(m - mm);
#pragma unroll
    for (int w = 0; w < kWaves - 1; ++w) {
      const float a = __builtin_amdgcn_exp2f(part[0][w][lane] - mm);
      L = fmaf(part[1][w][lane], a, L);
      A = fmaf(part[2][w][lane], a, A);
    }
    out[p] = A / L;
  }
}

}  // namespace

hipError_t launch_nw(int64_t n_targets, const float* tx, const float* ty, int64_t n_sources,
                     const float* sx, const float* sy, const float* sv, float denom, float* out,
                     hipStream_t stream, const Timers& tm) {
  const float kexp = (float)(1.4426950408889634 / (double)denom);  // log2(e) / denom
  const unsigned blocks = (unsigned)((n_targets + 63) / 64);
  // sources per wave: a quarter of them, rounded up to whole tiles
  const int64_t chunk = ((n_sources + kWaves - 1) / kWaves + kSrcTile - 1) / kSrcTile * kSrcTile;
  if (hipError_t e = mark(tm.start[kTimerNw], stream)) return e;
  hipLaunchKernelGGL(nw_kernel, dim3(blocks), dim3(kThreads), 0, stream, (int)n_targets, tx, ty,
                     (int)n_sources, sx, sy, sv, kexp, (int)chunk, out);
  if (hipError_t e = mark(tm.stop[kTimerNw], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
