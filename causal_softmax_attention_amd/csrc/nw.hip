// Nadaraya-Watson Gaussian-kernel average (pages: "Show HN: automatic deduction
// of FlashAttention kernel from 25 lines of SQL", the NADARAYA_WATSON query and
// check_nadaraya_watson): out_p = sum_q w_pq v_q / sum_q w_pq over every source,
// w_pq = exp(-((tx_p - sx_q)^2 + (ty_p - sy_q)^2) / denom).
//
// One lane per target; all lanes of a wave walk the same source, so the source
// columns are read with wave-uniform (scalar) loads and each pair costs only
// VALU work: 2 sub, mul, 2 fma, exp2, add, fma.  The distance is formed
// directly, (dx^2 + dy^2), not expanded into |t|^2 + |s|^2 - 2 t.s, which would
// cancel catastrophically at coordinates ~10.
//
// Running max, lazily: weights are exp2(e - m) in base 2, where m is a
// reference exponent that only ever equals the exact max of some source tile
// already seen, so sum_q w >= 1 holds and nothing underflows to 0/0.  A tile
// whose weights exceed 2^64 (including inf) is recomputed after m is raised to
// that tile's exact max and the running sums are rescaled; 2^64 times the
// number of sources stays far below float32's range.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;
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

__global__ __launch_bounds__(kThreads) void nw_kernel(int nt, const float* __restrict__ tx,
                                                      const float* __restrict__ ty, int ns,
                                                      const float* __restrict__ sx,
                                                      const float* __restrict__ sy,
                                                      const float* __restrict__ sv, float kexp,
                                                      float* __restrict__ out) {
  const int p = blockIdx.x * kThreads + threadIdx.x;
  const bool valid = p < nt;
  const float x = valid ? tx[p] : 0.f, y = valid ? ty[p] : 0.f;
  // m: reference exponent (base 2) = -kexp * (smallest d^2 in the first tile)
  float m = -kexp * tile_min_d2(x, y, sx, sy, 0, min(kSrcTile, ns));
  float l = 0.f, acc = 0.f;
  for (int j0 = 0; j0 < ns; j0 += kSrcTile) {
    const int jn = min(kSrcTile, ns - j0);
    float lt = 0.f, at = 0.f;
    const float nm = -m;
    if (jn == kSrcTile) {
#pragma unroll 16
      for (int jj = 0; jj < kSrcTile; ++jj) {
        const float dx = x - sx[j0 + jj], dy = y - sy[j0 + jj];
        const float d2 = fmaf(dy, dy, dx * dx);
        const float w = __builtin_amdgcn_exp2f(fmaf(d2, -kexp, nm));
        lt += w;
        at = fmaf(w, sv[j0 + jj], at);
      }
    } else {
      for (int jj = 0; jj < jn; ++jj) {
        const float dx = x - sx[j0 + jj], dy = y - sy[j0 + jj];
        const float d2 = fmaf(dy, dy, dx * dx);
        const float w = __builtin_amdgcn_exp2f(fmaf(d2, -kexp, nm));
        lt += w;
        at = fmaf(w, sv[j0 + jj], at);
      }
    }
    if (!(lt <= 0x1p64f)) {  // this tile holds a much larger weight: raise m, redo it
      const float mn = -kexp * tile_min_d2(x, y, sx, sy, j0, jn);
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      l *= alpha;
      acc *= alpha;
      m = mn;
      lt = 0.f;
      at = 0.f;
      for (int jj = 0; jj < jn; ++jj) {
        const float dx = x - sx[j0 + jj], dy = y - sy[j0 + jj];
        const float d2 = fmaf(dy, dy, dx * dx);
        const float w = __builtin_amdgcn_exp2f(fmaf(d2, -kexp, -m));
        lt += w;
        at = fmaf(w, sv[j0 + jj], at);
      }
    }
    l += lt;
    acc += at;
  }
  if (valid) out[p] = acc / l;
}

}  // namespace

hipError_t launch_nw(int64_t n_targets, const float* tx, const float* ty, int64_t n_sources,
                     const float* sx, const float* sy, const float* sv, float denom, float* out,
                     hipStream_t stream, const Timers& tm) {
  const float kexp = (float)(1.4426950408889634 / (double)denom);  // log2(e) / denom
  const unsigned blocks = (unsigned)((n_targets + kThreads - 1) / kThreads);
  if (hipError_t e = mark(tm.start[kTimerNw], stream)) return e;
  hipLaunchKernelGGL(nw_kernel, dim3(blocks), dim3(kThreads), 0, stream, (int)n_targets, tx, ty,
                     (int)n_sources, sx, sy, sv, kexp, out);
  if (hipError_t e = mark(tm.stop[kTimerNw], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
