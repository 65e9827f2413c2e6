// The long-table <-> matrix adapter (pages: "Show HN: automatic deduction of
// FlashAttention kernel from 25 lines of SQL", the demo script's helpers
// table() and matrix()): a T x D matrix is registered with the SQL engines as
// rows (t, d, x), one per cell, with t and d the row and column positions, and
// a (t, d, ...) result is pivoted back into a matrix.
//
// matrix -> rows: row r = t D + d is (t, d, m[t][d]), in (t, d) order (the
//   order of the forward's ORDER BY t, d).  One streaming pass.
// rows -> matrix: every cell starts as NaN (a cell no row names stays NaN, as
//   a pivot fills holes), then each row writes its cell.  A bitmap in the
//   caller's workspace (one bit per cell, set with atomicOr) catches a cell
//   named twice; a coordinate outside [0, T) x [0, D) is skipped.  Both set bits of a status word in device
//   memory (1: out of range, 2: named twice) that the caller reads after
//   synchronising; the matrix is unspecified when the status is not 0.
//
// Values are moved as raw bits (2, 4 or 8 bytes), so the pivot is bit-exact
// for every element type.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThr = 256;

// Fill the matrix with the NaN pattern and the bitmap (`words` 32-bit words)
// with 0, 16 bytes per store; thread 0 clears the status word.
template <typename U>
__global__ __launch_bounds__(kThr) void pivot_fill(U* __restrict__ out, uint32_t* __restrict__ seen,
                                                   int64_t cells, int64_t words, U nan_bits,
                                                   int32_t* __restrict__ status) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *status = 0;
  constexpr int kPer = 16 / sizeof(U);
  U pat[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) pat[e] = nan_bits;
  const uint4 nan16 = *(const uint4*)pat;
  const int64_t stride = (int64_t)gridDim.x * kThr;
  const int64_t vec = cells / kPer;
  for (int64_t i = (int64_t)blockIdx.x * kThr + threadIdx.x; i < vec; i += stride)
    ((uint4*)out)[i] = nan16;
  for (int64_t i = vec * kPer + (int64_t)blockIdx.x * kThr + threadIdx.x; i < cells; i += stride)
    out[i] = nan_bits;
  const int64_t wvec = words / 4;
  for (int64_t i = (int64_t)blockIdx.x * kThr + threadIdx.x; i < wvec; i += stride)
    ((uint4*)seen)[i] = make_uint4(0, 0, 0, 0);
  for (int64_t i = wvec * 4 + (int64_t)blockIdx.x * kThr + threadIdx.x; i < words; i += stride)
    seen[i] = 0;
}

// Each row writes its cell; the cell's bit, already set, tells a second write.
// A wave whose 64 rows name 64 consecutive cells (rows in (t, d) order, as the
// forward's ORDER BY returns them) sets the bits of that run with one atomicOr
// per 32-bit word it covers (at most three) instead of 64 on the same words.
template <typename U>
__global__ __launch_bounds__(kThr) void pivot_scatter(const int64_t* __restrict__ t,
                                                      const int64_t* __restrict__ d,
                                                      const U* __restrict__ x, int64_t rows,
                                                      int64_t T, int64_t D, U* __restrict__ out,
                                                      uint32_t* __restrict__ seen,
                                                      int32_t* __restrict__ status) {
  int flags = 0;
  const int lane = threadIdx.x & 63;
  const int64_t stride = (int64_t)gridDim.x * kThr;
  const int64_t first = (int64_t)blockIdx.x * kThr + (threadIdx.x & ~63);  // the wave's first row
  for (int64_t r0 = first; r0 < rows; r0 += stride) {
    const int64_t r = r0 + lane;
    const bool live = r < rows;
    int64_t cell = -1;
    bool ok = false;
    if (live) {
      const int64_t ti = t[r], di = d[r];
      ok = ti >= 0 && ti < T && di >= 0 && di < D;
      if (!ok) flags |= 1;
      cell = ok ? ti * D + di : -1;
    }
    // a run of 64 consecutive cells across the wave (all rows live and in range)
    const int64_t c0 = __shfl(cell, 0);
    const bool run = __all(live && ok && cell == c0 + lane);
    if (run) {
      // bits [c0, c0 + 64) span words w0 .. w0 + 2; lane k < 3 owns word w0 + k
      const int64_t w0 = c0 >> 5;
      const int sh = (int)(c0 & 31);
      if (lane < 3) {
        // bits of word w0 + lane covered by the run [sh, sh + 64) (relative to w0)
        const int lo = 32 * lane, hi = lo + 32;
        const int a = sh > lo ? sh : lo, b = sh + 64 < hi ? sh + 64 : hi;
        if (a < b) {
          const uint32_t mask = (b - a == 32 ? 0xffffffffu : ((1u << (b - a)) - 1u)) << (a - lo);
          if (atomicOr(seen + w0 + lane, mask) & mask) flags |= 2;
        }
      }
    } else if (live && ok) {
      const uint32_t bit = 1u << (cell & 31);
      if (atomicOr(seen + (cell >> 5), bit) & bit) flags |= 2;
    }
    if (live && ok) out[cell] = x[r];
  }
  // one status update per wave
  const int any1 = __any(flags & 1), any2 = __any(flags & 2);
  if (lane == 0 && (any1 | any2)) atomicOr(status, (any1 ? 1 : 0) | (any2 ? 2 : 0));
}

// Rows (t, d, x) of a T x D matrix in (t, d) order.  A thread handles pairs of
// consecutive cells, so consecutive lanes store consecutive 16-byte (t, d)
// pairs; it walks pairs i0, i0 + S, ... with (t, d) of the pair's first cell
// carried incrementally (no division per pair).
template <typename U>
__global__ __launch_bounds__(kThr) void matrix_rows(const U* __restrict__ m, int64_t cells, int64_t D,
                                                    int64_t* __restrict__ t, int64_t* __restrict__ d,
                                                    U* __restrict__ x) {
  typedef __attribute__((__vector_size__(2 * sizeof(U)))) U U2;
  const int64_t pairs = cells / 2;
  const int64_t S = (int64_t)gridDim.x * kThr;  // pairs per sweep
  int64_t p = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (p < pairs) {
    const int64_t step = 2 * S, sq = step / D, sr = step % D;
    int64_t ti = (2 * p) / D, di = (2 * p) % D;
    for (; p < pairs; p += S) {
      const int64_t i = 2 * p;
      const int64_t t1 = di + 1 == D ? ti + 1 : ti, d1 = di + 1 == D ? 0 : di + 1;
      *(longlong2*)(t + i) = make_longlong2(ti, t1);
      *(longlong2*)(d + i) = make_longlong2(di, d1);
      *(U2*)(x + i) = *(const U2*)(m + i);
      ti += sq;
      di += sr;
      if (di >= D) {
        di -= D;
        ti += 1;
      }
    }
  }
  // an odd last cell
  if (blockIdx.x == 0 && threadIdx.x == 0 && (cells & 1)) {
    const int64_t j = cells - 1;
    t[j] = j / D;
    d[j] = j % D;
    x[j] = m[j];
  }
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + kThr - 1) / kThr;
  return (unsigned)(b < 1 ? 1 : b > 8192 ? 8192 : b);
}

int64_t bitmap_words(int64_t cells) { return (cells + 31) / 32; }

template <typename U>
hipError_t pivot(int64_t rows, const int64_t* t, const int64_t* d, const void* x, int64_t T,
                 int64_t D, void* out, int32_t* status, void* workspace, U nan_bits,
                 hipStream_t stream, const Timers& tm) {
  const int64_t cells = T * D;
  uint32_t* seen = (uint32_t*)workspace;
  hipLaunchKernelGGL(pivot_fill<U>, dim3(grid_for(cells / 8 + 1)), dim3(kThr), 0, stream, (U*)out,
                     seen, cells, bitmap_words(cells), nan_bits, status);
  if (hipError_t e = mark(tm.start[kTimerTable], stream)) return e;
  hipLaunchKernelGGL(pivot_scatter<U>, dim3(grid_for(rows)), dim3(kThr), 0, stream, t, d,
                     (const U*)x, rows, T, D, (U*)out, seen, status);
  if (hipError_t e = mark(tm.stop[kTimerTable], stream)) return e;
  return hipGetLastError();
}

template <typename U>
hipError_t unpivot(int64_t T, int64_t D, const void* m, int64_t* t, int64_t* d, void* x,
                   hipStream_t stream) {
  const int64_t cells = T * D;
  hipLaunchKernelGGL(matrix_rows<U>, dim3(grid_for(cells / 2 + 1)), dim3(kThr), 0, stream,
                     (const U*)m, cells, D, t, d, (U*)x);
  return hipGetLastError();
}

}  // namespace

size_t table_workspace_bytes(int64_t T, int64_t D) {
  return (size_t)((bitmap_words(T * D) + 3) / 4 * 16);  // whole 16-byte stores
}

hipError_t launch_table_to_matrix(int elem_bytes, int64_t rows, const int64_t* t, const int64_t* d,
                                  const void* x, int64_t T, int64_t D, void* out, int32_t* status,
                                  void* workspace, hipStream_t stream, const Timers& tm) {
  // quiet NaN of float64, float32, bfloat16
  switch (elem_bytes) {
    case 8: return pivot<uint64_t>(rows, t, d, x, T, D, out, status, workspace,
                                   (uint64_t)0x7ff8000000000000ull, stream, tm);
    case 4: return pivot<uint32_t>(rows, t, d, x, T, D, out, status, workspace, 0x7fc00000u,
                                   stream, tm);
    default: return pivot<uint16_t>(rows, t, d, x, T, D, out, status, workspace,
                                    (uint16_t)0x7fc0u, stream, tm);
  }
}

hipError_t launch_matrix_to_table(int elem_bytes, int64_t T, int64_t D, const void* m, int64_t* t,
                                  int64_t* d, void* x, hipStream_t stream) {
  switch (elem_bytes) {
    case 8: return unpivot<uint64_t>(T, D, m, t, d, x, stream);
    case 4: return unpivot<uint32_t>(T, D, m, t, d, x, stream);
    default: return unpivot<uint16_t>(T, D, m, t, d, x, stream);
  }
}

}  // namespace attn
