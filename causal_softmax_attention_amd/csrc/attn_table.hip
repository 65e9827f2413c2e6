// The long-table <-> matrix adapter (pages: "Show HN: automatic deduction of
// FlashAttention kernel from 25 lines of SQL", the demo script's helpers
// table() and matrix()): a T x D matrix is registered with the SQL engines as
// rows (t, d, x), one per cell, with t and d the row and column positions, and
// a (t, d, ...) result is pivoted back into a matrix.
//
// matrix -> rows: row r = t D + d is (t, d, m[t][d]), in (t, d) order (the
//   order of the forward's ORDER BY t, d).  One streaming pass.
// rows -> matrix: every cell starts as NaN (a cell no row names stays NaN, as
//   a pivot fills holes), then each row writes its cell.  A per-cell counter
//   in the caller's workspace catches a cell named twice; a coordinate outside
//   [0, T) x [0, D) is skipped.  Both set bits of a status word in device
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

// Fill the matrix with the NaN pattern and the counters with 0, 16 bytes per
// store; thread 0 clears the status word.
template <typename U>
__global__ __launch_bounds__(kThr) void pivot_fill(U* __restrict__ out, int32_t* __restrict__ count,
                                                   int64_t cells, U nan_bits,
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
  const int64_t cvec = cells / 4;
  for (int64_t i = (int64_t)blockIdx.x * kThr + threadIdx.x; i < cvec; i += stride)
    ((uint4*)count)[i] = make_uint4(0, 0, 0, 0);
  for (int64_t i = cvec * 4 + (int64_t)blockIdx.x * kThr + threadIdx.x; i < cells; i += stride)
    count[i] = 0;
}

// Each row writes its cell; the counter's previous value tells a second write.
template <typename U>
__global__ __launch_bounds__(kThr) void pivot_scatter(const int64_t* __restrict__ t,
                                                      const int64_t* __restrict__ d,
                                                      const U* __restrict__ x, int64_t rows,
                                                      int64_t T, int64_t D, U* __restrict__ out,
                                                      int32_t* __restrict__ count,
                                                      int32_t* __restrict__ status) {
  int flags = 0;
  const int64_t stride = (int64_t)gridDim.x * kThr;
  for (int64_t r = (int64_t)blockIdx.x * kThr + threadIdx.x; r < rows; r += stride) {
    const int64_t ti = t[r], di = d[r];
    if (ti < 0 || ti >= T || di < 0 || di >= D) {
      flags |= 1;
      continue;
    }
    const int64_t cell = ti * D + di;
    if (atomicAdd(count + cell, 1) != 0) flags |= 2;
    out[cell] = x[r];
  }
  // one status update per wave
  const int any1 = __any(flags & 1), any2 = __any(flags & 2);
  if ((threadIdx.x & 63) == 0 && (any1 | any2)) atomicOr(status, (any1 ? 1 : 0) | (any2 ? 2 : 0));
}

// Rows (t, d, x) of a T x D matrix in (t, d) order.  Each thread walks the
// cells i0, i0 + S, ... with (t, d) carried incrementally (no division per cell).
template <typename U>
__global__ __launch_bounds__(kThr) void matrix_rows(const U* __restrict__ m, int64_t cells, int64_t D,
                                                    int64_t* __restrict__ t, int64_t* __restrict__ d,
                                                    U* __restrict__ x) {
  const int64_t S = (int64_t)gridDim.x * kThr;
  int64_t i = (int64_t)blockIdx.x * kThr + threadIdx.x;
  if (i >= cells) return;
  const int64_t sq = S / D, sr = S % D;
  int64_t ti = i / D, di = i % D;
  for (; i < cells; i += S) {
    t[i] = ti;
    d[i] = di;
    x[i] = m[i];
    ti += sq;
    di += sr;
    if (di >= D) {
      di -= D;
      ti += 1;
    }
  }
}

unsigned grid_for(int64_t n) {
  const int64_t b = (n + kThr - 1) / kThr;
  return (unsigned)(b < 1 ? 1 : b > 8192 ? 8192 : b);
}

template <typename U>
hipError_t pivot(int64_t rows, const int64_t* t, const int64_t* d, const void* x, int64_t T,
                 int64_t D, void* out, int32_t* status, void* workspace, U nan_bits,
                 hipStream_t stream, const Timers& tm) {
  const int64_t cells = T * D;
  int32_t* count = (int32_t*)workspace;
  hipLaunchKernelGGL(pivot_fill<U>, dim3(grid_for(cells / 4 + 1)), dim3(kThr), 0, stream, (U*)out,
                     count, cells, nan_bits, status);
  if (hipError_t e = mark(tm.start[kTimerTable], stream)) return e;
  hipLaunchKernelGGL(pivot_scatter<U>, dim3(grid_for(rows)), dim3(kThr), 0, stream, t, d,
                     (const U*)x, rows, T, D, (U*)out, count, status);
  if (hipError_t e = mark(tm.stop[kTimerTable], stream)) return e;
  return hipGetLastError();
}

template <typename U>
hipError_t unpivot(int64_t T, int64_t D, const void* m, int64_t* t, int64_t* d, void* x,
                   hipStream_t stream) {
  const int64_t cells = T * D;
  hipLaunchKernelGGL(matrix_rows<U>, dim3(grid_for(cells)), dim3(kThr), 0, stream, (const U*)m,
                     cells, D, t, d, (U*)x);
  return hipGetLastError();
}

}  // namespace

size_t table_workspace_bytes(int64_t T, int64_t D) { return (size_t)T * D * sizeof(int32_t); }

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
