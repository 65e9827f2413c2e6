// The long-table <-> matrix adapter (pages: "Show HN: automatic deduction of
// FlashAttention kernel from 25 lines of SQL", the demo script's helpers
// table() and matrix()): a T x D matrix is registered with the SQL engines as
// rows (t, d, x), one per cell, with t and d the row and column positions, and
// a (t, d, ...) result is pivoted back into a matrix.
//
// matrix -> rows: row r = t D + d is (t, d, m[t][d]), in (t, d) order (the
//   order of the forward's ORDER BY t, d).  One streaming pass.
// rows -> matrix: a cell no row names is NaN (a pivot fills holes), each row
//   gives its cell its x, a coordinate outside [0, T) x [0, D) is skipped, and
//   a cell named twice is an error.  Three passes and no per-row atomics
//   (scattered device atomics run at about a quarter of the rate of scattered
//   plain stores on this part):
//     1. clear a staging array in the caller's workspace (one word per cell:
//        the value's bits and a mark) and two counters;
//     2. each row stores its value, marked, into its cell's staging word (one
//        plain store, scattered unless the rows come in cell order) and counts
//        itself;
//     3. each cell takes its staged value, or NaN where unmarked, and the marked
//        cells are counted.
//   Two rows naming one cell leave one marked word for two counted rows, so
//   "some cell named twice" is exactly "marked cells < counted rows".
//   A first pass takes the common case whole: when there are T x D rows and
//   row r names cell r (the order of ORDER BY t, d), the matrix is a copy of
//   x.  That pass copies while it checks, and a workgroup stops as soon as any
//   row breaks the order; the three passes above then run only if one did
//   (each reads the flag and returns at once otherwise).  Status
//   bits in a device word (1: out of range, 2: named twice) are read by the
//   caller after synchronising; the matrix is unspecified when it is not 0.
//
// Values are moved as raw bits (2, 4 or 8 bytes), so the pivot is bit-exact
// for every element type.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThr = 256;
constexpr size_t kCounterBytes = 256;  // workspace head: two counters, then the order flag

// A cell's staging word: the value's bits and the mark of a row that named it.
template <typename U> struct StageOf;
template <> struct StageOf<uint16_t> {  // value | 1 << 16
  using type = uint32_t;
  __device__ static uint32_t make(uint16_t v) { return (uint32_t)v | 0x10000u; }
  __device__ static bool named(uint32_t s) { return (s >> 16) != 0; }
  __device__ static uint16_t value(uint32_t s) { return (uint16_t)(s & 0xffffu); }
};
template <> struct StageOf<uint32_t> {  // {value, 1}
  using type = uint2;
  __device__ static uint2 make(uint32_t v) { return make_uint2(v, 1u); }
  __device__ static bool named(uint2 s) { return s.y != 0; }
  __device__ static uint32_t value(uint2 s) { return s.x; }
};
template <> struct StageOf<uint64_t> {  // {low, high, 1, 0}
  using type = uint4;
  __device__ static uint4 make(uint64_t v) {
    return make_uint4((uint32_t)v, (uint32_t)(v >> 32), 1u, 0u);
  }
  __device__ static bool named(uint4 s) { return s.z != 0; }
  __device__ static uint64_t value(uint4 s) { return (uint64_t)s.x | ((uint64_t)s.y << 32); }
};

// Sum of one unsigned long long per thread over the workgroup, added to *dst
// by thread 0 (one device atomic per workgroup).
__device__ __forceinline__ void block_add(unsigned long long v, unsigned long long* dst) {
  __shared__ unsigned long long part[kThr / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
#pragma unroll
    for (int w = 0; w < kThr / 64; ++w) s += part[w];
    if (s) atomicAdd(dst, s);
  }
}

// Set-up: clear the counters and the status word; the order flag starts set
// unless there are exactly T x D rows.
__global__ void pivot_init(unsigned long long* __restrict__ counters, uint32_t* __restrict__ broken,
                           int32_t* __restrict__ status, int64_t rows, int64_t cells) {
  if (threadIdx.x == 0) {
    counters[0] = 0;
    counters[1] = 0;
    *broken = rows != cells;
    *status = 0;
  }
}

// The ordered pass: row r names cell r (and lies in range) -> copy its value;
// any other row sets the flag, and every workgroup returns once it sees the
// flag set.  (Element-sized accesses: t, d and x need only their natural
// alignment.)
template <typename U>
__global__ __launch_bounds__(kThr) void pivot_ordered(const int64_t* __restrict__ t,
                                                      const int64_t* __restrict__ d,
                                                      const U* __restrict__ x, int64_t rows,
                                                      int64_t T, int64_t D, U* __restrict__ out,
                                                      uint32_t* __restrict__ broken) {
  const int64_t stride = (int64_t)gridDim.x * kThr;
  for (int64_t r = (int64_t)blockIdx.x * kThr + threadIdx.x; r < rows; r += stride) {
    if (*(volatile uint32_t*)broken) return;
    const int64_t ti = t[r], di = d[r];
    if (ti >= 0 && ti < T && di >= 0 && di < D && ti * D + di == r) out[r] = x[r];
    else *broken = 1;
  }
}

// Pass 1: zero `words` 32-bit words of staging (16 bytes per store where it
// can).
__global__ __launch_bounds__(kThr) void pivot_clear(uint32_t* __restrict__ stage, int64_t words,
                                                    const uint32_t* __restrict__ broken) {
  if (!*broken) return;
  const int64_t stride = (int64_t)gridDim.x * kThr;
  const int64_t vec = words / 4;
  for (int64_t i = (int64_t)blockIdx.x * kThr + threadIdx.x; i < vec; i += stride)
    ((uint4*)stage)[i] = make_uint4(0, 0, 0, 0);
  for (int64_t i = vec * 4 + (int64_t)blockIdx.x * kThr + threadIdx.x; i < words; i += stride)
    stage[i] = 0;
}

// Pass 2: each row in range stores its marked value into its cell's staging
// word and counts itself (counters[0]); a row out of range sets status bit 1.
template <typename U>
__global__ __launch_bounds__(kThr) void pivot_stage(const int64_t* __restrict__ t,
                                                    const int64_t* __restrict__ d,
                                                    const U* __restrict__ x, int64_t rows,
                                                    int64_t T, int64_t D,
                                                    typename StageOf<U>::type* __restrict__ stage,
                                                    unsigned long long* __restrict__ counters,
                                                    int32_t* __restrict__ status,
                                                    const uint32_t* __restrict__ broken) {
  if (!*broken) return;
  using S = StageOf<U>;
  unsigned long long named = 0;
  int bad = 0;
  const int64_t stride = (int64_t)gridDim.x * kThr;
  for (int64_t r = (int64_t)blockIdx.x * kThr + threadIdx.x; r < rows; r += stride) {
    const int64_t ti = t[r], di = d[r];
    if (ti >= 0 && ti < T && di >= 0 && di < D) {
      stage[ti * D + di] = S::make(x[r]);
      ++named;
    } else {
      bad = 1;
    }
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(status, 1);
  block_add(named, counters);
}

// Pass 3: each cell takes its staged value, or the NaN pattern where no row
// named it; the named cells are counted (counters[1]).  kPer cells per step
// (16 bytes of staging words).
template <typename U>
__global__ __launch_bounds__(kThr) void pivot_emit(const typename StageOf<U>::type* __restrict__ stage,
                                                   int64_t cells, U* __restrict__ out, U nan_bits,
                                                   unsigned long long* __restrict__ counters,
                                                   const uint32_t* __restrict__ broken) {
  if (!*broken) return;
  using S = StageOf<U>;
  using W = typename S::type;
  constexpr int kPer = 16 / sizeof(W);
  unsigned long long named = 0;
  const int64_t stride = (int64_t)gridDim.x * kThr;
  const int64_t groups = cells / kPer;
  for (int64_t g = (int64_t)blockIdx.x * kThr + threadIdx.x; g < groups; g += stride) {
    W w[kPer];
    *(uint4*)w = ((const uint4*)stage)[g];
    U v[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const bool n = S::named(w[e]);
      named += n;
      v[e] = n ? S::value(w[e]) : nan_bits;
    }
    static_assert(kPer * sizeof(U) == 8, "a group is 8 bytes of output");
    *(uint2*)(out + g * kPer) = *(const uint2*)v;
  }
  for (int64_t c = groups * kPer + (int64_t)blockIdx.x * kThr + threadIdx.x; c < cells; c += stride) {
    const W w = stage[c];
    const bool n = S::named(w);
    named += n;
    out[c] = n ? S::value(w) : nan_bits;
  }
  block_add(named, counters + 1);
}

// Fewer marked cells than rows in range: some cell was named twice.
__global__ void pivot_check(const unsigned long long* __restrict__ counters,
                            int32_t* __restrict__ status) {
  if (threadIdx.x == 0 && counters[1] != counters[0]) atomicOr(status, 2);
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

size_t stage_bytes(int elem_bytes) { return elem_bytes == 8 ? 16 : elem_bytes == 4 ? 8 : 4; }

template <typename U>
hipError_t pivot(int64_t rows, const int64_t* t, const int64_t* d, const void* x, int64_t T,
                 int64_t D, void* out, int32_t* status, void* workspace, U nan_bits,
                 hipStream_t stream, const Timers& tm) {
  using W = typename StageOf<U>::type;
  const int64_t cells = T * D;
  unsigned long long* counters = (unsigned long long*)workspace;
  uint32_t* broken = (uint32_t*)(counters + 2);
  W* stage = (W*)((char*)workspace + kCounterBytes);
  const int64_t words = cells * (int64_t)(sizeof(W) / 4);
  if (hipError_t e = mark(tm.start[kTimerTable], stream)) return e;
  hipLaunchKernelGGL(pivot_init, dim3(1), dim3(64), 0, stream, counters, broken, status, rows,
                     cells);
  hipLaunchKernelGGL(pivot_ordered<U>, dim3(grid_for(rows)), dim3(kThr), 0, stream, t, d,
                     (const U*)x, rows, T, D, (U*)out, broken);
  hipLaunchKernelGGL(pivot_clear, dim3(grid_for(words / 4 + 1)), dim3(kThr), 0, stream,
                     (uint32_t*)stage, words, (const uint32_t*)broken);
  hipLaunchKernelGGL(pivot_stage<U>, dim3(grid_for(rows)), dim3(kThr), 0, stream, t, d,
                     (const U*)x, rows, T, D, stage, counters, status, (const uint32_t*)broken);
  hipLaunchKernelGGL(pivot_emit<U>, dim3(grid_for(cells / (16 / sizeof(W)) + 1)), dim3(kThr), 0,
                     stream, (const W*)stage, cells, (U*)out, nan_bits, counters,
                     (const uint32_t*)broken);
  hipLaunchKernelGGL(pivot_check, dim3(1), dim3(64), 0, stream, (const unsigned long long*)counters,
                     status);
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

size_t table_workspace_bytes(int elem_bytes, int64_t T, int64_t D) {
  // the counters, then one staging word per cell, in whole 16-byte stores
  return kCounterBytes + ((size_t)(T * D) * stage_bytes(elem_bytes) + 15) / 16 * 16;
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
