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
//   a cell named twice is an error.  No per-row device atomics (scattered
//   device atomics run at about a quarter of the rate of scattered plain
//   stores on this part).  Small tables take three passes (large ones their
//   binned form, below):
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

// Sum of one unsigned long long per thread over the workgroup of THR threads,
// added to *dst by thread 0 (one device atomic per workgroup).
template <int THR = kThr>
__device__ __forceinline__ void block_add(unsigned long long v, unsigned long long* dst) {
  __shared__ unsigned long long part[THR / 64];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
#pragma unroll
    for (int w = 0; w < THR / 64; ++w) s += part[w];
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

// ---- the binned form of passes 2 and 3, for large shuffled tables ----------
//
// The staging pass stores one scattered word per row, and a scattered store
// costs a whole 32-byte memory sector.  For large tables the rows are first
// sorted into bins of 2^bits consecutive cells (a counting sort: per-workgroup
// counts, their prefix sums, then a scatter into each bin's own range), so
// that one workgroup per bin can assemble its cells in LDS and write them out
// in order.  The counts and checks are those of the staging form.
constexpr int kBinThr = 1024;   // threads of the counting, scatter and emit passes
constexpr int kBinWGs = 256;    // workgroups of the counting and scatter passes
constexpr int kMaxBins = 4096;  // bins (LDS counters of the counting and scatter passes)
constexpr int kBinLds = 128 * 1024;  // bytes of one bin's staging words in LDS

// A sorted row: its cell within the bin (as index + 1, so 0 means empty) and
// its value's bits.
template <typename U> struct EntryOf;
template <> struct EntryOf<uint16_t> {  // value | (local + 1) << 16, local < 2^15
  using type = uint32_t;
  __device__ static uint32_t make(uint32_t local, uint16_t v) { return (uint32_t)v | ((local + 1) << 16); }
  __device__ static uint32_t local(uint32_t e) { return (e >> 16) - 1; }
  __device__ static uint16_t value(uint32_t e) { return (uint16_t)(e & 0xffffu); }
};
template <> struct EntryOf<uint32_t> {  // {value, local + 1}
  using type = uint2;
  __device__ static uint2 make(uint32_t local, uint32_t v) { return make_uint2(v, local + 1); }
  __device__ static uint32_t local(uint2 e) { return e.y - 1; }
  __device__ static uint32_t value(uint2 e) { return e.x; }
};
template <> struct EntryOf<uint64_t> {  // {low, high, local + 1, 0}
  using type = uint4;
  __device__ static uint4 make(uint32_t local, uint64_t v) {
    return make_uint4((uint32_t)v, (uint32_t)(v >> 32), local + 1, 0u);
  }
  __device__ static uint32_t local(uint4 e) { return e.z - 1; }
  __device__ static uint64_t value(uint4 e) { return (uint64_t)e.x | ((uint64_t)e.y << 32); }
};

// Counting: workgroup w counts its rows [w chunk, (w + 1) chunk) per bin in
// LDS and writes the counts to hist[w][bin]; a row out of range sets status
// bit 1.
__global__ __launch_bounds__(kBinThr) void bin_count(const int64_t* __restrict__ t,
                                                     const int64_t* __restrict__ d, int64_t rows,
                                                     int64_t T, int64_t D, int64_t chunk, int bits,
                                                     int nbins, uint32_t* __restrict__ hist,
                                                     int32_t* __restrict__ status,
                                                     const uint32_t* __restrict__ broken) {
  if (!*broken) return;
  __shared__ uint32_t h[kMaxBins];
  for (int i = threadIdx.x; i < nbins; i += kBinThr) h[i] = 0;
  __syncthreads();
  int bad = 0;
  const int64_t r0 = (int64_t)blockIdx.x * chunk, r1 = min(rows, r0 + chunk);
  for (int64_t r = r0 + threadIdx.x; r < r1; r += kBinThr) {
    const int64_t ti = t[r], di = d[r];
    if (ti >= 0 && ti < T && di >= 0 && di < D) atomicAdd(&h[(ti * D + di) >> bits], 1u);
    else bad = 1;
  }
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(status, 1);
  __syncthreads();
  for (int i = threadIdx.x; i < nbins; i += kBinThr) hist[(size_t)blockIdx.x * nbins + i] = h[i];
}

// Exclusive prefix of v over the workgroup's THR threads (all call it).
template <int THR>
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t& total) {
  __shared__ uint32_t wsum[THR / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t u = __shfl_up(inc, o);
    if (lane >= o) inc += u;
  }
  if (lane == 63) wsum[wave] = inc;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < THR / 64; ++w) {
    before += w < wave ? wsum[w] : 0u;
    total += wsum[w];
  }
  return before + inc - v;
}

// Per bin (workgroup b): the exclusive prefix of its counts over the counting
// workgroups, in place in hist[w][b], and the bin's total in base[b].
__global__ __launch_bounds__(kBinWGs) void bin_prefix(uint32_t* __restrict__ hist, int nwg,
                                                      int nbins, uint32_t* __restrict__ base,
                                                      const uint32_t* __restrict__ broken) {
  if (!*broken) return;
  const int b = blockIdx.x, w = threadIdx.x;
  const uint32_t v = w < nwg ? hist[(size_t)w * nbins + b] : 0u;
  uint32_t total;
  const uint32_t e = block_exclusive_scan<kBinWGs>(v, total);
  if (w < nwg) hist[(size_t)w * nbins + b] = e;
  if (w == 0) base[b] = total;
}

// The bins' first slots (exclusive prefix of their totals, in place in base,
// with base[nbins] = the rows in range, also counters[0]).  More rows in range
// than cells means a cell named twice: status bit 2, and the later passes stop
// (the sorted rows would not fit).
__global__ __launch_bounds__(kBinThr) void bin_bases(uint32_t* __restrict__ base, int nbins,
                                                     int64_t cells,
                                                     unsigned long long* __restrict__ counters,
                                                     uint32_t* __restrict__ overflow,
                                                     int32_t* __restrict__ status,
                                                     const uint32_t* __restrict__ broken) {
  if (!*broken) return;
  constexpr int kPer = kMaxBins / kBinThr;
  uint32_t v[kPer], sum = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = threadIdx.x * kPer + e;
    v[e] = i < nbins ? base[i] : 0u;
    sum += v[e];
  }
  uint32_t total;
  uint32_t run = block_exclusive_scan<kBinThr>(sum, total);
  __syncthreads();  // every thread has read base before it is overwritten
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = threadIdx.x * kPer + e;
    if (i < nbins) base[i] = run;
    run += v[e];
  }
  if (threadIdx.x == 0) {
    base[nbins] = total;
    counters[0] = total;
    const bool over = (int64_t)total > cells;
    *overflow = over;
    if (over) atomicOr(status, 2);
  }
}

// Scatter: workgroup w's rows (the counting pass's chunk) go to their bins'
// ranges.  A row's own scattered store would cost a whole memory sector, so
// the rows are taken kSub at a time and sorted by bin in LDS first (counts by
// LDS atomics, their prefix sum, then each row to its place); each wave then
// copies whole bins' runs to their global slots, so consecutive lanes store
// consecutive words.
template <typename U>
__global__ __launch_bounds__(kBinThr) void bin_scatter(const int64_t* __restrict__ t,
                                                       const int64_t* __restrict__ d,
                                                       const U* __restrict__ x, int64_t rows,
                                                       int64_t T, int64_t D, int64_t chunk,
                                                       int bits, int nbins,
                                                       const uint32_t* __restrict__ hist,
                                                       const uint32_t* __restrict__ base,
                                                       typename EntryOf<U>::type* __restrict__ sorted,
                                                       const uint32_t* __restrict__ broken,
                                                       const uint32_t* __restrict__ overflow) {
  if (!*broken || *overflow) return;
  using E = EntryOf<U>;
  using ET = typename E::type;
  constexpr int kSub = 96 * 1024 / sizeof(ET);  // rows per LDS-sorted batch
  constexpr int kPerThr = kSub / kBinThr;
  static_assert(kSub % kBinThr == 0, "whole rows per thread");
  __shared__ uint32_t cur[kMaxBins];        // each bin's next global slot
  __shared__ uint32_t start[kMaxBins + 1];  // the batch's count, then first LDS slot, per bin
  __shared__ uint4 buf_raw[kSub * sizeof(ET) / 16];
  ET* buf = (ET*)buf_raw;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < nbins; i += kBinThr)
    cur[i] = base[i] + hist[(size_t)blockIdx.x * nbins + i];
  const uint32_t mask = (1u << bits) - 1u;
  const int64_t r0 = (int64_t)blockIdx.x * chunk, r1 = min(rows, r0 + chunk);
  for (int64_t s0 = r0; s0 < r1; s0 += kSub) {
    for (int i = tid; i <= nbins; i += kBinThr) start[i] = 0;
    __syncthreads();
    // counts and ranks; a row out of range keeps bin -1
    int binr[kPerThr];
    uint32_t rank[kPerThr];
    ET ent[kPerThr];
#pragma unroll
    for (int k = 0; k < kPerThr; ++k) {
      const int64_t r = s0 + (int64_t)k * kBinThr + tid;
      binr[k] = -1;
      if (r < r1) {
        const int64_t ti = t[r], di = d[r];
        if (ti >= 0 && ti < T && di >= 0 && di < D) {
          const int64_t cell = ti * D + di;
          binr[k] = (int)(cell >> bits);
          ent[k] = E::make((uint32_t)cell & mask, x[r]);
          rank[k] = atomicAdd(&start[binr[k]], 1u);
        }
      }
    }
    __syncthreads();
    // counts -> first slots (exclusive prefix over the bins, start[nbins] = total)
    {
      constexpr int kPer = kMaxBins / kBinThr;
      uint32_t v[kPer], sum = 0;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int i = tid * kPer + e;
        v[e] = i < nbins ? start[i] : 0u;
        sum += v[e];
      }
      uint32_t total;
      uint32_t run = block_exclusive_scan<kBinThr>(sum, total);
      __syncthreads();
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int i = tid * kPer + e;
        if (i < nbins) start[i] = run;
        run += v[e];
      }
      if (tid == 0) start[nbins] = total;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPerThr; ++k)
      if (binr[k] >= 0) buf[start[binr[k]] + rank[k]] = ent[k];
    __syncthreads();
    // wave w copies bins w, w + 16, ...: lane j of a pass stores word j of the run
    for (int bn = wave; bn < nbins; bn += kBinThr / 64) {
      const uint32_t a = start[bn], n = start[bn + 1] - a, g = cur[bn];
      for (uint32_t j = lane; j < n; j += 64) sorted[g + j] = buf[a + j];
      if (lane == 0) cur[bn] = g + n;
    }
    __syncthreads();
  }
}

// Emit: workgroup b assembles bin b's cells in LDS from its sorted rows (a
// cell named twice keeps one of its values), writes them in order (NaN where
// unmarked), and counts the marked cells (counters[1]).
template <typename U>
__global__ __launch_bounds__(kBinThr) void bin_emit(const typename EntryOf<U>::type* __restrict__ sorted,
                                                    const uint32_t* __restrict__ base, int64_t cells,
                                                    int bits, U* __restrict__ out, U nan_bits,
                                                    unsigned long long* __restrict__ counters,
                                                    const uint32_t* __restrict__ broken,
                                                    const uint32_t* __restrict__ overflow) {
  if (!*broken || *overflow) return;
  using S = StageOf<U>;
  using W = typename S::type;
  using E = EntryOf<U>;
  __shared__ uint4 lds[kBinLds / 16];
  W* stg = (W*)lds;
  const int64_t c0 = (int64_t)blockIdx.x << bits;
  const int n = (int)min((int64_t)1 << bits, cells - c0);
  for (int i = threadIdx.x; i < n; i += kBinThr) stg[i] = W{};
  __syncthreads();
  for (uint32_t e = base[blockIdx.x] + threadIdx.x; e < base[blockIdx.x + 1]; e += kBinThr) {
    const typename E::type en = sorted[e];
    stg[E::local(en)] = S::make(E::value(en));
  }
  __syncthreads();
  unsigned long long named = 0;
  for (int i = threadIdx.x; i < n; i += kBinThr) {
    const W w = stg[i];
    const bool m = S::named(w);
    named += m;
    out[c0 + i] = m ? S::value(w) : nan_bits;
  }
  block_add<kBinThr>(named, counters + 1);
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

// The binned form runs for tables of at least kBinMin rows and cells.  Its
// bins are as large as LDS allows (2^bits cells whose staging words fill at
// most kBinLds bytes: the fewer the bins, the longer the runs the scatter
// stores), and there may be at most kMaxBins of them; bin_bits returns 0
// where that fails.
constexpr int64_t kBinMin = 65536;
int bin_bits(int elem_bytes, int64_t cells) {
  if (cells < kBinMin) return 0;
  int bits = 0;
  while (((int64_t)stage_bytes(elem_bytes) << (bits + 1)) <= kBinLds) ++bits;
  return (cells + ((int64_t)1 << bits) - 1) >> bits <= kMaxBins ? bits : 0;
}
// Workspace of the binned form after the staging words (which it uses for
// its sorted rows): hist [kBinWGs][kMaxBins] and base [kMaxBins + 1].
size_t bin_bytes() { return ((size_t)kBinWGs * kMaxBins + kMaxBins + 1) * 4; }

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
  // (row counts are 32-bit in the binned form)
  const int bits = rows >= kBinMin && rows < ((int64_t)1 << 31) ? bin_bits((int)sizeof(U), cells) : 0;
  if (bits) {
    using E = typename EntryOf<U>::type;
    static_assert(sizeof(E) == sizeof(W), "sorted rows reuse the staging words' space");
    uint32_t* overflow = broken + 1;
    uint32_t* hist = (uint32_t*)((char*)workspace + kCounterBytes +
                                 ((size_t)cells * sizeof(W) + 15) / 16 * 16);
    uint32_t* base = hist + (size_t)kBinWGs * kMaxBins;
    const int nbins = (int)((cells + ((int64_t)1 << bits) - 1) >> bits);
    const int64_t chunk = (rows + kBinWGs - 1) / kBinWGs;
    const int nwg = (int)((rows + chunk - 1) / chunk);
    const uint32_t* cbroken = broken;
    hipLaunchKernelGGL(bin_count, dim3(nwg), dim3(kBinThr), 0, stream, t, d, rows, T, D, chunk,
                       bits, nbins, hist, status, cbroken);
    hipLaunchKernelGGL(bin_prefix, dim3(nbins), dim3(kBinWGs), 0, stream, hist, nwg, nbins, base,
                       cbroken);
    hipLaunchKernelGGL(bin_bases, dim3(1), dim3(kBinThr), 0, stream, base, nbins, cells, counters,
                       overflow, status, cbroken);
    hipLaunchKernelGGL(bin_scatter<U>, dim3(nwg), dim3(kBinThr), 0, stream, t, d, (const U*)x,
                       rows, T, D, chunk, bits, nbins, (const uint32_t*)hist,
                       (const uint32_t*)base, (E*)stage, cbroken, (const uint32_t*)overflow);
    hipLaunchKernelGGL(bin_emit<U>, dim3(nbins), dim3(kBinThr), 0, stream, (const E*)stage,
                       (const uint32_t*)base, cells, bits, (U*)out, nan_bits, counters, cbroken,
                       (const uint32_t*)overflow);
  } else {
    hipLaunchKernelGGL(pivot_clear, dim3(grid_for(words / 4 + 1)), dim3(kThr), 0, stream,
                       (uint32_t*)stage, words, (const uint32_t*)broken);
    hipLaunchKernelGGL(pivot_stage<U>, dim3(grid_for(rows)), dim3(kThr), 0, stream, t, d,
                       (const U*)x, rows, T, D, stage, counters, status, (const uint32_t*)broken);
    hipLaunchKernelGGL(pivot_emit<U>, dim3(grid_for(cells / (16 / sizeof(W)) + 1)), dim3(kThr),
                       0, stream, (const W*)stage, cells, (U*)out, nan_bits, counters,
                       (const uint32_t*)broken);
  }
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
  // the counters, then one staging word per cell, in whole 16-byte stores,
  // then (tables large enough for the binned form) its counts and bin bases
  const int64_t cells = T * D;
  return kCounterBytes + ((size_t)cells * stage_bytes(elem_bytes) + 15) / 16 * 16 +
         (bin_bits(elem_bytes, cells) ? bin_bytes() : 0);
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
