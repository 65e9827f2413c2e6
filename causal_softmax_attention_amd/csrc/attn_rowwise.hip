// Row-per-group causal attention, forward and backward, for float64 (and the
// float32 backward).
//
// A group of 8 lanes owns one query row (forward, dQ) or one key row (dK/dV):
// lane g of the group holds features 8g .. 8g+7 of that row, partial dot
// products are summed across the group with three lane exchanges, and the
// group walks the other side's rows through LDS tiles.  When heads x rows are
// few, 8 or 32 groups share a row, each walking every 8th or 32nd row of the
// other side, and merge their partial states at the end (see Split below).  Every pair (i, j) with
// j <= i is visited by exactly the group that owns it and an absent pair
// (j > i) is never touched (pages: "Show HN: automatic deduction of
// FlashAttention kernel from 25 lines of SQL", the join predicate q.t >= k.t and
// the masks-are-absent-rows check).  The predicate is a parameter: causal
// (j <= i), every pair, or a causal window (j <= i and i - j < band); each row
// walks only the stretch of the other side its predicate admits.  The forward keeps a running max and
// denominator per row (the streaming plan the same page attributes to
// FlashAttention) and stores lse = m + ln l for the backward.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kG = 8;                    // lanes per row
constexpr int kF = kD / kG;              // features per lane
constexpr int kThr = 256;                // threads per workgroup
constexpr int kTile = 32;                // rows of the streamed side per LDS tile
constexpr int kFewBlocks = 2 * 256;      // fewer 32-row blocks than this (2 per CU): split

// S groups of 8 lanes share a row: group s walks tile rows s, s + S, ... and
// the S partial results are merged at the end.  S = 1 (32 rows per workgroup,
// each tile read by 32 rows) when heads x rows give the part enough
// workgroups; otherwise the walk's serial latency (a float64 exp per pair)
// sets the time and the rows' walks are split: S = 8 below 2 blocks of 32
// rows per CU, S = 32 (one row per workgroup) below 32 blocks.  Measured,
// float64 fwd+bwd: one head of 256 tokens 443 us unsplit, 138 us at S = 8,
// 97 us at S = 32; 4 heads of 1024 tokens 1846 us unsplit, 823 us at S = 8,
// 1210 us at S = 32.  16 heads of 2048 float32 tokens (1024 blocks) were
// 17 % slower at S = 8, so they stay unsplit.
__host__ __device__ constexpr int split_for(int64_t heads, int64_t N) {
  return heads * ((N + 31) / 32) < 32 ? 32 : heads * ((N + 31) / 32) < kFewBlocks ? 8 : 1;
}
template <int S>
struct Split {
  static constexpr int kRows = kThr / (kG * S);  // rows per workgroup
};

// Sum over the 8 lanes of a group (aligned groups: xor partners stay inside).
template <typename A>
__device__ __forceinline__ A group_sum(A x) {
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  x += __shfl_xor(x, 4);
  return x;
}

// Cooperative copy of rows [r0, r0 + kTile) of two [N][64] arrays into LDS
// (rows past the end read as zero).
template <typename T, typename A>
__device__ __forceinline__ void load_tiles(A (*xs)[kD], A (*ys)[kD], const T* x, const T* y,
                                           size_t base, int r0, int N) {
  for (int e = threadIdx.x; e < kTile * kD; e += kThr) {
    const int r = e / kD, c = e % kD, j = r0 + r;
    xs[r][c] = j < N ? widen(x[base + (size_t)j * kD + c]) : A(0);
    ys[r][c] = j < N ? widen(y[base + (size_t)j * kD + c]) : A(0);
  }
}

// Segment ids of rows [r0, r0 + kTile) into LDS (nothing without ids).
__device__ __forceinline__ void load_segs(int32_t* segs, const int32_t* segrow, int r0, int N) {
  if (segrow && threadIdx.x < kTile) {
    const int j = r0 + (int)threadIdx.x;
    segs[threadIdx.x] = j < N ? segrow[j] : 0;
  }
}

template <typename T, int S>
__global__ __launch_bounds__(kThr) void fwd_rowwise(const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const T* __restrict__ v, T* __restrict__ o,
                                                     acc_t<T>* __restrict__ lse, int N, int nqb,
                                                     acc_t<T> scale, int causal, int band,
                                                     acc_t<T>* __restrict__ delta,
                                                     const int32_t* __restrict__ seg, int hpb) {
  using A = acc_t<T>;
  constexpr int kRows = Split<S>::kRows;
  __shared__ A ks[kTile][kD];
  __shared__ A vs[kTile][kD];
  __shared__ int32_t segs[kTile];
  const int head = blockIdx.x / nqb;
  const int qb = nqb - 1 - (blockIdx.x % nqb);  // longest rows first
  const size_t base = (size_t)head * N * kD;
  const int32_t* segrow = seg ? seg + (size_t)(head / hpb) * N : nullptr;
  const int g = threadIdx.x % kG, f0 = kF * g;
  const int grp = threadIdx.x / kG, r = grp / S, sp = grp % S;  // row r of the block, split sp
  const int i = qb * kRows + r;
  const bool valid = i < N;
  const int jlo = band ? i - band + 1 : 0, jhi = causal ? i : N - 1;  // this row's keys

  A qr[kF], acc[kF];
#pragma unroll
  for (int f = 0; f < kF; ++f) {
    qr[f] = valid ? widen(q[base + (size_t)i * kD + f0 + f]) : A(0);
    acc[f] = 0;
  }
  A m = neg_inf<A>(), l = 0;
  const int32_t si = segrow && valid ? segrow[i] : 0;
  // keys of the block's rows: from its first row's window start to its last row
  const int kbeg = band ? max(0, qb * kRows - band + 1) / kTile * kTile : 0;
  const int kend = causal ? min(N, (qb + 1) * kRows) : N;
  for (int k0 = kbeg; k0 < kend; k0 += kTile) {
    __syncthreads();
    load_tiles(ks, vs, k, v, base, k0, N);
    load_segs(segs, segrow, k0, N);
    __syncthreads();
    const int jn = min(kTile, kend - k0);
    for (int jj = sp; jj < jn; jj += S) {
      const int j = k0 + jj;
      if (j > jhi) break;  // absent pairs past the row (the whole group leaves together)
      if (j < jlo || (segrow && segs[jj] != si)) continue;
      A s = 0;
#pragma unroll
      for (int f = 0; f < kF; ++f) s += qr[f] * ks[jj][f0 + f];
      s = group_sum(s) * scale;
      if (s > m) {
        const A alpha = exp_acc(m - s);
        l *= alpha;
#pragma unroll
        for (int f = 0; f < kF; ++f) acc[f] *= alpha;
        m = s;
      }
      const A p = exp_acc(s - m);
      l += p;
#pragma unroll
      for (int f = 0; f < kF; ++f) acc[f] += p * vs[jj][f0 + f];
    }
  }
  if (S > 1) {
    // merge the splits' (m, l, acc) against the largest m; the tiles' LDS is
    // free now (every group has left the walk at the barrier)
    A* mm = &ks[0][0];                     // [kRows][S]
    A* ll = mm + kRows * S;                // [kRows][S]
    A* aa = &vs[0][0];                     // [kRows][S][64]
    static_assert(2 * (kThr / (kG * S)) * S <= kTile * kD && (kThr / kG) * kD <= kTile * kD,
                  "merge buffers fit the tiles");
    __syncthreads();
    if (g == 0) {
      mm[r * S + sp] = m;
      ll[r * S + sp] = l;
    }
#pragma unroll
    for (int f = 0; f < kF; ++f) aa[(r * S + sp) * kD + f0 + f] = acc[f];
    __syncthreads();
    if (sp != 0) return;
    A mx = neg_inf<A>();
    for (int t = 0; t < S; ++t) mx = mx > mm[r * S + t] ? mx : mm[r * S + t];
    l = 0;
#pragma unroll
    for (int f = 0; f < kF; ++f) acc[f] = 0;
    for (int t = 0; t < S; ++t) {
      const A mt = mm[r * S + t];
      const A w = mt == neg_inf<A>() ? A(0) : exp_acc(mt - mx);  // a split that saw no key adds 0
      l += ll[r * S + t] * w;
#pragma unroll
      for (int f = 0; f < kF; ++f) acc[f] += aa[(r * S + t) * kD + f0 + f] * w;
    }
    m = mx;
  }
  if (valid) {
    const A inv = A(1) / l;
    A sq = 0;
#pragma unroll
    for (int f = 0; f < kF; ++f) {
      const T x = narrow<T>(acc[f] * inv);
      o[base + (size_t)i * kD + f0 + f] = x;
      sq += widen(x) * widen(x);
    }
    if (g == 0) lse[(size_t)head * N + i] = m + log_acc(l);
    if (delta) {  // the loss sum(o^2)/2: dO = O, so the backward's delta_i = |o_i|^2
      sq = group_sum(sq);
      if (g == 0) delta[(size_t)head * N + i] = sq;
    }
  }
}

// delta_i = sum_d dout_id * o_id
template <typename T>
__global__ __launch_bounds__(256) void bwd_delta(const T* __restrict__ o, const T* __restrict__ dout,
                                                 acc_t<T>* __restrict__ delta, int64_t rows) {
  using A = acc_t<T>;
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  A s = 0;
#pragma unroll 8
  for (int d = 0; d < kD; ++d) s += widen(o[r * kD + d]) * widen(dout[r * kD + d]);
  delta[r] = s;
}

// dK, dV: one group per key j, queries i >= j streamed through LDS.
template <typename T, int S>
__global__ __launch_bounds__(kThr) void bwd_dkdv_rowwise(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const acc_t<T>* __restrict__ lse,
    const acc_t<T>* __restrict__ delta, T* __restrict__ dk, T* __restrict__ dv, int N, int nkb,
    acc_t<T> scale, int causal, int band, const int32_t* __restrict__ seg, int hpb) {
  using A = acc_t<T>;
  constexpr int kRows = Split<S>::kRows;
  __shared__ A qs[kTile][kD];
  __shared__ A dos[kTile][kD];
  __shared__ A ls[kTile], ds_[kTile];
  __shared__ int32_t segs[kTile];
  const int head = blockIdx.x / nkb;
  const int32_t* segrow = seg ? seg + (size_t)(head / hpb) * N : nullptr;
  const int kb = blockIdx.x % nkb;  // low key blocks see the most queries: they come first
  const size_t base = (size_t)head * N * kD;
  const int g = threadIdx.x % kG, f0 = kF * g;
  const int grp = threadIdx.x / kG, r = grp / S, sp = grp % S;  // key r of the block, split sp
  const int j = kb * kRows + r;
  const bool valid = j < N;
  const int ilo = causal ? j : 0, ihi = band ? j + band - 1 : N - 1;  // this key's queries
  const int32_t sj = segrow && valid ? segrow[j] : 0;
  A kr[kF], vr[kF], gk[kF], gv[kF];
#pragma unroll
  for (int f = 0; f < kF; ++f) {
    kr[f] = valid ? widen(k[base + (size_t)j * kD + f0 + f]) : A(0);
    vr[f] = valid ? widen(v[base + (size_t)j * kD + f0 + f]) : A(0);
    gk[f] = 0;
    gv[f] = 0;
  }
  const int qbeg = causal ? kb * kRows : 0;
  const int qend = band ? min(N, (kb + 1) * kRows + band - 1) : N;
  for (int q0 = qbeg; q0 < qend; q0 += kTile) {
    __syncthreads();
    load_tiles(qs, dos, q, dout, base, q0, N);
    load_segs(segs, segrow, q0, N);
    if (threadIdx.x < kTile) {
      const int i = q0 + threadIdx.x;
      ls[threadIdx.x] = i < N ? lse[(size_t)head * N + i] : A(0);
      ds_[threadIdx.x] = i < N ? delta[(size_t)head * N + i] : A(0);
    }
    __syncthreads();
    const int in = min(kTile, qend - q0);
    for (int ii = sp; ii < in; ii += S) {
      if (q0 + ii < ilo || q0 + ii > ihi || (segrow && segs[ii] != sj)) continue;  // absent
      A s = 0, dp = 0;
#pragma unroll
      for (int f = 0; f < kF; ++f) {
        s += qs[ii][f0 + f] * kr[f];
        dp += dos[ii][f0 + f] * vr[f];
      }
      s = group_sum(s);
      dp = group_sum(dp);
      const A p = exp_acc(s * scale - ls[ii]);
      const A dsc = p * (dp - ds_[ii]) * scale;
#pragma unroll
      for (int f = 0; f < kF; ++f) {
        gv[f] += p * dos[ii][f0 + f];
        gk[f] += dsc * qs[ii][f0 + f];
      }
    }
  }
  if (S > 1) {
    // sum the splits' partial dK, dV (in split order) in the tiles' LDS
    A* pk = &qs[0][0];                     // [kRows][S][64]
    A* pv = &dos[0][0];
    __syncthreads();
#pragma unroll
    for (int f = 0; f < kF; ++f) {
      pk[(r * S + sp) * kD + f0 + f] = gk[f];
      pv[(r * S + sp) * kD + f0 + f] = gv[f];
    }
    __syncthreads();
    if (sp != 0) return;
    for (int t = 1; t < S; ++t)
#pragma unroll
      for (int f = 0; f < kF; ++f) {
        gk[f] += pk[(r * S + t) * kD + f0 + f];
        gv[f] += pv[(r * S + t) * kD + f0 + f];
      }
  }
  if (valid) {
#pragma unroll
    for (int f = 0; f < kF; ++f) {
      dk[base + (size_t)j * kD + f0 + f] = narrow<T>(gk[f]);
      dv[base + (size_t)j * kD + f0 + f] = narrow<T>(gv[f]);
    }
  }
}

// dQ: one group per query i, keys j <= i streamed through LDS.
template <typename T, int S>
__global__ __launch_bounds__(kThr) void bwd_dq_rowwise(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const acc_t<T>* __restrict__ lse,
    const acc_t<T>* __restrict__ delta, T* __restrict__ dq, int N, int nqb, acc_t<T> scale,
    int causal, int band, const int32_t* __restrict__ seg, int hpb) {
  using A = acc_t<T>;
  constexpr int kRows = Split<S>::kRows;
  __shared__ A ks[kTile][kD];
  __shared__ A vs[kTile][kD];
  __shared__ int32_t segs[kTile];
  const int head = blockIdx.x / nqb;
  const int32_t* segrow = seg ? seg + (size_t)(head / hpb) * N : nullptr;
  const int qb = nqb - 1 - (blockIdx.x % nqb);
  const size_t base = (size_t)head * N * kD;
  const int g = threadIdx.x % kG, f0 = kF * g;
  const int grp = threadIdx.x / kG, r = grp / S, sp = grp % S;  // query r of the block, split sp
  const int i = qb * kRows + r;
  const bool valid = i < N;
  A qr[kF], dor[kF], gq[kF];
#pragma unroll
  for (int f = 0; f < kF; ++f) {
    qr[f] = valid ? widen(q[base + (size_t)i * kD + f0 + f]) : A(0);
    dor[f] = valid ? widen(dout[base + (size_t)i * kD + f0 + f]) : A(0);
    gq[f] = 0;
  }
  const A li = valid ? lse[(size_t)head * N + i] : A(0);
  const A di = valid ? delta[(size_t)head * N + i] : A(0);
  const int32_t si = segrow && valid ? segrow[i] : 0;
  const int jlo = band ? i - band + 1 : 0, jhi = causal ? i : N - 1;
  const int kbeg = band ? max(0, qb * kRows - band + 1) / kTile * kTile : 0;
  const int kend = causal ? min(N, (qb + 1) * kRows) : N;
  for (int k0 = kbeg; k0 < kend; k0 += kTile) {
    __syncthreads();
    load_tiles(ks, vs, k, v, base, k0, N);
    load_segs(segs, segrow, k0, N);
    __syncthreads();
    const int jn = min(kTile, kend - k0);
    for (int jj = sp; jj < jn; jj += S) {
      const int j = k0 + jj;
      if (j > jhi) break;
      if (j < jlo || (segrow && segs[jj] != si)) continue;
      A s = 0, dp = 0;
#pragma unroll
      for (int f = 0; f < kF; ++f) {
        s += qr[f] * ks[jj][f0 + f];
        dp += dor[f] * vs[jj][f0 + f];
      }
      s = group_sum(s);
      dp = group_sum(dp);
      const A p = exp_acc(s * scale - li);
      const A dsc = p * (dp - di) * scale;
#pragma unroll
      for (int f = 0; f < kF; ++f) gq[f] += dsc * ks[jj][f0 + f];
    }
  }
  if (S > 1) {
    // sum the splits' partial dQ (in split order) in the tiles' LDS
    A* pq = &ks[0][0];                     // [kRows][S][64]
    __syncthreads();
#pragma unroll
    for (int f = 0; f < kF; ++f) pq[(r * S + sp) * kD + f0 + f] = gq[f];
    __syncthreads();
    if (sp != 0) return;
    for (int t = 1; t < S; ++t)
#pragma unroll
      for (int f = 0; f < kF; ++f) gq[f] += pq[(r * S + t) * kD + f0 + f];
  }
  if (valid) {
#pragma unroll
    for (int f = 0; f < kF; ++f) dq[base + (size_t)i * kD + f0 + f] = narrow<T>(gq[f]);
  }
}

}  // namespace

template <typename T>
hipError_t launch_fwd(const T* q, const T* k, const T* v, T* o, void* lse, int64_t heads,
                      int64_t N, double scale, const Mask& mk, void* bwd_ws, hipStream_t stream,
                      const Timers& tm) {
  using A = acc_t<T>;
  const int sp = split_for(heads, N);
  const int per = kThr / (kG * sp);
  const int nqb = (int)((N + per - 1) / per);
  auto kern = sp == 32 ? fwd_rowwise<T, 32> : sp == 8 ? fwd_rowwise<T, 8> : fwd_rowwise<T, 1>;
  if (hipError_t e = mark(tm.start[kTimerFwd], stream)) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(heads * nqb)), dim3(kThr), 0, stream, q, k, v, o,
                     (A*)lse, (int)N, nqb, (A)scale, mk.causal, mk.band, (A*)bwd_ws, mk.seg,
                     mk.hpb);
  if (hipError_t e = mark(tm.stop[kTimerFwd], stream)) return e;
  return hipGetLastError();
}

template <typename T>
size_t bwd_workspace_bytes(int64_t heads, int64_t N) {
  return (size_t)heads * N * sizeof(acc_t<T>);
}

template <typename T>
hipError_t launch_bwd(const T* q, const T* k, const T* v, const T* o, const T* dout,
                      const void* lse, T* dq, T* dk, T* dv, void* workspace, int64_t heads,
                      int64_t N, double scale, const Mask& mk, bool prepared,
                      hipStream_t stream, const Timers& tm) {
  using A = acc_t<T>;
  A* delta = (A*)workspace;
  const int64_t rows = heads * N;
  if (!prepared) {  // else the forward already wrote delta (dO = O)
    if (hipError_t e = mark(tm.start[kTimerBwdPre], stream)) return e;
    hipLaunchKernelGGL(bwd_delta<T>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream,
                       o, dout, delta, rows);
    if (hipError_t e = mark(tm.stop[kTimerBwdPre], stream)) return e;
  }
  const int sp = split_for(heads, N);
  const int per = kThr / (kG * sp);
  const int nb = (int)((N + per - 1) / per);
  auto kdkdv = sp == 32 ? bwd_dkdv_rowwise<T, 32>
               : sp == 8 ? bwd_dkdv_rowwise<T, 8> : bwd_dkdv_rowwise<T, 1>;
  auto kdq = sp == 32 ? bwd_dq_rowwise<T, 32> : sp == 8 ? bwd_dq_rowwise<T, 8> : bwd_dq_rowwise<T, 1>;
  if (hipError_t e = mark(tm.start[kTimerBwdDkdv], stream)) return e;
  hipLaunchKernelGGL(kdkdv, dim3((unsigned)(heads * nb)), dim3(kThr), 0, stream, q, k, v, dout,
                     (const A*)lse, delta, dk, dv, (int)N, nb, (A)scale, mk.causal, mk.band,
                     mk.seg, mk.hpb);
  if (hipError_t e = mark(tm.stop[kTimerBwdDkdv], stream)) return e;
  if (hipError_t e = mark(tm.start[kTimerBwdDq], stream)) return e;
  hipLaunchKernelGGL(kdq, dim3((unsigned)(heads * nb)), dim3(kThr), 0, stream, q, k, v, dout,
                     (const A*)lse, delta, dq, (int)N, nb, (A)scale, mk.causal, mk.band, mk.seg,
                     mk.hpb);
  if (hipError_t e = mark(tm.stop[kTimerBwdDq], stream)) return e;
  return hipGetLastError();
}

#define ATTN_INSTANTIATE(T)                                                                     \
  template hipError_t launch_fwd<T>(const T*, const T*, const T*, T*, void*, int64_t, int64_t, \
                                    double, const Mask&, void*, hipStream_t, const Timers&);    \
  template size_t bwd_workspace_bytes<T>(int64_t, int64_t);                                    \
  template hipError_t launch_bwd<T>(const T*, const T*, const T*, const T*, const T*,          \
                                    const void*, T*, T*, T*, void*, int64_t, int64_t, double,  \
                                    const Mask&, bool, hipStream_t, const Timers&);
ATTN_INSTANTIATE(double)
ATTN_INSTANTIATE(float)  // the float32 backward (its forward runs on MFMA, attn_fwd_f32.hip)

}  // namespace attn
