// Device-side helpers shared by the kernels of the attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kD = 64;  // features per head; the only D this library implements

// Accumulation / softmax type for each storage type: float64 stays float64,
// float32 and bfloat16 accumulate in float32.
template <typename T> struct AccOf;
template <> struct AccOf<double> { using type = double; };
template <> struct AccOf<float> { using type = float; };
template <> struct AccOf<__bf16> { using type = float; };
template <typename T> using acc_t = typename AccOf<T>::type;

__device__ __forceinline__ double widen(double x) { return x; }
__device__ __forceinline__ float widen(float x) { return x; }
__device__ __forceinline__ float widen(__bf16 x) { return (float)x; }

// Narrowing stores: float32 -> bfloat16 rounds to nearest even (v_cvt_pk_bf16_f32).
template <typename T> __device__ __forceinline__ T narrow(acc_t<T> x);
template <> __device__ __forceinline__ double narrow<double>(double x) { return x; }
template <> __device__ __forceinline__ float narrow<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 narrow<__bf16>(float x) { return (__bf16)x; }

// Natural exp / log in the accumulation type.  float32 uses the hardware base-2
// exponential with log2(e) folded into the argument.
__device__ __forceinline__ double exp_acc(double x) { return exp(x); }
__device__ __forceinline__ float exp_acc(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
__device__ __forceinline__ double log_acc(double x) { return log(x); }
__device__ __forceinline__ float log_acc(float x) { return __logf(x); }

template <typename A> __device__ __forceinline__ A neg_inf();
template <> __device__ __forceinline__ double neg_inf<double>() { return -__builtin_inf(); }
template <> __device__ __forceinline__ float neg_inf<float>() { return -__builtin_inff(); }

// Segment ids (one int32 per token): the tokens of [qs, qe) that can pair
// with the tokens [k0, k0 + nk) are those whose id lies in the id range
// [lo, hi] of the latter.  first / last: the first and one past the last such
// token (first = INT32_MAX, last = 0 if there is none); a token outside that
// span pairs with none of [k0, k0 + nk).  dense: every token of the span has
// its id in [lo, hi].  Workgroup-wide: every thread of the kThreads calls it;
// red is LDS for 2 x (kThreads / 64) x 4 ints.
struct SegSpan {
  int first, last;
  int32_t lo, hi;
  bool dense;
};

template <int kThreads>
__device__ __forceinline__ SegSpan seg_span(const int32_t* segrow, int N, int k0, int nk, int qs,
                                            int qe, int tid, int32_t (*red)[kThreads / 64][4]) {
  constexpr int kW = kThreads / 64;
  constexpr int kPer = 16;  // ids per thread per pass over [qs, qe)
  const int lane = tid & 63, wave = tid >> 6;
  // the first pass's loads are issued with the block's own ids, so the two
  // round trips overlap
  int32_t ids[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int i = qs + e * kThreads + tid;
    ids[e] = i < qe ? segrow[i] : 0;
  }
  int32_t lo = INT32_MAX, hi = INT32_MIN;
  for (int j = k0 + tid; j < min(k0 + nk, N); j += kThreads) {
    const int32_t id = segrow[j];
    lo = min(lo, id);
    hi = max(hi, id);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    lo = min(lo, __shfl_xor(lo, o));
    hi = max(hi, __shfl_xor(hi, o));
  }
  if (lane == 0) {
    red[0][wave][0] = lo;
    red[0][wave][1] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    lo = min(lo, red[0][w][0]);
    hi = max(hi, red[0][w][1]);
  }
  int f = INT32_MAX, l = -1, cnt = 0;
  for (int b = qs; b < qe; b += kPer * kThreads) {
    if (b != qs) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const int i = b + e * kThreads + tid;
        ids[e] = i < qe ? segrow[i] : 0;
      }
    }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int i = b + e * kThreads + tid;
      if (i < qe && ids[e] >= lo && ids[e] <= hi) {
        f = min(f, i);
        l = max(l, i);
        ++cnt;
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    f = min(f, __shfl_xor(f, o));
    l = max(l, __shfl_xor(l, o));
    cnt += __shfl_xor(cnt, o);
  }
  if (lane == 0) {
    red[1][wave][0] = f;
    red[1][wave][1] = l;
    red[1][wave][2] = cnt;
  }
  __syncthreads();
  cnt = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    f = min(f, red[1][w][0]);
    l = max(l, red[1][w][1]);
    cnt += red[1][w][2];
  }
  return SegSpan{f, l + 1, lo, hi, cnt == l + 1 - f};
}

}  // namespace attn
