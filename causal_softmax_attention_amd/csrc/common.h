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

}  // namespace attn
