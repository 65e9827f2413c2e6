// The loss of the pages' GRADIENT statement, loss = SUM(x * x) / 2 over every
// output value (pages: "Show HN: automatic deduction of FlashAttention kernel
// from 25 lines of SQL", the GRADIENT statement), from the per-row squared
// norms |o_i|^2 the forward already wrote for the backward (delta_i, or its
// negation for the bfloat16 path).
//
// Deterministic two-pass sum in float64: kLossParts workgroups each add a
// contiguous stretch of rows in a fixed order and write one partial; one
// workgroup then adds the partials in a fixed order.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

constexpr int kThreads = 256;

template <int N>
__device__ __forceinline__ double block_sum(double x, double (&red)[N]) {
  red[threadIdx.x] = x;
  __syncthreads();
#pragma unroll
  for (int w = N / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  return red[0];
}

template <typename V>
__global__ __launch_bounds__(kThreads) void loss_partials(const V* __restrict__ vals, int64_t rows,
                                                          double* __restrict__ parts) {
  __shared__ double red[kThreads];
  const int64_t per = (rows + kLossParts - 1) / kLossParts;
  const int64_t r0 = (int64_t)blockIdx.x * per, r1 = min(rows, r0 + per);
  double s = 0.0;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += kThreads) s += (double)vals[r];
  s = block_sum(s, red);
  if (threadIdx.x == 0) parts[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void loss_total(const double* __restrict__ parts,
                                                       double half_sign, double* __restrict__ loss) {
  __shared__ double red[kThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < kLossParts; i += kThreads) s += parts[i];
  s = block_sum(s, red);
  if (threadIdx.x == 0) *loss = half_sign * s;
}

}  // namespace

hipError_t launch_loss(int vals_kind, const void* vals, int64_t rows, double* parts, double* loss,
                       hipStream_t stream) {
  // vals_kind 0: float64 delta; 1: float32 delta; 2: float32 -delta
  const double half_sign = vals_kind == 2 ? -0.5 : 0.5;
  if (vals_kind == 0)
    hipLaunchKernelGGL(loss_partials<double>, dim3(kLossParts), dim3(kThreads), 0, stream,
                       (const double*)vals, rows, parts);
  else
    hipLaunchKernelGGL(loss_partials<float>, dim3(kLossParts), dim3(kThreads), 0, stream,
                       (const float*)vals, rows, parts);
  hipLaunchKernelGGL(loss_total, dim3(1), dim3(kThreads), 0, stream, (const double*)parts,
                     half_sign, loss);
  return hipGetLastError();
}

}  // namespace attn
