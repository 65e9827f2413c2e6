// Host-side launchers of the library's kernels.  Sizes are validated by the
// C ABI layer (attn_api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Caller-supplied timing events, one start/stop pair per kernel slot
// (ATTN_TIMER_* in include/attn.h); null events are skipped.
struct Timers {
  hipEvent_t start[7] = {};
  hipEvent_t stop[7] = {};
};
enum {
  kTimerFwd = 0,
  kTimerBwdPre = 1,
  kTimerBwdDkdv = 2,
  kTimerBwdDq = 3,
  kTimerNw = 4,
  kTimerTable = 5,
  kTimerProject = 6
};

inline hipError_t mark(hipEvent_t ev, hipStream_t s) { return ev ? hipEventRecord(ev, s) : hipSuccess; }

// Which (query i, key j) pairs exist (the join predicate): j < N and
//   causal != 0: j <= i;   band > 0: i - j < band   (band 0: no lower limit);
//   seg non-null: seg[b][i] == seg[b][j], where head h of the launch belongs to
//   batch b = h / hpb and seg is [B][N] int32 (segment ids of the tokens).
// causal = 1, band = 0 is the causal view; causal = 0, band = 0 every pair;
// causal = 1, band = w a causal window of w keys.  (causal = 0 with band > 0
// is not used.)
struct Mask {
  int causal = 1;
  int band = 0;
  const int32_t* seg = nullptr;
  int hpb = 1;  // heads per batch (the H of [B, H, N, D])
};

// Every forward launcher takes `bwd_ws`: null, or the backward workspace, which
// the forward then fills with the per-row values of the loss sum(o^2)/2
// (dO = O) so that the backward launchers can run `prepared` (without their
// first, per-row kernel).  Layouts: bfloat16 -delta_i then -lse_i / scale
// (float each); float32 / float64 delta_i in the accumulation type.

// Row-per-group kernels (attn_rowwise.hip): forward and backward of `heads`
// independent heads of N tokens, D = 64.  T is double or float; lse is double
// for double, float otherwise.
template <typename T>
hipError_t launch_fwd(const T* q, const T* k, const T* v, T* o, void* lse, int64_t heads,
                      int64_t N, double scale, const Mask& mk, void* bwd_ws, hipStream_t stream,
                      const Timers& tm);

// Backward workspace bytes and launch (dq, dk, dv from q, k, v, o, dout, lse).
template <typename T>
size_t bwd_workspace_bytes(int64_t heads, int64_t N);

template <typename T>
hipError_t launch_bwd(const T* q, const T* k, const T* v, const T* o, const T* dout,
                      const void* lse, T* dq, T* dk, T* dv, void* workspace, int64_t heads,
                      int64_t N, double scale, const Mask& mk, bool prepared,
                      hipStream_t stream, const Timers& tm);

// float32 forward on MFMA tiles (attn_fwd_f32.hip).
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int64_t heads, int64_t N, double scale, const Mask& mk, void* bwd_ws,
                          hipStream_t stream, const Timers& tm);

// bfloat16 forward on MFMA tiles (attn_fwd_bf16.hip).
hipError_t launch_fwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o,
                           float* lse, int64_t heads, int64_t N, double scale, const Mask& mk,
                           void* bwd_ws, hipStream_t stream, const Timers& tm);

// bfloat16 backward on MFMA tiles (attn_bwd_bf16.hip); the workspace holds two floats
// per row (-delta and -lse / scale).
size_t bwd_workspace_bytes_bf16(int64_t heads, int64_t N);
hipError_t launch_bwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* o,
                           const __bf16* dout, const float* lse, __bf16* dq, __bf16* dk,
                           __bf16* dv, void* workspace, int64_t heads, int64_t N, double scale,
                           const Mask& mk, bool prepared, hipStream_t stream, const Timers& tm);

// The dQ pass alone (attn_bwd_dq_bf16.hip), from the prep kernel's per-row values.
hipError_t launch_bwd_dq_bf16(const __bf16* q, const __bf16* k, const __bf16* v,
                              const __bf16* dout, const float* nlse, const float* ndelta,
                              __bf16* dq, int64_t heads, int64_t N, double scale,
                              const Mask& mk, hipStream_t stream, const Timers& tm);

// loss = sum(o^2)/2 from the per-row values a forward wrote (attn_loss.hip):
// vals_kind 0 float64 delta, 1 float32 delta, 2 float32 -delta; `parts` holds
// kLossParts doubles of scratch.
constexpr int kLossParts = 256;
hipError_t launch_loss(int vals_kind, const void* vals, int64_t rows, double* parts, double* loss,
                       hipStream_t stream);

hipError_t launch_nw(int64_t n_targets, const float* tx, const float* ty, int64_t n_sources,
                     const float* sx, const float* sy, const float* sv, float denom, float* out,
                     hipStream_t stream, const Timers& tm);

// Long-table <-> matrix adapter (attn_table.hip).  elem_bytes: 8, 4 or 2.
size_t table_workspace_bytes(int elem_bytes, int64_t T, int64_t D);
hipError_t launch_table_to_matrix(int elem_bytes, int64_t rows, const int64_t* t, const int64_t* d,
                                  const void* x, int64_t T, int64_t D, void* out, int32_t* status,
                                  void* workspace, hipStream_t stream, const Timers& tm);
hipError_t launch_matrix_to_table(int elem_bytes, int64_t T, int64_t D, const void* m, int64_t* t,
                                  int64_t* d, void* x, hipStream_t stream);

// Q / K / V input projections (attn_project.hip).  elem_bytes: 8, 4 or 2.
bool project_uses_mfma(int elem_bytes, int64_t M, int64_t Dm, int64_t H);
hipError_t launch_project(int elem_bytes, int64_t B, int64_t N, int64_t Dm, int64_t H,
                          const void* x, const void* wq, const void* wk, const void* wv, void* q,
                          void* k, void* v, hipStream_t stream, const Timers& tm);

}  // namespace attn
