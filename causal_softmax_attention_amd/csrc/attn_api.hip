// C ABI of the library (declared in include/attn.h): argument checks, dtype
// dispatch, and error reporting.  Every check happens before any launch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "../../include/attn.h"
#include "launch.h"

namespace {

thread_local std::string g_err;
thread_local attn::Timers g_tm;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) {
    g_err.clear();
    return ATTN_OK;
  }
  return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

size_t elem_size(int dtype) { return dtype == ATTN_BF16 ? 2 : dtype == ATTN_F32 ? 4 : 8; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Largest sizes the kernels index: a head's element count and the total
// element count must fit the int/int64 arithmetic used on the device.
constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxHeads = int64_t(1) << 24;
constexpr int64_t kMaxGroups = int64_t(1) << 24;  // x 256 threads = 2^32 work-items
// Largest element count of a matrix, table or weight the adapter and the
// projections index (int64 offsets; 2^40 elements is far beyond one GPU).
constexpr int64_t kMaxCells = int64_t(1) << 40;

int check_sizes(int dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale) {
  if (dtype != ATTN_F64 && dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_EINVAL, "unknown dtype %d", dtype);
  if (B < 1 || H < 1 || N < 1 || D < 1)
    return fail(ATTN_EINVAL, "sizes must be >= 1 (B=%lld H=%lld N=%lld D=%lld)", (long long)B,
                (long long)H, (long long)N, (long long)D);
  if (D != 64) return fail(ATTN_EUNSUPPORTED, "D=%lld: only D=64 is implemented", (long long)D);
  if (N > kMaxN) return fail(ATTN_EINVAL, "N=%lld exceeds %lld", (long long)N, (long long)kMaxN);
  if (B > kMaxHeads / H)
    return fail(ATTN_EINVAL, "B*H exceeds %lld", (long long)kMaxHeads);
  // Every launch over heads x row blocks takes at least 32 rows per 256-thread
  // workgroup, with heads padded to a multiple of 8; a launch's work-items
  // (workgroups x 256) must stay below 2^32.
  const int64_t padded = (B * H + 7) / 8 * 8, blocks = (N + 31) / 32;
  if (padded * blocks >= kMaxGroups)
    return fail(ATTN_EINVAL, "B*H=%lld heads of N=%lld need %lld workgroups of 32 rows; the limit is %lld",
                (long long)(B * H), (long long)N, (long long)(padded * blocks),
                (long long)kMaxGroups - 1);
  if (!(scale > 0.0) || !isfinite(scale)) return fail(ATTN_EINVAL, "scale must be finite and > 0");
  return ATTN_OK;
}

// The join predicate of a mask kind; a window at least N wide is the causal one.
int make_mask(int mask, int64_t window, int64_t N, attn::Mask& mk) {
  switch (mask) {
    case ATTN_MASK_CAUSAL: mk = attn::Mask{1, 0}; return ATTN_OK;
    case ATTN_MASK_FULL: mk = attn::Mask{0, 0}; return ATTN_OK;
    case ATTN_MASK_WINDOW:
      if (window < 1) return fail(ATTN_EINVAL, "window must be >= 1 (got %lld)", (long long)window);
      mk = attn::Mask{1, window >= N ? 0 : (int)window};
      return ATTN_OK;
    default: return fail(ATTN_EINVAL, "unknown mask kind %d", mask);
  }
}

// Workspace of the backward: its per-row values, then (from a 256-byte
// boundary) kLossParts doubles that the loss sum of attn_fwd_train uses.
size_t rows_bytes(int dtype, int64_t heads, int64_t N) {
  switch (dtype) {
    case ATTN_F64: return attn::bwd_workspace_bytes<double>(heads, N);
    case ATTN_F32: return attn::bwd_workspace_bytes<float>(heads, N);
    default: return attn::bwd_workspace_bytes_bf16(heads, N);
  }
}
size_t parts_offset(int dtype, int64_t heads, int64_t N) {
  return (rows_bytes(dtype, heads, N) + 255) / 256 * 256;
}
size_t workspace_bytes_for(int dtype, int64_t heads, int64_t N) {
  return parts_offset(dtype, heads, N) + attn::kLossParts * sizeof(double);
}

// Segment ids [B][N] (int32, one row per batch, shared by its H heads): the
// pointer must be 4-byte aligned and no output may overlap its B*N*4 bytes.
int add_segments(const int32_t* seg, int64_t H, attn::Mask& mk) {
  if ((uintptr_t)seg & 3u) return fail(ATTN_EINVAL, "segment ids must be 4-byte aligned");
  mk.seg = seg;
  mk.hpb = (int)H;
  return ATTN_OK;
}

size_t seg_bytes(int64_t B, int64_t N) { return (size_t)B * N * sizeof(int32_t); }

// attn_fwd, and with bwd_ws non-null the forward of attn_fwd_train (which
// checks the workspace itself); seg non-null adds the segment predicate.
int fwd_impl(int dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale, int mask,
             int64_t window, const int32_t* seg, const void* q, const void* k, const void* v,
             void* o, void* lse, void* bwd_ws, hipStream_t s) {
  if (int rc = check_sizes(dtype, B, H, N, D, scale)) return rc;
  attn::Mask mk;
  if (int rc = make_mask(mask, window, N, mk)) return rc;
  if (seg)
    if (int rc = add_segments(seg, H, mk)) return rc;
  if (!q || !k || !v || !o || !lse) return fail(ATTN_EINVAL, "null pointer argument");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return fail(ATTN_EINVAL, "pointers must be 16-byte aligned");
  const int64_t heads = B * H;
  const size_t tb = (size_t)heads * N * D * elem_size(dtype);
  const size_t lb = (size_t)heads * N * (dtype == ATTN_F64 ? 8 : 4);
  const void* ins[3] = {q, k, v};
  for (const void* p : ins)
    if (overlap(o, tb, p, tb) || overlap(lse, lb, p, tb))
      return fail(ATTN_EINVAL, "outputs must not alias inputs");
  if (overlap(o, tb, lse, lb)) return fail(ATTN_EINVAL, "o and lse overlap");
  if (seg && (overlap(o, tb, seg, seg_bytes(B, N)) || overlap(lse, lb, seg, seg_bytes(B, N))))
    return fail(ATTN_EINVAL, "outputs must not alias the segment ids");
  if (bwd_ws) {
    const size_t wb = workspace_bytes_for(dtype, heads, N);
    const void* all[] = {q, k, v, o};
    for (const void* p : all)
      if (overlap(bwd_ws, wb, p, tb)) return fail(ATTN_EINVAL, "workspace aliases a tensor");
    if (overlap(bwd_ws, wb, lse, lb)) return fail(ATTN_EINVAL, "workspace aliases lse");
  }
  hipError_t e;
  switch (dtype) {
    case ATTN_F64:
      e = attn::launch_fwd<double>((const double*)q, (const double*)k, (const double*)v,
                                   (double*)o, lse, heads, N, scale, mk, bwd_ws, s, g_tm);
      break;
    case ATTN_F32:
      e = attn::launch_fwd_f32((const float*)q, (const float*)k, (const float*)v, (float*)o,
                               (float*)lse, heads, N, scale, mk, bwd_ws, s, g_tm);
      break;
    default:
      e = attn::launch_fwd_bf16((const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                                (__bf16*)o, (float*)lse, heads, N, scale, mk, bwd_ws, s, g_tm);
  }
  return hip_status(e, "forward launch");
}

// attn_bwd; prepared: the workspace already holds the per-row values the
// forward of attn_fwd_train wrote (dout is o).
int bwd_impl(int dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale, int mask,
             int64_t window, const int32_t* seg, const void* q, const void* k, const void* v,
             const void* o, const void* dout, const void* lse, void* dq, void* dk, void* dv,
             void* workspace, size_t workspace_bytes, bool prepared, hipStream_t s) {
  if (int rc = check_sizes(dtype, B, H, N, D, scale)) return rc;
  attn::Mask mk;
  if (int rc = make_mask(mask, window, N, mk)) return rc;
  if (seg)
    if (int rc = add_segments(seg, H, mk)) return rc;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace)
    return fail(ATTN_EINVAL, "null pointer argument");
  const void* all[] = {q, k, v, o, dout, lse, dq, dk, dv, workspace};
  for (const void* p : all)
    if (!aligned16(p)) return fail(ATTN_EINVAL, "pointers must be 16-byte aligned");
  const int64_t heads = B * H;
  const size_t need = workspace_bytes_for(dtype, heads, N);
  if (workspace_bytes < need)
    return fail(ATTN_EINVAL, "workspace of %zu bytes is smaller than the %zu required",
                workspace_bytes, need);
  const size_t tb = (size_t)heads * N * D * elem_size(dtype);
  const size_t lb = (size_t)heads * N * (dtype == ATTN_F64 ? 8 : 4);
  const void* ins[] = {q, k, v, o, dout};
  void* outs[] = {dq, dk, dv};
  for (void* w : outs) {
    for (const void* r : ins)
      if (overlap(w, tb, r, tb)) return fail(ATTN_EINVAL, "outputs must not alias inputs");
    if (overlap(w, tb, lse, lb) || overlap(w, tb, workspace, need))
      return fail(ATTN_EINVAL, "outputs must not alias lse or the workspace");
  }
  if (overlap(dq, tb, dk, tb) || overlap(dq, tb, dv, tb) || overlap(dk, tb, dv, tb))
    return fail(ATTN_EINVAL, "dq, dk and dv must not overlap");
  if (seg) {
    void* written[] = {dq, dk, dv};
    for (void* w : written)
      if (overlap(w, tb, seg, seg_bytes(B, N)))
        return fail(ATTN_EINVAL, "outputs must not alias the segment ids");
    if (overlap(workspace, need, seg, seg_bytes(B, N)))
      return fail(ATTN_EINVAL, "workspace aliases the segment ids");
  }
  for (const void* r : ins)
    if (overlap(workspace, need, r, tb)) return fail(ATTN_EINVAL, "workspace aliases an input");
  if (overlap(workspace, need, lse, lb)) return fail(ATTN_EINVAL, "workspace aliases lse");
  hipError_t e;
  switch (dtype) {
    case ATTN_F64:
      e = attn::launch_bwd<double>((const double*)q, (const double*)k, (const double*)v,
                                   (const double*)o, (const double*)dout, lse, (double*)dq,
                                   (double*)dk, (double*)dv, workspace, heads, N, scale, mk,
                                   prepared, s, g_tm);
      break;
    case ATTN_F32:
      e = attn::launch_bwd<float>((const float*)q, (const float*)k, (const float*)v,
                                  (const float*)o, (const float*)dout, lse, (float*)dq,
                                  (float*)dk, (float*)dv, workspace, heads, N, scale, mk,
                                  prepared, s, g_tm);
      break;
    default:
      e = attn::launch_bwd_bf16((const __bf16*)q, (const __bf16*)k, (const __bf16*)v,
                                (const __bf16*)o, (const __bf16*)dout, (const float*)lse,
                                (__bf16*)dq, (__bf16*)dk, (__bf16*)dv, workspace, heads, N, scale,
                                mk, prepared, s, g_tm);
  }
  return hip_status(e, "backward launch");
}

// ---- the allocation-free backward ------------------------------------------
//
// attn_causal_bwd_noalloc runs the backward with its workspace in this
// statically allocated device array instead of a caller buffer.  Each GPU the
// library runs on holds its own copy for the life of the process.  The host
// name `scratch` is only a stand-in for the device symbol: host code uses the
// address hipGetSymbolAddress returns for the current device, never the name.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_at[kMaxDevices] = {};  // scratch's device address, per device

// scratch's address on the current device, looked up once per device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev)) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(ATTN_EUNSUPPORTED, "device %d: the scratch table holds %d devices", dev,
                kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_at[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)))
      return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(ATTN_EHIP, "hipGetSymbolAddress(scratch) returned a null address");
    g_scratch_at[dev] = p;
  }
  *out = g_scratch_at[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_causal_bwd_noalloc(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D,
                            double scale, const void* q, const void* k, const void* v,
                            const void* o, const void* dout, const void* lse, void* dq, void* dk,
                            void* dv, void* stream) {
  if (int rc = check_sizes(dtype, B, H, N, D, scale)) return rc;
  const size_t need = workspace_bytes_for(dtype, B * H, N);
  if (need > kScratchBytes)
    return fail(ATTN_EINVAL,
                "B*H*N = %lld rows need %zu bytes of backward workspace; the static scratch "
                "holds %zu (use attn_causal_bwd with a caller workspace)",
                (long long)(B * H * N), need, kScratchBytes);
  void* ws = nullptr;
  if (int rc = scratch_on_current_device(&ws)) return rc;
  // every per-row value the kernels read is written first by the backward's
  // own per-row pass, so the scratch needs no clearing between calls
  return bwd_impl(dtype, B, H, N, D, scale, ATTN_MASK_CAUSAL, 0, nullptr, q, k, v, o, dout, lse,
                  dq, dk, dv, ws, kScratchBytes, false, (hipStream_t)stream);
}

int attn_fwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale, attn_mask_t mask,
             int64_t window, const void* q, const void* k, const void* v, void* o, void* lse,
             void* stream) {
  return fwd_impl(dtype, B, H, N, D, scale, mask, window, nullptr, q, k, v, o, lse, nullptr,
                  (hipStream_t)stream);
}

int attn_fwd_seg(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                 attn_mask_t mask, int64_t window, const int32_t* seg, const void* q,
                 const void* k, const void* v, void* o, void* lse, void* stream) {
  if (!seg) return fail(ATTN_EINVAL, "null segment ids");
  return fwd_impl(dtype, B, H, N, D, scale, mask, window, seg, q, k, v, o, lse, nullptr,
                  (hipStream_t)stream);
}

int attn_causal_fwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                    const void* q, const void* k, const void* v, void* o, void* lse,
                    void* stream) {
  return attn_fwd(dtype, B, H, N, D, scale, ATTN_MASK_CAUSAL, 0, q, k, v, o, lse, stream);
}

size_t attn_causal_bwd_workspace_bytes(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D) {
  if (check_sizes(dtype, B, H, N, D, 1.0) != ATTN_OK) return 0;
  return workspace_bytes_for(dtype, B * H, N);
}

size_t attn_bwd_workspace_bytes(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D) {
  return attn_causal_bwd_workspace_bytes(dtype, B, H, N, D);
}

int attn_bwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale, attn_mask_t mask,
             int64_t window, const void* q, const void* k, const void* v, const void* o,
             const void* dout, const void* lse, void* dq, void* dk, void* dv, void* workspace,
             size_t workspace_bytes, void* stream) {
  return bwd_impl(dtype, B, H, N, D, scale, mask, window, nullptr, q, k, v, o, dout, lse, dq, dk,
                  dv, workspace, workspace_bytes, false, (hipStream_t)stream);
}

int attn_bwd_seg(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                 attn_mask_t mask, int64_t window, const int32_t* seg, const void* q,
                 const void* k, const void* v, const void* o, const void* dout, const void* lse,
                 void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                 void* stream) {
  if (!seg) return fail(ATTN_EINVAL, "null segment ids");
  return bwd_impl(dtype, B, H, N, D, scale, mask, window, seg, q, k, v, o, dout, lse, dq, dk, dv,
                  workspace, workspace_bytes, false, (hipStream_t)stream);
}

int attn_causal_bwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                    const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const void* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd(dtype, B, H, N, D, scale, ATTN_MASK_CAUSAL, 0, q, k, v, o, dout, lse, dq, dk,
                  dv, workspace, workspace_bytes, stream);
}

int attn_fwd_train(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale, attn_mask_t mask,
                   int64_t window, const void* q, const void* k, const void* v, void* o,
                   void* lse, void* workspace, size_t workspace_bytes, double* loss,
                   void* stream) {
  if (int rc = check_sizes(dtype, B, H, N, D, scale)) return rc;
  if (!workspace || !loss) return fail(ATTN_EINVAL, "null pointer argument");
  if (!aligned16(workspace) || ((uintptr_t)loss & 7u))
    return fail(ATTN_EINVAL, "workspace must be 16-byte and loss 8-byte aligned");
  const int64_t heads = B * H;
  const size_t need = workspace_bytes_for(dtype, heads, N);
  if (workspace_bytes < need)
    return fail(ATTN_EINVAL, "workspace of %zu bytes is smaller than the %zu required",
                workspace_bytes, need);
  const size_t tb = (size_t)heads * N * D * elem_size(dtype);
  const size_t lb = (size_t)heads * N * (dtype == ATTN_F64 ? 8 : 4);
  const void* all[] = {q, k, v, o};
  for (const void* p : all)
    if (overlap(loss, 8, p, tb)) return fail(ATTN_EINVAL, "loss aliases a tensor");
  if (overlap(loss, 8, lse, lb) || overlap(loss, 8, workspace, need))
    return fail(ATTN_EINVAL, "loss aliases lse or the workspace");
  hipStream_t s = (hipStream_t)stream;
  if (int rc = fwd_impl(dtype, B, H, N, D, scale, mask, window, nullptr, q, k, v, o, lse,
                        workspace, s))
    return rc;
  const int kind = dtype == ATTN_F64 ? 0 : dtype == ATTN_F32 ? 1 : 2;
  double* parts = (double*)((char*)workspace + parts_offset(dtype, heads, N));
  return hip_status(attn::launch_loss(kind, workspace, heads * N, parts, loss, s),
                    "attn_fwd_train loss launch");
}

int attn_bwd_from_fwd(attn_dtype_t dtype, int64_t B, int64_t H, int64_t N, int64_t D, double scale,
                      attn_mask_t mask, int64_t window, const void* q, const void* k, const void* v,
                      const void* o, const void* lse, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(dtype, B, H, N, D, scale, mask, window, nullptr, q, k, v, o, o, lse, dq, dk, dv,
                  workspace, workspace_bytes, true, (hipStream_t)stream);
}

int nw_gauss_average(int64_t n_targets, const float* tx, const float* ty, int64_t n_sources,
                     const float* sx, const float* sy, const float* sv, float denom,
                     float* out, void* stream) {
  if (n_targets < 1 || n_sources < 1)
    return fail(ATTN_EINVAL, "n_targets and n_sources must be >= 1");
  if (n_targets > (int64_t(1) << 30) || n_sources > (int64_t(1) << 30))
    return fail(ATTN_EINVAL, "at most 2^30 targets and sources");
  if (!(denom > 0.f) || !isfinite(denom)) return fail(ATTN_EINVAL, "denom must be finite and > 0");
  if (!tx || !ty || !sx || !sy || !sv || !out) return fail(ATTN_EINVAL, "null pointer argument");
  const void* cols[] = {tx, ty, sx, sy, sv, out};
  for (const void* p : cols)
    if ((uintptr_t)p & 3u) return fail(ATTN_EINVAL, "pointers must be 4-byte aligned");
  const size_t tb = (size_t)n_targets * 4, sb = (size_t)n_sources * 4;
  if (overlap(out, tb, tx, tb) || overlap(out, tb, ty, tb) || overlap(out, tb, sx, sb) ||
      overlap(out, tb, sy, sb) || overlap(out, tb, sv, sb))
    return fail(ATTN_EINVAL, "out must not alias an input");
  hipError_t e = attn::launch_nw(n_targets, tx, ty, n_sources, sx, sy, sv, denom, out,
                                 (hipStream_t)stream, g_tm);
  return hip_status(e, "nw_gauss_average launch");
}

size_t attn_table_workspace_bytes(attn_dtype_t dtype, int64_t T, int64_t D) {
  if (dtype != ATTN_F64 && dtype != ATTN_F32 && dtype != ATTN_BF16) {
    fail(ATTN_EINVAL, "unknown dtype %d", dtype);
    return 0;
  }
  if (T < 1 || D < 1 || T > kMaxCells / D) {
    fail(ATTN_EINVAL, "T and D must be >= 1 with at most %lld cells", (long long)kMaxCells);
    return 0;
  }
  return attn::table_workspace_bytes((int)elem_size(dtype), T, D);
}

int attn_table_to_matrix(attn_dtype_t dtype, int64_t rows, const int64_t* t, const int64_t* d,
                         const void* x, int64_t T, int64_t D, void* m, int32_t* status,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != ATTN_F64 && dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_EINVAL, "unknown dtype %d", dtype);
  if (rows < 1 || T < 1 || D < 1) return fail(ATTN_EINVAL, "rows, T and D must be >= 1");
  if (T > kMaxCells / D || rows > kMaxCells)
    return fail(ATTN_EINVAL, "at most %lld cells and rows", (long long)kMaxCells);
  if (!t || !d || !x || !m || !status || !workspace)
    return fail(ATTN_EINVAL, "null pointer argument");
  const size_t es = elem_size(dtype);
  if (((uintptr_t)t & 7u) || ((uintptr_t)d & 7u) || ((uintptr_t)x & (es - 1)) ||
      ((uintptr_t)status & 3u) || !aligned16(m) || !aligned16(workspace))
    return fail(ATTN_EINVAL, "misaligned pointer (t, d: 8; x: element; m, workspace: 16; status: 4)");
  const size_t need = attn::table_workspace_bytes((int)es, T, D);
  if (workspace_bytes < need)
    return fail(ATTN_EINVAL, "workspace of %zu bytes is smaller than the %zu required",
                workspace_bytes, need);
  const size_t ib = (size_t)rows * 8, xb = (size_t)rows * es, mb = (size_t)T * D * es;
  if (overlap(m, mb, t, ib) || overlap(m, mb, d, ib) || overlap(m, mb, x, xb) ||
      overlap(m, mb, workspace, need) || overlap(m, mb, status, 4))
    return fail(ATTN_EINVAL, "the matrix must not alias an input, the workspace or the status");
  if (overlap(workspace, need, t, ib) || overlap(workspace, need, d, ib) ||
      overlap(workspace, need, x, xb) || overlap(workspace, need, status, 4))
    return fail(ATTN_EINVAL, "the workspace must not alias an input or the status");
  if (overlap(status, 4, t, ib) || overlap(status, 4, d, ib) || overlap(status, 4, x, xb))
    return fail(ATTN_EINVAL, "the status must not alias an input");
  return hip_status(attn::launch_table_to_matrix((int)es, rows, t, d, x, T, D, m, status,
                                                 workspace, (hipStream_t)stream, g_tm),
                    "attn_table_to_matrix launch");
}

int attn_matrix_to_table(attn_dtype_t dtype, int64_t T, int64_t D, const void* m, int64_t* t, int64_t* d,
                         void* x, void* stream) {
  if (dtype != ATTN_F64 && dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_EINVAL, "unknown dtype %d", dtype);
  if (T < 1 || D < 1) return fail(ATTN_EINVAL, "T and D must be >= 1");
  if (T > kMaxCells / D) return fail(ATTN_EINVAL, "at most %lld cells", (long long)kMaxCells);
  if (!m || !t || !d || !x) return fail(ATTN_EINVAL, "null pointer argument");
  const size_t es = elem_size(dtype);
  if (!aligned16(t) || !aligned16(d) || !aligned16(x) || !aligned16(m))
    return fail(ATTN_EINVAL, "pointers must be 16-byte aligned");
  const size_t cells = (size_t)T * D, ib = cells * 8, xb = cells * es;
  if (overlap(t, ib, m, xb) || overlap(d, ib, m, xb) || overlap(x, xb, m, xb) ||
      overlap(t, ib, d, ib) || overlap(t, ib, x, xb) || overlap(d, ib, x, xb))
    return fail(ATTN_EINVAL, "t, d and x must not overlap each other or the matrix");
  return hip_status(attn::launch_matrix_to_table((int)es, T, D, m, t, d, x, (hipStream_t)stream),
                    "attn_matrix_to_table launch");
}

int attn_qkv_project(attn_dtype_t dtype, int64_t B, int64_t N, int64_t Dm, int64_t H, const void* x,
                     const void* wq, const void* wk, const void* wv, void* q, void* k, void* v,
                     void* stream) {
  if (dtype != ATTN_F64 && dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_EINVAL, "unknown dtype %d", dtype);
  if (B < 1 || N < 1 || Dm < 1 || H < 1)
    return fail(ATTN_EINVAL, "sizes must be >= 1 (B=%lld N=%lld Dm=%lld H=%lld)", (long long)B,
                (long long)N, (long long)Dm, (long long)H);
  if (H > 65535) return fail(ATTN_EINVAL, "at most 65535 heads");
  if (N > kMaxN || B > (int64_t(1) << 31) / N)
    return fail(ATTN_EINVAL, "B*N must be below 2^31 and N at most %lld", (long long)kMaxN);
  if (Dm > kMaxCells / (B * N) || Dm > kMaxCells / (H * 64))
    return fail(ATTN_EINVAL, "x or a weight matrix exceeds %lld elements", (long long)kMaxCells);
  if (!x || !wq || !wk || !wv || !q || !k || !v) return fail(ATTN_EINVAL, "null pointer argument");
  const void* all[] = {x, wq, wk, wv, q, k, v};
  for (const void* p : all)
    if (!aligned16(p)) return fail(ATTN_EINVAL, "pointers must be 16-byte aligned");
  const size_t es = elem_size(dtype);
  const size_t xb = (size_t)B * N * Dm * es, wb = (size_t)Dm * H * 64 * es,
               ob = (size_t)B * H * N * 64 * es;
  const void* ins[] = {wq, wk, wv};
  void* outs[] = {q, k, v};
  for (void* o : outs) {
    if (overlap(o, ob, x, xb)) return fail(ATTN_EINVAL, "outputs must not alias inputs");
    for (const void* w : ins)
      if (overlap(o, ob, w, wb)) return fail(ATTN_EINVAL, "outputs must not alias inputs");
  }
  if (overlap(q, ob, k, ob) || overlap(q, ob, v, ob) || overlap(k, ob, v, ob))
    return fail(ATTN_EINVAL, "q, k and v must not overlap");
  return hip_status(attn::launch_project((int)es, B, N, Dm, H, x, wq, wk, wv, q, k, v,
                                         (hipStream_t)stream, g_tm),
                    "attn_qkv_project launch");
}

int attn_set_kernel_timer(int slot, void* start, void* stop) {
  if (slot < 0 || slot >= ATTN_TIMER_SLOTS) return fail(ATTN_EINVAL, "unknown timer slot %d", slot);
  if ((start == nullptr) != (stop == nullptr))
    return fail(ATTN_EINVAL, "pass both events or neither");
  g_tm.start[slot] = (hipEvent_t)start;
  g_tm.stop[slot] = (hipEvent_t)stop;
  g_err.clear();
  return ATTN_OK;
}

const char* attn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
