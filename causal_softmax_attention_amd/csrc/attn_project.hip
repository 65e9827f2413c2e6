// Query, key and value input projections (pages: the "Wiki notes" page,
// brainpick-2k7.pages.dev, its MLIR functions @attention_head and
// @mini_attention: Q = x Wq, K = x Wk, V = x Wv, one matmul each, from the
// token embeddings x and three d_model x d_k weight matrices).
//
// Shapes: x [B, N, Dm] (one embedding row per token), W [Dm, H * 64] with
// head h in columns 64 h .. 64 h + 63, and Q, K, V written as the attention
// takes them, [B, H, N, 64] (head-major: the reshape and transpose of x W are
// folded into the stores).  The three products share one read of x: a single
// launch forms all three.
//
// bfloat16 with Dm a multiple of 64: one workgroup = 12 waves = 256 tokens x
// one head x all three matrices; wave w forms matrix w / 4 for 64 of the
// tokens.  A wave accumulates the transposed tiles C^T = W^T X^T
// (v_mfma_f32_32x32x16_bf16, float32 accumulators), so a lane holds one token
// and 16 of its features and stores them as 8-byte runs of one output row.
// K-chunks of 64 stream through two LDS stages filled by asynchronous
// bounds-checked buffer loads (rows past the last token read as zeros): the
// 256 x 64 slice of x and the 64 x 64 block of each weight matrix.  The W^T operand comes from transposing LDS reads
// (ds_read_b64_tr_b16: lane i gets column i, rows 4h..4h+3 and 8+4h..8+4h+3 of
// a 16-row chunk); the x operand is read with the same row order, two 8-byte
// reads per lane.  Workgroups of one XCD run in tiles of 4 token blocks x 8
// heads (the 32 it holds at once), so each tile reads its blocks of x and its
// heads' weights from HBM once and reuses them from that XCD's L2.
//
// Every other case (float32, float64, or a Dm that is not a multiple of 64):
// a tiled VALU kernel, 64 tokens x one head per workgroup, each thread 4
// tokens x 4 features of all three matrices, accumulating in float32
// (bfloat16, float32) or float64.
#include "common.h"
#include "launch.h"
#include "mfma_bf16.h"

namespace attn {
namespace {

using namespace mfma;

constexpr int kWaves = 12;               // 3 matrices x 4 token groups
constexpr int kThreads = 64 * kWaves;
constexpr int kTok = 256;                // tokens per workgroup (64 per wave)
constexpr int kKc = 64;                  // d_model per LDS stage

struct alignas(16) ProjStage {
  __bf16 x[kTok * kKc];     // 256 tokens x 64 (swizzled rows of 64)
  __bf16 w[3][kKc * 64];    // per matrix: 64 rows of d_model x the head's 64 columns
};

// One 1 KiB group s (rows 8s .. 8s + 7) of a swizzled LDS tile of 64-column
// bf16 rows, from rows row0 + 8s .. of a row-major matrix with a row pitch of
// `pitch` bytes, columns from byte `col_off` (lane l writes slot 64 s + l: row
// (64 s + l) / 8, physical chunk l % 8 holding logical chunk (l % 8) ^ swz(row)).
__device__ __forceinline__ void group_async(__amdgpu_buffer_rsrc_t rsrc, __bf16* tile, int row0,
                                            uint32_t pitch, uint32_t col_off, int s, int lane) {
  const int p = s * 64 + lane, row = p >> 3;
  const int logical = (p & 7) ^ swz(row);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(tile + s * 512), 16,
                                           (uint32_t)(row0 + row) * pitch + col_off + logical * 16,
                                           0, 0, 0);
}

// x operand of the token at `row` of the stage for 16-wide chunk c: d_model
// 16c + 4h .. +3 and 16c + 8 + 4h .. +3 (the row order of the transposing read).
__device__ __forceinline__ bf16x8_t read_x(const __bf16* tile, int row, int c, int h) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
  const bf16x4_t lo = *(const bf16x4_t*)(tile + lds_at(row, 16 * c + 4 * h));
  const bf16x4_t hi = *(const bf16x4_t*)(tile + lds_at(row, 16 * c + 8 + 4 * h));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Wave w forms matrix w / 4 for tokens 64 (w % 4) .. + 63 of the workgroup's
// 256; waves 0-7 stage the x slice (32 groups of 1 KiB), waves 8-11 the three
// weight blocks (24 groups).
__global__ __launch_bounds__(kThreads, 1) void project_bf16_mfma(
    const __bf16* __restrict__ x, const __bf16* __restrict__ w0, const __bf16* __restrict__ w1,
    const __bf16* __restrict__ w2, __bf16* __restrict__ o0, __bf16* __restrict__ o1,
    __bf16* __restrict__ o2, int M, int N, int Dm, int H, int nrt) {
  __shared__ ProjStage st0, st1;
  // workgroup b runs on XCD b % 8 and takes token block xcd + 8 k.  The XCD's
  // workgroups go in tiles of RB token blocks x HB heads (32 at most, as many
  // as the XCD runs at once), so a tile reads RB blocks of x and HB heads of
  // weights, each from HBM once and then from the XCD's L2
  const int HB = H < 8 ? H : 8, RB = 32 / HB, BS = HB * RB;
  const int hgroups = (H + HB - 1) / HB;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int blk = slot / BS, idx = slot - blk * BS;
  const int rtg = blk / hgroups, hgi = blk - rtg * hgroups;
  const int rt = (rtg * RB + idx / HB) * 8 + xcd, head = hgi * HB + idx % HB;
  if (rt >= nrt || head >= H) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mat = wave >> 2, tg = wave & 3;
  const int i32 = lane & 31, h = lane >> 5;
  const int m0 = rt * kTok;
  const uint32_t xpitch = (uint32_t)Dm * 2, wpitch = (uint32_t)H * 128;
  const __amdgpu_buffer_rsrc_t rx = head_rsrc(x, (uint32_t)M * xpitch);
  const uint32_t wbytes = (uint32_t)Dm * wpitch;
  const __amdgpu_buffer_rsrc_t rw[3] = {head_rsrc(w0, wbytes), head_rsrc(w1, wbytes),
                                        head_rsrc(w2, wbytes)};
  // waves 8-11 stage the weight blocks: group 4 (u & 1) + (wave - 8) of block
  // u >> 1 for u = 0..5
  auto issue = [&](ProjStage& s, int k0) {
    if (wave < 8) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        group_async(rx, s.x, m0, xpitch, (uint32_t)k0 * 2, 8 * u + wave, lane);
    } else {
#pragma unroll
      for (int u = 0; u < 6; ++u)
        group_async(rw[u >> 1], s.w[u >> 1], k0, wpitch, (uint32_t)head * 128,
                    4 * (u & 1) + (wave - 8), lane);
    }
  };

  floatx16 acc[2][2];  // [feature half nt][token half mt]: C^T tiles
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = floatx16{};

  auto compute = [&](const ProjStage& s) {
    const __bf16* wt = s.w[0] + mat * (kKc * 64);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      bf16x8_t xb[2], wa[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) xb[mt] = read_x(s.x, 64 * tg + 32 * mt + i32, c, h);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) wa[nt] = read_tr(wt, lane, c, 32 * nt);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[nt][mt] = mma(wa[nt], xb[mt], acc[nt][mt]);
    }
  };

  const int nk = Dm / kKc;
  issue(st0, 0);
  wait_vm_barrier<0>();
  for (int kc = 0; kc < nk; kc += 2) {
    if (kc + 1 < nk) issue(st1, (kc + 1) * kKc);
    compute(st0);
    wait_vm_barrier<0>();  // stage 1 has landed; every wave is done with stage 0
    if (kc + 1 >= nk) break;
    if (kc + 2 < nk) issue(st0, (kc + 2) * kKc);
    compute(st1);
    wait_vm_barrier<0>();
  }

  // epilogue: lane holds token m0 + 64 tg + 32 mt + i32, features
  // 32 nt + 8 g + 4 h .. +3 in registers 4 g .. 4 g + 3
  __bf16* out = mat == 0 ? o0 : mat == 1 ? o1 : o2;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int m = m0 + 64 * tg + 32 * mt + i32;
    if (m >= M) continue;
    const int b = m / N, n = m - b * N;
    __bf16* row = out + (((size_t)b * H + head) * N + n) * kD;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v;
        v.x = pack_bf16(acc[nt][mt][4 * g + 0], acc[nt][mt][4 * g + 1]);
        v.y = pack_bf16(acc[nt][mt][4 * g + 2], acc[nt][mt][4 * g + 3]);
        *(uint2*)(row + 32 * nt + 8 * g + 4 * h) = v;
      }
  }
}

// ---- tiled VALU kernel (any dtype, any Dm) -------------------------------
constexpr int kVT = 64;   // tokens per workgroup
constexpr int kVK = 16;   // d_model per LDS step

template <typename T>
__global__ __launch_bounds__(256) void project_valu(const T* __restrict__ x, const T* __restrict__ w0,
                                                    const T* __restrict__ w1,
                                                    const T* __restrict__ w2, T* __restrict__ o0,
                                                    T* __restrict__ o1, T* __restrict__ o2,
                                                    int64_t M, int64_t N, int64_t Dm, int64_t H) {
  using A = acc_t<T>;
  __shared__ A xs[kVK][kVT + 1];
  __shared__ A ws[3][kVK][kD];
  const int64_t m0 = (int64_t)blockIdx.x * kVT;
  const int64_t head = blockIdx.y;
  const int tid = threadIdx.x;
  const int tm = tid >> 4, tf = tid & 15;  // tokens 4 tm .. +3, features 4 tf .. +3
  const T* ws_src[3] = {w0, w1, w2};
  A acc[3][4][4];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) acc[j][a][b] = A(0);
  const int64_t ncol = H * kD;
  for (int64_t k0 = 0; k0 < Dm; k0 += kVK) {
    for (int e = tid; e < kVT * kVK; e += 256) {
      const int r = e / kVK, c = e % kVK;
      const int64_t m = m0 + r, k = k0 + c;
      xs[c][r] = (m < M && k < Dm) ? widen(x[m * Dm + k]) : A(0);
    }
    for (int e = tid; e < 3 * kVK * kD; e += 256) {
      const int j = e / (kVK * kD), rem = e % (kVK * kD), c = rem / kD, f = rem % kD;
      const int64_t k = k0 + c;
      ws[j][c][f] = k < Dm ? widen(ws_src[j][k * ncol + head * kD + f]) : A(0);
    }
    __syncthreads();
#pragma unroll 4
    for (int c = 0; c < kVK; ++c) {
      A xv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) xv[a] = xs[c][4 * tm + a];
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const A wv = ws[j][c][4 * tf + b];
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[j][a][b] = fma(xv[a], wv, acc[j][a][b]);
        }
    }
    __syncthreads();
  }
  T* outs[3] = {o0, o1, o2};
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int64_t m = m0 + 4 * tm + a;
    if (m >= M) continue;
    const int64_t b = m / N, n = m - b * N;
    T* row = nullptr;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      row = outs[j] + ((b * H + head) * N + n) * kD + 4 * tf;
#pragma unroll
      for (int f = 0; f < 4; ++f) row[f] = narrow<T>(acc[j][a][f]);
    }
  }
}

}  // namespace

bool project_uses_mfma(int elem_bytes, int64_t M, int64_t Dm, int64_t H) {
  return elem_bytes == 2 && Dm % kKc == 0 && M * Dm * 2 < (int64_t(1) << 31) &&
         Dm * H * 128 < (int64_t(1) << 31) && M < (int64_t(1) << 30);
}

hipError_t launch_project(int elem_bytes, int64_t B, int64_t N, int64_t Dm, int64_t H,
                          const void* x, const void* wq, const void* wk, const void* wv, void* q,
                          void* k, void* v, hipStream_t stream, const Timers& tm) {
  const int64_t M = B * N;
  if (hipError_t e = mark(tm.start[kTimerProject], stream)) return e;
  if (project_uses_mfma(elem_bytes, M, Dm, H)) {
    const int nrt = (int)((M + kTok - 1) / kTok);
    const int64_t HB = H < 8 ? H : 8, RB = 32 / HB, hgroups = (H + HB - 1) / HB;
    const int64_t per_xcd = (nrt + 7) / 8;   // token blocks of one XCD
    const unsigned grid = (unsigned)(8 * ((per_xcd + RB - 1) / RB) * hgroups * (HB * RB));
    hipLaunchKernelGGL(project_bf16_mfma, dim3(grid), dim3(kThreads), 0, stream,
                       (const __bf16*)x, (const __bf16*)wq, (const __bf16*)wk, (const __bf16*)wv,
                       (__bf16*)q, (__bf16*)k, (__bf16*)v, (int)M, (int)N, (int)Dm, (int)H, nrt);
  } else {
    const dim3 grid((unsigned)((M + kVT - 1) / kVT), (unsigned)H);
    switch (elem_bytes) {
      case 8:
        hipLaunchKernelGGL(project_valu<double>, grid, dim3(256), 0, stream, (const double*)x,
                           (const double*)wq, (const double*)wk, (const double*)wv, (double*)q,
                           (double*)k, (double*)v, M, N, Dm, H);
        break;
      case 4:
        hipLaunchKernelGGL(project_valu<float>, grid, dim3(256), 0, stream, (const float*)x,
                           (const float*)wq, (const float*)wk, (const float*)wv, (float*)q,
                           (float*)k, (float*)v, M, N, Dm, H);
        break;
      default:
        hipLaunchKernelGGL(project_valu<__bf16>, grid, dim3(256), 0, stream, (const __bf16*)x,
                           (const __bf16*)wq, (const __bf16*)wk, (const __bf16*)wv, (__bf16*)q,
                           (__bf16*)k, (__bf16*)v, M, N, Dm, H);
    }
  }
  if (hipError_t e = mark(tm.stop[kTimerProject], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
