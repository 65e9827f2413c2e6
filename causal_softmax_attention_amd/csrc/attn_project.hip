// Query, key and value input projections (pages: the "Wiki notes" page,
// brainpick-2k7.pages.dev, its MLIR functions @attention_head and
// @mini_attention: Q = x Wq, K = x Wk, V = x Wv, one matmul each, from the
// token embeddings x and three d_model x d_k weight matrices).
//
// Shapes: x [B, N, Dm] (one embedding row per token), W [Dm, H * 64] with
// head h in columns 64 h .. 64 h + 63, and Q, K, V written as the attention
// takes them, [B, H, N, 64] (head-major: the reshape and transpose of x W are
// folded into the stores).  One launch forms all three products.
//
// bfloat16 with Dm a multiple of 64: a GEMM over 256-token x 256-column tiles
// (4 heads of one matrix), 8 waves, 2 per SIMD.  Wave (wr, wc) accumulates the
// transposed tiles C^T = W^T X^T of tokens 128 wr .. + 127 and head wc of the
// tile (v_mfma_f32_32x32x16_bf16, float32 accumulators: 4 token x 2 column
// tiles, 128 registers), so a lane holds one token and 16 of its features and
// stores them as 8-byte runs of one output row.  64-wide slices of d_model
// stream through two LDS stages filled by asynchronous bounds-checked buffer
// loads (rows past the last token read as zeros).  Both operands are read in
// natural k order without bank conflicts: W^T by transposing reads
// (ds_read_b64_tr_b16) of 4 consecutive rows, x by 16-byte row reads.  An
// XCD's workgroups run in patches of 8 token blocks x 4 column groups, so each
// k-slice of x and W is read from L2 by several of the workgroups it holds at
// once.
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

constexpr int kKc = 64;                  // d_model per LDS stage

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

// W^T operand in natural k order: lane (h, i) gets column col0 + i, d_model
// rows 16 c + 8 h .. + 7 of a 64-row block (two transposing reads of 4 rows;
// each 16-lane group reads 4 consecutive rows x 32 bytes, which the swizzle
// puts in 32 different banks).  Its partner, the x operand, is then a plain
// 16-byte read of the token's row at 16 c + 8 h.
__device__ __forceinline__ bf16x8_t read_tr_nat(const __bf16* tile, int lane, int c, int col0) {
  const int g16 = lane >> 4, c16 = lane & 15;
  const int col = col0 + 16 * (g16 & 1) + 4 * (c16 & 3);
  const int row = 16 * c + 8 * (g16 >> 1) + (c16 >> 2);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + lds_at(row, col)));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + lds_at(row + 4, col)));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ---- 256 x 256 tiles, 4 x 2 MFMA tiles per wave ---------------------------
//
// Per 16-wide chunk of d_model a wave reads 4 x and 2 W^T operands for 8
// MFMAs (768 LDS bytes per MFMA); the next chunk's operands are read while
// this chunk's MFMAs run (5 % on the workload below).  Measured on
// x [8, 4096, 2048] with 32 heads: 0.82-0.87 ms.  Earlier forms: 12 waves of 2 x 2 tiles with x read in
// the accumulator-style k order (two 8-byte reads, 2-way bank conflicts),
// 0.96-1.10 ms; 4 waves of 4 x 4 tiles (256 accumulators, one wave per SIMD),
// 0.95 ms.
constexpr int gWaves = 8;
constexpr int gThreads = 64 * gWaves;
constexpr int gTok = 256;
constexpr int gHeads = 4;

struct alignas(16) GemmStage {
  __bf16 x[gTok * kKc];          // 256 tokens x 64 (swizzled rows of 64)
  __bf16 w[gHeads][kKc * 64];    // per head: 64 rows of d_model x its 64 columns
};

__global__ __launch_bounds__(gThreads, 2) void project_bf16_gemm(
    const __bf16* __restrict__ x, const __bf16* __restrict__ w0, const __bf16* __restrict__ w1,
    const __bf16* __restrict__ w2, __bf16* __restrict__ o0, __bf16* __restrict__ o1,
    __bf16* __restrict__ o2, int M, int N, int Dm, int H, int nrt, int ncg) {
  __shared__ GemmStage st0, st1;
  // workgroup b runs on XCD b % 8 and takes token blocks xcd + 8 k.  An XCD's
  // workgroups run in patches of 8 of its token blocks x 4 column
  // groups (the 32 it holds at once), so each k-slice of x is read by 4
  // workgroups and each k-slice of W by 8 while both sit in that XCD's L2
  constexpr int PR = 8, PC = 4;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int nrx = (nrt - xcd + 7) >> 3;     // token blocks of this XCD
  const int nct = 3 * ncg;                  // column groups (all three matrices)
  const int npc = (nct + PC - 1) / PC;
  const int patch = slot / (PR * PC), within = slot - patch * (PR * PC);
  const int rp = patch / npc, cp = patch - rp * npc;
  const int lr = rp * PR + within / PC, ct = cp * PC + within % PC;
  if (lr >= nrx || ct >= nct) return;
  const int rt = lr * 8 + xcd;
  const int mat = ct / ncg, head0 = (ct % ncg) * gHeads;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wave >> 2, wc = wave & 3;  // tokens 128 wr .., head head0 + wc
  const int i32 = lane & 31, h = lane >> 5;
  const int m0 = rt * gTok;
  const uint32_t xpitch = (uint32_t)Dm * 2, wpitch = (uint32_t)H * 128;
  const __amdgpu_buffer_rsrc_t rx = head_rsrc(x, (uint32_t)M * xpitch);
  const __amdgpu_buffer_rsrc_t rw =
      head_rsrc(mat == 0 ? w0 : mat == 1 ? w1 : w2, (uint32_t)Dm * wpitch);
  // 32 groups of 1 KiB for x (8 token rows each), 32 for W (8 rows of one
  // head's block each); wave w issues groups w, w + 8, ...
  auto issue = [&](GemmStage& s, int k0) {
#pragma unroll
    for (int u = 0; u < 32 / gWaves; ++u)
      group_async(rx, s.x, m0, xpitch, (uint32_t)k0 * 2, wave + gWaves * u, lane);
#pragma unroll
    for (int u = 0; u < 32 / gWaves; ++u) {
      const int g = wave + gWaves * u, hh = g >> 3;
      group_async(rw, s.w[hh], k0, wpitch, (uint32_t)(head0 + hh) * 128, g & 7, lane);
    }
  };

  floatx16 acc[2][4];  // [column tile nt][token tile mt]
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = floatx16{};

  auto compute = [&](const GemmStage& s) {
    // the lane as a value the compiler cannot see through: operand addresses
    // are formed per stage rather than hoisted for both stages (and held)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int li = ln & 31, lh = ln >> 5;
    // operands double-buffered: chunk c + 1 is read while chunk c's MFMAs run
    bf16x8_t xb[2][4], wa[2][2];
    auto load = [&](int c, int buf) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        xb[buf][mt] = read_row8(s.x, 128 * wr + 32 * mt + li, 16 * c + 8 * lh);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) wa[buf][nt] = read_tr_nat(s.w[wc], ln, c, 32 * nt);
    };
    load(0, 0);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c < 3) load(c + 1, (c + 1) & 1);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          acc[nt][mt] = mma(wa[c & 1][nt], xb[c & 1][mt], acc[nt][mt]);
      if (c < 3) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // the next chunk's 8 LDS reads
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // then this chunk's 8 MFMAs
      }
    }
  };

  // one loop body for both stages (a stage chosen at run time): an unrolled
  // pair with an exit between its halves made the compiler move the
  // accumulator registers between paths
  const int nk = Dm / kKc;
  issue(st0, 0);
  wait_vm_barrier<0>();
  for (int kc = 0; kc < nk; ++kc) {
    const bool odd = kc & 1;
    if (kc + 1 < nk) issue(odd ? st0 : st1, (kc + 1) * kKc);
    compute(odd ? st1 : st0);
    wait_vm_barrier<0>();  // the next stage has landed; every wave is done with this one
  }

  // epilogue: lane holds token m0 + 128 wr + 32 mt + i32, features 32 nt +
  // 8 g + 4 h .. +3 of head head0 + wc in registers 4 g .. 4 g + 3
  __bf16* out = mat == 0 ? o0 : mat == 1 ? o1 : o2;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int m = m0 + 128 * wr + 32 * mt + i32;
    if (m >= M) continue;
    const int b = m / N, n = m - b * N;
    const int head = head0 + wc;
    if (head >= H) continue;
    __bf16* row = out + (((size_t)b * H + head) * N + n) * kD;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 v;
        v.x = pack_bf16(acc[nt][mt][4 * g + 0], acc[nt][mt][4 * g + 1]);
        v.y = pack_bf16(acc[nt][mt][4 * g + 2], acc[nt][mt][4 * g + 3]);
        *(uint2*)(row + 32 * nt + 8 * g + 4 * h) = v;
      }
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
    const int nrt = (int)((M + gTok - 1) / gTok);
    const int ncg = (int)((H + gHeads - 1) / gHeads);
    const int64_t npr = ((nrt + 7) / 8 + 7) / 8, npc = (3 * ncg + 3) / 4;
    const unsigned grid = (unsigned)(8 * npr * npc * 32);
    hipLaunchKernelGGL(project_bf16_gemm, dim3(grid), dim3(gThreads), 0, stream,
                       (const __bf16*)x, (const __bf16*)wq, (const __bf16*)wk, (const __bf16*)wv,
                       (__bf16*)q, (__bf16*)k, (__bf16*)v, (int)M, (int)N, (int)Dm, (int)H, nrt,
                       ncg);
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
