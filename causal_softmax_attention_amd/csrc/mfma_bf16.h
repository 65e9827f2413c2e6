// bfloat16 MFMA building blocks for gfx950 shared by the attention kernels.
//
// v_mfma_f32_32x32x16_bf16 computes C[32x32] += A[32x16] B[16x32].  With lane
// l = 32 h + i (h in {0,1}, i in 0..31):
//   A operand: lane holds A[m = i][k = 8h .. 8h+7]       (8 bf16)
//   B operand: lane holds B[k = 8h .. 8h+7][n = i]       (8 bf16)
//   C / D    : lane holds C[m = 8(r/4) + 4h + r%4][n = i] for r = 0..15 (float)
// An accumulator C (M x N) is therefore usable, after rounding to bf16, as the
// B operand of a product that contracts over its M index: register r = 8c + t
// of the tile is contraction slot t of chunk c (16 rows), i.e. row
// 16c + 8(t/4) + 4h + t%4.  The matching A operand (the other factor, M' x that
// index) must present the same row order: slots 0..3 are rows 16c + 4h + 0..3,
// slots 4..7 rows 16c + 8 + 4h + 0..3.  ds_read_b64_tr_b16 produces exactly
// that from a row-major tile in LDS: the 16 lanes of a group each point at 4
// consecutive elements of a 4-row x 16-column block (lane c16: row c16/4,
// columns 4(c16%4)..+3) and lane c16 receives column c16, rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {
namespace mfma {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kRowElems = 64;  // one tile row: 64 bf16 = 128 B = eight 16-byte chunks

__device__ __forceinline__ floatx16 mma(bf16x8_t a, bf16x8_t b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tiles in LDS are row-major [rows][64] bf16 with chunk c of row r stored at
// chunk c ^ swz(r).  LDS has 64 four-byte banks (256 bytes a clock), so a
// row's physical chunk p lies in bank group 8 (r & 1) + p of sixteen.
//  - A 16-byte row read serves 16 lanes a clock: sixteen consecutive rows,
//    one logical chunk.  swz maps row bits 1-3 one-to-one onto three bits, so
//    the eight rows of either parity take eight different chunks: no two
//    lanes share a bank.
//  - A transposing 8-byte read serves 32 lanes a clock: four consecutive
//    rows (from a multiple of 4) x four chunks.  Rows r and r + 2 share a bank
//    half; row bit 1 flips swz's top bit and so moves them to opposite
//    halves of the eight chunks.
// (A swizzle over row bits 0-2 alone left the row reads two-way conflicted:
// rows r and r + 8 then collide.)
__device__ __forceinline__ int swz(int row) {
  return (((row >> 1) & 1) << 2) | (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
}
__device__ __forceinline__ int lds_at(int row, int col) {
  return row * kRowElems + (((col >> 3) ^ swz(row)) << 3) + (col & 7);
}

// A or B operand from the 16 bytes at (row, col..col+7) of a swizzled tile.
__device__ __forceinline__ bf16x8_t read_row8(const __bf16* tile, int row, int col) {
  return *(const bf16x8_t*)(tile + lds_at(row, col));
}

// Operand holding, for this lane's column `col0 + i`, rows (within chunk c of
// 16 rows) 16c + 4h + 0..3 and 16c + 8 + 4h + 0..3 of a row-major tile: the
// partner of a bf16-packed accumulator chunk (see the header comment).
__device__ __forceinline__ bf16x8_t read_tr(const __bf16* tile, int lane, int c, int col0) {
  const int g16 = lane >> 4, c16 = lane & 15;
  const int col = col0 + 16 * (g16 & 1) + 4 * (c16 & 3);
  const int row = 16 * c + 4 * (g16 >> 1) + (c16 >> 2);
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + lds_at(row, col)));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(tile + lds_at(row + 8, col)));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

// B operand of chunk c (rows 16c..16c+15 of a 32-row tile: c in {0,1}) from a
// bf16-packed accumulator tile held as 8 dwords.
__device__ __forceinline__ bf16x8_t chunk_op(const uint32_t* packed8, int c) {
  const uint4 w = make_uint4(packed8[4 * c + 0], packed8[4 * c + 1], packed8[4 * c + 2],
                             packed8[4 * c + 3]);
  return __builtin_bit_cast(bf16x8_t, w);
}

// Row of the accumulator register r held by lane-half h (within a 32-row tile).
__device__ __forceinline__ int acc_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Workgroup -> (head, block): workgroup b runs on XCD b % 8, so the blocks of
// head x, x + 8, ... go to XCD x (their shared K/V or Q/dO rows stay in that
// XCD's L2).  An XCD takes its heads in groups of `group`; within a group the
// blocks start heaviest first across the group's heads (rank 0 of every head,
// then rank 1, ...), where rank r is block nblk - 1 - r when `last_first` (the
// causal forward and dQ, whose last block walks the most keys) and block r
// otherwise.  Under a causal mask the light blocks then fill the end of the
// launch instead of one head's heavy block starting last.  With merge_tail,
// the last two whole groups and any remainder form one final group: a final
// group of few heads holds few blocks per slot of the XCD, so its heaviest
// blocks, starting near the end of the launch, would leave a tail.
__device__ __forceinline__ bool map_block(int b, int heads, int nblk, bool last_first, int group,
                                          int& head, int& blk, bool merge_tail = false) {
  const int xcd = b & 7, slot = b >> 3;
  const int hx = (heads - xcd + 7) >> 3;  // heads with head % 8 == xcd
  if (slot >= hx * nblk) return false;
  const int tail0 = merge_tail ? max(0, (hx / group - 2) * group) : hx;  // first head of the final group
  int h0, gc, within;
  if (slot >= tail0 * nblk) {
    h0 = tail0;
    gc = hx - tail0;
    within = slot - tail0 * nblk;
  } else {
    const int chunk = slot / (group * nblk);
    h0 = chunk * group;
    gc = min(group, hx - h0);             // heads in this group (the last may be short)
    within = slot - chunk * group * nblk;
  }
  const int r = within / gc, hi = h0 + within % gc;
  head = xcd + 8 * hi;
  blk = last_first ? nblk - 1 - r : r;
  return true;
}

__device__ __forceinline__ uint4 ldg16(const __bf16* p) { return *(const uint4*)p; }

// ---- asynchronous global -> LDS staging -----------------------------------
//
// buffer_load_dwordx4 ... lds writes lane i's 16 bytes to LDS at M0 + 16 i.
// A buffer resource covering exactly one head makes rows past its end read
// as zeros (no fault, no branch).  Tiles are staged with these loads two
// tiles ahead; the wait before each barrier leaves the newest tile's loads in
// flight (wait_vm_barrier), and the stages are distinct __shared__ objects
// referenced statically, so the compiler can tell a read of one stage from
// the copy still landing in another.

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Copy rows [row0, row0 + ROWS) (64 bf16 each) of the resource's head into a
// swizzled LDS tile.  Every thread of a WAVES-wave workgroup issues
// ROWS / (8 WAVES) loads; wave w fills the 1 KiB stretches u * WAVES + w, lane
// l slot l of it, and slot p of the tile holds row p / 8, physical chunk p % 8.
template <int ROWS, int WAVES = 4>
__device__ __forceinline__ void tile_async(__amdgpu_buffer_rsrc_t rsrc, __bf16* tile, int row0,
                                           int wave, int lane) {
  static_assert(ROWS % (8 * WAVES) == 0, "whole stretches per wave");
#pragma unroll
  for (int u = 0; u < ROWS / (8 * WAVES); ++u) {
    const int s = u * WAVES + wave;
    const int p = s * 64 + lane, row = p >> 3;
    const int logical = (p & 7) ^ swz(row);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(tile + s * 512), 16,
                                             (row0 + row) * 128 + logical * 16, 0, 0, 0);
  }
}

// Copy 64 floats [row0, row0 + 64) of a per-row array into LDS (one wave, one
// 4-byte load per lane).
__device__ __forceinline__ void rows_async(__amdgpu_buffer_rsrc_t rsrc, float* dst, int row0,
                                           int lane) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 4, (row0 + lane) * 4, 0, 0, 0);
}

// Wait until at most N of this wave's buffer loads are in flight and all its
// LDS accesses are done, then barrier (no release fence: the loads still in
// flight belong to a stage nobody reads before the next barrier).
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
  __builtin_amdgcn_s_barrier();
}

}  // namespace mfma
}  // namespace attn
