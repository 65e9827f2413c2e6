// Causal attention forward for bfloat16 inputs on gfx950 MFMA (float32
// accumulation and softmax).
//
// Method (pages: "Show HN: automatic deduction of FlashAttention kernel from 25
// lines of SQL", the view `attention` and the FlashAttention plan it describes:
// stream blocks of keys past blocks of queries with a running softmax instead
// of storing the N x N scores).  For each query i: s_ij = scale * q_i . k_j over
// keys j <= i, o_i = sum_j exp(s_ij - m_i) v_j / sum_j exp(s_ij - m_i), and
// lse_i = m_i + ln sum_j exp(s_ij - m_i).
//
// Layout of the work (one workgroup = 4 waves = 256 queries of one head):
//   * Each wave owns 64 queries (two 32-query MFMA columns).  Q stays in
//     registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so
//     every lane holds one query column of the score tile: the softmax state
//     (reference max m, running sum l) is per lane, no row reduction crosses
//     lanes except the final l_lane + l_(lane^32).
//   * Keys stream in tiles of 64 through LDS (double buffered, one barrier per
//     tile).  K rows feed the A operand with plain 16-byte reads; V rows are
//     read with ds_read_b64_tr_b16, which hands each lane 4 consecutive keys
//     of one feature column: exactly the A operand of O^T = V^T P^T.  The
//     bf16-rounded P accumulator registers are the B operand as they stand.
//   * Causal block skipping: a wave stops at the tile holding its last query;
//     only the diagonal tile and the ragged tail (keys >= N) are masked, by
//     setting those scores to -inf (an absent pair gets weight exactly 0).
//
// Lazy max: the row max only keeps exp from overflowing; it cancels from the
// ratio (the page's remark on the window spelling).  Weights are therefore
// taken as exp2(s*c - m_ref) against a reference m_ref, and a tile is redone
// with its exact max (rescaling the accumulators) only when some weight would
// exceed 2^8 - detected from the lane's tile sum, so the common path spends no
// instruction on a max.  m_ref starts at -inf, so the first tile always takes
// the exact path.  Products p * v are then bounded by 2^8 |v|.
//
// Absent rows with non-finite V: a masked pair must contribute nothing, but
// the MFMA would form 0 * inf = NaN.  While staging a V tile, a flag records
// whether it holds any non-finite value; a diagonal (masked) tile with the flag
// set takes a select-based VALU path that skips masked pairs.
#include "common.h"
#include "launch.h"

namespace attn {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short v4s __attribute__((__vector_size__(4 * sizeof(short))));
typedef __attribute__((address_space(3))) v4s lds_v4s;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 64;                 // queries per wave
constexpr int kBr = kQW * kWaves;       // queries per workgroup
constexpr int kBc = 64;                 // keys per tile
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 256.0f;           // lazy-max bound on a weight (2^8)

struct Smem {
  __bf16 k[2][kBc * kD];
  __bf16 v[2][kBc * kD];
  __bf16 p[kWaves][kQW * kBc];  // per-wave weights, used only by the select path
};

// LDS tiles hold 64 rows of 64 bf16 (128 B = eight 16-byte chunks).  Chunk c of
// row r is stored at chunk c ^ swz(r): eight consecutive rows then put a given
// chunk in eight different bank groups (the 16-byte K reads of 8 lanes), and
// four consecutive rows put a 32-byte pair of chunks in four different 32-byte
// bank ranges (the 8-byte transposing V reads of 16 lanes).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 1) | ((row >> 2) & 1); }
__device__ __forceinline__ int lds_at(int row, int col) {  // element offset of (row, col)
  return row * kD + ((((col >> 3) ^ swz(row))) << 3) + (col & 7);
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t p = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ float sum_bf16_pair(uint32_t p, float acc) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p), one, acc, false);
}

__device__ __forceinline__ bool all_finite_bf16x8(uint4 w) {
  // a bf16 value is non-finite when its 8 exponent bits are all ones
  const uint32_t e0 = w.x & 0x7f807f80u, e1 = w.y & 0x7f807f80u;
  const uint32_t e2 = w.z & 0x7f807f80u, e3 = w.w & 0x7f807f80u;
  auto bad = [](uint32_t e) { return (int)((e & 0xffffu) == 0x7f80u) | (int)((e >> 16) == 0x7f80u); };
  return (bad(e0) | bad(e1) | bad(e2) | bad(e3)) == 0;
}

// Map a linear workgroup id to (head, query block), longest block first within
// each head and the heads of one XCD grouped: workgroup b runs on XCD b % 8, so
// XCD x takes heads x, x + 8, ... in turn and their K/V stay in its L2.
__device__ __forceinline__ bool map_block(int b, int heads, int nqb, int& head, int& qb) {
  const int xcd = b & 7, slot = b >> 3;
  const int hx = (heads - xcd + 7) >> 3;  // heads with head % 8 == xcd
  if (slot >= hx * nqb) return false;
  head = xcd + 8 * (slot / nqb);
  qb = nqb - 1 - slot % nqb;
  return true;
}

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int heads, int N, int nqb, float c_scale) {
  __shared__ Smem sm;
  int head, qb;
  if (!map_block(blockIdx.x, heads, nqb, head, qb)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const int q0 = qb * kBr;
  const int qw = q0 + wave * kQW;                       // first query of this wave
  const int wq_last = min(qw + kQW, N) - 1;             // last valid query of the wave
  const int kend = min(N, q0 + kBr);                    // keys the workgroup needs
  const int ntiles = (kend + kBc - 1) / kBc;

  // Q operand: lane holds q[qw + 32*qt + i32][16*kk + 8*h .. +7]
  bf16x8_t qop[2][4];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = qw + 32 * qt + i32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (qi < N) w = *(const uint4*)(q + base + (size_t)qi * kD + 16 * kk + 8 * h);
      qop[qt][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  floatx16 oacc[2][2];  // [dt][qt]: O^T tile, lane holds query column
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) oacc[a][b] = floatx16{};
  float mref[2] = {-__builtin_inff(), -__builtin_inff()};
  float lsum[2] = {0.f, 0.f};

  // global -> register staging: each thread moves 2 x 16 B of K and of V per tile
  uint4 kreg[2], vreg[2];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * kThreads;          // 16-byte chunk index in the tile
      const int row = e >> 3, col = (e & 7) * 8;
      const int j = t * kBc + row;
      if (j < N) {
        kreg[u] = *(const uint4*)(k + base + (size_t)j * kD + col);
        vreg[u] = *(const uint4*)(v + base + (size_t)j * kD + col);
      } else {
        kreg[u] = make_uint4(0, 0, 0, 0);
        vreg[u] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  // returns whether the staged V chunks are all finite
  auto store_tile = [&](int buf) {
    bool fin = true;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + u * kThreads;
      const int off = lds_at(e >> 3, (e & 7) * 8);
      *(uint4*)(&sm.k[buf][off]) = kreg[u];
      *(uint4*)(&sm.v[buf][off]) = vreg[u];
      fin &= all_finite_bf16x8(vreg[u]);
    }
    return fin;
  };

  load_tile(0);
  // the barrier also ORs "this V tile holds a non-finite value" over the workgroup
  int vnonfinite = __syncthreads_or(!store_tile(0));

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(t + 1);
    const int k0 = t * kBc;
    if (k0 <= wq_last) {
      const __bf16* ks = sm.k[buf];
      const __bf16* vs = sm.v[buf];
      // ---- S^T = K Q^T : s[kt][qt] holds keys k0 + 32 kt + 8(r/4) + 4h + r%4, query column
      floatx16 s[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        bf16x8_t kop[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          kop[kk] = *(const bf16x8_t*)(ks + lds_at(32 * kt + i32, 16 * kk + 8 * h));
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          floatx16 acc = floatx16{};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qop[qt][kk], acc, 0, 0, 0);
          s[kt][qt] = acc;
        }
      }
      // ---- mask: the diagonal tile (keys beyond the wave's first query) and keys >= N
      const bool masked = (k0 + kBc - 1 > qw) || (k0 + kBc > N);
      if (masked) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const int qi = qw + 32 * qt + i32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int j = k0 + 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
              if (j > qi || j >= N) s[kt][qt][r] = -__builtin_inff();
            }
          }
      }
      // ---- weights against the reference max; P packed to bf16 (B operand layout)
      uint32_t p[2][2][8];  // [qt][kt][pair]
      float part[2];
      bool redo = false;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float nm = -mref[qt];
        float acc = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int pr = 0; pr < 8; ++pr) {
            const float a = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][2 * pr], c_scale, nm));
            const float b = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][2 * pr + 1], c_scale, nm));
            p[qt][kt][pr] = pack_bf16(a, b);
            acc = sum_bf16_pair(p[qt][kt][pr], acc);
          }
        part[qt] = acc;
        redo |= !(acc <= kTau);
      }
      if (__any(redo)) {
        // exact path: raise the reference to the tile max, rescale, recompute
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          float mx = -__builtin_inff();
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][qt][r]);
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mnew = fmaxf(mref[qt], mx * c_scale);
          const float alpha = __builtin_amdgcn_exp2f(mref[qt] - mnew);  // 0 when mref = -inf
          if (mnew != mref[qt]) {
            lsum[qt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[dt][qt][r] *= alpha;
            mref[qt] = mnew;
          }
          const float nm = -mref[qt];
          float acc = 0.f;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int pr = 0; pr < 8; ++pr) {
              const float a = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][2 * pr], c_scale, nm));
              const float b = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][2 * pr + 1], c_scale, nm));
              p[qt][kt][pr] = pack_bf16(a, b);
              acc = sum_bf16_pair(p[qt][kt][pr], acc);
            }
          part[qt] = acc;
        }
      }
      lsum[0] += part[0];
      lsum[1] += part[1];

      if (!(masked && vnonfinite)) {
        // ---- O^T += V^T P^T over 4 chunks of 16 keys
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int kt = c >> 1, half = c & 1;
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            // ds_read_b64_tr_b16: the 16 lanes of group g read a 4 (keys) x 16 (features)
            // block; lane c16 of the group receives feature column c16, keys row0..row0+3.
            const int g16 = lane >> 4, c16 = lane & 15;
            const int col = 32 * dt + 16 * (g16 & 1) + 4 * (c16 & 3);
            const int row = 16 * c + 4 * (g16 >> 1) + (c16 >> 2);
            const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s*)(vs + lds_at(row, col)));
            const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_v4s*)(vs + lds_at(row + 8, col)));
            const bf16x8_t vop = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
              const uint4 pw = make_uint4(p[qt][kt][4 * half + 0], p[qt][kt][4 * half + 1],
                                          p[qt][kt][4 * half + 2], p[qt][kt][4 * half + 3]);
              oacc[dt][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  vop, __builtin_bit_cast(bf16x8_t, pw), oacc[dt][qt], 0, 0, 0);
            }
          }
        }
      } else {
        // ---- select path: a masked pair never multiplies (V holds inf/NaN).
        // The wave's bf16 weights go to its own LDS area as [query][key], so
        // every lane can read the weight of any key with a plain address.
        __bf16* pw = sm.p[wave];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int pr = 0; pr < 8; ++pr) {
              const int r = 2 * pr;  // keys r, r+1 of the accumulator: consecutive
              const int jj = 32 * kt + 8 * (r >> 2) + 4 * h + (r & 3);
              *(uint32_t*)(pw + (32 * qt + i32) * kBc + jj) = p[qt][kt][pr];
            }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const int qi = qw + 32 * qt + i32;
          for (int jj = 0; jj < kBc; ++jj) {
            const int j = k0 + jj;
            const float pj = (float)pw[(32 * qt + i32) * kBc + jj];
            if (j > qi || j >= N) continue;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
              for (int r2 = 0; r2 < 16; ++r2) {
                const int d = 32 * dt + 8 * (r2 >> 2) + 4 * h + (r2 & 3);
                oacc[dt][qt][r2] += pj * (float)vs[lds_at(jj, d)];
              }
          }
        }
      }
    }
    const bool fin = more ? store_tile(buf ^ 1) : true;
    vnonfinite = __syncthreads_or(!fin);
  }

  // ---- epilogue: l over both lane halves, O = O^T / l, lse = (m + log2 l) ln 2
#pragma unroll
  for (int qt = 0; qt < 2; ++qt) {
    const int qi = qw + 32 * qt + i32;
    const float l = lsum[qt] + __shfl_xor(lsum[qt], 32);
    const float inv = 1.0f / l;
    if (qi < N) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * h;
          uint2 w;
          w.x = pack_bf16(oacc[dt][qt][4 * g + 0] * inv, oacc[dt][qt][4 * g + 1] * inv);
          w.y = pack_bf16(oacc[dt][qt][4 * g + 2] * inv, oacc[dt][qt][4 * g + 3] * inv);
          *(uint2*)(o + base + (size_t)qi * kD + d) = w;
        }
      if (h == 0) lse[(size_t)head * N + qi] = (mref[qt] + __log2f(l)) * kLn2;
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o,
                           float* lse, int64_t heads, int64_t N, double scale, hipStream_t stream,
                           const Timers& tm) {
  const int nqb = (int)((N + kBr - 1) / kBr);
  const int per_xcd = (int)((heads + 7) / 8) * nqb;
  const unsigned grid = (unsigned)(8 * per_xcd);
  const float c = (float)(scale * 1.4426950408889634);  // scale * log2(e)
  if (hipError_t e = mark(tm.start[kTimerFwd], stream)) return e;
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse,
                     (int)heads, (int)N, nqb, c);
  if (hipError_t e = mark(tm.stop[kTimerFwd], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
