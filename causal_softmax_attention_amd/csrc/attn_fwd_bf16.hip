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
// Layout of the work (one workgroup = 4 waves = 128 queries of one head):
//   * Each wave owns 32 queries (one 32-query MFMA column).  Q stays in
//     registers as the B operand of S^T = K Q^T (v_mfma_f32_32x32x16_bf16), so
//     every lane holds one query column of the score tile: the softmax state
//     (reference max m, running sum l) is per lane, no row reduction crosses
//     lanes except the final l_lane + l_(lane^32).
//   * Three workgroups share a CU: three waves per SIMD, each within 168
//     VGPRs, so while one wave waits on its score MFMAs another forms weights.
//     (Two waves of 64 queries each ran about 10 % slower: at 256 VGPRs the
//     compiler cannot hoist the V reads, and a third of the latency hiding is
//     lost.)
//   * Keys stream in tiles of 64 through a 3-stage LDS ring, filled by
//     asynchronous bounds-checked buffer loads two tiles ahead (one barrier per
//     tile; one tile ahead in the plain causal kernel, which runs each plain
//     tile's P V in the next tile's step and keeps that V in the third stage).
//     K rows feed the A operand with plain 16-byte reads; V rows are
//     read with ds_read_b64_tr_b16, which hands each lane 4 consecutive keys of
//     one feature column: exactly the A operand of O^T = V^T P^T.  The
//     bf16-rounded P accumulator registers are the B operand as they stand.
//   * Causal block skipping: a wave stops at the tile holding its last query;
//     only the diagonal tile and the ragged tail (keys >= N) are masked, by
//     setting those scores to -inf (an absent pair gets weight exactly 0).
//
// Lazy max: any offset common to a row's scores drops out of w / z, so the
// subtracted value need not be the exact maximum; it only has to keep the
// exponentials in float32 range (the demo script makes the same point beside
// its window spelling).  Weights are therefore
// taken as exp2(s*c - m_ref) against a reference m_ref, and a tile is redone
// with its exact max (rescaling the accumulators) only when some weight would
// exceed 2^8 - detected from the lane's tile sum, so the common path spends no
// instruction on a max.  m_ref starts at -inf, so the first tile always takes
// the exact path.  Products p * v are then bounded by 2^8 |v|.
//
// Absent rows with non-finite V: a masked pair must contribute nothing, but
// the MFMA would form 0 * inf = NaN.  On a masked tile each wave scans the V
// tile; if it holds any inf/NaN, that tile's P V is formed by a select-based
// VALU path that skips masked pairs.
#include "common.h"
#include "launch.h"
#include "mfma_bf16.h"

namespace attn {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = 1;                  // 32-query MFMA columns per wave (168 VGPRs hold one)
constexpr int kQW = 32 * kQT;           // queries per wave
constexpr int kBr = kQW * kWaves;       // queries per workgroup
constexpr int kBc = 64;                 // keys per tile
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kTau = 256.0f;          // lazy-max bound on a lane's tile sum (2^8)
constexpr float kRefInit = -1e30f;      // initial reference exponent (see the kernel)

// A pair (query i, key j) is absent when j >= N, or j > i under the causal
// predicate, or i - j >= band under a window of band keys.
__device__ __forceinline__ bool absent(int i, int j, int N, int causal, int band) {
  return j >= N || (causal && j > i) || (band && i - j >= band);
}

struct KVStage {
  __bf16 k[kBc * kD];
  __bf16 v[kBc * kD];
};

// Running maximum, per 16-bit half, of the magnitude bits (sign cleared) of
// bf16 pairs: a bf16 value is non-finite exactly when its magnitude bits reach
// 0x7f80 (all exponent bits set), so one compare of the maximum at the end
// tests every value (two instructions per word: an and, a packed max).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u16x2_t max_mag_bf16x8(u16x2_t acc, uint4 w) {
  acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2_t, w.x & 0x7fff7fffu));
  acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2_t, w.y & 0x7fff7fffu));
  acc = __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2_t, w.z & 0x7fff7fffu));
  return __builtin_elementwise_max(acc, __builtin_bit_cast(u16x2_t, w.w & 0x7fff7fffu));
}

// Weights of one 64-key tile against the lane's reference max, packed to
// bf16 pairs in B-operand order; returns the lane's sums of the float32
// weights per query column.  The sums use plain adds: a dot2 instruction
// (bf16 pair times ones) does not issue while the matrix pipe is busy, so it
// would hold this wave and the SIMD's other waves behind their MFMAs.
__device__ __forceinline__ void tile_weights(const floatx16 (&s)[2][kQT], float c_scale,
                                             const float (&mref)[kQT], uint32_t (&p)[kQT][2][8],
                                             float (&part)[kQT]) {
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const float nm = -mref[qt];
    float acc = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int pr = 0; pr < 8; ++pr) {
        const float a = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][2 * pr], c_scale, nm));
        const float b = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][2 * pr + 1], c_scale, nm));
        p[qt][kt][pr] = pack_bf16(a, b);
        acc += a + b;
      }
    part[qt] = acc;
  }
}

// One key tile for one wave (32 queries x 64 keys).  MASKED: the tile crosses
// the wave's diagonal or the end of the sequence.
// SEG: segment ids apply; segk holds the tile's 64 key ids (LDS) and sq the
// lane's query id, and a pair of different ids is absent.
template <bool MASKED, bool SEG>
__device__ __forceinline__ void fwd_tile(const __bf16* ks, const __bf16* vs, __bf16* pscr,
                                         int lane, int k0, int qw, int N, float c_scale,
                                         int causal, int band, const bf16x8_t (&qop)[kQT][4],
                                         floatx16 (&oacc)[2][kQT], float (&mref)[kQT],
                                         float (&lsum)[kQT], const int32_t* segk, int32_t sq) {
  const int i32 = lane & 31, h = lane >> 5;
  // ---- S^T = K Q^T: s[kt][qt] holds keys k0 + 32 kt + acc_row(r, h), query column
  floatx16 s[2][kQT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    bf16x8_t kop[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kop[kk] = read_row8(ks, 32 * kt + i32, 16 * kk + 8 * h);
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      floatx16 acc = floatx16{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) acc = mma(kop[kk], qop[qt][kk], acc);
      s[kt][qt] = acc;
    }
  }
  if (MASKED) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int qt = 0; qt < kQT; ++qt) {
        const int qi = qw + 32 * qt + i32;
        int32_t sk[16];  // ids of the lane's 16 keys of this half (rows acc_row(r, h))
        if (SEG) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int4 w = *(const int4*)(segk + 32 * kt + 8 * g + 4 * h);
            sk[4 * g + 0] = w.x; sk[4 * g + 1] = w.y; sk[4 * g + 2] = w.z; sk[4 * g + 3] = w.w;
          }
        }
        // register r holds key j = jb + acc_row(r, 0), so the predicate of
        // absent() becomes a range of that constant offset: lo < off < hi
        const int jb = k0 + 32 * kt + 4 * h;
        const int hi = causal ? min(N, qi + 1) - jb : N - jb;
        const int lo = band ? qi - band - jb : INT32_MIN;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = acc_row(r, 0);
          const bool gone = !(off < hi && off > lo) || (SEG && sk[r] != sq);
          s[kt][qt][r] = gone ? -__builtin_inff() : s[kt][qt][r];
        }
      }
  }
  // ---- weights against the reference max, exact max only when needed
  uint32_t p[kQT][2][8];
  float part[kQT];
  tile_weights(s, c_scale, mref, p, part);
  bool over = false;
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) over |= !(part[qt] <= kTau);
  if (__any(over)) {
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][qt][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mref[qt], mx * c_scale);
      if (mnew != mref[qt]) {
        const float alpha = __builtin_amdgcn_exp2f(mref[qt] - mnew);  // 0 from kRefInit
        lsum[qt] *= alpha;
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][qt][r] *= alpha;
        mref[qt] = mnew;
      }
    }
    tile_weights(s, c_scale, mref, p, part);
  }
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) lsum[qt] += part[qt];

  bool vbad = false;
  if (MASKED) {
    // lane l scans row l of the V tile for inf / NaN
    u16x2_t mag = {0, 0};
#pragma unroll
    for (int c = 0; c < 8; ++c) mag = max_mag_bf16x8(mag, *(const uint4*)(vs + lane * kD + 8 * c));
    vbad = __any(mag.x >= 0x7f80u || mag.y >= 0x7f80u);
  }
  if (!vbad) {
    // ---- O^T += V^T P^T over 4 chunks of 16 keys
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x8_t vop = read_tr(vs, lane, c, 32 * dt);
#pragma unroll
        for (int qt = 0; qt < kQT; ++qt)
          oacc[dt][qt] = mma(vop, chunk_op(p[qt][c >> 1], c & 1), oacc[dt][qt]);
      }
  } else {
    // ---- select path: a masked pair never multiplies (V holds inf/NaN).  The
    // weights of one 32-query column and 8 keys go to the wave's LDS area as
    // [query][key].
#pragma unroll
    for (int qt = 0; qt < kQT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int c8 = 0; c8 < 4; ++c8) {
#pragma unroll
          for (int pr = 2 * c8; pr < 2 * c8 + 2; ++pr) {
            const int jj = acc_row(2 * pr, h) - 8 * c8;  // keys 32 kt + 8 c8 + jj, + 1
            *(uint32_t*)(pscr + i32 * 8 + jj) = p[qt][kt][pr];
          }
          __builtin_amdgcn_wave_barrier();
          const int qi = qw + 32 * qt + i32;
#pragma unroll 1
          for (int jj = 0; jj < 8; ++jj) {
            const int j = k0 + 32 * kt + 8 * c8 + jj;
            const float pj = (float)pscr[i32 * 8 + jj];
            if (absent(qi, j, N, causal, band) || (SEG && segk[j - k0] != sq)) continue;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt)
#pragma unroll
              for (int r2 = 0; r2 < 16; ++r2)
                oacc[dt][qt][r2] +=
                    pj * (float)vs[lds_at(32 * kt + 8 * c8 + jj, 32 * dt + acc_row(r2, h))];
          }
          __builtin_amdgcn_wave_barrier();
        }
  }
}

// O^T += V^T P^T of one tile from its packed weights.
__device__ __forceinline__ void pv_mfma(const __bf16* vs, int lane, const uint32_t (&p)[2][8],
                                        floatx16 (&oacc)[2][kQT]) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      oacc[dt][0] = mma(read_tr(vs, lane, c, 32 * dt), chunk_op(p[c >> 1], c & 1), oacc[dt][0]);
}

// A tile with no absent pair whose own P V is left to the next tile: its
// score MFMAs, then the previous tile's P V (PEND) beside its weights.
template <bool PEND>
__device__ __forceinline__ void fwd_tile_defer(const __bf16* ks, const __bf16* vprev, int lane,
                                               float c_scale, const bf16x8_t (&qop)[kQT][4],
                                               floatx16 (&oacc)[2][kQT], float (&mref)[kQT],
                                               float (&lsum)[kQT], uint32_t (&pprev)[2][8]) {
  const int i32 = lane & 31, h = lane >> 5;
  floatx16 s[2][kQT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    bf16x8_t kop[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kop[kk] = read_row8(ks, 32 * kt + i32, 16 * kk + 8 * h);
    floatx16 acc = floatx16{};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) acc = mma(kop[kk], qop[0][kk], acc);
    s[kt][0] = acc;
  }
  if (PEND) pv_mfma(vprev, lane, pprev, oacc);
  uint32_t p[kQT][2][8];
  float part[kQT];
  // with nothing pending this is the wave's first tile (its plain tiles come
  // before every masked one), whose reference is still kRefInit: it takes the
  // exact max at once instead of after a lazy attempt that must overflow
  if (PEND) tile_weights(s, c_scale, mref, p, part);
  if (!PEND || __any(!(part[0] <= kTau))) {
    float mx = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][0][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mref[0], mx * c_scale);
    if (mnew != mref[0]) {
      const float alpha = __builtin_amdgcn_exp2f(mref[0] - mnew);
      lsum[0] *= alpha;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][0][r] *= alpha;
      mref[0] = mnew;
    }
    tile_weights(s, c_scale, mref, p, part);
  }
  lsum[0] += part[0];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int i = 0; i < 8; ++i) pprev[kt][i] = p[0][kt][i];
}

// CAUSAL: the causal predicate applies; BANDED: a window of band_arg keys does;
// SEG: only pairs of equal segment ids (seg, [B][N], batch = head / hpb) exist.
template <bool CAUSAL, bool BANDED, bool SEG>
__global__ __launch_bounds__(kThreads, 3) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    __bf16* __restrict__ o, float* __restrict__ lse, int heads, int N, int nqb, float c_scale,
    int band_arg, float* __restrict__ ndelta, float* __restrict__ nlse, float inv_scale,
    const int32_t* __restrict__ seg, int hpb) {
  constexpr int causal = CAUSAL;
  const int band = BANDED ? band_arg : 0;
  // one array, so the three stages' LDS addresses differ by immediate offsets
  // and share their per-lane address registers (separate objects took one
  // set per stage: 16 more VGPRs, and spills in the masked variants)
  __shared__ KVStage stg[3];
  KVStage &st0 = stg[0], &st1 = stg[1], &st2 = stg[2];
  // the select path's weights (32 queries x 8 keys a wave): at 32 x 16 the
  // segment variant's LDS (with its key ids) kept only 2 workgroups on a CU
  __shared__ __bf16 pscr[kWaves][32 * 8];
  __shared__ __attribute__((aligned(16))) int32_t sg[3][SEG ? kBc : 4];  // the stages' key ids
  static_assert(kQT == 1, "one query column per wave");
  int head, qb;
  // groups of 4 heads: an XCD holds 96 of these workgroups at once (32 CUs x
  // 3), a little under one group, whose K/V (4 x 1 MiB at N = 4096) about
  // fills its 4 MiB L2.  Measured at that size: groups of 8 read 2.6 times the
  // forward's Q, K and V bytes from beyond L2, groups of 4 1.5 times and groups
  // of 3 1.26 times; timed in alternating rounds, groups of 4 and 8 ran 3 %
  // faster than groups of 3, whose last group's heaviest blocks start late and
  // leave the launch a tail.
  if (!map_block(blockIdx.x, heads, nqb, true, 4, head, qb, true)) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const int qw = qb * kBr + wave * kQW;              // first query of this wave
  const int wq_last = min(qw + kQW, N) - 1;          // last valid query of the wave
  // keys the workgroup needs: tiles t0 .. ntiles-1
  int t0 = band ? max(0, qb * kBr - band + 1) / kBc : 0;
  const int kend = causal ? min(N, qb * kBr + kBr) : N;
  int ntiles = (kend + kBc - 1) / kBc;
  const int wlo = band ? qw - band + 1 : 0, whi = causal ? wq_last : N - 1;  // keys of this wave

  // Q operand: lane holds q[qw + 32 qt + i32][16 kk + 8 h .. +7]
  bf16x8_t qop[kQT][4];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qw + 32 * qt + i32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (qi < N) w = ldg16(q + base + (size_t)qi * kD + 16 * kk + 8 * h);
      qop[qt][kk] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  floatx16 oacc[2][kQT];  // [dt][qt]: O^T tile, lane holds query column
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < kQT; ++b) oacc[a][b] = floatx16{};
  // segment ids: the lane's query id, and the range of the wave's valid ids
  // (a tile none of whose key ids falls in it has no pair for this wave)
  const int32_t* segrow = SEG ? seg + (size_t)(head / hpb) * N : nullptr;
  int32_t sq = 0, sqlo = 0, sqhi = 0;
  if (SEG) {
    const int qi = qw + i32;
    sq = qi < N ? segrow[qi] : 0;
    sqlo = qi < N ? sq : INT32_MAX;
    sqhi = qi < N ? sq : INT32_MIN;
#pragma unroll
    for (int o2 = 16; o2 >= 1; o2 >>= 1) {
      sqlo = min(sqlo, __shfl_xor(sqlo, o2));
      sqhi = max(sqhi, __shfl_xor(sqhi, o2));
    }
    sqlo = __builtin_amdgcn_readfirstlane(sqlo);
    sqhi = __builtin_amdgcn_readfirstlane(sqhi);
    // only the key tiles within the span of keys whose ids fall in the
    // block's query-id range (never empty: each query is also a key)
    __shared__ int32_t red[2][kWaves][4];
    const SegSpan sp = seg_span<kThreads>(segrow, N, qb * kBr, kBr, t0 * kBc, kend, tid, red);
    t0 = __builtin_amdgcn_readfirstlane(sp.first / kBc);
    ntiles = __builtin_amdgcn_readfirstlane((sp.last + kBc - 1) / kBc);
  }
  // reference exponents start finite, so a tile whose pairs are all absent for
  // a lane gives it weights exp2(-inf) = 0, and its first present pair takes the
  // exact path (the weight overflows against kRefInit)
  float mref[kQT], lsum[kQT];
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    mref[qt] = kRefInit;
    lsum[qt] = 0.f;
  }

  const uint32_t tbytes = (uint32_t)N * kD * 2;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(k + base, tbytes), rv = head_rsrc(v + base, tbytes);
  __amdgpu_buffer_rsrc_t rs = rk;
  if (SEG) rs = head_rsrc(segrow, (uint32_t)N * 4);
  // wave 0 also copies the tile's key ids (one 4-byte load per lane); with its
  // one extra load per tile, the barrier waits below (at most the newest
  // tile's 4 loads in flight) still cover every older tile
  auto issue = [&](KVStage& s, int32_t* sgs, int t) {
    tile_async<kBc, kWaves>(rk, s.k, t * kBc, wave, lane);
    tile_async<kBc, kWaves>(rv, s.v, t * kBc, wave, lane);
    if (SEG && wave == 0) rows_async(rs, (float*)sgs, t * kBc, lane);
  };
  // The plain causal kernel runs a plain tile's P V in the next tile's step,
  // right after that tile's score MFMAs and beside its weights (1.5-2 % on
  // the 4096-token forward, same arithmetic in the same order).  The previous
  // tile's V then stays in its ring stage, so loads run one tile ahead.  With a
  // window or segment ids, whose walks are short or mostly masked, it lost.
  constexpr bool DEFER = CAUSAL && !BANDED && !SEG;
  if constexpr (!DEFER) {
    auto step = [&](KVStage& cur, int32_t* sgc, KVStage& ahead, int32_t* sga, int t) {
      const bool pre = t + 2 < ntiles;
      if (pre) issue(ahead, sga, t + 2);
      const int k0 = t * kBc;
      if (k0 <= whi && k0 + kBc - 1 >= wlo) {
        // segments: no key id in the wave's id range -> no pair; all ids one and
        // the same -> the ids mask nothing (keys past N are masked anyway)
        bool seg_some = true, seg_one = true;
        if (SEG) {
          const int32_t skey = sgc[lane];  // key k0 + lane
          const bool kin = k0 + lane < N;
          seg_some = __any(kin && skey >= sqlo && skey <= sqhi);
          seg_one = sqlo == sqhi && __all(!kin || skey == sqlo);
        }
        if (seg_some) {
          // masked: some pair of the tile is absent for some query of the wave
          if ((causal && k0 + kBc - 1 > qw) || (k0 + kBc > N) || (band && k0 < qw + kQW - band) ||
              !seg_one)
            fwd_tile<true, SEG>(cur.k, cur.v, pscr[wave], lane, k0, qw, N, c_scale, causal, band,
                                qop, oacc, mref, lsum, sgc, sq);
          else
            fwd_tile<false, SEG>(cur.k, cur.v, pscr[wave], lane, k0, qw, N, c_scale, causal, band,
                                 qop, oacc, mref, lsum, sgc, sq);
        }
      }
      if (pre) wait_vm_barrier<2 * kBc / (8 * kWaves)>();
      else wait_vm_barrier<0>();
    };

    issue(st0, sg[0], t0);
    if (t0 + 1 < ntiles) issue(st1, sg[1], t0 + 1);
    wait_vm_barrier<0>();
    for (int t = t0; t < ntiles; t += 3) {
      step(st0, sg[0], st2, sg[2], t);
      if (t + 1 < ntiles) step(st1, sg[1], st0, sg[0], t + 1);
      if (t + 2 < ntiles) step(st2, sg[2], st1, sg[1], t + 2);
    }

  } else {
    uint32_t pprev[2][8];  // weights of the tile whose P V is pending
    bool pend = false;
    auto step = [&](KVStage& cur, KVStage& ahead, int32_t* sga, KVStage& prv, int t) {
      if (t + 1 < ntiles) issue(ahead, sga, t + 1);
      const int k0 = t * kBc;
      const bool work = k0 <= whi;
      const bool masked = k0 + kBc - 1 > qw || k0 + kBc > N;
      if (work && !masked) {
        if (pend)
          fwd_tile_defer<true>(cur.k, prv.v, lane, c_scale, qop, oacc, mref, lsum, pprev);
        else
          fwd_tile_defer<false>(cur.k, prv.v, lane, c_scale, qop, oacc, mref, lsum, pprev);
        pend = true;
      } else {
        // masked or skipped: settle the pending P V first (its stage is
        // reloaded in the next step)
        if (pend) pv_mfma(prv.v, lane, pprev, oacc);
        pend = false;
        if (work)
          fwd_tile<true, false>(cur.k, cur.v, pscr[wave], lane, k0, qw, N, c_scale, causal, band,
                                qop, oacc, mref, lsum, nullptr, 0);
      }
      wait_vm_barrier<0>();  // tile t + 1 has landed; every wave is done with tile t - 1
    };

    issue(st0, sg[0], t0);
    wait_vm_barrier<0>();
    for (int t = t0; t < ntiles; t += 3) {
      step(st0, st1, sg[1], st2, t);
      if (t + 1 < ntiles) step(st1, st2, sg[2], st0, t + 1);
      if (t + 2 < ntiles) step(st2, st0, sg[0], st1, t + 2);
    }
    if (pend) pv_mfma(stg[(ntiles - 1 - t0) % 3].v, lane, pprev, oacc);
  }

  // ---- epilogue: l over both lane halves, O = O^T / l, lse = (m + log2 l) ln 2.
  // With ndelta given (the loss sum(o^2)/2, so dO = O), also the backward's
  // per-row values from the stored bf16 row: -delta_i = -|o_i|^2 and -lse_i / scale.
#pragma unroll
  for (int qt = 0; qt < kQT; ++qt) {
    const int qi = qw + 32 * qt + i32;
    const float l = lsum[qt] + __shfl_xor(lsum[qt], 32);
    const float inv = 1.0f / l;
    if (qi < N) {
      float sq = 0.f;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d = 32 * dt + 8 * g + 4 * h;
          uint2 w;
          w.x = pack_bf16(oacc[dt][qt][4 * g + 0] * inv, oacc[dt][qt][4 * g + 1] * inv);
          w.y = pack_bf16(oacc[dt][qt][4 * g + 2] * inv, oacc[dt][qt][4 * g + 3] * inv);
          *(uint2*)(o + base + (size_t)qi * kD + d) = w;
          if (ndelta) {
            const float x0 = __uint_as_float(w.x << 16), x1 = __uint_as_float(w.x & 0xffff0000u);
            const float x2 = __uint_as_float(w.y << 16), x3 = __uint_as_float(w.y & 0xffff0000u);
            sq = fmaf(x0, x0, fmaf(x1, x1, fmaf(x2, x2, fmaf(x3, x3, sq))));
          }
        }
      const float lse_i = (mref[qt] + __log2f(l)) * kLn2;
      if (h == 0) lse[(size_t)head * N + qi] = lse_i;
      if (ndelta) {
        sq += __shfl_xor(sq, 32);  // the partner lane holds the row's other 32 features
        if (h == 0) {
          ndelta[(size_t)head * N + qi] = -sq;
          nlse[(size_t)head * N + qi] = -lse_i * inv_scale;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, __bf16* o,
                           float* lse, int64_t heads, int64_t N, double scale, const Mask& mk,
                           void* bwd_ws, hipStream_t stream, const Timers& tm) {
  const int nqb = (int)((N + kBr - 1) / kBr);
  const unsigned grid = (unsigned)(8 * ((heads + 7) / 8) * nqb);
  const float c = (float)(scale * 1.4426950408889634);  // scale * log2(e)
  auto kern = mk.seg ? (mk.band > 0 ? attn_fwd_bf16_kernel<true, true, true>
                        : mk.causal ? attn_fwd_bf16_kernel<true, false, true>
                                    : attn_fwd_bf16_kernel<false, false, true>)
                     : (mk.band > 0 ? attn_fwd_bf16_kernel<true, true, false>
                        : mk.causal ? attn_fwd_bf16_kernel<true, false, false>
                                    : attn_fwd_bf16_kernel<false, false, false>);
  if (hipError_t e = mark(tm.start[kTimerFwd], stream)) return e;
  // the backward workspace: -delta per row, then -lse / scale per row
  float* ndelta = (float*)bwd_ws;
  float* nlse = ndelta ? ndelta + heads * N : nullptr;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, q, k, v, o, lse, (int)heads,
                     (int)N, nqb, c, mk.band, ndelta, nlse, (float)(1.0 / scale), mk.seg,
                     mk.hpb);
  if (hipError_t e = mark(tm.stop[kTimerFwd], stream)) return e;
  return hipGetLastError();
}

}  // namespace attn
