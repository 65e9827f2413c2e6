// Causal attention backward for bfloat16 on gfx950 MFMA (float32 accumulation).
//
// Gradient of a loss with upstream gradient dO (pages: "Show HN: automatic
// deduction of FlashAttention kernel from 25 lines of SQL", the GRADIENT
// statement: grad(loss, q.x), grad(loss, k.x), grad(loss, v.x) of
// loss = SUM(x * x) / 2, so dO = O there).  With P_ij = exp(s_ij - lse_i) over
// the pairs j <= i, s_ij = scale q_i . k_j:
//   delta_i = sum_d dO_id O_id            (= sum_j P_ij dP_ij)
//   dP_ij   = dO_i . v_j,   dS_ij = P_ij (dP_ij - delta_i)
//   dV_j = sum_{i>=j} P_ij dO_i,  dK_j = scale sum_{i>=j} dS_ij q_i,
//   dQ_i = scale sum_{j<=i} dS_ij k_j.
// Scores are recomputed from q, k and the forward's saved lse; nothing N x N is
// stored.
//
// Three launches, no atomics (float atomics in L2 run at about one 4-byte add
// per channel-clock on this part, far too slow for a dQ accumulated across key
// blocks):
//   1. prep: -delta_i and -lse_i / scale per row (one pass over O and dO),
//   2. dK/dV, key-stationary: a wave owns 32 keys whose K and V stay in
//      registers as MFMA B operands; 64-query stages (Q, dO, and the two
//      per-row values) stream through a 3-stage LDS ring filled by
//      asynchronous buffer loads.  S = Q K^T and dP = dO V^T are formed as
//      query x key accumulators, so after rounding to bf16 they are the B
//      operands of dV^T = dO^T P and dK^T = Q^T dS, whose A operands come from
//      transposing LDS reads of the same Q / dO rows.
//   3. dQ, query-stationary: a wave owns 32 queries (Q, dO in registers, its
//      two per-row values per lane); key tiles (K, V) stream through LDS.  S^T
//      and dP^T are key x query accumulators, so dS^T is the B operand of
//      dQ^T = K^T dS^T.
// A workgroup is 4 waves (128 stationary rows) and two workgroups share a CU:
// two waves per SIMD, each within 256 VGPRs, from workgroups that do not share
// barriers.  Every accumulator then stays in the VGPRs that the exp / VALU work
// reads, with no AGPR copies, and each SIMD's two waves overlap one another's
// MFMA and VALU phases.  (With 64 rows per wave and one wave per SIMD the
// working set passed 256 VGPRs, and the compiler moved about two accumulator
// registers between AGPRs and VGPRs per MFMA.)
#include "common.h"
#include "launch.h"
#include "mfma_bf16.h"

#include <type_traits>

namespace attn {
namespace {

using namespace mfma;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kKT = 1;                   // 32-row MFMA columns of stationary rows per wave
constexpr int kRowsW = 32 * kKT;         // stationary rows per wave
constexpr int kBlk = kRowsW * kWaves;    // stationary rows per workgroup
constexpr int kT = 64;                   // streamed rows per tile
constexpr int kT2 = kT;                  // streamed rows per LDS stage

// Per row: -delta_i = -sum_d dO_id O_id and -lse_i / scale, the values the
// score accumulators of both passes start from (so that they end as
// dP_ij - delta_i and s_ij - lse_i / scale, see below).  Eight lanes per row,
// 16 bytes each.  ALIAS: dO is O (one pointer, as for the loss sum(o^2)/2), so
// each row is read once and delta_i = |o_i|^2 (the same products in the same
// order as the general form).
template <bool ALIAS>
__global__ __launch_bounds__(256) void bwd_prep_bf16(const __bf16* __restrict__ o,
                                                     const __bf16* __restrict__ dout,
                                                     const float* __restrict__ lse,
                                                     float* __restrict__ ndelta,
                                                     float* __restrict__ nlse, float inv_scale,
                                                     int64_t rows) {
  // 32 R rows per workgroup: each thread has R rows' loads in flight (the
  // same bytes either way)
  constexpr int R = ALIAS ? 8 : 4;
  const int part = threadIdx.x & 7;
  const int64_t r0 = (int64_t)blockIdx.x * (32 * R) + (threadIdx.x >> 3);
  uint4 a[R], b[R];
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t r = r0 + 32 * i;
    a[i] = b[i] = make_uint4(0, 0, 0, 0);
    if (r < rows) {
      a[i] = ldg16(o + r * kD + part * 8);
      if (!ALIAS) b[i] = ldg16(dout + r * kD + part * 8);
    }
  }
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int64_t r = r0 + 32 * i;
    const __bf16* x = (const __bf16*)&a[i];
    const __bf16* y = ALIAS ? x : (const __bf16*)&b[i];
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf((float)x[e], (float)y[e], s);
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    if (r < rows && part == 0) {
      ndelta[r] = -s;
      nlse[r] = -lse[r] * inv_scale;
    }
  }
}

// ---- dK / dV, key-stationary -------------------------------------------------
//
// A wave owns 32 keys (K, V rows in registers as MFMA B operands) and walks the
// queries in 32-query halves.  Per half n:
//   A(n): S' = Q K^T - lse/scale and dP' = dO V^T - delta (query rows x key
//         columns), the accumulators starting from -lse/scale and -delta of
//         their rows, so the offsets cost no instruction;
//   B(n): P = exp2(c S') with c = scale log2(e), dS = P dP' (VALU), rounded to
//         bf16 and packed;
//   C(n): dV^T += dO^T P and dK^T += Q^T dS (the packed tiles are B operands,
//         the transposed Q / dO rows come from ds_read_b64_tr_b16).
// The three depend on one another in that order, so each step issues A(n+1),
// B(n) and C(n-1) together: the MFMAs of A and C overlap the exp / VALU work of
// B with no result waited on inside a step.
//
// Queries stream through a 3-stage LDS ring of 64-row stages (Q, dO, and
// -lse/scale, -delta), filled by asynchronous buffer loads.  Stage s holds
// halves 2s and 2s+1.  Step 0 of stage s forms A(2s+1) from its own rows
// 32.. and C(2s-1) from the previous stage's rows 32..; step 1 forms A(2s+2)
// from the next stage's rows 0.. and C(2s) from its own rows 0...  So one
// barrier per stage, between the two steps, both publishes stage s+1 and
// frees the previous stage's buffer for stage s+2.  All four waves of a
// workgroup walk the same halves from the workgroup's first key; halves before
// a wave's diagonal are fully masked (weight 0), so they add nothing.
// SEG: the stage also holds its queries' segment ids.
template <bool SEG>
struct alignas(16) QStageT {
  __bf16 q[kT2 * kD];
  __bf16 dout[kT2 * kD];
  float nlse[kT2];
  float ndelta[kT2];
  int32_t seg[SEG ? kT2 : 4];
};

template <bool SEG>
struct DkdvPipe {
  floatx16 s[kKT], dp[kKT];          // A(n) results, consumed by B(n)
  uint32_t pp[kKT][8], dsp[kKT][8];  // B(n-1) results, consumed by C(n-1)
  int32_t qs[SEG ? 16 : 1];          // A(n)'s query ids (rows acc_row(r, h)), for B(n)
};

// A: S' and dP' of the 32 queries at rows row0.. of a stage (and, with
// segment ids, the ids of the lane's rows).
template <bool SEG>
__device__ __forceinline__ void dkdv_scores(const QStageT<SEG>& st, int row0, int lane,
                                            const bf16x8_t (&kop)[kKT][4],
                                            const bf16x8_t (&vop)[kKT][4], floatx16 (&s)[kKT],
                                            floatx16 (&dp)[kKT], int32_t* qs) {
  const int i32 = lane & 31, h = lane >> 5;
  bf16x8_t qa[4], oa[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    qa[kk] = read_row8(st.q, row0 + i32, 16 * kk + 8 * h);
    oa[kk] = read_row8(st.dout, row0 + i32, 16 * kk + 8 * h);
  }
  floatx16 ls, ds;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (SEG) {
      const int4 w = *(const int4*)(st.seg + row0 + 8 * g + 4 * h);
      qs[4 * g + 0] = w.x; qs[4 * g + 1] = w.y; qs[4 * g + 2] = w.z; qs[4 * g + 3] = w.w;
    }
    const float4 a = *(const float4*)(st.nlse + row0 + 8 * g + 4 * h);
    const float4 b = *(const float4*)(st.ndelta + row0 + 8 * g + 4 * h);
    ls[4 * g + 0] = a.x; ls[4 * g + 1] = a.y; ls[4 * g + 2] = a.z; ls[4 * g + 3] = a.w;
    ds[4 * g + 0] = b.x; ds[4 * g + 1] = b.y; ds[4 * g + 2] = b.z; ds[4 * g + 3] = b.w;
  }
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
    floatx16 a = ls, b = ds;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      a = mma(qa[kk], kop[kt][kk], a);
      b = mma(oa[kk], vop[kt][kk], b);
    }
    s[kt] = a;
    dp[kt] = b;
  }
}

// B: packed bf16 P and dS of one half.  MASKED: absent pairs (key > query
// under the causal predicate, query - key >= band under a window) get weight 0
// (a select).  Queries past the end need no mask: their Q and dO rows read as
// zeros, so their dS is 0 and their P multiplies a zero dO row.
template <bool MASKED, bool SEG>
__device__ __forceinline__ void dkdv_softmax(const floatx16 (&s)[kKT], const floatx16 (&dp)[kKT],
                                             uint32_t (&pp)[kKT][8], uint32_t (&dsp)[kKT][8],
                                             int qrow0, int kw, int lane, float c_scale,
                                             int causal, int band, const int32_t* qs,
                                             int32_t sk) {
  const int i32 = lane & 31, h = lane >> 5;
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
    const int key = kw + 32 * kt + i32;
    // register r holds query qb + acc_row(r, 0): the pair is present when that
    // offset is at least lo (causal: query >= key) and below hi (window:
    // query - key < band)
    const int qb = qrow0 + 4 * h;
    const int lo = causal ? key - qb : INT32_MIN;
    const int hi = band ? key + band - qb : INT32_MAX;
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      float pv[2], dsv[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * pr + e;
        float p = __builtin_amdgcn_exp2f(s[kt][r] * c_scale);
        if (MASKED) {
          const int off = acc_row(r, 0);
          p = !(off >= lo && off < hi) || (SEG && qs[r] != sk) ? 0.f : p;
        }
        pv[e] = p;
        dsv[e] = p * dp[kt][r];
      }
      pp[kt][pr] = pack_bf16(pv[0], pv[1]);
      dsp[kt][pr] = pack_bf16(dsv[0], dsv[1]);
    }
  }
}

// C: dV^T += dO^T P and dK^T += Q^T dS over the 32 queries at rows row0.. of a stage.
template <class ST>
__device__ __forceinline__ void dkdv_accum(const ST& st, int row0, int lane,
                                           const uint32_t (&pp)[kKT][8],
                                           const uint32_t (&dsp)[kKT][8],
                                           floatx16 (&dkacc)[2][kKT], floatx16 (&dvacc)[2][kKT]) {
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const bf16x8_t otr = read_tr(st.dout, lane, row0 / 16 + half, 32 * dt);
      const bf16x8_t qtr = read_tr(st.q, lane, row0 / 16 + half, 32 * dt);
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        dvacc[dt][kt] = mma(otr, chunk_op(pp[kt], half), dvacc[dt][kt]);
        dkacc[dt][kt] = mma(qtr, chunk_op(dsp[kt], half), dkacc[dt][kt]);
      }
    }
}

// One pipelined step: A(n+1) from (sa, ra), B(n) of the half whose first query
// is qrow0, C(n-1) from (sc, rc).  SKIP_C: there is no half n-1.
template <bool MASKED, bool SKIP_C, bool SEG>
__device__ __forceinline__ void dkdv_step(const QStageT<SEG>& sa, int ra, const QStageT<SEG>& sc,
                                          int rc, int qrow0, int kw, int lane, float c_scale,
                                          int causal, int band, const bf16x8_t (&kop)[kKT][4],
                                          const bf16x8_t (&vop)[kKT][4], DkdvPipe<SEG>& pipe,
                                          floatx16 (&dkacc)[2][kKT], floatx16 (&dvacc)[2][kKT],
                                          int32_t sk) {
  uint32_t pp[kKT][8], dsp[kKT][8];
  if (!SKIP_C) dkdv_accum(sc, rc, lane, pipe.pp, pipe.dsp, dkacc, dvacc);
  dkdv_softmax<MASKED, SEG>(pipe.s, pipe.dp, pp, dsp, qrow0, kw, lane, c_scale, causal, band,
                            pipe.qs, sk);
  dkdv_scores<SEG>(sa, ra, lane, kop, vop, pipe.s, pipe.dp, pipe.qs);
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // empty asm on B's results: they are formed inside this step, so every
      // step carries its own softmax work beside its MFMAs
      asm volatile("" : "+v"(pp[kt][i]), "+v"(dsp[kt][i]));
      pipe.pp[kt][i] = pp[kt][i];
      pipe.dsp[kt][i] = dsp[kt][i];
    }
  __builtin_amdgcn_sched_barrier(0);  // keep each step's schedule to itself
}

// BANDED: a window of band keys; stages that reach its far edge take the
// masked body too.
// Without it the predicate is causal (causal = 1) or absent (causal = 0).
// SEG: only pairs of equal segment ids (seg, [B][N], batch = head / hpb)
// exist; the walk covers only the queries whose ids fall in the block's key-id
// range, and every stage takes the masked body.
template <bool BANDED, bool SEG>
__global__ __launch_bounds__(kThreads, 2) void bwd_dkdv_bf16(
    const __bf16* __restrict__ q, const __bf16* __restrict__ k, const __bf16* __restrict__ v,
    const __bf16* __restrict__ dout, const float* __restrict__ nlseg,
    const float* __restrict__ ndeltag, __bf16* __restrict__ dk, __bf16* __restrict__ dv,
    int heads, int N, int nkb, float c_scale, float scale, int causal, int band_arg,
    const int32_t* __restrict__ seg, int hpb) {
  using QStage = QStageT<SEG>;
  const int band = BANDED ? band_arg : 0;
  __shared__ QStage st0, st1, st2;
  int head, kb;
  if (!map_block(blockIdx.x, heads, nkb, false, 4, head, kb)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int i32 = lane & 31, h = lane >> 5;
  const size_t base = (size_t)head * N * kD;
  const size_t rbase = (size_t)head * N;
  const int kw = kb * kBlk + wave * kRowsW;  // first key of this wave

  // stationary B operands: lane holds X[key kw + 32 kt + i32][16 kk + 8 h .. +7]
  bf16x8_t kop[kKT][4], vop[kKT][4];
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
    const int key = kw + 32 * kt + i32;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 a = make_uint4(0, 0, 0, 0), b = a;
      if (key < N) {
        a = ldg16(k + base + (size_t)key * kD + 16 * kk + 8 * h);
        b = ldg16(v + base + (size_t)key * kD + 16 * kk + 8 * h);
      }
      kop[kt][kk] = __builtin_bit_cast(bf16x8_t, a);
      vop[kt][kk] = __builtin_bit_cast(bf16x8_t, b);
    }
  }
  floatx16 dkacc[2][kKT], dvacc[2][kKT];  // [dt][kt]: (feature x key) tiles, lane holds a key column
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < kKT; ++b) {
      dkacc[a][b] = floatx16{};
      dvacc[a][b] = floatx16{};
    }

  // queries that see these keys: from the block's first key (causal) or 0, to
  // the last key's window end or N (with segment ids, within their span)
  int qstart = causal ? kb * kBlk : 0;
  int qend = band ? min(N, kb * kBlk + kBlk - 1 + band) : N;
  const int32_t* segrow = SEG ? seg + (size_t)(head / hpb) * N : nullptr;
  bool seg_uniform = false;  // every query of the walk has the block's one key id
  if (SEG) {
    __shared__ int32_t red[2][kWaves][4];
    const SegSpan sp = seg_span<kThreads>(segrow, N, kb * kBlk, kBlk, qstart, qend, tid, red);
    // every key is also a query with its own id, so the span is never empty
    qstart = __builtin_amdgcn_readfirstlane(sp.first);
    qend = __builtin_amdgcn_readfirstlane(sp.last);
    seg_uniform = sp.lo == sp.hi && sp.dense;
  }
  const int nst = (qend - qstart + kT2 - 1) / kT2;  // stages of 64 queries
  const uint32_t tbytes = (uint32_t)N * kD * 2, rbytes = (uint32_t)N * 4;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(q + base, tbytes), ro = head_rsrc(dout + base, tbytes);
  const __amdgpu_buffer_rsrc_t rl = head_rsrc(nlseg + rbase, rbytes), rd = head_rsrc(ndeltag + rbase, rbytes);
  __amdgpu_buffer_rsrc_t rs = rl;
  if (SEG) rs = head_rsrc(segrow, rbytes);
  const int32_t sk = SEG && kw + i32 < N ? segrow[kw + i32] : 0;  // the lane's key id
  auto issue = [&](QStage& s, int t) {
    const int r0 = qstart + t * kT2;
    if (wave == 0) rows_async(rl, s.nlse, r0, lane);
    else if (wave == 1) rows_async(rd, s.ndelta, r0, lane);
    else if (SEG && wave == 2) rows_async(rs, (float*)s.seg, r0, lane);
    tile_async<kT2, kWaves>(rq, s.q, r0, wave, lane);
    tile_async<kT2, kWaves>(ro, s.dout, r0, wave, lane);
  };
  DkdvPipe<SEG> pipe;
  // stage s: cur holds it, nxt stage s + 1, prv stage s - 1 (and receives s + 2)
  auto stage = [&](auto masked, auto first, QStage& cur, QStage& nxt, QStage& prv, int s) {
    constexpr bool M = decltype(masked)::value, F = decltype(first)::value;
    const int q0 = qstart + s * kT2;
    dkdv_step<M, F, SEG>(cur, 32, prv, 32, q0, kw, lane, c_scale, causal, band, kop, vop, pipe,
                         dkacc, dvacc, sk);
    wait_vm_barrier<0>();  // stage s + 1 has landed; every wave is done with prv
    if (s + 2 < nst) issue(prv, s + 2);
    dkdv_step<M, false, SEG>(nxt, 0, cur, 0, q0 + 32, kw, lane, c_scale, causal, band, kop, vop,
                             pipe, dkacc, dvacc, sk);
  };
  // stages 0 and 1 hold the block's diagonal (masked body); later stages lie
  // wholly after every key of the block, so only a window's far edge masks
  // them: stage s does once its last query minus the block's first key
  // reaches band, i.e. from stage edge on.  Stages 2 .. edge - 1 (rounded down
  // to whole turns of the 3-stage ring) take the plain body, the rest the
  // masked one.  With segment ids the ids mask too, except where every query
  // of the walk shares the block's single key id: then the stages that lie
  // wholly inside the walk need only the base predicate.
  static_assert(kBlk == 2 * kT2, "the block's diagonal spans stages 0 and 1");
  using T = std::true_type;
  using Fl = std::false_type;
  const int edge = BANDED ? (band - kT2 + 1 + kb * kBlk - qstart + kT2 - 1) / kT2 : nst;
  const int whole = seg_uniform ? (qend - qstart) / kT2 : 2;  // segments: stages wholly inside
  const int plain_end = SEG ? 2 + 3 * (max(min(BANDED ? edge : nst, whole) - 2, 0) / 3)
                            : BANDED ? 2 + 3 * (max(edge - 2, 0) / 3) : nst;

  issue(st0, 0);
  if (nst > 1) issue(st1, 1);
  wait_vm_barrier<0>();
  if (causal && kw >= qstart + kT2 && nst > 1) {
    // no query of stage 0 sees this wave's keys: only the stage's barrier and
    // loads, A of stage 1's first half, and zero weights for the C of stage
    // 0's last half (issued by stage 1's first step)
    wait_vm_barrier<0>();
    if (2 < nst) issue(st2, 2);
    dkdv_scores<SEG>(st1, 0, lane, kop, vop, pipe.s, pipe.dp, pipe.qs);
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pipe.pp[kt][i] = 0u;
        pipe.dsp[kt][i] = 0u;
      }
  } else {
    dkdv_scores<SEG>(st0, 0, lane, kop, vop, pipe.s, pipe.dp, pipe.qs);  // A(0)
    stage(T{}, T{}, st0, st1, st2, 0);
  }
  if (nst > 1) stage(T{}, Fl{}, st1, st2, st0, 1);
  int s = 2;
  for (; s < min(plain_end, nst); s += 3) {
    stage(Fl{}, Fl{}, st2, st0, st1, s);
    if (s + 1 < nst) stage(Fl{}, Fl{}, st0, st1, st2, s + 1);
    if (s + 2 < nst) stage(Fl{}, Fl{}, st1, st2, st0, s + 2);
  }
  if (BANDED || SEG) {
    for (; s < nst; s += 3) {
      stage(T{}, Fl{}, st2, st0, st1, s);
      if (s + 1 < nst) stage(T{}, Fl{}, st0, st1, st2, s + 1);
      if (s + 2 < nst) stage(T{}, Fl{}, st1, st2, st0, s + 2);
    }
  }
  // C of the last half (rows 32.. of the last stage)
  {
    const int r = (nst - 1) % 3;
    const QStage& last = r == 0 ? st0 : r == 1 ? st1 : st2;
    dkdv_accum(last, 32, lane, pipe.pp, pipe.dsp, dkacc, dvacc);
  }

  // epilogue: lane holds key column kw + 32 kt + i32, feature rows 32 dt + acc_row(r, h)
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt) {
    const int key = kw + 32 * kt + i32;
    if (key >= N) continue;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = 32 * dt + 8 * g + 4 * h;
        uint2 wk, wv;
        wk.x = pack_bf16(dkacc[dt][kt][4 * g + 0] * scale, dkacc[dt][kt][4 * g + 1] * scale);
        wk.y = pack_bf16(dkacc[dt][kt][4 * g + 2] * scale, dkacc[dt][kt][4 * g + 3] * scale);
        wv.x = pack_bf16(dvacc[dt][kt][4 * g + 0], dvacc[dt][kt][4 * g + 1]);
        wv.y = pack_bf16(dvacc[dt][kt][4 * g + 2], dvacc[dt][kt][4 * g + 3]);
        *(uint2*)(dk + base + (size_t)key * kD + d) = wk;
        *(uint2*)(dv + base + (size_t)key * kD + d) = wv;
      }
  }
}

}  // namespace

size_t bwd_workspace_bytes_bf16(int64_t heads, int64_t N) {
  return (size_t)heads * N * 2 * sizeof(float);  // -delta, then -lse / scale
}

hipError_t launch_bwd_bf16(const __bf16* q, const __bf16* k, const __bf16* v, const __bf16* o,
                           const __bf16* dout, const float* lse, __bf16* dq, __bf16* dk,
                           __bf16* dv, void* workspace, int64_t heads, int64_t N, double scale,
                           const Mask& mk, bool prepared, hipStream_t stream, const Timers& tm) {
  const int64_t rows = heads * N;
  float* ndelta = (float*)workspace;
  float* nlse = ndelta + rows;
  const float c = (float)(scale * 1.4426950408889634);
  const int nb = (int)((N + kBlk - 1) / kBlk);
  const unsigned grid = (unsigned)(8 * ((heads + 7) / 8) * nb);
  if (!prepared) {  // else the forward already wrote both per-row values (dO = O)
    if (hipError_t e = mark(tm.start[kTimerBwdPre], stream)) return e;
    if (dout == o)
      hipLaunchKernelGGL(bwd_prep_bf16<true>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                         stream, o, dout, lse, ndelta, nlse, (float)(1.0 / scale), rows);
    else
      hipLaunchKernelGGL(bwd_prep_bf16<false>, dim3((unsigned)((rows + 127) / 128)), dim3(256), 0,
                         stream, o, dout, lse, ndelta, nlse, (float)(1.0 / scale), rows);
    if (hipError_t e = mark(tm.stop[kTimerBwdPre], stream)) return e;
  }
  if (hipError_t e = mark(tm.start[kTimerBwdDkdv], stream)) return e;
  auto kern = mk.seg ? (mk.band > 0 ? bwd_dkdv_bf16<true, true> : bwd_dkdv_bf16<false, true>)
                     : (mk.band > 0 ? bwd_dkdv_bf16<true, false> : bwd_dkdv_bf16<false, false>);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), 0, stream, q, k, v, dout, nlse, ndelta, dk,
                     dv, (int)heads, (int)N, nb, c, (float)scale, mk.causal, mk.band, mk.seg,
                     mk.hpb);
  if (hipError_t e = mark(tm.stop[kTimerBwdDkdv], stream)) return e;
  if (hipError_t e = hipGetLastError()) return e;
  return launch_bwd_dq_bf16(q, k, v, dout, nlse, ndelta, dq, heads, N, scale, mk, stream, tm);
}

}  // namespace attn
