// Softmax core and the interleaved 32-key step shared by the attention
// kernels for gfx950 (sliding-window / dense causal heads in attn_window.hip,
// block-sparse retrieval heads in attn.hip).
//
// What they compute (Synced RTPurbo article, "化繁为简，被低估的 SWA": most
// heads attend only a recent window; aitop.news summary of "Full Attention
// Strikes Back": retrieval heads run exact attention on an indexer-selected
// set): for query i and its key set J_i,
//     o_i = sum_{j in J_i} softmax_j(scale * q_i.k_j) v_j,
// with J_i = {i-w < j <= i} for a window head and J_i = {j <= i in the kept
// blocks} for a retrieval head.
//
// Shared design (MI355X-first):
//  * A wave owns 64 queries (one 64-token query block) of one head; its O
//    accumulator (64 x 128 fp32) lives in AGPRs. S^T = K Q^T runs on
//    v_mfma_f32_32x32x16_bf16 with queries along the lanes, so a query's
//    scores sit in one lane pair; every K or V^T operand read from LDS feeds
//    two MFMAs (two 32-query tiles), halving LDS traffic per flop.
//  * Key rows are placed so that the S^T accumulator is directly the B
//    operand of the P.V MFMA (no shuffles), and V arrives pre-transposed (V^T)
//    so its A operand is one 16-byte read.
//  * Softmax in base 2 against a fixed per-row reference taken from the
//    row's diagonal key block, so O is never rescaled; a rare second pass
//    covers rows whose scores climb far above that reference.
//  * Software pipeline: the QK MFMAs of tile t+1 are issued next to the
//    exp/pack VALU work of tile t, then P.V of tile t, so the matrix and vector
//    units overlap.
//  * Masks only on tiles that straddle the causal diagonal or the window's
//    lower edge; tiles outside a wave's set are skipped (the pages' point
//    about SWA without three-segment KV concat or a mask tensor, RTP-LLM
//    section of the Synced article).
//  * Work order: query blocks from last to first (heaviest first, the pages'
//    sparsity-aware scheduling).
#pragma once

#include "common.h"

namespace rtp {

// ------------------------------------------------------------ softmax core
// Base-2 softmax with a fixed reference per query: m is the max score of the
// query's own diagonal key half block (computed before the main pass), and
// p = 2^(c s - c m) may exceed 1: fp32 and bf16 share the exponent range, so
// values up to 2^64 lose nothing, and O and l share the reference, so O / l
// is exact. The main pass only records whether a lane's partial sum of some
// tile left that range (a score more than ~64 / c above m); if so (rare), a
// max-only pass finds every row's true maximum and the job is recomputed
// with it (then p <= 1). The O accumulator is touched only by MFMAs, which
// keeps it resident in AGPRs with no per-tile rescale.
constexpr float kSumLimit = 18446744073709551616.f;  // 2^64

// Row-sum update with one packed pair of p. F32: the two fp32 values, by
// plain adds. Otherwise the bf16-rounded pair that feeds the P.V MFMA, by one
// v_dot2_f32_bf16. Both give O / l within the bf16 rounding of p. On gfx950 a
// dot2 waits for the MFMA in flight, so the window kernel, whose steps keep
// the matrix pipe busy, uses the adds (2% faster at 128K); the sparse kernel
// measures faster with dot2.
template <bool F32>
__device__ __forceinline__ float row_add(float acc, float p0, float p1,
                                         uint32_t w) {
  if constexpr (F32) {
    return (acc + p0) + p1;
  } else {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one,
                                           acc, false);
  }
}

struct Soft {
  float mref[2];
  float lsum[2];
};

// max over the scores of a tile for query tile j (lane pair combined)
template <int NS>
__device__ __forceinline__ float tile_max(const f32x16 (&s)[NS][2], int j) {
  float m = -INFINITY;
#pragma unroll
  for (int u = 0; u < NS; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, s[u][j][i]);
  return fmaxf(m, __shfl_xor(m, 32));
}

// p = exp2(c s - c m) packed to bf16 (the B operand of P.V); ls = this
// lane's sum of p (row_add<F32>).
template <int NS, bool F32>
__device__ __forceinline__ void exp_pack(const f32x16 (&s)[NS][2],
                                         const Soft& sf, bf16x8 (&pb)[NS][2][2],
                                         float (&ls)[2], float c) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float mc = sf.mref[j] * c;
    float acc = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * h + 2 * e;
          const float p0 = fast_exp2(fmaf(s[u][j][i], c, -mc));
          const float p1 = fast_exp2(fmaf(s[u][j][i + 1], c, -mc));
          w[e] = pack_bf16x2(p0, p1);
          acc = row_add<F32>(acc, p0, p1, w[e]);
        }
        const uint4 q4 = make_uint4(w[0], w[1], w[2], w[3]);
        pb[u][j][h] = __builtin_bit_cast(bf16x8, q4);
      }
    ls[j] = acc;
  }
}

// One tile against the current references: packs P, adds the row sums and
// returns whether this lane's partial sum left the safe range. NaN (from NaN
// inputs) does not count: raising the reference cannot remove it, so it just
// propagates to the output.
template <int NS, bool F32>
__device__ __forceinline__ bool softmax_step(const f32x16 (&s)[NS][2],
                                             Soft& sf, bf16x8 (&pb)[NS][2][2],
                                             float c) {
  float ls[2];
  exp_pack<NS, F32>(s, sf, pb, ls, c);
  sf.lsum[0] += ls[0];
  sf.lsum[1] += ls[1];
  return (ls[0] > kSumLimit) || (ls[1] > kSumLimit);
}

template <int NS>
__device__ __forceinline__ void raise_refs(const f32x16 (&s)[NS][2],
                                           Soft& sf) {
#pragma unroll
  for (int j = 0; j < 2; ++j) sf.mref[j] = fmaxf(sf.mref[j], tile_max<NS>(s, j));
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[2][4]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x16 z = {};
      acc[j][mt] = z;
    }
}

// Mask scores of sub-tile starting at key kmin for query tiles with first
// query q0 (+32 for the second): valid iff key <= i and key > i - window.
__device__ __forceinline__ void mask_sub(f32x16 (&s)[2], int kmin, int q0,
                                         int window, int lane) {
  const int g = lane >> 5, n = lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qi = q0 + 32 * j + n;
    const int rel0 = qi - kmin - 8 * g;  // qi - key of element 0
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // key <= qi and key > qi - window, as one unsigned compare
      const unsigned rel = (unsigned)(rel0 - 16 * (i >> 3) - (i & 7));
      s[j][i] = rel < (unsigned)window ? s[j][i] : -INFINITY;
    }
  }
}

__device__ __forceinline__ void store_out(const f32x16 (&acc)[2][4],
                                          const Soft& sf, float c, u16* out,
                                          float* lse, int head, int q0, int S,
                                          int lane) {
  const int g = lane >> 5, n = lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qi = q0 + 32 * j + n;
    const float l = sf.lsum[j] + __shfl_xor(sf.lsum[j], 32);
    if (qi >= S) continue;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    u16* op = out + ((size_t)head * S + qi) * kD;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * mt + 8 * q4 + 4 * g;
        uint2 w;
        w.x = (uint32_t)f2bf(acc[j][mt][4 * q4 + 0] * inv) |
              ((uint32_t)f2bf(acc[j][mt][4 * q4 + 1] * inv) << 16);
        w.y = (uint32_t)f2bf(acc[j][mt][4 * q4 + 2] * inv) |
              ((uint32_t)f2bf(acc[j][mt][4 * q4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (lse && g == 0)
      lse[(size_t)head * S + qi] =
          (sf.mref[j] * c + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
  }
}

__device__ __forceinline__ void load_q(const u16* q, int head, int q0, int S,
                                       bf16x8 (&qf)[2][8], int lane) {
  const int g = lane >> 5, n = lane & 31;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qi = q0 + 32 * j + n;
    const u16* qp = q + ((size_t)head * S + (qi < S ? qi : 0)) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
      if (qi >= S) { bf16x8 z = {}; v = z; }
      qf[j][ks] = v;
    }
  }
}

// One 32-key step with the work interleaved by hand: the QK MFMAs of the next
// sub-tile (K operand kop(ks), ks = 0..7) and the P.V MFMAs of the current
// one (V^T operand vop(h, mt)) are issued in groups of 4, next to the
// exp/pack work of the current scores s and the operand reads of the next
// group. sched_barrier keeps the compiler from regrouping them (it otherwise
// issues all QK MFMAs, then all exps, then all P.V MFMAs). dop(i), i = 0..8,
// runs at the head of group i: the caller's staging loads for a later tile go
// there, one per group, because a burst of them stalls the wave's issue for
// several hundred cycles while spread out they hide behind the MFMAs. Row
// sums use row_add<F32>. Returns whether a row sum left the safe range.
template <bool F32, class KOp, class VOp, class DOp>
__device__ __forceinline__ bool attn_step(KOp kop, VOp vop, DOp dop,
                                          const bf16x8 (&qf)[2][8],
                                          const f32x16 (&s)[1][2],
                                          f32x16 (&sn)[1][2], Soft& sf,
                                          f32x16 (&acc)[2][4], float c) {
  const float mc[2] = {sf.mref[0] * c, sf.mref[1] * c};
  uint32_t w[2][2][4];  // packed P: [query tile j][key half h][pair]
  float ls[2] = {0.f, 0.f};
  // exp/pack of 4 scores (pairs e0, e0+1) of query tile j, key half h
  auto expq = [&](int j, int h, int e0) {
#pragma unroll
    for (int e = e0; e < e0 + 2; ++e) {
      const int i = 8 * h + 2 * e;
      const float p0 = fast_exp2(fmaf(s[0][j][i], c, -mc[j]));
      const float p1 = fast_exp2(fmaf(s[0][j][i + 1], c, -mc[j]));
      w[j][h][e] = pack_bf16x2(p0, p1);
      ls[j] = row_add<F32>(ls[j], p0, p1, w[j][h][e]);
    }
  };
  auto pb = [&](int j, int h) {
    return __builtin_bit_cast(
        bf16x8, make_uint4(w[j][h][0], w[j][h][1], w[j][h][2], w[j][h][3]));
  };
  f32x16 z = {};
  sn[0][0] = z;
  sn[0][1] = z;
  // Group g's MFMAs use operands read in group g-1, and each of groups 0-7
  // carries a quarter of one (query tile, key half) of exp/pack work:
  //   g0      read K ks 0,1                 | exp (j0,h0) and (j1,h0): q0
  //   g1-g3   read K 2g,2g+1; QK ks 2g-2,2g-1 | exp q1..q3 of h0
  //   g4      read V h0 mt0,1; QK ks 6,7    | exp (j0,h1) first half
  //   g5      read V h0 mt2,3; PV h0 mt0,1  | exp (j0,h1) second half
  //   g6      read V h1 mt0-3; PV h0 mt2,3  | exp (j1,h1) first half
  //   g7      PV h1 j0                      | exp (j1,h1) second half
  //   g8      PV h1 j1
  // Group 0 has no MFMA of its own: the previous step's last ones drain
  // while it runs. Each group's operand reads (and staging load) are fenced
  // off at its head: left to itself the scheduler sinks them to the end of
  // the group, right before the next group waits for them, which leaves
  // the LDS latency uncovered.
  dop(0);
  bf16x8 ka = kop(0), kb = kop(1);
  __builtin_amdgcn_sched_barrier(0);
  expq(0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    dop(q);
    const bf16x8 kc = kop(2 * q), kd = kop(2 * q + 1);
    __builtin_amdgcn_sched_barrier(0);
    sn[0][0] = mfma32(ka, qf[0][2 * q - 2], sn[0][0]);
    sn[0][1] = mfma32(ka, qf[1][2 * q - 2], sn[0][1]);
    sn[0][0] = mfma32(kb, qf[0][2 * q - 1], sn[0][0]);
    sn[0][1] = mfma32(kb, qf[1][2 * q - 1], sn[0][1]);
    expq(q >> 1, 0, 2 * (q & 1));
    ka = kc;
    kb = kd;
    __builtin_amdgcn_sched_barrier(0);
  }
  // g4
  dop(4);
  bf16x8 va = vop(0, 0), vb = vop(0, 1);
  __builtin_amdgcn_sched_barrier(0);
  sn[0][0] = mfma32(ka, qf[0][6], sn[0][0]);
  sn[0][1] = mfma32(ka, qf[1][6], sn[0][1]);
  sn[0][0] = mfma32(kb, qf[0][7], sn[0][0]);
  sn[0][1] = mfma32(kb, qf[1][7], sn[0][1]);
  expq(0, 1, 0);
  __builtin_amdgcn_sched_barrier(0);
  // g5
  dop(5);
  const bf16x8 vc = vop(0, 2), vd = vop(0, 3);
  __builtin_amdgcn_sched_barrier(0);
  {
    const bf16x8 p00 = pb(0, 0), p10 = pb(1, 0);
    acc[0][0] = mfma32(va, p00, acc[0][0]);
    acc[1][0] = mfma32(va, p10, acc[1][0]);
    acc[0][1] = mfma32(vb, p00, acc[0][1]);
    acc[1][1] = mfma32(vb, p10, acc[1][1]);
  }
  expq(0, 1, 2);
  __builtin_amdgcn_sched_barrier(0);
  // g6
  dop(6);
  const bf16x8 v10 = vop(1, 0), v11 = vop(1, 1), v12 = vop(1, 2),
               v13 = vop(1, 3);
  __builtin_amdgcn_sched_barrier(0);
  {
    const bf16x8 p00 = pb(0, 0), p10 = pb(1, 0);
    acc[0][2] = mfma32(vc, p00, acc[0][2]);
    acc[1][2] = mfma32(vc, p10, acc[1][2]);
    acc[0][3] = mfma32(vd, p00, acc[0][3]);
    acc[1][3] = mfma32(vd, p10, acc[1][3]);
  }
  expq(1, 1, 0);
  __builtin_amdgcn_sched_barrier(0);
  // g7
  dop(7);
  {
    const bf16x8 p = pb(0, 1);
    acc[0][0] = mfma32(v10, p, acc[0][0]);
    acc[0][1] = mfma32(v11, p, acc[0][1]);
    acc[0][2] = mfma32(v12, p, acc[0][2]);
    acc[0][3] = mfma32(v13, p, acc[0][3]);
  }
  expq(1, 1, 2);
  __builtin_amdgcn_sched_barrier(0);
  // g8
  dop(8);
  {
    const bf16x8 p = pb(1, 1);
    acc[1][0] = mfma32(v10, p, acc[1][0]);
    acc[1][1] = mfma32(v11, p, acc[1][1]);
    acc[1][2] = mfma32(v12, p, acc[1][2]);
    acc[1][3] = mfma32(v13, p, acc[1][3]);
  }
  sf.lsum[0] += ls[0];
  sf.lsum[1] += ls[1];
  return (ls[0] > kSumLimit) || (ls[1] > kSumLimit);
}

}  // namespace rtp
