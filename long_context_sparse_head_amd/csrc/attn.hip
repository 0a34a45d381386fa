// Attention kernels for gfx950: sliding-window / dense causal heads and
// block-sparse retrieval heads.
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
//
// Window kernel: 4 waves = 4 (head, query block) jobs of one KV group share
// one stream of 64-key tiles, staged by direct global->LDS loads
// (global_load_lds_dwordx4) into a 3-deep LDS ring of padded rows; a tile's
// loads are dealt one per MFMA group of a step, not issued in one burst. Each
// XCD takes a contiguous, equal share of all KV groups' work items.
//
// Sparse kernel: each wave runs its own (retrieval head, query block) job over
// its block list in 32-key half tiles: K goes straight into registers in MFMA
// operand layout (vector-memory path), V^T through a per-wave LDS slot (LDS
// DMA path), so the gather traffic is split over both paths.
#include <type_traits>

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
// keeps it resident in AGPRs with no per-tile rescale. Row sums use the
// bf16-rounded p that also feeds the P.V MFMA.
constexpr float kSumLimit = 18446744073709551616.f;  // 2^64

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

// p = exp2(c s - c m) packed to bf16 (the B operand of P.V); ls = sum of the
// packed values of this lane.

template <int NS>
__device__ __forceinline__ void exp_pack(const f32x16 (&s)[NS][2],
                                         const Soft& sf, bf16x8 (&pb)[NS][2][2],
                                         float (&ls)[2], float c) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
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
          acc = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2, w[e]), one, acc, false);
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
template <int NS>
__device__ __forceinline__ bool softmax_step(const f32x16 (&s)[NS][2],
                                             Soft& sf, bf16x8 (&pb)[NS][2][2],
                                             float c) {
  float ls[2];
  exp_pack<NS>(s, sf, pb, ls, c);
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

// =====================================================================
// Window / dense kernel
// =====================================================================
constexpr int WSTAGES = 3;
// Padded LDS rows (conflict-free for 8 consecutive rows, and every operand
// address of a lane is one base register plus an immediate offset).
constexpr int KROW_B = 272;                 // 256 B of K + 16 B pad
constexpr int VROW_B = 144;                 // 128 B of V^T + 16 B pad
constexpr int KTILE_B = 64 * KROW_B;        // 17408
constexpr int VTILE_B = 128 * VROW_B;       // 18432
constexpr int STAGE_B = KTILE_B + VTILE_B;  // 35840
constexpr int K_DMA = KTILE_B / 1024;       // 17 loads of 1 KB
constexpr int V_DMA = VTILE_B / 1024;       // 18 loads of 1 KB
constexpr int DMA_PER_WAVE = (K_DMA + V_DMA + 3) / 4;  // 9
static_assert(K_DMA == 17 && V_DMA == 18 && DMA_PER_WAVE == 9,
              "win_issue deals the loads for this split");

// Workgroups are dealt round-robin to the chip's 8 XCDs (each with its own
// L2). The work items of all KV groups are laid end to end and cut into 8
// contiguous ranges of equal estimated cost (tiles walked plus a per-item
// constant); XCD x runs range x. So the XCDs stay balanced when KV groups
// have different numbers of window heads or items differ in length (causal
// dense), and each XCD's concurrent workgroups cover neighbouring query
// blocks of one group.
constexpr int kXcds = 8;

// Heads are processed in packs: the window heads of one KV head that share
// a window size (so they share every K/V tile). With one window for all
// heads a pack is simply a KV group.
struct WinParams {
  const u16* q; const u16* k; const u16* vt; u16* out; float* lse;
  int S, S_pad, n_b, Hkv;
  float c;
  int per_xcd, n_items;
  int32_t xcd_begin[kXcds + 1];     // item range of each XCD
  uint8_t hlist[kMaxHeads];   // window heads, pack by pack
  int16_t hoff[kMaxHeads + 1];      // first hlist entry of each pack
  int32_t item_off[kMaxHeads + 1];  // first work item of each pack
  uint8_t pack_kv[kMaxHeads];       // KV head of each pack
  int32_t pack_win[kMaxHeads];      // window of each pack
};

// The 35 DMA loads of a tile (17 K, 18 V^T) are dealt round-robin to the 4
// waves. Load i writes LDS bytes [1024 i, 1024 i + 1024) of the stage (K rows
// first, then V^T rows); a lane's 16-byte unit either holds data or is a pad
// unit (then it re-reads a neighbouring chunk). A lane's global byte offset
// inside a tile does not depend on the tile, so it is computed once.
// K row r (MFMA row order) holds key (r & 32) + perm_row(r & 31).
struct WinLaneOffsets {
  uint32_t off[DMA_PER_WAVE];
};

__device__ __forceinline__ uint32_t win_unit_offset(int ld, int lane) {
  if (ld < K_DMA) {
    const int u = 64 * ld + lane;
    const int r = u / 17, c = min(u % 17, 15);
    return (uint32_t)(((r & 32) + perm_row(r & 31)) * 256 + c * 16);
  }
  const int u = 64 * (ld - K_DMA) + lane;
  const int d = u / 9, c = min(u % 9, 7);
  return (uint32_t)(d * 128 + c * 16);  // V^T block row d: 64 keys, 128 B
}

__device__ __forceinline__ WinLaneOffsets win_offsets(int wave, int lane) {
  WinLaneOffsets o;
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j) {
    const int ld = wave + 4 * j;
    o.off[j] = ld < K_DMA + V_DMA ? win_unit_offset(ld, lane) : 0u;
  }
  return o;
}

__device__ __attribute__((noinline)) void win_issue_ragged_k(
    const WinParams& p, int g, int kb, char* stage, int ld, int lane) {
  const int u = 64 * ld + lane;
  const int r = u / 17, c = min(u % 17, 15);
  int key = kb * 64 + (r & 32) + perm_row(r & 31);
  key = key < p.S ? key : p.S - 1;
  dma16(p.k + ((size_t)g * p.S + key) * kD + c * 8, stage + ld * 1024);
}

// First byte of a tile's K rows and of its V^T block.
__device__ __forceinline__ void win_tile_src(const WinParams& p, int g, int kb,
                                             const char*& kt, const char*& vt) {
  kt = reinterpret_cast<const char*>(p.k) +
       ((size_t)g * p.S + (size_t)kb * 64) * (kD * 2);
  vt = reinterpret_cast<const char*>(p.vt + ((size_t)g * p.n_b + kb) * 64 * kD);
}

// Load j (0..8) of this wave for a full tile: loads 0..3 are K rows, load 4 is
// K for wave 0 and V^T for the others, loads 5..8 are V^T. The stage has only
// 35 loads, so wave 3 repeats its load 7 as load 8 (same bytes, same place),
// which keeps the issue free of branches.
__device__ __forceinline__ void win_issue_one(const char* kt, const char* vt,
                                              char* stage,
                                              const WinLaneOffsets& o,
                                              int wave, int j) {
  if (j < 4) {
    dma16(kt + o.off[j], stage + wave * 1024 + j * 4096);
  } else if (j == 4) {
    dma16((wave == 0 ? kt : vt) + o.off[4], stage + wave * 1024 + 4 * 4096);
  } else if (j < 8) {
    dma16(vt + o.off[j], stage + wave * 1024 + j * 4096);
  } else {
    const int jj = wave < 3 ? 8 : 7;
    dma16(vt + o.off[jj], stage + wave * 1024 + jj * 4096);
  }
}

// All loads of this wave for tile kb, back to back.
__device__ __forceinline__ void win_issue(const WinParams& p, int g, int kb,
                                          char* stage, const WinLaneOffsets& o,
                                          int wave, int lane) {
  const char *kt, *vt;
  win_tile_src(p, g, kb, kt, vt);
  if ((kb + 1) * 64 > p.S) {  // last block of a ragged S: rows past S
#pragma unroll 1                // re-read row S-1 (masked anyway)
    for (int j = 0; j < DMA_PER_WAVE; ++j) {
      const int ld = wave + 4 * j;
      if (ld < K_DMA) win_issue_ragged_k(p, g, kb, stage, ld, lane);
      else if (ld < K_DMA + V_DMA) dma16(vt + o.off[j], stage + ld * 1024);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j) win_issue_one(kt, vt, stage, o, wave, j);
}

// S^T for one 32-key sub-tile st of a staged tile: s[0][j], j = query tile
__device__ __forceinline__ void win_qk(const char* stage, int st,
                                       const bf16x8 (&qf)[2][8],
                                       f32x16 (&s)[1][2], int lane) {
  const int g = lane >> 5, n = lane & 31;
  f32x16 z = {};
  s[0][0] = z;
  s[0][1] = z;
  const char* row = stage + (32 * st + n) * KROW_B + 16 * g;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(row + 32 * ks);
    s[0][0] = mfma32(a, qf[0][ks], s[0][0]);
    s[0][1] = mfma32(a, qf[1][ks], s[0][1]);
  }
}

__device__ __forceinline__ void win_pv(const char* stage, int st,
                                       const bf16x8 (&pb)[1][2][2],
                                       f32x16 (&acc)[2][4], int lane) {
  const int g = lane >> 5, n = lane & 31;
  const char* base = stage + KTILE_B + n * VROW_B + 16 * g + 64 * st;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(
          base + 32 * mt * VROW_B + 32 * ks);
      acc[0][mt] = mfma32(a, pb[0][0][ks], acc[0][mt]);
      acc[1][mt] = mfma32(a, pb[0][1][ks], acc[1][mt]);
    }
}

// K operand of a 32-key sub-tile straight from global memory: lane l holds
// the row of MFMA row l%32 (key perm_row(l%32)), 8 d-chunks. koff is the
// lane's byte offset inside a tile; rows past S (ragged last block) re-read
// row S-1 (they are masked).
__device__ __forceinline__ uint32_t k_lane_off(int lane) {
  return (uint32_t)(perm_row(lane & 31) * 256 + 16 * (lane >> 5));
}

__device__ __forceinline__ void load_k_sub(const u16* kbase, int S, int k0,
                                           uint32_t koff, bf16x8 (&kr)[8],
                                           int lane) {
  const char* kp;
  if (k0 + 32 <= S) {
    kp = reinterpret_cast<const char*>(kbase) + (size_t)k0 * 256 + koff;
  } else {
    int key = k0 + perm_row(lane & 31);
    key = key < S ? key : S - 1;
    kp = reinterpret_cast<const char*>(kbase + (size_t)key * kD) + 16 * (lane >> 5);
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
    kr[ks] = *reinterpret_cast<const bf16x8*>(kp + 32 * ks);
}

__device__ __forceinline__ void qk_regs(const bf16x8 (&kr)[8],
                                        const bf16x8 (&qf)[2][8],
                                        f32x16 (&s)[1][2]) {
  f32x16 z = {};
  s[0][0] = z;
  s[0][1] = z;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    s[0][0] = mfma32(kr[ks], qf[0][ks], s[0][0]);
    s[0][1] = mfma32(kr[ks], qf[1][ks], s[0][1]);
  }
}

// References of a 64-query block: each row's max over the keys it sees in its
// own diagonal key block (it always sees its own key there).
__device__ __forceinline__ void diag_refs(const u16* kbase, int S, int q0,
                                          int window, const bf16x8 (&qf)[2][8],
                                          Soft& sf, int lane) {
  const uint32_t koff = k_lane_off(lane);
  sf.mref[0] = sf.mref[1] = -INFINITY;
#pragma unroll 1
  for (int st = 0; st < 2; ++st) {
    bf16x8 kr[8];
    f32x16 s[1][2];
    load_k_sub(kbase, S, q0 + 32 * st, koff, kr, lane);
    qk_regs(kr, qf, s);
    mask_sub(s[0], q0 + 32 * st, q0, window, lane);
    raise_refs<1>(s, sf);
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
// several hundred cycles while spread out they hide behind the MFMAs. Returns
// whether a row sum left the safe range.
template <class KOp, class VOp, class DOp>
__device__ __forceinline__ bool attn_step(KOp kop, VOp vop, DOp dop,
                                          const bf16x8 (&qf)[2][8],
                                          const f32x16 (&s)[1][2],
                                          f32x16 (&sn)[1][2], Soft& sf,
                                          f32x16 (&acc)[2][4], float c) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
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
      ls[j] = __builtin_amdgcn_fdot2_f32_bf16(
          __builtin_bit_cast(bf16x2, w[j][h][e]), one, ls[j], false);
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
  // while it runs.
  dop(0);
  bf16x8 ka = kop(0), kb = kop(1);
  expq(0, 0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    dop(q);
    const bf16x8 kc = kop(2 * q), kd = kop(2 * q + 1);
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
  sn[0][0] = mfma32(ka, qf[0][6], sn[0][0]);
  sn[0][1] = mfma32(ka, qf[1][6], sn[0][1]);
  sn[0][0] = mfma32(kb, qf[0][7], sn[0][0]);
  sn[0][1] = mfma32(kb, qf[1][7], sn[0][1]);
  expq(0, 1, 0);
  __builtin_amdgcn_sched_barrier(0);
  // g5
  dop(5);
  const bf16x8 vc = vop(0, 2), vd = vop(0, 3);
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

// The window kernel's step: K rows of stage kst (half kh) and V^T rows of
// stage vst (half vh), both from the padded LDS tile.
template <class DOp>
__device__ __forceinline__ bool win_step(const char* kst, int kh,
                                         const char* vst, int vh,
                                         const bf16x8 (&qf)[2][8],
                                         const f32x16 (&s)[1][2],
                                         f32x16 (&sn)[1][2], Soft& sf,
                                         f32x16 (&acc)[2][4], float c,
                                         int lane, DOp dop) {
  const int g = lane >> 5, n = lane & 31;
  const char* krow = kst + (32 * kh + n) * KROW_B + 16 * g;
  const char* vrow = vst + KTILE_B + n * VROW_B + 16 * g + 64 * vh;
  return attn_step(
      [&](int ks) { return *reinterpret_cast<const bf16x8*>(krow + 32 * ks); },
      [&](int h, int mt) {
        return *reinterpret_cast<const bf16x8*>(vrow + 32 * mt * VROW_B +
                                                32 * h);
      },
      dop, qf, s, sn, sf, acc, c);
}

__global__ __launch_bounds__(256, 1) void attn_window_kernel(const WinParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[WSTAGES * STAGE_B];
  __shared__ int over_flag;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int xcd = blockIdx.x % kXcds;
  const int item = p.xcd_begin[xcd] + blockIdx.x / kXcds;
  if (item >= p.xcd_begin[xcd + 1]) return;  // whole workgroup
  int pk = 0;
  while (item >= p.item_off[pk + 1]) ++pk;
  const int ig = item - p.item_off[pk];
  const int h0 = p.hoff[pk], nsw = p.hoff[pk + 1] - h0;
  const int g = p.pack_kv[pk];  // KV head
  const int njobs = nsw * p.n_b;
  if (nsw == 0 || 4 * ig >= njobs) return;  // whole workgroup
  const int job = 4 * ig + wave;
  const bool active = job < njobs;  // idle waves still stage tiles
  const int jl = active ? job : njobs - 1;
  const int qb = p.n_b - 1 - jl / nsw;
  const int head = p.hlist[h0 + jl % nsw];
  const int q0 = qb * 64;
  const int w = p.pack_win[pk];
  // union tile range of the workgroup's jobs (up to four consecutive query
  // blocks when a KV group has fewer than four window heads), walked from the
  // top block down: tile t is key block qb_hi - t
  const int qb_hi = p.n_b - 1 - (4 * ig) / nsw;
  const int qb_lo = p.n_b - 1 - min(4 * ig + 3, njobs - 1) / nsw;
  const int lo = qb_lo * 64 - w + 1;
  const int kt_lo = lo > 0 ? (lo >> 6) : 0;
  const int nt = qb_hi - kt_lo + 1;
  // A 32-key sub-tile needs masking unless every key is inside every query's
  // window; sub-tiles entirely outside (edges only) are masked to nothing.
  auto mask = [&](f32x16 (&s)[1][2], int kmin) {
    const int kmax = kmin + 31, qmax = q0 + 63;
    if (!(kmax <= q0 && kmin > qmax - w)) mask_sub(s[0], kmin, q0, w, lane);
  };
  const WinLaneOffsets off = win_offsets(wave, lane);

  bf16x8 qf[2][8];
  load_q(p.q, head, q0, p.S, qf, lane);
  Soft sf;
  diag_refs(p.k + (size_t)g * p.S * kD, p.S, q0, w, qf, sf, lane);
  if (tid == 0) over_flag = 0;  // published by the first barrier below
  f32x16 acc[2][4];
  f32x16 sa[1][2], sb[1][2];
  for (int attempt = 0;; ++attempt) {
    zero_acc(acc);
    sf.lsum[0] = sf.lsum[1] = 0.f;
    bool over = false;
    // LDS ring: cur holds tile t, nxt tile t+1, spare the stage for t+2
    char* cur = smem;
    char* nxt = smem + STAGE_B;
    char* spare = smem + 2 * STAGE_B;
    win_issue(p, g, qb_hi, cur, off, wave, lane);
    if (nt > 1) win_issue(p, g, qb_hi - 1, nxt, off, wave, lane);
    wait_vm_all();
    __syncthreads();
    // Sub-tile u = 32 keys (tile u/2, half u%2). Step u runs the QK MFMAs of
    // sub-tile u+1 next to the exp/pack of sub-tile u, then P.V(u). One tile
    // (two steps) per iteration; the barrier sits between the steps, when QK
    // moves on to the next tile.
    bf16x8 pb[1][2][2];
    win_qk(cur, 0, qf, sa, lane);
    mask(sa, qb_hi * 64);
    // iteration t: tile t's second half and tile t+1's first half are
    // masked (edges) unless both tiles are clean for every wave
    auto iter = [&](auto with_mask, int t) {
      constexpr bool M = decltype(with_mask)::value;
      const int kb = qb_hi - t;
      if constexpr (M) {
        win_qk(cur, 1, qf, sb, lane);
        over |= softmax_step<1>(sa, sf, pb, p.c);
        win_pv(cur, 0, pb, acc, lane);
        mask(sb, kb * 64 + 32);
      } else {
        over |= win_step(cur, 1, cur, 0, qf, sa, sb, sf, acc, p.c, lane,
                         [](int) {});
      }
      wait_vm_all();
      __syncthreads();  // tile t+1 resident; spare (tile t-1) free
      const bool pf = t + 2 < nt;
      if constexpr (M) {
        if (pf) win_issue(p, g, kb - 2, spare, off, wave, lane);
        win_qk(nxt, 0, qf, sa, lane);
        over |= softmax_step<1>(sb, sf, pb, p.c);
        win_pv(cur, 1, pb, acc, lane);
        mask(sa, (kb - 1) * 64);
      } else {
        // Tile t+2's loads ride along with this step's MFMA groups, one per
        // group (a prefetched tile is below the top one, so never ragged).
        // Past the last tile they re-read tile t into the spare stage, which
        // is then never read, so the issue needs no branch.
        const char *kt, *vt;
        win_tile_src(p, g, pf ? kb - 2 : kb, kt, vt);
        over |= win_step(nxt, 0, cur, 1, qf, sb, sa, sf, acc, p.c, lane,
                         [&](int j) {
                           win_issue_one(kt, vt, spare, off, wave, j);
                         });
      }
      char* const done = cur;
      cur = nxt;
      nxt = spare;
      spare = done;
    };
    // Tiles clean for every wave of the workgroup: below the lowest query
    // block's diagonal and above the highest query block's window edge.
    const int edge = qb_hi * 64 + 63 - w;
    const int kc_lo = edge < 0 ? 0 : (edge >> 6) + 1;
    const int t_a = min(qb_hi - qb_lo + 1, nt - 1);
    const int t_b = min(max(qb_hi - kc_lo, t_a), nt - 1);
    int t = 0;
    for (; t < t_a; ++t) iter(std::true_type{}, t);
    for (; t < t_b; ++t) iter(std::false_type{}, t);
    for (; t < nt - 1; ++t) iter(std::true_type{}, t);
    win_qk(cur, 1, qf, sb, lane);
    over |= softmax_step<1>(sa, sf, pb, p.c);
    win_pv(cur, 0, pb, acc, lane);
    mask(sb, kt_lo * 64 + 32);
    over |= softmax_step<1>(sb, sf, pb, p.c);
    win_pv(cur, 1, pb, acc, lane);
    wait_vm_all();  // no load may still be writing the ring
    if (attempt > 0) break;  // exact references: nothing can overflow
    if (__any(over)) over_flag = 1;
    __syncthreads();  // also: every wave is done with the LDS ring
    if (!over_flag) break;
    // Rare: some score lies far above its row's reference. Find every row's
    // true maximum over the same tiles, then recompute with it.
    sf.mref[0] = sf.mref[1] = -INFINITY;
#pragma unroll 1
    for (int t = 0; t < nt; ++t) {
      win_issue(p, g, qb_hi - t, smem, off, wave, lane);
      wait_vm_all();
      __syncthreads();
#pragma unroll 1
      for (int st = 0; st < 2; ++st) {
        win_qk(smem, st, qf, sa, lane);
        mask(sa, (qb_hi - t) * 64 + 32 * st);
        raise_refs<1>(sa, sf);
      }
      __syncthreads();
    }
  }
  if (active) store_out(acc, sf, p.c, p.out, p.lse, head, q0, p.S, lane);
}

// =====================================================================
// Sparse kernel
// =====================================================================
constexpr int VHALF_B = 8192;  // V^T of 32 keys: 128 d x 64 B
constexpr int KHALF_B = 8192;  // K of 32 keys: 32 rows x 256 B
// per wave: a ring of 2 K and 3 V^T half tiles (4 waves: 160 KiB of LDS)
constexpr int SP_WAVE_B = 2 * KHALF_B + 3 * VHALF_B;

struct SparseParams {
  const u16* q; const u16* k; const u16* vt; u16* out; float* lse;
  const int32_t* sel; const int32_t* sel_cnt;
  int sel_stride, S, S_pad, n_b, G, n_ret, n_jobs;
  float c;
  // Retrieval heads are numbered in ascending head order, so those of one KV
  // group are consecutive: group slot i holds rho in [rho_begin[i],
  // rho_begin[i+1]) (only groups with retrieval heads get a slot).
  int n_grp;
  int16_t rho_begin[kMaxHeads + 1];
  uint8_t head_of_rho[kMaxHeads];
};

// V^T half tile (32 keys): row d x 4 chunks of 16 B, chunk c at
// c ^ ((d >> 2) & 3), so the 16 rows that 16 consecutive lanes read hit 16
// distinct bank groups. Load ins (0..7) covers rows 16 ins .. 16 ins + 15;
// the lane part of the global offset is the same for every load and tile.
__device__ __forceinline__ uint32_t sp_v_lane_off(int lane) {
  const int c = (lane & 3) ^ ((lane >> 4) & 3);
  return (uint32_t)((lane >> 2) * 128 + c * 16);
}

// vbase: the KV group's first V^T block; k0: first key of the half tile
__device__ __forceinline__ void sp_issue_v(const u16* vbase, int k0,
                                           uint32_t voff, char* slot) {
  const char* vb = reinterpret_cast<const char*>(
                       vbase + (size_t)(k0 >> 6) * 64 * kD) + (k0 & 63) * 2;
#pragma unroll
  for (int ins = 0; ins < 8; ++ins)
    dma16(vb + ins * 16 * 128 + voff, slot + ins * 1024);
}

// s_waitcnt vmcnt(24), other counters at their maximum (gfx9 encoding)
__device__ __forceinline__ void wait_vm24() {
  __builtin_amdgcn_s_waitcnt((24 & 15) | (7 << 4) | (15 << 8) | ((24 >> 4) << 14));
}

// K half tile (32 keys) in LDS: row r = key r, 16 chunks of 16 B, chunk c at
// position c ^ (r & 15) (16 consecutive lanes of an operand read then hit 16
// distinct bank groups). DMA ins (0..7), lane i fills position i & 15 of row
// 4 ins + i / 16; its global offset inside the half tile repeats every 4
// loads (+4 KiB), so 4 per-lane offsets cover all 8.
__device__ __forceinline__ void sp_k_lane_offs(int lane, uint32_t (&o)[4]) {
#pragma unroll
  for (int ins = 0; ins < 4; ++ins) {
    const int r = 4 * ins + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    o[ins] = (uint32_t)(r * 256 + c * 16);
  }
}

__device__ __attribute__((noinline)) void sp_issue_k_ragged(
    const u16* kbase, int S, int k0, char* slot, int lane) {
  for (int ins = 0; ins < 8; ++ins) {
    const int r = 4 * ins + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const int key = k0 + r < S ? k0 + r : S - 1;  // rows past S: masked
    dma16(kbase + (size_t)key * kD + c * 8, slot + ins * 1024);
  }
}

__device__ __forceinline__ void sp_issue_k(const u16* kbase, int S, int k0,
                                           const uint32_t (&o)[4], char* slot,
                                           int lane) {
  if (k0 + 32 > S) {
    sp_issue_k_ragged(kbase, S, k0, slot, lane);
    return;
  }
  const char* kb = reinterpret_cast<const char*>(kbase + (size_t)k0 * kD);
#pragma unroll
  for (int ins = 0; ins < 8; ++ins)
    dma16(kb + (ins >> 2) * 4096 + o[ins & 3], slot + ins * 1024);
}

__global__ __launch_bounds__(256, 1) void attn_sparse_kernel(const SparseParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[4 * SP_WAVE_B];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int job = 4 * blockIdx.x + wave;
  if (job >= p.n_jobs) return;  // waves are independent: no block barriers
  // Jobs run KV-group by KV-group (query blocks descending, the group's
  // heads interleaved), so the jobs in flight gather from one group's K/V
  // and share its frequently chosen blocks (sink, recent and strongly
  // scored ones) in L2.
  int gs = 0;
  while (job >= p.n_b * p.rho_begin[gs + 1]) ++gs;
  const int r0 = p.rho_begin[gs], nr = p.rho_begin[gs + 1] - r0;
  const int jj = job - p.n_b * r0;
  const int rho = r0 + jj % nr;
  const int qb = p.n_b - 1 - jj / nr;
  const int head = p.head_of_rho[rho];
  const int g = head / p.G;
  const int q0 = qb * 64;
  const int S = p.S;
  // The list is read-only here: reading it through the constant address
  // space lets the compiler use scalar loads, which leave vmcnt (the K/V
  // prefetch accounting) alone.
  typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
  const const_i32_ptr list =
      (const_i32_ptr)(p.sel + ((size_t)rho * p.n_b + qb) * p.sel_stride);
  int cnt = __builtin_amdgcn_readfirstlane(p.sel_cnt[(size_t)rho * p.n_b + qb]);
  cnt = cnt < 0 ? 0 : (cnt > p.sel_stride ? p.sel_stride : cnt);
  const int nt = 2 * cnt;  // 32-key half tiles (even)
  char* const kslots = smem + wave * SP_WAVE_B;
  char* const vslots = kslots + 2 * KHALF_B;
  const u16* kbase = p.k + (size_t)g * S * kD;
  const u16* vbase = p.vt + (size_t)g * p.n_b * 64 * kD;
  // Half tile t: blocks from the last (the diagonal) to the first, halves
  // ascending, so the first half tile holds every query's own key and sets
  // the reference. Indices past the end re-read the last half tile, so every
  // step issues the same loads (fixed wait counts); those are never used.
  auto tile_k0 = [&](int t) -> int {
    t = t < nt ? t : nt - 1;
    int kb = list[__builtin_amdgcn_readfirstlane(cnt - 1 - (t >> 1))];
    kb = kb < 0 ? 0 : (kb > qb ? qb : kb);  // memory-safe on bad input
    return kb * 64 + 32 * (t & 1);
  };
  // only half tiles of the diagonal block straddle the causal edge
  auto mask = [&](f32x16 (&sc)[1][2], int k0) {
    if (k0 + 31 > q0) mask_sub(sc[0], k0, q0, 1 << 30, lane);
  };
  uint32_t koffs[4];
  sp_k_lane_offs(lane, koffs);
  const uint32_t voff = sp_v_lane_off(lane);
  // this lane's operand rows: K row perm_row(n) (chunk 2 ks + g, swizzled),
  // V^T row 32 mt + n (chunk 2 h + g, swizzled)
  const int g2 = lane >> 5, n32 = lane & 31;
  const int kr_row = perm_row(n32);
  auto kop_at = [=](const char* slot) {
    return [=](int ks) {
      const int c = (2 * ks + g2) ^ (kr_row & 15);
      return *reinterpret_cast<const bf16x8*>(slot + kr_row * 256 + c * 16);
    };
  };
  auto vop_at = [=](const char* slot) {
    return [=](int h, int mt) {
      const int d = 32 * mt + n32;
      const int c = (2 * h + g2) ^ ((d >> 2) & 3);
      return *reinterpret_cast<const bf16x8*>(slot + d * 64 + c * 16);
    };
  };

  bf16x8 qf[2][8];
  load_q(p.q, head, q0, S, qf, lane);
  f32x16 acc[2][4];
  zero_acc(acc);
  Soft sf;
  sf.mref[0] = sf.mref[1] = -INFINITY;
  sf.lsum[0] = sf.lsum[1] = 0.f;
  if (nt == 0) {
    store_out(acc, sf, p.c, p.out, p.lse, head, q0, S, lane);
    return;
  }
  auto qk_lds = [&](const char* slot, f32x16 (&sc)[1][2]) {
    const auto kop = kop_at(slot);
    f32x16 z = {};
    sc[0][0] = z;
    sc[0][1] = z;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 a = kop(ks);
      sc[0][0] = mfma32(a, qf[0][ks], sc[0][0]);
      sc[0][1] = mfma32(a, qf[1][ks], sc[0][1]);
    }
  };

  // K of half tile t lives in K slot t % 2, V^T in V slot t % 3, both
  // staged by LDS DMA; every step issues one half tile (8 + 8 loads), three
  // ahead of the half tile whose P.V it runs.
  f32x16 sa[1][2], sb[1][2];
  for (int attempt = 0;; ++attempt) {
    const int k0_0 = tile_k0(0), k0_1 = tile_k0(1), k0_2 = tile_k0(2);
    sp_issue_k(kbase, S, k0_0, koffs, kslots, lane);
    sp_issue_v(vbase, k0_0, voff, vslots);
    sp_issue_k(kbase, S, k0_1, koffs, kslots + KHALF_B, lane);
    sp_issue_v(vbase, k0_1, voff, vslots + VHALF_B);
    wait_vm24();  // K(0) resident
    qk_lds(kslots, sa);
    mask(sa, k0_0);
    if (attempt == 0) raise_refs<1>(sa, sf);
    wait_lgkm0();  // reads of K slot 0 done
    sp_issue_k(kbase, S, k0_2, koffs, kslots, lane);
    sp_issue_v(vbase, k0_2, voff, vslots + 2 * VHALF_B);
    char* vcur = vslots;  // V slot of the current half tile t
    char* vn1 = vslots + VHALF_B;
    char* vn2 = vslots + 2 * VHALF_B;
    bool over = false;
    // step t: S(t) in sc -> P.V with V^T(t); QK(t+1) from K slot (t+1) % 2
    // -> sn; then the loads of half tile t+3 (K into that K slot, V^T into
    // t's V slot)
    auto step = [&](int t, char* kslot, f32x16 (&sc)[1][2],
                    f32x16 (&sn)[1][2]) {
      wait_vm24();  // K(t+1) and V^T(t) resident
      over |= attn_step(kop_at(kslot), vop_at(vcur), [](int) {}, qf, sc, sn,
                        sf, acc, p.c);
      const int k0f = tile_k0(t + 3);
      wait_lgkm0();  // this wave's reads of both slots are done
      sp_issue_k(kbase, S, k0f, koffs, kslot, lane);
      sp_issue_v(vbase, k0f, voff, vcur);
      char* const done = vcur;
      vcur = vn1;
      vn1 = vn2;
      vn2 = done;
    };
    // Rows are strictly ascending, so only the first block processed can be
    // the diagonal one: step 0 masks S(1), later steps need no masks.
    step(0, kslots + KHALF_B, sa, sb);
    mask(sb, k0_1);
    for (int t = 1; t + 1 < nt; t += 2) {
      step(t, kslots, sb, sa);
      step(t + 1, kslots + KHALF_B, sa, sb);
    }
    step(nt - 1, kslots, sb, sa);
    wait_vm_all();  // no DMA may still target this wave's LDS slots
    if (attempt > 0 || !__any(over)) break;
    // Rare: a score far above its row's reference. Find every row's true
    // maximum over the kept keys, then recompute with it.
#pragma unroll 1
    for (int t = 0; t < nt; ++t) {
      const int k0 = tile_k0(t);
      sp_issue_k(kbase, S, k0, koffs, kslots, lane);
      wait_vm_all();
      qk_lds(kslots, sa);
      mask(sa, k0);
      raise_refs<1>(sa, sf);
      wait_lgkm0();
    }
    zero_acc(acc);
    sf.lsum[0] = sf.lsum[1] = 0.f;
  }
  store_out(acc, sf, p.c, p.out, p.lse, head, q0, S, lane);
}

// =====================================================================
// V transpose: V [Hkv,S,128] -> V^T in 64-key blocks [Hkv][n_b][128][64]
// (zero beyond S), so every key block's V^T is one contiguous 16 KiB read
// =====================================================================
constexpr int TSTR = 136;
__global__ __launch_bounds__(256) void transpose_v_kernel(
    const u16* __restrict__ v, u16* __restrict__ vt, int S, int S_pad) {
  __shared__ __attribute__((aligned(16))) u16 t[64 * TSTR];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const u16* src = v + (size_t)g * S * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 4, ch = c & 15;
    const int key = kb * 64 + row;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (key < S) x = *reinterpret_cast<const uint4*>(src + (size_t)key * kD + ch * 8);
    *reinterpret_cast<uint4*>(t + row * TSTR + ch * 8) = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, dr = c >> 3, kc = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[(kc * 8 + 2 * e) * TSTR + dr] |
             ((uint32_t)t[(kc * 8 + 2 * e + 1) * TSTR + dr] << 16);
    *reinterpret_cast<uint4*>(
        vt + (((size_t)g * (S_pad / 64) + kb) * kD + dr) * 64 + kc * 8) =
        make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_transpose_v(const u16* v, u16* vt, int Hkv, int S, int S_pad,
                              hipStream_t st) {
  if (S_pad == 0) return hipSuccess;
  dim3 grid(S_pad / 64, Hkv);
  prof_begin("transpose_v", st);
  hipLaunchKernelGGL(transpose_v_kernel, grid, dim3(256), 0, st, v, vt, S, S_pad);
  prof_end(st);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnLaunch& a, const uint8_t* is_ret,
                            hipStream_t st, int parts) {
  if (a.n_b == 0) return hipSuccess;
  const int Hq = a.G * a.Hkv;
  const float c = a.scale * 1.4426950408889634f;
  // window heads
  WinParams wp;
  wp.q = a.q; wp.k = a.k; wp.vt = a.vt; wp.out = a.out; wp.lse = a.lse;
  wp.S = a.S; wp.S_pad = a.S_pad; wp.n_b = a.n_b; wp.Hkv = a.Hkv;
  wp.c = c;
  auto win_of = [&](int h) { return a.head_window ? a.head_window[h] : a.window; };
  // packs: per KV head, its window heads grouped by window size (first
  // appearance order)
  int nl = 0, n_items = 0, np = 0;
  for (int g = 0; g < a.Hkv; ++g) {
    bool taken[kMaxHeads] = {};
    for (int h0 = g * a.G; h0 < (g + 1) * a.G; ++h0) {
      if ((is_ret && is_ret[h0]) || taken[h0]) continue;
      const int w0 = win_of(h0);
      wp.hoff[np] = (int16_t)nl;
      wp.item_off[np] = n_items;
      wp.pack_kv[np] = (uint8_t)g;
      wp.pack_win[np] = w0;
      int cnt = 0;
      for (int h = h0; h < (g + 1) * a.G; ++h)
        if (!(is_ret && is_ret[h]) && !taken[h] && win_of(h) == w0) {
          taken[h] = true;
          wp.hlist[nl++] = (uint8_t)h;
          ++cnt;
        }
      n_items += (cnt * a.n_b + 3) / 4;
      ++np;
    }
  }
  wp.hoff[np] = (int16_t)nl;
  wp.item_off[np] = n_items;
  for (int i = np; i < kMaxHeads; ++i) {
    wp.pack_kv[i] = 0;
    wp.pack_win[i] = 1;
    wp.hoff[i + 1] = (int16_t)nl;
    wp.item_off[i + 1] = n_items;
  }
  for (int i = nl; i < kMaxHeads; ++i) wp.hlist[i] = 0;
  wp.n_items = n_items;
  // cost-balanced contiguous item ranges per XCD (the tile count of an item
  // follows the kernel's own range computation)
  {
    auto item_cost = [&](int pk, int ig) -> int64_t {
      const int w = wp.pack_win[pk];
      const int nsw = wp.hoff[pk + 1] - wp.hoff[pk];
      const int njobs = nsw * a.n_b;
      const int qb_hi = a.n_b - 1 - (4 * ig) / nsw;
      const int qb_lo = a.n_b - 1 - min(4 * ig + 3, njobs - 1) / nsw;
      const int64_t lo = (int64_t)qb_lo * 64 - w + 1;
      const int64_t kt_lo = lo > 0 ? (lo >> 6) : 0;
      return (qb_hi - kt_lo + 1) + 9;  // + per-item prologue/epilogue
    };
    int64_t total = 0;
    for (int pk = 0; pk < np; ++pk)
      for (int ig = 0; ig < wp.item_off[pk + 1] - wp.item_off[pk]; ++ig)
        total += item_cost(pk, ig);
    int x = 0, item = 0;
    int64_t run = 0;
    wp.xcd_begin[0] = 0;
    for (int pk = 0; pk < np; ++pk)
      for (int ig = 0; ig < wp.item_off[pk + 1] - wp.item_off[pk]; ++ig, ++item) {
        run += item_cost(pk, ig);
        while (x + 1 < kXcds && run * kXcds >= total * (x + 1))
          wp.xcd_begin[++x] = item + 1;
      }
    while (x < kXcds) wp.xcd_begin[++x] = n_items;
    int longest = 0;
    for (int i = 0; i < kXcds; ++i)
      longest = max(longest, wp.xcd_begin[i + 1] - wp.xcd_begin[i]);
    wp.per_xcd = longest;
  }
  if (nl > 0 && (parts & kAttnWindow)) {
    prof_begin("attn_window", st);
    hipLaunchKernelGGL(attn_window_kernel, dim3(wp.per_xcd * kXcds), dim3(256),
                       0, st, wp);
    prof_end(st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // retrieval heads
  if (!(parts & kAttnSparse)) return hipSuccess;
  int n_ret = 0;
  SparseParams sp;
  for (int h = 0; h < Hq; ++h)
    if (is_ret && is_ret[h]) sp.head_of_rho[n_ret++] = (uint8_t)h;
  if (n_ret == 0) return hipSuccess;
  for (int i = n_ret; i < kMaxHeads; ++i) sp.head_of_rho[i] = 0;
  sp.n_grp = 0;
  for (int rho = 0; rho < n_ret; ++rho)
    if (rho == 0 || sp.head_of_rho[rho] / a.G != sp.head_of_rho[rho - 1] / a.G)
      sp.rho_begin[sp.n_grp++] = (int16_t)rho;
  for (int i = sp.n_grp; i <= kMaxHeads; ++i) sp.rho_begin[i] = (int16_t)n_ret;
  sp.q = a.q; sp.k = a.k; sp.vt = a.vt; sp.out = a.out; sp.lse = a.lse;
  sp.sel = a.sel; sp.sel_cnt = a.sel_cnt; sp.sel_stride = a.sel_stride;
  sp.S = a.S; sp.S_pad = a.S_pad; sp.n_b = a.n_b; sp.G = a.G;
  sp.n_ret = n_ret;
  sp.n_jobs = n_ret * a.n_b;
  sp.c = c;
  prof_begin("attn_sparse", st);
  hipLaunchKernelGGL(attn_sparse_kernel, dim3((sp.n_jobs + 3) / 4), dim3(256), 0,
                     st, sp);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace rtp
