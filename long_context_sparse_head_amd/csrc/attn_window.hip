// Sliding-window / dense causal attention kernel for gfx950 (window heads,
// and retrieval heads in full mode). The softmax core and the interleaved
// step are in attn_core.h.
//
// 4 waves = 4 (head, query block) jobs of one KV group share one stream of
// 64-key tiles, staged by direct global->LDS loads (global_load_lds_dwordx4)
// into a 3-deep LDS ring of padded rows; a tile's loads are dealt one per MFMA
// group of a step, not issued in one burst. Each XCD takes a contiguous, equal
// share of all KV groups' work items.
//
// This file is compiled with the backend option that prefers the VGPR form
// of MFMA results: the score accumulators then land in VGPRs, where the
// softmax reads them, instead of in AGPRs that need a copy per value.
#include <type_traits>

#include "attn_core.h"

namespace rtp {

// =====================================================================
// Window / dense kernel
// =====================================================================
constexpr int WSTAGES = 3;
// Padded LDS rows (conflict-free for 8 consecutive rows, and every operand
// address of a lane is one base register plus an immediate offset).
constexpr int KROW_B = 272;                 // 256 B of K + 16 B pad
// V^T is staged as stored: a 64-key block in MFMA operand order, where each
// operand is one KiB read by the 64 lanes in order (conflict-free).
constexpr int KTILE_B = 64 * KROW_B;        // 17408
constexpr int VTILE_B = 64 * kD * 2;        // 16384
constexpr int STAGE_B = KTILE_B + VTILE_B;  // 33792
constexpr int K_DMA = KTILE_B / 1024;       // 17 loads of 1 KB
constexpr int V_DMA = VTILE_B / 1024;       // 16 loads of 1 KB
constexpr int DMA_PER_WAVE = (K_DMA + V_DMA + 3) / 4;  // 9
static_assert(K_DMA == 17 && V_DMA == 16 && DMA_PER_WAVE == 9,
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

// The 33 DMA loads of a tile (17 K, 16 V^T) are dealt round-robin to the 4
// waves. Load i writes LDS bytes [1024 i, 1024 i + 1024) of the stage (K rows
// first, then the V^T block); a lane's 16-byte K unit either holds data or is
// a pad unit (then it re-reads a neighbouring chunk). A lane's global byte offset
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
  return (uint32_t)((64 * (ld - K_DMA) + lane) * 16);  // V^T: as stored
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
  buf_dma16(buf_rsrc(p.k + (size_t)g * p.S * kD, (uint32_t)p.S * (kD * 2)),
            (uint32_t)key * (kD * 2) + c * 16, 0, stage + ld * 1024);
}

// Buffer descriptors of one KV head's K rows and V^T blocks; a tile's bytes
// start at kb * 16 KiB in both.
struct WinSrc {
  __amdgpu_buffer_rsrc_t k, v;
};
constexpr uint32_t kTileBytes = 64 * kD * 2;  // K rows or V^T of 64 keys
__device__ __forceinline__ WinSrc win_src(const WinParams& p, int g) {
  WinSrc r;
  r.k = buf_rsrc(p.k + (size_t)g * p.S * kD, (uint32_t)p.S * (kD * 2));
  r.v = buf_rsrc(p.vt + (size_t)g * p.n_b * 64 * kD,
                 (uint32_t)p.n_b * kTileBytes);
  return r;
}

// Load j (0..8) of this wave for a full tile: loads 0..3 are K rows, load 4 is
// K for wave 0 and V^T for the others, loads 5..8 are V^T. The stage has only
// 33 loads, so waves 1..3 repeat their load 7 as load 8 (same bytes, same
// place), which keeps the issue free of branches.
__device__ __forceinline__ void win_issue_one(const WinSrc& src, int kb,
                                              char* stage,
                                              const WinLaneOffsets& o,
                                              int wave, int j) {
  const uint32_t toff = (uint32_t)kb * kTileBytes;
  if (j < 4) {
    buf_dma16(src.k, o.off[j], toff, stage + wave * 1024 + j * 4096);
  } else if (j == 4) {
    buf_dma16(wave == 0 ? src.k : src.v, o.off[4], toff,
              stage + wave * 1024 + 4 * 4096);
  } else if (j < 8) {
    buf_dma16(src.v, o.off[j], toff, stage + wave * 1024 + j * 4096);
  } else {
    const int jj = wave == 0 ? 8 : 7;
    buf_dma16(src.v, o.off[jj], toff, stage + wave * 1024 + jj * 4096);
  }
}

// All loads of this wave for tile kb, back to back.
__device__ __forceinline__ void win_issue(const WinParams& p, const WinSrc& src,
                                          int g, int kb, char* stage,
                                          const WinLaneOffsets& o, int wave,
                                          int lane) {
  if ((kb + 1) * 64 > p.S) {  // last block of a ragged S: rows past S
#pragma unroll 1                // re-read row S-1 (masked anyway)
    for (int j = 0; j < DMA_PER_WAVE; ++j) {
      const int ld = wave + 4 * j;
      if (ld < K_DMA) win_issue_ragged_k(p, g, kb, stage, ld, lane);
      else if (ld < K_DMA + V_DMA)
        buf_dma16(src.v, o.off[j], (uint32_t)kb * kTileBytes,
                  stage + ld * 1024);
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < DMA_PER_WAVE; ++j)
    win_issue_one(src, kb, stage, o, wave, j);
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
  const char* base = stage + KTILE_B + st * 8192 + lane * 16;
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const bf16x8 a =
          *reinterpret_cast<const bf16x8*>(base + (ks * 4 + mt) * 1024);
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
  const char* vops = vst + KTILE_B + vh * 8192 + lane * 16;
  return attn_step<true>(
      [&](int ks) { return *reinterpret_cast<const bf16x8*>(krow + 32 * ks); },
      [&](int h, int mt) {
        return *reinterpret_cast<const bf16x8*>(vops + (h * 4 + mt) * 1024);
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
  const WinSrc src = win_src(p, g);

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
    win_issue(p, src, g, qb_hi, cur, off, wave, lane);
    if (nt > 1) win_issue(p, src, g, qb_hi - 1, nxt, off, wave, lane);
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
        over |= softmax_step<1, true>(sa, sf, pb, p.c);
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
        if (pf) win_issue(p, src, g, kb - 2, spare, off, wave, lane);
        win_qk(nxt, 0, qf, sa, lane);
        over |= softmax_step<1, true>(sb, sf, pb, p.c);
        win_pv(cur, 1, pb, acc, lane);
        mask(sa, (kb - 1) * 64);
      } else {
        // Tile t+2's loads ride along with this step's MFMA groups, one per
        // group (a prefetched tile is below the top one, so never ragged).
        // Past the last tile they re-read tile t into the spare stage, which
        // is then never read, so the issue needs no branch.
        const int kb_pf = pf ? kb - 2 : kb;
        over |= win_step(nxt, 0, cur, 1, qf, sb, sa, sf, acc, p.c, lane,
                         [&](int j) {
                           win_issue_one(src, kb_pf, spare, off, wave, j);
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
    over |= softmax_step<1, true>(sa, sf, pb, p.c);
    win_pv(cur, 0, pb, acc, lane);
    mask(sb, kt_lo * 64 + 32);
    over |= softmax_step<1, true>(sb, sf, pb, p.c);
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
      win_issue(p, src, g, qb_hi - t, smem, off, wave, lane);
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

hipError_t launch_window_heads(const AttnLaunch& a, const uint8_t* is_ret,
                               hipStream_t st) {
  if (a.n_b == 0) return hipSuccess;
  const float c = a.scale * 1.4426950408889634f;
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
  if (nl == 0) return hipSuccess;
  prof_begin("attn_window", st);
  hipLaunchKernelGGL(attn_window_kernel, dim3(wp.per_xcd * kXcds), dim3(256),
                     0, st, wp);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace rtp
