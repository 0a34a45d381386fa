// Block-sparse attention kernel for the retrieval heads on gfx950, the V
// transpose, and the attention launch. The softmax core and the interleaved
// step are in attn_core.h; the window kernel is in attn_window.hip.
//
// Each wave runs its own (retrieval head, query block) job over its block
// list in 32-key half tiles. K half tiles are staged per wave by LDS DMA;
// the V^T operands of a half tile are loaded straight into registers (V^T
// blocks are stored in MFMA operand order, one contiguous KiB per operand),
// four half tiles ahead of their P.V.
#include <type_traits>

#include "attn_core.h"

namespace rtp {

// =====================================================================
// Sparse kernel
// =====================================================================
constexpr int KHALF_B = 8192;  // K of 32 keys: 32 rows x 256 B
// per wave: a ring of 2 K half tiles (4 waves: 64 KiB of LDS)
constexpr int SP_WAVE_B = 2 * KHALF_B;

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
    __amdgpu_buffer_rsrc_t rk, int S, int k0, char* slot, int lane) {
  for (int ins = 0; ins < 8; ++ins) {
    const int r = 4 * ins + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const int key = k0 + r < S ? k0 + r : S - 1;  // rows past S: masked
    buf_dma16(rk, (uint32_t)key * (kD * 2) + c * 16, 0, slot + ins * 1024);
  }
}

// rk: buffer descriptor of the KV group's K rows
__device__ __forceinline__ void sp_issue_k(__amdgpu_buffer_rsrc_t rk, int S,
                                           int k0, const uint32_t (&o)[4],
                                           char* slot, int lane) {
  if (k0 + 32 > S) {
    sp_issue_k_ragged(rk, S, k0, slot, lane);
    return;
  }
  const uint32_t toff = (uint32_t)k0 * (kD * 2);
#pragma unroll
  for (int ins = 0; ins < 8; ++ins)
    buf_dma16(rk, (ins >> 2) * 4096 + o[ins & 3], toff, slot + ins * 1024);
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
  const int g = __builtin_amdgcn_readfirstlane(head / p.G);
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
  const __amdgpu_buffer_rsrc_t kbase =
      buf_rsrc(p.k + (size_t)g * S * kD, (uint32_t)S * (kD * 2));
  // this lane's 16 bytes of each V^T operand of the KV group's blocks
  const u16* const vblk = p.vt + (size_t)g * p.n_b * 64 * kD + lane * 8;
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
  // this lane's K operand row: perm_row(n) (chunk 2 ks + g, swizzled)
  const int g2 = lane >> 5, n32 = lane & 31;
  const int kr_row = perm_row(n32);
  auto kop_at = [=](const char* slot) {
    return [=](int ks) {
      const int c = (2 * ks + g2) ^ (kr_row & 15);
      return *reinterpret_cast<const bf16x8*>(slot + kr_row * 256 + c * 16);
    };
  };
  // the eight V^T operands (h = 0, 1; mt = 0..3, index 4 h + mt) of the
  // half tile starting at key k0
  auto load_v = [&](int k0, bf16x8 (&dst)[8]) {
    const u16* b = vblk + (size_t)(k0 >> 6) * (64 * kD) + ((k0 >> 5) & 1) * 4096;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      dst[i] = *reinterpret_cast<const bf16x8*>(b + i * 512);
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

  // K of half tile t lives in K slot t % 2 (LDS DMA, two half tiles ahead
  // of its QK), its V^T operands in register slot t % 4 (loaded four half
  // tiles ahead of its P.V). Issue order: V0 K0 V1 K1 V2, then K2 V3 after
  // the first QK, then step t issues K(t+3) and V(t+4) at its end, so
  // before step t everything up to K(t+1) has landed once at most 24 newer
  // loads remain (V(t+2), K(t+2), V(t+3)); V(t) is older than K(t+1).
  bf16x8 vr[4][8];
  f32x16 sa[1][2], sb[1][2];
  for (int attempt = 0;; ++attempt) {
    const int k0_0 = tile_k0(0), k0_1 = tile_k0(1);
    load_v(k0_0, vr[0]);
    sp_issue_k(kbase, S, k0_0, koffs, kslots, lane);
    load_v(k0_1, vr[1]);
    sp_issue_k(kbase, S, k0_1, koffs, kslots + KHALF_B, lane);
    load_v(tile_k0(2), vr[2]);
    wait_vm24();  // K(0) resident
    qk_lds(kslots, sa);
    mask(sa, k0_0);
    if (attempt == 0) raise_refs<1>(sa, sf);
    wait_lgkm0();  // reads of K slot 0 done
    sp_issue_k(kbase, S, tile_k0(2), koffs, kslots, lane);
    load_v(tile_k0(3), vr[3]);
    bool over = false;
    // step t: S(t) in sc -> P.V with V^T(t) (registers, slot t % 4); QK(t+1)
    // from K slot (t+1) % 2 -> sn; then K(t+3) into that K slot and V^T(t+4)
    // into register slot t % 4
    auto step = [&](auto ring, int t, f32x16 (&sc)[1][2],
                    f32x16 (&sn)[1][2]) {
      constexpr int R = decltype(ring)::value;
      char* const kslot = kslots + ((R + 1) & 1) * KHALF_B;
      wait_vm24();  // K(t+1) resident, and V^T(t) before it
      over |= attn_step<false>(
          kop_at(kslot), [&](int h, int mt) { return vr[R][4 * h + mt]; },
          [](int) {}, qf, sc, sn, sf, acc, p.c);
      const int k0k = tile_k0(t + 3), k0v = tile_k0(t + 4);
      wait_lgkm0();  // this wave's reads of the K slot are done
      sp_issue_k(kbase, S, k0k, koffs, kslot, lane);
      load_v(k0v, vr[R]);
    };
    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    using R2 = std::integral_constant<int, 2>;
    using R3 = std::integral_constant<int, 3>;
    // Rows are strictly ascending, so only the first block processed can be
    // the diagonal one: step 0 masks S(1), later steps need no masks.
    step(R0{}, 0, sa, sb);
    mask(sb, k0_1);
    int t = 1;
    for (; t + 4 <= nt; t += 4) {
      step(R1{}, t, sb, sa);
      step(R2{}, t + 1, sa, sb);
      step(R3{}, t + 2, sb, sa);
      step(R0{}, t + 3, sa, sb);
    }
    // nt is even, so 1 or 3 steps remain
    step(R1{}, t, sb, sa);
    if (t + 1 < nt) {
      step(R2{}, t + 1, sa, sb);
      step(R3{}, t + 2, sb, sa);
    }
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
// V transpose: V [Hkv,S,128] -> V^T in 64-key blocks of 16 KiB (zero
// beyond S), each block in MFMA operand order: unit u = ((hf * 2 + h) * 4 +
// mt) * 64 + 32 g + n (16 bytes) holds V[32 hf + 16 h + 8 g + e][32 mt + n],
// e = 0..7, the A operand of P.V for d 32 mt .. 32 mt + 31 and keys
// 32 hf + 16 h .. + 15. So one 32-key half tile's eight operands are eight
// contiguous KiB, and a lane's part of each is one 16-byte load.
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
  u16* dst = vt + ((size_t)g * (S_pad / 64) + kb) * (64 * kD);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int u = tid + 256 * i;  // consecutive threads: consecutive units
    const int n = u & 31, gg = (u >> 5) & 1, mt = (u >> 6) & 3;
    const int key0 = 16 * (u >> 8) + 8 * gg;  // 32 hf + 16 h + 8 g
    const int d = 32 * mt + n;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[(key0 + 2 * e) * TSTR + d] |
             ((uint32_t)t[(key0 + 2 * e + 1) * TSTR + d] << 16);
    *reinterpret_cast<uint4*>(dst + u * 8) = make_uint4(w[0], w[1], w[2], w[3]);
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
  if (parts & kAttnWindow) {
    hipError_t e = launch_window_heads(a, is_ret, st);
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
