// Retrieval-head indexer for gfx950: low-rank projection, and block scoring
// fused with the per-query-block top-k selection.
//
// What it computes (RTPurboV2 article, paragraph on the low-rank projector
// that maps the head dimension to r = 16; aitop.news summary of "Full
// Attention Strikes Back": a 16-dimensional indexer guesses which earlier
// tokens matter). This library's block rule:
//     k^_j   = P_k k_j                                  (every key)
//     q-_qb  = P_q mean_{i in qb} q_i                   (per query block; equal
//              to the mean of the projected queries by linearity)
//     sc(qb, kb) = max_{j in kb} q-_qb . k^_j           (1 <= kb <= qb-1)
//     Sel(qb) = {0} u top_k(sc(qb, .)) u {qb}           (ties: lower kb)
//
// Selection must agree with an fp32 computation except at near-ties, so the
// K = r contraction of the scores runs on bf16 MFMA with operands split into
// high and low bf16 parts (a = a_hi + a_lo): a.b ~ a_hi.b_hi + a_hi.b_lo +
// a_lo.b_hi, i.e. three MFMAs per tile (error ~1e-5 relative, well inside the
// 1e-4 tie band), instead of one fp32-VALU pass that would be ~5x slower.
//
// The RTPurboV2 article criticises fixed, materialised top-k budgets for
// their cost at long context; here the score rows are never written out.
// Each row's scores stream through a register of the lane that owns the row,
// and only the ones that can still enter its top k + 1 go to a small
// candidate buffer (see score_select_kernel). At 1M tokens that replaces
// 11.5 GiB of score rows by about 0.6 GB of buffers.
#include "common.h"
#include "proj.h"
#include "select.h"

namespace rtp {

struct ProjArgs {
  int S, n_b, r, n_ret;
  uint8_t head_of_rho[kMaxHeads];     // query head of retrieval index rho
  uint8_t grp_kvh[kMaxHeads];         // KV head of group slot j
  uint8_t grp_first[kMaxHeads + 1];   // retrieval indices of slot j:
                                      // grp_first[j] .. grp_first[j+1]-1
};

// k-th / (k+1)-th score slots are written as bit patterns: this file is
// built without NaN semantics, and an absent score is a quiet NaN.
constexpr uint32_t kQuietNaN = 0x7fc00000u;
__device__ __forceinline__ uint32_t order_key_bits(uint32_t key) {
  return (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
}
__device__ __forceinline__ void put_score(float* kth, size_t i, bool have,
                                          uint32_t key) {
  reinterpret_cast<uint32_t*>(kth)[i] = have ? order_key_bits(key) : kQuietNaN;
}

// Projected keys in the A-operand order of the scoring MFMA: for head rho
// and key block kb, 4*R16 chunks of 1 KiB; chunk ((mt*2 + part)*R16 + rs)
// holds, at 16-byte slot L (0..63), the 8 values
//     k^[64 kb + 32 mt + L%32][16 rs + 8 (L/32) + e], e = 0..7
// of the hi (part 0) or lo (part 1) bf16 part: exactly what lane L feeds to
// v_mfma_f32_32x32x16_bf16 for the 32-key tile mt, so every operand load is
// one contiguous 1 KiB read per wave.
__host__ __device__ inline size_t kop_block_elems(int r) { return 2048 * (r / 16); }

// ---- projection of keys: grid (ceil(n_b/4), groups), 4 waves, a wave per
// key block. The group's K is read once. The rows of P_k of the group's
// retrieval heads (r per head, heads in index order) are taken 32 at a
// time: each tile is staged in LDS as three bf16 parts and multiplied with
// the block's keys on the matrix cores (proj.h), which leaves each lane the
// eight consecutive projected values its slot of the operand layout holds.
// Optionally also the per-block centroids (mean of the projected keys over
// the block's tokens).
__global__ __launch_bounds__(256) void proj_keys_kernel(
    const u16* __restrict__ k, const float* __restrict__ p_k, const ProjArgs pa,
    u16* __restrict__ kop, float* __restrict__ cent) {
  __shared__ __attribute__((aligned(16))) char ptile[kProjTileB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kb = blockIdx.x * 4 + wave;
  const int j = blockIdx.y;
  const int S = pa.S, r = pa.r, n_b = pa.n_b;
  const int g = pa.grp_kvh[j];
  const bool kb_ok = kb < n_b;
  const int nvalid = kb_ok ? min(64, S - kb * 64) : 0;
  bf16x8 kbop[2][8];
  proj_keys_operands(k + ((size_t)g * S + (kb_ok ? (size_t)kb * 64 : 0)) * kD,
                     nvalid, kbop);
  const int rho0 = pa.grp_first[j];
  const int n_rows = (pa.grp_first[j + 1] - rho0) * r;
  const float* P = p_k + (size_t)rho0 * r * kD;
  const int R16 = r / 16, gq = lane >> 5, n = lane & 31;
  for (int m0 = 0; m0 < n_rows; m0 += 32) {
    __syncthreads();  // the previous tile is no longer read
    proj_stage(P, m0, n_rows, ptile);
    __syncthreads();
    if (!kb_ok) continue;
    f32x16 acc[2];
    proj_tile(ptile, kbop, acc);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int R = m0 + 16 * half;  // first row of this half (16 | r)
      if (R >= n_rows) break;
      const int rho = rho0 + R / r, rs = (R % r) / 16;
      float cs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) cs[e] = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = acc[mt][8 * half + e];
        if (kop) {
          uint32_t hw[4], lw[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const u16 h0 = f2bf(v[2 * e]), h1 = f2bf(v[2 * e + 1]);
            hw[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            lw[e] = pack_bf16x2(v[2 * e] - bf2f(h0), v[2 * e + 1] - bf2f(h1));
          }
          u16* kout = kop + ((size_t)rho * n_b + kb) * kop_block_elems(r);
          *reinterpret_cast<uint4*>(kout + (size_t)(((mt * 2 + 0) * R16 + rs) * 64 + lane) * 8) =
              make_uint4(hw[0], hw[1], hw[2], hw[3]);
          *reinterpret_cast<uint4*>(kout + (size_t)(((mt * 2 + 1) * R16 + rs) * 64 + lane) * 8) =
              make_uint4(lw[0], lw[1], lw[2], lw[3]);
        }
        if (cent) {  // keys past S project to 0
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            float x = v[e];
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) x += __shfl_xor(x, off);
            cs[e] += x;
          }
        }
      }
      if (cent && n == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          cent[((size_t)rho * n_b + kb) * r + 16 * rs + 8 * gq + e] = cs[e] / (float)nvalid;
      }
    }
  }
}

// ---- block means of queries, projected: grid (ceil(n_b/4), n_ret), 4
// waves, a wave per query block. Lane l reads 16 bytes (8 values of d) of
// rows 4i + l/16, i = 0..15: every load instruction reads 4 whole rows, and
// all 16 are in flight at once. Also clears the scoring kernel's work
// counter, so the two launches need nothing else between them.
__global__ __launch_bounds__(256) void proj_qmeans_kernel(
    const u16* __restrict__ q, const float* __restrict__ p_q, const ProjArgs pa,
    u16* __restrict__ qhi, u16* __restrict__ qlo, int* __restrict__ counter) {
  __shared__ float mean[4][kD];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qb = blockIdx.x * 4 + wave, rho = blockIdx.y;
  const int S = pa.S, r = pa.r, n_b = pa.n_b;
  if (counter && blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0)
    *counter = 0;
  if (qb < n_b) {
    const int h = pa.head_of_rho[rho];
    const int rows = min(64, S - qb * 64);
    const int c = lane & 15, s = lane >> 4;
    const u16* base = q + ((size_t)h * S + (size_t)qb * 64) * kD + 8 * c;
    uint4 w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 4 * i + s;
      w[i] = row < rows ? *reinterpret_cast<const uint4*>(base + (size_t)row * kD)
                        : make_uint4(0, 0, 0, 0);
    }
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t u[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[2 * e] += __uint_as_float(u[e] << 16);
        a[2 * e + 1] += __uint_as_float(u[e] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] += __shfl_xor(a[e], 16);
      a[e] += __shfl_xor(a[e], 32);
    }
    if (s == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) mean[wave][8 * c + e] = a[e] / (float)rows;
    }
  }
  __syncthreads();
  if (qb < n_b) {
    for (int rr = lane; rr < r; rr += 64) {
      const float4* prow =
          reinterpret_cast<const float4*>(p_q + ((size_t)rho * r + rr) * kD);
      float acc = 0.f;
#pragma unroll 8
      for (int d4 = 0; d4 < kD / 4; ++d4) {
        const float4 p = prow[d4];
        acc = fmaf(p.x, mean[wave][4 * d4], acc);
        acc = fmaf(p.y, mean[wave][4 * d4 + 1], acc);
        acc = fmaf(p.z, mean[wave][4 * d4 + 2], acc);
        acc = fmaf(p.w, mean[wave][4 * d4 + 3], acc);
      }
      const u16 hi = f2bf(acc);
      const size_t o = ((size_t)rho * n_b + qb) * r + rr;
      qhi[o] = hi;
      qlo[o] = f2bf(acc - bf2f(hi));
    }
  }
}

// ------------------------------------------- short sequences: score rows
// Up to kStreamMinBlocks key blocks (256K tokens) a head's score rows take at
// most 33.5 MB, and writing them out, then selecting each row in its own
// workgroup, keeps far more waves busy than one wave per 64 rows could: the
// rows are written as a lower triangle per head and the top k of each row
// found by the block-wide select. Longer sequences use the fused kernel
// below, whose memory does not grow with the square of the length.
// ---- block scores of short sequences (up to kStreamMinBlocks blocks):
// grid (ceil(n_b/128), ceil(n_b/KBC), n_ret), 4 waves.
// Workgroup = 128 query blocks (32 per wave, along the MFMA N dimension) x a
// chunk of KBC key blocks. Key blocks are staged in LDS KBI at a time (the
// 64 projected keys of each, hi and lo parts); each wave computes the 64 x 32
// dot products of a key block as two 32x32 tiles (keys along M) and
// max-pools its 64 keys. A stage is loaded into registers two stages ahead
// and written to LDS one stage ahead, so each global round trip is hidden
// behind two stages of MFMA work. The query tile is the fastest grid index,
// so the workgroups that share a key chunk run together and read it from
// L2. Scores are collected in LDS and written row by row, one contiguous run
// of up to KBC floats per row.
constexpr int KBC = 48;

template <int R16>
__global__ __launch_bounds__(256) void block_scores_kernel(
    const u16* __restrict__ kop, const u16* __restrict__ qhi,
    const u16* __restrict__ qlo, float* __restrict__ scores, int n_b) {
  constexpr int r = 16 * R16;
  constexpr int RS = r + 8;  // LDS row stride (bf16), 16-byte pad
  constexpr int KBI = R16 >= 4 ? 1 : 4 / R16;  // key blocks per stage
  static_assert(KBC % KBI == 0, "a chunk is whole stages");
  constexpr int SROWS = 64 * KBI;
  __shared__ __attribute__((aligned(16))) u16 st[2][2][SROWS * RS];
  __shared__ float scs[128][KBC + 1];
  const int qt = blockIdx.x, kc = blockIdx.y, rho = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const int qb0 = qt * 128;
  const int qb_last = min(qb0 + 127, n_b - 1);
  const int kb_begin = max(1, kc * KBC);
  const int kb_end = min((kc + 1) * KBC, qb_last);  // candidates kb < qb_last
  if (kb_begin >= kb_end) return;

  const int qb = qb0 + 32 * wave + n;
  const int wave_qmax = min(qb0 + 32 * wave + 31, n_b - 1);
  bf16x8 bh[R16], bl[R16];
#pragma unroll
  for (int rs = 0; rs < R16; ++rs) {
    bf16x8 z = {};
    bh[rs] = z;
    bl[rs] = z;
    if (qb < n_b) {
      const size_t o = ((size_t)rho * n_b + qb) * r + 16 * rs + 8 * g;
      bh[rs] = *reinterpret_cast<const bf16x8*>(qhi + o);
      bl[rs] = *reinterpret_cast<const bf16x8*>(qlo + o);
    }
  }
  const int64_t tri = tri_rows(n_b);
  float* srow_base = scores + (size_t)rho * tri;

  // a stage: SROWS rows x r bf16, hi and lo = SROWS * r / 4 chunks of 16 B
  constexpr int CH_PER_ROW = r / 8;
  constexpr int NCH = SROWS * CH_PER_ROW * 2;
  static_assert(NCH % 256 == 0, "whole chunks per thread");
  constexpr int PER_T = NCH / 256;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u16* kop_h = kop + (size_t)rho * n_b * kop_block_elems(r);
  const int nst = (kb_end - kb_begin + KBI - 1) / KBI;
  // key blocks past the chunk re-read its last block (never used)
  auto gload = [&](int stg, u32x4 (&reg)[PER_T]) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + 256 * i;
      const int part = c / (SROWS * CH_PER_ROW), cc = c % (SROWS * CH_PER_ROW);
      const int row = cc / CH_PER_ROW, ch = cc % CH_PER_ROW;
      const int kb = min(kb_begin + stg * KBI + row / 64, kb_end - 1);
      // (key m, values 8 ch .. 8 ch + 7) of block kb in the operand order
      const int m = row & 63;
      const int L = (m & 31) + 32 * (ch & 1);
      const u16* src = kop_h + (size_t)kb * kop_block_elems(r) +
                       ((((m >> 5) * 2 + part) * R16 + (ch >> 1)) * 64 + L) * 8;
      reg[i] = *reinterpret_cast<const u32x4*>(src);
    }
  };
  auto sstore = [&](int buf, const u32x4 (&reg)[PER_T]) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + 256 * i;
      const int part = c / (SROWS * CH_PER_ROW), cc = c % (SROWS * CH_PER_ROW);
      const int row = cc / CH_PER_ROW, ch = cc % CH_PER_ROW;
      *reinterpret_cast<u32x4*>(&st[buf][part][row * RS + ch * 8]) = reg[i];
    }
  };
  auto compute = [&](int stg, int buf) {
#pragma unroll
    for (int j = 0; j < KBI; ++j) {
      const int kb = kb_begin + stg * KBI + j;
      if (kb >= kb_end || kb >= wave_qmax) continue;  // wave-uniform
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 acc = {};
        const u16* ah = &st[buf][0][(64 * j + 32 * mt + n) * RS + 8 * g];
        const u16* al = &st[buf][1][(64 * j + 32 * mt + n) * RS + 8 * g];
#pragma unroll
        for (int rs = 0; rs < R16; ++rs) {
          const bf16x8 a_hi = *reinterpret_cast<const bf16x8*>(ah + 16 * rs);
          const bf16x8 a_lo = *reinterpret_cast<const bf16x8*>(al + 16 * rs);
          acc = mfma32(a_lo, bh[rs], acc);
          acc = mfma32(a_hi, bl[rs], acc);
          acc = mfma32(a_hi, bh[rs], acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[i]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (g == 0) scs[32 * wave + n][kb - kb_begin] = mx;
    }
  };

  // stage s sits in register set s % 2 until it is written to LDS buffer
  // s % 2; set (s + 2) % 2 is refilled as soon as stage s is in LDS
  u32x4 ra[PER_T], rb[PER_T];
  gload(0, ra);
  gload(min(1, nst - 1), rb);
  sstore(0, ra);
  __syncthreads();
  auto step = [&](int s, u32x4 (&cur)[PER_T], u32x4 (&nxt)[PER_T]) {
    // cur held stage s (already in LDS): refill it with stage s + 2
    gload(min(s + 2, nst - 1), cur);
    compute(s, s & 1);
    if (s + 1 < nst) sstore((s + 1) & 1, nxt);
    __syncthreads();
  };
  for (int s = 0; s < nst; s += 2) {
    step(s, ra, rb);
    if (s + 1 < nst) step(s + 1, rb, ra);
  }
  // write-out: row qb takes candidates kb_begin .. min(kb_end, qb) - 1
  for (int i = 0; i < 32; ++i) {
    const int row = 32 * wave + i, qbi = qb0 + row;
    if (qbi >= n_b) break;
    const int cnt = min(kb_end, qbi) - kb_begin;
    const int64_t off = qbi >= 2 ? (int64_t)(qbi - 2) * (qbi - 1) / 2 : 0;
    if (lane < cnt) srow_base[off + kb_begin + lane - 1] = scs[row][lane];
  }
}

// ---- top-k per (retrieval head, query block): grid (n_b, n_ret), 256 thr.
__global__ __launch_bounds__(256) void topk_kernel(
    const float* __restrict__ scores, int n_b, int top_k, int stride,
    int32_t* __restrict__ sel, int32_t* __restrict__ sel_cnt,
    float* __restrict__ kth) {
  // the row's keys (one pad word per 32): sized at launch for the longest
  // row, so short sequences keep several workgroups per CU
  extern __shared__ uint32_t keys[];
  __shared__ TopkShared sh;
  const int qb = blockIdx.x, rho = blockIdx.y, tid = threadIdx.x;
  const int n_c = max(qb - 1, 0);  // candidates 1 .. qb-1
  const size_t row_id = (size_t)rho * n_b + qb;
  int32_t* out = sel + row_id * stride;
  const float* row = scores + (size_t)rho * tri_rows(n_b) +
                     (qb >= 2 ? (int64_t)(qb - 2) * (qb - 1) / 2 : 0);
  uint32_t* kthb = reinterpret_cast<uint32_t*>(kth);

  if (n_c <= top_k || top_k == 0) {
    // keep every candidate, or none when top_k == 0
    const bool all = top_k > 0;
    for (int t = tid; t < stride; t += 256) {
      int v;
      if (all) v = t <= qb ? t : -1;
      else v = t == 0 ? 0 : ((t == 1 && qb >= 1) ? qb : -1);
      out[t] = v;
    }
    if (tid == 0) sel_cnt[row_id] = all ? qb + 1 : (qb >= 1 ? 2 : 1);
    if (kth) {
      // s_k exists iff 1 <= k <= n_c: here only k == n_c (the row minimum);
      // s_{k+1} exists iff k+1 <= n_c: here only k == 0 (the row maximum).
      uint32_t mn = 0xffffffffu, mx = 0u;
      for (int e = tid; e < n_c; e += 256) {
        const uint32_t kk = order_key(row[e]);
        mn = min(mn, kk);
        mx = max(mx, kk);
      }
      mn = block_min_u32(mn, sh.tmp);
      mx = block_max_u32(mx, sh.tmp);
      if (tid == 0) {  // absent scores are quiet NaNs, written as bits
        kthb[row_id * 2 + 0] = (top_k >= 1 && n_c == top_k) ? order_key_bits(mn) : kQuietNaN;
        kthb[row_id * 2 + 1] = (top_k == 0 && n_c >= 1) ? order_key_bits(mx) : kQuietNaN;
      }
    }
    return;
  }

  // 1 <= top_k < n_c
  const bool in_lds = n_c <= TK_LDS;
  if (in_lds) {
    // sixteen loads per thread in flight: a row of up to 4096 candidates
    // costs one memory round trip
    for (int e0 = tid; e0 < n_c; e0 += 16 * 256) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = row[min(e0 + 256 * u, n_c - 1)];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = e0 + 256 * u;
        if (e < n_c) keys[e + (e >> 5)] = order_key(v[u]);
      }
    }
    __syncthreads();
  }
  auto getk = [&](int e) -> uint32_t {
    return in_lds ? keys[e + (e >> 5)] : order_key(row[e]);
  };
  const TopkResult res = radix_topk(getk, n_c, top_k, out + 1, 1, sh);
  if (tid == 0) {
    out[0] = 0;
    out[top_k + 1] = qb;
    sel_cnt[row_id] = top_k + 2;
  }
  if (kth) {
    // (k+1)-th largest: T again if another key ties it, else the largest key
    // below T.
    uint32_t below = 0u;
    const int C = (n_c + 255) / 256;
    const int e0 = min(tid * C, n_c), e1 = min(e0 + C, n_c);
    for (int e = e0; e < e1; ++e) {
      const uint32_t key = getk(e);
      if (key < res.T) below = max(below, key);
    }
    below = block_max_u32(below, sh.tmp);
    const int count_ge = res.count_ge;
    if (tid == 0) {
      kthb[row_id * 2 + 0] = order_key_bits(res.T);
      kthb[row_id * 2 + 1] = order_key_bits(count_ge >= top_k + 1 ? res.T : below);
    }
  }
}

// ---------------------------------------------------------------- scoring
// Global-memory accesses of the scoring kernel go through address-space-1
// pointers, so they compile to global (not FLAT) instructions: a FLAT load
// also counts against the LDS wait counter, which would make every wait in
// the prefetch ring a full wait.
template <class T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem(T* p) {
  return (__attribute__((address_space(1))) T*)p;
}

// A candidate-buffer entry: (order key of the score, key block).
typedef uint32_t entry_t __attribute__((ext_vector_type(2)));

struct ScoreArgs {
  const u16* kop;               // projected keys, operand order
  const u16* qhi; const u16* qlo;
  entry_t* buf;                 // [4 n_wg][64][cap] (order key, block)
  int* counter;                 // next work item (cleared before launch)
  int32_t* sel; int32_t* sel_cnt; float* kth;
  int n_b, n_ret, top_k, cap, n_tiles, n_items;
};

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    v = min(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
    v = max(v, (uint32_t)__shfl_xor((int)v, off));
  return v;
}
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// Stores of one lane become visible to the other lanes of its wave (and
// workgroup) before the loads that follow.
__device__ __forceinline__ void fence_wg() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
}

__device__ __forceinline__ bool nan_key(uint32_t x) {
  return x > 0xff800000u || x < 0x007fffffu;
}

// Shrinks one row's candidate buffer rb[0..c) in place, in order, to a set
// that still holds the row's `need` best entries (order key descending, then
// lower position, i.e. lower block, first). Every entry removed is below
// every entry kept, so after it `thr` (returned) bounds what can still
// enter: a later block enters only with a key strictly above thr, because
// at least `need` kept entries are >= thr and come from lower blocks.
//
// Normally one histogram pass of the keys' values (256 bins between the
// row's minimum and maximum, as in the block-wide select) finds the bin
// holding the need-th best; everything from that bin up is kept and thr is
// the least kept key. When that frees fewer than 64 slots (many equal or
// crowded values), the exact need-th key T is found by radix select and
// exactly `need` entries are kept (those above T, then the first ones equal
// to T), with thr = T. One wave; returns the new count.
__device__ __forceinline__ int compact_row(entry_t* rb, int c, int need, int* hist,
                           uint32_t& thr) {
  const int lane = threadIdx.x & 63;
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int e = lane; e < c; e += 64) {
    const uint32_t x = rb[e].x;
    if (!nan_key(x)) {
      lo = min(lo, x);
      hi = max(hi, x);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  float flo = 0.f, scale = 0.f;
  if (lo <= hi) {
    flo = order_key_inv(lo);
    const float span = order_key_inv(hi) - flo;
    if (span > 0.f) scale = 255.99f / span;
    if (!(scale < 1e30f)) scale = 0.f;
  }
  auto bin = [&](uint32_t x) -> int {
    if (x > 0xff800000u) return 255;
    if (x < 0x007fffffu) return 0;
    float f = (order_key_inv(x) - flo) * scale;
    f = fminf(fmaxf(f, 0.f), 255.f);
    return (int)f;
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) hist[lane + 64 * j] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int e = lane; e < c; e += 64) atomicAdd(&hist[bin(rb[e].x)], 1);
  __builtin_amdgcn_wave_barrier();
  int h[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = hist[255 - 4 * lane - j];
    sum += h[j];
  }
  __builtin_amdgcn_wave_barrier();
  const int incl = wave_incl_scan(sum);
  const int excl = incl - sum;
  const bool mine = excl < need && need <= incl;
  int bstar = 0, kept = 0;
  if (mine) {
    int above = excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (above + h[j] >= need) {
        bstar = 255 - 4 * lane - j;
        kept = above + h[j];
        break;
      }
      above += h[j];
    }
  }
  const int src = (int)__builtin_ctzll(__ballot(mine));
  bstar = __shfl(bstar, src);
  kept = __shfl(kept, src);
  const bool exact = kept > c - 64;
  uint32_t T = 0u;
  int take_eq = 0;
  if (exact) {
    T = wave_kth([&](int i) { return rb[i].x; }, c, need, hist);
    int gt = 0;
    for (int e = lane; e < c; e += 64) gt += rb[e].x > T;
    take_eq = need - wave_sum(gt);
  }
  const uint64_t below = lanes_below();
  int w = 0, eq_seen = 0;
  uint32_t mn = 0xffffffffu;
  for (int e0 = 0; e0 < c; e0 += 64) {
    const int e = e0 + lane;
    const bool in = e < c;
    const entry_t v = in ? rb[e] : entry_t{0u, 0u};
    bool keep;
    if (exact) {
      const bool is_gt = in && v.x > T, is_eq = in && v.x == T;
      const uint64_t beq = __ballot(is_eq);
      keep = is_gt || (is_eq && eq_seen + __builtin_popcountll(beq & below) < take_eq);
      eq_seen += __builtin_popcountll(beq);
    } else {
      keep = in && bin(v.x) >= bstar;
    }
    const uint64_t bk = __ballot(keep);
    if (keep) {
      rb[w + __builtin_popcountll(bk & below)] = v;
      mn = min(mn, v.x);
    }
    w += __builtin_popcountll(bk);
  }
  thr = exact ? T : wave_min_u32(mn);
  return w;
}

// ---- the same two operations with the row held in registers (buffers of up
// to 64 * kRowRegs entries): one memory round trip per call instead of one
// per pass. Entry i of the row sits in slot i / 64 of lane i % 64.
constexpr int kRowRegs = 16;

struct RowRegs {
  uint32_t key[kRowRegs], kb[kRowRegs];
  int bn[kRowRegs];  // value bin of each entry (valid after row_bins)
  int c;
};

__device__ __forceinline__ void load_row(const entry_t* rb, int c, RowRegs& R) {
  const int lane = threadIdx.x & 63;
  R.c = c;
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) {
    const int i = lane + 64 * j;
    entry_t v = {0u, 0u};
    if (i < c) v = gmem(rb)[i];
    R.key[j] = v.x;
    R.kb[j] = v.y;
  }
}

// 256 bins of a linear quantisation of the entries' values between the
// row's least and greatest (non-NaN) value; NaN keys go to the end bins.
// Monotone: a greater value never lands in a lower bin.
__device__ __forceinline__ void row_bins(RowRegs& R) {
  const int lane = threadIdx.x & 63;
  uint32_t lo = 0xffffffffu, hi = 0u;
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) {
    const uint32_t x = R.key[j];
    if (lane + 64 * j < R.c && !nan_key(x)) {
      lo = min(lo, x);
      hi = max(hi, x);
    }
  }
  lo = wave_min_u32(lo);
  hi = wave_max_u32(hi);
  float flo = 0.f, scale = 0.f;
  if (lo <= hi) {
    flo = order_key_inv(lo);
    const float span = order_key_inv(hi) - flo;
    if (span > 0.f) scale = 255.99f / span;
    if (!(scale < 1e30f)) scale = 0.f;
  }
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) {
    const uint32_t x = R.key[j];
    int b;
    if (x > 0xff800000u) {
      b = 255;
    } else if (x < 0x007fffffu) {
      b = 0;
    } else {
      const float f = fminf(fmaxf((order_key_inv(x) - flo) * scale, 0.f), 255.f);
      b = min(max((int)f, 0), 255);
    }
    R.bn[j] = b;
  }
}

// The bin holding the rank-th best entry, the count of entries in higher
// bins and the count in that bin.
__device__ __forceinline__ void bin_threshold(const RowRegs& R, int rank,
                                              int* hist, int& bstar,
                                              int& above, int& nbin) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int j = 0; j < 4; ++j) hist[lane + 64 * j] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j)
    if (lane + 64 * j < R.c) atomicAdd(&hist[R.bn[j]], 1);
  __builtin_amdgcn_wave_barrier();
  int h[4], sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    h[j] = hist[255 - 4 * lane - j];
    sum += h[j];
  }
  __builtin_amdgcn_wave_barrier();
  const int incl = wave_incl_scan(sum);
  const int excl = incl - sum;
  const bool mine = excl < rank && rank <= incl;
  int b = 0, ab = 0, nb = 0;
  if (mine) {
    int run = excl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (run + h[j] >= rank) {
        b = 255 - 4 * lane - j;
        ab = run;
        nb = h[j];
        break;
      }
      run += h[j];
    }
  }
  const int src = (int)__builtin_ctzll(__ballot(mine));
  bstar = __shfl(b, src);
  above = __shfl(ab, src);
  nbin = __shfl(nb, src);
}

// The rank-th largest key among the entries of bin bstar (1 <= rank <= the
// bin's count): a 4-pass, 8-bit radix select over those entries only.
__device__ __forceinline__ uint32_t kth_in_bin(const RowRegs& R, int bstar, int rank,
                               int* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[lane + 64 * j] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < kRowRegs; ++j) {
      const uint32_t x = R.key[j];
      if (lane + 64 * j < R.c && R.bn[j] == bstar && (x & pmask) == prefix)
        atomicAdd(&hist[(x >> shift) & 255], 1);
    }
    __builtin_amdgcn_wave_barrier();
    int h[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = hist[255 - 4 * lane - j];
      sum += h[j];
    }
    __builtin_amdgcn_wave_barrier();
    const int incl = wave_incl_scan(sum);
    const int excl = incl - sum;
    const bool mine = excl < rank && rank <= incl;
    int digit = 0, run = excl;
    if (mine) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (run + h[j] >= rank) {
          digit = 255 - 4 * lane - j;
          break;
        }
        run += h[j];
      }
    }
    const int src = (int)__builtin_ctzll(__ballot(mine));
    digit = __shfl(digit, src);
    run = __shfl(run, src);
    prefix |= (uint32_t)digit << shift;
    pmask |= 0xffu << shift;
    rank -= run;
  }
  return prefix;
}

// compact_row for a row held in registers (same contract).
__device__ __forceinline__ int compact_regs(entry_t* rb, RowRegs& R, int need, int* hist,
                            uint32_t& thr) {
  const int lane = threadIdx.x & 63;
  row_bins(R);
  int bstar, above, nbin;
  bin_threshold(R, need, hist, bstar, above, nbin);
  const bool exact = above + nbin > R.c - 64;
  uint32_t T = 0u;
  int take_eq = 0;
  if (exact) {
    T = kth_in_bin(R, bstar, need - above, hist);
    int gt = 0;
#pragma unroll
    for (int j = 0; j < kRowRegs; ++j) gt += (lane + 64 * j < R.c) && R.key[j] > T;
    take_eq = need - wave_sum(gt);
  }
  const uint64_t below = lanes_below();
  int w = 0, eq_seen = 0;
  uint32_t mn = 0xffffffffu;
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) {
    if (64 * j >= R.c) break;  // wave-uniform
    const bool in = lane + 64 * j < R.c;
    const uint32_t x = R.key[j];
    bool keep;
    if (exact) {
      const bool is_gt = in && x > T, is_eq = in && x == T;
      const uint64_t beq = __ballot(is_eq);
      keep = is_gt || (is_eq && eq_seen + __builtin_popcountll(beq & below) < take_eq);
      eq_seen += __builtin_popcountll(beq);
    } else {
      keep = in && R.bn[j] >= bstar;
    }
    const uint64_t bk = __ballot(keep);
    if (keep) {
      gmem(rb)[w + __builtin_popcountll(bk & below)] = entry_t{x, R.kb[j]};
      mn = min(mn, x);
    }
    w += __builtin_popcountll(bk);
  }
  thr = exact ? T : wave_min_u32(mn);
  return w;
}

// finish_row for a row held in registers (same contract).
__device__ __forceinline__ void finish_regs(const ScoreArgs& a, RowRegs& R, int rho, int qb,
                            int* hist) {
  const int lane = threadIdx.x & 63;
  const int top_k = a.top_k, stride = top_k + 2;
  const int n_c = max(qb - 1, 0);
  const size_t row_id = (size_t)rho * a.n_b + qb;
  int32_t* out = a.sel + row_id * stride;
  if (n_c <= top_k || top_k == 0) {
    const bool all = top_k > 0;
    for (int t = lane; t < stride; t += 64) {
      int v;
      if (all) v = t <= qb ? t : -1;
      else v = t == 0 ? 0 : ((t == 1 && qb >= 1) ? qb : -1);
      out[t] = v;
    }
    if (lane == 0) a.sel_cnt[row_id] = all ? qb + 1 : (qb >= 1 ? 2 : 1);
    if (a.kth) {
      uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
      for (int j = 0; j < kRowRegs; ++j) {
        if (lane + 64 * j < R.c) {
          mn = min(mn, R.key[j]);
          mx = max(mx, R.key[j]);
        }
      }
      mn = wave_min_u32(mn);
      mx = wave_max_u32(mx);
      if (lane == 0) {
        put_score(a.kth, row_id * 2 + 0, top_k >= 1 && n_c == top_k, mn);
        put_score(a.kth, row_id * 2 + 1, top_k == 0 && n_c >= 1, mx);
      }
    }
    return;
  }
  // the k-th best key T, then every key above T and the first keys equal
  // to T, in block order
  row_bins(R);
  int bstar, above, nbin;
  bin_threshold(R, top_k, hist, bstar, above, nbin);
  const uint32_t T = kth_in_bin(R, bstar, top_k - above, hist);
  int gt = 0;
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) gt += (lane + 64 * j < R.c) && R.key[j] > T;
  const int take_eq = top_k - wave_sum(gt);
  const uint64_t below = lanes_below();
  int pos = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) {
    if (64 * j >= R.c) break;  // wave-uniform
    const bool in = lane + 64 * j < R.c;
    const uint32_t x = R.key[j];
    const bool is_gt = in && x > T, is_eq = in && x == T;
    const uint64_t beq = __ballot(is_eq);
    const bool t =
        is_gt || (is_eq && eq_seen + __builtin_popcountll(beq & below) < take_eq);
    const uint64_t bt = __ballot(t);
    if (t) out[1 + pos + __builtin_popcountll(bt & below)] = (int32_t)R.kb[j];
    pos += __builtin_popcountll(bt);
    eq_seen += __builtin_popcountll(beq);
  }
  if (lane == 0) {
    out[0] = 0;
    out[top_k + 1] = qb;
    a.sel_cnt[row_id] = top_k + 2;
  }
  if (a.kth) {
    int ge = 0;
    uint32_t bel = 0u;
#pragma unroll
    for (int j = 0; j < kRowRegs; ++j) {
      const uint32_t x = R.key[j];
      if (lane + 64 * j < R.c) {
        ge += x >= T;
        if (x < T) bel = max(bel, x);
      }
    }
    ge = wave_sum(ge);
    bel = wave_max_u32(bel);
    if (lane == 0) {
      put_score(a.kth, row_id * 2 + 0, true, T);
      put_score(a.kth, row_id * 2 + 1, true, ge >= top_k + 1 ? T : bel);
    }
  }
}

// Final choice of one row from its buffer rb[0..c) (which holds the row's
// top_k + 1 best candidates, in block order): the layout of the selection
// row and the k-th / (k+1)-th scores follow rtp_indexer_select.
__device__ __forceinline__ void finish_row(const ScoreArgs& a, entry_t* rb, int c, int rho,
                           int qb, int* hist) {
  const int lane = threadIdx.x & 63;
  const int top_k = a.top_k, stride = top_k + 2;
  const int n_c = max(qb - 1, 0);
  const size_t row_id = (size_t)rho * a.n_b + qb;
  int32_t* out = a.sel + row_id * stride;
  if (n_c <= top_k || top_k == 0) {
    // every candidate kept, or none when top_k == 0
    const bool all = top_k > 0;
    for (int t = lane; t < stride; t += 64) {
      int v;
      if (all) v = t <= qb ? t : -1;
      else v = t == 0 ? 0 : ((t == 1 && qb >= 1) ? qb : -1);
      out[t] = v;
    }
    if (lane == 0) a.sel_cnt[row_id] = all ? qb + 1 : (qb >= 1 ? 2 : 1);
    if (a.kth) {
      // s_k exists iff 1 <= k <= n_c (here k == n_c: the row minimum); s_{k+1}
      // iff k + 1 <= n_c (here k == 0: the row maximum). The buffer holds
      // every candidate (k == n_c) or the best one (k == 0).
      uint32_t mn = 0xffffffffu, mx = 0u;
      for (int e = lane; e < c; e += 64) {
        const uint32_t x = rb[e].x;
        mn = min(mn, x);
        mx = max(mx, x);
      }
      mn = wave_min_u32(mn);
      mx = wave_max_u32(mx);
      if (lane == 0) {
        put_score(a.kth, row_id * 2 + 0, top_k >= 1 && n_c == top_k, mn);
        put_score(a.kth, row_id * 2 + 1, top_k == 0 && n_c >= 1, mx);
      }
    }
    return;
  }
  // 1 <= top_k < n_c; shrink the buffer first when it is well above need
  if (c > top_k + 1 + 64) {
    uint32_t unused;
    c = compact_row(rb, c, top_k + 1, hist, unused);
  }
  const uint32_t T = wave_take(
      [&](int i) { return rb[i].x; }, c, top_k,
      [&](int p, int i, uint32_t) { out[1 + p] = (int32_t)rb[i].y; }, hist);
  if (lane == 0) {
    out[0] = 0;
    out[top_k + 1] = qb;
    a.sel_cnt[row_id] = top_k + 2;
  }
  if (a.kth) {
    // (k+1)-th best: T again if another key ties it, else the best key
    // below T (the buffer holds the top k + 1)
    int ge = 0;
    uint32_t bel = 0u;
    for (int e = lane; e < c; e += 64) {
      const uint32_t x = rb[e].x;
      ge += x >= T;
      if (x < T) bel = max(bel, x);
    }
    ge = wave_sum(ge);
    bel = wave_max_u32(bel);
    if (lane == 0) {
      put_score(a.kth, row_id * 2 + 0, true, T);
      put_score(a.kth, row_id * 2 + 1, true, ge >= top_k + 1 ? T : bel);
    }
  }
}

// ---- fused block scores and selection: a persistent grid of 4-wave
// workgroups; each workgroup repeatedly takes the next quad of work items
// from a counter (an item is one retrieval head's 64 consecutive query
// blocks, lane l owning query block 64 t + l; a quad is four adjacent items
// of one head, one per wave). Quads go from the longest rows to the
// shortest.
//
// Per candidate key block, the wave computes the 64 x 64 dot products of
// the block's keys with its 64 query-block means as 2 x 2 tiles of
// v_mfma_f32_32x32x16_bf16, three per tile (bf16 x 3 split), with the keys
// along M so that the max over a block's keys is a max over a lane's 16
// accumulator values plus one exchange with the other half of the wave
// (v_permlane32_swap). Each lane then holds its own row's score. A score
// that can still enter the row's top k + 1 is appended to the row's
// candidate buffer; a full buffer is shrunk by compact_row. The operands of
// the next key blocks are loaded PF blocks ahead; the wave never waits at a
// barrier, so a wave busy shrinking a buffer delays no other.
template <int R16, int PF>
__device__ __forceinline__ void run_tile(const ScoreArgs& a, int rho, int t,
                                         entry_t* wbuf, int* hist,
                                         int sync_until) {
  constexpr int r = 16 * R16;
  constexpr int NA = 4 * R16;  // 1 KiB operand chunks per key block
  const int lane = threadIdx.x & 63;
  const int n_b = a.n_b, cap = a.cap, need = a.top_k + 1;
  const int R0 = 64 * t;
  const int qb = R0 + lane;
  const bool row_ok = qb < n_b;
  const int qb_max = min(R0 + 63, n_b - 1);  // candidates: kb < qb_max
  // B operands: the query-block means of rows R0 + 32 nt + l%32
  bf16x8 bh[2][R16], bl[2][R16];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int row = R0 + 32 * nt + (lane & 31);
#pragma unroll
    for (int rs = 0; rs < R16; ++rs) {
      bf16x8 z = {};
      bh[nt][rs] = z;
      bl[nt][rs] = z;
      if (row < n_b) {
        const size_t o = ((size_t)rho * n_b + row) * r + 16 * rs + 8 * (lane >> 5);
        bh[nt][rs] = *reinterpret_cast<const bf16x8*>(a.qhi + o);
        bl[nt][rs] = *reinterpret_cast<const bf16x8*>(a.qlo + o);
      }
    }
  }
  const u16* kop = a.kop + (size_t)rho * n_b * kop_block_elems(r) + lane * 8;
  entry_t* rowbuf = wbuf + (size_t)lane * cap;
  int cnt = 0;
  uint32_t thr = 0u;
  bool armed = false;

  if (qb_max > 1) {
    const int last = qb_max - 1;
    bf16x8 ar[PF][NA];
    auto load_a = [&](int kb, bf16x8 (&dst)[NA]) {
      const u16* p = kop + (size_t)kb * kop_block_elems(r);
#pragma unroll
      for (int c = 0; c < NA; ++c)
        dst[c] = *gmem(reinterpret_cast<const bf16x8*>(p + c * 512));
    };
    // one key block: scores of the wave's 64 rows, the operands of block
    // kb + PF loaded into the freed slot, and the append
    auto step = [&](int kb, bf16x8 (&cur)[NA]) -> uint32_t {
      float mx[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) mx[nt] = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        f32x16 acc[2];
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          f32x16 z = {};
          acc[nt] = z;
        }
#pragma unroll
        for (int rs = 0; rs < R16; ++rs) {
          const bf16x8 ahi = cur[(mt * 2 + 0) * R16 + rs];
          const bf16x8 alo = cur[(mt * 2 + 1) * R16 + rs];
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma32(alo, bh[nt][rs], acc[nt]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma32(ahi, bl[nt][rs], acc[nt]);
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) acc[nt] = mfma32(ahi, bh[nt][rs], acc[nt]);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          float m = mx[nt];
#pragma unroll
          for (int i = 0; i < 16; i += 2) m = fmaxf(m, fmaxf(acc[nt][i], acc[nt][i + 1]));
          mx[nt] = m;
        }
      }
      load_a(min(kb + PF, last), cur);
      // lanes < 32 hold half-block maxima of rows R0 + l (tile 0) and lanes
      // >= 32 of rows R0 + 32 + l%32 (tile 1): one swap of the upper half of
      // mx[0] with the lower half of mx[1] lines the halves up, so lane l
      // ends with the score of row R0 + l
      const auto sw = __builtin_amdgcn_permlane32_swap(
          __float_as_uint(mx[0]), __float_as_uint(mx[1]), false, false);
      const float score = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      return order_key(score);
    };
    // (cnt < cap always holds here, as buffers are shrunk to at most
    // cap - 64 entries before they come within PF of full; the test keeps
    // every store in bounds regardless)
    auto append = [&](int kb, uint32_t key) {
      if (row_ok && kb < qb && (!armed || key > thr) && cnt < cap) {
        gmem(rowbuf)[cnt] = entry_t{key, (uint32_t)kb};
        ++cnt;
      }
    };
    // buffers that a group of PF more appends could fill are shrunk
    // between groups, so the groups themselves run without branches; the
    // group's appends come after all of its scores (in key-block order, so
    // the buffers hold what per-block appends would), which leaves the
    // group's 12 PF MFMAs and max reductions one scheduling region instead
    // of one per key block
    auto shrink = [&]() {
      uint64_t full = __ballot(cnt > cap - PF);
      if (full) {
        fence_wg();
        while (full) {
          const int rr = (int)__builtin_ctzll(full);
          full &= full - 1;
          uint32_t t_new;
          entry_t* rb = wbuf + (size_t)rr * cap;
          const int c_old = __builtin_amdgcn_readlane(cnt, rr);
          int c_new;
          if (cap <= 64 * kRowRegs) {
            RowRegs R;
            load_row(rb, c_old, R);
            c_new = compact_regs(rb, R, need, hist, t_new);
          } else {
            c_new = compact_row(rb, c_old, need, hist, t_new);
          }
          if (lane == rr) {
            cnt = c_new;
            thr = t_new;
            armed = true;
          }
        }
        fence_wg();
        // nothing of this branch stays in flight (it already waited for its
        // own loads), so the group loop keeps exact wait counts for the ring
        wait_vm_all();
      }
    };
    // the query-block operands arrive before the ring is filled: the wait
    // counts inside the loop then cover the ring's loads only
    wait_vm_all();
#pragma unroll
    for (int p = 0; p < PF; ++p) load_a(min(1 + p, last), ar[p]);
    // The workgroup's four waves meet at a barrier every 4 groups while all
    // of them are inside their common key range (sync_until, the same for
    // all four, so all four pass the same barriers): a wave delayed by
    // shrinking a buffer does not drift away from the others, and the key
    // blocks they share are still in cache when the last one reads them.
    int kb0 = 1;
    for (int grp = 0; kb0 + PF <= qb_max; kb0 += PF, ++grp) {
      uint32_t keys[PF];
#pragma unroll
      for (int p = 0; p < PF; ++p) keys[p] = step(kb0 + p, ar[p]);
#pragma unroll
      for (int p = 0; p < PF; ++p) append(kb0 + p, keys[p]);
      shrink();
      if ((grp & 3) == 3 && kb0 + PF <= sync_until) __syncthreads();
    }
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (kb0 + p < qb_max) append(kb0 + p, step(kb0 + p, ar[p]));
    shrink();
  }
  fence_wg();
  const int rows = min(64, n_b - R0);
  for (int rr = 0; rr < rows; ++rr) {
    const int c = __builtin_amdgcn_readlane(cnt, rr);
    entry_t* rb = wbuf + (size_t)rr * cap;
    if (cap <= 64 * kRowRegs) {
      RowRegs R;
      load_row(rb, c, R);
      finish_regs(a, R, rho, R0 + rr, hist);
    } else {
      finish_row(a, rb, c, rho, R0 + rr, hist);
    }
  }
  fence_wg();
}

template <int R16, int PF>
__global__ __launch_bounds__(256, 2) void score_select_kernel(const ScoreArgs a) {
  __shared__ int hist_all[4][256];
  __shared__ int s_quad;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int* hist = hist_all[wave];
  entry_t* wbuf = a.buf + (size_t)(blockIdx.x * 4 + wave) * 64 * a.cap;
  // Work is taken a quad at a time: one head's four adjacent 64-row tiles,
  // one per wave, started together after a barrier. The four waves then
  // stream the same projected keys at about the same time, so each key
  // block is fetched from memory about once per workgroup (taken one item
  // per wave, the waves of a workgroup read unrelated streams and every
  // read went to memory).
  const int n_quads = a.n_items / 4;
  for (;;) {
    if (threadIdx.x == 0) s_quad = atomicAdd(a.counter, 1);
    __syncthreads();
    const int quad = s_quad;
    __syncthreads();  // every wave has read s_quad before it is rewritten
    if (quad >= n_quads) break;
    const int u = quad / a.n_ret;
    const int rho = quad - u * a.n_ret;
    const int t = a.n_tiles - 1 - (4 * u + wave);
    // common key range of the quad's four tiles (none when the last quad
    // has fewer than four)
    const int t_min = a.n_tiles - 1 - (4 * u + 3);
    const int sync_until = t_min >= 0 ? min(64 * t_min + 63, a.n_b - 1) : 0;
    if (t >= 0) run_tile<R16, PF>(a, rho, t, wbuf, hist, sync_until);
  }
}

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t st) {
  if (a.n_ret == 0 || a.n_b == 0) return hipSuccess;
  ProjArgs pa;
  pa.S = a.S;
  pa.n_b = a.n_b;
  pa.r = a.r;
  pa.n_ret = a.n_ret;
  const int G = a.Hq / a.Hkv;
  int n_grp = 0;
  for (int i = 0; i < a.n_ret; ++i) {
    pa.head_of_rho[i] = a.ret_heads[i];
    const int g = a.ret_heads[i] / G;
    if (n_grp == 0 || pa.grp_kvh[n_grp - 1] != g) {
      pa.grp_kvh[n_grp] = (uint8_t)g;
      pa.grp_first[n_grp] = (uint8_t)i;
      ++n_grp;
    }
  }
  pa.grp_first[n_grp] = (uint8_t)a.n_ret;
  if (a.keys_only) {  // the centroids alone: no scratch
    prof_begin("proj_keys", st);
    hipLaunchKernelGGL(proj_keys_kernel, dim3((a.n_b + 3) / 4, n_grp),
                       dim3(256), 0, st, a.k, a.p_k, pa, (u16*)nullptr,
                       a.centroids);
    prof_end(st);
    return hipGetLastError();
  }
  const IndexerSizes z = indexer_sizes(a.n_ret, a.n_b, a.r, a.top_k);
  u16* kop = reinterpret_cast<u16*>(a.scratch);
  u16* qhi = reinterpret_cast<u16*>(a.scratch + z.kop);
  u16* qlo = reinterpret_cast<u16*>(a.scratch + z.kop + z.qpart);
  float* scores = reinterpret_cast<float*>(a.scratch + z.kop + 2 * z.qpart);
  entry_t* buf =
      reinterpret_cast<entry_t*>(a.scratch + z.kop + 2 * z.qpart + z.scores);
  int* counter = reinterpret_cast<int*>(a.scratch + z.kop + 2 * z.qpart +
                                        z.scores + z.buf);

  prof_begin("proj_keys", st);
  hipLaunchKernelGGL(proj_keys_kernel, dim3((a.n_b + 3) / 4, n_grp), dim3(256),
                     0, st, a.k, a.p_k, pa, kop, a.centroids);
  prof_end(st);
  prof_begin("proj_qmeans", st);
  hipLaunchKernelGGL(proj_qmeans_kernel, dim3((a.n_b + 3) / 4, a.n_ret),
                     dim3(256), 0, st, a.q, a.p_q, pa, qhi, qlo, counter);
  prof_end(st);
  if (!z.fused) {  // short sequence: score rows, then a top-k per row
    if (a.n_b >= 3) {
      dim3 grid((a.n_b + 127) / 128, (a.n_b + KBC - 1) / KBC, a.n_ret);
      prof_begin("block_scores", st);
      switch (a.r / 16) {
#define RTP_SCORE_CASE(R)                                                  \
  case R:                                                                  \
    hipLaunchKernelGGL(block_scores_kernel<R>, grid, dim3(256), 0, st, kop, \
                       qhi, qlo, scores, a.n_b);                           \
    break;
        RTP_SCORE_CASE(1) RTP_SCORE_CASE(2) RTP_SCORE_CASE(3) RTP_SCORE_CASE(4)
        RTP_SCORE_CASE(5) RTP_SCORE_CASE(6) RTP_SCORE_CASE(7) RTP_SCORE_CASE(8)
#undef RTP_SCORE_CASE
        default: return hipErrorInvalidValue;
      }
      prof_end(st);
    }
    prof_begin("topk", st);
    const int nk = a.n_b < TK_LDS ? a.n_b : TK_LDS;
    const size_t keys_bytes = ((size_t)nk + nk / 32 + 1) * 4;
    hipLaunchKernelGGL(topk_kernel, dim3(a.n_b, a.n_ret), dim3(256),
                       keys_bytes, st, scores, a.n_b, a.top_k, a.top_k + 2,
                       a.sel, a.sel_cnt, a.kth);
    prof_end(st);
    return hipGetLastError();
  }
  ScoreArgs sa;
  sa.kop = kop;
  sa.qhi = qhi;
  sa.qlo = qlo;
  sa.buf = buf;
  sa.counter = counter;
  sa.sel = a.sel;
  sa.sel_cnt = a.sel_cnt;
  sa.kth = a.kth;
  sa.n_b = a.n_b;
  sa.n_ret = a.n_ret;
  sa.top_k = a.top_k;
  sa.cap = z.cap;
  sa.n_tiles = (a.n_b + 63) / 64;
  sa.n_items = z.n_items;
  prof_begin("score_select", st);
  switch (a.r / 16) {
#define RTP_SCORE_CASE(R, PFN)                                                \
  case R:                                                                     \
    hipLaunchKernelGGL((score_select_kernel<R, PFN>), dim3(z.n_wg), dim3(256), \
                       0, st, sa);                                            \
    break;
    RTP_SCORE_CASE(1, 4) RTP_SCORE_CASE(2, 2) RTP_SCORE_CASE(3, 1)
    RTP_SCORE_CASE(4, 1) RTP_SCORE_CASE(5, 1) RTP_SCORE_CASE(6, 1)
    RTP_SCORE_CASE(7, 1) RTP_SCORE_CASE(8, 1)
#undef RTP_SCORE_CASE
    default: return hipErrorInvalidValue;
  }
  prof_end(st);
  return hipGetLastError();
}

}  // namespace rtp
