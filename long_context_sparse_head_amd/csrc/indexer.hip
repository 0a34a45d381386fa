// Retrieval-head indexer for gfx950: low-rank projection, block scoring and
// per-query-block top-k selection.
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
#include "common.h"
#include "select.h"

namespace rtp {

struct ProjArgs {
  int S, S_pad, n_b, r;
  uint8_t kvh_of_rho[kMaxHeads];
  uint8_t head_of_rho[kMaxHeads];
};

// ---- projection of keys: grid (n_ret, S_pad/64), one wave per 64 keys.
__global__ __launch_bounds__(64) void proj_keys_kernel(
    const u16* __restrict__ k, const float* __restrict__ p_k, const ProjArgs pa,
    u16* __restrict__ khi, u16* __restrict__ klo, float* __restrict__ cent) {
  __shared__ __attribute__((aligned(16))) float P[16 * kD];
  const int rho = blockIdx.x, kb = blockIdx.y, lane = threadIdx.x;
  const int S = pa.S, r = pa.r;
  const int g = pa.kvh_of_rho[rho];
  const int key = kb * 64 + lane;
  const u16* krow = k + ((size_t)g * S + (key < S ? key : 0)) * kD;
  for (int rc = 0; rc < r; rc += 16) {
    const float* src = p_k + ((size_t)rho * r + rc) * kD;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      reinterpret_cast<float4*>(P)[lane + 64 * i] =
          reinterpret_cast<const float4*>(src)[lane + 64 * i];
    __syncthreads();
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int dc = 0; dc < 16; ++dc) {
      uint4 raw = make_uint4(0, 0, 0, 0);
      if (key < S) raw = *reinterpret_cast<const uint4*>(krow + dc * 8);
      float kf[8];
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kf[2 * e] = __uint_as_float(w[e] << 16);
        kf[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        const float4 pa0 = *reinterpret_cast<const float4*>(P + rr * kD + dc * 8);
        const float4 pa1 = *reinterpret_cast<const float4*>(P + rr * kD + dc * 8 + 4);
        float x = acc[rr];
        x = fmaf(pa0.x, kf[0], x); x = fmaf(pa0.y, kf[1], x);
        x = fmaf(pa0.z, kf[2], x); x = fmaf(pa0.w, kf[3], x);
        x = fmaf(pa1.x, kf[4], x); x = fmaf(pa1.y, kf[5], x);
        x = fmaf(pa1.z, kf[6], x); x = fmaf(pa1.w, kf[7], x);
        acc[rr] = x;
      }
    }
    // split into high/low bf16 parts for the scoring MFMAs
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u16 h0 = f2bf(acc[2 * i]), h1 = f2bf(acc[2 * i + 1]);
      const u16 l0 = f2bf(acc[2 * i] - bf2f(h0));
      const u16 l1 = f2bf(acc[2 * i + 1] - bf2f(h1));
      hw[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lw[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    const size_t o = ((size_t)rho * pa.S_pad + key) * r + rc;
    uint4* dh = reinterpret_cast<uint4*>(khi + o);
    uint4* dl = reinterpret_cast<uint4*>(klo + o);
    dh[0] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
    dh[1] = make_uint4(hw[4], hw[5], hw[6], hw[7]);
    dl[0] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
    dl[1] = make_uint4(lw[4], lw[5], lw[6], lw[7]);
    if (cent) {
      const int cnt = min(64, S - kb * 64);
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float v = key < S ? acc[rr] : 0.f;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if (lane == 0) cent[((size_t)rho * pa.n_b + kb) * r + rc + rr] = v / (float)cnt;
      }
    }
    __syncthreads();
  }
}

// ---- block means of queries, projected: grid (n_ret, n_b), one wave each.
__global__ __launch_bounds__(64) void proj_qmeans_kernel(
    const u16* __restrict__ q, const float* __restrict__ p_q, const ProjArgs pa,
    u16* __restrict__ qhi, u16* __restrict__ qlo) {
  __shared__ float mean[kD];
  const int rho = blockIdx.x, qb = blockIdx.y, lane = threadIdx.x;
  const int S = pa.S, r = pa.r;
  const int h = pa.head_of_rho[rho];
  const int rows = min(64, S - qb * 64);
  const uint32_t* base = reinterpret_cast<const uint32_t*>(
      q + ((size_t)h * S + (size_t)qb * 64) * kD) + lane;
  float s0 = 0.f, s1 = 0.f;
  for (int i = 0; i < rows; ++i) {
    const uint32_t w = base[(size_t)i * (kD / 2)];
    s0 += __uint_as_float(w << 16);
    s1 += __uint_as_float(w & 0xffff0000u);
  }
  mean[2 * lane] = s0 / (float)rows;
  mean[2 * lane + 1] = s1 / (float)rows;
  __syncthreads();
  for (int rr = lane; rr < r; rr += 64) {
    const float* prow = p_q + ((size_t)rho * r + rr) * kD;
    float acc = 0.f;
    for (int d = 0; d < kD; ++d) acc = fmaf(prow[d], mean[d], acc);
    const u16 hi = f2bf(acc);
    const size_t o = ((size_t)rho * pa.n_b + qb) * r + rr;
    qhi[o] = hi;
    qlo[o] = f2bf(acc - bf2f(hi));
  }
}

// ---- block scores: grid (ceil(n_b/128), ceil(n_b/KBC), n_ret), 4 waves.
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
    const u16* __restrict__ khi, const u16* __restrict__ klo,
    const u16* __restrict__ qhi, const u16* __restrict__ qlo,
    float* __restrict__ scores, int S_pad, int n_b) {
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
  const u16* kh = khi + (size_t)rho * S_pad * r;
  const u16* kl = klo + (size_t)rho * S_pad * r;
  const int nst = (kb_end - kb_begin + KBI - 1) / KBI;
  // key blocks past the chunk re-read its last block (never used)
  auto gload = [&](int stg, u32x4 (&reg)[PER_T]) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = tid + 256 * i;
      const int part = c / (SROWS * CH_PER_ROW), cc = c % (SROWS * CH_PER_ROW);
      const int row = cc / CH_PER_ROW, ch = cc % CH_PER_ROW;
      const int kb = min(kb_begin + stg * KBI + row / 64, kb_end - 1);
      const u16* src = (part ? kl : kh) + ((size_t)kb * 64 + (row & 63)) * r + ch * 8;
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
  __shared__ uint32_t keys[TK_LDS + TK_LDS / 32];
  __shared__ TopkShared sh;
  const int qb = blockIdx.x, rho = blockIdx.y, tid = threadIdx.x;
  const int n_c = max(qb - 1, 0);  // candidates 1 .. qb-1
  const size_t row_id = (size_t)rho * n_b + qb;
  int32_t* out = sel + row_id * stride;
  const float* row = scores + (size_t)rho * tri_rows(n_b) +
                     (qb >= 2 ? (int64_t)(qb - 2) * (qb - 1) / 2 : 0);
  const float qnan = __builtin_nanf("");

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
      if (tid == 0) {
        kth[row_id * 2 + 0] = (top_k >= 1 && n_c == top_k) ? order_key_inv(mn) : qnan;
        kth[row_id * 2 + 1] = (top_k == 0 && n_c >= 1) ? order_key_inv(mx) : qnan;
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
      kth[row_id * 2 + 0] = order_key_inv(res.T);
      kth[row_id * 2 + 1] = count_ge >= top_k + 1 ? order_key_inv(res.T)
                                                  : order_key_inv(below);
    }
  }
}

hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t st) {
  if (a.n_ret == 0 || a.n_b == 0) return hipSuccess;
  ProjArgs pa;
  pa.S = a.S;
  pa.S_pad = a.S_pad;
  pa.n_b = a.n_b;
  pa.r = a.r;
  const int G = a.Hq / a.Hkv;
  for (int i = 0; i < kMaxHeads; ++i) {
    pa.head_of_rho[i] = i < a.n_ret ? a.ret_heads[i] : 0;
    pa.kvh_of_rho[i] = i < a.n_ret ? a.ret_heads[i] / G : 0;
  }
  prof_begin("proj_keys", st);
  hipLaunchKernelGGL(proj_keys_kernel, dim3(a.n_ret, a.S_pad / 64), dim3(64), 0,
                     st, a.k, a.p_k, pa, a.khi, a.klo, a.centroids);
  prof_end(st);
  if (a.keys_only) return hipGetLastError();
  prof_begin("proj_qmeans", st);
  hipLaunchKernelGGL(proj_qmeans_kernel, dim3(a.n_ret, a.n_b), dim3(64), 0, st,
                     a.q, a.p_q, pa, a.qhi, a.qlo);
  prof_end(st);
  if (a.n_b >= 3) {
    dim3 grid((a.n_b + 127) / 128, (a.n_b + KBC - 1) / KBC, a.n_ret);
    prof_begin("block_scores", st);
    switch (a.r / 16) {
#define RTP_SCORE_CASE(R)                                                    \
  case R:                                                                    \
    hipLaunchKernelGGL(block_scores_kernel<R>, grid, dim3(256), 0, st,       \
                       a.khi, a.klo, a.qhi, a.qlo, a.scores, a.S_pad, a.n_b); \
    break;
      RTP_SCORE_CASE(1) RTP_SCORE_CASE(2) RTP_SCORE_CASE(3) RTP_SCORE_CASE(4)
      RTP_SCORE_CASE(5) RTP_SCORE_CASE(6) RTP_SCORE_CASE(7) RTP_SCORE_CASE(8)
#undef RTP_SCORE_CASE
      default: return hipErrorInvalidValue;
    }
    prof_end(st);
  }
  prof_begin("topk", st);
  hipLaunchKernelGGL(topk_kernel, dim3(a.n_b, a.n_ret), dim3(256), 0, st,
                     a.scores, a.n_b, a.top_k, a.top_k + 2, a.sel, a.sel_cnt,
                     a.kth);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace rtp
