// Attention tile engine for gfx950: sliding-window heads, dense causal heads
// and block-sparse retrieval heads in one persistent-free launch.
//
// What it computes (Synced RTPurbo article, "化繁为简，被低估的 SWA": most
// heads attend only a recent window; aitop.news summary of "Full Attention
// Strikes Back": retrieval heads run exact attention on an indexer-selected
// set): for query i and its key set J_i,
//     o_i = sum_{j in J_i} softmax_j(scale * q_i.k_j) v_j,
// with J_i = {i-w < j <= i} for a window head and J_i = {j <= i in the kept
// blocks} for a retrieval head.
//
// Design (MI355X-first):
//  * One workgroup = 4 waves = 64 queries of one query block; key tiles are
//    64-token blocks, so a block-sparse list and a window range drive the same
//    loop. Work items: a PAIR of window heads of one KV group (each wave owns
//    32 queries of one head and the whole key tile), or a SINGLE head (each
//    wave owns 32 queries and one 32-key half of every tile; the two halves
//    are merged through LDS at the end).
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with the query along the lanes,
//    so a query's scores sit in one lane pair and the row max needs a single
//    cross-lane exchange. K rows are stored in LDS in an order that makes the
//    accumulator directly the B operand of the P.V MFMA (no shuffles), and V
//    arrives pre-transposed (V^T) so its A operand is one 16-byte LDS read.
//  * Online softmax in base 2 with lazy rescaling: the running max moves only
//    when a tile exceeds it by more than 8 (in log2 units), so the O rescale is
//    rare; exact because the final normalisation uses the same reference.
//  * Masks are evaluated only on tiles that straddle the causal diagonal or
//    the window's lower edge; tiles outside every query's set are skipped
//    (the pages' point about SWA without three-segment KV concat or a custom
//    mask tensor, RTP-LLM section of the Synced article).
//  * Work order: query blocks from last to first (heaviest first, the pages'
//    sparsity-aware scheduling), items of one query block grouped onto one
//    XCD so heads sharing a KV head share that XCD's L2.
#include "common.h"

namespace rtp {

constexpr int KSTR = 136;             // LDS row of K: 128 bf16 + 16 B pad
constexpr int VSTR = 72;              // LDS row of V^T: 64 bf16 + 16 B pad
constexpr int K_ELEMS = 64 * KSTR;
constexpr int V_ELEMS = 128 * VSTR;
constexpr int STAGE = K_ELEMS + V_ELEMS;  // bf16 elements per pipeline stage

struct AttnParams {
  AttnLaunch a;
  float c;      // scale * log2(e)
  float tau;    // lazy-rescale threshold, raw logit units
  int n_items, per_qb, chunk;
  uint32_t desc[kMaxHeads];
};

// Key row r of a 32-key sub-tile is stored at LDS row perm(r) (swap bits 2
// and 3). Then accumulator element i of lane l of S^T = K Q^T holds key
// 16*(i/8) + 8*(l/32) + i%8 of the sub-tile: the 8 values a lane feeds as the
// B operand of one P.V MFMA step are 8 consecutive keys.
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int NS>
__device__ __forceinline__ void process_tile(
    const u16* __restrict__ sk, const u16* __restrict__ sv, int k0, int sub0,
    const bf16x8 (&qf)[8], f32x16 (&acc)[4], float& m_ref, float& lsum,
    int qi, int qmin, int window, float c, float tau, int lane) {
  const int g = lane >> 5, n = lane & 31;
  const int qmax = qmin + 31;
  f32x16 s[NS];
  bool act[NS];
  bool any = false;
  float tmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int st = sub0 + u;
    const int kmin = k0 + 32 * st, kmax = kmin + 31;
    act[u] = !(kmin > qmax || kmax <= qmin - window);
    any |= act[u];
    if (act[u]) {
      f32x16 z = {};
      s[u] = z;
      const u16* arow = sk + (32 * st + n) * KSTR + 8 * g;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        s[u] = mfma32(*reinterpret_cast<const bf16x8*>(arow + 16 * ks), qf[ks],
                      s[u]);
      if (kmax > qmin || kmin <= qmax - window) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kmin + 16 * (i >> 3) + 8 * g + (i & 7);
          const bool ok = key <= qi && key > qi - window;
          s[u][i] = ok ? s[u][i] : -INFINITY;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[u][i]);
    }
  }
  if (!any) return;  // wave-uniform
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
  if (tmax > m_ref + tau) {
    const float alpha = fast_exp2((m_ref - tmax) * c);
    m_ref = tmax;
    lsum *= alpha;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][i] *= alpha;
  }
  const float mc = m_ref * c;
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    if (!act[u]) continue;
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float pv = fast_exp2(fmaf(s[u][i], c, -mc));
      lsum += pv;
      pb[i >> 3][i & 7] = (__bf16)pv;
    }
    const int st = sub0 + u;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u16* vrow = sv + (32 * mt + n) * VSTR + 32 * st + 16 * ks + 8 * g;
        acc[mt] = mfma32(*reinterpret_cast<const bf16x8*>(vrow), pb[ks],
                         acc[mt]);
      }
  }
}

__global__ __launch_bounds__(256, 2) void attn_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) u16 smem[2 * STAGE];
  const AttnLaunch& a = p.a;
  const int nb = a.n_b;
  const int S = a.S;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;

  // XCD-aware order: consecutive workgroups land on different XCDs, so give
  // each XCD runs of `chunk` consecutive logical items.
  int item = blockIdx.x;
  {
    const int grp = 8 * p.chunk;
    const int full = (p.n_items / grp) * grp;
    if (item < full) {
      const int x = item & 7, s = item >> 3;
      item = (s / p.chunk) * grp + x * p.chunk + (s % p.chunk);
    }
  }
  const int qb = nb - 1 - item / p.per_qb;  // heaviest (last) blocks first
  const uint32_t desc = p.desc[item % p.per_qb];
  const int kind = desc & 3;
  const int ha = (desc >> 8) & 255, hb = (desc >> 16) & 255;
  const int rho = desc >> 24;
  const int head = (kind == 0 && wave >= 2) ? hb : ha;
  const int kvh = ha / a.G;
  const int qmin = qb * 64 + 32 * (wave & 1);
  const int qi = qmin + n;
  const int window = (kind == 2) ? (1 << 30) : a.window;

  int kt_lo = 0, nt;
  const int32_t* sel_row = nullptr;
  if (kind == 2) {
    sel_row = a.sel + ((size_t)rho * nb + qb) * a.sel_stride;
    nt = a.sel_cnt[(size_t)rho * nb + qb];
    nt = nt < 0 ? 0 : (nt > a.sel_stride ? a.sel_stride : nt);
  } else {
    const int lo = qb * 64 - window + 1;
    kt_lo = lo > 0 ? (lo >> 6) : 0;
    nt = qb - kt_lo + 1;
  }
  auto tile_of = [&](int t) -> int {
    if (kind != 2) return kt_lo + t;
    int kb = sel_row[t];
    return kb < 0 ? 0 : (kb > qb ? qb : kb);  // memory-safe on bad input
  };

  bf16x8 qf[8];
  {
    const u16* qp = a.q + ((size_t)head * S + (qi < S ? qi : 0)) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
      if (qi >= S) { bf16x8 z = {}; v = z; }
      qf[ks] = v;
    }
  }

  const u16* kbase = a.k + (size_t)kvh * S * kD;
  const u16* vtbase = a.vt + (size_t)kvh * kD * a.S_pad;
  uint4 kreg[4], vreg[4];
  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 4, ch = cidx & 15;
      const int key = kb * 64 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (key < S)
        v = *reinterpret_cast<const uint4*>(kbase + (size_t)key * kD + ch * 8);
      kreg[i] = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i, dr = cidx >> 3, ch = cidx & 7;
      vreg[i] = *reinterpret_cast<const uint4*>(
          vtbase + (size_t)dr * a.S_pad + kb * 64 + ch * 8);
    }
  };
  auto sstore = [&](u16* st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 4, ch = cidx & 15;
      *reinterpret_cast<uint4*>(st + perm_row(row) * KSTR + ch * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int cidx = tid + 256 * i, dr = cidx >> 3, ch = cidx & 7;
      *reinterpret_cast<uint4*>(st + K_ELEMS + dr * VSTR + ch * 8) = vreg[i];
    }
  };

  f32x16 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    f32x16 z = {};
    acc[mt] = z;
  }
  float m_ref = -1e30f, lsum = 0.f;

  if (nt > 0) {
    gload(tile_of(0));
    sstore(smem);
  }
  __syncthreads();
  for (int t = 0; t < nt; ++t) {
    u16* cur = smem + (t & 1) * STAGE;
    u16* nxt = smem + ((t + 1) & 1) * STAGE;
    if (t + 1 < nt) gload(tile_of(t + 1));
    const int k0 = tile_of(t) * 64;
    if (kind == 0)
      process_tile<2>(cur, cur + K_ELEMS, k0, 0, qf, acc, m_ref, lsum, qi,
                      qmin, window, p.c, p.tau, lane);
    else
      process_tile<1>(cur, cur + K_ELEMS, k0, wave >> 1, qf, acc, m_ref, lsum,
                      qi, qmin, window, p.c, p.tau, lane);
    if (t + 1 < nt) sstore(nxt);
    __syncthreads();
  }

  lsum += __shfl_xor(lsum, 32);
  if (kind != 0) {
    // merge the two key halves: waves 2,3 hand (m, l, O) to waves 0,1
    float* xs = reinterpret_cast<float*>(smem);
    if (wave >= 2) {
      float* d = xs + (wave - 2) * 66 * 64 + lane;
      d[0] = m_ref;
      d[64] = lsum;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) d[(2 + mt * 16 + i) * 64] = acc[mt][i];
    }
    __syncthreads();
    if (wave < 2) {
      const float* s2 = xs + wave * 66 * 64 + lane;
      const float m2 = s2[0], l2 = s2[64];
      const float mm = fmaxf(m_ref, m2);
      const float a1 = fast_exp2((m_ref - mm) * p.c);
      const float a2 = fast_exp2((m2 - mm) * p.c);
      lsum = lsum * a1 + l2 * a2;
      m_ref = mm;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[mt][i] = acc[mt][i] * a1 + s2[(2 + mt * 16 + i) * 64] * a2;
    }
  }
  if (kind != 0 && wave >= 2) return;
  if (qi < S) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    u16* op = a.out + ((size_t)head * S + qi) * kD;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = 32 * mt + 8 * q4 + 4 * g;
        uint2 w;
        w.x = (uint32_t)f2bf(acc[mt][4 * q4 + 0] * inv) |
              ((uint32_t)f2bf(acc[mt][4 * q4 + 1] * inv) << 16);
        w.y = (uint32_t)f2bf(acc[mt][4 * q4 + 2] * inv) |
              ((uint32_t)f2bf(acc[mt][4 * q4 + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(op + d0) = w;
      }
    if (a.lse && g == 0)
      a.lse[(size_t)head * S + qi] =
          (m_ref * p.c + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f;
  }
}

// V [Hkv,S,128] -> V^T [Hkv,128,S_pad], zero beyond S.
__global__ __launch_bounds__(256) void transpose_v_kernel(
    const u16* __restrict__ v, u16* __restrict__ vt, int S, int S_pad) {
  __shared__ __attribute__((aligned(16))) u16 t[64 * KSTR];
  const int kb = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const u16* src = v + (size_t)g * S * kD;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, row = c >> 4, ch = c & 15;
    const int key = kb * 64 + row;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (key < S) x = *reinterpret_cast<const uint4*>(src + (size_t)key * kD + ch * 8);
    *reinterpret_cast<uint4*>(t + row * KSTR + ch * 8) = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + 256 * i, dr = c >> 3, kc = c & 7;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)t[(kc * 8 + 2 * e) * KSTR + dr] |
             ((uint32_t)t[(kc * 8 + 2 * e + 1) * KSTR + dr] << 16);
    *reinterpret_cast<uint4*>(vt + ((size_t)g * kD + dr) * S_pad + kb * 64 + kc * 8) =
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

hipError_t launch_attention(const AttnLaunch& a, const AttnItems& items,
                            hipStream_t st) {
  if (a.n_b == 0 || items.n == 0) return hipSuccess;
  AttnParams p;
  p.a = a;
  p.c = a.scale * 1.4426950408889634f;
  p.tau = 8.0f / p.c;
  p.per_qb = items.n;
  p.n_items = a.n_b * items.n;
  p.chunk = items.n;
  for (int i = 0; i < kMaxHeads; ++i) p.desc[i] = i < items.n ? items.desc[i] : 0;
  prof_begin("attn", st);
  hipLaunchKernelGGL(attn_kernel, dim3(p.n_items), dim3(256), 0, st, p);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace rtp
