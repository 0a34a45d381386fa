// Hybrid decode for gfx950: block-centroid selection for retrieval heads,
// sliding window for streaming heads, exact split-K attention, LSE merge.
//
// What it computes (RTPurboV2 article: keys cluster in the low-rank space, so
// whole groups of unrelated tokens can be skipped; for the Qwen3-Coder model
// the K cache is clustered at prefill and decode runs sparsely on the
// retrieval heads while the other heads keep an SWA window). This library's
// reading: groups are contiguous 64-token blocks with centroid
// c_kb = mean_{j in kb} P_k k_j; the projected query scores the candidates
// 1 .. n_b-n_recent-1; the sink block, the top_k candidates and the last
// n_recent blocks are attended exactly.
//
// Decode is bound by HBM bandwidth: every key/value byte is read once. The
// window heads of one KV group share one pass over the window (up to 32 heads
// per pass, GQA), retrieval heads gather their own blocks, and the keys of a
// (sequence, unit) are split over many workgroups whose partial softmax
// states are merged by log-sum-exp.
#include "common.h"
#include "select.h"

namespace rtp {

// Heads of one KV group that share a pass over its window: the N dimension
// of the MFMA tiles (32), so a group of up to 32 window heads reads its K/V
// once.
constexpr int kDecMaxUnitHeads = 32;

// ---------------------------------------------------------------- centroids
struct CentArgs {
  int Hkv, Lmax, n_ret, r, nbmax;
  KvView kv;
  uint8_t kvh_of_rho[kMaxHeads];
};

// Centroid of one full key block for one retrieval head, by one wave: the
// mean of the block's 64 keys (summed key by key, two dims per lane), then
// projected with P_k[rho] (equal to the mean of the projected keys by
// linearity). rows: the block's first key row; mean: kD floats of LDS.
__device__ __forceinline__ void block_centroid(const u16* rows_base,
                                               const float* prow0, int r,
                                               float* mean, float* out,
                                               int lane) {
  const uint32_t* rows = reinterpret_cast<const uint32_t*>(rows_base) + lane;
  float s0 = 0.f, s1 = 0.f;
  for (int i = 0; i < 64; ++i) {
    const uint32_t w = rows[(size_t)i * (kD / 2)];
    s0 += __uint_as_float(w << 16);
    s1 += __uint_as_float(w & 0xffff0000u);
  }
  mean[2 * lane] = s0 * (1.f / 64.f);
  mean[2 * lane + 1] = s1 * (1.f / 64.f);
  __syncthreads();
  for (int rr = lane; rr < r; rr += 64) {
    const float* prow = prow0 + (size_t)rr * kD;
    float acc = 0.f;
    for (int d = 0; d < kD; ++d) acc = fmaf(prow[d], mean[d], acc);
    out[rr] = acc;
  }
  __syncthreads();  // mean may be reused
}

// grid (nbmax, n_ret, B), one wave. Full blocks only.
__global__ __launch_bounds__(64) void build_centroids_kernel(
    const u16* __restrict__ kc, const int32_t* __restrict__ cache_len,
    const float* __restrict__ p_k, const CentArgs ca, float* __restrict__ cent) {
  __shared__ float mean[kD];
  const int kb = blockIdx.x, rho = blockIdx.y, b = blockIdx.z, lane = threadIdx.x;
  int L = cache_len[b];
  L = L < 0 ? 0 : (L > ca.Lmax ? ca.Lmax : L);
  if ((kb + 1) * 64 > L) return;
  const int g = ca.kvh_of_rho[rho];
  block_centroid(kc + kv_row(ca.kv, b, ca.Hkv, g, ca.Lmax, kb * 64),
                 p_k + (size_t)rho * ca.r * kD, ca.r, mean,
                 cent + (((size_t)b * ca.n_ret + rho) * ca.nbmax + kb) * ca.r,
                 lane);
}

// ------------------------------------------------------------- cache append
// grid (B, Hkv), one wave: k_new / v_new row of (b, g) -> position
// cache_len[b] of the cache (full caches are left unchanged).
__global__ __launch_bounds__(64) void append_kv_kernel(
    u16* __restrict__ kc, u16* __restrict__ vc,
    const int32_t* __restrict__ cache_len, const u16* __restrict__ k_new,
    const u16* __restrict__ v_new, int Hkv, int Lmax, const KvView kv) {
  const int b = blockIdx.x, g = blockIdx.y, lane = threadIdx.x;
  const int L = cache_len[b];
  if (L < 0 || L >= Lmax) return;
  const size_t src = ((size_t)b * Hkv + g) * kD;
  const size_t dst = kv_row(kv, b, Hkv, g, Lmax, L);
  reinterpret_cast<uint32_t*>(kc + dst)[lane] =
      reinterpret_cast<const uint32_t*>(k_new + src)[lane];
  reinterpret_cast<uint32_t*>(vc + dst)[lane] =
      reinterpret_cast<const uint32_t*>(v_new + src)[lane];
}

// grid (B), one wave: when the appended token completes a block, that
// block's centroid for every retrieval head; then cache_len[b] += 1.
__global__ __launch_bounds__(64) void append_centroids_kernel(
    const u16* __restrict__ kc, int32_t* __restrict__ cache_len,
    const float* __restrict__ p_k, const CentArgs ca, float* __restrict__ cent) {
  __shared__ float mean[kD];
  const int b = blockIdx.x, lane = threadIdx.x;
  const int L = cache_len[b];  // before the append
  if (L < 0 || L >= ca.Lmax) return;
  if ((L + 1) % 64 == 0) {
    const int kb = L / 64;
    for (int rho = 0; rho < ca.n_ret; ++rho) {
      const int g = ca.kvh_of_rho[rho];
      block_centroid(
          kc + kv_row(ca.kv, b, ca.Hkv, g, ca.Lmax, kb * 64),
          p_k + (size_t)rho * ca.r * kD, ca.r, mean,
          cent + (((size_t)b * ca.n_ret + rho) * ca.nbmax + kb) * ca.r, lane);
    }
  }
  if (lane == 0) cache_len[b] = L + 1;
}

hipError_t launch_decode_append(u16* kc, u16* vc, int32_t* cache_len,
                                const u16* k_new, const u16* v_new,
                                const float* p_k, float* cent, int B,
                                int Lmax, int Hkv, int n_ret, int r, int G,
                                const uint8_t* ret_heads, hipStream_t st,
                                KvView kv) {
  if (B == 0) return hipSuccess;
  CentArgs ca;
  ca.kv = kv;
  ca.Hkv = Hkv;
  ca.Lmax = Lmax;
  ca.n_ret = n_ret;
  ca.r = r;
  ca.nbmax = Lmax / 64;
  for (int i = 0; i < kMaxHeads; ++i)
    ca.kvh_of_rho[i] = i < n_ret ? ret_heads[i] / G : 0;
  prof_begin("append_kv", st);
  hipLaunchKernelGGL(append_kv_kernel, dim3(B, Hkv), dim3(64), 0, st, kc, vc,
                     cache_len, k_new, v_new, Hkv, Lmax, kv);
  prof_end(st);
  prof_begin("append_centroids", st);
  hipLaunchKernelGGL(append_centroids_kernel, dim3(B), dim3(64), 0, st, kc,
                     cache_len, p_k, ca, cent);
  prof_end(st);
  return hipGetLastError();
}

hipError_t launch_build_centroids(const u16* kc, const int32_t* cache_len,
                                  const float* p_k, float* cent, int B,
                                  int Lmax, int Hkv, int n_ret, int r, int G,
                                  const uint8_t* ret_heads, hipStream_t st,
                                  KvView kv) {
  const int nbmax = Lmax / 64;
  if (B == 0 || n_ret == 0 || nbmax == 0) return hipSuccess;
  CentArgs ca;
  ca.kv = kv;
  ca.Hkv = Hkv;
  ca.Lmax = Lmax;
  ca.n_ret = n_ret;
  ca.r = r;
  ca.nbmax = nbmax;
  for (int i = 0; i < kMaxHeads; ++i)
    ca.kvh_of_rho[i] = i < n_ret ? ret_heads[i] / G : 0;
  prof_begin("build_centroids", st);
  hipLaunchKernelGGL(build_centroids_kernel, dim3(nbmax, n_ret, B), dim3(64), 0,
                     st, kc, cache_len, p_k, ca, cent);
  prof_end(st);
  return hipGetLastError();
}

// --------------------------------------------------- clustered token list
struct DecTokArgs {
  const int32_t* cl_m; const int32_t* cl_off; const int32_t* cl_mem;
  int32_t* tok; int32_t* tok_cnt;  // tok == nullptr: block decode
};
struct TokShared {
  int tmp[4];
  int sid[256], spos[256];
  int carry;
};

// The tokens a retrieval head attends in the clustered decode, in the
// order of its kept ids (ascending): the members of a kept cluster
// (1 <= id < m, ascending token order) or every token of a kept block (the
// sink, blocks that left the recent window after the clustering, the recent
// blocks). Segment starts come from a block-wide scan of the segment
// lengths; then each thread fills output positions tid, tid + 256, ...:
// the segment of a position by binary search over the starts in LDS, and
// eight members' loads in flight before their stores. Run by the
// selection's 256 threads once the kept ids are written (ids, n_sel),
// after a barrier.
__device__ void build_token_list(const DecTokArgs& a, const int32_t* ids,
                                 int n_sel, int L, int n_b, int n_recent,
                                 int Lmax, int nbmax, size_t row, int b,
                                 TokShared& sh) {
  const int tid = threadIdx.x;
  const int m = min(a.cl_m[b], n_b - n_recent);  // recent blocks stay blocks
  const int32_t* off = a.cl_off + row * (nbmax + 1);
  const int32_t* mem = a.cl_mem + row * Lmax;
  int32_t* out = a.tok + row * Lmax;
  int carry = 0;
  for (int s0 = 0; s0 < n_sel; s0 += 256) {
    const int e = s0 + tid;
    const int id = e < n_sel ? ids[e] : -1;
    int len = 0, src = 0;  // src: first member slot, or first token
    if (id >= 0) {
      if (id >= 1 && id < m) {
        len = min(max(off[id + 1] - off[id], 0), Lmax);
        src = min(max(off[id], 0), Lmax - len);
      } else {
        len = max(0, min(L, 64 * id + 64) - 64 * id);
        src = 64 * id;
      }
    }
    const int incl = block_incl_scan(len, sh.tmp);
    sh.sid[tid] = (id >= 1 && id < m) ? src : -1 - src;  // member slot / ~token
    sh.spos[tid] = incl - len;
    if (tid == 255) sh.carry = incl;
    __syncthreads();
    const int nseg = min(256, n_sel - s0);
    const int total = sh.carry;
    // (the list holds at most Lmax ids and every id is a cached token, also
    // for tables that do not match this cache)
    for (int q0 = 0; q0 < total; q0 += 8 * 256) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + 256 * u + tid;
        v[u] = 0;
        if (q < total) {
          int lo = 0, hi = nseg;  // last segment starting at or before q
          while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (sh.spos[mid] <= q) lo = mid; else hi = mid;
          }
          const int sv = sh.sid[lo], i = q - sh.spos[lo];
          v[u] = sv >= 0 ? mem[sv + i] : (-1 - sv) + i;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int pos = carry + q0 + 256 * u + tid;
        if (q0 + 256 * u + tid < total && pos < Lmax)
          out[pos] = min(max(v[u], 0), L - 1);
      }
    }
    carry += total;
    __syncthreads();
  }
  if (tid == 0) a.tok_cnt[row] = min(carry, Lmax);
}

// ------------------------------------------------------------- block choice
struct DecSelArgs {
  int Hq, Lmax, n_ret, r, nbmax, top_k, n_recent, width;
  // clustered decode: cluster ids 1 .. cl_m[b]-1 with offsets cl_off
  // [B, n_ret, nbmax + 1]; an empty cluster is never chosen ahead of a
  // non-empty candidate (nullptr: block decode)
  const int32_t* cl_m; const int32_t* cl_off;
  uint8_t head_of_rho[kMaxHeads];
};

// grid (n_ret, B), 256 threads.
__global__ __launch_bounds__(256) void dec_select_kernel(
    const u16* __restrict__ q, const float* __restrict__ p_q,
    const float* __restrict__ cent, const int32_t* __restrict__ cache_len,
    const DecSelArgs a, float* __restrict__ cscores, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_cnt, const DecTokArgs ta) {
  __shared__ uint32_t keys[TK_LDS + TK_LDS / 32];
  __shared__ float qt[kD];
  // the selection workspaces and the token-list scan are never in use at
  // the same time
  __shared__ union {
    TopkShared block;
    WaveTopkShared wave;
    TokShared tok;
  } tsh;
  TopkShared& sh = tsh.block;
  WaveTopkShared& wsh = tsh.wave;
  const int rho = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  int L = cache_len[b];
  L = L < 1 ? 1 : (L > a.Lmax ? a.Lmax : L);
  const int n_b = (L + 63) / 64;
  const int n_c = max(n_b - a.n_recent - 1, 0);
  const size_t row_id = (size_t)b * a.n_ret + rho;
  int32_t* out = sel + row_id * a.width;
  if (n_c <= a.top_k) {  // short cache: every block
    for (int t = tid; t < a.width; t += 256) out[t] = t < n_b ? t : -1;
    if (tid == 0) sel_cnt[row_id] = n_b;
    if (ta.tok) {
      __syncthreads();  // the kept ids are written (read back by this block)
      build_token_list(ta, out, n_b, L, n_b, a.n_recent, a.Lmax, a.nbmax,
                       row_id, b, tsh.tok);
    }
    return;
  }
  const int h = a.head_of_rho[rho];
  const u16* qrow = q + ((size_t)b * a.Hq + h) * kD;
  // q~ = P_q q: thread (j, c) takes d = 8c .. 8c+7 of row j, 16 lanes sum
  // a row (r is a multiple of 16)
  for (int j0 = 0; j0 < a.r; j0 += 16) {
    const int j = j0 + (tid >> 4), c = tid & 15;
    float acc = 0.f;
    if (j < a.r) {
      const float4* pp =
          reinterpret_cast<const float4*>(p_q + ((size_t)rho * a.r + j) * kD + 8 * c);
      const float4 p0 = pp[0], p1 = pp[1];
      const uint4 qv = *reinterpret_cast<const uint4*>(qrow + 8 * c);
      acc = p0.x * bf2f(qv.x & 0xffffu);
      acc = fmaf(p0.y, bf2f(qv.x >> 16), acc);
      acc = fmaf(p0.z, bf2f(qv.y & 0xffffu), acc);
      acc = fmaf(p0.w, bf2f(qv.y >> 16), acc);
      acc = fmaf(p1.x, bf2f(qv.z & 0xffffu), acc);
      acc = fmaf(p1.y, bf2f(qv.z >> 16), acc);
      acc = fmaf(p1.z, bf2f(qv.w & 0xffffu), acc);
      acc = fmaf(p1.w, bf2f(qv.w >> 16), acc);
    }
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
    if (c == 0 && j < a.r) qt[j] = acc;
  }
  __syncthreads();
  const float* cb = cent + row_id * a.nbmax * a.r;
  float* srow = cscores + row_id * a.nbmax;
  const bool in_lds = n_c <= TK_LDS;
  // clustered decode: candidate e (id e + 1) is an empty cluster when
  // e + 1 < m and its offsets are equal; it then gets the lowest key (0,
  // the order key of the NaN bit pattern 0xffffffff), below every score
  const int32_t* coff = a.cl_off ? a.cl_off + row_id * (a.nbmax + 1) : nullptr;
  const int cm = a.cl_off ? min(a.cl_m[b], n_b - a.n_recent) : 0;
  // Candidate scores, several candidates per thread in flight; a centroid
  // row is r floats read as float4 (consecutive lanes read consecutive
  // rows). For r = 16 every load of a group of candidates is issued before
  // the first is used, so the row costs a few memory latencies, not one per
  // float4.
  auto empty_at = [&](int e) {
    return coff && e + 1 < cm && coff[e + 2] == coff[e + 1];
  };
  auto put = [&](int e, float v, bool empty) {
    if (empty) v = __uint_as_float(0xffffffffu);
    if (in_lds) keys[e + (e >> 5)] = order_key(v);
    else srow[e] = v;
  };
  if (a.r == 16) {
    constexpr int U = 8;
    for (int e0 = tid; e0 < n_c; e0 += U * 256) {
      float4 cv[U][4];
      bool emp[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int e = min(e0 + 256 * u, n_c - 1);
        const float4* crow = reinterpret_cast<const float4*>(cb + (size_t)(e + 1) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) cv[u][i] = crow[i];
        emp[u] = empty_at(e);  // loaded with the centroids
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float sc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc = fmaf(qt[4 * i], cv[u][i].x, sc);
          sc = fmaf(qt[4 * i + 1], cv[u][i].y, sc);
          sc = fmaf(qt[4 * i + 2], cv[u][i].z, sc);
          sc = fmaf(qt[4 * i + 3], cv[u][i].w, sc);
        }
        const int e = e0 + 256 * u;
        if (e < n_c) put(e, sc, emp[u]);
      }
    }
  } else {
    for (int e0 = tid; e0 < n_c; e0 += 4 * 256) {
      float sc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int rr = 0; rr < a.r; rr += 4) {
        float4 cv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int e = min(e0 + 256 * u, n_c - 1);
          cv[u] = *reinterpret_cast<const float4*>(cb + (size_t)(e + 1) * a.r + rr);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          sc[u] = fmaf(qt[rr], cv[u].x, sc[u]);
          sc[u] = fmaf(qt[rr + 1], cv[u].y, sc[u]);
          sc[u] = fmaf(qt[rr + 2], cv[u].z, sc[u]);
          sc[u] = fmaf(qt[rr + 3], cv[u].w, sc[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + 256 * u;
        if (e < n_c) put(e, sc[u], empty_at(e));
      }
    }
  }
  __syncthreads();
  auto getk = [&](int e) -> uint32_t {
    return in_lds ? keys[e + (e >> 5)] : order_key(srow[e]);
  };
  if (a.top_k > kWaveTopkMax) radix_topk(getk, n_c, a.top_k, out + 1, 1, sh);
  else if (a.top_k > 0 && n_c <= 4 * 64 * 16)
    wave_topk_regs<16>(getk, n_c, a.top_k, out + 1, 1, wsh);
  else if (a.top_k > 0) wave_topk(getk, n_c, a.top_k, out + 1, 1, wsh);
  const int n_rec = n_b - 1 - n_c;  // = n_recent here
  if (tid == 0) {
    out[0] = 0;
    sel_cnt[row_id] = 1 + a.top_k + n_rec;
  }
  for (int j = tid; j < n_rec; j += 256) out[1 + a.top_k + j] = n_c + 1 + j;
  if (ta.tok) {
    // the kept ids are written by this block: after the barrier its waves
    // read them back (one CU, one L1), and turn them into the token list
    __syncthreads();
    build_token_list(ta, out, 1 + a.top_k + n_rec, L, n_b, a.n_recent, a.Lmax,
                     a.nbmax, row_id, b, tsh.tok);
  }
}

// ---------------------------------------------------------------- attention
struct DecAttnArgs {
  const u16* q; const u16* kc; const u16* vc; const int32_t* cache_len;
  const int32_t* sel; const int32_t* sel_cnt;
  float* part_o; float* part_ml;
  int Hq, Hkv, Lmax, n_ret, window, n_split, sel_width, n_units;
  int unit_base;  // the launch covers units unit_base .. unit_base + gridDim.y - 1
  float c;  // scale * log2(e)
  // unit u: bits 0-1 kind (0 window heads of one KV group, 1 retrieval
  // head), bits 8-15 KV head, bits 16-23 head count, bits 24-31 first index
  // into hlist
  // clustered decode: per (sequence, retrieval head) a list of tok_width
  // token ids, tok_cnt of them used (read by the token-list instance)
  const int32_t* tok; const int32_t* tok_cnt; int tok_width;
  KvView kv;  // paged cache (read by the kPaged instances)
  uint32_t desc[2 * kMaxHeads];
  uint8_t rho[2 * kMaxHeads];
  uint8_t hlist[kMaxHeads];
};

// K and V tiles of 32 keys in a wave's LDS, 256 B per key row in 16 chunks
// of 16 B. Both come from global memory in whole rows (load ins, 0..7, covers
// rows 4 ins .. 4 ins + 3: lane i takes position i & 15 of row 4 ins + i / 16,
// so each load and each LDS write is 1 KiB contiguous) and are stored
// swizzled so the MFMA operand reads hit distinct banks:
//  K: position p of row r holds d-chunk p ^ (r & 15) (an operand read takes
//     one chunk of 16 consecutive rows);
//  V: position p of row r holds d-chunk p ^ (4 ((r >> 3) & 1)) (a P.V operand
//     read takes one d of rows 8 apart).
constexpr int kDecTile = 32 * kD * 2;

// grid (n_split, n_units, B), 256 threads. Each wave takes 32-key tiles in
// turn (tiles wave, wave + 4, ...), independently of the other waves until
// the final merge. Both products run on MFMA with the unit's heads along N
// (so up to 32 heads share every K/V byte): S^T = K Q^T with K rows read in
// perm_row order, which makes the accumulator of S^T the B operand of
// O^T += V^T P; that product wants 8 consecutive keys of one d per lane, so V
// is read transposed from LDS. The next tile's K and V are loaded into
// registers (a whole iteration ahead) and written to LDS at the start of
// the next iteration; plain loads, not LDS DMA, keep the compiler's wait
// counts exact.
//
// kTok (clustered decode, retrieval units only): the keys are a list of
// token ids instead of blocks. Tile t of the list is entries 32 t .. 32 t +
// 31; splits take whole pairs of tiles, so with clusters equal to blocks
// every tile, split and wave sees exactly the keys of the block walk. Row r
// of a tile is gathered from token id (entry r), the ids of the next tile
// having been loaded one iteration ahead.
//
// kPaged: the cache is paged (KvView); a row's address goes through the
// block table, and a tile that straddles two pages takes the per-row loads.
template <bool kTok, bool kPaged>
__global__ __launch_bounds__(256, 2) void dec_attn_kernel(const DecAttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char kvbuf[4][2][kDecTile];
  __shared__ float red_ml[4][kDecMaxUnitHeads][2];
  const int s = blockIdx.x, u = a.unit_base + blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, n = lane & 31;
  const uint32_t desc = a.desc[u];
  const int kind = desc & 3, kvh = (desc >> 8) & 255, nh = (desc >> 16) & 255,
            first = desc >> 24;
  int L = a.cache_len[b];
  L = L < 1 ? 1 : (L > a.Lmax ? a.Lmax : L);

  // key tiles of this split
  int nt = 0, k_begin = 0, k_end = 0, blk0 = 0;
  // The selection is read-only here: the constant address space lets the
  // compiler use scalar loads, which leave the K/V prefetch waits alone.
  typedef __attribute__((address_space(4))) const int32_t* const_i32_ptr;
  const_i32_ptr list = nullptr;
  if (kind == 0) {
    const int lo = max(0, L - a.window);
    const int nk = L - lo;
    const int per = ((nk + a.n_split - 1) / a.n_split + 31) & ~31;
    k_begin = min(lo + s * per, L);
    k_end = min(lo + (s + 1) * per, L);
    nt = (k_end - k_begin + 31) / 32;
  } else if (!kTok) {
    const int rho = a.rho[u];
    const int nsel = a.sel_cnt[(size_t)b * a.n_ret + rho];
    list = (const_i32_ptr)(a.sel + ((size_t)b * a.n_ret + rho) * a.sel_width);
    const int bps = (nsel + a.n_split - 1) / a.n_split;
    blk0 = min(s * bps, nsel);
    const int blk1 = min(blk0 + bps, nsel);
    nt = 2 * (blk1 - blk0);
  }
  // token-list mode: entries T0*32 .. of a list of n_tok token ids
  const int32_t* tl = nullptr;
  int n_tok = 0, T0 = 0;
  if (kTok && kind == 1) {
    const size_t row = (size_t)b * a.n_ret + a.rho[u];
    n_tok = a.tok_cnt[row];
    tl = a.tok + row * a.tok_width;
    const int ntile = (n_tok + 31) / 32;
    const int per = 2 * (((ntile + 1) / 2 + a.n_split - 1) / a.n_split);
    T0 = min(s * per, ntile);
    nt = min(per, ntile - T0);
  }

  // rows: contiguous, kbase + key * kD; paged, the pool base plus the
  // offset of the key's page row
  const size_t kv_off = kPaged ? 0 : ((size_t)b * a.Hkv + kvh) * a.Lmax * kD;
  const u16* kbase = a.kc + kv_off;
  const u16* vbase = a.vc + kv_off;
  auto roff = [&](int key) -> size_t {
    if constexpr (kPaged) return kv_row(a.kv, b, a.Hkv, kvh, a.Lmax, key);
    else return (size_t)key * kD;
  };

  // B operand of S^T: Q^T, column n = head n of the unit (zero beyond nh)
  bf16x8 qf[8];
  {
    const int h = n < nh ? a.hlist[first + n] : a.hlist[first];
    const u16* qp = a.q + ((size_t)b * a.Hq + h) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(qp + 16 * ks);
      if (n >= nh) { bf16x8 z = {}; v = z; }
      qf[ks] = v;
    }
  }

  // tile t: first key and number of keys (0: past this wave's work)
  auto tile_at = [&](int t, int& base, int& nvalid) {
    base = 0;
    nvalid = 0;
    if (t < nt) {
      if (kTok) {
        nvalid = min(32, n_tok - 32 * (T0 + t));
      } else if (kind == 0) {
        base = k_begin + 32 * t;
        nvalid = min(32, k_end - base);
      } else {
        const int blk = list[__builtin_amdgcn_readfirstlane(blk0 + (t >> 1))];
        base = blk * 64 + 32 * (t & 1);
        nvalid = max(0, min(32, L - base));
        if (nvalid == 0) base = 0;
      }
    }
  };
  // whole-row loads of one tile (K or V, by swizzle); rows past nvalid
  // re-read the tile's first row (never NaN garbage: their P is exactly 0)
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  // Full tiles: one uniform tile address plus per-lane offsets (the
  // swizzle of row 4 ins + lane / 16 repeats every 4 loads for K and every
  // 2 for V, and each load is 1 KiB further on).
  uint32_t koff[4], voff[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * j + (lane >> 4);
    koff[j] = (uint32_t)(r * 256 + (((lane & 15) ^ (r & 15)) << 4));
  }
#pragma unroll
  for (int j = 0; j < 2; ++j)
    voff[j] = (uint32_t)((lane >> 4) * 256 + (((lane & 15) ^ (4 * j)) << 4));
  auto load_rows = [&](const u16* src, int base, int nvalid, bool kswz,
                       u32x4 (&st)[8]) {
    // wave-uniform: a full tile inside one page (always, unpaged)
    if (nvalid == 32 && (!kPaged || (base & 63) <= 32)) {
      const char* t = reinterpret_cast<const char*>(src + roff(base));
#pragma unroll
      for (int ins = 0; ins < 8; ++ins) {
        const uint32_t off = kswz ? koff[ins & 3] + (ins >> 2) * 4096
                                  : voff[(ins >> 1) & 1] + (ins >> 1) * 2048 +
                                        (ins & 1) * 1024;
        st[ins] = *reinterpret_cast<const u32x4*>(t + off);
      }
    } else {
#pragma unroll
      for (int ins = 0; ins < 8; ++ins) {
        const int r = 4 * ins + (lane >> 4);
        const int chunk = (lane & 15) ^ (kswz ? (r & 15) : 4 * ((r >> 3) & 1));
        const u16* p = src + roff(r < nvalid ? base + r : base) + chunk * 8;
        st[ins] = *reinterpret_cast<const u32x4*>(p);
      }
    }
  };
  // token-list mode: lane l < 32 holds the id of entry l of tile t (past
  // the list: the last entry, a valid row whose weight is 0); ids of the 32
  // rows of a tile then come from that lane by a cross-lane read
  auto ids_of = [&](int t) -> int {
    if (t >= nt) return 0;
    return tl[min(32 * (T0 + t) + (lane & 31), n_tok - 1)];
  };
  auto load_rows_tok = [&](const u16* src, int idv, bool kswz, u32x4 (&st)[8]) {
#pragma unroll
    for (int ins = 0; ins < 8; ++ins) {
      const int r = 4 * ins + (lane >> 4);
      const int id = __shfl(idv, r);
      const int chunk = (lane & 15) ^ (kswz ? (r & 15) : 4 * ((r >> 3) & 1));
      st[ins] = *reinterpret_cast<const u32x4*>(src + roff(id) + chunk * 8);
    }
  };
  char* const ktile = kvbuf[wave][0];
  char* const vtile = kvbuf[wave][1];
  auto store_rows = [&](char* tile, const u32x4 (&st)[8]) {
#pragma unroll
    for (int ins = 0; ins < 8; ++ins)
      *reinterpret_cast<u32x4*>(tile + ins * 1024 + lane * 16) = st[ins];
  };
  // A operand of S^T, step ks: lane (g, n) holds K[perm_row(n)][16 ks + 8 g
  // .. + 7]
  auto k_frag = [&](int ks) {
    const int r = perm_row(n);
    return *reinterpret_cast<const bf16x8*>(ktile + r * 256 +
                                            (((2 * ks + g) ^ (r & 15)) << 4));
  };
  // A operand of O^T += V^T P for keys 16 c .. 16 c + 15 and d 32 mt ..
  // 32 mt + 31: lane (g, n) holds V[16 c + 8 g + e][32 mt + n], e = 0..7
  auto v_frag = [&](const char* buf, int c, int mt) {
    const int d = 32 * mt + n;
    const char* p = buf + (16 * c + 8 * g) * 256 + (((d >> 3) ^ (4 * g)) << 4) +
                    (d & 7) * 2;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)*reinterpret_cast<const u16*>(p + 2 * e * 256) |
             ((uint32_t)*reinterpret_cast<const u16*>(p + (2 * e + 1) * 256) << 16);
    return __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  };

  float m_run = -1e30f, l_run = 0.f;  // softmax state of head n (lane pair)
  f32x16 o[4];  // O^T: element i of o[mt] is d = 32 mt + 8 (i/4) + 4 g + i%4
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) o[mt] = f32x16{};

  int base, nvalid;
  tile_at(wave, base, nvalid);
  u32x4 kst[8], vst[8];
  int idn = 0;
  if (kTok) {
    const int idv = ids_of(wave);
    load_rows_tok(kbase, idv, true, kst);
    load_rows_tok(vbase, idv, false, vst);
    idn = ids_of(4 + wave);
  } else {
    load_rows(kbase, base, nvalid, true, kst);
    load_rows(vbase, base, nvalid, false, vst);
  }
  const int iters = (nt + 3) / 4;
  for (int it = 0; it < iters; ++it) {
    // this tile to LDS (the previous tile's reads are done: a wave's LDS
    // operations complete in order), then the next tile into the registers,
    // in flight for the whole iteration. Past the wave's last tile the loads
    // re-read one row (cache hits), so every iteration issues the same loads.
    store_rows(ktile, kst);
    store_rows(vtile, vst);
    int nbase, nnvalid;
    tile_at((it + 1) * 4 + wave, nbase, nnvalid);
    if (kTok) {
      load_rows_tok(kbase, idn, true, kst);
      load_rows_tok(vbase, idn, false, vst);
      idn = ids_of((it + 2) * 4 + wave);
    } else {
      load_rows(kbase, nbase, nnvalid, true, kst);
      load_rows(vbase, nbase, nnvalid, false, vst);
    }
    if (nvalid > 0) {  // wave-uniform
      f32x16 sacc = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) sacc = mfma32(k_frag(ks), qf[ks], sacc);
      // element i: key 16 (i/8) + 8 g + i%8 of the tile, head n
      if (nvalid < 32) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (16 * (i >> 3) + 8 * g + (i & 7) >= nvalid) sacc[i] = -INFINITY;
      }
      float tmax = sacc[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, sacc[i]);
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
      const float m_new = fmaxf(m_run, tmax);
      if (__any(m_new > m_run)) {  // rescale only when some head's max rose
        const float alpha = fast_exp2((m_run - m_new) * a.c);
        l_run *= alpha;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[mt][i] *= alpha;
        m_run = m_new;
      }
      const float mc = m_run * a.c;
      const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
      bf16x8 pb[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        uint32_t w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 8 * c + 2 * e;
          w[e] = pack_bf16x2(fast_exp2(fmaf(sacc[i], a.c, -mc)),
                             fast_exp2(fmaf(sacc[i + 1], a.c, -mc)));
          // l sums the rounded weights that P.V uses
          l_run = __builtin_amdgcn_fdot2_f32_bf16(
              __builtin_bit_cast(bf16x2, w[e]), one, l_run, false);
        }
        pb[c] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
      }
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          o[mt] = mfma32(v_frag(vtile, c, mt), pb[c], o[mt]);
    }
    base = nbase;
    nvalid = nnvalid;
  }

  // wave-level totals: l over the lane pair; O^T columns of the unit's heads
  // go to this wave's own (now idle) K and V tiles (16 KiB: 32 heads x 128 d)
  l_run += __shfl_xor(l_run, 32);
  float* const red_o = reinterpret_cast<float*>(ktile);  // [head][d]
  static_assert(kDecMaxUnitHeads * kD * 4 <= 2 * kDecTile, "fits the tiles");
  if (n < nh) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float4 w;
        w.x = o[mt][4 * q + 0];
        w.y = o[mt][4 * q + 1];
        w.z = o[mt][4 * q + 2];
        w.w = o[mt][4 * q + 3];
        *reinterpret_cast<float4*>(red_o + n * kD + 32 * mt + 8 * q + 4 * g) = w;
      }
  }
  if (g == 0 && n < kDecMaxUnitHeads) {
    red_ml[wave][n][0] = m_run;
    red_ml[wave][n][1] = l_run;
  }
  __syncthreads();
  // merge the 4 waves and write this split's partial state
  for (int idx = tid; idx < nh * kD; idx += 256) {
    const int j = idx / kD, d = idx % kD;
    float M = -1e30f;
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red_ml[w][j][0]);
    float acc = 0.f, lsum = 0.f;
    for (int w = 0; w < 4; ++w) {
      const float f = fast_exp2((red_ml[w][j][0] - M) * a.c);
      acc += f * reinterpret_cast<const float*>(kvbuf[w][0])[j * kD + d];
      lsum += f * red_ml[w][j][1];
    }
    const int h = a.hlist[first + j];
    const size_t pidx = ((size_t)b * a.Hq + h) * a.n_split + s;
    a.part_o[pidx * kD + d] = acc;
    if (d == 0) {
      a.part_ml[pidx * 2 + 0] = M;
      a.part_ml[pidx * 2 + 1] = lsum;
    }
  }
}

// grid (Hq, B), 128 threads: combine the splits of one (sequence, head).
__global__ __launch_bounds__(128) void dec_merge_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_ml,
    int Hq, int n_split, float c, u16* __restrict__ out, float* __restrict__ lse) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const size_t p0 = ((size_t)b * Hq + h) * n_split;
  float M = -1e30f;
  for (int s = 0; s < n_split; ++s) M = fmaxf(M, part_ml[(p0 + s) * 2]);
  float acc = 0.f, l = 0.f;
  for (int s = 0; s < n_split; ++s) {
    const float f = fast_exp2((part_ml[(p0 + s) * 2] - M) * c);
    acc += f * part_o[(p0 + s) * kD + d];
    l += f * part_ml[(p0 + s) * 2 + 1];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  out[((size_t)b * Hq + h) * kD + d] = f2bf(acc * inv);
  if (lse && d == 0)
    lse[(size_t)b * Hq + h] = (M * c + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
}

// Streaming-head attention needs no block choice, so it runs on the
// device's auxiliary stream (AuxFork), concurrently with the block choice and
// the retrieval-head attention on the caller's stream; the merge waits for
// both.
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t st) {
  if (a.B == 0) return hipSuccess;
  const int G = a.Hq / a.Hkv;
  const int nbmax = a.Lmax / 64;
  const int width = a.top_k + 1 + a.n_recent;
  DecSelArgs sa;
  sa.Hq = a.Hq;
  sa.Lmax = a.Lmax;
  sa.n_ret = a.n_ret;
  sa.r = a.r;
  sa.nbmax = nbmax;
  sa.top_k = a.top_k;
  sa.n_recent = a.n_recent;
  sa.width = width;
  sa.cl_m = a.cl_m;
  sa.cl_off = a.cl_off;
  for (int i = 0; i < kMaxHeads; ++i) sa.head_of_rho[i] = i < a.n_ret ? a.ret_heads[i] : 0;
  const bool clustered = a.cl_off != nullptr;
  DecAttnArgs da;
  da.q = a.q;
  da.kc = a.kc;
  da.vc = a.vc;
  da.cache_len = a.cache_len;
  da.sel = a.sel;
  da.sel_cnt = a.sel + (size_t)a.B * a.n_ret * width;
  da.part_o = a.part_o;
  da.part_ml = a.part_ml;
  da.Hq = a.Hq;
  da.Hkv = a.Hkv;
  da.Lmax = a.Lmax;
  da.n_ret = a.n_ret;
  da.window = a.window;
  da.n_split = a.n_split;
  da.sel_width = width;
  da.c = a.scale * 1.4426950408889634f;
  da.tok = a.tok;
  da.tok_cnt = a.tok_cnt;
  da.tok_width = a.Lmax;
  da.kv = a.kv;
  const bool paged = a.kv.table != nullptr;
  // units: window heads of each KV group (up to kDecMaxUnitHeads per unit)
  // first, then one unit per retrieval head
  int nu = 0, nl = 0, rho = 0;
  for (int g = 0; g < a.Hkv; ++g) {
    int cnt = 0, start = nl;
    for (int h = g * G; h < (g + 1) * G; ++h) {
      if (a.is_ret[h]) continue;
      da.hlist[nl++] = (uint8_t)h;
      if (++cnt == kDecMaxUnitHeads) {
        da.desc[nu] = 0u | ((uint32_t)g << 8) | ((uint32_t)cnt << 16) | ((uint32_t)start << 24);
        da.rho[nu++] = 0;
        cnt = 0;
        start = nl;
      }
    }
    if (cnt) {
      da.desc[nu] = 0u | ((uint32_t)g << 8) | ((uint32_t)cnt << 16) | ((uint32_t)start << 24);
      da.rho[nu++] = 0;
    }
  }
  const int n_win_units = nu;
  for (int h = 0; h < a.Hq; ++h) {
    if (!a.is_ret[h]) continue;
    da.hlist[nl] = (uint8_t)h;
    da.desc[nu] = 1u | ((uint32_t)(h / G) << 8) | (1u << 16) | ((uint32_t)nl << 24);
    da.rho[nu++] = (uint8_t)rho++;
    ++nl;
  }
  da.n_units = nu;
  const int n_ret_units = nu - n_win_units;

  DecTokArgs ta;
  ta.cl_m = a.cl_m;
  ta.cl_off = a.cl_off;
  ta.cl_mem = a.cl_mem;
  ta.tok = clustered ? a.tok : nullptr;
  ta.tok_cnt = a.tok_cnt;
  auto select = [&]() {
    prof_begin("dec_select", st);
    hipLaunchKernelGGL(dec_select_kernel, dim3(a.n_ret, a.B), dim3(256), 0, st,
                       a.q, a.p_q, a.cent, a.cache_len, sa, a.cscores, a.sel,
                       a.sel + (size_t)a.B * a.n_ret * width, ta);
    prof_end(st);
  };
  auto attend = [&](const char* name, int base, int n, hipStream_t on) {
    DecAttnArgs d = da;
    d.unit_base = base;
    prof_begin(name, on);
    const dim3 grid(a.n_split, n, a.B);
    const bool tok = clustered && base >= n_win_units;  // retrieval units
    if (tok && paged)
      hipLaunchKernelGGL((dec_attn_kernel<true, true>), grid, dim3(256), 0, on, d);
    else if (tok)
      hipLaunchKernelGGL((dec_attn_kernel<true, false>), grid, dim3(256), 0, on, d);
    else if (paged)
      hipLaunchKernelGGL((dec_attn_kernel<false, true>), grid, dim3(256), 0, on, d);
    else
      hipLaunchKernelGGL((dec_attn_kernel<false, false>), grid, dim3(256), 0, on, d);
    prof_end(on);
  };
  hipError_t e = hipSuccess;
  if (!a.one_stream && n_win_units > 0 && n_ret_units > 0) {
    AuxFork fork(st);
    if ((e = fork.status()) != hipSuccess) return e;
    attend("dec_attn_window", 0, n_win_units, fork.stream());
    if ((e = hipGetLastError()) != hipSuccess) return e;
    select();
    attend("dec_attn_retrieval", n_win_units, n_ret_units, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = fork.join()) != hipSuccess) return e;
  } else {
    if (a.n_ret > 0) select();
    if (n_win_units > 0) attend("dec_attn_window", 0, n_win_units, st);
    if (n_ret_units > 0) attend("dec_attn_retrieval", n_win_units, n_ret_units, st);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin("dec_merge", st);
  hipLaunchKernelGGL(dec_merge_kernel, dim3(a.Hq, a.B), dim3(kD), 0, st,
                     a.part_o, a.part_ml, a.Hq, a.n_split, da.c, a.out, a.lse);
  prof_end(st);
  return hipGetLastError();
}

}  // namespace rtp
