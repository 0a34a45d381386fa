// Semantic K-cache clustering for gfx950: k-means (Lloyd) of the projected
// keys of every (sequence, retrieval head), seeded by the block centroids.
//
// What it computes (RTPurboV2 article, paragraph on the synergy of feature
// and sequence compression: after the low-rank projection, keys of related
// meaning lie close together and unrelated ones far apart, so whole groups
// of unrelated tokens can be skipped; Qwen3-Coder recipe paragraph: the K
// cache is clustered in prefill and decode runs sparsely). The pages give no
// algorithm; this library's reading:
//   points   x_t = P_k k_t, t in blocks 1 .. m-1, m = max(n_b - n_recent, 1)
//            (fp32, projected on the matrix cores as in the indexer)
//   clusters ids 1 .. m-1, id c starting from the centroid table's entry c
//            (the block centroid after rtp_build_centroids)
//   one step assign every point to the nearest centroid (Euclidean; ties:
//            lower id), then move every cluster with members to their mean;
//            a cluster without members keeps its centroid
//   tables   members of each cluster, ascending token order, and offsets.
//
// Kernels of one step:
//   cl_assign_kernel  nearest centroid, as argmax_c x.mu_c - |mu_c|^2 / 2: a
//                     K = r contraction on bf16 MFMA with split operands
//                     (x_hi.mu_hi + x_hi.mu_lo + x_lo.mu_hi, and the bias by
//                     one more MFMA against a constant operand), the running
//                     best per (token, cluster column) in registers, one
//                     cross-lane reduction at the end; member counts per
//                     (chunk of tokens, cluster) by atomics (order-free).
//   cl_scan_kernel    cluster offsets and each chunk's first slot per
//                     cluster (exclusive scans).
//   cl_place_kernel   members grouped by cluster in ascending token order:
//                     one wave per chunk walks its tokens in order.
//   cl_update_kernel  the mean of each cluster's members, summed in fp64 in
//                     a fixed order.
// Everything is deterministic: no atomic takes part in a floating-point sum
// or decides an order.
#include "common.h"
#include "proj.h"
#include "select.h"

namespace rtp {

struct ClArgs {
  const u16* kc; const int32_t* cache_len; const float* p_k;
  KvView kv;
  float* x;         // [B, n_ret, Lmax, r] projected keys (rows of clustered tokens)
  int32_t* assign;  // [B, n_ret, Lmax] cluster id of each clustered token
  int32_t* hist;    // [B, n_ret, kClChunks, nbmax] counts, then first slots
  float* cent;      // [B, n_ret, nbmax, r]
  int32_t* cl_m;    // [B]
  int32_t* cl_off;  // [B, n_ret, nbmax + 1]
  int32_t* cl_mem;  // [B, n_ret, Lmax]
  int Hkv, Lmax, nbmax, n_ret, r, n_recent;
  uint8_t kvh_of_rho[kMaxHeads];
};

__device__ __forceinline__ int cl_count(const ClArgs& a, int b) {
  int L = a.cache_len[b];
  L = L < 0 ? 0 : (L > a.Lmax ? a.Lmax : L);
  return max((L + 63) / 64 - a.n_recent, 1);
}

// Tokens 64 .. 64m-1 (candidate index t = token - 64) are split into at most
// kClChunks chunks of cl_chunk_len(m) tokens (a multiple of 64).
__device__ __forceinline__ int cl_chunk_len(int m) {
  return 64 * ((m - 1 + kClChunks - 1) / kClChunks);
}

// ------------------------------------------------------------ projection
// grid (ceil(nbmax / 4), n_ret, B), 4 waves, a wave per 64-token block kb
// (1 <= kb < m): x_t = P_k k_t in fp32, as in the indexer's projection: the
// head's rows of P_k staged 32 at a time in LDS as three bf16 parts and
// multiplied with the block's keys on the matrix cores (proj.h).
__global__ __launch_bounds__(256) void cl_project_kernel(const ClArgs a) {
  __shared__ __attribute__((aligned(16))) char ptile[kProjTileB];
  const int rho = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kb = 4 * blockIdx.x + wave;
  const int m = cl_count(a, b);
  if (4 * blockIdx.x >= m) return;  // whole workgroup
  const bool ok = kb >= 1 && kb < m;
  bf16x8 kbop[2][8];
  proj_keys_operands(a.kc + kv_row(a.kv, b, a.Hkv, a.kvh_of_rho[rho], a.Lmax,
                                   ok ? kb * 64 : 0),
                     ok ? 64 : 0, kbop);
  const float* P = a.p_k + (size_t)rho * a.r * kD;
  const int gq = lane >> 5, n = lane & 31;
  for (int m0 = 0; m0 < a.r; m0 += 32) {
    __syncthreads();
    proj_stage(P, m0, a.r, ptile);
    __syncthreads();
    if (!ok) continue;
    f32x16 acc[2];
    proj_tile(ptile, kbop, acc);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int R = m0 + 16 * half;
      if (R >= a.r) break;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        float* xo = a.x + (((size_t)b * a.n_ret + rho) * a.Lmax + (size_t)kb * 64 +
                           32 * mt + n) * a.r + R + 8 * gq;
        *reinterpret_cast<float4*>(xo) =
            make_float4(acc[mt][8 * half], acc[mt][8 * half + 1],
                        acc[mt][8 * half + 2], acc[mt][8 * half + 3]);
        *reinterpret_cast<float4*>(xo + 4) =
            make_float4(acc[mt][8 * half + 4], acc[mt][8 * half + 5],
                        acc[mt][8 * half + 6], acc[mt][8 * half + 7]);
      }
    }
  }
}

// -------------------------------------------------------------- E-step
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], bf16x8& hi,
                                             bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const u16 h0 = f2bf(v[2 * e]), h1 = f2bf(v[2 * e + 1]);
    h[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    l[e] = pack_bf16x2(v[2 * e] - bf2f(h0), v[2 * e + 1] - bf2f(h1));
  }
  hi = __builtin_bit_cast(bf16x8, make_uint4(h[0], h[1], h[2], h[3]));
  lo = __builtin_bit_cast(bf16x8, make_uint4(l[0], l[1], l[2], l[3]));
}

// grid (ceil(nbmax / 4), n_ret, B), 256 threads: 256 clustered tokens per
// workgroup, 64 per wave as two 32-token tiles (the A operand: token rows,
// kept in registers). Clusters stream through LDS, 256 per stage; each
// 32-cluster tile is the B operand (cluster columns). Accumulator element i
// of lane (g, n) scores token row 8 (i/4) + 4 g + i%4 against cluster
// column n; the lane keeps, per token row, the best score over the tiles
// and the tile it came from (strictly greater only: ties keep the earlier,
// lower cluster).
template <int R16>
__global__ __launch_bounds__(256, 2) void cl_assign_kernel(const ClArgs a) {
  constexpr int R = 16 * R16;
  constexpr int ROWB = 32 * R16 + 16;  // bytes per cluster row (padded: the
                                       // 16-byte operand reads of 8 lanes
                                       // then hit distinct banks)
  constexpr int CS = 256;              // clusters per stage
  __shared__ __attribute__((aligned(16))) char hi_s[CS * ROWB];
  __shared__ __attribute__((aligned(16))) char lo_s[CS * ROWB];
  __shared__ __attribute__((aligned(16))) uint32_t nb_s[CS][2];
  const int rho = blockIdx.y, b = blockIdx.z;
  const int m = cl_count(a, b);
  const int C = m - 1, n_tok = 64 * C;
  const int t_base = 256 * blockIdx.x;
  if (t_base >= n_tok) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, n = lane & 31;
  const size_t bh = (size_t)b * a.n_ret + rho;
  const float* xb = a.x + (bh * a.Lmax + 64) * R;
  const float* cb = a.cent + (bh * a.nbmax + 1) * R;

  bf16x8 xh[2][R16], xl[2][R16];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int t = min(t_base + 64 * wave + 32 * j + n, n_tok - 1);
    const float* xp = xb + (size_t)t * R + 8 * g;
#pragma unroll
    for (int ks = 0; ks < R16; ++ks) {
      const float4 v0 = *reinterpret_cast<const float4*>(xp + 16 * ks);
      const float4 v1 = *reinterpret_cast<const float4*>(xp + 16 * ks + 4);
      const float v[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      split_bf16x8(v, xh[j][ks], xl[j][ks]);
    }
  }
  // A operand of the bias product: ones at k = 0, 1, 2 of every row
  bf16x8 ones = {};
  if (g == 0) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    const uint32_t o1 = __builtin_bit_cast(uint32_t, one);
    ones = __builtin_bit_cast(bf16x8, make_uint4(o1, o1 & 0xffffu, 0u, 0u));
  }
  float best[2][16];
  int bidx[2][16];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      best[j][i] = -INFINITY;
      bidx[j][i] = 0;
    }

  for (int c0 = 0; c0 < C; c0 += CS) {
    __syncthreads();  // the previous stage has been read
    {
      // thread tid stages cluster c0 + tid: hi / lo parts and the bias
      // -|mu|^2 / 2 as three bf16 parts (columns past C score -inf)
      const int c = c0 + tid;
      float s2 = 0.f;
      char* hrow = hi_s + tid * ROWB;
      char* lrow = lo_s + tid * ROWB;
#pragma unroll
      for (int q = 0; q < 2 * R16; ++q) {
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (c < C) {
          const float4 v0 = *reinterpret_cast<const float4*>(cb + (size_t)c * R + 8 * q);
          const float4 v1 = *reinterpret_cast<const float4*>(cb + (size_t)c * R + 8 * q + 4);
          v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w;
          v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) s2 = fmaf(v[e], v[e], s2);
        bf16x8 h, l;
        split_bf16x8(v, h, l);
        *reinterpret_cast<bf16x8*>(hrow + 16 * q) = h;
        *reinterpret_cast<bf16x8*>(lrow + 16 * q) = l;
      }
      uint32_t w0 = 0xff80u, w1 = 0u;  // -inf, 0, 0
      if (c < C) {
        const float nb = -0.5f * s2;
        const u16 p0 = f2bf(nb);
        const float r1 = nb - bf2f(p0);
        const u16 p1 = f2bf(r1);
        const u16 p2 = f2bf(r1 - bf2f(p1));
        w0 = (uint32_t)p0 | ((uint32_t)p1 << 16);
        w1 = p2;
      }
      nb_s[tid][0] = w0;
      nb_s[tid][1] = w1;
    }
    __syncthreads();
    const int n_ct = (min(CS, C - c0) + 31) / 32;
    for (int ct = 0; ct < n_ct; ++ct) {
      const int cl = 32 * ct + n;
      bf16x8 mh[R16], ml[R16];
#pragma unroll
      for (int ks = 0; ks < R16; ++ks) {
        mh[ks] = *reinterpret_cast<const bf16x8*>(hi_s + cl * ROWB + 32 * ks + 16 * g);
        ml[ks] = *reinterpret_cast<const bf16x8*>(lo_s + cl * ROWB + 32 * ks + 16 * g);
      }
      bf16x8 nbo = {};
      if (g == 0) {
        const uint2 w = *reinterpret_cast<const uint2*>(nb_s[cl]);
        nbo = __builtin_bit_cast(bf16x8, make_uint4(w.x, w.y, 0u, 0u));
      }
      const int tile = (c0 >> 5) + ct;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        f32x16 acc = mfma32(ones, nbo, f32x16{});
#pragma unroll
        for (int ks = 0; ks < R16; ++ks) {
          acc = mfma32(xl[j][ks], mh[ks], acc);
          acc = mfma32(xh[j][ks], ml[ks], acc);
          acc = mfma32(xh[j][ks], mh[ks], acc);
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const bool up = acc[i] > best[j][i];
          best[j][i] = up ? acc[i] : best[j][i];
          bidx[j][i] = up ? tile : bidx[j][i];
        }
      }
    }
  }

  // best over the 32 columns of each row (lanes n of one half g): larger
  // score, or equal score and lower cluster
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = best[j][i];
      int c = 32 * bidx[j][i] + n;
#pragma unroll
      for (int off = 16; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(v, off);
        const int oc = __shfl_xor(c, off);
        const bool take = ov > v || (ov == v && oc < c);
        v = take ? ov : v;
        c = take ? oc : c;
      }
      bidx[j][i] = c;
    }
  // lane (g, n < 16) writes token row 8 (n/4) + 4 g + n%4 of each tile
  const int CL = cl_chunk_len(m);
  int32_t* asg = a.assign + bh * a.Lmax;
  int32_t* hist = a.hist + bh * kClChunks * a.nbmax;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    int c = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) c = (i == n) ? bidx[j][i] : c;
    // a row whose scores all fail the comparisons (NaN inputs) keeps its
    // lane's column, possibly past C: it is then given cluster 0
    c = c < C ? c : 0;
    const int t = t_base + 64 * wave + 32 * j + 8 * (n >> 2) + 4 * g + (n & 3);
    if (n < 16 && t < n_tok) {
      asg[t] = c + 1;
      atomicAdd(&hist[(size_t)(t / CL) * a.nbmax + c], 1);
    }
  }
}

// ----------------------------------------------------------------- scans
// grid (n_ret, B), 256 threads: member count of every cluster (summed over
// the chunks), cluster offsets (cl_off[id] = first member slot of cluster
// id; cl_off[m] and later entries = the number of clustered tokens), and,
// in place of each chunk's counts, the first slot of that chunk's members
// of each cluster.
__global__ __launch_bounds__(256) void cl_scan_kernel(const ClArgs a) {
  __shared__ int tmp[4];
  __shared__ int carry_s;
  const int rho = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int m = cl_count(a, b), C = m - 1;
  const size_t bh = (size_t)b * a.n_ret + rho;
  int32_t* hist = a.hist + bh * kClChunks * a.nbmax;
  int32_t* off = a.cl_off + bh * (a.nbmax + 1);
  const int CL = cl_chunk_len(m);
  const int nch = C > 0 ? (64 * C + CL - 1) / CL : 0;
  if (rho == 0 && tid == 0) a.cl_m[b] = m;
  int carry = 0;
  for (int c0 = 0; c0 < C; c0 += 256) {
    const int c = c0 + tid;
    int tot = 0;
    if (c < C)
      for (int j = 0; j < nch; ++j) tot += hist[(size_t)j * a.nbmax + c];
    const int incl = block_incl_scan(tot, tmp);
    if (c < C) {
      int run = carry + incl - tot;
      off[c + 1] = run;
      for (int j = 0; j < nch; ++j) {
        const int h = hist[(size_t)j * a.nbmax + c];
        hist[(size_t)j * a.nbmax + c] = run;
        run += h;
      }
    }
    if (tid == 255) carry_s = carry + incl;
    __syncthreads();
    carry = carry_s;
    __syncthreads();
  }
  if (tid == 0) off[0] = 0;
  for (int id = m + tid; id <= a.nbmax; id += 256) off[id] = 64 * C;
}

// grid (kClChunks, n_ret, B), one wave: the members of chunk j, placed at
// their clusters' slots in ascending token order. The wave walks the
// chunk's tokens in order, 64 at a time. Lanes with the same cluster find
// each other with one ballot per bit of the cluster index; the lowest of
// them reserves the group's slots with one atomic on the chunk's next slot
// for that cluster (only this wave touches it, and each step waits for its
// atomics), and each lane takes the slot after those of the lower lanes.
__global__ __launch_bounds__(64) void cl_place_kernel(const ClArgs a) {
  const int j = blockIdx.x, rho = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int m = cl_count(a, b), C = m - 1, n_tok = 64 * C;
  const int CL = cl_chunk_len(m);
  const int t0 = j * CL, t1 = min(t0 + CL, n_tok);
  if (t0 >= t1) return;
  const size_t bh = (size_t)b * a.n_ret + rho;
  const int32_t* asg = a.assign + bh * a.Lmax;
  int32_t* next = a.hist + (bh * kClChunks + j) * a.nbmax;
  int32_t* mem = a.cl_mem + bh * a.Lmax;
  const int nbits = C > 1 ? 32 - __builtin_clz((unsigned)(C - 1)) : 0;
  const uint64_t below = lanes_below();
  for (int s = t0; s < t1; s += 64) {
    const int t = s + lane;
    const bool valid = t < t1;
    const int c = valid ? asg[t] - 1 : 0;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
      const bool set = (c >> bit) & 1;
      const uint64_t bl = __ballot(set);
      peers &= set ? bl : ~bl;
    }
    const int leader = peers ? __builtin_ctzll(peers) : 0;
    int pos = 0;
    if (valid && lane == leader) pos = atomicAdd(&next[c], __popcll(peers));
    pos = __shfl(pos, leader);
    if (valid) mem[pos + __popcll(peers & below)] = 64 + t;
  }
}

// -------------------------------------------------------------- M-step
// grid (ceil(nbmax / 4), n_ret, B), 256 threads, one wave per cluster: the
// mean of its members' projected keys. Lane (s, d) sums dim d of members
// s, s + 4, ... in fp64; the four partial sums are added pairwise. A cluster
// without members keeps its centroid.
__global__ __launch_bounds__(256) void cl_update_kernel(const ClArgs a) {
  const int rho = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int c = 4 * blockIdx.x + wave;  // cluster id c + 1
  const int m = cl_count(a, b), C = m - 1;
  if (c >= C) return;
  const size_t bh = (size_t)b * a.n_ret + rho;
  const int32_t* off = a.cl_off + bh * (a.nbmax + 1);
  const int o0 = off[c + 1], cnt = off[c + 2] - o0;
  if (cnt <= 0) return;
  const int32_t* mem = a.cl_mem + bh * a.Lmax + o0;
  const float* xb = a.x + bh * a.Lmax * a.r;
  float* out = a.cent + (bh * a.nbmax + c + 1) * a.r;
  const int s = lane >> 4, d = lane & 15;
  for (int d0 = 0; d0 < a.r; d0 += 16) {
    double acc = 0.0;
    for (int i = s; i < cnt; i += 4) acc += (double)xb[(size_t)mem[i] * a.r + d0 + d];
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    if (s == 0) out[d0 + d] = (float)(acc / (double)cnt);
  }
}

// --------------------------------------------------------- no Lloyd step
// grid (ceil((nbmax * 64) / 256), n_ret, B), 256 threads: the tables of
// clusters equal to the blocks (cluster id c holds the tokens of block c).
__global__ __launch_bounds__(256) void cl_identity_kernel(const ClArgs a) {
  const int rho = blockIdx.y, b = blockIdx.z;
  const int i = 256 * blockIdx.x + threadIdx.x;
  const int m = cl_count(a, b), n_tok = 64 * (m - 1);
  const size_t bh = (size_t)b * a.n_ret + rho;
  if (i < n_tok) a.cl_mem[bh * a.Lmax + i] = 64 + i;
  if (i <= a.nbmax) a.cl_off[bh * (a.nbmax + 1) + i] = i == 0 ? 0 : 64 * (min(i, m) - 1);
  if (rho == 0 && i == 0) a.cl_m[b] = m;
}

__global__ __launch_bounds__(256) void cl_zero_kernel(int32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n;
       i += (size_t)gridDim.x * 256)
    p[i] = 0;
}

template <int R16>
static void launch_steps(const ClArgs& a, int B, int iters, hipStream_t st) {
  const int gb = (a.nbmax + 3) / 4;
  prof_begin("cl_project", st);
  hipLaunchKernelGGL(cl_project_kernel, dim3(gb, a.n_ret, B), dim3(256), 0, st, a);
  prof_end(st);
  const size_t nh = (size_t)B * a.n_ret * kClChunks * a.nbmax;
  for (int it = 0; it < iters; ++it) {
    const size_t zb = (nh + 255) / 256;
    hipLaunchKernelGGL(cl_zero_kernel, dim3((unsigned)(zb < 8192 ? zb : 8192)),
                       dim3(256), 0, st, a.hist, nh);
    prof_begin("cl_assign", st);
    hipLaunchKernelGGL(cl_assign_kernel<R16>, dim3(gb, a.n_ret, B), dim3(256), 0,
                       st, a);
    prof_end(st);
    prof_begin("cl_scan", st);
    hipLaunchKernelGGL(cl_scan_kernel, dim3(a.n_ret, B), dim3(256), 0, st, a);
    prof_end(st);
    prof_begin("cl_place", st);
    hipLaunchKernelGGL(cl_place_kernel, dim3(kClChunks, a.n_ret, B), dim3(64), 0,
                       st, a);
    prof_end(st);
    prof_begin("cl_update", st);
    hipLaunchKernelGGL(cl_update_kernel, dim3(gb, a.n_ret, B), dim3(256), 0, st,
                       a);
    prof_end(st);
  }
}

hipError_t launch_cluster(const ClusterLaunch& L, hipStream_t st) {
  if (L.B == 0 || L.n_ret == 0 || L.Lmax < 64) return hipSuccess;
  ClArgs a;
  a.kc = L.kc;
  a.kv = L.kv;
  a.cache_len = L.cache_len;
  a.p_k = L.p_k;
  a.cent = L.cent;
  a.cl_m = L.cl_m;
  a.cl_off = L.cl_off;
  a.cl_mem = L.cl_mem;
  a.Hkv = L.Hkv;
  a.Lmax = L.Lmax;
  a.nbmax = L.Lmax / 64;
  a.n_ret = L.n_ret;
  a.r = L.r;
  a.n_recent = L.n_recent;
  for (int i = 0; i < kMaxHeads; ++i)
    a.kvh_of_rho[i] = i < L.n_ret ? L.ret_heads[i] / L.G : 0;
  const ClusterSizes z = cluster_sizes(L.B, L.Lmax, L.n_ret, L.r);
  a.x = reinterpret_cast<float*>(L.scratch + z.x);
  a.assign = reinterpret_cast<int32_t*>(L.scratch + z.assign);
  a.hist = reinterpret_cast<int32_t*>(L.scratch + z.hist);
  if (L.iters == 0) {
    prof_begin("cl_identity", st);
    hipLaunchKernelGGL(cl_identity_kernel, dim3((a.nbmax * 64 + 255) / 256, a.n_ret, L.B),
                       dim3(256), 0, st, a);
    prof_end(st);
    return hipGetLastError();
  }
  switch (L.r / 16) {
    case 1: launch_steps<1>(a, L.B, L.iters, st); break;
    case 2: launch_steps<2>(a, L.B, L.iters, st); break;
    case 3: launch_steps<3>(a, L.B, L.iters, st); break;
    case 4: launch_steps<4>(a, L.B, L.iters, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace rtp
