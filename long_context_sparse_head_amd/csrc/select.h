// Block-wide exact top-k selection (256 threads), shared by the prefill
// indexer and the decode block choice.
//
// The k largest of n candidate scores (ties: lower candidate index first) are
// found by a 4-pass, 8-bit radix select on order-preserving 32-bit keys, then
// written in ascending index order by a prefix sum over thread-contiguous
// chunks. The result is exact and deterministic (LDS atomics only build
// histograms, whose totals do not depend on order).
#pragma once
#include "common.h"

namespace rtp {

constexpr int TK_LDS = 16384;  // candidates held in LDS (longer rows: global)

__device__ __forceinline__ uint32_t order_key(float f) {
  if (f == 0.f) f = 0.f;  // -0 and +0 compare equal
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Inclusive scan of one int per thread over a 256-thread block.
__device__ __forceinline__ int block_incl_scan(int v, int* tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  if (lane == 63) tmp[wave] = v;
  __syncthreads();
  int add = 0;
  for (int w = 0; w < wave; ++w) add += tmp[w];
  __syncthreads();
  return v + add;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, int* tmp) {
  for (int off = 32; off >= 1; off >>= 1)
    v = max(v, (uint32_t)__shfl_xor((int)v, off));
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = (int)v;
  __syncthreads();
  uint32_t r = 0u;
  for (int w = 0; w < 4; ++w) r = max(r, (uint32_t)tmp[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, int* tmp) {
  for (int off = 32; off >= 1; off >>= 1)
    v = min(v, (uint32_t)__shfl_xor((int)v, off));
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = (int)v;
  __syncthreads();
  uint32_t r = 0xffffffffu;
  for (int w = 0; w < 4; ++w) r = min(r, (uint32_t)tmp[w]);
  __syncthreads();
  return r;
}

struct TopkShared {
  int hist[256];
  int tmp[8];
  int bcast[4];
};

struct TopkResult {
  uint32_t T;       // key of the k-th largest candidate
  int count_ge;     // candidates with key >= T (block-uniform)
};

// Requires 1 <= k < n. getk(e) returns the key of candidate e (0 <= e < n).
// Writes out[0..k-1] = idx_base + chosen e, ascending. Every thread of the
// block must call it.
template <class GetK>
__device__ TopkResult radix_topk(GetK getk, int n, int k, int32_t* out,
                                 int idx_base, TopkShared& sh) {
  const int tid = threadIdx.x;
  const int C = (n + 255) / 256;
  const int e0 = min(tid * C, n), e1 = min(e0 + C, n);
  uint32_t prefix = 0, pmask = 0;
  int kk = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    sh.hist[tid] = 0;
    __syncthreads();
    for (int e = e0; e < e1; ++e) {
      const uint32_t key = getk(e);
      if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    const int b = 255 - tid;  // thread t covers bin 255-t: scan from the top
    const int h = sh.hist[b];
    const int incl = block_incl_scan(h, sh.tmp);  // keys with digit >= b
    const int gt = incl - h;                      // keys with digit > b
    if (h > 0 && gt < kk && kk <= incl) {
      sh.bcast[0] = b;
      sh.bcast[1] = gt;
    }
    __syncthreads();
    prefix |= (uint32_t)sh.bcast[0] << shift;
    pmask |= 0xffu << shift;
    kk -= sh.bcast[1];
    __syncthreads();
  }
  const uint32_t T = prefix;  // kk = how many keys equal to T are taken
  int ngt = 0, neq = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t key = getk(e);
    ngt += key > T;
    neq += key == T;
  }
  const int eq_incl = block_incl_scan(neq, sh.tmp);
  const int take_eq = max(0, min(kk - (eq_incl - neq), neq));
  const int ntake = ngt + take_eq;
  const int pos_incl = block_incl_scan(ntake, sh.tmp);
  const int ge_incl = block_incl_scan(ngt + neq, sh.tmp);
  if (tid == 255) sh.bcast[2] = ge_incl;
  int pos = pos_incl - ntake;
  int eq_seen = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t key = getk(e);
    bool t = key > T;
    if (key == T) {
      t = eq_seen < take_eq;
      ++eq_seen;
    }
    if (t) out[pos++] = idx_base + e;
  }
  __syncthreads();
  TopkResult res;
  res.T = T;
  res.count_ge = sh.bcast[2];
  return res;
}

}  // namespace rtp
