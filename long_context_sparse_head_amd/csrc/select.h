// Block-wide exact top-k selection (256 threads), shared by the prefill
// indexer and the decode block choice.
//
// The k largest of n candidate scores (ties: lower candidate index first) are
// found on order-preserving 32-bit keys (a value histogram locates the bin
// of the threshold, an exact radix select inside it finds the threshold),
// then written in ascending index order by a prefix sum over
// thread-contiguous chunks. The result is exact and deterministic (LDS
// atomics only build histograms and a candidate set whose order does not
// matter).
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

constexpr int TK_CAND = 2048;  // keys of the threshold bin held in LDS

struct TopkShared {
  int hist[256];
  int tmp[8];
  int bcast[4];
  int ncand;
  uint32_t cand[TK_CAND];
};

struct TopkResult {
  uint32_t T;       // key of the k-th largest candidate
  int count_ge;     // candidates with key >= T (block-uniform)
};

// The kk-th largest (1 <= kk <= count) of the keys key(i), i < m, for which
// pred(i) holds: a 4-pass, 8-bit radix select. Every thread of the block
// must call it; the result is block-uniform.
template <class Key, class Pred>
__device__ uint32_t radix_kth(Key key, Pred pred, int m, int kk,
                              TopkShared& sh) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    sh.hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < m; i += 256) {
      if (!pred(i)) continue;
      const uint32_t x = key(i);
      if ((x & pmask) == prefix) atomicAdd(&sh.hist[(x >> shift) & 255], 1);
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
  return prefix;
}

// Requires 1 <= k < n. getk(e) returns the key of candidate e (0 <= e < n).
// Writes out[0..k-1] = idx_base + chosen e, ascending (ties: lower e first).
// Every thread of the block must call it.
//
// The threshold T (the k-th largest key) is found in two steps: keys are
// histogrammed into 256 bins of a linear quantisation of their values
// between the row's minimum and maximum (order-preserving, and spread even
// when the values share a few exponents, unlike the top bits of the key),
// which fixes the bin holding T; the keys of that bin alone are then
// gathered in LDS and searched exactly. A bin too large to gather is
// searched in place.
template <class GetK>
__device__ TopkResult radix_topk(GetK getk, int n, int k, int32_t* out,
                                 int idx_base, TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int C = (n + 255) / 256;
  const int e0 = min(tid * C, n), e1 = min(e0 + C, n);
  // range of the non-NaN keys (NaN keys lie above +inf or below -inf)
  auto is_nan_key = [](uint32_t x) {
    return x > 0xff800000u || x < 0x007fffffu;
  };
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int e = e0; e < e1; ++e) {
    const uint32_t x = getk(e);
    if (!is_nan_key(x)) {
      lo = min(lo, x);
      hi = max(hi, x);
    }
  }
  lo = block_min_u32(lo, sh.tmp);
  hi = block_max_u32(hi, sh.tmp);
  float flo = 0.f, scale = 0.f;
  if (lo <= hi) {
    flo = order_key_inv(lo);
    const float span = order_key_inv(hi) - flo;
    if (span > 0.f) scale = 255.99f / span;
    if (!(scale < 1e30f)) scale = 0.f;  // inf span or tiny span: one bin
  }
  auto bin = [&](uint32_t x) -> int {
    if (x > 0xff800000u) return 255;  // +NaN keys
    if (x < 0x007fffffu) return 0;    // -NaN keys
    float f = (order_key_inv(x) - flo) * scale;
    f = fminf(fmaxf(f, 0.f), 255.f);  // NaN (inf * 0) -> 0
    return (int)f;
  };
  sh.hist[tid] = 0;
  __syncthreads();
  for (int e = e0; e < e1; ++e) atomicAdd(&sh.hist[bin(getk(e))], 1);
  __syncthreads();
  {
    const int b = 255 - tid;
    const int h = sh.hist[b];
    const int incl = block_incl_scan(h, sh.tmp);
    const int gt = incl - h;
    if (h > 0 && gt < k && k <= incl) {
      sh.bcast[0] = b;
      sh.bcast[1] = gt;
      sh.bcast[2] = h;
    }
    if (tid == 0) sh.ncand = 0;
    __syncthreads();
  }
  const int bstar = sh.bcast[0], kk = k - sh.bcast[1], nbin = sh.bcast[2];
  uint32_t T;
  if (nbin <= TK_CAND) {
    // gather the bin's keys (wave-aggregated appends)
    for (int i = 0; i < C; ++i) {
      const int e = e0 + i;
      const uint32_t x = e < e1 ? getk(e) : 0u;
      const bool in = e < e1 && bin(x) == bstar;
      const uint64_t bal = __ballot(in);
      if (bal) {
        int base = 0;
        if (lane == __builtin_ctzll(bal))
          base = atomicAdd(&sh.ncand, (int)__builtin_popcountll(bal));
        base = __shfl(base, (int)__builtin_ctzll(bal));
        const uint64_t below = lane ? (bal & ((1ull << lane) - 1)) : 0ull;
        if (in) sh.cand[base + __builtin_popcountll(below)] = x;
      }
    }
    __syncthreads();
    T = radix_kth([&](int i) { return sh.cand[i]; }, [](int) { return true; },
                  nbin, kk, sh);
  } else {
    T = radix_kth(getk, [&](int e) { return bin(getk(e)) == bstar; }, n, kk,
                  sh);
  }
  // take every key above T and the first (by index) keys equal to T: one
  // scan of the packed counts (greater in the low half, equal in the high
  // half). Both totals are below n < 2^15 there, so every partial sum stays
  // below 2^31 and the signed scan cannot overflow. Equal keys are taken in
  // index order, so those taken before thread t number
  // min(equal before t, keq).
  int ngt = 0, neq = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t x = getk(e);
    ngt += x > T;
    neq += x == T;
  }
  int gt_before, eq_before, tot_gt, tot_eq;
  if (n < 32768) {
    const int both = ngt | (neq << 16);
    const int incl = block_incl_scan(both, sh.tmp);
    if (tid == 255) sh.bcast[3] = incl;
    __syncthreads();
    tot_gt = sh.bcast[3] & 0xffff;
    tot_eq = sh.bcast[3] >> 16;
    const int excl = incl - both;
    gt_before = excl & 0xffff;
    eq_before = excl >> 16;
  } else {  // longer rows: one scan per count
    const int gi = block_incl_scan(ngt, sh.tmp);
    const int ei = block_incl_scan(neq, sh.tmp);
    if (tid == 255) {
      sh.bcast[3] = gi;
      sh.bcast[2] = ei;
    }
    __syncthreads();
    tot_gt = sh.bcast[3];
    tot_eq = sh.bcast[2];
    gt_before = gi - ngt;
    eq_before = ei - neq;
  }
  const int keq = k - tot_gt;  // keys equal to T to take
  const int take_eq = max(0, min(keq - eq_before, neq));
  int pos = gt_before + min(eq_before, keq);
  int eq_seen = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t x = getk(e);
    bool t = x > T;
    if (x == T) {
      t = eq_seen < take_eq;
      ++eq_seen;
    }
    if (t) out[pos++] = idx_base + e;
  }
  __syncthreads();
  TopkResult res;
  res.T = T;
  res.count_ge = tot_gt + tot_eq;
  return res;
}

// ------------------------------------------------- wave-synchronous top-k
// For small k: each wave of the block selects in its own range with no block
// barriers (a wave's LDS operations complete in order), then one wave
// selects among the survivors. Used by the decode block choice (k <= 64).

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(v, off);
    if (lane >= off) v += y;
  }
  return v;
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = threadIdx.x & 63;
  return lane ? (~0ull >> (64 - lane)) : 0ull;
}

// The kk-th largest (1 <= kk <= m) of key(i), i < m, found by one wave: a
// 4-pass, 8-bit radix select on a 256-bin histogram of its own.
template <class Key>
__device__ uint32_t wave_kth(Key key, int m, int kk, int* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[lane + 64 * j] = 0;
    __builtin_amdgcn_wave_barrier();
    for (int i = lane; i < m; i += 64) {
      const uint32_t x = key(i);
      if ((x & pmask) == prefix) atomicAdd(&hist[(x >> shift) & 255], 1);
    }
    __builtin_amdgcn_wave_barrier();
    // lane l covers bins 255 - 4l .. 252 - 4l, from the top
    int h[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = hist[255 - 4 * lane - j];
      sum += h[j];
    }
    __builtin_amdgcn_wave_barrier();
    const int incl = wave_incl_scan(sum);
    const int excl = incl - sum;
    const bool mine = excl < kk && kk <= incl;  // exactly one lane
    int bin = 0, above = excl;
    if (mine) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above + h[j] >= kk) {
          bin = 255 - 4 * lane - j;
          break;
        }
        above += h[j];
      }
    }
    const int src = (int)__builtin_ctzll(__ballot(mine));
    bin = __shfl(bin, src);
    above = __shfl(above, src);
    prefix |= (uint32_t)bin << shift;
    pmask |= 0xffu << shift;
    kk -= above;
  }
  return prefix;
}

// Hands the k largest of key(i), i < m (1 <= k <= m; ties: lower i first)
// to emit(p, i, key) with p = 0..k-1 in ascending i, and returns the k-th
// largest key. One wave.
template <class Key, class Emit>
__device__ uint32_t wave_take(Key key, int m, int k, Emit emit, int* hist) {
  const int lane = threadIdx.x & 63;
  const uint32_t T = wave_kth(key, m, k, hist);
  int gt = 0;
  for (int i = lane; i < m; i += 64) gt += key(i) > T;
  gt = __shfl(wave_incl_scan(gt), 63);
  const int take_eq = k - gt;  // keys equal to T to take, lowest i first
  const uint64_t below = lanes_below();
  int pos = 0, eq_seen = 0;
  for (int i0 = 0; i0 < m; i0 += 64) {
    const int i = i0 + lane;
    const uint32_t x = i < m ? key(i) : 0u;
    const bool is_gt = i < m && x > T, is_eq = i < m && x == T;
    const uint64_t beq = __ballot(is_eq);
    const bool t =
        is_gt || (is_eq && eq_seen + __builtin_popcountll(beq & below) < take_eq);
    const uint64_t bt = __ballot(t);
    if (t) emit(pos + __builtin_popcountll(bt & below), i, x);
    pos += __builtin_popcountll(bt);
    eq_seen += __builtin_popcountll(beq);
  }
  return T;
}

// The per-wave selection suits small budgets over a few thousand keys (the
// decode block choice): its first radix pass bins on the top key bits, where
// scores of one row crowd into a few bins, so its LDS atomics serialise as
// rows and budgets grow. Prefill rows use the block-wide select above.
constexpr int kWaveTopkMax = 64;

struct WaveTopkShared {
  int hist[4][256];
  uint32_t ckey[4 * kWaveTopkMax];
  int cidx[4 * kWaveTopkMax];
  uint32_t T;
};

// Requires 1 <= k <= kWaveTopkMax and k < n; 256 threads. Writes out[0..k)
// = idx_base + chosen e, ascending (ties: lower e first), and returns the
// k-th largest key (block-uniform). The four waves take consecutive
// quarters of [0, n); every member of the final top k is in its quarter's
// top k, and the survivors are stored in quarter order, i.e. in ascending
// e, so the last selection keeps the tie order.
template <class GetK>
__device__ uint32_t wave_topk(GetK getk, int n, int k, int32_t* out,
                              int idx_base, WaveTopkShared& sh) {
  const int wave = threadIdx.x >> 6;
  const int C = (n + 3) / 4;
  auto kw_of = [&](int w) {
    return min(k, max(0, min(n, (w + 1) * C) - w * C));
  };
  const int lo = min(wave * C, n), m = min(n, lo + C) - lo;
  int off = 0;
  for (int w = 0; w < wave; ++w) off += kw_of(w);
  const int kw = kw_of(wave);
  if (kw > 0)
    wave_take([&](int i) { return getk(lo + i); }, m, kw,
              [&](int p, int i, uint32_t x) {
                sh.ckey[off + p] = x;
                sh.cidx[off + p] = lo + i;
              },
              sh.hist[wave]);
  __syncthreads();
  if (wave == 0) {
    const int M = kw_of(0) + kw_of(1) + kw_of(2) + kw_of(3);
    const uint32_t T = wave_take(
        [&](int i) { return sh.ckey[i]; }, M, k,
        [&](int p, int i, uint32_t) { out[p] = idx_base + sh.cidx[i]; },
        sh.hist[0]);
    if ((threadIdx.x & 63) == 0) sh.T = T;
  }
  __syncthreads();
  return sh.T;
}

// The same selection with each lane's keys held in registers (NPL per lane
// and wave, so n <= 4 * 64 * NPL): every radix pass and the collection then
// read registers, and only the histogram atomics touch LDS. Same contract
// and result as wave_topk.
template <int NPL>
__device__ uint32_t wave_kth_regs(const uint32_t (&kr)[NPL], int m, int kk,
                                  int* hist) {
  const int lane = threadIdx.x & 63;
  uint32_t prefix = 0, pmask = 0;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
#pragma unroll
    for (int j = 0; j < 4; ++j) hist[lane + 64 * j] = 0;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int i = lane + 64 * j;
      if (i < m && (kr[j] & pmask) == prefix)
        atomicAdd(&hist[(kr[j] >> shift) & 255], 1);
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
    const bool mine = excl < kk && kk <= incl;  // exactly one lane
    int bin = 0, above = excl;
    if (mine) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above + h[j] >= kk) {
          bin = 255 - 4 * lane - j;
          break;
        }
        above += h[j];
      }
    }
    const int src = (int)__builtin_ctzll(__ballot(mine));
    bin = __shfl(bin, src);
    above = __shfl(above, src);
    prefix |= (uint32_t)bin << shift;
    pmask |= 0xffu << shift;
    kk -= above;
  }
  return prefix;
}

// key i = lane + 64 j of the wave's range sits in kr[j] (i < m valid)
template <int NPL, class Emit>
__device__ uint32_t wave_take_regs(const uint32_t (&kr)[NPL], int m, int k,
                                   Emit emit, int* hist) {
  const uint32_t T = wave_kth_regs<NPL>(kr, m, k, hist);
  const int lane = threadIdx.x & 63;
  int gt = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) gt += (lane + 64 * j < m) && kr[j] > T;
  gt = __shfl(wave_incl_scan(gt), 63);
  const int take_eq = k - gt;
  const uint64_t below = lanes_below();
  int pos = 0, eq_seen = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int i = lane + 64 * j;
    const bool valid = i < m;
    const bool is_gt = valid && kr[j] > T, is_eq = valid && kr[j] == T;
    const uint64_t beq = __ballot(is_eq);
    const bool t =
        is_gt || (is_eq && eq_seen + __builtin_popcountll(beq & below) < take_eq);
    const uint64_t bt = __ballot(t);
    if (t) emit(pos + __builtin_popcountll(bt & below), i, kr[j]);
    pos += __builtin_popcountll(bt);
    eq_seen += __builtin_popcountll(beq);
  }
  return T;
}

// wave_topk for n <= 4 * 64 * NPL, with register-held keys
template <int NPL, class GetK>
__device__ uint32_t wave_topk_regs(GetK getk, int n, int k, int32_t* out,
                                   int idx_base, WaveTopkShared& sh) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int C = (n + 3) / 4;
  auto kw_of = [&](int w) {
    return min(k, max(0, min(n, (w + 1) * C) - w * C));
  };
  const int lo = min(wave * C, n), m = min(n, lo + C) - lo;
  int off = 0;
  for (int w = 0; w < wave; ++w) off += kw_of(w);
  const int kw = kw_of(wave);
  if (kw > 0) {
    uint32_t kr[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int i = lane + 64 * j;
      kr[j] = i < m ? getk(lo + i) : 0u;
    }
    wave_take_regs<NPL>(kr, m, kw,
                        [&](int p, int i, uint32_t x) {
                          sh.ckey[off + p] = x;
                          sh.cidx[off + p] = lo + i;
                        },
                        sh.hist[wave]);
  }
  __syncthreads();
  if (wave == 0) {
    constexpr int NS = (4 * kWaveTopkMax + 63) / 64;
    const int M = kw_of(0) + kw_of(1) + kw_of(2) + kw_of(3);
    uint32_t kr[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int i = lane + 64 * j;
      kr[j] = i < M ? sh.ckey[i] : 0u;
    }
    const uint32_t T = wave_take_regs<NS>(
        kr, M, k,
        [&](int p, int i, uint32_t) { out[p] = idx_base + sh.cidx[i]; },
        sh.hist[0]);
    if (lane == 0) sh.T = T;
  }
  __syncthreads();
  return sh.T;
}

}  // namespace rtp
