// Low-rank projection of key rows on the matrix cores (gfx950):
//     x_j = P k_j,  P fp32 [rows, 128], k_j bf16 [128].
//
// P is split into three bf16 parts, P = p1 + p2 + p3 (p2, p3 the bf16
// roundings of what the earlier parts leave, so the split keeps all 24 bits
// of P's significand); a bf16 key times a bf16 part is exact in fp32, so
// the three v_mfma_f32_32x32x16_bf16 products summed in fp32 give the fp32
// projection (only the order of the fp32 additions differs from a plain
// dot product).
//
// The product is C^T = P K^T: 32 rows of P (M) against 32 keys (N), K = 128
// in 8 steps. A workgroup stages one 32-row tile of the three parts in LDS
// (rows padded to 272 bytes, so the 16-byte operand reads of 8 consecutive
// rows hit distinct banks); each wave holds its 64-key block's keys as the
// B operand. After cl_rows_of_lane, lane (g, n) holds, for key 32 mt + n of
// the block, rows 8 g .. 8 g + 7 of the tile in acc[mt][0..7] and rows
// 16 + 8 g .. 16 + 8 g + 7 in acc[mt][8..15]: eight consecutive rows of one
// key per lane, as the indexer's operand layout and the clustering's fp32
// rows both want.
#pragma once

#include "common.h"

namespace rtp {

constexpr int kProjRowB = 272;                 // LDS bytes per P row
constexpr int kProjPartB = 32 * kProjRowB;     // one part of a 32-row tile
constexpr int kProjTileB = 3 * kProjPartB;     // 26112

// Stage rows m0 .. m0 + 31 of P (rows >= n_rows are zero) as three bf16
// parts, by the workgroup's 256 threads (16 values each). The caller
// separates stages with barriers.
__device__ __forceinline__ void proj_stage(const float* P, int m0, int n_rows,
                                           char* lds) {
  const int t = threadIdx.x, row = t >> 3, c0 = 16 * (t & 7);
  const int gr = m0 + row;
  float v[16];
  if (gr < n_rows) {
    const float4* src = reinterpret_cast<const float4*>(P + (size_t)gr * kD + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 f = src[i];
      v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.f;
  }
  uint32_t w[3][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float a = v[2 * e], b = v[2 * e + 1];
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const u16 ha = f2bf(a), hb = f2bf(b);
      w[part][e] = (uint32_t)ha | ((uint32_t)hb << 16);
      a -= bf2f(ha);
      b -= bf2f(hb);
    }
  }
#pragma unroll
  for (int part = 0; part < 3; ++part) {
    char* dst = lds + part * kProjPartB + row * kProjRowB + 2 * c0;
    *reinterpret_cast<uint4*>(dst) = make_uint4(w[part][0], w[part][1], w[part][2], w[part][3]);
    *reinterpret_cast<uint4*>(dst + 16) =
        make_uint4(w[part][4], w[part][5], w[part][6], w[part][7]);
  }
}

// B operands of a 64-key block (first row `krows`, `nvalid` keys present,
// the rest zero): lane (g, n) holds K[32 mt + n][16 ks + 8 g .. + 7].
__device__ __forceinline__ void proj_keys_operands(const u16* krows, int nvalid,
                                                   bf16x8 (&kb)[2][8]) {
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int key = 32 * mt + n;
    const u16* p = krows + (size_t)(key < nvalid ? key : 0) * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8 v = *reinterpret_cast<const bf16x8*>(p + 16 * ks);
      if (key >= nvalid) { bf16x8 z = {}; v = z; }
      kb[mt][ks] = v;
    }
  }
}

// The staged tile times the block's keys (two accumulators per key tile,
// even and odd steps, so four product chains interleave), then the halves
// exchanged so each lane holds eight consecutive rows of its key.
__device__ __forceinline__ void proj_tile(const char* lds,
                                          const bf16x8 (&kb)[2][8],
                                          f32x16 (&acc)[2]) {
  const int lane = threadIdx.x & 63, g = lane >> 5, n = lane & 31;
  f32x16 a[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    a[mt][0] = f32x16{};
    a[mt][1] = f32x16{};
  }
#pragma unroll
  for (int ks = 0; ks < 8; ++ks)
#pragma unroll
    for (int part = 0; part < 3; ++part) {
      const bf16x8 pa = *reinterpret_cast<const bf16x8*>(
          lds + part * kProjPartB + n * kProjRowB + 32 * ks + 16 * g);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        a[mt][ks & 1] = mfma32(pa, kb[mt][ks], a[mt][ks & 1]);
    }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    f32x16 c;
#pragma unroll
    for (int i = 0; i < 16; ++i) c[i] = a[mt][0][i] + a[mt][1][i];
    // rows: lane (g, n) element i holds row 8 (i/4) + 4 g + i%4; swapping
    // the upper half of element i with the lower half of element i + 4
    // (i = 0..3 and 8..11) leaves rows 8 g + e in elements e = 0..7 and
    // rows 16 + 8 g + e in elements 8 + e
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 8 * q + e;
        const auto sw = __builtin_amdgcn_permlane32_swap(
            __float_as_uint(c[i]), __float_as_uint(c[i + 4]), false, false);
        c[i] = __uint_as_float(sw[0]);
        c[i + 4] = __uint_as_float(sw[1]);
      }
    acc[mt] = c;
  }
}

}  // namespace rtp
