// Shared device helpers and internal launcher declarations (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace rtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;

constexpr int kD = 128;      // head dim
constexpr int kBlk = 64;     // indexer block = attention key tile
constexpr int kMaxHeads = 128;
// Longest prefill: one KV head's K (S x 256 B) must fit a buffer descriptor.
constexpr int kMaxSeq = (1 << 24) - 64;
// the most 64-token blocks a sequence has; top_k and n_recent are capped by it
constexpr int kMaxBlocks = kMaxSeq / 64;

// MFMA lane layouts on gfx950 (checked on hardware against a CPU matmul):
//  v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8*(l/32)+e] and
//  B[8*(l/32)+e][l%32] (e = 0..7); accumulator element i of lane l is
//  C[8*(i/4) + 4*(l/32) + i%4][l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf2f(u16 b) {
  return __uint_as_float(((uint32_t)b) << 16);
}
__device__ __forceinline__ u16 f2bf(float f) {  // round to nearest even
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(u16, b);
}
__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {  // RNE
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// LDS DMA: lane i's 16 bytes from g land at lds_base + 16 i.
typedef __attribute__((address_space(3))) void* lds_ptr_t;
__device__ __forceinline__ void dma16(const void* g, void* lds_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds_base, 16, 0, 0);
}
// The same LDS DMA through a buffer descriptor (the MUBUF "lds" form):
// 16 bytes per lane from base + voff + soff land at lds_base + 16 i. The FLAT
// form above counts, for the compiler, as possibly touching LDS, and while
// one is in flight every LDS wait it inserts is a full lgkmcnt(0); with the
// buffer form the waits stay exact, so operand reads issued ahead really do
// overlap the MFMAs. A descriptor covers at most 4 GiB (bytes < 2^32).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)bytes, 0x00020000);
}
__device__ __forceinline__ void buf_dma16(__amdgpu_buffer_rsrc_t r,
                                          uint32_t voff, uint32_t soff,
                                          void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base, 16, voff,
                                           soff, 0, 0);
}
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0); }
// s_waitcnt vmcnt(N), other counters at their maximum (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14));  // lgkmcnt(0)
}

// Row of a 32-key sub-tile that MFMA row m reads: swap bits 2 and 3. Then
// accumulator element i of lane l of S^T holds key 16*(i/8) + 8*(l/32) + i%8
// of the sub-tile, i.e. the 8 values a lane feeds to one P.V step are 8
// consecutive keys.
__device__ __forceinline__ int perm_row(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Optional per-kernel timing (off unless rtp_profile(1) was called): HIP
// events recorded on the launch stream right before and after a kernel.
void prof_begin(const char* name, hipStream_t st);
void prof_end(hipStream_t st);

// Fork and join with the device's auxiliary stream: a library-owned stream
// (default priority, created on first use) on which independent work runs
// concurrently with the caller's stream. Constructing an AuxFork records an
// event on `st` that the auxiliary stream waits for, so work put on
// stream() starts after everything enqueued on `st` before; join() makes
// `st` wait for that work. Holds a process-wide lock from construction to
// join() (or destruction), so the events are never shared by two calls.
// If the auxiliary stream cannot be created, stream() is `st` itself.
class AuxFork {
 public:
  explicit AuxFork(hipStream_t st);
  ~AuxFork();
  AuxFork(const AuxFork&) = delete;
  AuxFork& operator=(const AuxFork&) = delete;
  hipStream_t stream() const { return aux_; }
  hipError_t status() const { return err_; }
  hipError_t join();

 private:
  hipStream_t st_, aux_;
  void* slot_ = nullptr;
  hipError_t err_ = hipSuccess;
  bool locked_ = false, joined_ = false;
};

__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline int64_t tri_rows(int64_t n_b) {  // candidates of rows 2..n_b-1
  return n_b >= 3 ? (n_b - 2) * (n_b - 1) / 2 : 0;
}

// ---------------------------------------------------------------- launchers
// All launchers enqueue on `stream` and return the launch status.

struct AttnLaunch {
  const u16* q; const u16* k; const u16* vt; u16* out; float* lse;
  const int32_t* sel; const int32_t* sel_cnt; int sel_stride;
  int S, S_pad, n_b, G, Hkv, window;
  float scale;
  // HOST [Hq] window of each head attended by the window kernel, or NULL
  // (then `window` for every such head)
  const int32_t* head_window = nullptr;
};

hipError_t launch_transpose_v(const u16* v, u16* vt, int Hkv, int S, int S_pad,
                              hipStream_t st);
// is_ret: host [Hq]; nullptr means every head is a window head. parts: 1 =
// window heads only, 2 = retrieval heads only, 3 = both.
constexpr int kAttnWindow = 1, kAttnSparse = 2, kAttnAll = 3;
// The window / dense heads of a launch (attn_window.hip); launch_attention
// calls it for the kAttnWindow part.
hipError_t launch_window_heads(const AttnLaunch& a, const uint8_t* is_ret,
                               hipStream_t st);
hipError_t launch_attention(const AttnLaunch& a, const uint8_t* is_ret,
                            hipStream_t st, int parts = kAttnAll);

// Scratch of the indexer, per call:
//  - projected keys of every retrieval head in the MFMA operand order of
//    the scoring kernel: per (head, key block) 4*r/16 KiB (hi and lo bf16
//    parts of 64 keys x r);
//  - projected query-block means, hi and lo bf16 parts, [n_ret, n_b, r];
//  - up to kStreamMinBlocks key blocks: the score rows (fp32, the lower
//    triangle of each head);
//  - longer sequences: the fused kernel's candidate buffers, one per row of
//    each wave slot, `cap` entries of 8 bytes (order key, block), and a work
//    counter.
constexpr int kScoreMaxWG = 512;  // persistent workgroups (2 per CU)
constexpr int kStreamMinBlocks = 4097;
struct IndexerSizes {
  size_t kop, qpart, scores, buf, counter, total;
  int cap, n_items, n_wg;
  bool fused;
};
__host__ inline IndexerSizes indexer_sizes(int n_ret, int n_b, int r,
                                           int top_k) {
  IndexerSizes z;
  const int need = top_k + 1;  // the top_k + 1 best are kept (for s_{k+1})
  // (4 need entries, hence fewer shrinks, measured no faster at 1M tokens:
  // each shrink then handles more entries)
  const int c = 2 * need > need + 64 ? 2 * need : need + 64;
  z.cap = (c + 63) / 64 * 64;
  // a row has at most n_b - 2 candidates: a buffer with 64 slots more than
  // that is never shrunk (so cap >= need + 64 wherever shrinking happens)
  const int all = (n_b + 63) / 64 * 64 + 64;
  if (z.cap > all) z.cap = all;
  const int tiles = (n_b + 63) / 64;
  z.n_items = 4 * n_ret * ((tiles + 3) / 4);
  int wg = (z.n_items + 3) / 4;
  z.n_wg = wg < 1 ? 1 : (wg > kScoreMaxWG ? kScoreMaxWG : wg);
  z.fused = n_b >= kStreamMinBlocks;
  z.kop = align256((size_t)n_ret * n_b * 256 * r);
  z.qpart = align256((size_t)n_ret * n_b * r * 2);
  z.scores = z.fused ? 0 : align256((size_t)n_ret * tri_rows(n_b) * 4);
  z.buf = z.fused ? align256((size_t)z.n_wg * 4 * 64 * z.cap * 8) : 0;
  z.counter = 256;
  z.total = z.kop + 2 * z.qpart + z.scores + z.buf + z.counter;
  return z;
}

struct IndexerLaunch {
  const u16* q; const u16* k; const float* p_q; const float* p_k;
  int S, n_b, Hq, Hkv, n_ret, r, top_k;
  const uint8_t* ret_heads;  // host: query head of each retrieval index
  char* scratch;             // indexer_sizes(...).total bytes, 256-aligned
  int32_t* sel; int32_t* sel_cnt; float* kth; float* centroids;
  bool keys_only = false;  // only the key projection (and centroids)
};
hipError_t launch_indexer(const IndexerLaunch& a, hipStream_t st);

// Decode K/V cache view. Contiguous (table == nullptr): [B, Hkv, Lmax, d].
// Paged: pages of 64 tokens [n_pages, Hkv, 64, d] and a block table
// [B, max_blocks] whose entry (b, j) is the page holding tokens 64 j ..
// 64 j + 63 of sequence b (Lmax = 64 max_blocks). Page ids outside
// [0, n_pages) are clamped, so a bad table stays inside the pool.
struct KvView {
  const int32_t* table = nullptr;
  int max_blocks = 0, n_pages = 0;
};
// element offset of token j of (sequence b, KV head g)
__device__ __forceinline__ size_t kv_row(const KvView& v, int b, int Hkv,
                                         int g, int Lmax, int j) {
  if (!v.table) return (((size_t)b * Hkv + g) * Lmax + j) * kD;
  int page = v.table[(size_t)b * v.max_blocks + (j >> 6)];
  page = min(max(page, 0), v.n_pages - 1);
  return (((size_t)page * Hkv + g) * 64 + (j & 63)) * kD;
}

struct DecodeLaunch {
  const u16* q; const u16* kc; const u16* vc; const int32_t* cache_len;
  const float* p_q; const float* cent;
  int B, Lmax, Hq, Hkv, n_ret, r, window, top_k, n_recent, n_split;
  float scale;
  const uint8_t* ret_heads;  // host
  const uint8_t* is_ret;     // host [Hq]
  u16* out; float* lse; int32_t* sel; float* cscores; float* part_o;
  float* part_ml;
  // every kernel on `st` (no auxiliary stream, so nothing is created)
  bool one_stream = false;
  // clustered decode (cl_off != nullptr): the cluster tables of
  // launch_cluster, and space for the token lists [B, n_ret, Lmax] and
  // their lengths [B, n_ret]
  const int32_t* cl_m = nullptr; const int32_t* cl_off = nullptr;
  const int32_t* cl_mem = nullptr;
  int32_t* tok = nullptr; int32_t* tok_cnt = nullptr;
  KvView kv;  // paged cache when kv.table is set
};

// K-cache clustering: the clustered tokens of one (sequence, retrieval
// head) are split into at most kClChunks chunks for the stable grouping.
constexpr int kClChunks = 64;
struct ClusterSizes {
  size_t x, assign, hist, total;  // byte offsets in the workspace
};
inline ClusterSizes cluster_sizes(int B, int Lmax, int n_ret, int r) {
  const size_t rows = (size_t)B * n_ret * Lmax, nbmax = (size_t)Lmax / 64;
  ClusterSizes z;
  size_t off = 0;
  z.x = off;      off += align256(rows * r * 4);
  z.assign = off; off += align256(rows * 4);
  z.hist = off;   off += align256((size_t)B * n_ret * kClChunks * nbmax * 4);
  z.total = off;
  return z;
}
struct ClusterLaunch {
  const u16* kc; const int32_t* cache_len; const float* p_k;
  KvView kv;  // paged cache when kv.table is set
  float* cent; int32_t* cl_m; int32_t* cl_off; int32_t* cl_mem;
  int B, Lmax, Hkv, n_ret, r, n_recent, iters, G;
  const uint8_t* ret_heads;  // host
  char* scratch;             // cluster_sizes(...).total bytes, 256-aligned
};
hipError_t launch_cluster(const ClusterLaunch& a, hipStream_t st);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t st);

hipError_t launch_build_centroids(const u16* kc, const int32_t* cache_len,
                                  const float* p_k, float* cent, int B,
                                  int Lmax, int Hkv, int n_ret, int r, int G,
                                  const uint8_t* ret_heads, hipStream_t st,
                                  KvView kv = KvView());

hipError_t launch_decode_append(u16* kc, u16* vc, int32_t* cache_len,
                                const u16* k_new, const u16* v_new,
                                const float* p_k, float* cent, int B,
                                int Lmax, int Hkv, int n_ret, int r, int G,
                                const uint8_t* ret_heads, hipStream_t st,
                                KvView kv = KvView());


}  // namespace rtp
