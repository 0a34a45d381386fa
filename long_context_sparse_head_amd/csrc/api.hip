// C ABI of the hybrid attention library: argument validation, workspace
// layout and kernel sequencing. Declarations and semantics: include/rtp.h.
#include "common.h"
#include "../../include/rtp.h"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <string>
#include <vector>

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  g_err = std::string(where) + ": " + hipGetErrorString(e);
  return RTP_EHIP;
}

struct HeadInfo {
  int n_ret = 0;
  std::vector<uint8_t> ret_heads;  // query head of each retrieval index
};

HeadInfo scan_mask(const uint8_t* m, int Hq) {
  HeadInfo hi;
  for (int h = 0; h < Hq; ++h)
    if (m[h]) {
      hi.ret_heads.push_back((uint8_t)h);
      ++hi.n_ret;
    }
  return hi;
}

// Shape checks shared by every entry point.
int check_shape(int S, int Hq, int Hkv, int d) {
  if (S < 0 || Hq <= 0 || Hkv <= 0)
    return fail(RTP_EINVAL, "sizes must satisfy S >= 0, Hq > 0, Hkv > 0");
  if (Hq % Hkv)
    return fail(RTP_EINVAL, "Hq must be a multiple of Hkv");
  if (d != rtp::kD) return fail(RTP_EUNSUPPORTED, "only d = 128 is supported");
  if (Hq > rtp::kMaxHeads)
    return fail(RTP_EUNSUPPORTED, "at most 128 query heads are supported");
  if (S > rtp::kMaxSeq)
    return fail(RTP_EUNSUPPORTED, "S must be at most 16777152 tokens");
  return RTP_OK;
}

int check_indexer(int n_ret, int r, int block, int top_k) {
  if (block != rtp::kBlk) return fail(RTP_EUNSUPPORTED, "only block = 64 is supported");
  if (top_k < 0 || top_k > rtp::kMaxBlocks)
    return fail(RTP_EINVAL, "top_k must be in [0, 262143] (the most blocks a sequence has)");
  if (n_ret > 0 && (r < 16 || r > 128 || r % 16))
    return fail(RTP_EUNSUPPORTED, "r must be a multiple of 16 in [16, 128]");
  return RTP_OK;
}

// Prefill workspace. The indexer's scratch and V^T share the first region:
// the indexer runs first, and V^T (needed only by the attention kernels) is
// written after it has finished, on the same stream.
struct PrefillLayout {
  size_t vt, idx, sel, cnt, total;
};

// n_sel: retrieval heads that select (0 when none runs the indexer)
PrefillLayout prefill_layout(int S, int Hkv, int n_ret, int r, int top_k,
                             int n_sel) {
  using rtp::align256;
  const size_t n_b = (size_t)(S + 63) / 64, S_pad = n_b * 64;
  PrefillLayout L;
  const size_t vt_bytes = align256((size_t)Hkv * rtp::kD * S_pad * 2);
  const size_t idx_bytes =
      n_sel ? rtp::indexer_sizes(n_sel, (int)n_b, r, top_k).total : 0;
  size_t off = 0;
  L.vt = 0;
  L.idx = 0;
  off = std::max(vt_bytes, idx_bytes);
  L.sel = off; off += align256((size_t)n_sel * n_b * (top_k + 2) * 4);
  L.cnt = off; off += align256((size_t)n_sel * n_b * 4);
  L.total = off;
  (void)n_ret;
  return L;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return RTP_OK;
  if (!ws || ws_bytes < need)
    return fail(RTP_EWORKSPACE, "workspace too small: need " + std::to_string(need) +
                                    " bytes, got " + std::to_string(ws_bytes));
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(RTP_EWORKSPACE, "workspace must be 256-byte aligned");
  return RTP_OK;
}

float resolve_scale(float scale, int d) {
  return scale > 0.f ? scale : 1.0f / std::sqrt((float)d);
}

// ------------------------------------------------------- kernel timing
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_prof_pool;
std::vector<ProfRec> g_prof_recs;
constexpr size_t kProfMax = 1 << 14;

}  // namespace

namespace {
struct AuxSlot {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;
};
constexpr int kMaxDevices = 64;
std::mutex g_aux_mu;
AuxSlot g_aux[kMaxDevices];
}  // namespace

namespace rtp {
AuxFork::AuxFork(hipStream_t st) : st_(st), aux_(st) {
  g_aux_mu.lock();
  locked_ = true;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return;
  }
  AuxSlot& x = g_aux[dev];
  if (x.failed) return;
  if (!x.s) {
    if (hipStreamCreateWithFlags(&x.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&x.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&x.join, hipEventDisableTiming) != hipSuccess) {
      x.failed = true;
      (void)hipGetLastError();
      return;
    }
  }
  err_ = hipEventRecord(x.fork, st);
  if (err_ == hipSuccess) err_ = hipStreamWaitEvent(x.s, x.fork, 0);
  if (err_ == hipSuccess) {
    aux_ = x.s;
    slot_ = &x;
  }
}

hipError_t AuxFork::join() {
  hipError_t e = hipSuccess;
  if (!joined_ && slot_) {
    AuxSlot& x = *static_cast<AuxSlot*>(slot_);
    e = hipEventRecord(x.join, aux_);
    if (e == hipSuccess) e = hipStreamWaitEvent(st_, x.join, 0);
  }
  joined_ = true;
  if (locked_) {
    locked_ = false;
    g_aux_mu.unlock();
  }
  return e;
}

AuxFork::~AuxFork() { (void)join(); }

void prof_begin(const char* name, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || g_prof_recs.size() >= kProfMax) return;
  if (g_prof_recs.size() == g_prof_pool.size()) {
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess) return;
    if (hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      return;
    }
    g_prof_pool.push_back({a, b});
  }
  const auto& ev = g_prof_pool[g_prof_recs.size()];
  if (hipEventRecord(ev.first, st) != hipSuccess) return;
  g_prof_recs.push_back({name, ev.first, ev.second});
}
void prof_end(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || g_prof_recs.empty()) return;
  (void)hipEventRecord(g_prof_recs.back().b, st);
}
}  // namespace rtp

extern "C" {

int rtp_profile(int enable) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_on = enable != 0;
  g_prof_recs.clear();
  return RTP_OK;
}

int rtp_profile_read(const char** names, float* ms, int max) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int n = 0;
  for (const auto& r : g_prof_recs) {
    if (n >= max) break;
    hipError_t e = hipEventSynchronize(r.b);
    float t = -1.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess) return hip_fail(e, "rtp_profile_read");
    if (names) names[n] = r.name;
    if (ms) ms[n] = t;
    ++n;
  }
  g_prof_recs.clear();
  return n;
}


const char* rtp_status_string(int s) {
  switch (s) {
    case RTP_OK: return "ok";
    case RTP_EINVAL: return "invalid argument";
    case RTP_EUNSUPPORTED: return "unsupported configuration";
    case RTP_EWORKSPACE: return "workspace too small or misaligned";
    case RTP_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* rtp_last_error(void) { return g_err.c_str(); }

const char* rtp_version(void) { return "rtp-hybrid-attn 0.1 (gfx950)"; }

size_t rtp_prefill_workspace_bytes(int S, int Hq, int Hkv, int d,
                                   const uint8_t* is_retrieval, int r,
                                   int block, int top_k) {
  if (check_shape(S, Hq, Hkv, d) || !is_retrieval) return 0;
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (check_indexer(hi.n_ret, r, block, top_k)) return 0;
  return prefill_layout(S, Hkv, hi.n_ret, r, top_k, hi.n_ret).total;
}

size_t rtp_dense_workspace_bytes(int S, int Hq, int Hkv, int d) {
  if (check_shape(S, Hq, Hkv, d)) return 0;
  return prefill_layout(S, Hkv, 0, 16, 0, 0).total;
}

static int run_indexer(const void* q, const void* k, int S, int Hq, int Hkv,
                       const HeadInfo& hi, const float* p_q, const float* p_k,
                       int r, int top_k, int32_t* sel, int32_t* sel_count,
                       float* kth, float* cent, char* scratch, hipStream_t st,
                       bool keys_only) {
  rtp::IndexerLaunch a;
  a.q = static_cast<const rtp::u16*>(q);
  a.k = static_cast<const rtp::u16*>(k);
  a.p_q = p_q;
  a.p_k = p_k;
  a.S = S;
  a.n_b = (S + 63) / 64;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_ret = hi.n_ret;
  a.r = r;
  a.top_k = top_k;
  a.ret_heads = hi.ret_heads.data();
  a.scratch = scratch;
  a.sel = sel;
  a.sel_cnt = sel_count;
  a.kth = kth;
  a.centroids = cent;
  a.keys_only = keys_only;
  hipError_t e = rtp::launch_indexer(a, st);
  if (e != hipSuccess) return hip_fail(e, "indexer launch");
  return RTP_OK;
}

int rtp_indexer_select(const void* q, const void* k, int S, int Hq, int Hkv,
                       int d, const uint8_t* is_retrieval, const float* p_q,
                       const float* p_k, int r, int block, int top_k,
                       int32_t* sel, int32_t* sel_count, float* kth_scores,
                       float* centroids, void* ws, size_t ws_bytes,
                       rtp_stream_t stream) {
  g_err.clear();
  if (int e = check_shape(S, Hq, Hkv, d)) return e;
  if (!is_retrieval) return fail(RTP_EINVAL, "is_retrieval is NULL");
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (int e = check_indexer(hi.n_ret, r, block, top_k)) return e;
  if (S == 0 || hi.n_ret == 0) return RTP_OK;
  if (!q || !k || !p_q || !p_k || !sel || !sel_count)
    return fail(RTP_EINVAL, "q, k, p_q, p_k, sel and sel_count must be non-NULL");
  const PrefillLayout L = prefill_layout(S, Hkv, hi.n_ret, r, top_k, hi.n_ret);
  if (int e = check_ws(ws, ws_bytes, L.total)) return e;
  return run_indexer(q, k, S, Hq, Hkv, hi, p_q, p_k, r, top_k, sel, sel_count,
                     kth_scores, centroids, static_cast<char*>(ws) + L.idx,
                     reinterpret_cast<hipStream_t>(stream), false);
}

}  // extern "C"

namespace {
// Shared body of rtp_hybrid_attn_prefill (one window, sparse retrieval
// heads) and rtp_headwise_prefill (a window per head, retrieval heads
// sparse or full, optional centroids).
int prefill_impl(const void* q, const void* k, const void* v, int S, int Hq,
                 int Hkv, int d, const uint8_t* is_retrieval, int window,
                 const int32_t* windows, int mode, const float* p_q,
                 const float* p_k, int r, int block, int top_k, float scale,
                 const int32_t* sel_in, const int32_t* sel_count_in,
                 void* out, float* lse, int32_t* sel_out,
                 int32_t* sel_count_out, float* centroids, void* ws,
                 size_t ws_bytes, rtp_stream_t stream) {
  if (int e = check_shape(S, Hq, Hkv, d)) return e;
  if (!is_retrieval) return fail(RTP_EINVAL, "is_retrieval is NULL");
  if (mode != RTP_RETRIEVAL_SPARSE && mode != RTP_RETRIEVAL_FULL)
    return fail(RTP_EINVAL, "retrieval must be RTP_RETRIEVAL_SPARSE or RTP_RETRIEVAL_FULL");
  const bool full = mode == RTP_RETRIEVAL_FULL;
  if (windows) {
    for (int h = 0; h < Hq; ++h)
      if (!is_retrieval[h] && windows[h] < 1)
        return fail(RTP_EINVAL, "every streaming head's window must be >= 1");
  } else if (window < 1) {
    return fail(RTP_EINVAL, "window must be >= 1");
  }
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (int e = check_indexer(hi.n_ret, r, block, full ? 0 : top_k)) return e;
  if ((sel_in == nullptr) != (sel_count_in == nullptr))
    return fail(RTP_EINVAL, "sel_in and sel_count_in must both be given or both NULL");
  if ((sel_out == nullptr) != (sel_count_out == nullptr))
    return fail(RTP_EINVAL, "sel_out and sel_count_out must both be given or both NULL");
  if (full && (sel_in || sel_out))
    return fail(RTP_EINVAL, "full retrieval heads take and give no selection");
  if (S == 0) return RTP_OK;
  if (!q || !k || !v || !out) return fail(RTP_EINVAL, "q, k, v and out must be non-NULL");
  const bool select = !full && hi.n_ret > 0 && !sel_in;
  if (select && (!p_q || !p_k))
    return fail(RTP_EINVAL, "p_q and p_k must be non-NULL when retrieval heads select");
  if (centroids && hi.n_ret > 0 && !p_k)
    return fail(RTP_EINVAL, "p_k must be non-NULL when centroids are requested");
  const PrefillLayout L = prefill_layout(S, Hkv, hi.n_ret, r, full ? 0 : top_k,
                                         full ? 0 : hi.n_ret);
  if (int e = check_ws(ws, ws_bytes, L.total)) return e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const int n_b = (S + 63) / 64, S_pad = n_b * 64;

  // The indexer (or the key projection alone, for the centroids) runs
  // first: its scratch is the region V^T takes afterwards.
  const int32_t* sel_use = sel_in;
  const int32_t* cnt_use = sel_count_in;
  hipError_t e = hipSuccess;
  if (select) {
    int32_t* s = sel_out ? sel_out : reinterpret_cast<int32_t*>(w + L.sel);
    int32_t* c = sel_count_out ? sel_count_out : reinterpret_cast<int32_t*>(w + L.cnt);
    if (int err = run_indexer(q, k, S, Hq, Hkv, hi, p_q, p_k, r, top_k, s, c,
                              nullptr, centroids, w + L.idx, st, false))
      return err;
    sel_use = s;
    cnt_use = c;
  } else {
    if (!full && hi.n_ret > 0 && sel_out) {
      const size_t n = (size_t)hi.n_ret * n_b;
      e = hipMemcpyAsync(sel_out, sel_in, n * (top_k + 2) * 4,
                         hipMemcpyDeviceToDevice, st);
      if (e == hipSuccess)
        e = hipMemcpyAsync(sel_count_out, sel_count_in, n * 4,
                           hipMemcpyDeviceToDevice, st);
      if (e != hipSuccess) return hip_fail(e, "selection copy");
    }
    if (centroids && hi.n_ret > 0) {  // the key projection alone
      if (int err = run_indexer(q, k, S, Hq, Hkv, hi, p_q, p_k, r, 0, nullptr,
                                nullptr, nullptr, centroids, nullptr, st, true))
        return err;
    }
  }
  // V^T: both attention kernels read it
  rtp::u16* vt = reinterpret_cast<rtp::u16*>(w + L.vt);
  e = rtp::launch_transpose_v(static_cast<const rtp::u16*>(v), vt, Hkv, S,
                              S_pad, st);
  if (e != hipSuccess) return hip_fail(e, "transpose launch");
  // Full retrieval heads join the window kernel with a window of S.
  std::vector<int32_t> head_window;
  if (windows || full) {
    head_window.resize(Hq);
    for (int h = 0; h < Hq; ++h)
      head_window[h] = full && is_retrieval[h] ? std::max(S, 1)
                                               : (windows ? windows[h] : window);
  }
  rtp::AttnLaunch a;
  a.q = static_cast<const rtp::u16*>(q);
  a.k = static_cast<const rtp::u16*>(k);
  a.vt = vt;
  a.out = static_cast<rtp::u16*>(out);
  a.lse = lse;
  a.sel = sel_use;
  a.sel_cnt = cnt_use;
  a.sel_stride = top_k + 2;
  a.S = S;
  a.S_pad = S_pad;
  a.n_b = n_b;
  a.G = Hq / Hkv;
  a.Hkv = Hkv;
  a.window = windows ? 1 : window;
  a.scale = resolve_scale(scale, d);
  a.head_window = head_window.empty() ? nullptr : head_window.data();
  const uint8_t* sparse_heads = full ? nullptr : is_retrieval;

  // On long sequences the window heads attend on the device's auxiliary
  // stream while the block-sparse heads run on the caller's stream: the
  // window kernel is bound by the matrix cores, the block-sparse kernel at
  // 1M tokens by its K/V gathers, so the two share the GPU well. Up to 4096
  // blocks every kernel fills the GPU alone; there they run one after the
  // other (which also keeps each kernel's time measurable on its own).
  constexpr int kForkMinBlocks = 4096;
  const bool sparse_part = !full && hi.n_ret > 0;
  const bool fork = sparse_part && hi.n_ret < Hq && n_b > kForkMinBlocks;
  if (fork) {
    rtp::AuxFork aux(st);
    if ((e = aux.status()) != hipSuccess) return hip_fail(e, "stream fork");
    e = rtp::launch_attention(a, sparse_heads, aux.stream(), rtp::kAttnWindow);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    e = rtp::launch_attention(a, sparse_heads, st, rtp::kAttnSparse);
    if (e != hipSuccess) return hip_fail(e, "attention launch");
    if ((e = aux.join()) != hipSuccess) return hip_fail(e, "stream join");
    return RTP_OK;
  }
  e = rtp::launch_attention(a, sparse_heads, st, rtp::kAttnAll);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return RTP_OK;
}
}  // namespace

extern "C" {

int rtp_hybrid_attn_prefill(const void* q, const void* k, const void* v,
                            int S, int Hq, int Hkv, int d,
                            const uint8_t* is_retrieval, int window,
                            const float* p_q, const float* p_k, int r,
                            int block, int top_k, float scale,
                            const int32_t* sel_in,
                            const int32_t* sel_count_in, void* out,
                            float* lse, int32_t* sel_out,
                            int32_t* sel_count_out, void* ws, size_t ws_bytes,
                            rtp_stream_t stream) {
  g_err.clear();
  return prefill_impl(q, k, v, S, Hq, Hkv, d, is_retrieval, window, nullptr,
                      RTP_RETRIEVAL_SPARSE, p_q, p_k, r, block, top_k, scale,
                      sel_in, sel_count_in, out, lse, sel_out, sel_count_out,
                      nullptr, ws, ws_bytes, stream);
}

size_t rtp_headwise_prefill_workspace_bytes(int S, int Hq, int Hkv, int d,
                                            const uint8_t* is_retrieval,
                                            int retrieval, int r, int block,
                                            int top_k) {
  if (check_shape(S, Hq, Hkv, d) || !is_retrieval) return 0;
  if (retrieval != RTP_RETRIEVAL_SPARSE && retrieval != RTP_RETRIEVAL_FULL) return 0;
  const bool full = retrieval == RTP_RETRIEVAL_FULL;
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (check_indexer(hi.n_ret, r, block, full ? 0 : top_k)) return 0;
  return prefill_layout(S, Hkv, hi.n_ret, r, full ? 0 : top_k,
                        full ? 0 : hi.n_ret).total;
}

int rtp_headwise_prefill(const void* q, const void* k, const void* v, int S,
                         int Hq, int Hkv, int d, const uint8_t* is_retrieval,
                         const int32_t* windows, int retrieval,
                         const float* p_q, const float* p_k, int r, int block,
                         int top_k, float scale, const int32_t* sel_in,
                         const int32_t* sel_count_in, void* out, float* lse,
                         int32_t* sel_out, int32_t* sel_count_out,
                         float* centroids, void* ws, size_t ws_bytes,
                         rtp_stream_t stream) {
  g_err.clear();
  if (!windows) return fail(RTP_EINVAL, "windows is NULL");
  return prefill_impl(q, k, v, S, Hq, Hkv, d, is_retrieval, 1, windows,
                      retrieval, p_q, p_k, r, block, top_k, scale, sel_in,
                      sel_count_in, out, lse, sel_out, sel_count_out,
                      centroids, ws, ws_bytes, stream);
}

int rtp_dense_attn_prefill(const void* q, const void* k, const void* v,
                           int S, int Hq, int Hkv, int d, float scale,
                           void* out, float* lse, void* ws, size_t ws_bytes,
                           rtp_stream_t stream) {
  g_err.clear();
  if (int e = check_shape(S, Hq, Hkv, d)) return e;
  if (S == 0) return RTP_OK;
  if (!q || !k || !v || !out) return fail(RTP_EINVAL, "q, k, v and out must be non-NULL");
  const PrefillLayout L = prefill_layout(S, Hkv, 0, 16, 0, 0);
  if (int e = check_ws(ws, ws_bytes, L.total)) return e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const int n_b = (S + 63) / 64, S_pad = n_b * 64;
  rtp::u16* vt = reinterpret_cast<rtp::u16*>(w + L.vt);
  hipError_t e = rtp::launch_transpose_v(static_cast<const rtp::u16*>(v), vt,
                                         Hkv, S, S_pad, st);
  if (e != hipSuccess) return hip_fail(e, "transpose launch");
  rtp::AttnLaunch a;
  a.q = static_cast<const rtp::u16*>(q);
  a.k = static_cast<const rtp::u16*>(k);
  a.vt = vt;
  a.out = static_cast<rtp::u16*>(out);
  a.lse = lse;
  a.sel = nullptr;
  a.sel_cnt = nullptr;
  a.sel_stride = 0;
  a.S = S;
  a.S_pad = S_pad;
  a.n_b = n_b;
  a.G = Hq / Hkv;
  a.Hkv = Hkv;
  a.window = S;  // window >= S: full causal attention
  a.scale = resolve_scale(scale, d);
  e = rtp::launch_attention(a, nullptr, st);
  if (e != hipSuccess) return hip_fail(e, "attention launch");
  return RTP_OK;
}

}  // extern "C"

namespace {
// Paged-cache arguments: a block table [B, max_blocks] of page ids into a
// pool of n_pages pages (64 tokens of every KV head each).
int check_pages(const int32_t* table, int max_blocks, int n_pages) {
  if (!table) return fail(RTP_EINVAL, "block_table is NULL");
  if (max_blocks < 1 || n_pages < 1)
    return fail(RTP_EINVAL, "max_blocks and n_pages must be >= 1");
  if ((int64_t)max_blocks * 64 > INT32_MAX)
    return fail(RTP_EUNSUPPORTED, "max_blocks * 64 must fit an int");
  return RTP_OK;
}

int build_centroids_impl(const void* k_cache, const int32_t* cache_len, int B,
                         int Lmax, int Hq, int Hkv, int d,
                         const uint8_t* is_retrieval, const float* p_k, int r,
                         int block, float* centroids, rtp_stream_t stream,
                         rtp::KvView kv) {
  if (int e = check_shape(0, Hq, Hkv, d)) return e;
  if (B < 0 || Lmax < 0) return fail(RTP_EINVAL, "B and Lmax must be >= 0");
  if (!is_retrieval) return fail(RTP_EINVAL, "is_retrieval is NULL");
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (int e = check_indexer(hi.n_ret, r, block, 0)) return e;
  if (B == 0 || hi.n_ret == 0 || Lmax < 64) return RTP_OK;
  if (!k_cache || !cache_len || !p_k || !centroids)
    return fail(RTP_EINVAL, "k_cache, cache_len, p_k and centroids must be non-NULL");
  hipError_t e = rtp::launch_build_centroids(
      static_cast<const rtp::u16*>(k_cache), cache_len, p_k, centroids, B, Lmax,
      Hkv, hi.n_ret, r, Hq / Hkv, hi.ret_heads.data(),
      reinterpret_cast<hipStream_t>(stream), kv);
  if (e != hipSuccess) return hip_fail(e, "centroid launch");
  return RTP_OK;
}

int decode_append_impl(void* k_cache, void* v_cache, int32_t* cache_len,
                       const void* k_new, const void* v_new, int B, int Lmax,
                       int Hq, int Hkv, int d, const uint8_t* is_retrieval,
                       const float* p_k, int r, int block, float* centroids,
                       rtp_stream_t stream, rtp::KvView kv) {
  if (int e = check_shape(0, Hq, Hkv, d)) return e;
  if (B < 0 || Lmax < 0) return fail(RTP_EINVAL, "B and Lmax must be >= 0");
  if (!is_retrieval) return fail(RTP_EINVAL, "is_retrieval is NULL");
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (int e = check_indexer(hi.n_ret, r, block, 0)) return e;
  if (B == 0) return RTP_OK;
  if (!k_cache || !v_cache || !cache_len || !k_new || !v_new)
    return fail(RTP_EINVAL, "cache, cache_len and new-token pointers must be non-NULL");
  if (hi.n_ret > 0 && (!p_k || !centroids))
    return fail(RTP_EINVAL, "p_k and centroids must be non-NULL with retrieval heads");
  hipError_t e = rtp::launch_decode_append(
      static_cast<rtp::u16*>(k_cache), static_cast<rtp::u16*>(v_cache),
      cache_len, static_cast<const rtp::u16*>(k_new),
      static_cast<const rtp::u16*>(v_new), p_k, centroids, B, Lmax, Hkv,
      hi.n_ret, r, Hq / Hkv, hi.ret_heads.data(),
      reinterpret_cast<hipStream_t>(stream), kv);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return RTP_OK;
}
}  // namespace

extern "C" {

int rtp_build_centroids(const void* k_cache, const int32_t* cache_len, int B,
                        int Lmax, int Hq, int Hkv, int d,
                        const uint8_t* is_retrieval, const float* p_k, int r,
                        int block, float* centroids, rtp_stream_t stream) {
  g_err.clear();
  return build_centroids_impl(k_cache, cache_len, B, Lmax, Hq, Hkv, d,
                              is_retrieval, p_k, r, block, centroids, stream,
                              rtp::KvView());
}

int rtp_build_centroids_paged(const void* k_pages, const int32_t* block_table,
                              int max_blocks, int n_pages,
                              const int32_t* cache_len, int B, int Hq, int Hkv,
                              int d, const uint8_t* is_retrieval,
                              const float* p_k, int r, int block,
                              float* centroids, rtp_stream_t stream) {
  g_err.clear();
  if (B > 0)
    if (int e = check_pages(block_table, max_blocks, n_pages)) return e;
  rtp::KvView kv;
  kv.table = block_table;
  kv.max_blocks = max_blocks;
  kv.n_pages = n_pages;
  return build_centroids_impl(k_pages, cache_len, B, 64 * max_blocks, Hq, Hkv,
                              d, is_retrieval, p_k, r, block, centroids,
                              stream, kv);
}

int rtp_decode_append(void* k_cache, void* v_cache, int32_t* cache_len,
                      const void* k_new, const void* v_new, int B, int Lmax,
                      int Hq, int Hkv, int d, const uint8_t* is_retrieval,
                      const float* p_k, int r, int block, float* centroids,
                      rtp_stream_t stream) {
  g_err.clear();
  return decode_append_impl(k_cache, v_cache, cache_len, k_new, v_new, B, Lmax,
                            Hq, Hkv, d, is_retrieval, p_k, r, block, centroids,
                            stream, rtp::KvView());
}

int rtp_decode_append_paged(void* k_pages, void* v_pages,
                            const int32_t* block_table, int max_blocks,
                            int n_pages, int32_t* cache_len, const void* k_new,
                            const void* v_new, int B, int Hq, int Hkv, int d,
                            const uint8_t* is_retrieval, const float* p_k,
                            int r, int block, float* centroids,
                            rtp_stream_t stream) {
  g_err.clear();
  if (B > 0)
    if (int e = check_pages(block_table, max_blocks, n_pages)) return e;
  rtp::KvView kv;
  kv.table = block_table;
  kv.max_blocks = max_blocks;
  kv.n_pages = n_pages;
  return decode_append_impl(k_pages, v_pages, cache_len, k_new, v_new, B,
                            64 * max_blocks, Hq, Hkv, d, is_retrieval, p_k, r,
                            block, centroids, stream, kv);
}

static const int kDecSplit = 8;

struct DecodeLayout {
  size_t cs, sel, po, pml, tok, tcnt, total;
};

// clustered: room for the token lists of the clustered decode
static DecodeLayout decode_layout(int B, int Lmax, int Hq, int n_ret, int top_k,
                                  int n_recent, bool clustered = false) {
  using rtp::align256;
  const size_t nbmax = (size_t)Lmax / 64, width = (size_t)top_k + 1 + n_recent;
  DecodeLayout L;
  size_t off = 0;
  L.cs = off;  off += align256((size_t)B * n_ret * nbmax * 4);
  L.sel = off; off += align256((size_t)B * n_ret * (width + 1) * 4);
  L.po = off;  off += align256((size_t)B * Hq * kDecSplit * rtp::kD * 4);
  L.pml = off; off += align256((size_t)B * Hq * kDecSplit * 2 * 4);
  L.tok = L.tcnt = off;
  if (clustered) {
    L.tok = off;  off += align256((size_t)B * n_ret * Lmax * 4);
    L.tcnt = off; off += align256((size_t)B * n_ret * 4);
  }
  L.total = off;
  return L;
}

size_t rtp_decode_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int d,
                                  const uint8_t* is_retrieval, int r,
                                  int block, int top_k, int n_recent) {
  if (check_shape(0, Hq, Hkv, d) || !is_retrieval || B < 0 || Lmax < 0 ||
      n_recent < 1 || n_recent > rtp::kMaxBlocks)
    return 0;
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (check_indexer(hi.n_ret, r, block, top_k)) return 0;
  return decode_layout(B, Lmax, Hq, hi.n_ret, top_k, n_recent).total;
}

size_t rtp_decode_clustered_workspace_bytes(int B, int Lmax, int Hq, int Hkv,
                                            int d, const uint8_t* is_retrieval,
                                            int r, int block, int top_k,
                                            int n_recent) {
  if (check_shape(0, Hq, Hkv, d) || !is_retrieval || B < 0 || Lmax < 0 ||
      n_recent < 1 || n_recent > rtp::kMaxBlocks)
    return 0;
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (check_indexer(hi.n_ret, r, block, top_k)) return 0;
  return decode_layout(B, Lmax, Hq, hi.n_ret, top_k, n_recent, true).total;
}

size_t rtp_cluster_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int d,
                                   const uint8_t* is_retrieval, int r,
                                   int block) {
  if (check_shape(0, Hq, Hkv, d) || !is_retrieval || B < 0 || Lmax < 0)
    return 0;
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (check_indexer(hi.n_ret, r, block, 0) || r > 64) return 0;
  return rtp::cluster_sizes(B, Lmax, hi.n_ret, r).total;
}

}  // extern "C"

namespace {
int cluster_keys_impl(const void* k_cache, const int32_t* cache_len, int B,
                      int Lmax, int Hq, int Hkv, int d,
                      const uint8_t* is_retrieval, const float* p_k, int r,
                      int block, int n_recent, int iters, float* centroids,
                      int32_t* cl_m, int32_t* cl_off, int32_t* cl_members,
                      void* ws, size_t ws_bytes, rtp_stream_t stream,
                      rtp::KvView kv) {
  if (int e = check_shape(0, Hq, Hkv, d)) return e;
  if (B < 0 || Lmax < 0) return fail(RTP_EINVAL, "B and Lmax must be >= 0");
  if (!is_retrieval) return fail(RTP_EINVAL, "is_retrieval is NULL");
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (int e = check_indexer(hi.n_ret, r, block, 0)) return e;
  if (hi.n_ret > 0 && r > 64)
    return fail(RTP_EUNSUPPORTED, "clustering supports r in {16, 32, 48, 64}");
  if (n_recent < 1 || n_recent > rtp::kMaxBlocks)
    return fail(RTP_EINVAL, "n_recent must be in [1, 262143]");
  if (iters < 0 || iters > 1000) return fail(RTP_EINVAL, "iters must be in [0, 1000]");
  if (B == 0 || hi.n_ret == 0 || Lmax < 64) return RTP_OK;
  if (!k_cache || !cache_len || !p_k || !centroids || !cl_m || !cl_off ||
      !cl_members)
    return fail(RTP_EINVAL, "k_cache, cache_len, p_k, centroids and the cluster tables must be non-NULL");
  const rtp::ClusterSizes z = rtp::cluster_sizes(B, Lmax, hi.n_ret, r);
  if (iters > 0)
    if (int e = check_ws(ws, ws_bytes, z.total)) return e;
  rtp::ClusterLaunch a;
  a.kc = static_cast<const rtp::u16*>(k_cache);
  a.kv = kv;
  a.cache_len = cache_len;
  a.p_k = p_k;
  a.cent = centroids;
  a.cl_m = cl_m;
  a.cl_off = cl_off;
  a.cl_mem = cl_members;
  a.B = B;
  a.Lmax = Lmax;
  a.Hkv = Hkv;
  a.n_ret = hi.n_ret;
  a.r = r;
  a.n_recent = n_recent;
  a.iters = iters;
  a.G = Hq / Hkv;
  a.ret_heads = hi.ret_heads.data();
  a.scratch = static_cast<char*>(ws);
  hipError_t e = rtp::launch_cluster(a, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cluster launch");
  return RTP_OK;
}
}  // namespace

extern "C" {

int rtp_cluster_keys(const void* k_cache, const int32_t* cache_len, int B,
                     int Lmax, int Hq, int Hkv, int d,
                     const uint8_t* is_retrieval, const float* p_k, int r,
                     int block, int n_recent, int iters, float* centroids,
                     int32_t* cl_m, int32_t* cl_off, int32_t* cl_members,
                     void* ws, size_t ws_bytes, rtp_stream_t stream) {
  g_err.clear();
  return cluster_keys_impl(k_cache, cache_len, B, Lmax, Hq, Hkv, d,
                           is_retrieval, p_k, r, block, n_recent, iters,
                           centroids, cl_m, cl_off, cl_members, ws, ws_bytes,
                           stream, rtp::KvView());
}

int rtp_cluster_keys_paged(const void* k_pages, const int32_t* block_table,
                           int max_blocks, int n_pages,
                           const int32_t* cache_len, int B, int Hq, int Hkv,
                           int d, const uint8_t* is_retrieval,
                           const float* p_k, int r, int block, int n_recent,
                           int iters, float* centroids, int32_t* cl_m,
                           int32_t* cl_off, int32_t* cl_members, void* ws,
                           size_t ws_bytes, rtp_stream_t stream) {
  g_err.clear();
  if (B > 0)
    if (int e = check_pages(block_table, max_blocks, n_pages)) return e;
  rtp::KvView kv;
  kv.table = block_table;
  kv.max_blocks = max_blocks;
  kv.n_pages = n_pages;
  return cluster_keys_impl(k_pages, cache_len, B, 64 * max_blocks, Hq, Hkv, d,
                           is_retrieval, p_k, r, block, n_recent, iters,
                           centroids, cl_m, cl_off, cl_members, ws, ws_bytes,
                           stream, kv);
}

}  // extern "C"

namespace {
// Shared body of rtp_hybrid_attn_decode (caller's workspace) and
// rtp_hybrid_attn_decode_noalloc (the library's static scratch). `need`
// receives the scratch bytes the call uses (0 when nothing is launched);
// with ws == nullptr the call stops after validation and sizing.
int decode_impl(const void* q, const void* k_cache, const void* v_cache,
                const int32_t* cache_len, int B, int Lmax, int Hq, int Hkv,
                int d, const uint8_t* is_retrieval, int window,
                const float* p_q, const float* centroids, int r, int block,
                int top_k, int n_recent, float scale, void* out, float* lse,
                int32_t* sel_out, void* ws, size_t ws_bytes, bool one_stream,
                size_t* need, rtp_stream_t stream,
                const int32_t* cl_m = nullptr, const int32_t* cl_off = nullptr,
                const int32_t* cl_mem = nullptr, bool clustered = false,
                rtp::KvView kv = rtp::KvView()) {
  *need = 0;
  if (int e = check_shape(0, Hq, Hkv, d)) return e;
  if (B < 0 || Lmax < 1) return fail(RTP_EINVAL, "B must be >= 0 and Lmax >= 1");
  if (!is_retrieval) return fail(RTP_EINVAL, "is_retrieval is NULL");
  if (window < 1) return fail(RTP_EINVAL, "window must be >= 1");
  if (n_recent < 1 || n_recent > rtp::kMaxBlocks)
    return fail(RTP_EINVAL, "n_recent must be in [1, 262143] (the block of the new token is always kept)");
  const HeadInfo hi = scan_mask(is_retrieval, Hq);
  if (int e = check_indexer(hi.n_ret, r, block, top_k)) return e;
  if (B == 0) return RTP_OK;
  if (!q || !k_cache || !v_cache || !cache_len || !out)
    return fail(RTP_EINVAL, "q, k_cache, v_cache, cache_len and out must be non-NULL");
  if (hi.n_ret > 0 && (!p_q || !centroids))
    return fail(RTP_EINVAL, "p_q and centroids must be non-NULL with retrieval heads");
  if (clustered && hi.n_ret > 0 && (!cl_m || !cl_off || !cl_mem))
    return fail(RTP_EINVAL, "the cluster tables must be non-NULL with retrieval heads");
  const DecodeLayout L = decode_layout(B, Lmax, Hq, hi.n_ret, top_k, n_recent,
                                       clustered);
  *need = L.total;
  if (!ws) return RTP_OK;
  if (int e = check_ws(ws, ws_bytes, L.total)) return e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  rtp::DecodeLaunch a;
  a.q = static_cast<const rtp::u16*>(q);
  a.kc = static_cast<const rtp::u16*>(k_cache);
  a.vc = static_cast<const rtp::u16*>(v_cache);
  a.cache_len = cache_len;
  a.p_q = p_q;
  a.cent = centroids;
  a.B = B;
  a.Lmax = Lmax;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.n_ret = hi.n_ret;
  a.r = r;
  a.window = window;
  a.top_k = top_k;
  a.n_recent = n_recent;
  a.n_split = kDecSplit;
  a.scale = resolve_scale(scale, d);
  a.ret_heads = hi.ret_heads.data();
  a.is_ret = is_retrieval;
  a.out = static_cast<rtp::u16*>(out);
  a.lse = lse;
  a.sel = reinterpret_cast<int32_t*>(w + L.sel);
  a.cscores = reinterpret_cast<float*>(w + L.cs);
  a.part_o = reinterpret_cast<float*>(w + L.po);
  a.part_ml = reinterpret_cast<float*>(w + L.pml);
  a.one_stream = one_stream;
  a.kv = kv;
  if (clustered && hi.n_ret > 0) {
    a.cl_m = cl_m;
    a.cl_off = cl_off;
    a.cl_mem = cl_mem;
    a.tok = reinterpret_cast<int32_t*>(w + L.tok);
    a.tok_cnt = reinterpret_cast<int32_t*>(w + L.tcnt);
  }
  hipError_t e = rtp::launch_decode(a, st);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  if (sel_out && hi.n_ret > 0) {
    const size_t width = (size_t)top_k + 1 + n_recent;
    e = hipMemcpyAsync(sel_out, a.sel, (size_t)B * hi.n_ret * width * 4,
                       hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return hip_fail(e, "selection copy");
  }
  return RTP_OK;
}

// Scratch of rtp_hybrid_attn_decode_noalloc: a device array of the library
// (each GPU the library runs on holds its own copy until the process ends).
// Host code never uses the array's name as an address: its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept in g_scratch_ptr.
static __device__ __align__(256) char scratch[RTP_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RTP_EUNSUPPORTED, "device index beyond the library's table");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return RTP_OK;
}
}  // namespace

extern "C" {

int rtp_hybrid_attn_decode(const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* cache_len,
                           int B, int Lmax, int Hq, int Hkv, int d,
                           const uint8_t* is_retrieval, int window,
                           const float* p_q, const float* centroids, int r,
                           int block, int top_k, int n_recent, float scale,
                           void* out, float* lse, int32_t* sel_out, void* ws,
                           size_t ws_bytes, rtp_stream_t stream) {
  g_err.clear();
  size_t need = 0;
  if (!ws) {  // validate and size first: a missing workspace is EWORKSPACE
    int e = decode_impl(q, k_cache, v_cache, cache_len, B, Lmax, Hq, Hkv, d,
                        is_retrieval, window, p_q, centroids, r, block, top_k,
                        n_recent, scale, out, lse, sel_out, nullptr, 0, false,
                        &need, stream);
    if (e) return e;
    return check_ws(ws, ws_bytes, need);
  }
  return decode_impl(q, k_cache, v_cache, cache_len, B, Lmax, Hq, Hkv, d,
                     is_retrieval, window, p_q, centroids, r, block, top_k,
                     n_recent, scale, out, lse, sel_out, ws, ws_bytes, false,
                     &need, stream);
}

int rtp_hybrid_attn_decode_noalloc(const void* q, const void* k_cache,
                                   const void* v_cache,
                                   const int32_t* cache_len, int B, int Lmax,
                                   int Hq, int Hkv, int d,
                                   const uint8_t* is_retrieval, int window,
                                   const float* p_q, const float* centroids,
                                   int r, int block, int top_k, int n_recent,
                                   float scale, void* out, float* lse,
                                   int32_t* sel_out, rtp_stream_t stream) {
  g_err.clear();
  size_t need = 0;
  int e = decode_impl(q, k_cache, v_cache, cache_len, B, Lmax, Hq, Hkv, d,
                      is_retrieval, window, p_q, centroids, r, block, top_k,
                      n_recent, scale, out, lse, sel_out, nullptr, 0, true,
                      &need, stream);
  if (e || need == 0) return e;
  if (need > RTP_NOALLOC_SCRATCH_BYTES)
    return fail(RTP_EWORKSPACE,
                "this decode step needs " + std::to_string(need) +
                    " bytes of scratch; rtp_hybrid_attn_decode_noalloc has " +
                    std::to_string((size_t)RTP_NOALLOC_SCRATCH_BYTES) +
                    " (use rtp_hybrid_attn_decode with a workspace)");
  void* ptr = nullptr;
  if ((e = scratch_of_current_device(&ptr))) return e;
  return decode_impl(q, k_cache, v_cache, cache_len, B, Lmax, Hq, Hkv, d,
                     is_retrieval, window, p_q, centroids, r, block, top_k,
                     n_recent, scale, out, lse, sel_out, ptr,
                     RTP_NOALLOC_SCRATCH_BYTES, true, &need, stream);
}

int rtp_hybrid_attn_decode_clustered(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* cache_len, int B, int Lmax, int Hq, int Hkv, int d,
    const uint8_t* is_retrieval, int window, const float* p_q,
    const float* centroids, const int32_t* cl_m, const int32_t* cl_off,
    const int32_t* cl_members, int r, int block, int top_k, int n_recent,
    float scale, void* out, float* lse, int32_t* sel_out, void* ws,
    size_t ws_bytes, rtp_stream_t stream) {
  g_err.clear();
  size_t need = 0;
  if (!ws) {
    int e = decode_impl(q, k_cache, v_cache, cache_len, B, Lmax, Hq, Hkv, d,
                        is_retrieval, window, p_q, centroids, r, block, top_k,
                        n_recent, scale, out, lse, sel_out, nullptr, 0, false,
                        &need, stream, cl_m, cl_off, cl_members, true);
    if (e) return e;
    return check_ws(ws, ws_bytes, need);
  }
  return decode_impl(q, k_cache, v_cache, cache_len, B, Lmax, Hq, Hkv, d,
                     is_retrieval, window, p_q, centroids, r, block, top_k,
                     n_recent, scale, out, lse, sel_out, ws, ws_bytes, false,
                     &need, stream, cl_m, cl_off, cl_members, true);
}

// Paged twins: the cache is a pool of pages and a block table; Lmax is
// 64 * max_blocks. cl_m == nullptr: the block decode.
static int decode_paged(const void* q, const void* k_pages,
                        const void* v_pages, const int32_t* block_table,
                        int max_blocks, int n_pages, const int32_t* cache_len,
                        int B, int Hq, int Hkv, int d,
                        const uint8_t* is_retrieval, int window,
                        const float* p_q, const float* centroids,
                        const int32_t* cl_m, const int32_t* cl_off,
                        const int32_t* cl_members, bool clustered, int r,
                        int block, int top_k, int n_recent, float scale,
                        void* out, float* lse, int32_t* sel_out, void* ws,
                        size_t ws_bytes, rtp_stream_t stream) {
  if (B > 0)
    if (int e = check_pages(block_table, max_blocks, n_pages)) return e;
  rtp::KvView kv;
  kv.table = block_table;
  kv.max_blocks = max_blocks;
  kv.n_pages = n_pages;
  const int Lmax = 64 * max_blocks;
  size_t need = 0;
  if (!ws) {
    int e = decode_impl(q, k_pages, v_pages, cache_len, B, Lmax, Hq, Hkv, d,
                        is_retrieval, window, p_q, centroids, r, block, top_k,
                        n_recent, scale, out, lse, sel_out, nullptr, 0, false,
                        &need, stream, cl_m, cl_off, cl_members, clustered, kv);
    if (e) return e;
    return check_ws(ws, ws_bytes, need);
  }
  return decode_impl(q, k_pages, v_pages, cache_len, B, Lmax, Hq, Hkv, d,
                     is_retrieval, window, p_q, centroids, r, block, top_k,
                     n_recent, scale, out, lse, sel_out, ws, ws_bytes, false,
                     &need, stream, cl_m, cl_off, cl_members, clustered, kv);
}

int rtp_hybrid_attn_decode_paged(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, int max_blocks, int n_pages,
    const int32_t* cache_len, int B, int Hq, int Hkv, int d,
    const uint8_t* is_retrieval, int window, const float* p_q,
    const float* centroids, int r, int block, int top_k, int n_recent,
    float scale, void* out, float* lse, int32_t* sel_out, void* ws,
    size_t ws_bytes, rtp_stream_t stream) {
  g_err.clear();
  return decode_paged(q, k_pages, v_pages, block_table, max_blocks, n_pages,
                      cache_len, B, Hq, Hkv, d, is_retrieval, window, p_q,
                      centroids, nullptr, nullptr, nullptr, false, r, block,
                      top_k, n_recent, scale, out, lse, sel_out, ws, ws_bytes,
                      stream);
}

int rtp_hybrid_attn_decode_clustered_paged(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, int max_blocks, int n_pages,
    const int32_t* cache_len, int B, int Hq, int Hkv, int d,
    const uint8_t* is_retrieval, int window, const float* p_q,
    const float* centroids, const int32_t* cl_m, const int32_t* cl_off,
    const int32_t* cl_members, int r, int block, int top_k, int n_recent,
    float scale, void* out, float* lse, int32_t* sel_out, void* ws,
    size_t ws_bytes, rtp_stream_t stream) {
  g_err.clear();
  return decode_paged(q, k_pages, v_pages, block_table, max_blocks, n_pages,
                      cache_len, B, Hq, Hkv, d, is_retrieval, window, p_q,
                      centroids, cl_m, cl_off, cl_members, true, r, block,
                      top_k, n_recent, scale, out, lse, sel_out, ws, ws_bytes,
                      stream);
}

}  // extern "C"
