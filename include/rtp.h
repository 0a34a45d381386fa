/*
 * rtp.h - C ABI of the headwise hybrid attention library for MI355X (gfx950).
 *
 * What it computes (the pages are web articles, cited by title and section):
 *
 *  - "阿里Qwen3 RTPurbo：15%全量Attention长文本5倍压缩方案", section
 *    "化繁为简，被低估的 SWA": each query head is fixed to one of two kinds. A
 *    small share keeps long-range access; the rest ("streaming heads") use
 *    causal sliding-window attention (SWA): query i attends keys
 *    i - window < j <= i.
 *  - "阿里RTPurboV2：Transformer再次崛起，百步训练实现10倍稀少把稳",
 *    paragraph on the low-rank projector (D -> r = 16), and the aitop.news
 *    summary of "Full Attention Strikes Back": long-range ("retrieval")
 *    heads use a 16-dimensional indexer to guess which earlier tokens
 *    matter, then run exact softmax attention only on that selected set.
 *    This library's indexer rule: blocks of `block` tokens; the query block
 *    qb scores every candidate key block 1 <= kb <= qb-1 by
 *        sc(qb,kb) = max_{j in kb} ( mean_{i in qb} P_q q_i ) . ( P_k k_j ),
 *    keeps the top_k candidates (ties: lower block index), and always adds
 *    the sink block 0 and the diagonal block qb. Query i of block qb then
 *    attends every key j <= i of the kept blocks.
 *  - Same RTPurboV2 article, paragraphs on clustering in the low-rank space
 *    and on the decode recipe: decode scores per-block key centroids
 *    c_kb = mean_{j in kb} P_k k_j with the projected query, keeps the sink,
 *    the last n_recent blocks and the top_k candidates, and attends exactly.
 *  - Same article, paragraph on feature and sequence compression working
 *    together (related keys gather in the low-rank space): rtp_cluster_keys
 *    groups the projected keys by k-means (Lloyd's algorithm, seeded by the
 *    blocks), and rtp_hybrid_attn_decode_clustered lets the retrieval heads
 *    choose among those clusters instead of blocks.
 *
 * Softmax everywhere: s_j = scale * q.k_j, lse = log sum_j exp(s_j),
 * out = sum_j exp(s_j - lse) v_j, computed with fp32 accumulation.
 *
 * Conventions (every entry point):
 *  - All tensors are dense, row-major, device memory owned by the caller.
 *    bf16 tensors are passed as raw 16-bit storage (`const void*`).
 *  - `is_retrieval` is a HOST array of Hq bytes (nonzero = retrieval head).
 *    n_ret = number of nonzero entries. Projections p_q/p_k are fp32
 *    [n_ret, r, d] device arrays for the retrieval heads in ascending head
 *    order.
 *  - GQA: query head h reads KV head h / (Hq / Hkv).
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). The library allocates no device memory: scratch space comes
 *    from the caller's workspace `ws` of `ws_bytes` bytes (256-byte aligned),
 *    sized by the matching *_workspace_bytes query (the one exception,
 *    rtp_hybrid_attn_decode_noalloc, uses a fixed array loaded with the
 *    library). Calls never synchronise.
 *    Some calls also run part of their work on a library-owned auxiliary
 *    stream of the device (default priority, created on first use):
 *    rtp_hybrid_attn_decode, and the prefills on sequences of more than
 *    4096 blocks. Events order that work after what was enqueued on
 *    `stream` before the call, and the rest of the call after it, so each
 *    call stays ordered on `stream` as a whole.
 *  - Arguments are validated on the host before anything is enqueued. On an
 *    error nothing is launched, outputs are untouched, and a negative status
 *    is returned; rtp_last_error() gives a thread-local message.
 *  - Results are deterministic: no atomics take part in any reduction.
 *  - Supported shapes: d = 128, block = 64, r a multiple of 16 in [16, 128],
 *    Hq <= 128, Hq % Hkv == 0. A prefill's S may be any size from 0 to
 *    16 777 152 = 2^24 - 64 (a ragged last block is handled; one KV head's
 *    K must fit a 4 GiB buffer descriptor; that largest S is tested against
 *    the oracle); larger S returns RTP_EUNSUPPORTED. top_k and n_recent are at most 262 143 (the most
 *    64-token blocks such a sequence has); larger values return RTP_EINVAL.
 *  - Two calls that share a workspace must not overlap in time.
 */
#ifndef RTP_H
#define RTP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define RTP_OK 0
#define RTP_EINVAL (-1)       /* null pointer, negative, too large or
                                 inconsistent size */
#define RTP_EUNSUPPORTED (-2) /* d != 128, block != 64, bad r, Hq > 128,
                                prefill S > 2^24 - 64 */
#define RTP_EWORKSPACE (-3)   /* ws too small or not 256-byte aligned */
#define RTP_EHIP (-4)         /* HIP runtime or launch error */

typedef struct ihipStream_t* rtp_stream_t; /* hipStream_t */

/* Human-readable name of a status code (static string). */
const char* rtp_status_string(int status);
/* Message of the last error on the calling thread ("" if none). */
const char* rtp_last_error(void);
/* Library version string. */
const char* rtp_version(void);

/* Kernel timing for measurement tools. rtp_profile(1) clears the record and
 * makes every later call record a pair of HIP events on its stream around
 * each kernel it launches; rtp_profile(0) stops. rtp_profile_read() waits for
 * the recorded events, writes up to `max` kernel names (static strings) and
 * elapsed milliseconds, clears the record and returns the count (or a
 * negative status). Not meant to be used while calls run on other threads. */
int rtp_profile(int enable);
int rtp_profile_read(const char** names, float* ms, int max);

/* Workspace bytes needed by rtp_indexer_select / rtp_hybrid_attn_prefill
 * for these sizes (0 on invalid arguments). Linear in S: V^T of every KV
 * head, the projected keys (4 r bytes per token per retrieval head) and
 * the selections; up to 4096 blocks also the score rows of each retrieval
 * head (a lower triangle, at most 33.5 MB per head), past them fixed-size
 * candidate buffers instead (0.56 GiB for top_k = 256). For example 0.13 GiB
 * at S = 128K with 5 retrieval heads and 2.39 GiB at S = 1M with 23. */
size_t rtp_prefill_workspace_bytes(int S, int Hq, int Hkv, int d,
                                   const uint8_t* is_retrieval, int r,
                                   int block, int top_k);

/*
 * rtp_indexer_select - the retrieval-head indexer alone (project, score,
 * select). Defined by the RTPurboV2 low-rank projector paragraph and the
 * aitop.news indexer summary, with the block rule stated at the top.
 *
 *  q [Hq,S,d] bf16, k [Hkv,S,d] bf16           inputs (only retrieval heads
 *                                               of q are read)
 *  p_q, p_k [n_ret,r,d] fp32                    projections
 *  sel [n_ret,n_b,top_k+2] int32   (out)        kept blocks per query block,
 *                                               ascending, padded with -1
 *  sel_count [n_ret,n_b] int32     (out)        number of kept blocks
 *  kth_scores [n_ret,n_b,2] fp32   (out, may be NULL)
 *        the k-th and (k+1)-th largest candidate scores (NaN when the row
 *        has fewer candidates), for logging near-ties
 *  centroids [n_ret,n_b,r] fp32    (out, may be NULL)
 *        per-block mean of the projected keys P_k k_j
 *  n_b = ceil(S / block). A row with no more candidates than top_k keeps
 *  them all.
 */
int rtp_indexer_select(const void* q, const void* k, int S, int Hq, int Hkv,
                       int d, const uint8_t* is_retrieval, const float* p_q,
                       const float* p_k, int r, int block, int top_k,
                       int32_t* sel, int32_t* sel_count, float* kth_scores,
                       float* centroids, void* ws, size_t ws_bytes,
                       rtp_stream_t stream);

/*
 * rtp_hybrid_attn_prefill - one layer of headwise hybrid attention over a
 * whole sequence. Streaming heads: SWA with `window` (window >= S gives
 * full causal attention). Retrieval heads: indexer selection, then exact
 * attention on the kept blocks.
 *
 *  q [Hq,S,d], k/v [Hkv,S,d] bf16
 *  scale            softmax scale; <= 0 means 1/sqrt(d)
 *  sel_in, sel_count_in   (may both be NULL) a selection in the layout of
 *        rtp_indexer_select; when given, the indexer is skipped and these
 *        blocks are used (each row strictly ascending, within 0..qb;
 *        rows that break this are read memory-safely but give undefined
 *        outputs)
 *  out [Hq,S,d] bf16 (out)        attention output, rounded to nearest even
 *  lse [Hq,S] fp32 (out, may be NULL)   natural-log sum of exp of scaled
 *                                        logits over the attended keys
 *  sel_out, sel_count_out (out, may be NULL) the selection used
 */
int rtp_hybrid_attn_prefill(const void* q, const void* k, const void* v,
                            int S, int Hq, int Hkv, int d,
                            const uint8_t* is_retrieval, int window,
                            const float* p_q, const float* p_k, int r,
                            int block, int top_k, float scale,
                            const int32_t* sel_in,
                            const int32_t* sel_count_in, void* out,
                            float* lse, int32_t* sel_out,
                            int32_t* sel_count_out, void* ws, size_t ws_bytes,
                            rtp_stream_t stream);

/* Retrieval-head modes of rtp_headwise_prefill. */
#define RTP_RETRIEVAL_SPARSE 0  /* indexer selection + exact attention on it */
#define RTP_RETRIEVAL_FULL 1    /* causal full attention */

/* Workspace bytes for rtp_headwise_prefill (0 on invalid arguments). In
 * RTP_RETRIEVAL_FULL mode no selection workspace is needed. */
size_t rtp_headwise_prefill_workspace_bytes(int S, int Hq, int Hkv, int d,
                                            const uint8_t* is_retrieval,
                                            int retrieval, int r, int block,
                                            int top_k);

/*
 * rtp_headwise_prefill - rtp_hybrid_attn_prefill with a window per head, a
 * per-call choice of how retrieval heads attend, and the decode centroids
 * as an epilogue. This follows the RTPurboV2 article's paragraph on the
 * Qwen3-Coder-30B-A3B deployment: retrieval heads use full attention in
 * prefill together with K-cache clustering and run sparse only in decode;
 * streaming heads use SWA with windows that may differ (8192 for some).
 *
 *  windows [Hq] int32, HOST (each >= 1): streaming head h attends keys
 *        i - windows[h] < j <= i (windows[h] >= S: causal full attention).
 *        Entries of retrieval heads are not used.
 *  retrieval  RTP_RETRIEVAL_SPARSE: retrieval heads select blocks as in
 *        rtp_hybrid_attn_prefill (p_q, p_k, top_k, sel_in/sel_count_in and
 *        sel_out/sel_count_out as there);
 *        RTP_RETRIEVAL_FULL: retrieval heads attend every key j <= i;
 *        p_q and top_k are not used and sel_in/sel_out must be NULL.
 *  centroids [n_ret,n_b,r] fp32 (out, may be NULL): per-block mean of the
 *        projected keys P_k k_j of each retrieval head (as in
 *        rtp_indexer_select; a ragged last block averages its tokens). For a
 *        decode cache holding this sequence, the full blocks' rows equal
 *        what rtp_build_centroids computes, up to fp32 rounding. Needs p_k.
 *  Other arguments as in rtp_hybrid_attn_prefill; ws is sized by
 *  rtp_headwise_prefill_workspace_bytes. A NULL `windows` or an unknown
 *  mode is RTP_EINVAL.
 */
int rtp_headwise_prefill(const void* q, const void* k, const void* v, int S,
                         int Hq, int Hkv, int d, const uint8_t* is_retrieval,
                         const int32_t* windows, int retrieval,
                         const float* p_q, const float* p_k, int r, int block,
                         int top_k, float scale, const int32_t* sel_in,
                         const int32_t* sel_count_in, void* out, float* lse,
                         int32_t* sel_out, int32_t* sel_count_out,
                         float* centroids, void* ws, size_t ws_bytes,
                         rtp_stream_t stream);

/* Workspace bytes for rtp_dense_attn_prefill. */
size_t rtp_dense_workspace_bytes(int S, int Hq, int Hkv, int d);

/*
 * rtp_dense_attn_prefill - dense causal attention on the same tile engine:
 * the full-attention baseline the pages compare against (FlashAttention-2
 * in the aitop.news summary). Same layouts as rtp_hybrid_attn_prefill.
 */
int rtp_dense_attn_prefill(const void* q, const void* k, const void* v,
                           int S, int Hq, int Hkv, int d, float scale,
                           void* out, float* lse, void* ws, size_t ws_bytes,
                           rtp_stream_t stream);

/*
 * rtp_build_centroids - decode-side key clustering (RTPurboV2, K-cache
 * clustering): for every sequence b, retrieval head rho and FULL block kb
 * (kb < cache_len[b] / block):
 *     centroids[b,rho,kb,:] = mean_{j in kb} P_k[rho] k_cache[b,g,j,:]
 * where g is the KV head of retrieval head rho. Entries of partial or
 * absent blocks are left untouched.
 *
 *  k_cache [B,Hkv,Lmax,d] bf16; cache_len [B] int32 DEVICE array
 *  (0 <= cache_len[b] <= Lmax); p_k [n_ret,r,d] fp32;
 *  centroids [B,n_ret,Lmax/block,r] fp32 (out)
 */
int rtp_build_centroids(const void* k_cache, const int32_t* cache_len, int B,
                        int Lmax, int Hq, int Hkv, int d,
                        const uint8_t* is_retrieval, const float* p_k, int r,
                        int block, float* centroids, rtp_stream_t stream);

/*
 * rtp_decode_append - appends one token per sequence to the decode cache and
 * keeps the centroids of rtp_build_centroids current (RTPurboV2: the K
 * cache stays clustered in the low-rank space during decode; here a block's
 * centroid is added when its last token arrives):
 *   k_cache[b,g,L_b,:] = k_new[b,g,:], v_cache[b,g,L_b,:] = v_new[b,g,:]
 *   with L_b = cache_len[b]; if L_b + 1 is a multiple of block, the
 *   centroids of block L_b / block are computed for every retrieval head
 *   exactly as rtp_build_centroids would; then cache_len[b] = L_b + 1.
 *
 *  k_cache, v_cache [B,Hkv,Lmax,d] bf16 (in/out); cache_len [B] int32
 *  DEVICE array (in/out); k_new, v_new [B,Hkv,d] bf16;
 *  p_k [n_ret,r,d] fp32 and centroids [B,n_ret,Lmax/block,r] fp32 (in/out;
 *  both may be NULL when no head is a retrieval head).
 *  The caller keeps cache_len[b] < Lmax; a sequence whose cache is full is
 *  left unchanged. Two kernels on `stream`, nothing allocated.
 */
int rtp_decode_append(void* k_cache, void* v_cache, int32_t* cache_len,
                      const void* k_new, const void* v_new, int B, int Lmax,
                      int Hq, int Hkv, int d, const uint8_t* is_retrieval,
                      const float* p_k, int r, int block, float* centroids,
                      rtp_stream_t stream);

/* Workspace bytes for rtp_hybrid_attn_decode. */
size_t rtp_decode_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int d,
                                  const uint8_t* is_retrieval, int r,
                                  int block, int top_k, int n_recent);

/*
 * rtp_hybrid_attn_decode - one decode step for a batch of sequences
 * (RTPurboV2 decode recipe: sparse retrieval heads via key clustering, SWA
 * for streaming heads). The new token's K/V are already appended, so
 * sequence b has L = cache_len[b] >= 1 tokens and the query sits at L-1.
 *
 *  Streaming head: attends keys max(0, L-window) .. L-1.
 *  Retrieval head rho: n_b = ceil(L/block); q~ = P_q[rho] q; candidates
 *    1 .. n_b-n_recent-1 scored by q~ . centroids[b,rho,kb]; keeps block 0,
 *    the top_k candidates (ties: lower index) and blocks n_b-n_recent ..
 *    n_b-1; attends every cached token of the kept blocks. n_recent >= 1:
 *    the block holding the new token (possibly partial, so without a
 *    centroid) is always kept.
 *
 *  q [B,Hq,d] bf16; k_cache/v_cache [B,Hkv,Lmax,d] bf16;
 *  cache_len [B] int32 DEVICE array (1 <= cache_len[b] <= Lmax);
 *  p_q [n_ret,r,d] fp32; centroids [B,n_ret,Lmax/block,r] fp32 from
 *  rtp_build_centroids;
 *  out [B,Hq,d] bf16 (out); lse [B,Hq] fp32 (out, may be NULL);
 *  sel_out [B,n_ret,top_k+1+n_recent] int32 (out, may be NULL): kept blocks
 *  ascending, -1 padded.
 *
 *  Streams: when both kinds of head are present, the streaming-head
 *  attention runs on an auxiliary stream that the library creates once per
 *  device (default priority), concurrently with the block choice on
 *  `stream`. Events order it after the work enqueued on `stream` before the
 *  call, and the rest of the call after it, so the step as a whole is
 *  ordered on `stream` like any other asynchronous call; the host never
 *  waits. If the auxiliary stream cannot be created, everything runs on
 *  `stream`.
 */
int rtp_hybrid_attn_decode(const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* cache_len,
                           int B, int Lmax, int Hq, int Hkv, int d,
                           const uint8_t* is_retrieval, int window,
                           const float* p_q, const float* centroids, int r,
                           int block, int top_k, int n_recent, float scale,
                           void* out, float* lse, int32_t* sel_out, void* ws,
                           size_t ws_bytes, rtp_stream_t stream);

/* Scratch bytes held by the library for rtp_hybrid_attn_decode_noalloc on
 * each GPU it runs on (64 MiB). */
#define RTP_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * rtp_hybrid_attn_decode_noalloc - rtp_hybrid_attn_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc). Same arguments, results
 * and validation as rtp_hybrid_attn_decode, without ws / ws_bytes: the
 * scratch space comes from a device array of the library, fixed at
 * RTP_NOALLOC_SCRATCH_BYTES per GPU, that lives until the process ends.
 * Nothing is allocated or created: no device memory, and no auxiliary
 * stream (every kernel runs on `stream`, in order).
 *
 *  A step whose scratch need (rtp_decode_workspace_bytes of the same sizes)
 *  exceeds RTP_NOALLOC_SCRATCH_BYTES returns RTP_EWORKSPACE with nothing
 *  launched. (For example, 32 sequences of 256K tokens with 32 query / 4 KV
 *  heads, 5 retrieval heads and top_k 64 need about 7 MB.)
 *  All calls on one GPU share that GPU's array, and no call needs it to
 *  start cleared: two calls that overlap in time on one GPU (on different
 *  streams, or from different threads) race and give undefined results.
 */
int rtp_hybrid_attn_decode_noalloc(const void* q, const void* k_cache,
                                   const void* v_cache,
                                   const int32_t* cache_len, int B, int Lmax,
                                   int Hq, int Hkv, int d,
                                   const uint8_t* is_retrieval, int window,
                                   const float* p_q, const float* centroids,
                                   int r, int block, int top_k, int n_recent,
                                   float scale, void* out, float* lse,
                                   int32_t* sel_out, rtp_stream_t stream);

/* Workspace bytes for rtp_cluster_keys (0 on invalid arguments). */
size_t rtp_cluster_workspace_bytes(int B, int Lmax, int Hq, int Hkv, int d,
                                   const uint8_t* is_retrieval, int r,
                                   int block);

/*
 * rtp_cluster_keys - semantic clustering of the decode K cache
 * ("阿里RTPurboV2：Transformer再次崛起，百步训练实现10倍稀少把稳", paragraph
 * on the synergy of feature and sequence compression: after the low-rank
 * projection, related keys lie close together and unrelated ones far apart,
 * so the sequence can be compressed by clustering; Qwen3-Coder recipe
 * paragraph: the K cache is clustered during prefill and decode runs
 * sparsely). The pages give no algorithm; this library's reading is k-means
 * by Lloyd's algorithm, seeded by the blocks:
 *
 *  For sequence b and retrieval head rho, with L = cache_len[b],
 *  n_b = ceil(L / block) and m = max(n_b - n_recent, 1): the points are the
 *  projected keys x_t = P_k[rho] k_cache[b,g,t] of tokens block .. block*m-1
 *  (blocks 1 .. m-1; the sink block and the last n_recent blocks are always
 *  attended and are not clustered). Cluster ids are 1 .. m-1; cluster c
 *  starts from centroids[b,rho,c,:] (its block centroid after
 *  rtp_build_centroids, or the result of an earlier call). Each of the
 *  `iters` steps assigns every point to the nearest centroid (squared
 *  Euclidean distance; ties: the lower id), then moves every cluster that
 *  has members to their mean; a cluster without members keeps its
 *  centroid. With iters = 0 the clusters are the blocks.
 *
 *  k_cache [B,Hkv,Lmax,d] bf16; cache_len [B] int32 DEVICE array;
 *  p_k [n_ret,r,d] fp32 with r in {16, 32, 48, 64}; n_recent >= 1;
 *  0 <= iters <= 1000.
 *  centroids [B,n_ret,Lmax/block,r] fp32 (in/out): entries 1 .. m-1 become
 *    the cluster centroids (each the mean of its members); others untouched.
 *  cl_m [B] int32 (out): m of each sequence.
 *  cl_off [B,n_ret,Lmax/block+1] int32 (out): the members of cluster c are
 *    cl_members[b,rho, cl_off[c] .. cl_off[c+1]-1]; cl_off[0] = cl_off[1] =
 *    0, and the entries from m on hold the number of clustered tokens.
 *  cl_members [B,n_ret,Lmax] int32 (out): token ids grouped by cluster,
 *    ascending within each cluster.
 *  ws: rtp_cluster_workspace_bytes bytes (may be NULL when iters = 0).
 *
 *  Precision: the nearest centroid is taken as the largest
 *  x . mu_c - |mu_c|^2 / 2, with the products formed from split bf16 parts
 *  (about 2^-16 of |x| |mu_c|), so a point that close to equidistant from
 *  two centroids may take either; the means are summed in fp64. Results are
 *  deterministic.
 */
int rtp_cluster_keys(const void* k_cache, const int32_t* cache_len, int B,
                     int Lmax, int Hq, int Hkv, int d,
                     const uint8_t* is_retrieval, const float* p_k, int r,
                     int block, int n_recent, int iters, float* centroids,
                     int32_t* cl_m, int32_t* cl_off, int32_t* cl_members,
                     void* ws, size_t ws_bytes, rtp_stream_t stream);

/* Workspace bytes for rtp_hybrid_attn_decode_clustered. */
size_t rtp_decode_clustered_workspace_bytes(int B, int Lmax, int Hq, int Hkv,
                                            int d, const uint8_t* is_retrieval,
                                            int r, int block, int top_k,
                                            int n_recent);

/*
 * rtp_hybrid_attn_decode_clustered - rtp_hybrid_attn_decode whose retrieval
 * heads choose among the clusters of rtp_cluster_keys (same RTPurboV2
 * paragraphs: decode skips whole groups of unrelated tokens and attends the
 * kept ones exactly).
 *
 *  Retrieval head rho of sequence b, with L = cache_len[b] (which may have
 *  grown since the clustering), n_b = ceil(L/block) and m = cl_m[b]: the
 *  candidates are 1 .. n_b-n_recent-1; a candidate c < m is cluster c,
 *  scored by q~ . centroids[b,rho,c] where q~ = P_q[rho] q, and is skipped
 *  when it has no members; a candidate c >= m (a block that left the recent
 *  window after the clustering) is block c with its block centroid (kept
 *  current by rtp_decode_append). The sink block 0, the top_k candidates
 *  (ties: lower id) and the blocks n_b-n_recent .. n_b-1 are kept; the head
 *  attends every member token of a kept cluster and every token of a kept
 *  block, exactly. Streaming heads as in rtp_hybrid_attn_decode.
 *
 *  cl_m, cl_off, cl_members: the tables of rtp_cluster_keys. sel_out
 *  [B,n_ret,top_k+1+n_recent] (may be NULL): kept ids ascending, -1 padded
 *  (an empty cluster appears only when fewer than top_k candidates have
 *  members; it adds no token). Other arguments, streams and validation as
 *  in rtp_hybrid_attn_decode; ws of rtp_decode_clustered_workspace_bytes
 *  bytes. With the tables of iters = 0 the result equals
 *  rtp_hybrid_attn_decode bit for bit.
 */
int rtp_hybrid_attn_decode_clustered(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* cache_len, int B, int Lmax, int Hq, int Hkv, int d,
    const uint8_t* is_retrieval, int window, const float* p_q,
    const float* centroids, const int32_t* cl_m, const int32_t* cl_off,
    const int32_t* cl_members, int r, int block, int top_k, int n_recent,
    float scale, void* out, float* lse, int32_t* sel_out, void* ws,
    size_t ws_bytes, rtp_stream_t stream);

/*
 * Paged decode cache (the survey's incremental-cache step with paged KV; a
 * serving engine keeps the K/V of many sequences in fixed-size pages). The
 * *_paged calls below are the calls of the same name without the suffix,
 * with the contiguous cache [B,Hkv,Lmax,d] replaced by:
 *
 *  k_pages, v_pages [n_pages,Hkv,block,d] bf16: a pool of pages, each
 *    holding `block` (= 64) consecutive tokens of every KV head;
 *  block_table [B,max_blocks] int32 DEVICE array: entry (b, j) is the page
 *    holding tokens 64 j .. 64 j + 63 of sequence b (the caller owns page
 *    allocation; entries past the sequence's last block are not read);
 *  Lmax = 64 * max_blocks everywhere the unpaged call uses it (centroid
 *    table [B,n_ret,max_blocks,r], cluster tables, workspace queries).
 *
 *  Page ids outside [0, n_pages) are clamped into the pool, so a bad table
 *  gives wrong results but no access outside the pool. Results equal those
 *  of the unpaged call on the cache the table describes, bit for bit.
 *  Extra errors: RTP_EINVAL for a NULL block_table, max_blocks < 1 or
 *  n_pages < 1 (when B > 0).
 */
int rtp_build_centroids_paged(const void* k_pages, const int32_t* block_table,
                              int max_blocks, int n_pages,
                              const int32_t* cache_len, int B, int Hq, int Hkv,
                              int d, const uint8_t* is_retrieval,
                              const float* p_k, int r, int block,
                              float* centroids, rtp_stream_t stream);

/* Appends at token cache_len[b], i.e. into page block_table[b, L_b / 64]
 * at row L_b % 64 (that page must be allocated in the table). */
int rtp_decode_append_paged(void* k_pages, void* v_pages,
                            const int32_t* block_table, int max_blocks,
                            int n_pages, int32_t* cache_len, const void* k_new,
                            const void* v_new, int B, int Hq, int Hkv, int d,
                            const uint8_t* is_retrieval, const float* p_k,
                            int r, int block, float* centroids,
                            rtp_stream_t stream);

/* ws: rtp_decode_workspace_bytes(B, 64 * max_blocks, ...) bytes. */
int rtp_hybrid_attn_decode_paged(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, int max_blocks, int n_pages,
    const int32_t* cache_len, int B, int Hq, int Hkv, int d,
    const uint8_t* is_retrieval, int window, const float* p_q,
    const float* centroids, int r, int block, int top_k, int n_recent,
    float scale, void* out, float* lse, int32_t* sel_out, void* ws,
    size_t ws_bytes, rtp_stream_t stream);

/* ws: rtp_cluster_workspace_bytes(B, 64 * max_blocks, ...) bytes. */
int rtp_cluster_keys_paged(const void* k_pages, const int32_t* block_table,
                           int max_blocks, int n_pages,
                           const int32_t* cache_len, int B, int Hq, int Hkv,
                           int d, const uint8_t* is_retrieval,
                           const float* p_k, int r, int block, int n_recent,
                           int iters, float* centroids, int32_t* cl_m,
                           int32_t* cl_off, int32_t* cl_members, void* ws,
                           size_t ws_bytes, rtp_stream_t stream);

/* ws: rtp_decode_clustered_workspace_bytes(B, 64 * max_blocks, ...) bytes. */
int rtp_hybrid_attn_decode_clustered_paged(
    const void* q, const void* k_pages, const void* v_pages,
    const int32_t* block_table, int max_blocks, int n_pages,
    const int32_t* cache_len, int B, int Hq, int Hkv, int d,
    const uint8_t* is_retrieval, int window, const float* p_q,
    const float* centroids, const int32_t* cl_m, const int32_t* cl_off,
    const int32_t* cl_members, int r, int block, int top_k, int n_recent,
    float scale, void* out, float* lse, int32_t* sel_out, void* ws,
    size_t ws_bytes, rtp_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RTP_H */
