/*
 * rkv.h - C ABI of an MI355X (gfx950) implementation of RocketKV's hot path:
 * SnapKV++ permanent KV eviction at prefill and hybrid sparse attention at each decode step.
 *
 * Method: "RocketKV: Accelerating Long-Context LLM Inference via Two-Stage KV Cache
 * Compression" (arXiv 2502.14051). Passages cited below by page and section:
 *   [summary]   summarizepaper.com summary, "Key points"
 *   [rebuttal]  paperhub.cn, the authors' rebuttal, by section heading
 *   [abstract]  pith.science record, abstract (v3)
 *
 * Conventions shared by every call
 *   - Pointers are DEVICE pointers to dense row-major arrays unless stated otherwise. The caller
 *     owns every buffer, workspaces included; the library never allocates or frees, and it
 *     synchronises only in rkv_hybrid_decode_status. It keeps no state between calls apart from
 *     what a workspace holds (and the fixed scratch of rkv_hybrid_decode_step_noalloc), so
 *     concurrent calls on different streams are safe as long as their output and workspace
 *     buffers do not overlap (and they are not both rkv_hybrid_decode_step_noalloc on one GPU).
 *   - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued asynchronously.
 *   - dtype: RKV_F32 (float) or RKV_BF16 (bfloat16 stored as uint16 bit patterns). q, K, V,
 *     summaries and attention outputs share the call's dtype; scores, pooled scores and all
 *     accumulation are float32; indices are int32.
 *   - GQA: query head g uses KV head g / (Hq / Hkv); Hq must be a multiple of Hkv.
 *   - Return value: RKV_OK (0) or a negative RKV_ERR_* code. All argument checks run on the
 *     host before anything is enqueued, so a failed call has no side effects. RKV_ERR_LAUNCH
 *     reports an enqueue failure; faults inside kernels surface at the caller's next
 *     synchronisation.
 *   - Every index selection breaks score ties toward the lower index and returns indices in
 *     ascending order.
 */
#ifndef RKV_H
#define RKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RKV_VERSION 1

enum rkv_status {
  RKV_OK = 0,
  RKV_ERR_NULL = -1,        /* a required pointer is NULL */
  RKV_ERR_SHAPE = -2,       /* a size or parameter is out of range or inconsistent */
  RKV_ERR_DTYPE = -3,       /* unknown dtype */
  RKV_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than the matching *_workspace_bytes */
  RKV_ERR_UNSUPPORTED = -5, /* valid but not implemented here (e.g. head dim not 64 or 128) */
  RKV_ERR_LAUNCH = -6,      /* the HIP runtime refused to enqueue a kernel */
  RKV_ERR_SCRATCH = -7      /* the shape needs more than RKV_NOALLOC_SCRATCH_BYTES of scratch */
};

enum rkv_dtype { RKV_F32 = 0, RKV_BF16 = 1 };
enum rkv_pool { RKV_POOL_AVG = 0, RKV_POOL_MAX = 1 };

/* Library version (RKV_VERSION). */
int rkv_version(void);

/* Static English description of a status code; never NULL. */
const char* rkv_status_string(int status);

/* ------------------------------------------------------------------------------------------
 * Budget planner (host only, no GPU work). The pages' rule for turning a token budget into the
 * two stages' settings ([rebuttal] "Is Page Always Divided Into 4?": the compression ratio
 * C = L / token_budget is split evenly between SnapKV++ and hybrid attention, and hybrid
 * attention's share again evenly between the sequence (page size) and head (channels)
 * dimensions; "Lack of Direct Latency Comparison": the budget counts the approximation's
 * traffic, so with pages of ps tokens and r of D channels the approximation costs
 * keep*r/(ps*2*D) tokens and the rest goes to sparse attention; "Potential Sensitivity to
 * Kernel Size in SnapKV++": longer inputs take larger pooling kernels).
 *
 * With s = sqrt(C) per stage and d = sqrt(s) per dimension of the second stage:
 *   keep          = round(L / s), clamped to [W, L]
 *   page_size     = max(1, round(d))
 *   r             = round(D / d), clamped to [1, D]
 *   approx_tokens = ceil(keep * r / (page_size * 2 * D))
 *   topk          = token_budget - approx_tokens, rounded down to a multiple of page_size and
 *                   clamped to [page_size, keep rounded up to a page]
 *   pool_kernel   = 7 for L <= 4096, 15 for L <= 16384, 31 for L <= 65536, else 63
 * A budget of at least L compresses nothing: keep = L, page_size = 1, r = D, topk = L,
 * approx_tokens = 0. Requires L >= 1, D >= 1, 1 <= W <= L, token_budget >= 1; every output
 * pointer non-NULL. Outputs are written only on success.
 * ------------------------------------------------------------------------------------------ */
int rkv_plan_budget(int L, int D, int W, int token_budget, int* keep, int* page_size, int* r,
                    int* topk, int* pool_kernel, int* approx_tokens);

/* ------------------------------------------------------------------------------------------
 * Stage 1 - SnapKV++ permanent eviction ([rebuttal] "Measurement of Exact-TopK": one-time top-k
 * filtering of the prompt; "SCBench Results": driven by the queries at the end of the prompt;
 * "Is Needle Among Evicted Tokens": independent per KV head and layer; [summary] and [rebuttal]
 * "Novelty of SnapKV++": the GQA enhancement; "Potential Sensitivity to Kernel Size in
 * SnapKV++": the pooling kernel size).
 *
 * For every sequence b and KV head h:
 *   s[g,i,j] = scale * <q_win[b,g,i,:], k[b,h,j,:]>   for the group's query heads g, window row
 *              i (prompt position L-W+i) and keys j <= L-W+i (causal);
 *   A = row softmax of s;  c[j] = sum_{g,i} A[g,i,j] for prefix keys j < L-W;
 *   pooled = same-size 1D pooling of c with kernel `pool_kernel` (odd) and zero padding
 *            (RKV_POOL_AVG: box sum / pool_kernel; RKV_POOL_MAX: box maximum);
 *   kept = the keep-W prefix positions with the highest pooled score, ascending, followed by
 *          the W window positions L-W .. L-1.  When keep >= L nothing is evicted: kept = 0..L-1.
 * Lc = min(keep, L) slots per head are produced.
 *
 * q_win      [B, Hq, W, D]   queries of the last W prompt positions
 * k, v       [B, Hkv, L, D]  the prompt's keys and values
 * kept_idx   [B, Hkv, Lc]    int32 out: kept prompt positions
 * k_out,v_out[B, Hkv, Lc, D] out: the compressed cache (rows of k, v at kept_idx); both NULL
 *                            to compute indices only, otherwise both non-NULL
 * pooled_out [B, Hkv, L-W]   float out, may be NULL: the pooled scores (unused when keep >= L)
 * scale      softmax scale (1/sqrt(D) for standard attention); must be finite and > 0
 * Requires 1 <= W <= L, W <= keep, D in {64, 128}, pool_kernel odd >= 1.
 * ws         device workspace of at least rkv_snapkvpp_workspace_bytes(...) bytes (16-byte
 *            aligned); contents on entry are ignored.
 * ------------------------------------------------------------------------------------------ */
int rkv_snapkvpp_workspace_bytes(int B, int Hq, int Hkv, int L, int D, int W, int keep,
                                 int dtype, size_t* bytes);
int rkv_snapkvpp_evict(const void* q_win, const void* k, const void* v, int B, int Hq, int Hkv,
                       int L, int D, int W, int keep, int pool_kernel, int pool_type, float scale,
                       int dtype, int32_t* kept_idx, void* k_out, void* v_out, float* pooled_out,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Page summaries ([rebuttal] "Explanation of Calculating Approximate Attention Scores", paper
 * Figure 3: K is split into pages of consecutive tokens and each page keeps its element-wise
 * minimum and maximum).
 *
 * k_c            [B, Hkv, Lc, D]  compressed keys
 * kmin_t, kmax_t [B, Hkv, D, P]   out, channel-major, P = ceil(Lc / page_size):
 *                kmin_t[b,h,c,p] = min over slots t of page p (t < Lc) of k_c[b,h,t,c]; same
 *                for max. Values are copied exactly (no rounding).
 * Requires Lc >= 1, page_size >= 1, D in {64, 128}.
 * ------------------------------------------------------------------------------------------ */
int rkv_build_page_summaries(const void* k_c, int B, int Hkv, int Lc, int D, int page_size,
                             int dtype, void* kmin_t, void* kmax_t, void* stream);

/* ------------------------------------------------------------------------------------------
 * Hybrid approximate page scores ([rebuttal] "Explanation of Calculating Approximate Attention
 * Scores": the bound max(q*Kmin, q*Kmax) per page, computed only on the head-dim positions
 * where |q| is large, fetching Kmin or Kmax per position by the sign of q, and GQA-consistent
 * through the group sums of q and |q|; "Novelty": reduction along both sequence and head dims).
 *
 * For every sequence b and KV head h with query heads g of its group:
 *   a[c] = sum_g |q[b,g,c]|, qbar[c] = sum_g q[b,g,c]    (float32)
 *   C    = the r channels with the largest a (ties: lower channel), ascending
 *   page_scores[b,h,p] = sum_{c in C} (qbar[c] >= 0 ? qbar[c]*kmax_t[b,h,c,p]
 *                                                   : qbar[c]*kmin_t[b,h,c,p])
 *        which equals sum_{c in C} max(qbar[c]*kmin, qbar[c]*kmax).
 * q              [B, Hq, D]       decode queries
 * kmin_t, kmax_t [B, Hkv, D, P]   from rkv_build_page_summaries
 * chan_idx       [B, Hkv, r]      int32 out, may be NULL: C
 * page_scores    [B, Hkv, P]      float out
 * Requires 1 <= r <= D, D in {64, 128}, Hq / Hkv <= 8, P >= 1.
 * ------------------------------------------------------------------------------------------ */
int rkv_hybrid_approx_scores(const void* q, const void* kmin_t, const void* kmax_t, int B,
                             int Hq, int Hkv, int D, int P, int r, int dtype, int32_t* chan_idx,
                             float* page_scores, void* stream);

/* ------------------------------------------------------------------------------------------
 * Top-k selection ([rebuttal] "Explanation of Calculating Approximate Attention Scores": select
 * the pages with higher scores; "Measurement of Exact-TopK": SnapKV's one-time top-k filter).
 *
 * scores  [rows, n] float (finite; -0.0 and +0.0 are equal)
 * idx_out [rows, min(k, n)] int32 out: per row, the indices of the min(k, n) largest scores,
 *         ties to the lower index, in ascending index order.
 * Requires rows >= 1, n >= 1, k >= 0 (k == 0 does nothing and idx_out may be NULL). ws may be
 * NULL when the workspace size is 0.
 * ------------------------------------------------------------------------------------------ */
int rkv_topk_workspace_bytes(int rows, int n, int k, size_t* bytes);
int rkv_topk_select(const float* scores, int rows, int n, int k, int32_t* idx_out, void* ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Sparse exact attention over the selected pages ([rebuttal] "Lack of Direct Latency
 * Comparison": Step 3, sparse attention on the selected tokens; "Explanation of Calculating
 * Approximate Attention Scores": all heads of a GQA group share the selection).
 *
 * For every sequence b, query head g and its KV head h:
 *   T = slots t of the listed pages (t = page*page_size + u, u < page_size, t < Lc)
 *   out[b,g,:] = sum_{t in T} softmax_t(scale * <q[b,g,:], k_c[b,h,t,:]>) * v_c[b,h,t,:]
 * q         [B, Hq, D]
 * k_c, v_c  [B, Hkv, Lc, D]
 * page_idx  [B, Hkv, n_pages] int32 page numbers in [0, ceil(Lc/page_size)), each at most
 *           once (entries outside that range are ignored)
 * out       [B, Hq, D] out (dtype of the call; bf16 rounds to nearest even). Scores, softmax
 *           and sums are float32; for bf16 with D = 128 the product with V runs on matrix cores
 *           with the softmax weights rounded to bf16.
 * Requires 1 <= n_pages <= ceil(Lc/page_size), n_pages <= 262144, D in {64, 128},
 * Hq / Hkv <= 8, scale finite.
 * ws        workspace of rkv_sparse_attend_workspace_bytes(...) bytes (may be 0, then NULL ok).
 * ------------------------------------------------------------------------------------------ */
int rkv_sparse_attend_workspace_bytes(int B, int Hq, int Hkv, int D, int page_size, int n_pages,
                                      int dtype, size_t* bytes);
int rkv_sparse_attend_decode(const void* q, const void* k_c, const void* v_c,
                             const int32_t* page_idx, int B, int Hq, int Hkv, int Lc, int D,
                             int page_size, int n_pages, float scale, int dtype, void* out,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * One hybrid decode step: the approximate page scores, the page top-k (k = n_pages) and the
 * sparse attention of the three calls above, in a single kernel launch when B*Hkv <= 256, and as
 * those three calls' launches (with the scores, pages and attention partials in the workspace)
 * when more heads than that fill the GPU with one block each ([rebuttal]
 * "Explanation of Calculating Approximate Attention Scores", "Lack of Direct Latency
 * Comparison": Steps 1-2 approximate and select, Step 3 attends). Scores and selected pages are
 * bit-identical to those of the separate calls; the output equals theirs up to float rounding
 * order.
 *
 * q, kmin_t, kmax_t, k_c, v_c, out as in the three calls; n_pages = pages to select (1..P).
 * chan_idx    [B, Hkv, r]       int32 out, may be NULL
 * page_scores [B, Hkv, P]       float out, may be NULL
 * page_idx    [B, Hkv, n_pages] int32 out, may be NULL: the selected pages, ascending
 * Requires P = ceil(Lc/page_size) <= 8192 and the limits of the three calls.
 * ws          rkv_hybrid_decode_workspace_bytes(...) bytes (its size depends on the shape B,
 *             Hq, Hkv, Lc, D, page_size and dtype, not on n_pages), zero-filled ONCE by
 *             rkv_hybrid_decode_workspace_init before its first use, and again before it is used
 *             for a different shape. The workspace holds, per KV head, a call counter and a
 *             count of started blocks. The blocks of a head exchange scores and partial results
 *             through the workspace as 64-bit words tagged with the call counter, and a block
 *             that still misses another block's result after about 20 us of wall-clock time
 *             (the environment variable RKV_STEAL_US, read at each call, sets this deadline;
 *             a negative value makes waiting blocks redo all such work, for testing)
 *             computes it itself (bit-identical); so a call finishes however its blocks are
 *             scheduled, also while other work shares the GPU, and leaves the counters ready for
 *             the next call (no call has to clear anything). Waits for words that must already be
 *             on their way are bounded by about 1 ms; one that runs out sets a bit of the
 *             workspace's status word and that call's output is not valid: read it with
 *             rkv_hybrid_decode_status, and initialise the workspace again before reusing it.
 *             Calls that overlap in time must not share a workspace; calls on different
 *             workspaces may run concurrently on any streams.
 * ------------------------------------------------------------------------------------------ */
int rkv_hybrid_decode_workspace_bytes(int B, int Hq, int Hkv, int Lc, int D, int page_size,
                                      int n_pages, int dtype, size_t* bytes);
int rkv_hybrid_decode_workspace_init(void* ws, size_t ws_bytes, void* stream);
int rkv_hybrid_decode_step(const void* q, const void* kmin_t, const void* kmax_t,
                           const void* k_c, const void* v_c, int B, int Hq, int Hkv, int Lc,
                           int D, int page_size, int r, int n_pages, float scale, int dtype,
                           int32_t* chan_idx, float* page_scores, int32_t* page_idx, void* out,
                           void* ws, size_t ws_bytes, void* stream);

/* The fused step's status word: *status (host memory) receives the bits set by calls on this
 * workspace since it was initialised or last cleared: 1 = a wait for page scores ran out of time,
 * 2 = a wait for attention partials ran out of time (either makes that call's output invalid);
 * informational, outputs valid: 16 = a block scored pages whose scoring block had not delivered
 * within the steal deadline, 32 = the same for an attention slice. (status & 15) == 0 means every
 * call's output is valid. clear != 0 zeroes the word after reading it. The read is enqueued on `stream` after the
 * work already there, and this call SYNCHRONISES the stream before returning. */
int rkv_hybrid_decode_status(void* ws, size_t ws_bytes, int clear, uint32_t* status, void* stream);

/* ------------------------------------------------------------------------------------------
 * rkv_hybrid_decode_step without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, limits, results and errors are those of rkv_hybrid_decode_step, except:
 *   - The workspace is the library's own scratch: a fixed RKV_NOALLOC_SCRATCH_BYTES (8 MiB) of
 *     device memory per GPU, part of the loaded library and held until the process ends. A shape
 *     whose rkv_hybrid_decode_workspace_bytes exceeds it is refused with RKV_ERR_SCRATCH before
 *     anything is enqueued (every shape with 128 < B*Hkv <= 256 fits, and so does any with
 *     B*Hkv <= 128 and B*Hkv*ceil(Lc/page_size) <= 2^19 pages, e.g. 8 heads of 16384-token
 *     caches at page 4; more than 256 heads need about B*Hkv*(8*ceil(Lc/page_size) +
 *     4*(Hq/Hkv)*(D+2)*s) bytes, s <= 8 attention splits, which 640 heads of 8192 pages exceed).
 *   - The call allocates and frees nothing. On its first call on a device it looks up that
 *     device's scratch address; whenever B*Hkv, Hq/Hkv, D, ceil(Lc/page_size) or dtype differ
 *     from the previous call's on the same device (and on the first call), it first enqueues a
 *     fill kernel that zeroes the part of the scratch the shape uses.
 *   - Every call on a GPU shares that GPU's scratch and leaves its counters there for the next
 *     call: calls that overlap in time on one GPU (other streams, other host threads) race and
 *     their results are undefined. Issue them in order on one stream, or synchronise between.
 *   - status: NULL, or DEVICE memory for one uint32: after the step the scratch's status word
 *     (bits as in rkv_hybrid_decode_status) is moved there and cleared. Bits 1 and 2 mark that
 *     call's output invalid; the counters stay consistent, so later calls are unaffected.
 * ------------------------------------------------------------------------------------------ */
#define RKV_NOALLOC_SCRATCH_BYTES (8u << 20)
int rkv_hybrid_decode_step_noalloc(const void* q, const void* kmin_t, const void* kmax_t,
                                   const void* k_c, const void* v_c, int B, int Hq, int Hkv,
                                   int Lc, int D, int page_size, int r, int n_pages, float scale,
                                   int dtype, int32_t* chan_idx, float* page_scores,
                                   int32_t* page_idx, void* out, uint32_t* status, void* stream);

/* ------------------------------------------------------------------------------------------
 * Decode-time append into a compressed cache that grows ([rebuttal] "SCBench Results": plain
 * SnapKV compresses only the prompt's KV, so generated tokens join the cache as decoding goes
 * on; "Explanation of Calculating Approximate Attention Scores": each page of consecutive
 * tokens keeps its element-wise minimum and maximum). The caches and summaries are laid out for
 * a fixed capacity of cap token slots per (b, h), of which the first Lc are valid:
 *
 * k_c, v_c       [B, Hkv, cap, D]           compressed keys and values
 * kmin_t, kmax_t [B, Hkv, D, Pcap]          channel-major summaries, Pcap = ceil(cap/page_size);
 *                                           page p holds the summary of slots [p*page_size,
 *                                           min((p+1)*page_size, Lc)) for p < ceil(Lc/page_size)
 *
 * rkv_build_page_summaries_cap: rkv_build_page_summaries over the first Lc slots of a cache of
 *   capacity cap (1 <= Lc <= cap); pages from ceil(Lc/page_size) on are not written.
 * rkv_kv_append: k_new, v_new [B, Hkv, D] go to slot Lc (0 <= Lc < cap), and k_new folds into
 *   page Lc/page_size: a slot at a page boundary starts the page (min = max = k_new), any other
 *   replaces the page's min (max) where k_new is strictly smaller (larger). The result is
 *   bit-identical to rkv_build_page_summaries_cap over Lc + 1 slots. The caller then uses Lc + 1.
 * rkv_hybrid_decode_step_cap: rkv_hybrid_decode_step over the first Lc slots (P =
 *   ceil(Lc/page_size) pages) of caches and summaries of capacity cap. Size its workspace with
 *   rkv_hybrid_decode_workspace_bytes(B, Hq, Hkv, cap, ...): the workspace is laid out for the
 *   capacity, so one workspace serves every Lc <= cap of that capacity (initialised once).
 * Requires the limits of the calls they extend, Pcap <= 8192 for the step, pointers to
 * 16-byte-aligned memory. Errors as everywhere: nothing is written when a call returns nonzero.
 * ------------------------------------------------------------------------------------------ */
int rkv_build_page_summaries_cap(const void* k_c, int B, int Hkv, int Lc, int cap, int D,
                                 int page_size, int dtype, void* kmin_t, void* kmax_t,
                                 void* stream);
int rkv_kv_append(const void* k_new, const void* v_new, int B, int Hkv, int Lc, int cap, int D,
                  int page_size, int dtype, void* k_c, void* v_c, void* kmin_t, void* kmax_t,
                  void* stream);
int rkv_hybrid_decode_step_cap(const void* q, const void* kmin_t, const void* kmax_t,
                               const void* k_c, const void* v_c, int B, int Hq, int Hkv, int Lc,
                               int cap, int D, int page_size, int r, int n_pages, float scale,
                               int dtype, int32_t* chan_idx, float* page_scores,
                               int32_t* page_idx, void* out, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------------------------
 * RocketKV-MT, the multi-turn variant ([rebuttal] "SCBench Results": SnapKV++ does not evict
 * permanently; every prompt token stays in memory, and each decode step selects only among the
 * tokens SnapKV++ kept). The compressed cache is a view: slot t of (b, h) is row
 * kept_idx[b,h,t] of the full cache.
 *
 * k, v      [B, Hkv, L, D]   the full caches
 * kept_idx  [B, Hkv, Lc]     int32 rows of the view, e.g. rkv_snapkvpp_evict's kept_idx with
 *                            k_out = v_out = NULL; values outside [0, L) are clamped into it
 * rkv_build_page_summaries_indexed: rkv_build_page_summaries of the view (kmin_t, kmax_t
 *   [B, Hkv, D, ceil(Lc/page_size)]); bit-identical to summarising the gathered rows.
 * rkv_hybrid_decode_step_indexed: rkv_hybrid_decode_step over the view; its workspace is
 *   rkv_hybrid_decode_workspace_bytes(B, Hq, Hkv, Lc, ...). Channels, scores, pages and outputs
 *   are bit-identical to rkv_hybrid_decode_step on the gathered caches.
 * Requires the limits of the calls they extend.
 * ------------------------------------------------------------------------------------------ */
int rkv_build_page_summaries_indexed(const void* k, const int32_t* kept_idx, int B, int Hkv,
                                     int L, int Lc, int D, int page_size, int dtype, void* kmin_t,
                                     void* kmax_t, void* stream);
int rkv_hybrid_decode_step_indexed(const void* q, const void* kmin_t, const void* kmax_t,
                                   const void* k, const void* v, const int32_t* kept_idx, int B,
                                   int Hq, int Hkv, int L, int Lc, int D, int page_size, int r,
                                   int n_pages, float scale, int dtype, int32_t* chan_idx,
                                   float* page_scores, int32_t* page_idx, void* out, void* ws,
                                   size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RKV_H */
