/*
 * dash.h -- C ABI of the DashAttention forward library for AMD Instinct MI355X
 * (gfx950).
 *
 * The method ("DashAttention: Differentiable and Adaptive Sparse Hierarchical
 * Attention", explainer pages for arXiv 2605.18753, section "Technical
 * summary") computes attention in three stages:
 *   Stage 0  summaries of contiguous key blocks (chunks of block_size keys);
 *   Stage 1  coarse scores of each query against the summaries and
 *            w = alpha-entmax(gamma * zbar), a sparse probability vector over
 *            blocks whose support size follows the scores; GQA query heads
 *            that share a KV head average their probabilities;
 *   Stage 2  softmax attention restricted to the routed blocks, with the
 *            routing probability as a prior (added as a log bias before the
 *            softmax); blocks of probability 0 are masked; the block holding
 *            the query (near the diagonal, no summary yet) is handled apart.
 * The pages state one fused kernel per stage, with prefill and incremental
 * decoding ("Technical summary", Contributions, efficient GPU implementation).
 *
 * Fixed readings (the pages leave them open):
 *   - summary s_j = (mean of block j's keys) . W_s, W_s a d x d float32 matrix,
 *     row-major [d_in][d_out], shared by all heads;
 *   - zbar_j = q . s_j / sqrt(d); entmax input x_j = (alpha - 1) gamma zbar_j;
 *     p_j = [x_j - tau]_+^(1/(alpha-1)) with sum_j p_j = 1 (Tsallis entmax);
 *   - causal attention: the routing candidates of a query at position i are
 *     the complete blocks j < floor(i / block_size); the query's own block is
 *     always attended (keys t <= i) with bias 0; a routed block adds
 *     log pbar_j to q.k/sqrt(d); pbar is the mean of p over the heads of a
 *     GQA group.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers unless stated, 16-byte aligned
 *     (DASH_ERR_INVALID_ARG otherwise); tensors are dense row-major with the
 *     shapes given.  q, o: [B, H, n, d]; k, v:
 *     [B, Hkv, kv_len, d] (one block of one head is a contiguous run).  Query
 *     head h reads KV head h / (H / Hkv).
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  The library never allocates, frees or synchronises; the
 *     caller owns every buffer, including workspaces.  Calls are re-entrant
 *     across streams; concurrent calls must not share output buffers.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is launched and the status says why.  A failed launch is
 *     reported as DASH_ERR_HIP; faults during execution surface at the
 *     caller's next synchronisation.  Device data is never inspected: NaN and
 *     Inf propagate.
 *   - Results are bitwise reproducible for fixed inputs and launch shapes
 *     (no floating-point atomics).
 */
#ifndef DASH_H_
#define DASH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARG = 1,        /* null pointer, negative size, bad shape */
  DASH_ERR_UNSUPPORTED = 2,        /* valid but not built (head_dim, block_size, ...) */
  DASH_ERR_WORKSPACE_TOO_SMALL = 3,
  DASH_ERR_HIP = 4                 /* a HIP runtime call or launch failed */
} dash_status;

typedef enum { DASH_F32 = 0, DASH_BF16 = 1 } dash_dtype;

/* Problem description shared by every call.
 *   batch       B >= 1 sequences
 *   n_heads     H query heads; n_kv_heads Hkv divides H; G = H / Hkv must be
 *               1, 2, 4 or 8
 *   head_dim    d: 64 or 128
 *   block_size  key block ("chunk") size: 64 or 128
 *   alpha       entmax exponent, 1 < alpha <= 2
 *   gamma       routing scale, finite and > 0
 *   dtype       element type of q, k, v and o (DASH_F32 or DASH_BF16); the
 *               summaries and W_s are always float32
 *   sigma       prior strength (Stage 2, "prior-induced sparse softmax"): the
 *               bias of a routed block is sigma * log pbar, i.e. the reference
 *               distribution is proportional to pbar^sigma on the support;
 *               finite and >= 0; 1 = the routing distribution itself, 0 = only
 *               its support (a mask)
 *   window      near-diagonal branch in blocks, >= 1: the query's own block and
 *               the window - 1 blocks before it are attended token-causally
 *               with bias 0 and are never routed; routing candidates are the
 *               complete blocks j < own - (window - 1) */
typedef struct {
  int32_t batch;
  int32_t n_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  float alpha;
  float gamma;
  int32_t dtype;
  float sigma;
  int32_t window;
} dash_params;

/* Query tile of the prefill path: 64 consecutive positions of one sequence
 * and one KV head (all G query heads of the group).  The routing result is
 * stored per tile: the union of the tile's selected blocks and, for each
 * selected block, the prior bias of every position of the tile. */
#define DASH_QUERY_TILE 64

/* Storage of the routing result (Stage 1 -> Stage 2 hand-over), caller-owned.
 * For prefill over n positions: n_qt = ceil(n / 64) tiles, nb = ceil(n / bs)
 * blocks, QT = 64.  For decode (one query per sequence): n = 1, n_qt = 1,
 * QT = 1, nb = ceil(max_len / bs).
 *   tau          [B, H, n]            float; entmax threshold per (head, query),
 *                                     NaN for queries without a candidate block
 *   sel_count    [B, Hkv, n_qt]       int32; number of selected blocks
 *   sel_idx      [B, Hkv, n_qt, nb]   int32; ascending selected block ids,
 *                                     the first sel_count entries are valid
 *   sel_logp     [B, Hkv, n_qt, nb, QT] float; the Stage 2 bias
 *                                     sigma * log pbar(block, query) indexed by
 *                                     BLOCK ID, -inf where pbar = 0; valid for
 *                                     the candidate blocks of the tile
 *   support_bits [B, H, n, ceil(nb/32)] uint32, optional (NULL = not written);
 *                                     bit j set iff block j is in that head's own
 *                                     entmax support (x_j > tau), before the GQA
 *                                     average
 *   tile_bits    [B, Hkv, n_qt, ceil(nb/32)] uint32, optional (NULL = not
 *                                     written); the bit-packed mask of active
 *                                     chunks handed to Stage 2: bit j (word j/32,
 *                                     bit j%32) set iff block j is in the tile's
 *                                     list, every other bit 0 */
typedef struct {
  float* tau;
  int32_t* sel_count;
  int32_t* sel_idx;
  float* sel_logp;
  uint32_t* support_bits;
  uint32_t* tile_bits;
} dash_route_buf;

/* Element counts of each dash_route_buf array (not bytes). */
typedef struct {
  int64_t n_qt, nb, qt;
  int64_t tau, sel_count, sel_idx, sel_logp, support_bits, tile_bits;
} dash_route_sizes;

const char* dash_status_string(dash_status s);

/* Library version string, e.g. "dash-mi355x 0.1.0 gfx950". */
const char* dash_version(void);

/* Sizes of the prefill routing buffers for n query positions. */
dash_status dash_route_sizes_prefill(const dash_params* p, int64_t n, dash_route_sizes* out);

/* Sizes of the decode routing buffers for caches of max_len tokens. */
dash_status dash_route_sizes_decode(const dash_params* p, int64_t max_len, dash_route_sizes* out);

/* Workspace bytes needed by dash_prefill (n positions) and dash_decode
 * (caches of max_len tokens).  The workspace must be 256-byte aligned. */
dash_status dash_prefill_workspace_bytes(const dash_params* p, int64_t n, size_t* bytes);
dash_status dash_decode_workspace_bytes(const dash_params* p, int64_t max_len, size_t* bytes);

/* Stage 0 ("local chunk summarization", DashAttention explainer, Technical
 * summary; summaries are computed once a chunk is complete and then cached).
 * For every sequence b, KV head g and block j in [blk_begin, blk_end), with
 * K = k[b, g, j*bs:(j+1)*bs, :]:
 *   q_bar NULL    summ[b, g, j, :] = mean_t(K[t]) . w_s
 *   q_bar given   summ[b, g, j, :] = (sum_t a_t K[t]) . w_s,
 *                 a = softmax_t(q_bar[g] . K[t] / sqrt(d))
 * (the learned summary query attending to the chunk's keys by local scaled
 * dot-product attention; a zero query is the mean), accumulated in float32.
 *   k      [B, Hkv, kv_len, d] dtype; (blk_end * bs) <= kv_len
 *   w_s    [d, d] float32
 *   q_bar  NULL or [Hkv, d] float32 summary queries
 *   summ   [B, Hkv, summ_blocks, d] float32, blk_end <= summ_blocks
 * Blocks outside [blk_begin, blk_end) are left untouched. */
dash_status dash_summarize(const dash_params* p, const void* k, int64_t kv_len, int64_t blk_begin,
                           int64_t blk_end, const float* w_s, const float* q_bar, float* summ,
                           int64_t summ_blocks, void* stream);

/* Stage 1 for causal prefill of positions 0..n-1: coarse scores, alpha-entmax
 * per (query, head), GQA average, per-tile union and compaction.
 *   q      [B, H, n, d] dtype
 *   summ   [B, Hkv, summ_blocks, d] float32 holding blocks 0 .. floor(n/bs)-1
 *   route  buffers sized by dash_route_sizes_prefill(p, n) */
dash_status dash_route(const dash_params* p, const void* q, int64_t n, const float* summ,
                       int64_t summ_blocks, const dash_route_buf* route, void* stream);

/* Stage 2 for causal prefill: for each query, softmax over the keys of its
 * tile's selected blocks (logit q.k/sqrt(d) + sel_logp, -inf masks) and the
 * keys t <= i of its own block (bias 0); o = weights . v.
 *   q, o   [B, H, n, d] dtype;  k, v [B, Hkv, n, d] dtype
 *   route  as written by dash_route (tau and support_bits are not read)
 * DASH_ERR_UNSUPPORTED when one (sequence, KV head)'s keys span 2 GiB or more
 * ((n + 64) * d * element size >= 2^31). */
dash_status dash_attend(const dash_params* p, const void* q, const void* k, const void* v,
                        int64_t n, const dash_route_buf* route, void* o, void* stream);

/* Bit-packed mask -> Stage 2 lists, for prefill (the DashAttention explainer,
 * Technical summary, Stage 2: the attention kernel walks the active chunks
 * that a bit-packed mask defines).  For every tile, the set bits of
 * route->tile_bits that fall on the tile's routing candidates (blocks
 * j < floor(64 qt / bs) - (window - 1)) become sel_idx (ascending) and
 * sel_count; bits on any other block are ignored.  dash_attend then runs on
 * route, with sel_logp (the bias of each listed block, -inf to mask a
 * position) supplied by the caller.
 *   route  tile_bits (read), sel_count and sel_idx (written); sized by
 *          dash_route_sizes_prefill(p, n) */
dash_status dash_mask_to_list(const dash_params* p, int64_t n, const dash_route_buf* route,
                              void* stream);

/* Fused causal prefill: dash_summarize of blocks [0, floor(n/bs)) into summ
 * (with the summary queries q_bar, NULL = mean pooling), dash_route into the
 * workspace, dash_attend into o.
 *   summ   [B, Hkv, summ_blocks, d] float32, summ_blocks >= floor(n/bs)
 *   q_bar  NULL or [Hkv, d] float32 summary queries
 *   ws     >= dash_prefill_workspace_bytes(p, n) bytes, 256-byte aligned
 * Same size limit as dash_attend. */
dash_status dash_prefill(const dash_params* p, const void* q, const void* k, const void* v,
                         int64_t n, const float* w_s, const float* q_bar, float* summ,
                         int64_t summ_blocks, void* o, void* ws, size_t ws_bytes, void* stream);

/* dash_prefill for a batch of sequences of different lengths (a ragged
 * batch): sequence b has seq_lens[b] positions, stored in the first rows of
 * its n_max-row slices,
 *   q, o   [B, H, n_max, d] dtype;  k, v [B, Hkv, n_max, d] dtype
 *   seq_lens [B] int32 DEVICE array, values clamped into [0, n_max]
 * Every sequence is computed exactly as dash_prefill would compute it alone
 * (its complete blocks summarised into summ, routing and attention over its
 * own positions); rows at or past seq_lens[b] of o and summaries of blocks
 * past its last complete block are not written.  Query tiles past a
 * sequence's end exit at once, so the work follows the real lengths.
 * Workspace and limits as dash_prefill with n = n_max. */
dash_status dash_prefill_varlen(const dash_params* p, const void* q, const void* k, const void* v,
                                int64_t n_max, const int32_t* seq_lens, const float* w_s,
                                const float* q_bar, float* summ, int64_t summ_blocks, void* o,
                                void* ws, size_t ws_bytes, void* stream);

/* Backward pass of the causal prefill (the pages stress that alpha-entmax
 * keeps the hierarchy differentiable: gradients flow from the attention
 * output back through the routing into the chunk summaries).  For mean-pooled
 * summaries (no summary query), given the forward's inputs, its output o, its
 * summaries and routing result, and dO = dL/do:
 *   q, o, d_o  [B, H, n, d] dtype;  k, v [B, Hkv, n, d] dtype
 *   summ       [B, Hkv, summ_blocks, d] float32 as dash_summarize wrote it
 *   route      as dash_route wrote it for these inputs (tau, sel_count,
 *              sel_idx, sel_logp)
 *   dq         [B, H, n, d] float32;  dk, dv [B, Hkv, n, d] float32;
 *   dw_s       [d, d] float32 -- all written (not accumulated)
 *   ws         >= dash_prefill_backward_workspace_bytes(p, n), 256-byte aligned
 * The gradient reaches q through both the fine attention and the coarse
 * scores, k through the attention and the block means, and W_s through the
 * summaries.  Blocks with pbar = 0 take no gradient.  Accumulation in float32
 * (bf16 inputs: the attention products on bf16 MFMA), every sum in a fixed
 * order (bitwise reproducible, like the forward).  The per-query-tile arrays
 * of the workspace hold one slab of tiles at a time, sized so that they stay
 * within about 1 GiB; the rest grows as n.  DASH_ERR_UNSUPPORTED under the
 * same 2 GiB per-(sequence, KV head) limit as dash_attend. */
dash_status dash_prefill_backward_workspace_bytes(const dash_params* p, int64_t n,
                                                  size_t* bytes);
dash_status dash_prefill_backward(const dash_params* p, const void* q, const void* k,
                                  const void* v, const void* o, const void* d_o, int64_t n,
                                  const float* w_s, const float* summ, int64_t summ_blocks,
                                  const dash_route_buf* route, float* dq, float* dk, float* dv,
                                  float* dw_s, void* ws, size_t ws_bytes, void* stream);

/* One incremental decoding step for every sequence b: the query q[b] sits at
 * position L = cache_len[b] - 1 and its key/value are already in the caches.
 * Routes over the cached summaries of blocks j < floor(L / bs), attends to the
 * selected blocks plus keys [floor(L/bs)*bs, L] of the own block, and, when
 * cache_len[b] % bs == 0 (the step completes a block), writes the summary of
 * block cache_len[b]/bs - 1 into summ (as dash_summarize with q_bar).
 *   q, o            [B, H, d] dtype
 *   k_cache, v_cache [B, Hkv, max_len, d] dtype
 *   cache_len       [B] int32 DEVICE array, 1 <= cache_len[b] <= max_len
 *   q_bar           NULL or [Hkv, d] float32 summary queries
 *   summ            [B, Hkv, summ_blocks, d] float32, summ_blocks >= ceil(max_len/bs),
 *                   read for blocks < floor((cache_len-1)/bs), written as above
 *   route           optional (NULL = use the workspace): where the routing
 *                   result goes, sized by dash_route_sizes_decode
 *   ws              >= dash_decode_workspace_bytes(p, max_len) bytes
 * Values of cache_len outside [1, max_len] are clamped into that range.
 * DASH_ERR_UNSUPPORTED when (max_len + 64) * d * element size >= 2^31, when
 * (H / Hkv) * ceil(max_len / block_size) * 4 bytes (one routing
 * workgroup's LDS) exceed 160 KiB, when B * Hkv > 65535, or for bf16 when
 * B * Hkv > 8192. */
dash_status dash_decode(const dash_params* p, const void* q, const void* k_cache,
                        const void* v_cache, const int32_t* cache_len, int64_t max_len,
                        const float* w_s, const float* q_bar, float* summ, int64_t summ_blocks,
                        void* o, const dash_route_buf* route, void* ws, size_t ws_bytes,
                        void* stream);

/* dash_decode over a paged KV cache (serving layout; DashAttention explainer,
 * Contributions: the kernels support incremental decoding).  One page holds
 * one block of bs keys of every KV head:
 *   k_pages, v_pages [num_pages, Hkv, bs, d] dtype
 *   block_table      [B, max_blocks] int32 DEVICE array: block j of sequence b
 *                    (j < ceil(cache_len[b] / bs)) is in page block_table[b, j];
 *                    max_blocks >= ceil(max_len / bs)
 * Every other argument, the result and the summary written for a completed
 * block are as in dash_decode (the summaries stay per sequence,
 * [B, Hkv, summ_blocks, d]).  Page ids outside [0, num_pages) are clamped into
 * that range: a bad table gives wrong results but no access outside the
 * pages.  No 2 GiB limit on the cache. */
dash_status dash_decode_paged(const dash_params* p, const void* q, const void* k_pages,
                              const void* v_pages, int64_t num_pages, const int32_t* block_table,
                              int64_t max_blocks, const int32_t* cache_len, int64_t max_len,
                              const float* w_s, const float* q_bar, float* summ,
                              int64_t summ_blocks, void* o, const dash_route_buf* route,
                              void* ws, size_t ws_bytes, void* stream);

/* dash_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same step, kernels and result as dash_decode (bitwise), but the workspace
 * is the library's own static device scratch, 32 MiB per GPU, held until the
 * process ends; nothing is allocated or freed.  DASH_ERR_WORKSPACE_TOO_SMALL
 * (nothing launched) when dash_decode_workspace_bytes(p, max_len) exceeds
 * 32 MiB, which covers e.g. 32 sequences x 32K and 8 x 128K with 64 query
 * heads.  The first call on a device looks up that device's scratch address
 * (once per device, with the device current).  Every call on one GPU shares
 * its scratch: calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller.  The scratch keeps the last call's
 * contents; no part of it needs to start at zero. */
dash_status dash_decode_noalloc(const dash_params* p, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* cache_len, int64_t max_len,
                                const float* w_s, const float* q_bar, float* summ,
                                int64_t summ_blocks, void* o, const dash_route_buf* route,
                                void* stream);

/* ---- Measurement helpers (not part of the attention computation) ---------
 * What this GPU attains, in the same process, for stating each kernel's
 * roofline fraction against a measured ceiling beside the nominal one.
 *
 * dash_peak_stream: one grid-stride pass of 16-byte loads over `bytes` bytes
 * of src (a multiple of 16, both pointers 16-byte aligned).  mode 0 copies
 * them to dst (dst holds `bytes` bytes); modes 1 and 2 only read them and
 * store one 16-byte value per thread, so dst must hold
 * 16 * dash_peak_stream_grid() bytes.  Mode 1 loads allocate in the caches
 * (a read of more than their size empties them); mode 2 loads use the
 * non-temporal policy of the decode step's K/V loads.  Other modes return
 * DASH_ERR_INVALID_ARG.  dash_peak_mfma: every wave of a chip-filling grid runs `iters`
 * rounds of eight independent v_mfma_f32_32x32x16_bf16 on register operands
 * (no memory traffic in the loop); *flops receives the flop count of the
 * launch (host pointer), sink (device) one float per wave, sized by
 * dash_peak_mfma_grid(). */
dash_status dash_peak_stream_grid(int64_t* threads);
dash_status dash_peak_stream(const void* src, void* dst, int64_t bytes, int32_t mode,
                             void* stream);
dash_status dash_peak_mfma_grid(int64_t* waves);
dash_status dash_peak_mfma(int64_t iters, float* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H_ */
