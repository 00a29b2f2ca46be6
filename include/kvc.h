/*
 * kvc.h -- C ABI of the MI355X (gfx950) KV-cache compression hot path.
 *
 * Four steps shared by observation-window KV eviction (SnapKV-style), FastKV's
 * token-selective propagation and per-step KV retrieval (FreeKV):
 *
 *   kvc_score_window    saliency of every cached token from the attention of the
 *                       last w queries, summed over the window and over the query
 *                       heads of each GQA group, then max-pooled in 1-D
 *   kvc_select_topk     per-KV-head top-k under a retention budget, plus the
 *                       trailing window, lower index first on equal scores
 *   kvc_select_core     the same with role-based retention: core tokens always
 *                       kept, the budget over the scratch tokens (CASK)
 *   kvc_gather_compact  copy of the kept rows into a compacted cache that keeps
 *                       the original positions
 *   kvc_decode_attn     GQA decode attention of one query per head over the
 *                       compacted cache
 *   kvc_block_landmarks, kvc_block_scores, kvc_expand_blocks
 *                       landmark-guided block selection (xKV, ShadowKV-style):
 *                       block means of K, the group's logit per block, kept blocks
 *                       back to token indices (the block top-k is kvc_select_topk)
 *   kvc_query_similarity  cosine of the queries of two adjacent decode steps and
 *                       the KV heads whose selection is redone before attention
 *                       (speculative retrieval with fine-grained correction)
 *
 * Pages these calls follow (cited by title and section):
 *   [FastKV]   "FastKV: Decoupling of Context Reduction and KV Cache Compression for
 *              Prefill-Decoding Acceleration", section 2.A (saliency from the recent
 *              window's attention; the selected tokens and the sliding-window tokens
 *              propagate) and section 2.B (TSP rate and KV retention rate are two
 *              independent budgets).
 *   [Tutorial] "Variantes de l'attention et compression du cache KV", sections
 *              "MHA et GQA" (L, S, n_h, n_kv, d_h, b; query heads sharing a KV head),
 *              "Quand la reutilisation est-elle exacte ?" (causal alignment of rows
 *              appended after S cached tokens; keep original positions after
 *              eviction) and "Compresser un cache existant" (observation-window
 *              scoring, keep a subset of past keys and values).
 *   [xKV]      "xKV: Compression de Cache KV Inter-couche par Extraction de Vecteurs
 *              Singuliers Alignes", section 2.3 (Reconstruction Selective: a sparse
 *              subset of tokens found by landmark-guided block selection, as in
 *              ShadowKV; the low-rank reconstruction itself is not part of this path).
 *   [FreeKV]   "FreeKV: Boosting KV Cache Retrieval for Efficient LLM Inference",
 *              technical summary section 2.A (select a subset with the current
 *              query, then attend over it, at every decode step; speculative
 *              retrieval reuses the previous step's subset and fine-grained
 *              correction redoes the selection of the heads whose query drifted).
 *
 * Conventions for every call:
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The library
 *     allocates no memory; scratch space is the caller's `ws` buffer, sized by the
 *     matching *_workspace() query.  Where a call says so, its workspace must be
 *     zero-filled once before first use (hipMemset, torch.zeros): every call that
 *     completes leaves the parts it uses as counters and accumulators zero again,
 *     so the workspace may be reused between calls of the same kind that are
 *     ordered on one stream, under the shape rule stated with the call.  Such a
 *     workspace written by anything else, used under another shape, or whose last
 *     call did not complete, must be zero-filled again.  Other workspaces are
 *     scratch: any contents will do.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL is the
 *     default stream).  Nothing blocks the host.  Calls sharing a workspace must
 *     be ordered on one stream.
 *   - Layouts are head-major, contiguous, row-major, exactly as written below.
 *     bf16 means the 16-bit bfloat format stored as uint16 bit patterns.
 *   - Every precondition that the host can check is checked before any HIP call;
 *     on failure the call returns KVC_ERR_INVALID_ARG, KVC_ERR_UNSUPPORTED or
 *     KVC_ERR_WORKSPACE and launches nothing.  A failed launch returns KVC_ERR_HIP.
 *   - Device-resident sequence lengths are a caller contract: kernels clamp each
 *     to [0, s_max].
 *   - No C++ exception crosses this interface.  The library keeps no state
 *     between calls apart from a cache of device attributes.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 4

typedef enum kvc_status {
    KVC_OK = 0,
    KVC_ERR_INVALID_ARG = 1,  /* a null pointer, a size out of range, inconsistent shapes */
    KVC_ERR_UNSUPPORTED = 2,  /* a valid shape or dtype this build has no kernel for      */
    KVC_ERR_WORKSPACE = 3,    /* ws is NULL or smaller than the *_workspace() size         */
    KVC_ERR_HIP = 4           /* the HIP runtime reported an error (no device, launch)    */
} kvc_status;

typedef enum kvc_dtype {
    KVC_F32 = 0,              /* 4-byte IEEE float                                        */
    KVC_BF16 = 1              /* 2-byte bfloat16 (uint16 bit patterns), fp32 arithmetic   */
} kvc_dtype;

/*
 * Problem dimensions (Tutorial, "MHA et GQA": S cached tokens, n_h query heads,
 * n_kv KV heads, head width d_h, b bytes per element).  Layers are not a
 * dimension: call once per layer, or fold independent layers into `batch`.
 */
typedef struct kvc_dims {
    int32_t batch;            /* B >= 1 sequences (or sequence-layer pairs)                 */
    int32_t s_max;            /* S >= 1: token capacity, the leading token dim of K/V/scores */
    const int32_t *seq_lens;  /* device int32[B] cached lengths S_b; NULL: every S_b = s_max */
    int32_t n_h;              /* query heads, a multiple of n_kv                             */
    int32_t n_kv;             /* KV heads; query head h reads KV head h / (n_h / n_kv)       */
    int32_t d_h;              /* head width: 64 or 128                                       */
    int32_t dtype;            /* kvc_dtype of Q, K, V and the decode output                  */
    const int32_t *unit_mask; /* device int32[B][n_kv] or NULL (every unit).  kvc_score_window
                                 and kvc_select_topk skip unit (b, g) when its entry is 0 and
                                 leave its outputs as they were (FreeKV 2.A: selection runs
                                 again only for the heads that need correction); not allowed
                                 with KVC_SELECT_SHARED_HEADS; kvc_decode_attn ignores it     */
} kvc_dims;

/* kvc_select_topk flag: one selection per sequence from the sum of the pooled
 * scores over all KV heads, added in double and rounded to float (FastKV 2.A: the tokens
 * chosen at the propagation layer are the same for every head). */
#define KVC_SELECT_SHARED_HEADS 1

/* kvc_score_window flag: use the portable VALU kernels (any R, d_h, dtype) instead
 * of the bf16 MFMA kernels.  Results agree to the same tolerance; meant for tests. */
#define KVC_SCORE_GENERIC 1
/* kvc_score_window flag, for tests: the single-pass kernel does not wait for the row
 * statistics of any KV head and leaves every item to its follow-up kernel (the path
 * an item takes when its bounded wait runs out).  Results are identical. */
#define KVC_SCORE_DEFER_ALL 2

int32_t kvc_abi_version(void);
const char *kvc_status_str(kvc_status status);

/*
 * kvc_score_window -- observation-window saliency (FastKV 2.A; Tutorial,
 * "Compresser un cache existant"), R = (n_h/n_kv) * w rows per KV head.
 *
 * For sequence b and KV head g, with r = n_h/n_kv, every query head h in
 * [g*r, g*r + r) and every window row i < w:
 *   x[h,i,t] = scale * <q_win[b][h][i], k[b][g][t]>            for visible t < S_b
 *   raw[b][g][t] = sum over (h, i) of exp(x[h,i,t] - M[h,i]) / L[h,i]
 * with M, L the max and the sum of exp(x - M) over the visible t of that row.
 * Visibility (Tutorial, "Quand la reutilisation est-elle exacte ?"): when
 * window_in_cache != 0 the window rows are the last w cached tokens, so row i sees
 * t <= S_b - w + i; otherwise (a new query that is not in the cache) every
 * t < S_b is visible.  A row that sees no key adds nothing.
 * Pooling over the candidate region C = [0, max(0, S_b - n_keep)):
 *   pooled[b][g][t] = max of raw[b][g][u] over u in [t - p/2, t + p/2] intersect C, t in C
 *   pooled[b][g][t] = raw[b][g][t] for t in [max(0, S_b - n_keep), S_b)
 *   raw and pooled are 0 for t in [S_b, s_max).
 *
 * q_win      [B][n_h][w][d_h] dtype      window queries
 * k          [B][n_kv][s_max][d_h] dtype  keys
 * w          1 <= w <= 1024, and (n_h/n_kv)*w <= 1024; s_max <= 2^22 (else
 *            KVC_ERR_UNSUPPORTED)
 * pool_kernel odd, 1 <= p <= 63 (1: no pooling)
 * scale      > 0; 0 means 1/sqrt(d_h)
 * raw        [B][n_kv][s_max] float, written (required)
 * pooled     [B][n_kv][s_max] float, written (required)
 * flags      0, or KVC_SCORE_GENERIC and/or KVC_SCORE_DEFER_ALL
 * ws         at least kvc_score_window_workspace(dims, w, flags) bytes, 16-byte
 *            aligned, zero-filled before first use: per-item row statistics, per-KV-head
 *            arrival counters and, for the single-pass kernel, a deferred-item count
 *            (returned to zero by each call that completes) and a call tag (advanced
 *            by each call; the final row statistics carry it); calls with the same
 *            dims (seq_lens and unit_mask aside), w and flags may share one workspace
 *            without zero-filling it again
 * Arithmetic: fp32 logits (bf16 products are exact), fp32 exp2-based softmax with
 * the row sums accumulated per lane and merged in double; raw agrees with a
 * double-precision evaluation to about 1e-6 relative.  Probabilities below the
 * fp32 normal range are flushed to zero.
 */
size_t kvc_score_window_workspace(const kvc_dims *dims, int32_t w, int32_t flags);
kvc_status kvc_score_window(const kvc_dims *dims, const void *q_win, const void *k, int32_t w,
                            int32_t window_in_cache, int32_t n_keep, int32_t pool_kernel,
                            float scale, float *raw, float *pooled, int32_t flags,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * kvc_score_window_plan -- the launch configuration kvc_score_window takes for these
 * arguments (it depends on the shapes only), for tests and profiling:
 *   out[0]  1 when the bf16 MFMA kernels run, 0 for the portable kernels
 *   out[1]  MFMA path: blocks of 16 window rows per KV head (1, 2, 4 or 8), else 0
 *   out[2]  MFMA path: tokens per work-group item, else 0
 *   out[3]  MFMA path: work-group items per KV head, else 0
 *   out[4]  1 when K is read in a single pass (16 < R <= 32, s_max <= 131072: the row
 *           statistics are exchanged between the work-groups of a resident grid), 0
 *           for the two-pass kernels, which a device that cannot hold one work-group
 *           per 1024-token item of a KV head at once also takes.  Work-groups that
 *           wait too long for the statistics (two such calls running at the same time
 *           on other streams, for instance) leave their items to a follow-up kernel
 *           that re-reads their K: slower, same results
 *   out[5]  1 when the two-pass kernels merge the row statistics of a KV head's items
 *           in the last of its first-pass work-groups to finish (at most 8 items per KV
 *           head, all work-groups resident at once), 0 when a kernel of its own merges
 *           them (or for the single-pass and portable kernels)
 * out  int32[6], host memory.  Same argument checks as kvc_score_window_workspace.
 */
kvc_status kvc_score_window_plan(const kvc_dims *dims, int32_t w, int32_t flags, int32_t *out);

/*
 * kvc_select_topk -- per-KV-head selection under the retention budget (FastKV 2.B),
 * plus the always-kept trailing tokens (FastKV 2.A), in ascending original order.
 *
 * For each unit (b, g) (or b alone with KVC_SELECT_SHARED_HEADS, score = the sum
 * over g, in double, rounded to float), with C = max(0, S_b - n_keep) candidates [0, C) and the
 * unit's budget k_u = k, or k_per_unit[u] clamped to [0, k] (PyramidKV-style budgets
 * that differ per layer or head: Tutorial, "Compresser un cache existant"):
 *   k_eff = min(k_u, C); the first k_eff candidates in the total order
 *   (score descending, index ascending) are selected;
 *   idx[0 .. k_eff) = those indices ascending; idx[k_eff ..) = C, C+1, ..., S_b - 1;
 *   count = k_eff + (S_b - C); idx entries past count are -1.
 *
 * scores [B][n_kv][s_max] float (the pooled output of kvc_score_window); must not
 *        hold NaN; -0.0 and +0.0 are equal
 * k, n_keep  >= 0, cap = k + n_keep >= 1 (k: the largest budget)
 * k_per_unit  [B][H] int32 or NULL (every unit takes k)
 * idx    [B][H][k + n_keep] int32, H = n_kv, or 1 with KVC_SELECT_SHARED_HEADS
 * count  [B][H] int32
 * ws     at least kvc_select_topk_workspace(dims, k, n_keep, flags) bytes, 16-byte
 *        aligned, zero-filled before first use: per-unit radix histograms and a
 *        completion counter (returned to zero by each call), per-chunk counts (and
 *        the head sum when shared); the size depends on batch, n_kv, s_max, n_keep
 *        and flags.  Calls with the same batch, n_kv and flags may share one
 *        workspace without zero-filling it again (s_max, n_keep, k and seq_lens may
 *        differ if it is large enough for each)
 * The result is unique (ties are ordered by index) and bit-reproducible.
 */
size_t kvc_select_topk_workspace(const kvc_dims *dims, int32_t k, int32_t n_keep, int32_t flags);
kvc_status kvc_select_topk(const kvc_dims *dims, const float *scores, int32_t k, int32_t n_keep,
                           int32_t flags, const int32_t *k_per_unit, int32_t *idx, int32_t *count,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * kvc_select_core -- role-based retention (CASK: "Core" tokens, which carry the
 * reasoning state, are always kept; "Scratch" tokens are the target of compression):
 * the budget k applies to the scratch tokens only.
 *
 * For each unit (b, g), with C = max(0, S_b - n_keep), Core = {t < C : core[b][t] != 0},
 * Scratch = [0, C) minus Core:
 *   k_eff = min(k, |Scratch|); Sel = the first k_eff scratch tokens in the order
 *   (score descending, index ascending);
 *   idx = ascending(Sel u Core), then C, C+1, ..., S_b - 1; -1 padded
 *   count = k_eff + |Core| + (S_b - C)
 * |Core| <= core_cap is the caller's contract; a unit with more core candidates keeps
 * the k + core_cap lowest-indexed of them and no scratch token.
 *
 * scores  [B][n_kv][s_max] float, finite (the pooled output of kvc_score_window)
 * core    [B][s_max] uint8 role of each token, shared by the heads of a sequence
 * k, core_cap, n_keep >= 0, k + core_cap + n_keep >= 1
 * idx     [B][n_kv][k + core_cap + n_keep] int32; count [B][n_kv] int32
 * dims->unit_mask is honoured as in kvc_select_topk
 * ws      at least kvc_select_core_workspace(dims, n_keep) bytes, 16-byte aligned,
 *         zero-filled before first use; its first part is a kvc_select_topk workspace
 *         (same reuse rule: calls with the same batch and n_kv), then scratch
 */
size_t kvc_select_core_workspace(const kvc_dims *dims, int32_t n_keep);
kvc_status kvc_select_core(const kvc_dims *dims, const float *scores, const uint8_t *core, int32_t k,
                           int32_t core_cap, int32_t n_keep, int32_t *idx, int32_t *count,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * kvc_gather_compact -- compacted cache that keeps original positions (Tutorial,
 * "Quand la reutilisation est-elle exacte ?"; FreeKV 2.B on keeping the GPU copy in
 * one layout).  A byte copy: any row type works.
 *
 * For unit u = (b, h), h < heads, and j < count[b][h'] (clamped to [0, cap]):
 *   dst0[b][h][j] = src0[b][h][idx[b][h'][j]]    (row_bytes bytes)
 *   dst1[b][h][j] = src1[b][h][idx[b][h'][j]]    (when src1/dst1 are given)
 *   pos_out[b][h][j] = src_pos[b][idx[b][h'][j]]  (idx itself when src_pos is NULL)
 * where h' = h when idx_heads == heads and h' = 0 when idx_heads == 1 (one list
 * shared by every head).  Rows j >= count are not written; their pos_out is -1.
 * An index outside [0, s_max) copies nothing and gets pos_out -1.  With unit_mask,
 * a list whose entry is 0 is skipped: its dst rows and pos_out are left as they were.
 *
 * src0, src1   [B][heads][s_max][row_bytes]; src1 may be NULL (then dst1 must be NULL)
 * src_pos      [B][s_max] int32 or NULL
 * idx          [B][idx_heads][cap] int32; count [B][idx_heads] int32
 * dst0, dst1   [B][heads][cap][row_bytes]
 * pos_out      [B][heads][cap] int32 or NULL
 * unit_mask    [B][idx_heads] int32 or NULL (every list is copied)
 * row_bytes    a multiple of 16; row_bytes/16 a power of two or a multiple of 256;
 *              every row pointer 16-byte aligned
 */
kvc_status kvc_gather_compact(int32_t batch, int32_t heads, int32_t s_max, int32_t row_bytes,
                              const void *src0, const void *src1, const int32_t *src_pos,
                              const int32_t *idx, const int32_t *count, int32_t idx_heads,
                              int32_t cap, void *dst0, void *dst1, int32_t *pos_out,
                              const int32_t *unit_mask, void *stream);

/*
 * kvc_decode_attn -- GQA decode attention over the compacted cache (FreeKV 2.A:
 * attend over the selected subset; Tutorial, "MHA et GQA").
 *
 * For each (b, h), g = h / (n_h/n_kv), n = count[b][g] clamped to [0, cap]:
 *   y_t = scale * <q[b][h], kc[b][g][t]>, t < n
 *   out[b][h] = sum_t softmax(y)_t * vc[b][g][t]     (count 0: zeros)
 *   lse[b][h] = max_t y_t + log(sum_t exp(y_t - max_t y_t))   (count 0: -inf)
 *
 * dims       batch, n_h, n_kv, d_h and dtype are used (s_max and seq_lens are not)
 * q          [B][n_h][d_h] dtype
 * kc, vc     [B][n_kv][cap][d_h] dtype
 * count      [B][n_kv] int32
 * out        [B][n_h][d_h] dtype (bf16: round to nearest even)
 * lse        [B][n_h] float or NULL
 * q, kc, vc and out 16-byte aligned
 * ws         at least kvc_decode_attn_workspace(dims, cap) bytes, 16-byte aligned,
 *            zero-filled before first use: its first 65536 bytes hold arrival counters
 *            (one per KV head and chunk of query heads) that every completed call
 *            leaves at zero, the rest the split partials.  One workspace of the
 *            largest size needed serves calls of any shape in stream order; calls
 *            that overlap on one workspace race
 * Splits over t are merged in a fixed order: results are bit-reproducible.
 */
size_t kvc_decode_attn_workspace(const kvc_dims *dims, int32_t cap);
kvc_status kvc_decode_attn(const kvc_dims *dims, const void *q, const void *kc, const void *vc,
                           const int32_t *count, int32_t cap, float scale, void *out, float *lse,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * kvc_decode_attn_plan -- the launch configuration kvc_decode_attn takes for these
 * shapes, for tests and profiling:
 *   out[0]  token splits per KV head (work-groups along t)
 *   out[1]  tokens per split
 *   out[2]  query heads per work-group (the rest of a group in further chunks)
 *   out[3]  1 when the last work-group of a (KV head, chunk) to finish folds the
 *           splits itself (up to 64 splits for one head per work-group, fewer for
 *           more heads: 8 for eight heads of 128 elements), 0 when a second kernel does
 * out  int32[4], host memory.  KVC_ERR_INVALID_ARG for invalid dims, cap < 1 or a
 * NULL out.
 */
kvc_status kvc_decode_attn_plan(const kvc_dims *dims, int32_t cap, int32_t *out);

/*
 * kvc_decode_attn_noalloc -- kvc_decode_attn for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and kernels as kvc_decode_attn, without the
 * workspace: the split partials go to a static device array of the library, one per
 * GPU, of 4 MiB (4194304 bytes), held until the process ends.
 * A shape whose kvc_decode_attn_workspace() exceeds that limit returns
 * KVC_ERR_WORKSPACE and launches nothing.  The call allocates nothing; the array is
 * zero when the library loads and every call leaves its counters at zero, as
 * kvc_decode_attn does those of its workspace.  Every call on a GPU uses that GPU's
 * one array: calls that may overlap on one GPU (other streams, other threads) race
 * and must be ordered by the caller.
 */
kvc_status kvc_decode_attn_noalloc(const kvc_dims *dims, const void *q, const void *kc, const void *vc,
                                   const int32_t *count, int32_t cap, float scale, void *out, float *lse,
                                   void *stream);

/*
 * Landmark-guided block selection (xKV 2.3).  The cache of each KV head is cut into
 * n_blk = ceil(s_max / block) blocks of `block` tokens.
 *
 * kvc_block_landmarks: landmarks[b][g][j] = mean of k[b][g][t] over the block's tokens
 *   t < S_b (0 for a block with none), summed in token order in double, rounded to float.
 *   k [B][n_kv][s_max][d_h] dtype; landmarks [B][n_kv][n_blk][d_h] float.
 * kvc_block_scores: for the candidate blocks j < cand[b] = floor(max(0, S_b - n_keep) /
 *   block): scores[b][g][j] = scale * sum over the query heads h of g, then over d, of
 *   q[b][h][d] * landmarks[b][g][j][d] (exact products added in that order in double,
 *   rounded to float); 0 for the other blocks.  scale 0 selects 1/sqrt(d_h) (in double);
 *   q [B][n_h][d_h] dtype; scores [B][n_kv][n_blk] float; cand [B] int32.
 *   Select the blocks with kvc_select_topk(dims with s_max = n_blk, seq_lens = cand,
 *   k = blocks to keep, n_keep = 0).
 * kvc_expand_blocks: for unit u = (b, h): the count_blk[u] kept blocks (ascending in
 *   idx_blk) give tokens idx_blk[u][j] * block + i at position j * block + i, then the
 *   tail [cand[b] * block, S_b) (the trailing tokens that start no candidate block);
 *   -1 past count; count[u] = min(cap, count_blk[u] * block + S_b - cand[b] * block).
 *   cap = k_blocks * block + n_keep + block - 1 holds every case.
 */
kvc_status kvc_block_landmarks(const kvc_dims *dims, const void *k, int32_t block, float *landmarks, void *stream);
kvc_status kvc_block_scores(const kvc_dims *dims, const void *q, const float *landmarks, int32_t block,
                            int32_t n_keep, float scale, float *scores, int32_t *cand, void *stream);
kvc_status kvc_expand_blocks(int32_t batch, int32_t heads, int32_t s_max, const int32_t *seq_lens, int32_t block,
                             int32_t n_keep, const int32_t *idx_blocks, const int32_t *count_blocks,
                             int32_t cap_blocks, int32_t *idx, int32_t *count, int32_t cap, void *stream);

/*
 * kvc_query_similarity -- which KV heads must select again before attention at this
 * decode step (FreeKV, technical summary 2.A).  Queries of adjacent steps are very
 * similar, so a step may attend over the subset selected with the previous step's
 * query (speculative retrieval); where the similarity of a head's two queries falls
 * below a threshold tau, the selection is redone for that head first (fine-grained
 * correction).  Selection is per KV head, so a KV head is corrected as soon as one
 * of its query heads drifted.
 *
 * For each (b, h), g = h / (n_h/n_kv):
 *   cos[b][h] = <q_cur[b][h], q_prev[b][h]> / (|q_cur[b][h]| |q_prev[b][h]|),
 *               0 when either norm is 0 (sums in double, rounded to float)
 *   refresh[b][g] = 1 iff cos[b][h] < tau (compared in double) for some h of g, else 0
 *   keep[b][g] = 1 - refresh[b][g]
 * refresh (keep) is a unit_mask for the calls that redo (skip) the selection.
 *
 * dims           batch, n_h, n_kv, d_h and dtype are used
 * q_cur, q_prev  [B][n_h][d_h] dtype, 16-byte aligned
 * tau            any finite value: tau > 1 corrects every head, tau <= -1 none
 * cos            [B][n_h] float or NULL
 * refresh        [B][n_kv] int32
 * keep           [B][n_kv] int32 or NULL
 * No workspace.
 */
kvc_status kvc_query_similarity(const kvc_dims *dims, const void *q_cur, const void *q_prev, double tau,
                                float *cos, int32_t *refresh, int32_t *keep, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
