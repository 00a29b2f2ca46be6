/*
 * kvc_oracle.c -- plain, slow, fp64 CPU oracle of the KV-cache compression hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file.  It shares no code,
 * header, table or helper with the HIP implementation, and it never calls it.
 *
 * What it computes, step by step, and where the pages state it:
 *
 *   [FastKV]   "FastKV: Decoupling of Context Reduction and KV Cache Compression
 *              for Prefill-Decoding Acceleration", section 2.A (Token-Selective
 *              Propagation: token saliency is computed from the attention of the
 *              recent-window tokens; only the selected tokens and the sliding-window
 *              tokens are propagated) and section 2.B (the TSP rate and the KV
 *              retention rate are two independent budgets).
 *   [Tutorial] "Variantes de l'attention et compression du cache KV":
 *              section "MHA et GQA" (cache size 2*L*S*n_kv*d_h*b, several query
 *              heads share one KV head), section "Quand la reutilisation est-elle
 *              exacte ?" (causal alignment of new rows after S cached tokens; keep
 *              the original position indices after eviction), section "Compresser
 *              un cache existant" (SnapKV scores prompt positions from the attention
 *              of an observation window and keeps a subset of past keys/values).
 *   [FreeKV]   "FreeKV: Boosting KV Cache Retrieval for Efficient LLM Inference",
 *              technical summary section 2.A (each decode step selects a subset of
 *              the cache with the current query, then attends over it).
 *
 * Readings where the pages leave a step open:
 *   logit scale 1/sqrt(d_h) unless given; query head h uses KV head h / (n_h/n_kv);
 *   window rows are the last w cached tokens, so window row i sees key t iff
 *   t <= S_b - w + i (a query that is not in the cache sees every key); the window
 *   and the GQA group are reduced by a plain sum of softmax probabilities; pooling
 *   is a centred stride-1 max over the candidate region [0, S_b - n_keep) only;
 *   the budget k counts candidates and the n_keep trailing tokens are kept on top;
 *   ties go to the lower index; kept indices are emitted in ascending order.
 *
 * Arithmetic: logits, softmax and probability sums in double; the window score is
 * rounded to float once at the end.  Pooling and selection compare those float
 * scores exactly (the decision is taken in the precision the scores are stored
 * in), and the head-shared (TSP) score is the sum over KV heads in double.  Decode
 * attention is accumulated in double.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KVO_API __attribute__((visibility("default")))

/* Tutorial, "MHA et GQA": bytes of a KV cache for one sequence, 2 * L * S * n_kv * d_h * b
 * (the factor two counts keys and values). */
KVO_API uint64_t kvo_cache_bytes(int64_t L, int64_t S, int64_t n_kv, int64_t d_h, int64_t b)
{
    return (uint64_t)2 * (uint64_t)L * (uint64_t)S * (uint64_t)n_kv * (uint64_t)d_h * (uint64_t)b;
}

/* Sets the OpenMP thread count (n <= 0 keeps the default) and returns the count in use. */
KVO_API int kvo_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
    return omp_get_max_threads();
#else
    (void)n;
    return 1;
#endif
}

static int seq_len_of(const int32_t *seq_lens, int b, int s_max)
{
    int s = seq_lens ? seq_lens[b] : s_max;
    if (s < 0) s = 0;
    if (s > s_max) s = s_max;
    return s;
}

/*
 * Observation-window saliency of one layer (FastKV 2.A; Tutorial, "Compresser un
 * cache existant"), then the max pool over the candidate region.
 *
 * q_win  [B][n_h][w][d_h]   window queries (row i of head h)
 * k      [B][n_kv][s_max][d_h]
 * raw64  [B][n_kv][s_max]   optional: the probability sums in double
 * raw    [B][n_kv][s_max]   the same rounded to float; 0 for t >= S_b
 * pooled [B][n_kv][s_max]   candidates t < S_b - n_keep: max of raw over the centred
 *                           window of width pool clipped to the candidate region;
 *                           other t < S_b: raw[t]; t >= S_b: 0
 */
KVO_API void kvo_score_window(int B, int s_max, const int32_t *seq_lens, int n_h, int n_kv, int d_h,
                              const float *q_win, const float *k, int w, int window_in_cache,
                              int n_keep, int pool, double scale,
                              double *raw64, float *raw, float *pooled)
{
    const int r = n_h / n_kv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < n_kv; ++g) {
            const int S = seq_len_of(seq_lens, b, s_max);
            const size_t unit = (size_t)b * n_kv + g;
            const float *kb = k + unit * (size_t)s_max * d_h;
            double *acc = (double *)calloc((size_t)S + 1, sizeof(double));
            double *x = (double *)malloc(((size_t)S + 1) * sizeof(double));

            /* Query heads g*r .. g*r + r - 1 share KV head g (Tutorial, "MHA et GQA"). */
            for (int hh = 0; hh < r; ++hh) {
                const int h = g * r + hh;
                for (int i = 0; i < w; ++i) {
                    const float *q = q_win + (((size_t)b * n_h + h) * w + i) * d_h;
                    /* Causal alignment (Tutorial, "Quand la reutilisation ..."): window
                     * row i is the token at position S - w + i and sees keys up to it. */
                    long last = window_in_cache ? (long)S - w + i : (long)S - 1;
                    if (last > (long)S - 1) last = (long)S - 1;
                    if (last < 0) continue; /* a row that sees no key adds nothing */
                    double M = -INFINITY;
                    for (long t = 0; t <= last; ++t) {
                        double dot = 0.0;
                        const float *kr = kb + (size_t)t * d_h;
                        for (int d = 0; d < d_h; ++d) dot += (double)q[d] * (double)kr[d];
                        x[t] = scale * dot;
                        if (x[t] > M) M = x[t];
                    }
                    double L = 0.0;
                    for (long t = 0; t <= last; ++t) L += exp(x[t] - M);
                    /* Window and group reduction: plain sum of the probabilities. */
                    for (long t = 0; t <= last; ++t) acc[t] += exp(x[t] - M) / L;
                }
            }

            float *rw = raw + unit * (size_t)s_max;
            float *pl = pooled + unit * (size_t)s_max;
            for (int t = 0; t < s_max; ++t) {
                rw[t] = t < S ? (float)acc[t] : 0.0f;
                if (raw64) raw64[unit * (size_t)s_max + t] = t < S ? acc[t] : 0.0;
            }
            /* Candidate region: every cached token except the n_keep trailing ones,
             * which are always kept (FastKV 2.A: the sliding-window tokens propagate). */
            const int cand_end = S - n_keep > 0 ? S - n_keep : 0;
            const int half = pool / 2;
            for (int t = 0; t < s_max; ++t) {
                if (t < cand_end) {
                    int lo = t - half < 0 ? 0 : t - half;
                    int hi = t + half > cand_end - 1 ? cand_end - 1 : t + half;
                    float m = rw[lo];
                    for (int u = lo + 1; u <= hi; ++u)
                        if (rw[u] > m) m = rw[u];
                    pl[t] = m;
                } else {
                    pl[t] = t < S ? rw[t] : 0.0f;
                }
            }
            free(acc);
            free(x);
        }
    }
}

typedef struct {
    double key; /* a float score widened exactly, or the double head sum (TSP) */
    int32_t t;
} kvo_item;

/* Total order of the selection: higher score first, lower index first on equal scores. */
static int by_score_desc_index_asc(const void *pa, const void *pb)
{
    const kvo_item *a = (const kvo_item *)pa, *b = (const kvo_item *)pb;
    if (a->key > b->key) return -1;
    if (a->key < b->key) return 1;
    return (a->t > b->t) - (a->t < b->t);
}

static int by_int_asc(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

/*
 * Per-KV-head top-k under the retention budget (FastKV 2.B), plus the n_keep
 * trailing tokens (FastKV 2.A), in ascending original order (Tutorial, "Quand la
 * reutilisation ...": keep the original positions).
 *
 * scores [B][H][s_max] float; shared_heads != 0 selects one set per sequence from
 *        the sum over the H heads (TSP, FastKV 2.A: one token set is propagated for
 *        every head), taken in double (every addend is exact in double, and the sum's
 *        rounding error stays far below the spacing of the float scores).
 * idx    [B][H_out][k + n_keep], H_out = shared_heads ? 1 : H; -1 past count
 * count  [B][H_out] = min(k, C) + (S_b - C), C = max(0, S_b - n_keep)
 */
KVO_API void kvo_select_topk(int B, int H, int s_max, const int32_t *seq_lens, const float *scores,
                             int k, int n_keep, int shared_heads, int32_t *idx, int32_t *count)
{
    const int H_out = shared_heads ? 1 : H;
    const int cap = k + n_keep;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H_out; ++h) {
            const int S = seq_len_of(seq_lens, b, s_max);
            const int cand_end = S - n_keep > 0 ? S - n_keep : 0;
            const int k_eff = k < cand_end ? k : cand_end;
            kvo_item *items = (kvo_item *)malloc(((size_t)cand_end + 1) * sizeof(kvo_item));
            for (int t = 0; t < cand_end; ++t) {
                double s;
                if (shared_heads) {
                    s = 0.0;
                    for (int g = 0; g < H; ++g) s += (double)scores[((size_t)b * H + g) * s_max + t];
                } else {
                    s = (double)scores[((size_t)b * H + h) * s_max + t];
                }
                items[t].key = s;
                items[t].t = t;
            }
            qsort(items, (size_t)cand_end, sizeof(kvo_item), by_score_desc_index_asc);
            int32_t *out = idx + ((size_t)b * H_out + h) * cap;
            for (int j = 0; j < k_eff; ++j) out[j] = items[j].t;
            qsort(out, (size_t)k_eff, sizeof(int32_t), by_int_asc);
            int n = k_eff;
            for (int t = cand_end; t < S; ++t) out[n++] = t;
            count[(size_t)b * H_out + h] = n;
            for (int j = n; j < cap; ++j) out[j] = -1;
            free(items);
        }
    }
}

/*
 * Compacting gather that keeps original positions (Tutorial, "Quand la
 * reutilisation ..."): row j of unit (b, h) is row idx[j] of the source;
 * pos_out[j] = src_pos[b][idx[j]] (idx[j] itself when src_pos is NULL).
 * Rows j >= count are left untouched and get pos_out -1.
 */
KVO_API void kvo_gather(int B, int heads, int s_max, int row_bytes, const uint8_t *src,
                        const int32_t *src_pos, const int32_t *idx, const int32_t *count, int cap,
                        uint8_t *dst, int32_t *pos_out)
{
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < heads; ++h) {
            const size_t unit = (size_t)b * heads + h;
            int n = count[unit];
            if (n < 0) n = 0;
            if (n > cap) n = cap;
            for (int j = 0; j < cap; ++j) {
                if (j < n) {
                    const int t = idx[unit * cap + j];
                    if (dst)
                        memcpy(dst + (unit * cap + j) * (size_t)row_bytes,
                               src + (unit * s_max + t) * (size_t)row_bytes, (size_t)row_bytes);
                    if (pos_out) pos_out[unit * cap + j] = src_pos ? src_pos[(size_t)b * s_max + t] : t;
                } else if (pos_out) {
                    pos_out[unit * cap + j] = -1;
                }
            }
        }
    }
}

/*
 * GQA decode attention of one new query per head over the compacted cache
 * (FreeKV technical summary 2.A: attend over the selected subset; Tutorial,
 * "MHA et GQA": query head h reads KV head h / (n_h/n_kv)).
 *
 * q [B][n_h][d_h]; kc, vc [B][n_kv][cap][d_h]; count [B][n_kv]
 * out [B][n_h][d_h] = sum_t softmax(y)_t vc[t], y_t = scale <q, kc[t]>, t < count
 * lse [B][n_h] = M + log(sum_t exp(y_t - M)); count 0 gives out 0 and lse -inf.
 */
KVO_API void kvo_decode(int B, int n_h, int n_kv, int d_h, const float *q, const float *kc,
                        const float *vc, const int32_t *count, int cap, double scale,
                        double *out, double *lse)
{
    const int r = n_h / n_kv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < n_h; ++h) {
            const int g = h / r;
            const size_t unit = (size_t)b * n_kv + g;
            int n = count[unit];
            if (n < 0) n = 0;
            if (n > cap) n = cap;
            const float *qh = q + ((size_t)b * n_h + h) * d_h;
            double *o = out + ((size_t)b * n_h + h) * d_h;
            for (int d = 0; d < d_h; ++d) o[d] = 0.0;
            if (n == 0) {
                if (lse) lse[(size_t)b * n_h + h] = -INFINITY;
                continue;
            }
            double *y = (double *)malloc((size_t)n * sizeof(double));
            double M = -INFINITY;
            for (int t = 0; t < n; ++t) {
                const float *kr = kc + (unit * cap + t) * (size_t)d_h;
                double dot = 0.0;
                for (int d = 0; d < d_h; ++d) dot += (double)qh[d] * (double)kr[d];
                y[t] = scale * dot;
                if (y[t] > M) M = y[t];
            }
            double L = 0.0;
            for (int t = 0; t < n; ++t) L += exp(y[t] - M);
            for (int t = 0; t < n; ++t) {
                const double p = exp(y[t] - M) / L;
                const float *vr = vc + (unit * cap + t) * (size_t)d_h;
                for (int d = 0; d < d_h; ++d) o[d] += p * (double)vr[d];
            }
            if (lse) lse[(size_t)b * n_h + h] = M + log(L);
            free(y);
        }
    }
}

/*
 * Query similarity of two adjacent decode steps and the heads it sends to
 * correction (FreeKV technical summary 2.A: queries of adjacent steps are very
 * similar, so step i attends over the subset selected with the query of step
 * i - 1; when the cosine similarity of the two queries of a head falls below a
 * threshold tau, selection and retrieval run again for that head before attention).
 *
 * q_cur, q_prev [B][n_h][d_h]
 * cos_out [B][n_h] = <q_cur, q_prev> / (|q_cur| |q_prev|), 0 when either norm is 0
 * refresh [B][n_kv] = 1 iff some query head h of KV head g (h / (n_h/n_kv) == g)
 *                     has cos_out < tau, else 0 (selection is per KV head, so a KV
 *                     head is corrected as soon as one of its query heads drifted)
 * Sums in double; the comparison with tau is on the double cosine.
 */
KVO_API void kvo_query_similarity(int B, int n_h, int n_kv, int d_h, const float *q_cur,
                                  const float *q_prev, double tau, double *cos_out, int32_t *refresh)
{
    const int r = n_h / n_kv;
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < n_kv; ++g) refresh[(size_t)b * n_kv + g] = 0;
        for (int h = 0; h < n_h; ++h) {
            const float *x = q_cur + ((size_t)b * n_h + h) * d_h;
            const float *y = q_prev + ((size_t)b * n_h + h) * d_h;
            double xy = 0.0, xx = 0.0, yy = 0.0;
            for (int d = 0; d < d_h; ++d) {
                xy += (double)x[d] * (double)y[d];
                xx += (double)x[d] * (double)x[d];
                yy += (double)y[d] * (double)y[d];
            }
            const double c = (xx > 0.0 && yy > 0.0) ? xy / (sqrt(xx) * sqrt(yy)) : 0.0;
            cos_out[(size_t)b * n_h + h] = c;
            if (c < tau) refresh[(size_t)b * n_kv + h / r] = 1;
        }
    }
}

/*
 * Role-based retention (CASK, "Core" and "Scratch" tokens): core tokens are always
 * kept; the budget k applies to the scratch tokens only.  The n_keep trailing tokens
 * stay kept as in kvo_select_topk.
 *
 * scores [B][H][s_max] float; core [B][s_max] uint8, nonzero = core token (a role of
 * the token, shared by every head of the sequence).
 * With C = max(0, S_b - n_keep), Core = {t < C : core[b][t]}, Scratch = [0, C) \ Core:
 *   k_eff = min(k, |Scratch|); Sel = the first k_eff scratch tokens in the order
 *   (score desc, index asc); idx = sort_asc(Sel u Core) ++ [C, S_b);
 *   count = k_eff + |Core| + (S_b - C); -1 past count.
 * The output holds cap = k + core_cap + n_keep indices per unit.  When the caller's
 * core_cap is smaller than |Core| the candidates cannot all fit: the unit then keeps
 * the first k + core_cap candidates of the list "Core by ascending index, then Scratch
 * in the selection order" (every core token while they fit, the best scratch tokens
 * in what is left), so count never exceeds cap.  Otherwise this is the rule above.
 */
KVO_API void kvo_select_core(int B, int H, int s_max, const int32_t *seq_lens, const float *scores,
                             const uint8_t *core, int k, int core_cap, int n_keep, int32_t *idx, int32_t *count)
{
    const int cap = k + core_cap + n_keep;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < H; ++h) {
            const int S = seq_len_of(seq_lens, b, s_max);
            const int C = S - n_keep > 0 ? S - n_keep : 0;
            kvo_item *items = (kvo_item *)malloc(((size_t)C + 1) * sizeof(kvo_item));
            int32_t *keep = (int32_t *)malloc(((size_t)S + 1) * sizeof(int32_t));
            int n_scratch = 0, n_core = 0;
            for (int t = 0; t < C; ++t) {
                if (core[(size_t)b * s_max + t]) {
                    keep[n_core++] = t;                 /* core: always kept (ascending) */
                } else {
                    items[n_scratch].key = (double)scores[((size_t)b * H + h) * s_max + t];
                    items[n_scratch].t = t;
                    ++n_scratch;
                }
            }
            qsort(items, (size_t)n_scratch, sizeof(kvo_item), by_score_desc_index_asc);
            const int k_eff = k < n_scratch ? k : n_scratch;
            int n_cand = n_core + k_eff;                /* the rule's kept candidates */
            if (n_cand > k + core_cap) n_cand = k + core_cap;   /* what the output can hold */
            int n = n_core < n_cand ? n_core : n_cand;  /* core first, lowest index first */
            for (int j = 0; n < n_cand; ++j) keep[n++] = items[j].t;
            qsort(keep, (size_t)n, sizeof(int32_t), by_int_asc);
            for (int t = C; t < S; ++t) keep[n++] = t;
            int32_t *out = idx + ((size_t)b * H + h) * cap;
            for (int j = 0; j < n; ++j) out[j] = keep[j];
            for (int j = n; j < cap; ++j) out[j] = -1;
            count[(size_t)b * H + h] = n;
            free(items);
            free(keep);
        }
    }
}

/*
 * Landmark-guided block selection (xKV, section 2.3 "Reconstruction Selective": the
 * tokens most relevant to the current query are found by a block selection guided by
 * landmarks, as in ShadowKV).  The cache of each KV head is cut into blocks of `block`
 * consecutive tokens; a block's landmark is the mean of its keys; a block's score is
 * the group's attention logit for its landmark; the best blocks are kept whole.
 */

/* landmarks [B][n_kv][n_blk][d_h], n_blk = ceil(s_max / block): the mean of the keys
 * t < S_b of each block (0 for a block with none), in double, rounded to float. */
KVO_API void kvo_block_landmarks(int B, int n_kv, int s_max, int d_h, const int32_t *seq_lens,
                                 const float *k, int block, float *landmarks)
{
    const int n_blk = (s_max + block - 1) / block;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < n_kv; ++g) {
            const int S = seq_len_of(seq_lens, b, s_max);
            for (int j = 0; j < n_blk; ++j) {
                float *lm = landmarks + (((size_t)b * n_kv + g) * n_blk + j) * d_h;
                const int t0 = j * block;
                const int t1 = t0 + block < S ? t0 + block : S;
                for (int d = 0; d < d_h; ++d) {
                    double s = 0.0;
                    for (int t = t0; t < t1; ++t) s += (double)k[(((size_t)b * n_kv + g) * s_max + t) * d_h + d];
                    lm[d] = t1 > t0 ? (float)(s / (double)(t1 - t0)) : 0.0f;
                }
            }
        }
    }
}

/* scores [B][n_kv][n_blk] = scale * sum over the query heads h of KV head g of
 * <q[b][h], landmark[b][g][j]> (in double, rounded to float) for the candidate blocks
 * j < cand[b] = floor(max(0, S_b - n_keep) / block), 0 elsewhere. */
KVO_API void kvo_block_scores(int B, int n_h, int n_kv, int s_max, int d_h, const int32_t *seq_lens,
                              const float *q, const float *landmarks, int block, int n_keep, double scale,
                              float *scores, int32_t *cand)
{
    const int r = n_h / n_kv;
    const int n_blk = (s_max + block - 1) / block;
    for (int b = 0; b < B; ++b) {
        const int S = seq_len_of(seq_lens, b, s_max);
        const int C = S - n_keep > 0 ? S - n_keep : 0;
        cand[b] = C / block;
        for (int g = 0; g < n_kv; ++g) {
            for (int j = 0; j < n_blk; ++j) {
                double s = 0.0;
                if (j < cand[b]) {
                    const float *lm = landmarks + (((size_t)b * n_kv + g) * n_blk + j) * d_h;
                    for (int h = g * r; h < (g + 1) * r; ++h) {
                        const float *qh = q + ((size_t)b * n_h + h) * d_h;
                        for (int d = 0; d < d_h; ++d) s += (double)qh[d] * (double)lm[d];
                    }
                }
                scores[((size_t)b * n_kv + g) * n_blk + j] = (float)(scale * s);
            }
        }
    }
}

/* Token list of the kept blocks: for unit u, the count_blk[u] selected blocks (their
 * indices ascending in idx_blk) expand to their `block` tokens each, in order, then the
 * tail [cand * block, S_b) that is not a candidate block is kept; -1 past count. */
KVO_API void kvo_expand_blocks(int B, int H, int s_max, const int32_t *seq_lens, int block, int n_keep,
                               const int32_t *idx_blk, const int32_t *count_blk, int cap_blk,
                               int32_t *idx, int32_t *count, int cap)
{
    for (int b = 0; b < B; ++b) {
        const int S = seq_len_of(seq_lens, b, s_max);
        const int C = S - n_keep > 0 ? S - n_keep : 0;
        const int tail0 = (C / block) * block;
        for (int h = 0; h < H; ++h) {
            const size_t u = (size_t)b * H + h;
            int n = 0;
            for (int j = 0; j < count_blk[u]; ++j)
                for (int i = 0; i < block; ++i)
                    if (n < cap) idx[u * cap + n++] = idx_blk[u * cap_blk + j] * block + i;
            for (int t = tail0; t < S; ++t)
                if (n < cap) idx[u * cap + n++] = t;
            count[u] = n;
            for (int j = n; j < cap; ++j) idx[u * cap + j] = -1;
        }
    }
}
