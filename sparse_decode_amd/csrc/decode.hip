// decode.hip -- GQA decode attention of one query per head over the compacted cache
// (FreeKV technical summary section 2.A: attend over the selected subset; Tutorial
// "Variantes de l'attention et compression du cache KV", section "MHA et GQA":
// query head h reads KV head h / (n_h / n_kv)).
//
// Split-K over tokens.  A work-group per (token split, KV head, head chunk) loads
// each K/V row of its split once and uses it for every query head of the chunk (up
// to 8), so the compacted cache is streamed exactly once.  A lane owns 16 bytes of a
// row (8 bf16 or 4 fp32); a row is spread over d_h/8 (d_h/4) lanes, a lane group.
// Each lane group keeps an online softmax state (max m, sum l, output o); the groups
// are folded in group order into the split's partial state.  The splits of a
// (KV head, chunk) are folded in split order by whichever of its work-groups arrives
// last (an arrival counter per chunk; up to kFuseSplits splits, fewer for many heads
// per work-group), or, for more splits, by a second kernel.  Either way the result does not depend on scheduling.  Logits
// are kept in log2 units: q is pre-multiplied by scale * log2(e).  The arrival
// counters open the workspace in a region of fixed size that no partial ever
// overwrites; the last arrival returns its counter to zero, so one zero-filled
// workspace serves calls of any shape.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;

template <bool BF16>
struct RowVec;
template <>
struct RowVec<true> {
    static constexpr int kElems = 8;
    __device__ static void unpack(const u32x4 &v, float *f)
    {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    }
};
template <>
struct RowVec<false> {
    static constexpr int kElems = 4;
    __device__ static void unpack(const u32x4 &v, float *f)
    {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
};

// Merges online-softmax state (m2, l2, o2) into (m, l, o); m = -inf means empty.
template <int E>
__device__ __forceinline__ void merge_state(float &m, float &l, float *o, float m2, float l2, const float *o2)
{
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) return;
    const float a = fast_exp2(m - M), a2 = fast_exp2(m2 - M);
    l = l * a + l2 * a2;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = o[e] * a + o2[e] * a2;
    m = M;
}

struct DecArgs {
    const void *q, *kc, *vc;
    const int32_t *count;
    int cap, n_h, n_kv, r, n_splits, split_tokens, head_chunks;
    float c;                  // scale * log2(e)
    float *part_o;            // [units][r][n_splits][D]
    float2 *part_ml;          // [units][r][n_splits] (max, sum) in log2 units
    int32_t *arrive;          // [units][head_chunks] arrivals, or null: the merge kernel folds
    void *out;                // [B][n_h][D]
    float *lse;               // [B][n_h] or null
};

constexpr int kMaxSplits = 1024;   // longer caches take longer splits
constexpr int kFuseSplits = 64;    // at most this many splits are folded by their last arrival
constexpr int kDecWgPerCu = 2;     // work-groups per CU the split count aims at
constexpr int kUnroll = 4;          // token rows per lane group and batch (two batches in flight)

// Writes one output element and, for d == 0, the log-sum-exp (natural log).
template <bool BF16>
__device__ __forceinline__ void store_out(void *out, float *lse, size_t bh, int D, int d, float M, float L, float O)
{
    const float y = (L > 0.f) ? O / L : 0.f;
    if (BF16)
        ((uint16_t *)out)[bh * D + d] = f32_to_bf16(y);
    else
        ((float *)out)[bh * D + d] = y;
    if (lse && d == 0) lse[bh] = (L > 0.f) ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// Fold of a few splits (at most kFoldSmall) when a thread per (head, element) pair
// fits the work-group: each thread loads every split's (max, sum) of its head and its
// element of every split's output at once, forms the weights itself and adds the
// splits in split order; no LDS, no barrier.
constexpr int kFoldSmall = 16;

template <bool BF16, int D, int RH>
__device__ __forceinline__ void fold_small(const DecArgs &a, int unit, int hc, int heads)
{
    static_assert(RH * D <= kDecThreads, "a thread per pair");
    const int tid = kvc_tid();
    if (tid >= heads * D) return;
    const int j = tid / D, d = tid - j * D;
    const int NS = a.n_splits;
    const size_t base = ((size_t)unit * a.r + hc * RH + j) * NS;   // slot of (head j, split 0)
    const unsigned long long *ml = (const unsigned long long *)a.part_ml + base;
    const float *po = a.part_o + base * D + d;
    unsigned long long mlv[kFoldSmall];
    float v[kFoldSmall];
#pragma unroll
    for (int q = 0; q < kFoldSmall; ++q) {
        if (q < NS) {
            mlv[q] = ld_dev(ml + q);
            v[q] = ld_dev(po + (size_t)q * D);
        }
    }
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < kFoldSmall; ++q)
        if (q < NS) M = fmaxf(M, unpack_lo(mlv[q]));
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int q = 0; q < kFoldSmall; ++q) {
        if (q < NS) {
            const float m = unpack_lo(mlv[q]);
            const float w = (M == -INFINITY || m == -INFINITY) ? 0.f : fast_exp2(m - M);
            L = fmaf(w, unpack_hi(mlv[q]), L);
            O = fmaf(w, v[q], O);
        }
    }
    const int b = unit / a.n_kv;
    const int g = unit - b * a.n_kv;
    store_out<BF16>(a.out, a.lse, (size_t)b * a.n_h + g * a.r + hc * RH + j, D, d, M, L, O);
}

// Split-fold geometry of a chunk of RH heads of D elements: the kDecThreads threads
// take (head, element) pairs, SG split groups per pair when there are fewer pairs
// than threads, PPT pairs per thread otherwise.  A thread holds every partial value it
// folds in registers at once (at most kFoldVals), which bounds the splits a last
// arrival folds: fold_limit(RH * D) splits, at most kFuseSplits.
constexpr int kFoldVals = 32;
__host__ __device__ constexpr int fold_sg(int pt) { return pt >= kDecThreads ? 1 : kDecThreads / pt; }
__host__ __device__ constexpr int fold_ppt(int pt) { return pt >= kDecThreads ? pt / kDecThreads : 1; }
__host__ __device__ constexpr int fold_limit(int pt)
{
    return kFoldVals * fold_sg(pt) / fold_ppt(pt) < kFuseSplits ? kFoldVals * fold_sg(pt) / fold_ppt(pt) : kFuseSplits;
}

// The last work-group to arrive for (unit, head chunk) folds the chunk's split
// partials in split order.  Every load (split maxima and sums, the partial outputs)
// is issued first, so the fold costs one memory round trip; the maxima and sums go to
// LDS, where a wave per head forms the weights exp2(m_s - M) and L; each thread folds
// its pairs' values over its strided subset of the splits and the split groups are
// added in group order.  `lds` holds at least
// 2 * RH * n_splits + kDecThreads floats; n_splits <= fold_limit(RH * D).
template <bool BF16, int D, int RH>
__device__ void fold_splits(const DecArgs &a, int unit, int hc, int heads, float *lds, float *sM, float *sL)
{
    constexpr int PT = RH * D;                // (head, element) pairs
    constexpr int SG = fold_sg(PT);
    constexpr int PPT = fold_ppt(PT);
    constexpr int VPP = kFoldVals / PPT;      // split values per pair and thread
    constexpr int MLT = (RH * kFuseSplits + kDecThreads - 1) / kDecThreads;
    static_assert(PT % kDecThreads == 0 || kDecThreads % PT == 0, "pairs and threads");
    const int NS = a.n_splits;
    const int tid = kvc_tid();
    const int lane = tid & (kWave - 1);
    const int wv = tid >> 6;
    const int sg = tid / (PT < kDecThreads ? PT : kDecThreads);
    float *wm = lds;                  // [heads][NS] split maxima, then weights
    float *wl = lds + RH * NS;        // [heads][NS] split sums
    float *red = wl + RH * NS;        // [SG][PT] group sums
    const size_t base = ((size_t)unit * a.r + hc * RH) * NS;    // slot of (head 0, split 0)
    unsigned long long *ml = (unsigned long long *)a.part_ml;
    unsigned long long mlv[MLT];
#pragma unroll
    for (int i = 0; i < MLT; ++i) {
        const int x = tid + i * kDecThreads;
        if (x < heads * NS) mlv[i] = ld_dev(ml + base + x);
    }
    float v[PPT][VPP];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = PT >= kDecThreads ? tid + i * kDecThreads : tid - sg * PT;
        const int j = p / D;
        const float *po = a.part_o + (base + (size_t)j * NS) * D + (p - j * D);
#pragma unroll
        for (int q = 0; q < VPP; ++q) {
            const int s = sg + q * SG;
            if (j < heads && s < NS) v[i][q] = ld_dev(po + (size_t)s * D);
        }
    }
#pragma unroll
    for (int i = 0; i < MLT; ++i) {
        const int x = tid + i * kDecThreads;
        if (x < heads * NS) {
            wm[x] = unpack_lo(mlv[i]);
            wl[x] = unpack_hi(mlv[i]);
        }
    }
    __syncthreads();
    for (int j = wv; j < heads; j += kDecWaves) {               // NS <= 64: a split per lane
        const bool on = lane < NS;
        const float ms = on ? wm[j * NS + lane] : -INFINITY;
        float M = ms;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) M = fmaxf(M, shfl_xor_f(M, o));
        const float w = (M == -INFINITY || ms == -INFINITY) ? 0.f : fast_exp2(ms - M);
        float L = on ? w * wl[j * NS + lane] : 0.f;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) L += shfl_xor_f(L, o);
        if (on) wm[j * NS + lane] = w;
        if (lane == 0) {
            sM[j] = M;
            sL[j] = L;
        }
    }
    __syncthreads();
    float acc[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = PT >= kDecThreads ? tid + i * kDecThreads : tid - sg * PT;
        const int j = p / D;
        acc[i] = 0.f;
#pragma unroll
        for (int q = 0; q < VPP; ++q) {
            const int s = sg + q * SG;
            if (j < heads && s < NS) acc[i] = fmaf(wm[j * NS + s], v[i][q], acc[i]);
        }
    }
    if (SG > 1) {
        red[sg * PT + (tid - sg * PT)] = acc[0];
        __syncthreads();
        if (sg != 0) return;
        for (int g2 = 1; g2 < SG; ++g2) acc[0] += red[g2 * PT + tid];
    }
    const int b = unit / a.n_kv;
    const int g = unit - b * a.n_kv;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int p = PT >= kDecThreads ? tid + i * kDecThreads : tid;
        const int j = p / D;
        const int d = p - j * D;
        if (j < heads) store_out<BF16>(a.out, a.lse, (size_t)b * a.n_h + g * a.r + hc * RH + j, D, d, sM[j], sL[j], acc[i]);
    }
}

// One work-group per (token split, KV head, head chunk) streams the split's K and V
// rows once (the first rows are requested before the queries) and keeps an online
// softmax state per lane group, updated once per kUnroll rows; the lane groups are
// folded through LDS in group order and the split's partial state is stored.
template <bool BF16, int D, int RH>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecArgs a)
{
    using RV = RowVec<BF16>;
    constexpr int E = RV::kElems;           // elements per lane
    constexpr int LPT = D / E;              // lanes per token row
    constexpr int TPW = kWave / LPT;        // token rows per wave step
    constexpr int VPR = D / E;              // 16-byte vectors per row (== LPT)
    constexpr int G = kDecWaves * TPW;      // lane groups per work-group
    static_assert(LPT <= kWave && (kWave % LPT) == 0, "row must fit a wave");

    __shared__ float sm_o[G][RH][D];
    __shared__ float sm_m[G][RH];
    __shared__ float sm_l[G][RH];
    __shared__ float sm_w[G][RH];
    __shared__ float sm_M[RH];

    const int split = kvc_bid_x();
    const int unit = kvc_bid_y();            // b * n_kv + g
    const int hc = kvc_bid_z();
    const int b = unit / a.n_kv;
    const int g = unit - b * a.n_kv;
    const int tid = kvc_tid();
    const int lane = tid & (kWave - 1);
    const int wv = tid >> 6;
    const int li = lane % LPT;
    const int ts = lane / LPT;
    const int grp = wv * TPW + ts;
    const int r = a.r;
    const int heads = min(RH, r - hc * RH);  // query heads of this chunk

    // ---- phase 1: this split.  Its first rows are requested before the count is
    // known and zeroed past the count once it arrives, so count, rows and queries
    // share one round trip.  Every load is unconditional (row indices clamped below
    // cap, head indices to the chunk's last head) and out-of-range values are dropped
    // afterwards: a load under a branch would be waited for inside it.
    const int s0 = split * a.split_tokens;
    constexpr int step = G;                 // token rows per work-group step
    const u32x4 *krow = (const u32x4 *)a.kc + (size_t)unit * a.cap * VPR + li;
    const u32x4 *vrow = (const u32x4 *)a.vc + (size_t)unit * a.cap * VPR + li;
    u32x4 kv[kUnroll], vv[kUnroll];
    int t = s0 + grp;
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
        const int tq = min(t + q * step, a.cap - 1);
        kv[q] = ld_stream(krow + (size_t)tq * VPR);
        vv[q] = ld_stream(vrow + (size_t)tq * VPR);
    }
    int n = ld_uniform(a.count, unit);
    // queries of this chunk of the group
    const int h_first = g * r + hc * RH;
    u32x4 qv[RH];
#pragma unroll
    for (int j = 0; j < RH; ++j) qv[j] = *((const u32x4 *)a.q + ((size_t)(b * a.n_h + h_first + min(j, heads - 1))) * VPR + li);
    // the rows count as used here, unconditionally: otherwise the compiler moves their
    // loads under the branch on the count below, a round trip later
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) asm volatile("" ::"v"(kv[q]), "v"(vv[q]));
    n = n < 0 ? 0 : (n > a.cap ? a.cap : n);
    const int s1 = min(s0 + a.split_tokens, n);
    // pre-scaled into log2 units; heads past the chunk's end are zero
    float qf[RH][E];
#pragma unroll
    for (int j = 0; j < RH; ++j) {
        RV::unpack(qv[j], qf[j]);
#pragma unroll
        for (int e = 0; e < E; ++e) qf[j][e] = j < heads ? qf[j][e] * a.c : 0.f;
    }
#pragma unroll
    for (int q = 0; q < kUnroll; ++q) {
        if (t + q * step >= s1) {           // past the count: those rows may hold any bits
            kv[q] = u32x4{0u, 0u, 0u, 0u};
            vv[q] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    float m[RH], l[RH], o[RH][E];
#pragma unroll
    for (int j = 0; j < RH; ++j) {
        m[j] = -INFINITY;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) o[j][e] = 0.f;
    }
    // A lane group is entirely in or out of range (t depends on the group only), so
    // the row sums inside the loop always see a whole group.
    for (; t < s1; t += kUnroll * step) {
        u32x4 kn[kUnroll], vn[kUnroll];
        const int tn = t + kUnroll * step;
        if (tn < s1) {                       // next rows, requested before this batch is used
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {
                const int tq = min(tn + q * step, a.cap - 1);   // rows past s1 are masked below
                kn[q] = ld_stream(krow + (size_t)tq * VPR);
                vn[q] = ld_stream(vrow + (size_t)tq * VPR);
            }
        }
        float x[kUnroll][RH];
#pragma unroll
        for (int q = 0; q < kUnroll; ++q) {
            float kf[E];
            RV::unpack(kv[q], kf);
#pragma unroll
            for (int j = 0; j < RH; ++j) {
                float sdot = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) sdot = fmaf(qf[j][e], kf[e], sdot);
                if (LPT == 16) {
                    sdot = row16_sum(sdot);
                } else {
#pragma unroll
                    for (int off = LPT / 2; off > 0; off >>= 1) sdot += shfl_xor_f(sdot, off);
                }
                x[q][j] = t + q * step < s1 ? sdot : -INFINITY;
            }
        }
#pragma unroll
        for (int j = 0; j < RH; ++j) {
            float mx = m[j];
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) mx = fmaxf(mx, x[q][j]);
            const float al = fast_exp2(m[j] - mx);           // m = -inf: 0 (l, o are 0 too)
            float p[kUnroll], ps = 0.f;
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {
                p[q] = fast_exp2(x[q][j] - mx);                // invalid rows: exp2(-inf) = 0
                ps += p[q];
            }
            l[j] = fmaf(l[j], al, ps);
#pragma unroll
            for (int e = 0; e < E; ++e) o[j][e] *= al;
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {
                float vf[E];
                RV::unpack(vv[q], vf);
#pragma unroll
                for (int e = 0; e < E; ++e) o[j][e] = fmaf(p[q], vf[e], o[j][e]);
            }
            m[j] = mx;
        }
        if (tn < s1) {
#pragma unroll
            for (int q = 0; q < kUnroll; ++q) {       // rows past the count may hold any bits
                const bool in = tn + q * step < s1;
                kv[q] = in ? kn[q] : u32x4{0u, 0u, 0u, 0u};
                vv[q] = in ? vn[q] : u32x4{0u, 0u, 0u, 0u};
            }
        }
    }
    // lane-group states -> LDS; the groups are folded in group order
#pragma unroll
    for (int j = 0; j < RH; ++j) {
#pragma unroll
        for (int e = 0; e < E; ++e) sm_o[grp][j][li * E + e] = o[j][e];
        if (li == 0) {
            sm_m[grp][j] = m[j];
            sm_l[grp][j] = l[j];
        }
    }
    __syncthreads();
    if (tid < G * RH) {
        const int g2 = tid / RH, j = tid - (tid / RH) * RH;
        float M = -INFINITY;
        for (int x2 = 0; x2 < G; ++x2) M = fmaxf(M, sm_m[x2][j]);
        const float mg = sm_m[g2][j];
        sm_w[g2][j] = mg == -INFINITY ? 0.f : fast_exp2(mg - M);
        if (g2 == 0) sm_M[j] = M;
    }
    __syncthreads();
    const bool fuse = a.arrive != nullptr;
    for (int x2 = tid; x2 < heads * D; x2 += kDecThreads) {
        const int j = x2 / D;
        const int d = x2 - j * D;
        float L = 0.f, O = 0.f;
        for (int g2 = 0; g2 < G; ++g2) {
            L = fmaf(sm_w[g2][j], sm_l[g2][j], L);
            O = fmaf(sm_w[g2][j], sm_o[g2][j][d], O);
        }
        const size_t slot = ((size_t)unit * r + hc * RH + j) * a.n_splits + split;
        if (fuse) {
            st_dev(a.part_o + slot * D + d, O);
            if (d == 0) st_dev((unsigned long long *)a.part_ml + slot, pack2(sm_M[j], L));
        } else {
            a.part_o[slot * D + d] = O;
            if (d == 0) a.part_ml[slot] = make_float2(sm_M[j], L);
        }
    }
    if (!fuse) return;
    // count this split's arrival once its partial state has landed; the last arrival folds
    stores_done();
    __shared__ int sm_last;
    __syncthreads();
    if (tid == 0) {
        int32_t *cnt = a.arrive + (size_t)unit * a.head_chunks + hc;
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = old == a.n_splits - 1;
        if (sm_last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!sm_last) return;
    if constexpr (RH * D <= kDecThreads) {
        if (a.n_splits <= kFoldSmall) {
            fold_small<BF16, D, RH>(a, unit, hc, heads);
            return;
        }
    }
    fold_splits<BF16, D, RH>(a, unit, hc, heads, &sm_o[0][0][0], sm_M, &sm_w[0][0]);
}

constexpr int kMergeThreads = 256;

// Deterministic block reductions (fixed shuffle tree, then waves in order).
__device__ __forceinline__ float block_max(float v, float *red)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
    if ((kvc_tid() & 63) == 0) red[kvc_tid() >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kMergeThreads / kWave; ++i) r = fmaxf(r, red[i]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ float block_sum(float v, float *red)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += shfl_xor_f(v, o);
    if ((kvc_tid() & 63) == 0) red[kvc_tid() >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kMergeThreads / kWave; ++i) r += red[i];
    __syncthreads();
    return r;
}

// One work-group per (b, h).  Every split's (m, l) and the first kMergeBatch split
// outputs of each thread are requested together up front (one dependent round trip
// for up to G * kMergeBatch splits); the split weights exp2(m_s - M) go to LDS, the
// kMergeThreads / D thread groups fold their strided subsets of the splits and the
// groups are added in group order.
constexpr int kMergeBatch = 32;

template <bool BF16, int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float *__restrict__ part_o,
                                                                     const float2 *__restrict__ part_ml, int n_h,
                                                                     int n_kv, int r, int n_splits,
                                                                     void *__restrict__ out, float *__restrict__ lse)
{
    constexpr int G = kMergeThreads / D;
    constexpr int MLPT = kMaxSplits / kMergeThreads;       // (m, l) pairs per thread
    __shared__ float sw[kMaxSplits];
    __shared__ float red[kMergeThreads / kWave];
    __shared__ float so[G][D];
    const int bh = kvc_bid_x();              // b * n_h + h
    const int b = bh / n_h;
    const int h = bh - b * n_h;
    const int g = h / r;
    const int hl = h - g * r;
    const size_t base = ((size_t)(b * n_kv + g) * r + hl) * n_splits;
    const int d = kvc_tid() % D;
    const int grp = kvc_tid() / D;
    float v[kMergeBatch];
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) {
        const int s = grp + q * G;
        v[q] = s < n_splits ? part_o[(base + s) * D + d] : 0.f;
    }
    float2 ml[MLPT];
#pragma unroll
    for (int i = 0; i < MLPT; ++i) {
        const int s = (int)kvc_tid() + i * kMergeThreads;
        ml[i] = s < n_splits ? part_ml[base + s] : make_float2(-INFINITY, 0.f);
    }

    float mloc = -INFINITY;
#pragma unroll
    for (int i = 0; i < MLPT; ++i) mloc = fmaxf(mloc, ml[i].x);
    const float M = block_max(mloc, red);
    float lloc = 0.f;
#pragma unroll
    for (int i = 0; i < MLPT; ++i) {
        const int s = (int)kvc_tid() + i * kMergeThreads;
        const float wgt = (M == -INFINITY || ml[i].x == -INFINITY) ? 0.f : fast_exp2(ml[i].x - M);
        if (s < n_splits) sw[s] = wgt;
        lloc += wgt * ml[i].y;
    }
    const float L = block_sum(lloc, red);   // also orders the sw[] writes before their reads
    float O = 0.f;
#pragma unroll
    for (int q = 0; q < kMergeBatch; ++q) {
        const int s = grp + q * G;
        if (s < n_splits) O = fmaf(sw[s], v[q], O);
    }
    for (int s0 = grp + kMergeBatch * G; s0 < n_splits; s0 += kMergeBatch * G) {
#pragma unroll
        for (int q = 0; q < kMergeBatch; ++q) {
            const int s = s0 + q * G;
            v[q] = s < n_splits ? part_o[(base + s) * D + d] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < kMergeBatch; ++q) {
            const int s = s0 + q * G;
            if (s < n_splits) O = fmaf(sw[s], v[q], O);
        }
    }
    so[grp][d] = O;
    __syncthreads();
    if (grp != 0) return;
    float Ot = so[0][d];
    for (int g2 = 1; g2 < G; ++g2) Ot += so[g2][d];
    store_out<BF16>(out, lse, bh, D, d, M, L, Ot);
}

template <bool BF16, int D>
hipError_t launch_rh(int rh, dim3 grid, hipStream_t stream, const DecArgs &a)
{
    switch (rh) {
    case 1: hipLaunchKernelGGL((decode_kernel<BF16, D, 1>), grid, dim3(kDecThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<BF16, D, 2>), grid, dim3(kDecThreads), 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<BF16, D, 4>), grid, dim3(kDecThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_kernel<BF16, D, 8>), grid, dim3(kDecThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace

DecodePlan plan_decode(int batch, int n_h, int n_kv, int d_h, int cap, int cus)
{
    DecodePlan p;
    const int r = n_h / n_kv;
    p.head_chunk = r >= 8 ? 8 : (r >= 4 ? 4 : (r >= 2 ? 2 : 1));
    if (p.head_chunk < r && r < 8) p.head_chunk *= 2;   // r = 3, 5, 6, 7 -> next power of two
    p.head_chunks = (r + p.head_chunk - 1) / p.head_chunk;
    const long units = (long)batch * n_kv * p.head_chunks;
    // about kDecWgPerCu work-groups per CU, splits of a multiple of 64 tokens (one
    // unrolled iteration of the work-group), at most kMaxSplits
    long splits = ((long)kDecWgPerCu * cus + units - 1) / units;
    const long max_splits = (cap + 63) / 64;
    if (splits > max_splits) splits = max_splits;
    if (splits > kMaxSplits) splits = kMaxSplits;
    if (splits < 1) splits = 1;
    long tok = (cap + splits - 1) / splits;
    tok = ((tok + 63) / 64) * 64;
    p.split_tokens = (int)tok;
    p.n_splits = (int)((cap + tok - 1) / tok);
    if (p.n_splits < 1) p.n_splits = 1;
    p.fused = p.n_splits <= fold_limit(p.head_chunk * d_h) && units <= kDecCounters;
    const size_t slots = (size_t)batch * n_kv * r * p.n_splits;
    p.o_off = (size_t)kDecCounters * sizeof(int32_t);
    p.ml_off = p.o_off + (slots * (size_t)d_h * sizeof(float) + 255) / 256 * 256;
    p.ws_bytes = p.ml_off + slots * sizeof(float2);
    return p;
}

hipError_t launch_decode(int batch, int n_h, int n_kv, int d_h, bool bf16, const void *q, const void *kc,
                         const void *vc, const int32_t *count, int cap, float scale, void *out, float *lse,
                         void *ws, const DecodePlan &plan, hipStream_t stream)
{
    DecArgs a;
    a.q = q;
    a.kc = kc;
    a.vc = vc;
    a.count = count;
    a.cap = cap;
    a.n_h = n_h;
    a.n_kv = n_kv;
    a.r = n_h / n_kv;
    a.n_splits = plan.n_splits;
    a.split_tokens = plan.split_tokens;
    a.c = scale * 1.4426950408889634f;
    a.head_chunks = plan.head_chunks;
    a.part_o = (float *)((char *)ws + plan.o_off);
    a.part_ml = (float2 *)((char *)ws + plan.ml_off);
    a.arrive = plan.fused ? (int32_t *)ws : nullptr;
    a.out = out;
    a.lse = lse;
    const dim3 grid(plan.n_splits, batch * n_kv, plan.head_chunks);
    hipError_t e = bf16 ? (d_h == 128 ? launch_rh<true, 128>(plan.head_chunk, grid, stream, a)
                                      : launch_rh<true, 64>(plan.head_chunk, grid, stream, a))
                        : (d_h == 128 ? launch_rh<false, 128>(plan.head_chunk, grid, stream, a)
                                      : launch_rh<false, 64>(plan.head_chunk, grid, stream, a));
    if (e != hipSuccess || plan.fused) return e;
    const dim3 mgrid(batch * n_h);
    if (bf16) {
        if (d_h == 128) hipLaunchKernelGGL((decode_merge_kernel<true, 128>), mgrid, dim3(kMergeThreads), 0, stream, a.part_o, a.part_ml, n_h, n_kv, a.r, a.n_splits, out, lse);
        else hipLaunchKernelGGL((decode_merge_kernel<true, 64>), mgrid, dim3(kMergeThreads), 0, stream, a.part_o, a.part_ml, n_h, n_kv, a.r, a.n_splits, out, lse);
    } else {
        if (d_h == 128) hipLaunchKernelGGL((decode_merge_kernel<false, 128>), mgrid, dim3(kMergeThreads), 0, stream, a.part_o, a.part_ml, n_h, n_kv, a.r, a.n_splits, out, lse);
        else hipLaunchKernelGGL((decode_merge_kernel<false, 64>), mgrid, dim3(kMergeThreads), 0, stream, a.part_o, a.part_ml, n_h, n_kv, a.r, a.n_splits, out, lse);
    }
    return hipGetLastError();
}

}  // namespace kvc
