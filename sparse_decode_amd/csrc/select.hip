// select.hip -- per-KV-head top-k under the retention budget (FastKV section 2.B)
// plus the always-kept trailing window (FastKV section 2.A), emitted in ascending
// original order (Tutorial "Variantes de l'attention et compression du cache KV",
// section "Quand la reutilisation est-elle exacte ?": keep original positions).
//
// Scores become order-preserving uint32 keys (-0.0 folded onto +0.0).  The exact
// k-th largest key T of a unit, and how many keys equal to T are still needed, come
// from a three-level radix select over the key bits [21, 32), [10, 21) and [0, 10);
// the selected set is every key > T plus the lowest-indexed keys == T, written in
// index order.  One work-group alone streams a unit's keys far below the chip's
// bandwidth (a CU keeps only so many cache lines in flight), so every pass is spread
// over the unit's chunks of 2048 keys, or 8192 when the call has at least 512 such
// larger chunks (one work-group each, every key loaded once into registers), and the
// levels meet through per-unit histograms in global memory:
//
//   level1  grid (chunks, units): histogram of the top 11 bits of the chunk's keys,
//           added into the unit histogram H1
//   level2  finds the H1 bin d1 that holds T, histograms the next 11 bits of the
//           chunk's keys in bin d1, adds into H2
//   level3  finds d1 and d2, histograms the low 10 bits of the chunk's keys with
//           prefix (d1, d2) into H3; stores the chunk's count of keys above that
//           prefix and the suffix sums of its own level-3 histogram
//   write   finds T and the ties to take; every chunk's count above T and at T
//           follows from the stored per-chunk figures, so each work-group derives
//           its output offset from the chunks before it and compacts its chunk in
//           order (ballots give in-wave prefix counts); chunk 0 also writes the
//           window, the padding and the count
//
// The unit histograms and a per-unit counter live in the workspace, which must be
// zero when a call starts: the last write work-group of each unit clears them again.
// Every figure is an integer count, so the result does not depend on scheduling.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

constexpr int kB1 = 2048;           // key bits [21, 32)
constexpr int kB2 = 2048;           // key bits [10, 21)
constexpr int kB3 = 1024;           // key bits [0, 10)
constexpr int kHistInts = kB1 + kB2 + kB3;
constexpr int kSfx = kB3 + 4;       // suffix sums [0, kB3] of one chunk, padded
constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
// Candidates per work-group of the chunked kernels: kThreads * KPT, KPT = 8 (2048) or,
// when the call has many chunks anyway, 32 (8192): fewer work-groups, each reading the
// unit histograms and scanning them once for four times as many keys.
constexpr int kKptSmall = 8;
constexpr int kKptLarge = 32;
constexpr int kCoreChunk = 2048;    // tokens per work-group of the core-mask kernel
constexpr int kCopies = 4;          // LDS histogram copies, picked by lane & 3

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                      // -0.0 == +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

struct UnitShape {
    int S, C, k_eff;
};

__device__ __forceinline__ UnitShape unit_shape(const int32_t *seq_lens, int b, int s_max, int k, int n_keep)
{
    UnitShape s;
    s.S = clamp_len(seq_lens, b, s_max);
    s.C = s.S - n_keep > 0 ? s.S - n_keep : 0;
    s.k_eff = k < s.C ? k : s.C;
    return s;
}

struct SelArgs {
    const float *scores;      // [units][s_max]
    const int32_t *seq_lens;
    int s_max, H, k, n_keep, cap;
    int n_chunks;
    int32_t *hist;            // [units][kHistInts]: H1, H2, H3 (zero between calls)
    int32_t *done;            // [units]: write work-groups past their histogram reads (zero between calls)
    int32_t *above12;         // [units][n_chunks]: chunk keys above prefix (d1, d2)
    int32_t *sfx3;            // [units][n_chunks][kSfx]: suffix sums of the chunk's H3 part
    int32_t *idx;             // [units][cap]
    int32_t *count;           // [units]
    const int32_t *mask;      // [units] or null: units with 0 are skipped by every kernel
    const int32_t *kpu;       // [units] or null: the unit's budget, clamped to [0, k]
};

// The unit's budget: its own entry of kpu (clamped to [0, k]) or k.
__device__ __forceinline__ int unit_budget(const SelArgs &a, int u)
{
    if (!a.kpu) return a.k;
    const int v = ld_uniform(a.kpu, u);
    return v < 0 ? 0 : (v > a.k ? a.k : v);
}

// Histogram increment with leader aggregation: the lanes whose bin equals the first
// active lane's bin add their count with one atomic (neighbouring tokens often share
// a bin); the others add into their own histogram copy.
__device__ __forceinline__ void hist_add(int *h_copy, int *h_lead, int bin)
{
    const int lane = kvc_tid() & (kWave - 1);
    const int lead = __builtin_amdgcn_readfirstlane(bin);
    const unsigned long long act = __ballot(1);
    const unsigned long long m = __ballot(bin == lead);
    if (bin == lead) {
        if (lane == __ffsll((long long)act) - 1) atomicAdd(&h_lead[lead], __popcll(m));
    } else {
        atomicAdd(&h_copy[bin], 1);
    }
}

__device__ __forceinline__ void lds_clear(int (*h)[kB1])
{
    for (int i = kvc_tid(); i < kCopies * kB1 / 4; i += kThreads)
        reinterpret_cast<int4 *>(&h[0][0])[i] = make_int4(0, 0, 0, 0);
}

// Adds the non-zero bins of the LDS histogram copies into the global histogram g.
template <int NB>
__device__ __forceinline__ void flush_hist(int (*h)[kB1], int32_t *g)
{
    for (int b = kvc_tid(); b < NB; b += kThreads) {
        int s = 0;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) s += h[c][b];
        if (s) atomicAdd(&g[b], s);
    }
}

struct Digit {
    int digit, above;
};

// Thread i owns bins NB-1-i*per down to NB-per-i*per of a histogram; c[p] receives
// the count of bin (NB-1-i*per) - p.  Two 16-byte loads per 8 bins.
template <int NB>
__device__ __forceinline__ void load_bins(const int32_t *__restrict__ g, int (&c)[NB / kThreads])
{
    constexpr int per = NB / kThreads;
    const int top = NB - 1 - (int)kvc_tid() * per;
    const int4 *g4 = reinterpret_cast<const int4 *>(g + top - per + 1);
#pragma unroll
    for (int v = 0; v < per / 4; ++v) {
        const int4 x = g4[v];                            // bins top-per+1+4v .. top-per+4+4v
        c[per - 1 - 4 * v] = x.x;
        c[per - 2 - 4 * v] = x.y;
        c[per - 3 - 4 * v] = x.z;
        c[per - 4 - 4 * v] = x.w;
    }
}

// The bin that holds the k_rem-th largest key (counting from the top bin) and the
// number of keys in the bins above it, from the counts load_bins gave every thread.
template <int NB>
__device__ __forceinline__ Digit find_digit(const int (&c)[NB / kThreads], int k_rem, int *scan, Digit *out)
{
    constexpr int per = NB / kThreads;
    const int top = NB - 1 - (int)kvc_tid() * per;
    int cnt = 0;
#pragma unroll
    for (int p = 0; p < per; ++p) cnt += c[p];
    int tot;
    int above = block_exclusive_scan(cnt, scan, &tot);
#pragma unroll
    for (int p = 0; p < per; ++p) {
        if (above < k_rem && above + c[p] >= k_rem) *out = Digit{top - p, above};
        above += c[p];
    }
    __syncthreads();
    const Digit d = *out;
    __syncthreads();
    return d;
}

// A chunk is KPT * kThreads consecutive candidates; thread i holds keys
// t0 + i + q * kThreads (q < KPT), loaded once.  Slots past the chunk's end hold key 0
// and are masked by `valid`.
template <int KPT>
struct ChunkKeys {
    uint32_t key[KPT];
    int t0, t1;
};

template <int KPT>
__device__ __forceinline__ void load_chunk(const float *__restrict__ sc, int t0, int t1, ChunkKeys<KPT> &ck)
{
    ck.t0 = t0;
    ck.t1 = t1;
    float v[KPT];
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        const int t = t0 + (int)kvc_tid() + q * kThreads;
        v[q] = t < t1 ? sc[t] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < KPT; ++q) ck.key[q] = order_key(v[q]);
}

template <int KPT>
__device__ __forceinline__ bool chunk_valid(const ChunkKeys<KPT> &ck, int q)
{
    return ck.t0 + (int)kvc_tid() + q * kThreads < ck.t1;
}

// ------------------------------------------------------------------------------ kernels
// The work-group's unit and chunk; false when the chunk has nothing to histogram.
template <int KPT>
__device__ __forceinline__ bool chunk_of(const SelArgs &a, UnitShape &us, int &t0, int &t1)
{
    constexpr int kChunk = KPT * kThreads;
    us = unit_shape(a.seq_lens, (int)kvc_bid_y() / a.H, a.s_max, unit_budget(a, kvc_bid_y()), a.n_keep);
    t0 = (int)kvc_bid_x() * kChunk;
    t1 = min(us.C, t0 + kChunk);
    if (a.mask && !ld_uniform(a.mask, kvc_bid_y())) return false;
    return us.k_eff > 0 && us.k_eff < us.C && t0 < us.C;
}

template <int KPT>
__global__ __launch_bounds__(kThreads) void sel_level1_kernel(SelArgs a)
{
    __shared__ int h[kCopies][kB1];
    const int u = kvc_bid_y();
    UnitShape us;
    int t0, t1;
    if (!chunk_of<KPT>(a, us, t0, t1)) return;
    ChunkKeys<KPT> ck;
    load_chunk(a.scores + (size_t)u * a.s_max, t0, t1, ck);
    lds_clear(h);
    __syncthreads();
    int *hc = h[kvc_tid() & (kCopies - 1)];
#pragma unroll
    for (int q = 0; q < KPT; ++q)
        if (chunk_valid(ck, q)) hist_add(hc, h[0], (int)(ck.key[q] >> 21));
    __syncthreads();
    flush_hist<kB1>(h, a.hist + (size_t)u * kHistInts);
}

template <int KPT>
__global__ __launch_bounds__(kThreads) void sel_level2_kernel(SelArgs a)
{
    __shared__ int h[kCopies][kB1];
    __shared__ int scan[16];
    __shared__ Digit dg;
    const int u = kvc_bid_y();
    UnitShape us;
    int t0, t1;
    if (!chunk_of<KPT>(a, us, t0, t1)) return;
    const int32_t *H = a.hist + (size_t)u * kHistInts;
    int c1[kB1 / kThreads];
    load_bins<kB1>(H, c1);
    ChunkKeys<KPT> ck;
    load_chunk(a.scores + (size_t)u * a.s_max, t0, t1, ck);
    lds_clear(h);
    const Digit d1 = find_digit<kB1>(c1, us.k_eff, scan, &dg);
    int *hc = h[kvc_tid() & (kCopies - 1)];
#pragma unroll
    for (int q = 0; q < KPT; ++q)
        if (chunk_valid(ck, q) && (int)(ck.key[q] >> 21) == d1.digit)
            hist_add(hc, h[0], (int)((ck.key[q] >> 10) & (kB2 - 1)));
    __syncthreads();
    flush_hist<kB2>(h, a.hist + (size_t)u * kHistInts + kB1);
}

template <int KPT>
__global__ __launch_bounds__(kThreads) void sel_level3_kernel(SelArgs a)
{
    __shared__ int h[kCopies][kB1];
    __shared__ int scan[16];
    __shared__ int wave_above[kWaves];
    __shared__ Digit dg;
    const int u = kvc_bid_y();
    const int j = kvc_bid_x();
    UnitShape us;
    int t0, t1;
    if (!chunk_of<KPT>(a, us, t0, t1)) return;
    const int tid = kvc_tid();
    const int lane = tid & (kWave - 1);
    const int32_t *H = a.hist + (size_t)u * kHistInts;
    int c1[kB1 / kThreads], c2[kB2 / kThreads];
    load_bins<kB1>(H, c1);
    load_bins<kB2>(H + kB1, c2);
    ChunkKeys<KPT> ck;
    load_chunk(a.scores + (size_t)u * a.s_max, t0, t1, ck);
    lds_clear(h);
    const Digit d1 = find_digit<kB1>(c1, us.k_eff, scan, &dg);
    const Digit d2 = find_digit<kB2>(c2, us.k_eff - d1.above, scan, &dg);
    const uint32_t pre2 = ((uint32_t)d1.digit << 11) | (uint32_t)d2.digit;
    int *hc = h[tid & (kCopies - 1)];
    int above = 0;                                       // keys whose top 22 bits exceed pre2
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        if (!chunk_valid(ck, q)) continue;
        const uint32_t k22 = ck.key[q] >> 10;
        above += k22 > pre2;
        if (k22 == pre2) hist_add(hc, h[0], (int)(ck.key[q] & (kB3 - 1)));
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) above += shfl_xor_i(above, o);
    if (lane == 0) wave_above[tid >> 6] = above;
    __syncthreads();
    flush_hist<kB3>(h, a.hist + (size_t)u * kHistInts + kB1 + kB2);
    // suffix sums of the chunk's own level-3 histogram: sfx[b] = keys with low bits >= b
    constexpr int per = kB3 / kThreads;
    const int top = kB3 - 1 - tid * per;
    int c[per], cnt = 0;
#pragma unroll
    for (int p = 0; p < per; ++p) {
        int s2 = 0;
#pragma unroll
        for (int cc = 0; cc < kCopies; ++cc) s2 += h[cc][top - p];
        c[p] = s2;
        cnt += s2;
    }
    int tot;
    int run = block_exclusive_scan(cnt, scan, &tot);
    int32_t *sfx = a.sfx3 + ((size_t)u * a.n_chunks + j) * kSfx;
#pragma unroll
    for (int p = 0; p < per; ++p) {
        run += c[p];
        sfx[top - p] = run;
    }
    if (tid == 0) {
        sfx[kB3] = 0;
        int s2 = 0;
        for (int w = 0; w < kWaves; ++w) s2 += wave_above[w];
        a.above12[(size_t)u * a.n_chunks + j] = s2;
    }
}

template <int KPT>
__global__ __launch_bounds__(kThreads) void sel_write_kernel(SelArgs a)
{
    constexpr int kChunk = KPT * kThreads;
    __shared__ int scan[16];
    __shared__ Digit dg;
    __shared__ int wave_gt[kWaves], wave_eq[kWaves];
    __shared__ int chunk_take, is_last;
    const int u = kvc_bid_y();
    const int j = kvc_bid_x();
    const int tid = kvc_tid();
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    if (a.mask && !ld_uniform(a.mask, u)) return;
    const UnitShape us = unit_shape(a.seq_lens, u / a.H, a.s_max, unit_budget(a, u), a.n_keep);
    int32_t *out = a.idx + (size_t)u * a.cap;
    if (j == 0) {
        // the always-kept trailing tokens, the -1 padding and the count
        const int nw = us.S - us.C;
        for (int i = tid; i < nw; i += kThreads) out[us.k_eff + i] = us.C + i;
        for (int i = us.k_eff + nw + tid; i < a.cap; i += kThreads) out[i] = -1;
        if (tid == 0) a.count[u] = us.k_eff + nw;
    }
    const int t0 = j * kChunk;
    if (us.k_eff == 0 || t0 >= us.C) return;
    const int t1 = min(us.C, t0 + kChunk);
    if (us.k_eff == us.C) {
        for (int t = t0 + tid; t < t1; t += kThreads) out[t] = t;
        return;
    }
    // wave w owns the contiguous quarter [w0, w0 + kChunk/4) of the chunk; lane l holds
    // keys w0 + l + 64 q
    const int w0 = t0 + wid * (kChunk / kWaves);
    const float *sc = a.scores + (size_t)u * a.s_max;
    const int32_t *H = a.hist + (size_t)u * kHistInts;
    int c1[kB1 / kThreads], c2[kB2 / kThreads], c3[kB3 / kThreads];
    load_bins<kB1>(H, c1);
    load_bins<kB2>(H + kB1, c2);
    load_bins<kB3>(H + kB1 + kB2, c3);
    uint32_t key[KPT];
    {
        float v[KPT];
#pragma unroll
        for (int q = 0; q < KPT; ++q) {
            const int t = w0 + lane + q * kWave;
            v[q] = t < t1 ? sc[t] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < KPT; ++q) key[q] = order_key(v[q]);
    }
    const Digit d1 = find_digit<kB1>(c1, us.k_eff, scan, &dg);
    const Digit d2 = find_digit<kB2>(c2, us.k_eff - d1.above, scan, &dg);
    const Digit d3 = find_digit<kB3>(c3, us.k_eff - d1.above - d2.above, scan, &dg);
    const uint32_t T = ((uint32_t)d1.digit << 21) | ((uint32_t)d2.digit << 10) | (uint32_t)d3.digit;
    const int ties = us.k_eff - d1.above - d2.above - d3.above;     // keys == T to take, lowest index first
    // the last of the unit's work-groups to get here (all others have read H) returns
    // the histograms and the counter to zero for the next call
    if (tid == 0) {
        const int n_wg = (us.C + kChunk - 1) / kChunk;
        is_last = atomicAdd(&a.done[u], 1) == n_wg - 1;
    }
    __syncthreads();
    if (is_last) {
        int4 *h4 = reinterpret_cast<int4 *>(a.hist + (size_t)u * kHistInts);
        for (int i = tid; i < kHistInts / 4; i += kThreads) h4[i] = make_int4(0, 0, 0, 0);
        if (tid == 0) a.done[u] = 0;
    }
    __syncthreads();

    // output offset of this chunk: the chunks before it contribute their keys above T
    // and, lowest chunk first, their keys equal to T until `ties` are taken.  Thread i
    // of each block of kThreads chunks holds one chunk.
    int base = 0, eq_run = 0;
    for (int jb = 0; jb <= j; jb += kThreads) {
        const int jj = jb + tid;
        int gt = 0, eq = 0;
        if (jj <= j) {
            const int32_t *sfx = a.sfx3 + ((size_t)u * a.n_chunks + jj) * kSfx;
            const int s_hi = sfx[d3.digit + 1], s_at = sfx[d3.digit];
            gt = a.above12[(size_t)u * a.n_chunks + jj] + s_hi;
            eq = s_at - s_hi;
        }
        int eq_tot;
        const int eq_before = eq_run + block_exclusive_scan(eq, scan, &eq_tot);
        int take = ties - eq_before;
        take = take < 0 ? 0 : (take > eq ? eq : take);
        if (jj == j) {
            chunk_take = take;
        }
        int sel_tot;
        block_exclusive_scan(jj < j ? gt + take : 0, scan, &sel_tot);
        base += sel_tot;
        eq_run += eq_tot;
    }
    __syncthreads();
    const int take_j = chunk_take;

    // ordered compaction: per-wave counts, then ballots give in-wave prefix counts
    int gt = 0, eq = 0;
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        const bool ok = w0 + lane + q * kWave < t1;
        gt += ok && key[q] > T;
        eq += ok && key[q] == T;
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        gt += shfl_xor_i(gt, o);
        eq += shfl_xor_i(eq, o);
    }
    if (lane == 0) {
        wave_gt[wid] = gt;
        wave_eq[wid] = eq;
    }
    __syncthreads();
    int pos = base, eq_seen = 0;
    for (int w = 0; w < wid; ++w) {
        int take = take_j - eq_seen;
        take = take < 0 ? 0 : (take > wave_eq[w] ? wave_eq[w] : take);
        pos += wave_gt[w] + take;
        eq_seen += wave_eq[w];
    }
    const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int q = 0; q < KPT; ++q) {
        const int t = w0 + lane + q * kWave;
        const bool ok = t < t1;
        const bool is_gt = ok && key[q] > T;
        const bool is_eq = ok && key[q] == T;
        const unsigned long long m_eq = __ballot(is_eq);
        const int rank = eq_seen + __popcll(m_eq & below);
        const bool sel = is_gt || (is_eq && rank < take_j);
        const unsigned long long m_sel = __ballot(sel);
        const int p = pos + __popcll(m_sel & below);
        if (sel && p < us.k_eff) out[p] = t;                     // never past the budget
        pos += __popcll(m_sel);
        eq_seen += __popcll(m_eq);
    }
}

// ------------------------------------------------------------- one work-group per unit
// When a unit has at most 32768 candidates and there are enough units to occupy the
// chip, one work-group of 512 threads holds all of a unit's candidates in registers
// (16 bytes per load, every load in flight at once) and runs the three radix levels
// and the ordered write in LDS: one launch, every key read once.  (A CU keeps only so
// many loads in flight, so with few units the chunked kernels, which spread a unit
// over many CUs, finish first.)  The levels, the tie rule and the output are those of
// the chunked kernels above.
constexpr int kUnitThreads = 512;

// Bin of the k_rem-th largest key of an LDS histogram (summed over its first NC
// copies) and the number of keys above that bin; thread i owns bins NB-1-i*per down to
// NB-per-i*per.
template <int NB, int NC>
__device__ __forceinline__ Digit unit_digit(int (*h)[kB1], int k_rem, int *scan, Digit *out)
{
    constexpr int per = NB / kUnitThreads;
    const int top = NB - 1 - (int)kvc_tid() * per;
    int c[per], cnt = 0;
#pragma unroll
    for (int p = 0; p < per; ++p) {
        int s = 0;
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) s += h[cc][top - p];
        c[p] = s;
        cnt += s;
    }
    int tot;
    int above = block_exclusive_scan(cnt, scan, &tot);
#pragma unroll
    for (int p = 0; p < per; ++p) {
        if (above < k_rem && above + c[p] >= k_rem) *out = Digit{top - p, above};
        above += c[p];
    }
    __syncthreads();
    const Digit d = *out;
    // the histogram is free again: clear the copy the next levels use
    for (int i = kvc_tid(); i < kB1 / 4; i += kUnitThreads) reinterpret_cast<int4 *>(&h[0][0])[i] = make_int4(0, 0, 0, 0);
    __syncthreads();
    return d;
}

// Thread i holds the K = 4 NQ consecutive candidates [K i, K i + K), so one block
// scan orders the write.  VEC: rows of a multiple of 4 floats, 16-byte loads.
template <int NQ, bool VEC>
__global__ __launch_bounds__(kUnitThreads) void sel_unit_kernel(SelArgs a)
{
    constexpr int K = 4 * NQ;
    __shared__ int h[kCopies][kB1];
    __shared__ int scan[16];
    __shared__ Digit dg;
    const int u = kvc_bid_x();
    const int tid = kvc_tid();
    if (a.mask && !ld_uniform(a.mask, u)) return;
    const UnitShape us = unit_shape(a.seq_lens, u / a.H, a.s_max, unit_budget(a, u), a.n_keep);
    int32_t *out = a.idx + (size_t)u * a.cap;
    // the always-kept trailing tokens, the -1 padding and the count
    const int nw = us.S - us.C;
    for (int i = tid; i < nw; i += kUnitThreads) out[us.k_eff + i] = us.C + i;
    for (int i = us.k_eff + nw + tid; i < a.cap; i += kUnitThreads) out[i] = -1;
    if (tid == 0) a.count[u] = us.k_eff + nw;
    if (us.k_eff == 0) return;
    if (us.k_eff == us.C) {
        for (int t = tid; t < us.C; t += kUnitThreads) out[t] = t;
        return;
    }
    const float *sc = a.scores + (size_t)u * a.s_max;
    const int t0 = K * tid;
    uint32_t key[K];
    {
        float v[K];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int t = t0 + 4 * q;
            if constexpr (VEC) {
                // t < C <= s_max and s_max % 4 == 0: the whole vector is inside the row
                const float4 x = t < us.C ? *(const float4 *)(sc + t) : make_float4(0.f, 0.f, 0.f, 0.f);
                v[4 * q] = x.x;
                v[4 * q + 1] = x.y;
                v[4 * q + 2] = x.z;
                v[4 * q + 3] = x.w;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * q + e] = t + e < us.C ? sc[t + e] : 0.f;
            }
        }
        // past the candidates the key is 0, below every key of a non-NaN score: the
        // histograms may count those slots, since the k_eff-th largest key (k_eff < C)
        // and the counts above its bins do not change; the write checks validity
#pragma unroll
        for (int i = 0; i < K; ++i) key[i] = t0 + i < us.C ? order_key(v[i]) : 0u;
    }
    for (int i = tid; i < kCopies * kB1 / 4; i += kUnitThreads)
        reinterpret_cast<int4 *>(&h[0][0])[i] = make_int4(0, 0, 0, 0);
    __syncthreads();
    int *hc = h[tid & (kCopies - 1)];

    // level 1: key bits [21, 32)
#pragma unroll
    for (int i = 0; i < K; ++i) hist_add(hc, h[0], (int)(key[i] >> 21));
    __syncthreads();
    const Digit d1 = unit_digit<kB1, kCopies>(h, us.k_eff, scan, &dg);
    // level 2: bits [10, 21) of the keys in bin d1.  Those spread over many bins, so
    // plain LDS atomics into one copy beat the wave-level aggregation here.
#pragma unroll
    for (int i = 0; i < K; ++i)
        if ((int)(key[i] >> 21) == d1.digit) atomicAdd(&h[0][(key[i] >> 10) & (kB2 - 1)], 1);
    __syncthreads();
    const Digit d2 = unit_digit<kB2, 1>(h, us.k_eff - d1.above, scan, &dg);
    // level 3: bits [0, 10) of the keys with prefix (d1, d2)
    const uint32_t pre2 = ((uint32_t)d1.digit << 11) | (uint32_t)d2.digit;
#pragma unroll
    for (int i = 0; i < K; ++i)
        if ((key[i] >> 10) == pre2) atomicAdd(&h[0][key[i] & (kB3 - 1)], 1);
    __syncthreads();
    const Digit d3 = unit_digit<kB3, 1>(h, us.k_eff - d1.above - d2.above, scan, &dg);
    const uint32_t T = (pre2 << 10) | (uint32_t)d3.digit;
    const int ties = us.k_eff - d1.above - d2.above - d3.above;     // keys == T to take, lowest index first

    // ordered write: one block scan of (keys > T, keys == T) per thread
    int gt = 0, eq = 0;
#pragma unroll
    for (int i = 0; i < K; ++i) {
        const bool ok = t0 + i < us.C;
        gt += ok && key[i] > T;
        eq += ok && key[i] == T;
    }
    int tot;
    const int before = block_exclusive_scan(gt | (eq << 16), scan, &tot);
    int eq_before = before >> 16;
    int pos = (before & 0xffff) + min(ties, eq_before);
#pragma unroll
    for (int i = 0; i < K; ++i) {
        if (t0 + i >= us.C) break;
        bool sel = key[i] > T;
        if (key[i] == T) sel = eq_before++ < ties;
        if (sel) {
            if (pos < us.k_eff) out[pos] = t0 + i;                    // never past the budget
            ++pos;
        }
    }
}

// TSP score: float sum over KV heads in head order (one selection per sequence).
__global__ __launch_bounds__(256) void head_sum_kernel(const float *__restrict__ scores, int n_kv, int s_max,
                                                       float *__restrict__ out)
{
    const int b = kvc_bid_y();
    const int t = kvc_bid_x() * 256 + kvc_tid();
    if (t >= s_max) return;
    const float *p = scores + (size_t)b * n_kv * s_max + t;
    // eight heads' scores requested together, then added in head order
    float s = 0.f;
    int g0 = 0;
    for (; g0 + 8 <= n_kv; g0 += 8) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = p[(size_t)(g0 + i) * s_max];
#pragma unroll
        for (int i = 0; i < 8; ++i) s += v[i];
    }
    for (; g0 < n_kv; ++g0) s += p[(size_t)g0 * s_max];
    out[(size_t)b * s_max + t] = s;
}

// ---------------------------------------------------------------- role-based retention
// CASK's core tokens are always kept and the budget applies to the scratch tokens: a
// core candidate's score becomes +inf (the largest key), and the unit's budget grows
// by its number of core candidates, so the ordinary selection of k + |core| keys takes
// every core token plus the best k scratch tokens.  One work-group per (2048-token
// chunk, unit) writes the masked scores and counts the chunk's core candidates.
__global__ __launch_bounds__(kThreads) void core_scores_kernel(const float *__restrict__ scores,
                                                               const uint8_t *__restrict__ core,
                                                               const int32_t *__restrict__ seq_lens, int H,
                                                               int s_max, int n_keep, int n_chunks,
                                                               const int32_t *__restrict__ mask,
                                                               float *__restrict__ masked,
                                                               int32_t *__restrict__ chunk_core)
{
    __shared__ int wave_n[kWaves];
    const int u = kvc_bid_y();
    if (mask && !ld_uniform(mask, u)) return;
    const int b = u / H;
    const int S = clamp_len(seq_lens, b, s_max);
    const int C = S - n_keep > 0 ? S - n_keep : 0;
    const int t0 = kvc_bid_x() * kCoreChunk;
    int n = 0;
    // every load of the thread's kCoreChunk / kThreads tokens goes out before the first
    // use (indices clamped into the row; the stores check the range)
    constexpr int kPer = kCoreChunk / kThreads;
    float sc[kPer];
    uint8_t cr[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int t = min(t0 + (int)kvc_tid() + i * kThreads, s_max - 1);
        sc[i] = scores[(size_t)u * s_max + t];
        cr[i] = core[(size_t)b * s_max + t];
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int t = t0 + (int)kvc_tid() + i * kThreads;
        if (t >= s_max) break;
        const bool c = t < C && cr[i] != 0;
        n += c;
        masked[(size_t)u * s_max + t] = c ? INFINITY : sc[i];
    }
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) n += __shfl_xor(n, o, kWave);
    if ((kvc_tid() & (kWave - 1)) == 0) wave_n[kvc_tid() >> 6] = n;
    __syncthreads();
    if (kvc_tid() == 0) {
        int tot = 0;
        for (int w = 0; w < kWaves; ++w) tot += wave_n[w];
        chunk_core[(size_t)u * n_chunks + kvc_bid_x()] = tot;
    }
}

// budget[u] = k + min(|core candidates of u|, core_cap)
__global__ __launch_bounds__(256) void core_budget_kernel(const int32_t *__restrict__ chunk_core, int units,
                                                          int n_chunks, int k, int core_cap,
                                                          int32_t *__restrict__ budget)
{
    const int u = kvc_bid_x() * 256 + kvc_tid();
    if (u >= units) return;
    int n = 0;
    for (int j = 0; j < n_chunks; ++j) n += chunk_core[(size_t)u * n_chunks + j];
    budget[u] = k + (n < core_cap ? n : core_cap);
}

struct SelLayout {
    int kpt;                  // keys per thread of the chunked kernels
    int n_chunks;
    size_t sum_off, hist_off, done_off, above_off, sfx_off, bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The parts that must be zero when a call starts (counters, histograms) come first and
// depend only on the number of units, so calls with the same batch, n_kv and flags
// can share a workspace whatever their s_max, n_keep, k and lengths; the per-call
// scratch follows.
SelLayout sel_layout(int batch, int n_kv, int s_max, int n_keep, bool shared)
{
    SelLayout L;
    const long units = shared ? batch : (long)batch * n_kv;
    const long c_max = s_max - n_keep > 1 ? (long)s_max - n_keep : 1;
    const long big = kKptLarge * kThreads;
    L.kpt = units * ((c_max + big - 1) / big) >= 512 ? kKptLarge : kKptSmall;
    const long chunk = (long)L.kpt * kThreads;
    L.n_chunks = (int)((c_max + chunk - 1) / chunk);
    size_t off = 0;
    L.done_off = off;
    off += align256((size_t)units * sizeof(int32_t));
    L.hist_off = off;
    off += align256((size_t)units * kHistInts * sizeof(int32_t));
    L.sum_off = off;
    if (shared) off += align256((size_t)batch * s_max * sizeof(float));
    L.above_off = off;
    off += align256((size_t)units * L.n_chunks * sizeof(int32_t));
    L.sfx_off = off;
    off += align256((size_t)units * L.n_chunks * kSfx * sizeof(int32_t));
    L.bytes = off;
    return L;
}

static_assert((kKptSmall * kThreads) % (kWaves * kWave) == 0 && (kKptLarge * kThreads) % (kWaves * kWave) == 0,
              "chunk shape");
static_assert(kHistInts % 4 == 0 && kSfx % 4 == 0 && kB1 % 4 == 0, "16-byte aligned histogram parts");

}  // namespace

size_t select_ws_bytes(int batch, int n_kv, int s_max, int n_keep, bool shared)
{
    return sel_layout(batch, n_kv, s_max, n_keep, shared).bytes;
}

// [selection workspace][masked scores][per-chunk core counts][budgets]
struct CoreLayout {
    size_t masked_off, chunk_off, budget_off, bytes;
    int n_chunks;
};

static CoreLayout core_layout(int batch, int n_kv, int s_max, int n_keep)
{
    CoreLayout L;
    const size_t units = (size_t)batch * n_kv;
    L.n_chunks = (s_max + kCoreChunk - 1) / kCoreChunk;
    size_t off = align256(select_ws_bytes(batch, n_kv, s_max, n_keep, false));
    L.masked_off = off;
    off += align256(units * s_max * sizeof(float));
    L.chunk_off = off;
    off += align256(units * L.n_chunks * sizeof(int32_t));
    L.budget_off = off;
    off += align256(units * sizeof(int32_t));
    L.bytes = off;
    return L;
}

size_t select_core_ws_bytes(int batch, int n_kv, int s_max, int n_keep)
{
    return core_layout(batch, n_kv, s_max, n_keep).bytes;
}

hipError_t launch_select_core(int batch, int n_kv, int s_max, const int32_t *seq_lens, const float *scores,
                              const uint8_t *core, int k, int core_cap, int n_keep, int32_t *idx, int32_t *count,
                              const int32_t *unit_mask, void *ws, const DeviceInfo &dev, hipStream_t stream)
{
    const CoreLayout L = core_layout(batch, n_kv, s_max, n_keep);
    char *w = (char *)ws;
    float *masked = (float *)(w + L.masked_off);
    int32_t *chunk_core = (int32_t *)(w + L.chunk_off);
    int32_t *budget = (int32_t *)(w + L.budget_off);
    const int units = batch * n_kv;
    hipLaunchKernelGGL(core_scores_kernel, dim3(L.n_chunks, units), dim3(kThreads), 0, stream, scores, core,
                       seq_lens, n_kv, s_max, n_keep, L.n_chunks, unit_mask, masked, chunk_core);
    hipLaunchKernelGGL(core_budget_kernel, dim3((units + 255) / 256), dim3(256), 0, stream, chunk_core, units,
                       L.n_chunks, k, core_cap, budget);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_select(batch, n_kv, s_max, seq_lens, masked, k + core_cap, n_keep, false, idx, count, unit_mask,
                         budget, ws, dev, stream);
}

hipError_t launch_select(int batch, int n_kv, int s_max, const int32_t *seq_lens, const float *scores,
                         int k, int n_keep, bool shared, int32_t *idx, int32_t *count,
                         const int32_t *unit_mask, const int32_t *k_per_unit, void *ws, const DeviceInfo &dev,
                         hipStream_t stream)
{
    const SelLayout L = sel_layout(batch, n_kv, s_max, n_keep, shared);
    char *w = (char *)ws;
    SelArgs a;
    a.scores = scores;
    a.H = n_kv;
    if (shared) {
        float *sum = (float *)(w + L.sum_off);
        hipLaunchKernelGGL(head_sum_kernel, dim3((s_max + 255) / 256, batch), dim3(256), 0, stream, scores,
                           n_kv, s_max, sum);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        a.scores = sum;
        a.H = 1;
    }
    const int units = batch * a.H;
    a.seq_lens = seq_lens;
    a.s_max = s_max;
    a.k = k;
    a.n_keep = n_keep;
    a.cap = k + n_keep;
    a.n_chunks = L.n_chunks;
    a.hist = (int32_t *)(w + L.hist_off);
    a.done = (int32_t *)(w + L.done_off);
    a.above12 = (int32_t *)(w + L.above_off);
    a.sfx3 = (int32_t *)(w + L.sfx_off);
    a.idx = idx;
    a.count = count;
    a.mask = shared ? nullptr : unit_mask;
    a.kpu = k_per_unit;

    const long c_max = (long)s_max - n_keep;
    if (c_max <= 32768 && units >= dev.cus / 2) {
        // every unit's candidates fit one work-group's registers, and the units fill the chip
        const bool vec = s_max % 4 == 0 && ((uintptr_t)a.scores & 15) == 0;
        const dim3 g1(units), b1(kUnitThreads);
        if (c_max <= 8192) {
            if (vec) hipLaunchKernelGGL((sel_unit_kernel<4, true>), g1, b1, 0, stream, a);
            else hipLaunchKernelGGL((sel_unit_kernel<4, false>), g1, b1, 0, stream, a);
        } else if (c_max <= 16384) {
            if (vec) hipLaunchKernelGGL((sel_unit_kernel<8, true>), g1, b1, 0, stream, a);
            else hipLaunchKernelGGL((sel_unit_kernel<8, false>), g1, b1, 0, stream, a);
        } else {
            if (vec) hipLaunchKernelGGL((sel_unit_kernel<16, true>), g1, b1, 0, stream, a);
            else hipLaunchKernelGGL((sel_unit_kernel<16, false>), g1, b1, 0, stream, a);
        }
        return hipGetLastError();
    }
    const dim3 grid(L.n_chunks, units);
    if (L.kpt == kKptLarge) {
        hipLaunchKernelGGL(sel_level1_kernel<kKptLarge>, grid, dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(sel_level2_kernel<kKptLarge>, grid, dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(sel_level3_kernel<kKptLarge>, grid, dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(sel_write_kernel<kKptLarge>, grid, dim3(kThreads), 0, stream, a);
    } else {
        hipLaunchKernelGGL(sel_level1_kernel<kKptSmall>, grid, dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(sel_level2_kernel<kKptSmall>, grid, dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(sel_level3_kernel<kKptSmall>, grid, dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(sel_write_kernel<kKptSmall>, grid, dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
}

}  // namespace kvc
