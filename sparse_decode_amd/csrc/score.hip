// score.hip -- observation-window saliency of every cached token (FastKV section
// 2.A: token saliency from the attention of the recent-window tokens; Tutorial
// "Variantes de l'attention et compression du cache KV", section "Compresser un
// cache existant": score prompt positions from an observation window), with the
// causal alignment of the window rows (same page, section "Quand la reutilisation
// est-elle exacte ?": row i of the last w tokens sees keys up to S - w + i).
//
// For KV head g of sequence b the R = (n_h/n_kv) * w window rows of the group's
// query heads are scored against every key; each row is softmax-normalised over
// the keys it sees and the probabilities are summed per key over all R rows.  The
// row normalisers (max M_r, sum L_r) depend on every key, so the score takes two
// passes over K:
//   pass 1  logits -> per-row (max, sum of exp) for one chunk of tokens (for one
//           block of 16 rows: per 256-token block of the chunk)
//   merge   partials -> (M_r, 1/L_r) per row, in token order, in double
//   pass 2  logits again -> sum_r exp(x - M_r) / L_r per token
//   pool    centred max over the candidate region
// All units go into one launch of each kernel.  Both passes stream K from HBM; on
// this chip the second read is not served faster by the MALL, so nothing is gained
// by grouping units to fit it.
//
// The bf16 path computes logits with v_mfma_f32_16x16x32_bf16 (16 tokens x 16 rows
// per tile).  K is staged through LDS with coalesced 16-byte loads, a register ring
// keeping several stages in flight; each wave holds its rows' Q^T operands in
// registers for the whole chunk.  Pass 1 keeps the row statistics in-lane (tokens
// on the M side give each lane one row); pass 2 sums over rows across lanes with a
// transposed butterfly of DPP lane exchanges.  Both passes evaluate exactly the
// same MFMA sequence, so their logits are identical.  Exponentials use exp2 with
// scale * log2(e) folded into one FMA.
#include <mutex>

#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

// ====================================================================================
// Portable VALU path: any R, d_h in {64, 128}, fp32 or bf16.  Logits are stored.
// ====================================================================================
constexpr int kGenThreads = 256;
constexpr int kGenRowsLds = 64;   // Q rows staged in LDS at a time

template <bool BF16, int D>
__device__ __forceinline__ void load_row_f32(const void *base, size_t row, float *dst)
{
    if (BF16) {
        const u32x4 *p = (const u32x4 *)((const uint16_t *)base + row * D);
#pragma unroll
        for (int v = 0; v < D / 8; ++v) {
            const u32x4 x = p[v];
            dst[8 * v + 0] = bf16_lo(x.x); dst[8 * v + 1] = bf16_hi(x.x);
            dst[8 * v + 2] = bf16_lo(x.y); dst[8 * v + 3] = bf16_hi(x.y);
            dst[8 * v + 4] = bf16_lo(x.z); dst[8 * v + 5] = bf16_hi(x.z);
            dst[8 * v + 6] = bf16_lo(x.w); dst[8 * v + 7] = bf16_hi(x.w);
        }
    } else {
        const float4 *p = (const float4 *)((const float *)base + row * D);
#pragma unroll
        for (int v = 0; v < D / 4; ++v) {
            const float4 x = p[v];
            dst[4 * v + 0] = x.x; dst[4 * v + 1] = x.y; dst[4 * v + 2] = x.z; dst[4 * v + 3] = x.w;
        }
    }
}

// logits[u][rr][t] = scale * <q_rr, k_t> for visible t, -inf otherwise.
template <bool BF16, int D>
__global__ __launch_bounds__(kGenThreads) void gen_logits_kernel(
    const void *__restrict__ q_win, const void *__restrict__ k, const int32_t *__restrict__ seq_lens,
    int s_max, int n_h, int n_kv, int w, int wic, int R, int unit0, float scale, const int32_t *__restrict__ mask,
    float *__restrict__ logits)
{
    __shared__ float qs[kGenRowsLds][D];
    const int u = unit0 + kvc_bid_y();
    if (mask && !ld_uniform(mask, u)) return;
    const int b = u / n_kv;
    const int g = u - b * n_kv;
    const int r = n_h / n_kv;
    const int S = clamp_len(seq_lens, b, s_max);
    const int t = kvc_bid_x() * kGenThreads + kvc_tid();
    float kr[D];
    if (t < S) load_row_f32<BF16, D>(k, (size_t)u * s_max + t, kr);
    const size_t qrow0 = (size_t)(b * n_h + g * r) * w;     // the R rows are contiguous
    float *lg = logits + (size_t)kvc_bid_y() * R * s_max;
    for (int r0 = 0; r0 < R; r0 += kGenRowsLds) {
        const int nr = min(kGenRowsLds, R - r0);
        __syncthreads();
        for (int x = kvc_tid(); x < nr * D; x += kGenThreads) {
            const int rr = x / D, d = x - rr * D;
            const size_t off = (qrow0 + r0 + rr) * D + d;
            qs[rr][d] = BF16 ? bf16_to_f32(((const uint16_t *)q_win)[off]) : ((const float *)q_win)[off];
        }
        __syncthreads();
        if (t >= s_max) continue;
        for (int rr = 0; rr < nr; ++rr) {
            const int row = r0 + rr;
            const int i = row % w;
            const int last = wic ? min(S - w + i, S - 1) : S - 1;
            float x = -INFINITY;
            if (t <= last) {
                float acc = 0.f;
#pragma unroll
                for (int d = 0; d < D; ++d) acc = fmaf(qs[rr][d], kr[d], acc);
                x = acc * scale;
            }
            lg[(size_t)row * s_max + t] = x;
        }
    }
}

// Per row: M = max logit, L = sum exp(x - M); fin = (-M*log2e, 1/L), or (0, 0) when
// the row sees no key.
__global__ __launch_bounds__(kGenThreads) void gen_rowstats_kernel(const float *__restrict__ logits, int s_max,
                                                                   int R, const int32_t *__restrict__ mask,
                                                                   float2 *__restrict__ fin)
{
    if (mask && !ld_uniform(mask, kvc_bid_y())) return;
    __shared__ float red_m[kGenThreads / kWave];
    __shared__ double red_l[kGenThreads / kWave];
    const int row = kvc_bid_x();
    const int ul = kvc_bid_y();
    const float *lg = logits + ((size_t)ul * R + row) * s_max;
    float m = -INFINITY;
    for (int t = kvc_tid(); t < s_max; t += kGenThreads) m = fmaxf(m, lg[t]);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) m = fmaxf(m, shfl_xor_f(m, o));
    if ((kvc_tid() & 63) == 0) red_m[kvc_tid() >> 6] = m;
    __syncthreads();
    m = red_m[0];
    for (int i = 1; i < kGenThreads / kWave; ++i) m = fmaxf(m, red_m[i]);
    if (m == -INFINITY) {
        if (kvc_tid() == 0) fin[(size_t)ul * R + row] = make_float2(0.f, 0.f);
        return;
    }
    const float nmc = -m * kLog2e;
    double sd = 0.0;
    for (int t = kvc_tid(); t < s_max; t += kGenThreads) sd += (double)fast_exp2(fmaf(lg[t], kLog2e, nmc));
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) sd += __shfl_xor(sd, o, kWave);
    if ((kvc_tid() & 63) == 0) red_l[kvc_tid() >> 6] = sd;
    __syncthreads();
    if (kvc_tid() == 0) {
        double L = 0.0;
        for (int i = 0; i < kGenThreads / kWave; ++i) L += red_l[i];
        fin[(size_t)ul * R + row] = make_float2(nmc, (float)(1.0 / L));
    }
}

// raw[t] = sum_rows exp(x - M) / L, 0 beyond S_b.
__global__ __launch_bounds__(kGenThreads) void gen_probsum_kernel(const float *__restrict__ logits,
                                                                  const float2 *__restrict__ fin,
                                                                  const int32_t *__restrict__ seq_lens,
                                                                  int s_max, int n_kv, int R, int unit0,
                                                                  const int32_t *__restrict__ mask,
                                                                  float *__restrict__ raw)
{
    const int ul = kvc_bid_y();
    const int u = unit0 + ul;
    if (mask && !ld_uniform(mask, u)) return;
    const int S = clamp_len(seq_lens, u / n_kv, s_max);
    const int t = kvc_bid_x() * kGenThreads + kvc_tid();
    if (t >= s_max) return;
    float acc = 0.f;
    if (t < S) {
        const float *lg = logits + (size_t)ul * R * s_max + t;
        for (int row = 0; row < R; ++row) {
            const float2 f = fin[(size_t)ul * R + row];
            const float e = fast_exp2(fmaf(lg[(size_t)row * s_max], kLog2e, f.x));
            acc = fmaf(e, f.y, acc);
        }
    }
    raw[(size_t)u * s_max + t] = acc;
}

// ====================================================================================
// Pooling: centred max of raw over the candidate region (shared by both paths)
// ====================================================================================
constexpr int kPoolThreads = 256;
constexpr int kPoolTile = 1024;     // tokens per work-group, 4 per thread
constexpr int kMaxHalf = 31;        // pool kernels up to 63

__device__ __forceinline__ float pool_at(const float *tile, int base, int t, int half, int C, int S)
{
    if (t < C) {
        const int lo = t - half < 0 ? 0 : t - half;
        const int hi = t + half > C - 1 ? C - 1 : t + half;
        float v = tile[lo - base];
        for (int x = lo + 1; x <= hi; ++x) v = fmaxf(v, tile[x - base]);
        return v;
    }
    return t < S ? tile[t - base] : 0.f;
}

// The pooled outputs of one tile: tile[i] holds raw[base + i] for the kPoolTile tokens
// from t0 and their halo; this thread's 4 tokens start at t = t0 + 4 tid.
template <bool VEC, int HALF>
__device__ __forceinline__ void pool_tile(const float *tile, int base, int t, int s_max, int half, int C, int S,
                                          float *__restrict__ out)
{
    if (t >= s_max) return;
    float o[4];
    if (HALF >= 0 && t - HALF >= 0 && t + 3 + HALF <= C - 1) {
        // the 4 windows are whole: [t - HALF, t + 3 + HALF] inside [0, C)
        constexpr int NW = HALF >= 0 ? 4 + 2 * HALF : 1;
        float win[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) win[i] = tile[t - HALF + i - base];
#pragma unroll
        for (int k = 0; k < 4; ++k) {                      // token t + k: win[k .. k + 2 HALF]
            float v = win[k];
#pragma unroll
            for (int i = k + 1; i <= k + 2 * HALF; ++i) v = fmaxf(v, win[i]);
            o[k] = v;
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = pool_at(tile, base, t + k, half, C, S);
    }
    if constexpr (VEC) {
        *(float4 *)(out + t) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (t + k < s_max) out[t + k] = o[k];
    }
}

// LDS tile of the pooling kernels: 2 kMaxHalf + 2 slots (left halo, then 16-byte
// alignment), the body, the right halo
constexpr int kPoolLds = 2 * kMaxHalf + 2 + kPoolTile + kMaxHalf + 1;

// One work-group per kPoolTile tokens of a unit: the tile and its halo are staged in
// LDS once (coalesced), then each output is the max over its window.  Each thread
// owns 4 consecutive tokens (one 16-byte load and store when a row is a multiple of 4
// floats).  HALF >= 0 is the half-width known at compile time: where the 4 windows
// lie inside [0, C), the thread reads the 4 + 2 HALF values once into registers and
// takes the 4 maxima there; elsewhere, and for HALF < 0, every window is walked.
template <bool VEC, int HALF>
__global__ __launch_bounds__(kPoolThreads) void pool_kernel(const float *__restrict__ raw,
                                                            const int32_t *__restrict__ seq_lens, int s_max,
                                                            int n_kv, int n_keep, int half,
                                                            const int32_t *__restrict__ mask,
                                                            float *__restrict__ pooled, int32_t *reset, int n_reset)
{
    // the single-pass kernels' counters go back to zero here, after their last use, and
    // the tag word that follows them advances to this call's tag
    if (reset && kvc_bid_x() == 0 && kvc_bid_y() == 0) {
        for (int i = kvc_tid(); i < n_reset; i += kPoolThreads) reset[i] = 0;
        if (kvc_tid() == 0) reset[n_reset] += 1;
    }
    __shared__ __attribute__((aligned(16))) float tile[kPoolLds];
    if constexpr (HALF >= 0) half = HALF;
    const int u = kvc_bid_y();
    if (mask && !ld_uniform(mask, u)) return;
    const int S = clamp_len(seq_lens, u / n_kv, s_max);
    const int C = S - n_keep > 0 ? S - n_keep : 0;
    const int t0 = kvc_bid_x() * kPoolTile;
    const float *rw = raw + (size_t)u * s_max;
    const int tid = kvc_tid();
    const int base = t0 - (2 * kMaxHalf + 2);               // tile[i] holds raw[base + i]
    float *body = tile + 2 * kMaxHalf + 2;                  // 16-byte aligned: 64 floats in
    const int t = t0 + 4 * tid;                             // this thread's 4 tokens
    if constexpr (VEC) {
        *(float4 *)(body + 4 * tid) = t < s_max ? *(const float4 *)(rw + t) : make_float4(0.f, 0.f, 0.f, 0.f);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) body[4 * tid + k] = t + k < s_max ? rw[t + k] : 0.f;
    }
    if (tid < half) {
        const int th = t0 - half + tid;
        tile[th - base] = th >= 0 ? rw[th] : 0.f;
    } else if (tid < 2 * half) {
        const int th = t0 + kPoolTile + (tid - half);
        tile[th - base] = th < s_max ? rw[th] : 0.f;
    }
    __syncthreads();
    pool_tile<VEC, HALF>(tile, base, t, s_max, half, C, S, pooled + (size_t)u * s_max);
}

template <bool VEC>
void launch_pool_vec(dim3 grid, const float *raw, const int32_t *seq_lens, int s_max, int n_kv, int n_keep, int half,
                     const int32_t *mask, float *pooled, int32_t *reset, int n_reset, hipStream_t stream)
{
    switch (half) {
    case 0: hipLaunchKernelGGL((pool_kernel<VEC, 0>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, reset, n_reset); break;
    case 1: hipLaunchKernelGGL((pool_kernel<VEC, 1>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, reset, n_reset); break;
    case 2: hipLaunchKernelGGL((pool_kernel<VEC, 2>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, reset, n_reset); break;
    case 3: hipLaunchKernelGGL((pool_kernel<VEC, 3>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, reset, n_reset); break;
    default: hipLaunchKernelGGL((pool_kernel<VEC, -1>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, reset, n_reset); break;
    }
}

void launch_pool(const float *raw, const int32_t *seq_lens, int s_max, int units, int n_kv, int n_keep, int half,
                 const int32_t *mask, float *pooled, int32_t *reset, int n_reset, hipStream_t stream)
{
    const dim3 grid((s_max + kPoolTile - 1) / kPoolTile, units);
    if (s_max % 4 == 0 && ((uintptr_t)raw & 15) == 0 && ((uintptr_t)pooled & 15) == 0)
        launch_pool_vec<true>(grid, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, reset, n_reset, stream);
    else
        launch_pool_vec<false>(grid, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, reset, n_reset, stream);
}

// ====================================================================================
// bf16 MFMA path
// ====================================================================================
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfThreads = 256;
constexpr int kStatBlock = 256;     // tokens per row partial of the one-row-block statistics
constexpr int kMaxChunk = 2048;     // tokens per work-group of the two-pass kernels at most
constexpr int kMfWaves = kMfThreads / kWave;

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8_t, v); }

// Raw buffer resource (gfx9 descriptor word 3) over `bytes` bytes from p, and the
// cache-policy bit of a streamed (non-temporal) buffer load.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kAuxNt = 2;
// Every argument is wave-uniform; readfirstlane lets the compiler keep the
// descriptor in scalar registers (a vector one would need a waterfall loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void *p, int bytes)
{
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    void *q = (void *)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes), kBufferWord3);
}

struct MfArgs {
    const uint16_t *q_win;
    const uint16_t *k;
    const int32_t *seq_lens;
    int s_max, n_h, n_kv, w, wic, R, unit0, n_chunks, chunk_tokens;
    float c;                 // scale * log2(e)
    int n_parts;             // row partials per unit: one per chunk, or per 256-token block (RT = 1)
    int compact_batch;       // one row block, ragged lengths: B, the work-groups of the valid (KV head,
                             // chunk) pairs first (see mfma_stats_kernel); 0: one work-group per pair
    float2 *part;            // pass 1 out: [group][n_parts][RT*16] (m, l)
    float2 *fin;             // merged row statistics, pass 2 in: [group][RT*16] (-M*c, 1/L)
    int32_t *arrive;         // [group] chunk arrival counters (zero between calls) when the last
                             // arriving pass-1 work-group merges its unit's chunks, else null
    float *raw;              // pass 2 out: [B*n_kv][s_max]
    float *pooled;           // one row block: pooled out of the fused pass 2 [B*n_kv][s_max]
    int n_keep, half;        // its pooling: trailing tokens kept, half-width
    float *logits;           // one row block only: pass 1 keeps its logits [B*n_kv][s_max][rs], or null
    int rs;                  // rows kept per token (R rounded up to 4)
    const int32_t *mask;     // [B*n_kv] or null: units with 0 are skipped
};

// Work decomposition shared by both passes (a work-group is four waves).  Logits come from
// v_mfma_f32_16x16x32_bf16 with 16 keys on M and 16 query rows on N: lane
// l = 16 kg + t supplies token t and elements [32 s + 8 kg, +8) at k-step s for both
// operands (the dot product runs over the same permutation of d on both sides), and
// receives row n = l % 16 for tokens 4 kg + j, j < 4.
//   * The R rows (RT blocks of 16) are split over WPR waves, CPW blocks each; their
//     B operands (Q^T) are loaded once into registers.  With fewer than four row
//     blocks the remaining waves form TG token groups.
//   * K is staged through LDS one stage of ST tokens at a time with coalesced
//     16-byte loads (every load instruction reads 8 KB contiguous), double
//     buffered: the next stage's loads are in flight while the current one is
//     multiplied.  Rows are padded by 16 bytes so the 16 rows a wave reads for one
//     A operand fall in distinct banks.
template <int D, int RT>
struct Sc {
    static constexpr int KS = D / 32;                    // MFMA k-steps
    static constexpr int WPR = RT < 4 ? RT : 4;          // waves sharing one token tile
    static constexpr int CPW = RT / WPR;                 // row blocks per wave
    static constexpr int TG = kMfWaves / WPR;            // token groups
    static constexpr int ST = 16 * (TG > 2 ? TG : 2);    // tokens per stage (8 KB at d_h = 128)
    static constexpr int P = RT == 8 ? 2 : 4;            // stages in flight (register ring; 2 measured best at RT = 8)
    static constexpr int TPG = ST / 16 / TG;             // 16-token tiles per group per stage
    static constexpr int ROWB = 2 * D + 16;              // LDS bytes per row
    static constexpr int VPR = D / 8;                    // 16-byte vectors per row
    static constexpr int LOADS = ST * VPR / kMfThreads;  // 16-byte loads per thread per stage
    static constexpr int STAGE_BYTES = ST * ROWB;
    static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
    static constexpr int PAIR = TPG < 2 ? TPG : 2;       // tiles whose logits share one max/rescale
    static_assert(LOADS >= 1 && ST * VPR % kMfThreads == 0, "stage must split evenly over the threads");

    // Coalesced loads of one stage through a buffer resource over the unit's S cached
    // rows: every offset is a vector offset (the range check covers the vector and
    // instruction offsets, so the stage's first row is added there, not as a scalar
    // offset), and rows at or past S read as zero.  KEEP: ordinary loads, which leave
    // K in the caches for the second pass; else loads hinted as streamed (K's last use).
    template <bool KEEP>
    __device__ static void load_stage(__amdgpu_buffer_rsrc_t rsrc, int st0, u32x4 *reg)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int gid = i * kMfThreads + kvc_tid();
            const int row = gid / VPR, col = gid - row * VPR;
            reg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                rsrc, (st0 + row) * (2 * D) + col * 16, 0, KEEP ? 0 : kAuxNt));
        }
    }

    __device__ static void store_stage(unsigned char *buf, const u32x4 *reg)
    {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int gid = i * kMfThreads + kvc_tid();
            const int row = gid / VPR, col = gid - row * VPR;
            *(u32x4 *)(buf + row * ROWB + col * 16) = reg[i];
        }
    }

    // This wave's B operands (its CPW row blocks of the group's queries) straight
    // into registers; rows >= R are zero.
    __device__ static void load_q(const MfArgs &a, int b, int g, int wr, int n, int kg, u32x4 (*qb)[KS])
    {
        const int r = a.n_h / a.n_kv;
        const uint16_t *q0 = a.q_win + (size_t)(b * a.n_h + g * r) * a.w * D;
#pragma unroll
        for (int cb = 0; cb < CPW; ++cb) {
            const int row = (wr * CPW + cb) * 16 + n;
#pragma unroll
            for (int s = 0; s < KS; ++s)
                qb[cb][s] = row < a.R ? *((const u32x4 *)(q0 + (size_t)row * D + 32 * s + 8 * kg))
                                      : u32x4{0u, 0u, 0u, 0u};
        }
    }

    __device__ static void load_a(const unsigned char *buf, int tile, int n, int kg, u32x4 *ka)
    {
#pragma unroll
        for (int s = 0; s < KS; ++s) ka[s] = *(const u32x4 *)(buf + (tile * 16 + n) * ROWB + (4 * s + kg) * 16);
    }

    __device__ static f32x4_t mma(const u32x4 *ka, const u32x4 *qb)
    {
        f32x4_t acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[s]), as_bf16x8(qb[s]), acc, 0, 0, 0);
        return acc;
    }

    // The same tile with the operands swapped (query rows on M, tokens on N): lane
    // l = 16 kg + n receives token n for rows 4 kg + j, j < 4.
    __device__ static f32x4_t mma_rows(const u32x4 *qb, const u32x4 *ka)
    {
        f32x4_t acc = {};
#pragma unroll
        for (int s = 0; s < KS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qb[s]), as_bf16x8(ka[s]), acc, 0, 0, 0);
        return acc;
    }
};

// Pass 1: per row, max logit m and sum of exp2((x - m) c) over one chunk's visible
// tokens, merged across lane groups and token groups in a fixed order.
// Streams stages [0, n_st) of a chunk through LDS.  Stage j's loads are issued P - 1
// steps before it is stored to LDS (register ring ring[j % P]), so every work-group
// keeps up to P stages of K in flight.  BODY(buf, st) runs on the stage in LDS;
// POST(st) runs after the barrier that ends step st.  The loop is unrolled by P so
// the ring index is a compile-time constant, and every load and LDS store in it is
// unconditional (look-ahead past the last stage re-reads the last stage, skipped
// steps only skip BODY/POST): the compiler can then count outstanding loads exactly
// instead of draining the ring at every step.
template <int D, int RT, bool KEEP, typename BODY, typename POST>
__device__ __forceinline__ void stream_stages(__amdgpu_buffer_rsrc_t kunit, int ch0, int n_st,
                                              unsigned char *kbuf, BODY body, POST post)
{
    using C = Sc<D, RT>;
    constexpr int P = C::P;
    if (n_st <= 0) return;
    const int last_st = n_st - 1;
    u32x4 ring[P][C::LOADS];
#pragma unroll
    for (int q = 0; q < P; ++q) C::template load_stage<KEEP>(kunit, ch0 + min(q, last_st) * C::ST, ring[q]);
    C::store_stage(kbuf, ring[0]);
    __syncthreads();
    for (int base = 0; base < n_st; base += P) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const int st = base + q;
            C::template load_stage<KEEP>(kunit, ch0 + min(st + P, last_st) * C::ST, ring[q]);
            if (st < n_st) body(kbuf + (st & 1) * C::STAGE_BYTES, st);
            C::store_stage(kbuf + ((st + 1) & 1) * C::STAGE_BYTES, ring[(q + 1) % P]);
            __syncthreads();
            if (st < n_st) post(st);
        }
    }
}

template <int D, int RT, bool MASK>
__device__ __forceinline__ void stats_stage(const unsigned char *buf, int st0, int tg, int n, int kg,
                                            const u32x4 (*qb)[Sc<D, RT>::KS], const int *last, float c,
                                            float *m, double *l, float *lg, int rs, int S)
{
    using C = Sc<D, RT>;
    constexpr int NV = 4 * C::PAIR;                      // logits per lane per row block per max
#pragma unroll
    for (int p0 = 0; p0 < C::TPG; p0 += C::PAIR) {
        float x[C::CPW][NV];
#pragma unroll
        for (int pp = 0; pp < C::PAIR; ++pp) {
            const int tile = tg + (p0 + pp) * C::TG;
            u32x4 ka[C::KS];
            C::load_a(buf, tile, n, kg, ka);
#pragma unroll
            for (int cb = 0; cb < C::CPW; ++cb) {
                const f32x4_t x4 = C::mma(ka, qb[cb]);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    x[cb][4 * pp + j] = x4[j];
                    if (MASK && st0 + tile * 16 + 4 * kg + j > last[cb]) x[cb][4 * pp + j] = -INFINITY;
                }
                if constexpr (RT == 1) {
                    // few rows: keep the logits (rs floats per token) for pass 2 instead of K
                    if (lg && n < rs) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int tok = st0 + tile * 16 + 4 * kg + j;
                            if (tok < S) lg[(size_t)tok * rs + n] = x[cb][4 * pp + j];
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int cb = 0; cb < C::CPW; ++cb) {
            float mx = m[cb];
#pragma unroll
            for (int j = 0; j < NV; ++j) mx = fmaxf(mx, x[cb][j]);
            if (!MASK || mx != -INFINITY) {
                const float nmc = -mx * c;
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int j = 0; j < NV; j += 2) {
                    s0 += fast_exp2(fmaf(x[cb][j], c, nmc));
                    s1 += fast_exp2(fmaf(x[cb][j + 1], c, nmc));
                }
                // rescale by exp2((m_old - mx) c): exactly 1 while the max stands (an
                // fma against the rounded -mx c would be 1 +- 1e-6 and, applied at every
                // update of a long chunk, drift the sum past 1e-5); the running sum is
                // kept in double for the same reason
                l[cb] = fma(l[cb], (double)fast_exp2((m[cb] - mx) * c), (double)(s0 + s1));
                m[cb] = mx;
            }
        }
    }
}

// Merges the partials (m, l) of every row of unit ul in a fixed order, by the unit's
// last arriving pass-1 work-group or by mfma_merge_parts_kernel (kMfThreads threads
// either way, so both give the same bits): thread (slice, row) folds partials slice,
// slice + slices, ... online (rescale factors in fp32, sums in double), and the slices
// are then folded in slice order.  The partials may have been published with st_dev by
// the work-groups of other XCDs, hence ld_dev.  buf: 3 KB of LDS.
// Chunks of a unit with S tokens that pass 1 visits: every chunk, or with compact_batch
// only those holding tokens (at least one, so a unit with no token still publishes).
__device__ __forceinline__ int chunks_of(const MfArgs &a, int S)
{
    if (!a.compact_batch) return a.n_chunks;
    const int n = (S + a.chunk_tokens - 1) / a.chunk_tokens;
    return n < 1 ? 1 : n;
}

template <int RPAD>
__device__ __forceinline__ void merge_chunks(const MfArgs &a, int ul, unsigned char *buf)
{
    constexpr int slices = kMfThreads / RPAD;
    static_assert(slices * RPAD == kMfThreads, "rows must split the work-group evenly");
    float *sm_M = (float *)buf;
    double *sm_L = (double *)(buf + kMfThreads * sizeof(float));
    const int row = kvc_tid() % RPAD;
    const int slice = kvc_tid() / RPAD;
    const unsigned long long *p = (const unsigned long long *)(a.part + (size_t)ul * a.n_parts * RPAD) + row;
    // the partials written by this call: those of the chunks pass 1 visited
    int n_parts = a.n_parts;
    if (a.compact_batch) {
        const int S = clamp_len(a.seq_lens, (a.unit0 + ul) / a.n_kv, a.s_max);
        n_parts = min(n_parts, chunks_of(a, S) * (RPAD == 16 ? a.chunk_tokens / kStatBlock : 1));
    }
    float Mx = -INFINITY;
    double L = 0.0;
    constexpr int kBatch = 8;               // partials requested together per thread
    for (int ch0 = slice; ch0 < n_parts; ch0 += kBatch * slices) {
        unsigned long long v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int ch = min(ch0 + q * slices, n_parts - 1);    // unconditional: one round trip
            v[q] = ld_dev(p + (size_t)ch * RPAD);
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (ch0 + q * slices >= n_parts) continue;
            const float vm = unpack_lo(v[q]), vl = unpack_hi(v[q]);
            if (vm == -INFINITY) continue;
            if (vm > Mx) {
                L = L * (double)fast_exp2((Mx - vm) * a.c) + (double)vl;
                Mx = vm;
            } else {
                L += (double)vl * (double)fast_exp2((vm - Mx) * a.c);
            }
        }
    }
    sm_M[kvc_tid()] = Mx;
    sm_L[kvc_tid()] = L;
    __syncthreads();
    if (slice != 0) return;
    float Mt = -INFINITY;
    for (int s2 = 0; s2 < slices; ++s2) Mt = fmaxf(Mt, sm_M[s2 * RPAD + row]);
    float2 res = make_float2(0.f, 0.f);
    if (row < a.R && Mt != -INFINITY) {
        double Lt = 0.0;
        for (int s2 = 0; s2 < slices; ++s2) {
            const float ms = sm_M[s2 * RPAD + row];
            if (ms != -INFINITY) Lt += sm_L[s2 * RPAD + row] * (double)fast_exp2((ms - Mt) * a.c);
        }
        if (Lt > 0.0) res = make_float2(-Mt * a.c, (float)(1.0 / Lt));
    }
    a.fin[(size_t)ul * RPAD + row] = res;
}

template <int D, int RT>
__global__ __launch_bounds__(kMfThreads) __attribute__((amdgpu_waves_per_eu(4))) void mfma_stats_kernel(MfArgs a)
{
    using C = Sc<D, RT>;
    constexpr int KS = C::KS;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *kbuf = lds;                           // 2 stages
    __shared__ float sm_m[C::TG][RT * 16];
    __shared__ float sm_l[C::TG][RT * 16];
    // One row block (RT = 1): a partial per 256-token block rather than per chunk, so
    // the statistics do not depend on how the tokens are cut into chunks (a call that
    // scores a few KV heads cuts them finer and gets the same bits).  At a block's last
    // stage each wave merges a row's four lane groups with lane swaps (VALU only),
    // keeps the result in LDS per (block, token group) and starts afresh; after the
    // loop the token groups of every block are merged in order.
    constexpr bool kBlocks = RT == 1;
    constexpr int kBlkSt = kStatBlock / C::ST;           // stages per block
    constexpr int kMaxBlk = kMaxChunk / kStatBlock;      // blocks per chunk at most
    static_assert(!kBlocks || (kStatBlock % C::ST == 0 && C::CPW == 1), "a block is whole stages");
    __shared__ float sm_bm[kBlocks ? kMaxBlk : 1][C::TG][16], sm_bl[kBlocks ? kMaxBlk : 1][C::TG][16];

    int chunk = kvc_bid_x();
    int ul = kvc_bid_y();
    if (RT == 1 && a.compact_batch) {
        // ragged lengths: work-group L of the grid takes the L-th (KV head, chunk) pair
        // holding tokens, KV heads in order, and the ones past the last pair exit; the
        // work that exists then fills the first work-groups, which the dispatcher spreads
        // evenly over the CUs (a pair per work-group in grid order left whole CUs with
        // four long chunks and others with four empty ones)
        int L = (int)kvc_bid_y() * a.n_chunks + (int)kvc_bid_x();
        bool found = false;
        for (int bb = 0; bb < a.compact_batch; ++bb) {
            const int nch = chunks_of(a, clamp_len(a.seq_lens, bb, a.s_max));
            if (L < nch * a.n_kv) {
                ul = bb * a.n_kv + L / nch;
                chunk = L % nch;
                found = true;
                break;
            }
            L -= nch * a.n_kv;
        }
        if (!found) return;
    }
    const int u = a.unit0 + ul;
    if (a.mask && !ld_uniform(a.mask, u)) return;
    const int b = u / a.n_kv;
    const int g = u - b * a.n_kv;
    const int S = __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens, b, a.s_max));   // uniform: scalar offsets below
    const int lane = kvc_tid() & 63, wv = kvc_tid() >> 6;
    const int n = lane & 15, kg = lane >> 4;
    const int wr = wv % C::WPR, tg = wv / C::WPR;
    const __amdgpu_buffer_rsrc_t kunit = buffer_rsrc(a.k + (size_t)u * a.s_max * D, S * (2 * D));
    const int ch0 = chunk * a.chunk_tokens;
    int n_st = (min(ch0 + a.chunk_tokens, S) - ch0 + C::ST - 1) / C::ST;
    n_st = n_st < 0 ? 0 : n_st;

    u32x4 qb[C::CPW][KS];
    C::load_q(a, b, g, wr, n, kg, qb);
    int last[C::CPW];
#pragma unroll
    for (int cb = 0; cb < C::CPW; ++cb) {
        const int i = ((wr * C::CPW + cb) * 16 + n) % a.w;
        last[cb] = a.wic ? min(S - a.w + i, S - 1) : S - 1;
    }
    const int all_vis = a.wic ? S - a.w : S - 1;          // every row sees tokens <= all_vis
    float *lg = a.logits ? a.logits + (size_t)u * a.s_max * a.rs : nullptr;
    float m[C::CPW];
    double l[C::CPW];
#pragma unroll
    for (int cb = 0; cb < C::CPW; ++cb) {
        m[cb] = -INFINITY;
        l[cb] = 0.0;
    }
    auto store_partial = [&](float Mx, float L, int idx, int row) {
        float2 *dst = a.part + ((size_t)ul * a.n_parts + idx) * (RT * 16) + row;
        if (a.arrive) st_dev((unsigned long long *)dst, pack2(Mx, L));
        else *dst = make_float2(Mx, L);
    };
    auto block_end = [&](int st) { return st % kBlkSt == kBlkSt - 1 || st == n_st - 1; };
    // (m, l) merged with the lane l ^ 32, then l ^ 16 (a symmetric expression: both
    // lanes of a pair get the same bits)
    auto lane_merge = [&](float &mm, double &ll) {
#pragma unroll
        for (int sw = 0; sw < 2; ++sw) {
            const uint32_t mb = __float_as_uint(mm);
            const uint32_t lo = (uint32_t)__double_as_longlong(ll), hi = (uint32_t)(__double_as_longlong(ll) >> 32);
            uint32_t pm, plo, phi;
            if (sw == 0) {
                const bool low = (kvc_tid() & 63) < 32;
                const auto x = __builtin_amdgcn_permlane32_swap(mb, mb, false, false);
                const auto y = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
                const auto z = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
                pm = low ? x[1] : x[0];
                plo = low ? y[1] : y[0];
                phi = low ? z[1] : z[0];
            } else {
                const bool even = ((kvc_tid() >> 4) & 1) == 0;
                const auto x = __builtin_amdgcn_permlane16_swap(mb, mb, false, false);
                const auto y = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
                const auto z = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
                pm = even ? x[1] : x[0];
                plo = even ? y[1] : y[0];
                phi = even ? z[1] : z[0];
            }
            const float m2 = __uint_as_float(pm);
            const double l2 = __longlong_as_double((long long)(((unsigned long long)phi << 32) | plo));
            const float Mx = fmaxf(mm, m2);
            if (Mx != -INFINITY) {
                ll = ll * (double)fast_exp2((mm - Mx) * a.c) + l2 * (double)fast_exp2((m2 - Mx) * a.c);
                mm = Mx;
            }
        }
    };
    stream_stages<D, RT, true>(kunit, ch0, n_st, kbuf,
        [&](const unsigned char *cur, int st) {
            const int st0 = ch0 + st * C::ST;
            if (st0 + C::ST - 1 <= all_vis)
                stats_stage<D, RT, false>(cur, st0, tg, n, kg, qb, last, a.c, m, l, lg, a.rs, S);
            else
                stats_stage<D, RT, true>(cur, st0, tg, n, kg, qb, last, a.c, m, l, lg, a.rs, S);
            if constexpr (kBlocks) {
                if (block_end(st)) {
                    lane_merge(m[0], l[0]);
                    const int bl = (st0 - ch0) / kStatBlock;
                    if (kg == 0) {
                        sm_bm[bl][tg][n] = m[0];
                        sm_bl[bl][tg][n] = (float)l[0];
                    }
                    m[0] = -INFINITY;
                    l[0] = 0.0;
                }
            }
        },
        [&](int) {});
    if constexpr (kBlocks) {
        // every block of the chunk: its token groups in order; blocks past the
        // sequence hold no token
        const int nb = (n_st * C::ST + kStatBlock - 1) / kStatBlock;      // blocks with stages
        const int b1 = min(a.chunk_tokens / kStatBlock, a.n_parts - ch0 / kStatBlock);
        __syncthreads();
        for (int i = kvc_tid(); i < b1 * 16; i += kMfThreads) {
            const int bl = i / 16, row = i % 16;
            float Mx = -INFINITY, L = 0.f;
            if (bl < nb) {
                for (int t2 = 0; t2 < C::TG; ++t2) Mx = fmaxf(Mx, sm_bm[bl][t2][row]);
                if (Mx != -INFINITY)
                    for (int t2 = 0; t2 < C::TG; ++t2) L += sm_bl[bl][t2][row] * fast_exp2((sm_bm[bl][t2][row] - Mx) * a.c);
            }
            store_partial(Mx, L, ch0 / kStatBlock + bl, row);
        }
    } else {
        // merge the four lane groups of a row (lanes n, n+16, n+32, n+48), then the
        // token groups
#pragma unroll
        for (int cb = 0; cb < C::CPW; ++cb) {
#pragma unroll
            for (int off = 16; off < 64; off <<= 1) {
                const float m2 = shfl_xor_f(m[cb], off);
                const double l2 = __shfl_xor(l[cb], off, kWave);
                const float Mx = fmaxf(m[cb], m2);
                if (Mx != -INFINITY) {
                    l[cb] = l[cb] * (double)fast_exp2((m[cb] - Mx) * a.c) + l2 * (double)fast_exp2((m2 - Mx) * a.c);
                    m[cb] = Mx;
                }
            }
            if (kg == 0) {
                sm_m[tg][(wr * C::CPW + cb) * 16 + n] = m[cb];
                sm_l[tg][(wr * C::CPW + cb) * 16 + n] = (float)l[cb];
            }
        }
        __syncthreads();
        for (int row = kvc_tid(); row < RT * 16; row += kMfThreads) {
            float Mx = -INFINITY;
            for (int t2 = 0; t2 < C::TG; ++t2) Mx = fmaxf(Mx, sm_m[t2][row]);
            float L = 0.f;
            if (Mx != -INFINITY)
                for (int t2 = 0; t2 < C::TG; ++t2) L += sm_l[t2][row] * fast_exp2((sm_m[t2][row] - Mx) * a.c);
            store_partial(Mx, L, chunk, row);
        }
    }
    if (!a.arrive) return;                  // a merge kernel merges the partials
    // count this chunk's arrival once its partials have landed; the unit's last arrival
    // merges every chunk (the K stage buffers are free by now and hold the merge's state)
    stores_done();
    __shared__ int sm_last;
    __syncthreads();
    if (kvc_tid() == 0) {
        const int old = __hip_atomic_fetch_add(a.arrive + ul, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sm_last = old == chunks_of(a, S) - 1;
        if (sm_last) __hip_atomic_store(a.arrive + ul, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (sm_last) merge_chunks<RT * 16>(a, ul, lds);
}

// The merge of one row block's partials as a kernel of its own: the arithmetic of the
// merge in the last pass-1 work-group.
template <int RPAD>
__global__ __launch_bounds__(kMfThreads) void mfma_merge_parts_kernel(MfArgs a)
{
    __shared__ __attribute__((aligned(16))) unsigned char buf[kMfThreads * (sizeof(float) + sizeof(double))];
    const int ul = kvc_bid_x();
    if (a.mask && !ld_uniform(a.mask, a.unit0 + ul)) return;
    merge_chunks<RPAD>(a, ul, buf);
}

// Merges the chunk partials of every row in a fixed order, as a kernel of its own
// (launches with many chunks or work-group rounds).  blockDim = 1024:
// thread (slice, row) folds chunks slice, slice + slices, ... online (rescale factors
// in fp32, sums in double); the slices are then folded in slice order.
constexpr int kMergeThreads = 1024;

__global__ __launch_bounds__(kMergeThreads) void mfma_merge_kernel(const float2 *__restrict__ part, int n_chunks,
                                                                    int rpad, int R, float c,
                                                                    const int32_t *__restrict__ mask,
                                                                    float2 *__restrict__ fin)
{
    __shared__ float sm_M[kMergeThreads];
    __shared__ double sm_L[kMergeThreads];
    const int ul = kvc_bid_x();
    if (mask && !ld_uniform(mask, ul)) return;
    const int slices = kMergeThreads / rpad;
    const int row = kvc_tid() % rpad;
    const int slice = kvc_tid() / rpad;
    const float2 *p = part + (size_t)ul * n_chunks * rpad + row;
    float Mx = -INFINITY;
    double L = 0.0;
    constexpr int kBatch = 16;              // chunk partials requested together per thread
    for (int ch0 = slice; slice < slices && ch0 < n_chunks; ch0 += kBatch * slices) {
        float2 v[kBatch];
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            const int ch = min(ch0 + q * slices, n_chunks - 1);      // unconditional: one round trip
            v[q] = p[(size_t)ch * rpad];
        }
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
            if (ch0 + q * slices >= n_chunks) continue;
            if (v[q].x == -INFINITY) continue;
            if (v[q].x > Mx) {
                L = L * (double)fast_exp2((Mx - v[q].x) * c) + (double)v[q].y;
                Mx = v[q].x;
            } else {
                L += (double)v[q].y * (double)fast_exp2((v[q].x - Mx) * c);
            }
        }
    }
    sm_M[kvc_tid()] = Mx;
    sm_L[kvc_tid()] = L;
    __syncthreads();
    if (slice != 0) return;
    float Mt = -INFINITY;
    for (int s2 = 0; s2 < slices; ++s2) Mt = fmaxf(Mt, sm_M[s2 * rpad + row]);
    float2 res = make_float2(0.f, 0.f);
    if (row < R && Mt != -INFINITY) {
        double Lt = 0.0;
        for (int s2 = 0; s2 < slices; ++s2) {
            const float ms = sm_M[s2 * rpad + row];
            if (ms != -INFINITY) Lt += sm_L[s2 * rpad + row] * (double)fast_exp2((ms - Mt) * c);
        }
        if (Lt > 0.0) res = make_float2(-Mt * c, (float)(1.0 / Lt));
    }
    fin[(size_t)ul * rpad + row] = res;
}

// Pass 2: raw[t] = sum over rows of exp2((x - M) c) / L for one chunk.  The tiles
// are multiplied with the query rows on M and the tokens on N, so each lane holds one
// token of a tile for four rows of every row block and sums them in-lane; the four
// lane groups of a token (lanes n, n + 16, n + 32, n + 48) are added with two lane
// swaps (rows of 32, then of 16 lanes), and the WPR row slices in LDS, in a fixed
// order, once per stage.
template <int D, int RT, bool MASK>
__device__ __forceinline__ void probsum_stage(const unsigned char *buf, int st0, int tg, int wr, int n, int kg,
                                              const u32x4 (*qb)[Sc<D, RT>::KS], const int (*last)[4],
                                              const float (*nmc)[4], const float (*il)[4], float c, float *red)
{
    using C = Sc<D, RT>;
#pragma unroll
    for (int p = 0; p < C::TPG; ++p) {
        const int tile = tg + p * C::TG;
        u32x4 ka[C::KS];
        C::load_a(buf, tile, n, kg, ka);
        const int tok = st0 + tile * 16 + n;
        float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
        for (int cb = 0; cb < C::CPW; ++cb) {
            const f32x4_t x = C::mma_rows(qb[cb], ka);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float e = fast_exp2(fmaf(x[j], c, nmc[cb][j]));
                if (MASK && tok > last[cb][j]) e = 0.f;
                if (j & 1) acc1 = fmaf(e, il[cb][j], acc1);
                else acc0 = fmaf(e, il[cb][j], acc0);
            }
        }
        const float v = acc0 + acc1;
        const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const float v2 = __uint_as_float(h[0]) + __uint_as_float(h[1]);   // + lane l ^ 32
        const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2), false, false);
        const float v4 = __uint_as_float(q[0]) + __uint_as_float(q[1]);   // + lane l ^ 16
        if (kg == 0) red[wr * C::ST + tile * 16 + n] = v4;                // [row slice][token]
    }
}

template <int D, int RT>
__global__ __launch_bounds__(kMfThreads) __attribute__((amdgpu_waves_per_eu(4))) void mfma_probsum_kernel(MfArgs a)
{
    using C = Sc<D, RT>;
    constexpr int KS = C::KS;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *kbuf = lds;
    float *rawbuf = (float *)(lds + C::LDS_BYTES);       // the chunk's scores, written once at the end
    __shared__ float red[2][C::WPR * C::ST];

    const int chunk = kvc_bid_x();
    const int ul = kvc_bid_y();
    const int u = a.unit0 + ul;
    if (a.mask && !ld_uniform(a.mask, u)) return;
    const int b = u / a.n_kv;
    const int g = u - b * a.n_kv;
    const int S = __builtin_amdgcn_readfirstlane(clamp_len(a.seq_lens, b, a.s_max));   // uniform: scalar offsets below
    const int lane = kvc_tid() & 63, wv = kvc_tid() >> 6;
    const int n = lane & 15, kg = lane >> 4;
    const int wr = wv % C::WPR, tg = wv / C::WPR;
    const __amdgpu_buffer_rsrc_t kunit = buffer_rsrc(a.k + (size_t)u * a.s_max * D, S * (2 * D));
    float *rawu = a.raw + (size_t)u * a.s_max;
    const int ch0 = chunk * a.chunk_tokens;
    const int ch1 = min(ch0 + a.chunk_tokens, a.s_max);
    int n_st = (min(ch1, S) - ch0 + C::ST - 1) / C::ST;   // stages holding cached tokens
    n_st = n_st < 0 ? 0 : n_st;

    u32x4 qb[C::CPW][KS];
    C::load_q(a, b, g, wr, n, kg, qb);
    // row constants of this lane's rows (4 kg + j of each row block)
    float nmc[C::CPW][4], il[C::CPW][4];
    int last[C::CPW][4];
#pragma unroll
    for (int cb = 0; cb < C::CPW; ++cb) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (wr * C::CPW + cb) * 16 + 4 * kg + j;
            const float2 f = a.fin[(size_t)ul * (RT * 16) + row];
            nmc[cb][j] = f.x;
            il[cb][j] = f.y;
            const int i = row % a.w;
            last[cb][j] = a.wic ? min(S - a.w + i, S - 1) : S - 1;
        }
    }
    const int all_vis = a.wic ? S - a.w : S - 1;
    stream_stages<D, RT, false>(kunit, ch0, n_st, kbuf,
        [&](const unsigned char *cur, int st) {
            const int st0 = ch0 + st * C::ST;
            float *rd = red[st & 1];
            if (st0 + C::ST - 1 <= all_vis)
                probsum_stage<D, RT, false>(cur, st0, tg, wr, n, kg, qb, last, nmc, il, a.c, rd);
            else
                probsum_stage<D, RT, true>(cur, st0, tg, wr, n, kg, qb, last, nmc, il, a.c, rd);
        },
        [&](int st) {
            // add the row slices of this stage in order; red[st & 1] is rewritten two
            // steps later
            const float *rd = red[st & 1];
            for (int t = kvc_tid(); t < C::ST; t += kMfThreads) {
                float v = 0.f;
                for (int r2 = 0; r2 < C::WPR; ++r2) v += rd[r2 * C::ST + t];
                rawbuf[st * C::ST + t] = v;
            }
        });
    __syncthreads();
    // the chunk's scores, 0 past the cached length
    for (int t = kvc_tid(); ch0 + t < ch1; t += kMfThreads) {
        const int tok = ch0 + t;
        rawu[tok] = (tok < S && t < n_st * C::ST) ? rawbuf[t] : 0.f;
    }
}

// One row block (R <= 16): pass 2, from the logits pass 1 kept (no K is read again),
// and the pooling in one kernel.  A work-group takes kPoolTile tokens of a unit and
// the pooling halo around them, scores each token from its rs consecutive logits (sum
// over rows, in row order, of exp2(x c - M c) / L), writes the tile's scores and pools
// them from LDS as pool_kernel does.
template <bool VEC, int HALF>
__global__ __launch_bounds__(kPoolThreads) void logit_pool_kernel(MfArgs a)
{
    __shared__ float2 f[16];
    __shared__ __attribute__((aligned(16))) float tile[kPoolLds];
    int half = a.half;
    if constexpr (HALF >= 0) half = HALF;
    const int ul = kvc_bid_y();
    const int u = a.unit0 + ul;
    if (a.mask && !ld_uniform(a.mask, u)) return;
    const int tid = kvc_tid();
    if (tid < 16) f[tid] = tid < a.R ? a.fin[(size_t)ul * 16 + tid] : make_float2(0.f, 0.f);
    __syncthreads();
    const int S = clamp_len(a.seq_lens, u / a.n_kv, a.s_max);
    const int C = S - a.n_keep > 0 ? S - a.n_keep : 0;
    const float *lg = a.logits + (size_t)u * a.s_max * a.rs;
    auto score = [&](int t) {               // 0 outside [0, S)
        float acc = 0.f;
        if (t >= 0 && t < S) {
            const float4 *x4 = (const float4 *)(lg + (size_t)t * a.rs);
            float x[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (4 * q < a.rs) {
                    const float4 v = x4[q];
                    x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
                }
            }
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (r < a.R) acc = fmaf(fast_exp2(fmaf(x[r], a.c, f[r].x)), f[r].y, acc);
        }
        return acc;
    };
    const int t0 = kvc_bid_x() * kPoolTile;
    const int base = t0 - (2 * kMaxHalf + 2);               // tile[i] holds raw[base + i]
    float *body = tile + 2 * kMaxHalf + 2;
    const int t = t0 + 4 * tid;                             // this thread's 4 tokens
    float v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = score(t + k);
    *(float4 *)(body + 4 * tid) = make_float4(v[0], v[1], v[2], v[3]);
    float *rw = a.raw + (size_t)u * a.s_max;
    if constexpr (VEC) {
        if (t < a.s_max) *(float4 *)(rw + t) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (t + k < a.s_max) rw[t + k] = v[k];
    }
    if (tid < half) {
        const int th = t0 - half + tid;
        tile[th - base] = score(th);
    } else if (tid < 2 * half) {
        const int th = t0 + kPoolTile + (tid - half);
        tile[th - base] = score(th);                        // 0 past S, so past s_max
    }
    __syncthreads();
    pool_tile<VEC, HALF>(tile, base, t, a.s_max, half, C, S, a.pooled + (size_t)u * a.s_max);
}

template <bool VEC>
void launch_logit_pool(dim3 grid, const MfArgs &a, hipStream_t stream)
{
    switch (a.half) {
    case 0: hipLaunchKernelGGL((logit_pool_kernel<VEC, 0>), grid, dim3(kPoolThreads), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((logit_pool_kernel<VEC, 1>), grid, dim3(kPoolThreads), 0, stream, a); break;
    case 2: hipLaunchKernelGGL((logit_pool_kernel<VEC, 2>), grid, dim3(kPoolThreads), 0, stream, a); break;
    case 3: hipLaunchKernelGGL((logit_pool_kernel<VEC, 3>), grid, dim3(kPoolThreads), 0, stream, a); break;
    default: hipLaunchKernelGGL((logit_pool_kernel<VEC, -1>), grid, dim3(kPoolThreads), 0, stream, a); break;
    }
}

// ====================================================================================
// Single-pass MFMA path for 17..32 rows per KV head (MHA windows, small groups): K is
// read once.
//
// An item is 1024 consecutive tokens of one unit; each of the four waves of a
// work-group takes 256 of them (16 tiles of 16 tokens).  K reaches LDS by direct
// buffer-to-LDS loads, four tiles ahead in a per-wave ring, laid out so that every
// lane reads back exactly the 16 bytes it loaded as its MFMA operand: no registers
// hold K in flight and no barrier orders it.  The item's R x 1024 logits stay in
// registers (query rows on M, tokens on N, as in pass 2 above).
//
// A persistent grid of G work-groups takes items j = blockIdx.x, + G, + 2G, ... with
// G a multiple of the items per unit, so all items of a unit fall in one round and
// every work-group of a round is resident at once.  For its item a work-group
//   A  computes the logits, reduces them to the item's per-row (max, sum of exp),
//      publishes that record and counts the unit's arrival; the unit's last arrival
//      merges the unit's records in item order into the final per-row (M, 1/L) and
//      publishes them;
//   B  one round later, once the next item's first K tiles are in flight, waits for
//      the unit's final statistics and turns the logits still in registers into the
//      probability sums of the item's tokens.
// A never waits and B waits only for items of an earlier round, so the grid cannot
// deadlock while all of it is resident.  A wait that does not end within a bounded
// time (a work-group not resident, for instance) puts the item on a deferred list; a
// follow-up kernel recomputes those items from K once every record is written.
// Records, final statistics and arrival counters are written and read with
// device-scope atomics (coherent across the XCDs' L2 caches); a writer waits for its
// record stores to complete before the arrival that announces them.  Every final
// statistic word carries the call's tag (one more than a word of the workspace that
// the pooling kernel advances after each call), so a waiting work-group polls the
// final statistics themselves: the merging work-group neither waits for their stores
// nor raises a separate flag, and the waiter needs no second load.
// ====================================================================================
constexpr int kSpThreads = 256;
constexpr int kSpWaves = kSpThreads / kWave;
constexpr int kSpTiles = 16;                             // 16-token tiles per wave per item
constexpr int kSpRing = 4;                               // K tiles in flight per wave
constexpr int kSpItem = 16 * kSpTiles * kSpWaves;        // 1024 tokens
constexpr int kSpFixGroups = 64;                          // work-groups of the follow-up kernel

struct SpArgs {
    const uint16_t *q_win;
    const uint16_t *k;
    const int32_t *seq_lens;
    const int32_t *mask;
    int s_max, n_h, n_kv, w, wic, R, n_chunks, n_items, G;
    int spin;                 // bound of a wait, 100 MHz ticks (0: defer every item)
    int fix_g;                // work-groups of the follow-up kernel
    float c;                  // scale * log2(e)
    float *raw;               // [units][s_max]
    int32_t *arrive;          // [units] items that published their record (zero between calls)
    int32_t *defer_n;         // deferred items (zero between calls)
    const int32_t *tag;       // the previous call's tag (advanced by the pooling kernel)
    int32_t *defer;           // [n_items]
    unsigned long long *rec;  // [units][n_chunks][16 RT] packed (m, l) per item and row
    unsigned long long *fin;  // [units][16 RT][2] tagged final -M c, 1/L
};

// A record word: the value's bits low, the call's tag high.
__device__ __forceinline__ unsigned long long tagged(float v, uint32_t tag)
{
    return (unsigned long long)__float_as_uint(v) | ((unsigned long long)tag << 32);
}
__device__ __forceinline__ uint32_t tag_of(unsigned long long w) { return (uint32_t)(w >> 32); }

template <int CTRL>
__device__ __forceinline__ float dpp_max(float v)
{
    return fmaxf(v, dpp_f<CTRL>(v));
}
// Max over the 16 lanes of a row (same pairings as row16_sum).
__device__ __forceinline__ float row16_max(float v)
{
    v = dpp_max<kDppRowMirror>(v);
    v = dpp_max<kDppHalfMirror>(v);
    v = dpp_max<kDppXor2>(v);
    v = dpp_max<kDppXor1>(v);
    return v;
}

typedef __attribute__((address_space(3))) void lds_void;

// Waits until at most N vector memory operations of this wave are outstanding (the
// direct-to-LDS loads of a ring slot have landed once the later ones are all that is
// left); N is a constant after unrolling.
template <int N>
__device__ __forceinline__ void vm_wait()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Waits until this wave's LDS reads have returned (before a ring slot is refilled).
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Work-group barrier that orders LDS accesses only: the direct-to-LDS loads of K stay in
// flight across it (a full barrier would wait for every outstanding load).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct SpItem {
    int u, b, g, ch, t0, S;
    bool active;              // unit not masked and the item holds cached tokens
    bool zero;                // unit not masked, item past the cached tokens: raw = 0
};

__device__ __forceinline__ SpItem sp_item(const SpArgs &a, int j)
{
    SpItem it;
    it.u = j / a.n_chunks;
    it.ch = j - it.u * a.n_chunks;
    it.b = it.u / a.n_kv;
    it.g = it.u - it.b * a.n_kv;
    it.t0 = it.ch * kSpItem;
    it.S = clamp_len(a.seq_lens, it.b, a.s_max);
    const bool on = !a.mask || ld_uniform(a.mask, it.u) != 0;
    it.active = on && it.t0 < it.S;
    it.zero = on && !it.active && it.t0 < a.s_max;
    return it;
}

template <int D, int RT>
struct Sp {
    static constexpr int KS = D / 32;
    static constexpr int ROWS = 16 * RT;
    static constexpr int QROWB = 2 * D + 16;             // LDS bytes per query row (padded: distinct banks)
    static constexpr int SLOT = 16 * 2 * D;              // LDS bytes of one wave's tile

    // First token of the wave's share of an item.
    __device__ static int wave_t0(const SpItem &it, int wv) { return it.t0 + wv * 16 * kSpTiles; }

    // Direct loads of one 16-token tile of the wave's share into its LDS slot.  Every
    // load instruction reads 1 KB of contiguous rows (64 / CPR whole rows of CPR 16-byte
    // chunks); lane l's chunk lands at slot + 1024 i + 16 l.  Chunk c of row r is stored
    // at position c ^ (r % CPR) of the row (an XOR swizzle), so that the 16 lanes reading
    // one chunk column of 16 rows as an MFMA operand hit distinct banks.  Rows at or past
    // S read as zero.
    static constexpr int CPR = D / 8;                    // 16-byte chunks per row
    __device__ static void load_tile(__amdgpu_buffer_rsrc_t rs, int tb, int n, int kg, unsigned char *slot)
    {
        const int l = 16 * kg + n;
        constexpr int RPI = kWave / CPR;                 // rows per load instruction
#pragma unroll
        for (int i = 0; i < 16 / RPI; ++i) {
            const int row = RPI * i + l / CPR;
            const int chunk = (l % CPR) ^ (row % CPR);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)(slot + i * kWave * 16), 16,
                                                     (tb + row) * (2 * D) + chunk * 16, 0, 0, kAuxNt);
        }
    }

    // This thread's share of the unit's query rows (rows >= R repeat row R - 1; they are
    // masked out): QV 16-byte vectors, fetched ahead of the item and stored to LDS later.
    static constexpr int QV = (ROWS * (D / 8) + kSpThreads - 1) / kSpThreads;
    __device__ static void fetch_q(const SpArgs &a, const SpItem &it, u32x4 *qr)
    {
        const int r = a.n_h / a.n_kv;
        const uint16_t *q0 = a.q_win + (size_t)(it.b * a.n_h + it.g * r) * a.w * D;
        constexpr int VPR = D / 8;
#pragma unroll
        for (int v = 0; v < QV; ++v) {
            const int i = min((int)kvc_tid() + v * kSpThreads, ROWS * VPR - 1);
            const int row = i / VPR, col = i - row * VPR;
            qr[v] = *((const u32x4 *)(q0 + (size_t)min(row, a.R - 1) * D) + col);
        }
    }
    __device__ static void store_q(const u32x4 *qr, unsigned char *q_lds)
    {
        constexpr int VPR = D / 8;
#pragma unroll
        for (int v = 0; v < QV; ++v) {
            const int i = (int)kvc_tid() + v * kSpThreads;
            const int row = i / VPR, col = i - row * VPR;
            if ((ROWS * VPR) % kSpThreads == 0 || i < ROWS * VPR) *(u32x4 *)(q_lds + row * QROWB + col * 16) = qr[v];
        }
    }

    // Which (row, token) pairs are visible: row r < R sees token t when t <= last(r)
    // (the causal window mask); every row r < R sees every token t <= lo.
    struct Vis {
        int R, S, w, wic, lo;
        __device__ Vis(const SpArgs &a, const SpItem &it)
            : R(a.R), S(it.S), w(a.w), wic(a.wic), lo(a.wic ? it.S - a.w : it.S - 1) {}
        __device__ int last(int r) const { return r >= R ? -1 : (wic ? min(S - w + r % w, S - 1) : S - 1); }
    };

    // Logits of one tile from its LDS slot: lane (kg, n) holds token t = tb + n for rows
    // cb*16 + 4 kg + jj; invisible (row, token) pairs are -inf.  Tiles wholly at or before
    // vis.lo mask only rows >= R; the others (the window's tail) evaluate the mask per row.
    __device__ static void tile_logits(const unsigned char *slot, const unsigned char *q_lds, int tb, int n, int kg,
                                       const Vis &vis, float (*lg)[4])
    {
        u32x4 kb[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s)
            kb[s] = *(const u32x4 *)(slot + n * (2 * D) + (((4 * s + kg) ^ (n % CPR)) * 16));
        const int t = tb + n;
#pragma unroll
        for (int cb = 0; cb < RT; ++cb) {
            f32x4_t acc = {};
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4 qv = *(const u32x4 *)(q_lds + (cb * 16 + n) * QROWB + (4 * s + kg) * 16);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qv), as_bf16x8(kb[s]), acc, 0, 0, 0);
            }
            if (tb + 15 <= vis.lo) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) lg[cb][jj] = cb * 16 + 4 * kg + jj < vis.R ? acc[jj] : -INFINITY;
            } else {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) lg[cb][jj] = t <= vis.last(cb * 16 + 4 * kg + jj) ? acc[jj] : -INFINITY;
            }
        }
    }

    // The item's raw scores from its logits and the unit's final (-M c, 1/L).
    __device__ static void finish(const SpArgs &a, const SpItem &it, const float (*lg)[RT][4], const float2 *fin,
                                  int wv, int n, int kg)
    {
        float nmc[RT][4], il[RT][4];
#pragma unroll
        for (int cb = 0; cb < RT; ++cb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float2 f = fin[cb * 16 + 4 * kg + jj];
                nmc[cb][jj] = f.x;
                il[cb][jj] = f.y;
            }
        const int tw = wave_t0(it, wv);
        float *out = a.raw + (size_t)it.u * a.s_max;
#pragma unroll
        for (int p = 0; p < kSpTiles; ++p) {
            float v0 = 0.f, v1 = 0.f;
#pragma unroll
            for (int cb = 0; cb < RT; ++cb) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float e = fast_exp2(fmaf(lg[p][cb][jj], a.c, nmc[cb][jj]));   // -inf: 0
                    if (jj & 1) v1 = fmaf(e, il[cb][jj], v1);
                    else v0 = fmaf(e, il[cb][jj], v0);
                }
            }
            const float v = v0 + v1;
            const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            const float v2 = __uint_as_float(h[0]) + __uint_as_float(h[1]);
            const auto q = __builtin_amdgcn_permlane16_swap(__float_as_uint(v2), __float_as_uint(v2), false, false);
            const float v4 = __uint_as_float(q[0]) + __uint_as_float(q[1]);
            const int t = tw + 16 * p + n;
            if (kg == 0 && t < a.s_max) out[t] = t < it.S ? v4 : 0.f;
        }
    }
};

// The unit's final per-row (-M c, 1/L) from its items' records, merged in item order
// (a thread per (row, slice of items), every record load of a thread in flight at
// once, then the slices in order); left in fin[ROWS] in LDS.  Every thread calls it.
template <int ROWS>
__device__ __forceinline__ void sp_merge(const SpArgs &a, int u, int n_u, bool dev, float *mg_m, double *mg_l,
                                         float2 *fin)
{
    constexpr int SL = kSpThreads / ROWS;
    constexpr int PER = 8;                                // records per thread per batch
    const int tid = kvc_tid();
    const int row = tid % ROWS, sl = tid / ROWS;
    const unsigned long long *rp = a.rec + (size_t)u * a.n_chunks * ROWS + row;
    float M = -INFINITY;
    double L = 0.0;
    for (int c0 = sl; c0 < n_u; c0 += PER * SL) {
        unsigned long long v[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const unsigned long long *p = rp + (size_t)min(c0 + q * SL, n_u - 1) * ROWS;
            v[q] = dev ? ld_dev(p) : *p;
        }
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (c0 + q * SL >= n_u) continue;
            const float m2 = unpack_lo(v[q]), l2 = unpack_hi(v[q]);
            if (m2 == -INFINITY) continue;
            if (m2 > M) {
                L = L * (double)fast_exp2((M - m2) * a.c) + (double)l2;
                M = m2;
            } else {
                L += (double)l2 * (double)fast_exp2((m2 - M) * a.c);
            }
        }
    }
    mg_m[tid] = M;
    mg_l[tid] = L;
    __syncthreads();
    if (tid < ROWS) {
        float Mt = -INFINITY;
        for (int s2 = 0; s2 < SL; ++s2) Mt = fmaxf(Mt, mg_m[s2 * ROWS + tid]);
        float2 res = make_float2(0.f, 0.f);
        if (tid < a.R && Mt != -INFINITY) {
            double Lt = 0.0;
            for (int s2 = 0; s2 < SL; ++s2) {
                const float ms = mg_m[s2 * ROWS + tid];
                if (ms != -INFINITY) Lt += mg_l[s2 * ROWS + tid] * (double)fast_exp2((ms - Mt) * a.c);
            }
            if (Lt > 0.0) res = make_float2(-Mt * a.c, (float)(1.0 / Lt));
        }
        fin[tid] = res;
    }
    __syncthreads();
}

// The item's 16 tiles of one wave through the ring: before tile P is read, only the
// loads of the tiles issued after it may still be in flight; once its LDS reads have
// returned, its slot is refilled with tile P + 4.
template <int D, int RT, int P>
__device__ __forceinline__ void sp_tiles(__amdgpu_buffer_rsrc_t rs, unsigned char *const *slot,
                                         const unsigned char *q_lds, int tw, int n, int kg,
                                         const typename Sp<D, RT>::Vis &vis, float (*lg)[RT][4])
{
    if constexpr (P < kSpTiles) {
        using S = Sp<D, RT>;
        constexpr int later = (P + kSpRing < kSpTiles ? P + kSpRing : kSpTiles) - (P + 1);
        vm_wait<S::KS * later>();
        S::tile_logits(slot[P % kSpRing], q_lds, tw + 16 * P, n, kg, vis, lg[P]);
        if constexpr (P + kSpRing < kSpTiles) {
            lds_reads_done();
            S::load_tile(rs, tw + 16 * (P + kSpRing), n, kg, slot[P % kSpRing]);
        }
        sp_tiles<D, RT, P + 1>(rs, slot, q_lds, tw, n, kg, vis, lg);
    }
}

template <int D, int RT>
__global__ __launch_bounds__(kSpThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_single_kernel(SpArgs a)
{
    using P = Sp<D, RT>;
    constexpr int ROWS = P::ROWS;
    __shared__ __attribute__((aligned(16))) unsigned char ring0[kSpWaves * P::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char ring1[kSpWaves * P::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char ring2[kSpWaves * P::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char ring3[kSpWaves * P::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char q_lds[ROWS * P::QROWB];
    __shared__ float sm_m[kSpWaves][ROWS];
    __shared__ float sm_l[kSpWaves][ROWS];
    __shared__ double mg_l[kSpThreads];
    __shared__ float mg_m[kSpThreads];
    __shared__ float2 sh_fin[ROWS];
    __shared__ int sh_int[2];

    const int tid = kvc_tid();
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, kg = lane >> 4;
    // the wave's four ring slots, one LDS array each so that reading one slot waits only
    // for the loads into it
    unsigned char *const slot[kSpRing] = {ring0 + wv * P::SLOT, ring1 + wv * P::SLOT, ring2 + wv * P::SLOT,
                                          ring3 + wv * P::SLOT};

    float lg[kSpTiles][RT][4];
    u32x4 qr[P::QV];
    SpItem prev;
    prev.active = false;
    // this call's tag: the pooling kernel advances the word after every call
    const uint32_t tag = (uint32_t)ld_uniform(a.tag, 0) + 1u;

    // an item's query rows (to registers) and first ring of K tiles, issued ahead of it;
    // issued for every item (an inactive one reads unit 0's queries and no K: an empty
    // range), so that the same number of loads is in flight on every path
    auto prefetch = [&](const SpItem &x) {
        SpItem y = x;
        if (!x.active) {
            y.u = y.b = y.g = 0;
            y.t0 = 0;
        }
        P::fetch_q(a, y, qr);
        const __amdgpu_buffer_rsrc_t rs =
            buffer_rsrc(a.k + (size_t)y.u * a.s_max * D, x.active ? x.S * (2 * D) : 0);
#pragma unroll
        for (int p = 0; p < kSpRing; ++p) P::load_tile(rs, P::wave_t0(y, wv) + 16 * p, n, kg, slot[p]);
    };

    SpItem it;
    it.active = false;
    it.zero = false;
    if ((int)kvc_bid_x() < a.n_items) it = sp_item(a, kvc_bid_x());
    prefetch(it);
    for (int j = kvc_bid_x();; j += a.G) {
        const bool have = j < a.n_items;

        // ---- B: the previous item, once its unit's statistics are final
        if (prev.active) {
            if (wv == 0) {
                // lane l < 2 ROWS polls word l of the unit's final statistics until every
                // word carries this call's tag, for at most a.spin ticks of the 100 MHz
                // real-time counter
                const bool mine = lane < 2 * ROWS;
                const unsigned long long *fp = a.fin + (size_t)prev.u * ROWS * 2 + (mine ? lane : 0);
                unsigned long long f = 0;
                int ok = 0;
                if (a.spin) {
                    const uint64_t t_end = __builtin_amdgcn_s_memrealtime() + (uint64_t)a.spin;
                    for (;;) {
                        f = ld_dev(fp);
                        if (__builtin_amdgcn_ballot_w64(mine && tag_of(f) != tag) == 0) {
                            ok = 1;
                            break;
                        }
                        if (__builtin_amdgcn_s_memrealtime() >= t_end) break;
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                if (ok) {
                    if (mine) reinterpret_cast<float *>(sh_fin)[lane] = __uint_as_float((uint32_t)f);
                } else if (lane == 0) {
                    const int slot_i = __hip_atomic_fetch_add(a.defer_n, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    a.defer[slot_i] = (int)(prev.u * a.n_chunks + prev.ch);
                }
                if (lane == 0) sh_int[0] = ok;
            }
            lds_barrier();
            if (sh_int[0]) P::finish(a, prev, lg, sh_fin, wv, n, kg);
        }
        if (!have) break;
        if (it.zero) {
            float *out = a.raw + (size_t)it.u * a.s_max;
            for (int t = it.t0 + tid; t < it.t0 + kSpItem && t < a.s_max; t += kSpThreads) out[t] = 0.f;
        }
        prev = it;
        const int jn = j + a.G;
        SpItem nx;
        nx.active = false;
        nx.zero = false;
        if (jn < a.n_items) nx = sp_item(a, jn);
        if (!it.active) {
            prefetch(nx);
            it = nx;
            continue;
        }

        // ---- A: this item's logits and per-row statistics, published as its record
        lds_barrier();                   // no wave still reads the previous item's queries
        P::store_q(qr, q_lds);
        lds_barrier();
        {
            const typename P::Vis vis(a, it);
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.k + (size_t)it.u * a.s_max * D, it.S * (2 * D));
            sp_tiles<D, RT, 0>(rs, slot, q_lds, P::wave_t0(it, wv), n, kg, vis, lg);
        }
#pragma unroll
        for (int cb = 0; cb < RT; ++cb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float m = lg[0][cb][jj];
#pragma unroll
                for (int p = 1; p < kSpTiles; ++p) m = fmaxf(m, lg[p][cb][jj]);
                m = row16_max(m);
                if (n == 0) sm_m[wv][cb * 16 + 4 * kg + jj] = m;
            }
        lds_barrier();
#pragma unroll
        for (int cb = 0; cb < RT; ++cb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int r = cb * 16 + 4 * kg + jj;
                float m = sm_m[0][r];
#pragma unroll
                for (int x = 1; x < kSpWaves; ++x) m = fmaxf(m, sm_m[x][r]);
                float s0 = 0.f, s1 = 0.f;
                if (m != -INFINITY) {
                    const float nm = -m * a.c;
#pragma unroll
                    for (int p = 0; p < kSpTiles; p += 2) {
                        s0 += fast_exp2(fmaf(lg[p][cb][jj], a.c, nm));
                        s1 += fast_exp2(fmaf(lg[p + 1][cb][jj], a.c, nm));
                    }
                }
                const float s = row16_sum(s0 + s1);
                if (n == 0) sm_l[wv][r] = s;
            }
        lds_barrier();
        if (tid < ROWS) {
            float m = sm_m[0][tid];
            for (int x = 1; x < kSpWaves; ++x) m = fmaxf(m, sm_m[x][tid]);
            float l = 0.f;
            for (int x = 0; x < kSpWaves; ++x) l += sm_l[x][tid];
            st_dev(a.rec + ((size_t)it.u * a.n_chunks + it.ch) * ROWS + tid, pack2(m, l));
            stores_done();               // the record lands before the arrival announces it
        }
        lds_barrier();
        const int n_u = (it.S + kSpItem - 1) / kSpItem;
        int old = 0;
        if (tid == 0) old = __hip_atomic_fetch_add(a.arrive + it.u, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the next item's queries and first K tiles fly from here on, across the previous
        // item's wait and finish
        prefetch(nx);
        if (tid == 0) sh_int[1] = old == n_u - 1;
        lds_barrier();
        if (sh_int[1]) {
            // the unit's last item: merge the records, publish the tagged final statistics
            sp_merge<ROWS>(a, it.u, n_u, true, mg_m, mg_l, sh_fin);
            if (tid < 2 * ROWS) {
                const float2 f = sh_fin[tid >> 1];
                st_dev(a.fin + ((size_t)it.u * ROWS + (tid >> 1)) * 2 + (tid & 1), tagged((tid & 1) ? f.y : f.x, tag));
            }
        }
        it = nx;
    }
}

// Items whose wait ran out: recomputed from K (the same logits) with the unit's
// statistics merged from its records, every record being written by now (a kernel
// boundary later).  Work-group i takes deferred items i, i + grid, ...; the pooling
// kernel that follows returns the arrival counters and the deferred count to zero.
template <int D, int RT>
__global__ __launch_bounds__(kSpThreads) void mfma_single_fixup_kernel(SpArgs a)
{
    using P = Sp<D, RT>;
    constexpr int ROWS = P::ROWS;
    __shared__ __attribute__((aligned(16))) unsigned char ring0[kSpWaves * P::SLOT];
    __shared__ __attribute__((aligned(16))) unsigned char q_lds[ROWS * P::QROWB];
    __shared__ double mg_l[kSpThreads];
    __shared__ float mg_m[kSpThreads];
    __shared__ float2 sh_fin[ROWS];
    const int tid = kvc_tid();
    const int lane = tid & 63, wv = tid >> 6;
    const int n = lane & 15, kg = lane >> 4;
    unsigned char *const slot = ring0 + wv * P::SLOT;
    const int nd = *a.defer_n;
    for (int i = kvc_bid_x(); i < nd; i += a.fix_g) {
        const SpItem it = sp_item(a, a.defer[i]);
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(a.k + (size_t)it.u * a.s_max * D, it.S * (2 * D));
        const int tw = P::wave_t0(it, wv);
        float lg[kSpTiles][RT][4];
        u32x4 qr[P::QV];
        P::fetch_q(a, it, qr);
        P::store_q(qr, q_lds);
        sp_merge<ROWS>(a, it.u, (it.S + kSpItem - 1) / kSpItem, false, mg_m, mg_l, sh_fin);   // orders q_lds too
        const typename P::Vis vis(a, it);
#pragma unroll
        for (int p = 0; p < kSpTiles; ++p) {
            lds_reads_done();
            P::load_tile(rs, tw + 16 * p, n, kg, slot);
            vm_wait<0>();
            P::tile_logits(slot, q_lds, tw + 16 * p, n, kg, vis, lg[p]);
        }
        P::finish(a, it, lg, sh_fin, wv, n, kg);
        __syncthreads();
    }
}

template <int D, int RT>
void launch_mfma_group(const MfArgs &a, int group_units, hipStream_t stream)
{
    using C = Sc<D, RT>;
    dim3 grid(a.n_chunks, group_units);
    static_assert(C::LDS_BYTES >= kMfThreads * (sizeof(float) + sizeof(double)), "merge state fits the stages");
    hipLaunchKernelGGL((mfma_stats_kernel<D, RT>), grid, dim3(kMfThreads), C::LDS_BYTES, stream, a);
    if (!a.arrive) {
        if constexpr (RT == 1)
            hipLaunchKernelGGL((mfma_merge_parts_kernel<RT * 16>), dim3(group_units), dim3(kMfThreads), 0, stream, a);
        else
            hipLaunchKernelGGL(mfma_merge_kernel, dim3(group_units), dim3(kMergeThreads), 0, stream,
                               (const float2 *)a.part, a.n_parts, RT * 16, a.R, a.c,
                               a.mask ? a.mask + a.unit0 : nullptr, a.fin);
    }
    if (RT == 1 && a.logits) {
        // pass 2 fused with the pooling
        const dim3 pgrid((a.s_max + kPoolTile - 1) / kPoolTile, group_units);
        if (a.s_max % 4 == 0 && ((uintptr_t)a.raw & 15) == 0 && ((uintptr_t)a.pooled & 15) == 0)
            launch_logit_pool<true>(pgrid, a, stream);
        else
            launch_logit_pool<false>(pgrid, a, stream);
    } else {
        hipLaunchKernelGGL((mfma_probsum_kernel<D, RT>), grid, dim3(kMfThreads),
                           C::LDS_BYTES + (size_t)a.chunk_tokens * sizeof(float), stream, a);
    }
}

template <int D>
void launch_mfma_group_rt(int rt, const MfArgs &a, int group_units, hipStream_t stream)
{
    switch (rt) {
    case 1: launch_mfma_group<D, 1>(a, group_units, stream); break;
    case 2: launch_mfma_group<D, 2>(a, group_units, stream); break;
    case 4: launch_mfma_group<D, 4>(a, group_units, stream); break;
    default: launch_mfma_group<D, 8>(a, group_units, stream); break;
    }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the single-pass path: the words that must be zero between calls come
// first and depend on the unit count only.
struct SpLayout {
    size_t arrive_off, defer_n_off, tag_off, defer_off, rec_off, fin_off, bytes;
};

// The arrival counters and the deferred count (units + 1 words, zero between calls)
// open the workspace; the tag word follows (zero before first use, advanced by the
// pooling kernel after every call).  Final statistics are two tagged words per row.
SpLayout sp_layout(int units, int n_chunks, int rows)
{
    SpLayout L;
    size_t off = 0;
    L.arrive_off = off;
    off += (size_t)units * sizeof(int32_t);
    L.defer_n_off = off;
    off += sizeof(int32_t);
    L.tag_off = off;
    off = align256(off + sizeof(int32_t));
    L.defer_off = off;
    off = align256(off + (size_t)units * n_chunks * sizeof(int32_t));
    L.rec_off = off;
    off = align256(off + (size_t)units * n_chunks * rows * sizeof(unsigned long long));
    L.fin_off = off;
    off = align256(off + (size_t)units * rows * 2 * sizeof(unsigned long long));
    L.bytes = off;
    return L;
}

// Work-groups of the single-pass kernel that fit the current device at once (cached
// per device and instance).
template <int D, int RT>
hipError_t sp_capacity(long *cap)
{
    static std::mutex mu;
    static long cache[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 64 && cache[dev]) {
        *cap = cache[dev];
        return hipSuccess;
    }
    DeviceInfo di;
    if ((e = device_info(&di)) != hipSuccess) return e;
    int nb = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void *>(mfma_single_kernel<D, RT>),
                                                     kSpThreads, 0);
    if (e != hipSuccess) return e;
    *cap = (long)nb * di.cus;
    if (dev >= 0 && dev < 64) cache[dev] = *cap;
    return hipSuccess;
}

// Launches the single-pass kernel and its follow-up; *done = false (nothing launched)
// when a unit's items would not fit one resident round.
template <int D, int RT>
hipError_t launch_single(const SpArgs &a0, bool *done, hipStream_t stream)
{
    *done = false;
    long cap = 0;
    hipError_t e = sp_capacity<D, RT>(&cap);
    if (e != hipSuccess) return e;
    if (cap < a0.n_chunks) return hipSuccess;
    SpArgs a = a0;
    long G = cap < a.n_items ? cap : a.n_items;
    G = G / a.n_chunks * a.n_chunks;
    a.G = (int)G;
    // the follow-up kernel usually finds no deferred item: a small grid keeps its launch
    // cheap, and its work-groups stride over whatever was deferred
    a.fix_g = (int)(G < kSpFixGroups ? G : kSpFixGroups);
    hipLaunchKernelGGL((mfma_single_kernel<D, RT>), dim3((unsigned)G), dim3(kSpThreads), 0, stream, a);
    hipLaunchKernelGGL((mfma_single_fixup_kernel<D, RT>), dim3((unsigned)a.fix_g), dim3(kSpThreads), 0, stream, a);
    *done = true;
    return hipGetLastError();
}

}  // namespace

ScorePlan plan_score(int batch, int s_max, int n_h, int n_kv, int d_h, bool bf16, int w, bool generic, int cus)
{
    ScorePlan p;
    p.R = (n_h / n_kv) * w;
    const int units = batch * n_kv;
    p.mfma = !generic && bf16 && (d_h == 64 || d_h == 128) && p.R <= 128;
    if (p.mfma) {
        const int rt = p.R <= 16 ? 1 : (p.R <= 32 ? 2 : (p.R <= 64 ? 4 : 8));
        p.rt = rt;
        const int rpad = rt * 16;
        // every unit in one launch: the second pass streams K from HBM again either
        // way (measured: keeping a group's K within the MALL size does not make the
        // re-read faster), and one launch amortises the kernel boundaries
        p.group_units = units;
        // tokens per work-group: the largest of 2048, 1024, 512, 256 that still gives
        // at least four work-groups per CU (a multiple of every stage size)
        int ct_tok = kMaxChunk;
        while (ct_tok > 256) {
            const long chunks = (s_max + ct_tok - 1) / ct_tok;
            if (chunks * p.group_units >= 4L * cus) break;
            ct_tok >>= 1;
        }
        p.tiles_per_wave = 0;
        p.chunk_tokens = ct_tok;
        p.n_chunks = (s_max + ct_tok - 1) / ct_tok;
        p.n_parts = rt == 1 ? (s_max + kStatBlock - 1) / kStatBlock : p.n_chunks;
        // a few chunks per unit in one round of work-groups: the unit's last arriving
        // pass-1 work-group merges the chunks, one launch less.  With more chunks or
        // rounds, publishing every work-group's partials device-coherently and waiting
        // for its arrival count cost more than the merge kernel (measured: twice the
        // pass-1 time at 128 chunks of a KV head, +15% over four rounds)
        p.fold_merge = p.n_chunks <= 8 && (long)p.n_chunks * p.group_units <= 4L * cus;
        // row partials, merged row statistics, chunk arrival counters (zero between calls)
        p.ws_bytes = align256((size_t)p.group_units * p.n_parts * rpad * sizeof(float2)) +
                     align256((size_t)p.group_units * rpad * sizeof(float2)) +
                     align256((size_t)p.group_units * sizeof(int32_t)) + 256;
        // a single row block (R <= 16): pass 1 keeps its logits, 4 * rs bytes per token,
        // and pass 2 reads those instead of K's 2 * d_h bytes
        p.logit_rows = rt == 1 ? (p.R + 3) / 4 * 4 : 0;
        p.logits_off = p.ws_bytes;
        if (p.logit_rows) p.ws_bytes += align256((size_t)units * s_max * p.logit_rows * sizeof(float));
        const long items = ((long)s_max + kSpItem - 1) / kSpItem;
        if (rt == 2 && items <= 128) {
            // one pass over K for 17..32 rows: a resident grid of at least half a
            // work-group per CU holds a unit's items (at most 128 of 1024 tokens) in one
            // round.  A single row block (R <= 16) keeps the two-kernel path above, whose
            // second kernel reads 4 R bytes of logits per token instead of K: measured
            // faster for one query per head of the batched ragged decode
            p.single = true;
            p.sp_chunks = (int)items;
            p.sp_item = kSpItem;
            const SpLayout L = sp_layout(units, p.sp_chunks, rpad);
            p.two_pass_off = L.bytes;
            p.logits_off += L.bytes;
            p.ws_bytes += L.bytes;
        }
    } else {
        p.group_units = units;
        p.ws_bytes = align256((size_t)units * p.R * s_max * sizeof(float)) +
                     align256((size_t)units * p.R * sizeof(float2)) + 256;
    }
    return p;
}

hipError_t launch_score(int batch, int s_max, const int32_t *seq_lens, int n_h, int n_kv, int d_h, bool bf16,
                        const void *q_win, const void *k, int w, bool window_in_cache, int n_keep, int pool,
                        float scale, float *raw, float *pooled, const int32_t *unit_mask, void *ws,
                        const ScorePlan &plan, hipStream_t stream)
{
    const int units = batch * n_kv;
    void *const ws_base = ws;
    bool single_done = false;
    if (plan.mfma && plan.single) {
        const SpLayout L = sp_layout(units, plan.sp_chunks, plan.rt * 16);
        char *w8 = (char *)ws;
        SpArgs a;
        a.q_win = (const uint16_t *)q_win;
        a.k = (const uint16_t *)k;
        a.seq_lens = seq_lens;
        a.mask = unit_mask;
        a.s_max = s_max;
        a.n_h = n_h;
        a.n_kv = n_kv;
        a.w = w;
        a.wic = window_in_cache ? 1 : 0;
        a.R = plan.R;
        a.n_chunks = plan.sp_chunks;
        a.n_items = units * plan.sp_chunks;
        a.G = 0;
        a.spin = plan.sp_spin;
        a.c = scale * kLog2e;
        a.raw = raw;
        a.arrive = (int32_t *)(w8 + L.arrive_off);
        a.defer_n = (int32_t *)(w8 + L.defer_n_off);
        a.tag = (const int32_t *)(w8 + L.tag_off);
        a.fin = (unsigned long long *)(w8 + L.fin_off);
        a.defer = (int32_t *)(w8 + L.defer_off);
        a.rec = (unsigned long long *)(w8 + L.rec_off);
        hipError_t e;
        if (d_h == 128) e = plan.rt == 1 ? launch_single<128, 1>(a, &single_done, stream)
                                         : launch_single<128, 2>(a, &single_done, stream);
        else e = plan.rt == 1 ? launch_single<64, 1>(a, &single_done, stream)
                              : launch_single<64, 2>(a, &single_done, stream);
        if (e != hipSuccess) return e;
    }
    if (plan.mfma && !single_done) {
        const int rt = plan.rt;
        const int rpad = rt * 16;
        ws = (char *)ws + plan.two_pass_off;
        MfArgs a;
        a.q_win = (const uint16_t *)q_win;
        a.k = (const uint16_t *)k;
        a.seq_lens = seq_lens;
        a.s_max = s_max;
        a.n_h = n_h;
        a.n_kv = n_kv;
        a.w = w;
        a.wic = window_in_cache ? 1 : 0;
        a.R = plan.R;
        a.n_chunks = plan.n_chunks;
        a.chunk_tokens = plan.chunk_tokens;
        a.n_parts = plan.n_parts;
        // ragged lengths with one row block: the valid chunks first (units in one group).
        // Not for a masked call, whose work-groups mostly exit at their first load: the
        // mapping's walk over the lengths would delay every one of them
        a.compact_batch = rt == 1 && seq_lens && !unit_mask && batch <= 64 && plan.group_units == units ? batch : 0;
        a.c = scale * kLog2e;
        const size_t fin_off = align256((size_t)plan.group_units * plan.n_parts * rpad * sizeof(float2));
        a.part = (float2 *)ws;
        a.fin = (float2 *)((char *)ws + fin_off);
        int32_t *arrive = (int32_t *)((char *)ws + fin_off + align256((size_t)plan.group_units * rpad * sizeof(float2)));
        a.arrive = plan.fold_merge ? arrive : nullptr;
        if (rt == 1 && unit_mask) {
            // a call for some KV heads (a correction): work-groups of one 256-token block,
            // so a KV head is spread over many CUs, and the last one merges.  The
            // partials are per block whatever the chunks: the same bits as a full call
            a.chunk_tokens = kStatBlock;
            a.n_chunks = (s_max + kStatBlock - 1) / kStatBlock;
            a.arrive = arrive;
        }
        a.raw = raw;
        a.pooled = pooled;
        a.n_keep = n_keep;
        a.half = pool / 2;
        a.mask = unit_mask;
        a.rs = plan.logit_rows;
        a.logits = plan.logit_rows ? (float *)((char *)ws + plan.logits_off - plan.two_pass_off) : nullptr;
        for (int u0 = 0; u0 < units; u0 += plan.group_units) {
            const int gu = min(plan.group_units, units - u0);
            a.unit0 = u0;
            if (d_h == 128) launch_mfma_group_rt<128>(rt, a, gu, stream);
            else launch_mfma_group_rt<64>(rt, a, gu, stream);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    } else if (!plan.mfma) {
        float *logits = (float *)ws;
        float2 *fin = (float2 *)((char *)ws + align256((size_t)units * plan.R * s_max * sizeof(float)));
        dim3 gtok((s_max + kGenThreads - 1) / kGenThreads, units);
        if (bf16) {
            if (d_h == 128) hipLaunchKernelGGL((gen_logits_kernel<true, 128>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, unit_mask, logits);
            else hipLaunchKernelGGL((gen_logits_kernel<true, 64>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, unit_mask, logits);
        } else {
            if (d_h == 128) hipLaunchKernelGGL((gen_logits_kernel<false, 128>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, unit_mask, logits);
            else hipLaunchKernelGGL((gen_logits_kernel<false, 64>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, unit_mask, logits);
        }
        hipLaunchKernelGGL(gen_rowstats_kernel, dim3(plan.R, units), dim3(kGenThreads), 0, stream, logits, s_max,
                           plan.R, unit_mask, fin);
        hipLaunchKernelGGL(gen_probsum_kernel, gtok, dim3(kGenThreads), 0, stream, logits, (const float2 *)fin,
                           seq_lens, s_max, n_kv, plan.R, 0, unit_mask, raw);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // the two-pass kernels of one row block pool in their second pass
    if (plan.mfma && !single_done && plan.logit_rows) return hipGetLastError();
    // after the single-pass kernels the pooling kernel zeroes their arrival counters and
    // deferred count (laid out first in the workspace: units + 1 words) and advances the
    // tag word after them
    int32_t *reset = single_done ? (int32_t *)ws_base : nullptr;
    launch_pool(raw, seq_lens, s_max, units, n_kv, n_keep, pool / 2, unit_mask, pooled, reset, units + 1, stream);
    return hipGetLastError();
}

}  // namespace kvc
