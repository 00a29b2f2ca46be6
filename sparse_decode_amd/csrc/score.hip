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
//   pass 1  logits -> per-row (max, sum of exp) for one chunk of tokens
//   merge   chunk partials -> (M_r, 1/L_r) per row, in chunk order, in double
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
                                                            float *__restrict__ pooled)
{
    // 2 kMaxHalf + 2 slots (left halo, then 16-byte alignment), the body, the right halo
    __shared__ __attribute__((aligned(16))) float tile[2 * kMaxHalf + 2 + kPoolTile + kMaxHalf + 1];
    if constexpr (HALF >= 0) half = HALF;
    const int u = kvc_bid_y();
    if (mask && !ld_uniform(mask, u)) return;
    const int S = clamp_len(seq_lens, u / n_kv, s_max);
    const int C = S - n_keep > 0 ? S - n_keep : 0;
    const int t0 = kvc_bid_x() * kPoolTile;
    const float *rw = raw + (size_t)u * s_max;
    float *out = pooled + (size_t)u * s_max;
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

template <bool VEC>
void launch_pool_vec(dim3 grid, const float *raw, const int32_t *seq_lens, int s_max, int n_kv, int n_keep, int half,
                     const int32_t *mask, float *pooled, hipStream_t stream)
{
    switch (half) {
    case 0: hipLaunchKernelGGL((pool_kernel<VEC, 0>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled); break;
    case 1: hipLaunchKernelGGL((pool_kernel<VEC, 1>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled); break;
    case 2: hipLaunchKernelGGL((pool_kernel<VEC, 2>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled); break;
    case 3: hipLaunchKernelGGL((pool_kernel<VEC, 3>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled); break;
    default: hipLaunchKernelGGL((pool_kernel<VEC, -1>), grid, dim3(kPoolThreads), 0, stream, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled); break;
    }
}

void launch_pool(const float *raw, const int32_t *seq_lens, int s_max, int units, int n_kv, int n_keep, int half,
                 const int32_t *mask, float *pooled, hipStream_t stream)
{
    const dim3 grid((s_max + kPoolTile - 1) / kPoolTile, units);
    if (s_max % 4 == 0 && ((uintptr_t)raw & 15) == 0 && ((uintptr_t)pooled & 15) == 0)
        launch_pool_vec<true>(grid, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, stream);
    else
        launch_pool_vec<false>(grid, raw, seq_lens, s_max, n_kv, n_keep, half, mask, pooled, stream);
}

// ====================================================================================
// bf16 MFMA path
// ====================================================================================
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kMfThreads = 256;
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
    float2 *part;            // pass 1 out: [group][chunk][RT*16] (m, l)
    const float2 *fin;       // pass 2 in:  [group][RT*16] (-M*c, 1/L)
    float *raw;              // pass 2 out: [B*n_kv][s_max]
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

template <int D, int RT>
__global__ __launch_bounds__(kMfThreads) __attribute__((amdgpu_waves_per_eu(4))) void mfma_stats_kernel(MfArgs a)
{
    using C = Sc<D, RT>;
    constexpr int KS = C::KS;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    unsigned char *kbuf = lds;                           // 2 stages
    __shared__ float sm_m[C::TG][RT * 16];
    __shared__ float sm_l[C::TG][RT * 16];

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
    stream_stages<D, RT, true>(kunit, ch0, n_st, kbuf,
        [&](const unsigned char *cur, int st) {
            const int st0 = ch0 + st * C::ST;
            if (st0 + C::ST - 1 <= all_vis)
                stats_stage<D, RT, false>(cur, st0, tg, n, kg, qb, last, a.c, m, l, lg, a.rs, S);
            else
                stats_stage<D, RT, true>(cur, st0, tg, n, kg, qb, last, a.c, m, l, lg, a.rs, S);
        },
        [&](int) {});
    // merge the four lane groups of a row (lanes n, n+16, n+32, n+48), then the token groups
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
        a.part[((size_t)ul * a.n_chunks + chunk) * (RT * 16) + row] = make_float2(Mx, L);
    }
}

// Merges the chunk partials of every row in a fixed order.  blockDim = 1024:
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

// Pass 2 from the logits pass 1 kept (a single row block of at most 16 rows): per
// token, raw = sum over rows, in row order, of exp2(x c - M c) / L.  Each thread reads
// one token's rs consecutive logits; no K is read again.
constexpr int kLogitThreads = 256;

__global__ __launch_bounds__(kLogitThreads) void logit_probsum_kernel(const float *__restrict__ logits,
                                                                      const float2 *__restrict__ fin,
                                                                      const int32_t *__restrict__ seq_lens,
                                                                      int s_max, int n_kv, int R, int rs, int rpad,
                                                                      int unit0, float c,
                                                                      const int32_t *__restrict__ mask,
                                                                      float *__restrict__ raw)
{
    __shared__ float2 f[16];
    const int ul = kvc_bid_y();
    const int u = unit0 + ul;
    if (mask && !ld_uniform(mask, u)) return;
    if (kvc_tid() < 16) f[kvc_tid()] = kvc_tid() < R ? fin[(size_t)ul * rpad + kvc_tid()] : make_float2(0.f, 0.f);
    __syncthreads();
    const int S = clamp_len(seq_lens, u / n_kv, s_max);
    const int t = kvc_bid_x() * kLogitThreads + kvc_tid();
    if (t >= s_max) return;
    float acc = 0.f;
    if (t < S) {
        const float4 *x4 = (const float4 *)(logits + ((size_t)u * s_max + t) * rs);
        float x[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (4 * q < rs) {
                const float4 v = x4[q];
                x[4 * q] = v.x; x[4 * q + 1] = v.y; x[4 * q + 2] = v.z; x[4 * q + 3] = v.w;
            }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (r < R) acc = fmaf(fast_exp2(fmaf(x[r], c, f[r].x)), f[r].y, acc);
    }
    raw[(size_t)u * s_max + t] = acc;
}

template <int D, int RT>
void launch_mfma_group(const MfArgs &a, int group_units, hipStream_t stream)
{
    using C = Sc<D, RT>;
    dim3 grid(a.n_chunks, group_units);
    hipLaunchKernelGGL((mfma_stats_kernel<D, RT>), grid, dim3(kMfThreads), C::LDS_BYTES, stream, a);
    hipLaunchKernelGGL(mfma_merge_kernel, dim3(group_units), dim3(kMergeThreads), 0, stream,
                       (const float2 *)a.part, a.n_chunks, RT * 16, a.R, a.c, a.mask ? a.mask + a.unit0 : nullptr,
                       (float2 *)a.fin);
    if (RT == 1 && a.logits) {
        const dim3 lgrid((a.s_max + kLogitThreads - 1) / kLogitThreads, group_units);
        hipLaunchKernelGGL(logit_probsum_kernel, lgrid, dim3(kLogitThreads), 0, stream, (const float *)a.logits,
                           a.fin, a.seq_lens, a.s_max, a.n_kv, a.R, a.rs, RT * 16, a.unit0, a.c, a.mask, a.raw);
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

}  // namespace

ScorePlan plan_score(int batch, int s_max, int n_h, int n_kv, int d_h, bool bf16, int w, bool generic, int cus)
{
    ScorePlan p;
    p.R = (n_h / n_kv) * w;
    const int units = batch * n_kv;
    p.mfma = !generic && bf16 && (d_h == 64 || d_h == 128) && p.R <= 128;
    if (p.mfma) {
        const int rt = p.R <= 16 ? 1 : (p.R <= 32 ? 2 : (p.R <= 64 ? 4 : 8));
        const int rpad = rt * 16;
        // every unit in one launch: the second pass streams K from HBM again either
        // way (measured: keeping a group's K within the MALL size does not make the
        // re-read faster), and one launch amortises the kernel boundaries
        p.group_units = units;
        // tokens per work-group: the largest of 2048, 1024, 512, 256 that still gives
        // at least four work-groups per CU (a multiple of every stage size)
        int ct_tok = 2048;
        while (ct_tok > 256) {
            const long chunks = (s_max + ct_tok - 1) / ct_tok;
            if (chunks * p.group_units >= 4L * cus) break;
            ct_tok >>= 1;
        }
        p.tiles_per_wave = 0;
        p.chunk_tokens = ct_tok;
        p.n_chunks = (s_max + ct_tok - 1) / ct_tok;
        p.ws_bytes = align256((size_t)p.group_units * p.n_chunks * rpad * sizeof(float2)) +
                     align256((size_t)p.group_units * rpad * sizeof(float2)) + 256;
        // a single row block (R <= 16): pass 1 keeps its logits, 4 * rs bytes per token,
        // and pass 2 reads those instead of K's 2 * d_h bytes
        p.logit_rows = rt == 1 ? (p.R + 3) / 4 * 4 : 0;
        p.logits_off = p.ws_bytes;
        if (p.logit_rows) p.ws_bytes += align256((size_t)units * s_max * p.logit_rows * sizeof(float));
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
    if (plan.mfma) {
        const int rt = plan.R <= 16 ? 1 : (plan.R <= 32 ? 2 : (plan.R <= 64 ? 4 : 8));
        const int rpad = rt * 16;
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
        a.c = scale * kLog2e;
        a.part = (float2 *)ws;
        a.fin = (const float2 *)((char *)ws + align256((size_t)plan.group_units * plan.n_chunks * rpad * sizeof(float2)));
        a.raw = raw;
        a.mask = unit_mask;
        a.rs = plan.logit_rows;
        a.logits = plan.logit_rows ? (float *)((char *)ws + plan.logits_off) : nullptr;
        for (int u0 = 0; u0 < units; u0 += plan.group_units) {
            const int gu = min(plan.group_units, units - u0);
            a.unit0 = u0;
            if (d_h == 128) launch_mfma_group_rt<128>(rt, a, gu, stream);
            else launch_mfma_group_rt<64>(rt, a, gu, stream);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    } else {
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
    launch_pool(raw, seq_lens, s_max, units, n_kv, n_keep, pool / 2, unit_mask, pooled, stream);
    return hipGetLastError();
}

}  // namespace kvc
