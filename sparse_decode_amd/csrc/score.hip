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
// Units are processed in groups whose K fits the 256 MB MALL, so pass 2 re-reads K
// from the MALL rather than from HBM.
//
// The bf16 path computes logits with v_mfma_f32_32x32x16_bf16: a wave multiplies a
// 32-token K tile (A operand, loaded straight from HBM into registers, 128
// contiguous bytes per lane) by the group's Q^T (B operand, resident in registers
// for the whole chunk), giving a 32-token x 32-row fp32 tile per row block.  With
// tokens on the M side each lane owns one row, so the row statistics of pass 1 stay
// in-lane; pass 2 sums over rows across lanes with a transposed butterfly.  Both
// passes evaluate exactly the same MFMA sequence, so their logits are identical.
// Exponentials use exp2 with scale * log2(e) folded into one FMA.
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
    int s_max, int n_h, int n_kv, int w, int wic, int R, int unit0, float scale, float *__restrict__ logits)
{
    __shared__ float qs[kGenRowsLds][D];
    const int u = unit0 + blockIdx.y;
    const int b = u / n_kv;
    const int g = u - b * n_kv;
    const int r = n_h / n_kv;
    const int S = clamp_len(seq_lens, b, s_max);
    const int t = blockIdx.x * kGenThreads + threadIdx.x;
    float kr[D];
    if (t < S) load_row_f32<BF16, D>(k, (size_t)u * s_max + t, kr);
    const size_t qrow0 = (size_t)(b * n_h + g * r) * w;     // the R rows are contiguous
    float *lg = logits + (size_t)blockIdx.y * R * s_max;
    for (int r0 = 0; r0 < R; r0 += kGenRowsLds) {
        const int nr = min(kGenRowsLds, R - r0);
        __syncthreads();
        for (int x = threadIdx.x; x < nr * D; x += kGenThreads) {
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
                                                                   int R, float2 *__restrict__ fin)
{
    __shared__ float red_m[kGenThreads / kWave];
    __shared__ double red_l[kGenThreads / kWave];
    const int row = blockIdx.x;
    const int ul = blockIdx.y;
    const float *lg = logits + ((size_t)ul * R + row) * s_max;
    float m = -INFINITY;
    for (int t = threadIdx.x; t < s_max; t += kGenThreads) m = fmaxf(m, lg[t]);
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) m = fmaxf(m, shfl_xor_f(m, o));
    if ((threadIdx.x & 63) == 0) red_m[threadIdx.x >> 6] = m;
    __syncthreads();
    m = red_m[0];
    for (int i = 1; i < kGenThreads / kWave; ++i) m = fmaxf(m, red_m[i]);
    if (m == -INFINITY) {
        if (threadIdx.x == 0) fin[(size_t)ul * R + row] = make_float2(0.f, 0.f);
        return;
    }
    const float nmc = -m * kLog2e;
    float s = 0.f;
    for (int t = threadIdx.x; t < s_max; t += kGenThreads) s += fast_exp2(fmaf(lg[t], kLog2e, nmc));
    double sd = s;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) sd += __shfl_xor(sd, o, kWave);
    if ((threadIdx.x & 63) == 0) red_l[threadIdx.x >> 6] = sd;
    __syncthreads();
    if (threadIdx.x == 0) {
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
                                                                  float *__restrict__ raw)
{
    const int ul = blockIdx.y;
    const int u = unit0 + ul;
    const int S = clamp_len(seq_lens, u / n_kv, s_max);
    const int t = blockIdx.x * kGenThreads + threadIdx.x;
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
__global__ __launch_bounds__(256) void pool_kernel(const float *__restrict__ raw, const int32_t *__restrict__ seq_lens,
                                                   int s_max, int n_kv, int n_keep, int half,
                                                   float *__restrict__ pooled)
{
    const int u = blockIdx.y;
    const int S = clamp_len(seq_lens, u / n_kv, s_max);
    const int C = S - n_keep > 0 ? S - n_keep : 0;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= s_max) return;
    const float *rw = raw + (size_t)u * s_max;
    float v;
    if (t < C) {
        const int lo = t - half < 0 ? 0 : t - half;
        const int hi = t + half > C - 1 ? C - 1 : t + half;
        v = rw[lo];
        for (int x = lo + 1; x <= hi; ++x) v = fmaxf(v, rw[x]);
    } else {
        v = t < S ? rw[t] : 0.f;
    }
    pooled[(size_t)u * s_max + t] = v;
}

// ====================================================================================
// bf16 MFMA path
// ====================================================================================
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMfThreads = 256;
constexpr int kMfWaves = kMfThreads / kWave;

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4 &v) { return __builtin_bit_cast(bf16x8_t, v); }

// Token (M index) held by accumulator element j of a lane in half `h`.
__device__ __forceinline__ int acc_token(int j, int h) { return 8 * (j >> 2) + 4 * h + (j & 3); }

template <int D, int RT>
struct MfmaTile {
    static constexpr int KS = D / 16;   // MFMA k-steps; a lane covers D/2 contiguous elements

    // A operand: token row t0 + n, elements [h*D/2, h*D/2 + D/2).
    __device__ static void load_k(const uint16_t *__restrict__ kunit, int t_row, int h, u32x4 *dst)
    {
        const u32x4 *p = (const u32x4 *)(kunit + (size_t)t_row * D + h * (D / 2));
#pragma unroll
        for (int s = 0; s < KS; ++s) dst[s] = ld_stream(p + s);
    }

    __device__ static void mma(const u32x4 *ka, const bf16x8_t (*qb)[KS], f32x16_t *acc)
    {
#pragma unroll
        for (int ct = 0; ct < RT; ++ct) {
            f32x16_t a = {};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[s]), qb[ct][s], a, 0, 0, 0);
            acc[ct] = a;
        }
    }
};

struct MfArgs {
    const uint16_t *q_win;
    const uint16_t *k;
    const int32_t *seq_lens;
    int s_max, n_h, n_kv, w, wic, R, unit0, n_chunks, chunk_tokens, tiles_per_wave;
    float c;                 // scale * log2(e)
    float2 *part;            // pass 1 out: [group][chunk][RT*32] (m, l)
    const float2 *fin;       // pass 2 in:  [group][RT*32] (-M*c, 1/L)
    float *raw;              // pass 2 out: [B*n_kv][s_max]
};

// Loads this lane's B operands (Q^T) for all row blocks: row ct*32 + n, elements
// [h*D/2, h*D/2 + D/2).  Rows >= R are zero.
template <int D, int RT>
__device__ __forceinline__ void load_q(const MfArgs &a, int b, int g, int n, int h,
                                       bf16x8_t (*qb)[D / 16])
{
    constexpr int KS = D / 16;
    const int r = a.n_h / a.n_kv;
    const uint16_t *q0 = a.q_win + (size_t)(b * a.n_h + g * r) * a.w * D;
#pragma unroll
    for (int ct = 0; ct < RT; ++ct) {
        const int row = ct * 32 + n;
        if (row < a.R) {
            const u32x4 *p = (const u32x4 *)(q0 + (size_t)row * D + h * (D / 2));
#pragma unroll
            for (int s = 0; s < KS; ++s) qb[ct][s] = as_bf16x8(p[s]);
        } else {
#pragma unroll
            for (int s = 0; s < KS; ++s) qb[ct][s] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
        }
    }
}

template <int D, int RT>
__global__ __launch_bounds__(kMfThreads, 1) void mfma_stats_kernel(MfArgs a)
{
    using T = MfmaTile<D, RT>;
    constexpr int KS = T::KS;
    __shared__ float sm_m[kMfWaves][RT * 32];
    __shared__ float sm_l[kMfWaves][RT * 32];

    const int chunk = blockIdx.x;
    const int ul = blockIdx.y;
    const int u = a.unit0 + ul;
    const int b = u / a.n_kv;
    const int g = u - b * a.n_kv;
    const int S = clamp_len(a.seq_lens, b, a.s_max);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 31, h = lane >> 5;

    bf16x8_t qb[RT][KS];
    load_q<D, RT>(a, b, g, n, h, qb);

    // last visible token of this lane's row in each row block
    int last[RT];
#pragma unroll
    for (int ct = 0; ct < RT; ++ct) {
        const int row = ct * 32 + n;
        const int i = row % a.w;
        last[ct] = a.wic ? min(S - a.w + i, S - 1) : S - 1;
    }
    const int all_vis = a.wic ? S - a.w : S - 1;   // every row sees tokens <= all_vis

    float m[RT], l[RT];
#pragma unroll
    for (int ct = 0; ct < RT; ++ct) {
        m[ct] = -INFINITY;
        l[ct] = 0.f;
    }
    const uint16_t *kunit = a.k + (size_t)u * a.s_max * D;
    const int tile0 = chunk * a.chunk_tokens;

    for (int it = 0; it < a.tiles_per_wave; ++it) {
        const int t0 = tile0 + (it * kMfWaves + wv) * 32;
        if (t0 >= S) break;
        u32x4 ka[KS];
        T::load_k(kunit, min(t0 + n, S - 1), h, ka);
        f32x16_t acc[RT];
        T::mma(ka, qb, acc);
        const bool full = t0 + 31 <= all_vis;
#pragma unroll
        for (int ct = 0; ct < RT; ++ct) {
            float x[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) x[j] = acc[ct][j];
            if (!full) {
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    if (t0 + acc_token(j, h) > last[ct]) x[j] = -INFINITY;
            }
            float lm = x[0];
#pragma unroll
            for (int j = 1; j < 16; ++j) lm = fmaxf(lm, x[j]);
            const float mn = fmaxf(m[ct], lm);
            if (mn != -INFINITY) {
                const float nmc = -mn * a.c;
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) s += fast_exp2(fmaf(x[j], a.c, nmc));
                l[ct] = fmaf(l[ct], fast_exp2(fmaf(m[ct], a.c, nmc)), s);
                m[ct] = mn;
            }
        }
    }
    // merge the two lane halves (same rows, different tokens), then the waves
#pragma unroll
    for (int ct = 0; ct < RT; ++ct) {
        const float m2 = shfl_xor_f(m[ct], 32);
        const float l2 = shfl_xor_f(l[ct], 32);
        const float M = fmaxf(m[ct], m2);
        if (M != -INFINITY) {
            l[ct] = l[ct] * fast_exp2((m[ct] - M) * a.c) + l2 * fast_exp2((m2 - M) * a.c);
            m[ct] = M;
        }
        if (h == 0) {
            sm_m[wv][ct * 32 + n] = m[ct];
            sm_l[wv][ct * 32 + n] = l[ct];
        }
    }
    __syncthreads();
    for (int row = threadIdx.x; row < RT * 32; row += kMfThreads) {
        float M = -INFINITY;
        for (int w2 = 0; w2 < kMfWaves; ++w2) M = fmaxf(M, sm_m[w2][row]);
        float L = 0.f;
        if (M != -INFINITY)
            for (int w2 = 0; w2 < kMfWaves; ++w2) L += sm_l[w2][row] * fast_exp2((sm_m[w2][row] - M) * a.c);
        a.part[((size_t)ul * a.n_chunks + chunk) * (RT * 32) + row] = make_float2(M, L);
    }
}

// Merges the chunk partials of each row in chunk order, in double.
__global__ __launch_bounds__(128) void mfma_merge_kernel(const float2 *__restrict__ part, int n_chunks, int rpad,
                                                         int R, float c, float2 *__restrict__ fin)
{
    const int ul = blockIdx.y;
    const int row = blockIdx.x * 128 + threadIdx.x;
    if (row >= rpad) return;
    const float2 *p = part + (size_t)ul * n_chunks * rpad + row;
    float M = -INFINITY;
    for (int ch = 0; ch < n_chunks; ++ch) M = fmaxf(M, p[(size_t)ch * rpad].x);
    float2 res = make_float2(0.f, 0.f);
    if (row < R && M != -INFINITY) {
        double L = 0.0;
        for (int ch = 0; ch < n_chunks; ++ch) {
            const float2 v = p[(size_t)ch * rpad];
            if (v.x != -INFINITY) L += (double)v.y * exp2((double)(v.x - M) * (double)c);
        }
        if (L > 0.0) res = make_float2(-M * c, (float)(1.0 / L));
    }
    fin[(size_t)ul * rpad + row] = res;
}

template <int D, int RT>
__global__ __launch_bounds__(kMfThreads, 1) void mfma_probsum_kernel(MfArgs a)
{
    using T = MfmaTile<D, RT>;
    constexpr int KS = T::KS;
    const int chunk = blockIdx.x;
    const int ul = blockIdx.y;
    const int u = a.unit0 + ul;
    const int b = u / a.n_kv;
    const int g = u - b * a.n_kv;
    const int S = clamp_len(a.seq_lens, b, a.s_max);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n = lane & 31, h = lane >> 5;

    bf16x8_t qb[RT][KS];
    load_q<D, RT>(a, b, g, n, h, qb);
    float nmc[RT], il[RT];
    int last[RT];
#pragma unroll
    for (int ct = 0; ct < RT; ++ct) {
        const int row = ct * 32 + n;
        const float2 f = a.fin[(size_t)ul * (RT * 32) + row];
        nmc[ct] = f.x;
        il[ct] = f.y;
        const int i = row % a.w;
        last[ct] = a.wic ? min(S - a.w + i, S - 1) : S - 1;
    }
    const int all_vis = a.wic ? S - a.w : S - 1;
    const uint16_t *kunit = a.k + (size_t)u * a.s_max * D;
    float *rawu = a.raw + (size_t)u * a.s_max;
    const int tile0 = chunk * a.chunk_tokens;
    // this lane's token after the transposed reduction, and whether it writes
    const int v = 8 * ((n >> 4) & 1) + 4 * ((n >> 3) & 1) + 2 * ((n >> 2) & 1) + ((n >> 1) & 1);
    const int my_tok = acc_token(v, h);
    const bool writer = (n & 1) == 0;

    for (int it = 0; it < a.tiles_per_wave; ++it) {
        const int t0 = tile0 + (it * kMfWaves + wv) * 32;
        if (t0 >= a.s_max) break;
        if (t0 >= S) {
            if (writer && t0 + my_tok < a.s_max) rawu[t0 + my_tok] = 0.f;
            continue;
        }
        u32x4 ka[KS];
        T::load_k(kunit, min(t0 + n, S - 1), h, ka);
        f32x16_t acc[RT];
        T::mma(ka, qb, acc);
        const bool full = t0 + 31 <= all_vis;
        float cs[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) cs[j] = 0.f;
#pragma unroll
        for (int ct = 0; ct < RT; ++ct) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float e = fast_exp2(fmaf(acc[ct][j], a.c, nmc[ct]));
                if (!full && t0 + acc_token(j, h) > last[ct]) e = 0.f;
                cs[j] = fmaf(e, il[ct], cs[j]);
            }
        }
        // transposed butterfly over the 32 lanes of each half: 16 -> 8 -> 4 -> 2 -> 1
#pragma unroll
        for (int step = 0; step < 4; ++step) {
            const int mask = 16 >> step;
            const int half_n = 8 >> step;
            const bool upper = (n & mask) != 0;
#pragma unroll
            for (int i = 0; i < half_n; ++i) {
                const float send = upper ? cs[i] : cs[i + half_n];
                const float keep = upper ? cs[i + half_n] : cs[i];
                cs[i] = keep + shfl_xor_f(send, mask);
            }
        }
        cs[0] += shfl_xor_f(cs[0], 1);
        const int t = t0 + my_tok;
        if (writer && t < a.s_max) rawu[t] = t < S ? cs[0] : 0.f;
    }
}

template <int D, int RT>
void launch_mfma_group(const MfArgs &a, int group_units, hipStream_t stream)
{
    dim3 grid(a.n_chunks, group_units);
    hipLaunchKernelGGL((mfma_stats_kernel<D, RT>), grid, dim3(kMfThreads), 0, stream, a);
    hipLaunchKernelGGL(mfma_merge_kernel, dim3((RT * 32 + 127) / 128, group_units), dim3(128), 0, stream,
                       (const float2 *)a.part, a.n_chunks, RT * 32, a.R, a.c, (float2 *)a.fin);
    hipLaunchKernelGGL((mfma_probsum_kernel<D, RT>), grid, dim3(kMfThreads), 0, stream, a);
}

template <int D>
void launch_mfma_group_rt(int rt, const MfArgs &a, int group_units, hipStream_t stream)
{
    switch (rt) {
    case 1: launch_mfma_group<D, 1>(a, group_units, stream); break;
    case 2: launch_mfma_group<D, 2>(a, group_units, stream); break;
    case 3: launch_mfma_group<D, 3>(a, group_units, stream); break;
    default: launch_mfma_group<D, 4>(a, group_units, stream); break;
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
        const int rpad = (p.R + 31) / 32 * 32;
        // group of units whose K (bf16) fits comfortably in the MALL between passes
        const size_t unit_k = (size_t)s_max * d_h * 2;
        size_t gu = (size_t)(128u << 20) / (unit_k ? unit_k : 1);
        if (gu < 1) gu = 1;
        if (gu > (size_t)units) gu = units;
        p.group_units = (int)gu;
        // tiles per wave: largest in {8,4,2,1} that still gives >= 2 work-groups per CU
        int tpw = 8;
        while (tpw > 1) {
            const long chunks = (s_max + 128L * tpw - 1) / (128L * tpw);
            if (chunks * p.group_units >= 2L * cus) break;
            tpw >>= 1;
        }
        p.tiles_per_wave = tpw;
        p.chunk_tokens = 128 * tpw;
        p.n_chunks = (s_max + p.chunk_tokens - 1) / p.chunk_tokens;
        p.ws_bytes = align256((size_t)p.group_units * p.n_chunks * rpad * sizeof(float2)) +
                     align256((size_t)p.group_units * rpad * sizeof(float2)) + 256;
    } else {
        p.group_units = units;
        p.ws_bytes = align256((size_t)units * p.R * s_max * sizeof(float)) +
                     align256((size_t)units * p.R * sizeof(float2)) + 256;
    }
    return p;
}

hipError_t launch_score(int batch, int s_max, const int32_t *seq_lens, int n_h, int n_kv, int d_h, bool bf16,
                        const void *q_win, const void *k, int w, bool window_in_cache, int n_keep, int pool,
                        float scale, float *raw, float *pooled, void *ws, const ScorePlan &plan,
                        hipStream_t stream)
{
    const int units = batch * n_kv;
    if (plan.mfma) {
        const int rpad = (plan.R + 31) / 32 * 32;
        const int rt = rpad / 32;
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
        a.tiles_per_wave = plan.tiles_per_wave;
        a.c = scale * kLog2e;
        a.part = (float2 *)ws;
        a.fin = (const float2 *)((char *)ws + align256((size_t)plan.group_units * plan.n_chunks * rpad * sizeof(float2)));
        a.raw = raw;
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
            if (d_h == 128) hipLaunchKernelGGL((gen_logits_kernel<true, 128>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, logits);
            else hipLaunchKernelGGL((gen_logits_kernel<true, 64>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, logits);
        } else {
            if (d_h == 128) hipLaunchKernelGGL((gen_logits_kernel<false, 128>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, logits);
            else hipLaunchKernelGGL((gen_logits_kernel<false, 64>), gtok, dim3(kGenThreads), 0, stream, q_win, k, seq_lens, s_max, n_h, n_kv, w, window_in_cache ? 1 : 0, plan.R, 0, scale, logits);
        }
        hipLaunchKernelGGL(gen_rowstats_kernel, dim3(plan.R, units), dim3(kGenThreads), 0, stream, logits, s_max,
                           plan.R, fin);
        hipLaunchKernelGGL(gen_probsum_kernel, gtok, dim3(kGenThreads), 0, stream, logits, (const float2 *)fin,
                           seq_lens, s_max, n_kv, plan.R, 0, raw);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(pool_kernel, dim3((s_max + 255) / 256, units), dim3(256), 0, stream, raw, seq_lens, s_max,
                       n_kv, n_keep, pool / 2, pooled);
    return hipGetLastError();
}

}  // namespace kvc
