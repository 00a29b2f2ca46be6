// decode.hip -- GQA decode attention of one query per head over the compacted cache
// (FreeKV technical summary section 2.A: attend over the selected subset; Tutorial
// "Variantes de l'attention et compression du cache KV", section "MHA et GQA":
// query head h reads KV head h / (n_h / n_kv)).
//
// Split-K over tokens.  One work-group per (KV head, token split, head chunk) loads
// each K/V row once from HBM and uses it for every query head of the GQA group it
// holds (up to 8), so the kernel streams the compacted cache exactly once.  A lane
// owns 16 bytes of a row (8 bf16 or 4 fp32); a row is split over d_h/8 lanes and a
// wave works on 64/(d_h/8) tokens at a time.  Each lane group keeps an online
// softmax state (running max m, sum l, output o), merged across lane groups, then
// waves, then splits -- always in the same order, so results are reproducible.
// Logits are kept in log2 units: q is pre-multiplied by scale * log2(e).
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

template <bool BF16, int D, int RH>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(
    const void *__restrict__ q_, const void *__restrict__ kc_, const void *__restrict__ vc_,
    const int32_t *__restrict__ count, int cap, int n_h, int n_kv, int r, int n_splits,
    int split_tokens, float c, float *__restrict__ part_o, float2 *__restrict__ part_ml)
{
    using RV = RowVec<BF16>;
    constexpr int E = RV::kElems;           // elements per lane
    constexpr int LPT = D / E;              // lanes per token row
    constexpr int TPW = kWave / LPT;        // token rows per wave step
    constexpr int VPR = D / E;              // 16-byte vectors per row (== LPT)
    static_assert(LPT <= kWave && (kWave % LPT) == 0, "row must fit a wave");

    __shared__ float sm_o[kDecWaves][RH][D];
    __shared__ float sm_m[kDecWaves][RH];
    __shared__ float sm_l[kDecWaves][RH];

    const int split = blockIdx.x;
    const int unit = blockIdx.y;            // b * n_kv + g
    const int hc = blockIdx.z;
    const int b = unit / n_kv;
    const int g = unit - b * n_kv;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x >> 6;
    const int li = lane % LPT;
    const int ts = lane / LPT;

    int n = count[unit];
    n = n < 0 ? 0 : (n > cap ? cap : n);
    const int s0 = split * split_tokens;
    int s1 = s0 + split_tokens;
    s1 = s1 > n ? n : s1;

    // queries of this chunk of the group, pre-scaled into log2 units
    float qf[RH][E];
    const int h_first = g * r + hc * RH;
#pragma unroll
    for (int j = 0; j < RH; ++j) {
        const int hl = hc * RH + j;
        if (hl < r) {
            const u32x4 v = *((const u32x4 *)q_ + ((size_t)(b * n_h + h_first + j)) * VPR + li);
            RV::unpack(v, qf[j]);
#pragma unroll
            for (int e = 0; e < E; ++e) qf[j][e] *= c;
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e) qf[j][e] = 0.f;
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

    const u32x4 *krow = (const u32x4 *)kc_ + (size_t)unit * cap * VPR + li;
    const u32x4 *vrow = (const u32x4 *)vc_ + (size_t)unit * cap * VPR + li;
    constexpr int UNR = 4;                  // tokens in flight per lane group
    const int step = kDecWaves * TPW;
    for (int t = s0 + wv * TPW + ts; t < s1; t += UNR * step) {
        u32x4 kv[UNR], vv[UNR];
#pragma unroll
        for (int q = 0; q < UNR; ++q) {
            const int tq = t + q * step;
            if (tq < s1) {
                kv[q] = ld_stream(krow + (size_t)tq * VPR);
                vv[q] = ld_stream(vrow + (size_t)tq * VPR);
            }
        }
#pragma unroll
        for (int q = 0; q < UNR; ++q) {
            if (t + q * step >= s1) break;
            float kf[E], vf[E];
            RV::unpack(kv[q], kf);
            RV::unpack(vv[q], vf);
#pragma unroll
            for (int j = 0; j < RH; ++j) {
                float s = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e) s = fmaf(qf[j][e], kf[e], s);
                if (LPT == 16) {
                    s = row16_sum(s);
                } else {
#pragma unroll
                    for (int off = LPT / 2; off > 0; off >>= 1) s += shfl_xor_f(s, off);
                }
                const float mn = fmaxf(m[j], s);
                const float a = fast_exp2(m[j] - mn);
                const float p = fast_exp2(s - mn);
                l[j] = l[j] * a + p;
#pragma unroll
                for (int e = 0; e < E; ++e) o[j][e] = fmaf(o[j][e], a, p * vf[e]);
                m[j] = mn;
            }
        }
    }
    // Lanes whose group saw no token jump here with m = -inf.  The loop above only
    // runs for valid tokens, but the shuffles inside it need every lane of a token
    // group: a group is either entirely in range or entirely out, since t depends
    // on ts and the wave only.

    // merge the token groups of the wave (lanes li, li + LPT, li + 2 LPT, ...)
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
#pragma unroll
        for (int j = 0; j < RH; ++j) {
            const float m2 = shfl_xor_f(m[j], off);
            const float l2 = shfl_xor_f(l[j], off);
            float o2[E];
#pragma unroll
            for (int e = 0; e < E; ++e) o2[e] = shfl_xor_f(o[j][e], off);
            merge_state<E>(m[j], l[j], o[j], m2, l2, o2);
        }
    }
    if (ts == 0) {
#pragma unroll
        for (int j = 0; j < RH; ++j) {
#pragma unroll
            for (int e = 0; e < E; ++e) sm_o[wv][j][li * E + e] = o[j][e];
            if (li == 0) {
                sm_m[wv][j] = m[j];
                sm_l[wv][j] = l[j];
            }
        }
    }
    __syncthreads();
    // merge the waves in order and write this split's partial state
    for (int x = threadIdx.x; x < RH * D; x += kDecThreads) {
        const int j = x / D;
        const int d = x - j * D;
        const int hl = hc * RH + j;
        if (hl >= r) continue;
        float M = -INFINITY;
        for (int w2 = 0; w2 < kDecWaves; ++w2) M = fmaxf(M, sm_m[w2][j]);
        float L = 0.f, O = 0.f;
        if (M != -INFINITY) {
            for (int w2 = 0; w2 < kDecWaves; ++w2) {
                const float a = fast_exp2(sm_m[w2][j] - M);
                L += sm_l[w2][j] * a;
                O += sm_o[w2][j][d] * a;
            }
        }
        const size_t slot = ((size_t)unit * r + hl) * n_splits + split;
        part_o[slot * D + d] = O;
        if (d == 0) part_ml[slot] = make_float2(M, L);
    }
}

constexpr int kMergeThreads = 256;
constexpr int kMaxSplits = 1024;

// Deterministic block reductions (fixed shuffle tree, then waves in order).
__device__ __forceinline__ float block_max(float v, float *red)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, shfl_xor_f(v, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
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
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < kMergeThreads / kWave; ++i) r += red[i];
    __syncthreads();
    return r;
}

// One work-group per (b, h): split weights exp2(m_s - M) staged in LDS, then
// kMergeThreads / D thread groups each fold a strided subset of the splits (8 loads
// in flight per thread) and the groups are added in group order.
template <bool BF16, int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(const float *__restrict__ part_o,
                                                                     const float2 *__restrict__ part_ml, int n_h,
                                                                     int n_kv, int r, int n_splits,
                                                                     void *__restrict__ out, float *__restrict__ lse)
{
    constexpr int G = kMergeThreads / D;
    __shared__ float sw[kMaxSplits];
    __shared__ float red[kMergeThreads / kWave];
    __shared__ float so[G][D];
    const int bh = blockIdx.x;              // b * n_h + h
    const int b = bh / n_h;
    const int h = bh - b * n_h;
    const int g = h / r;
    const int hl = h - g * r;
    const size_t base = ((size_t)(b * n_kv + g) * r + hl) * n_splits;
    float mloc = -INFINITY;
    for (int s = threadIdx.x; s < n_splits; s += kMergeThreads) mloc = fmaxf(mloc, part_ml[base + s].x);
    const float M = block_max(mloc, red);
    float lloc = 0.f;
    for (int s = threadIdx.x; s < n_splits; s += kMergeThreads) {
        const float2 ml = part_ml[base + s];
        const float wgt = (M == -INFINITY || ml.x == -INFINITY) ? 0.f : fast_exp2(ml.x - M);
        sw[s] = wgt;
        lloc += wgt * ml.y;
    }
    const float L = block_sum(lloc, red);   // also orders the sw[] writes before their reads
    const int d = threadIdx.x % D;
    const int grp = threadIdx.x / D;
    float O = 0.f;
    for (int s0 = grp; s0 < n_splits; s0 += 8 * G) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int s = s0 + q * G;
            v[q] = s < n_splits ? part_o[(base + s) * D + d] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int s = s0 + q * G;
            if (s < n_splits) O = fmaf(sw[s], v[q], O);
        }
    }
    so[grp][d] = O;
    __syncthreads();
    if (grp != 0) return;
    float Ot = so[0][d];
    for (int g2 = 1; g2 < G; ++g2) Ot += so[g2][d];
    const float y = (L > 0.f) ? Ot / L : 0.f;
    if (BF16)
        ((uint16_t *)out)[(size_t)bh * D + d] = f32_to_bf16(y);
    else
        ((float *)out)[(size_t)bh * D + d] = y;
    if (lse && d == 0) lse[bh] = (L > 0.f) ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

template <bool BF16, int D, int RH>
void launch_split(dim3 grid, hipStream_t stream, const void *q, const void *kc, const void *vc,
                  const int32_t *count, int cap, int n_h, int n_kv, int r, int n_splits, int split_tokens,
                  float c, float *part_o, float2 *part_ml)
{
    hipLaunchKernelGGL((decode_split_kernel<BF16, D, RH>), grid, dim3(kDecThreads), 0, stream, q, kc, vc,
                       count, cap, n_h, n_kv, r, n_splits, split_tokens, c, part_o, part_ml);
}

template <bool BF16, int D>
void launch_split_rh(int rh, dim3 grid, hipStream_t stream, const void *q, const void *kc, const void *vc,
                     const int32_t *count, int cap, int n_h, int n_kv, int r, int n_splits,
                     int split_tokens, float c, float *part_o, float2 *part_ml)
{
    switch (rh) {
    case 1: launch_split<BF16, D, 1>(grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, n_splits, split_tokens, c, part_o, part_ml); break;
    case 2: launch_split<BF16, D, 2>(grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, n_splits, split_tokens, c, part_o, part_ml); break;
    case 4: launch_split<BF16, D, 4>(grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, n_splits, split_tokens, c, part_o, part_ml); break;
    default: launch_split<BF16, D, 8>(grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, n_splits, split_tokens, c, part_o, part_ml); break;
    }
}

}  // namespace

DecodePlan plan_decode(int batch, int n_h, int n_kv, int d_h, int cap, int cus)
{
    (void)d_h;
    DecodePlan p;
    const int r = n_h / n_kv;
    p.head_chunk = r >= 8 ? 8 : (r >= 4 ? 4 : (r >= 2 ? 2 : 1));
    if (p.head_chunk < r && r < 8) p.head_chunk *= 2;   // r = 3, 5, 6, 7 -> next power of two
    p.head_chunks = (r + p.head_chunk - 1) / p.head_chunk;
    const long units = (long)batch * n_kv * p.head_chunks;
    // about two work-groups per CU, splits of at least 64 tokens (one unrolled
    // iteration of the work-group), at most kMaxSplits
    long splits = (2L * cus + units - 1) / units;
    const long max_splits = (cap + 63) / 64;
    if (splits > max_splits) splits = max_splits;
    if (splits > kMaxSplits) splits = kMaxSplits;
    if (splits < 1) splits = 1;
    long tok = (cap + splits - 1) / splits;
    tok = ((tok + 63) / 64) * 64;
    p.split_tokens = (int)tok;
    p.n_splits = (int)((cap + tok - 1) / tok);
    if (p.n_splits < 1) p.n_splits = 1;
    if (p.n_splits > kMaxSplits) {           // only for caps beyond 64 * kMaxSplits tokens
        p.split_tokens = (int)(((cap + kMaxSplits - 1) / kMaxSplits + 63) / 64 * 64);
        p.n_splits = (cap + p.split_tokens - 1) / p.split_tokens;
    }
    const size_t slots = (size_t)batch * n_kv * r * p.n_splits;
    p.ws_bytes = slots * (size_t)d_h * sizeof(float) + slots * sizeof(float2) + 256;
    return p;
}

hipError_t launch_decode(int batch, int n_h, int n_kv, int d_h, bool bf16, const void *q, const void *kc,
                         const void *vc, const int32_t *count, int cap, float scale, void *out, float *lse,
                         void *ws, const DecodePlan &plan, hipStream_t stream)
{
    const int r = n_h / n_kv;
    const size_t slots = (size_t)batch * n_kv * r * plan.n_splits;
    float *part_o = (float *)ws;
    float2 *part_ml = (float2 *)((char *)ws + ((slots * d_h * sizeof(float) + 255) / 256) * 256);
    const float c = scale * 1.4426950408889634f;
    dim3 grid(plan.n_splits, batch * n_kv, plan.head_chunks);
    if (bf16) {
        if (d_h == 128) launch_split_rh<true, 128>(plan.head_chunk, grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, plan.n_splits, plan.split_tokens, c, part_o, part_ml);
        else launch_split_rh<true, 64>(plan.head_chunk, grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, plan.n_splits, plan.split_tokens, c, part_o, part_ml);
    } else {
        if (d_h == 128) launch_split_rh<false, 128>(plan.head_chunk, grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, plan.n_splits, plan.split_tokens, c, part_o, part_ml);
        else launch_split_rh<false, 64>(plan.head_chunk, grid, stream, q, kc, vc, count, cap, n_h, n_kv, r, plan.n_splits, plan.split_tokens, c, part_o, part_ml);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 mgrid(batch * n_h);
    if (bf16) {
        if (d_h == 128) hipLaunchKernelGGL((decode_merge_kernel<true, 128>), mgrid, dim3(kMergeThreads), 0, stream, part_o, part_ml, n_h, n_kv, r, plan.n_splits, out, lse);
        else hipLaunchKernelGGL((decode_merge_kernel<true, 64>), mgrid, dim3(kMergeThreads), 0, stream, part_o, part_ml, n_h, n_kv, r, plan.n_splits, out, lse);
    } else {
        if (d_h == 128) hipLaunchKernelGGL((decode_merge_kernel<false, 128>), mgrid, dim3(kMergeThreads), 0, stream, part_o, part_ml, n_h, n_kv, r, plan.n_splits, out, lse);
        else hipLaunchKernelGGL((decode_merge_kernel<false, 64>), mgrid, dim3(kMergeThreads), 0, stream, part_o, part_ml, n_h, n_kv, r, plan.n_splits, out, lse);
    }
    return hipGetLastError();
}

}  // namespace kvc
