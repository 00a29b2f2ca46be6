// blocks.hip -- landmark-guided block selection (xKV section 2.3, "Reconstruction
// Selective": the tokens most relevant to the current query are found by a block
// selection guided by landmarks, as in ShadowKV).  Each KV head's cache is cut into
// blocks of `block` tokens; a block's landmark is the mean of its keys, its score the
// group's attention logit for that landmark; the best blocks are kept whole and
// expanded back into token indices for the compacting gather.
//
// Landmarks and block scores are sums of exact products (bf16 * bf16 / fp32 in
// double), added in a fixed order in double: the scores the selection compares are
// reproducible bit for bit.  All three kernels are memory-bound streams; landmarks are
// built once per cache and read (1/block of K's rows, in fp32) at every step.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

constexpr int kBlkThreads = 256;

template <bool BF16>
__device__ __forceinline__ void widen(const u32x4 &v, double *f)
{
    if (BF16) {
        f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
    } else {
        f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
        f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
    }
}

// One thread per (unit, block, 16-byte vector of the row): the mean over the block's
// cached tokens, summed in token order in double.
template <bool BF16>
__global__ __launch_bounds__(kBlkThreads) void block_landmarks_kernel(const u32x4 *__restrict__ k,
                                                                      const int32_t *__restrict__ seq_lens,
                                                                      int n_kv, int s_max, int vpr, int block,
                                                                      int n_blk, float *__restrict__ landmarks)
{
    constexpr int E = BF16 ? 8 : 4;                 // elements per vector
    const long gid = (long)kvc_bid_x() * kBlkThreads + kvc_tid();
    const int u = kvc_bid_y();
    if (gid >= (long)n_blk * vpr) return;
    const int j = (int)(gid / vpr), c = (int)(gid - (long)j * vpr);
    const int S = clamp_len(seq_lens, u / n_kv, s_max);
    const int t0 = j * block, t1 = min(t0 + block, S);
    double acc[E] = {};
    for (int t = t0; t < t1; ++t) {
        double f[E];
        widen<BF16>(k[((size_t)u * s_max + t) * vpr + c], f);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] += f[e];
    }
    float *out = landmarks + (((size_t)u * n_blk + j) * vpr + c) * E;
#pragma unroll
    for (int e = 0; e < E; ++e) out[e] = t1 > t0 ? (float)(acc[e] / (double)(t1 - t0)) : 0.f;
}

// One thread per (unit, block): scale * sum over the group's query heads, then over d,
// of q * landmark, in double, for the candidate blocks j < floor((S_b - n_keep) / block);
// 0 elsewhere.  Unit (b, 0)'s block-0 thread also writes the candidate block count.
// Two waves per SIMD: a thread holds its 512-byte landmark row in registers, and
// without the bound the compiler's allocation left one wave per SIMD (a few registers
// spill instead).
template <bool BF16, int D>
__global__ __launch_bounds__(kBlkThreads) __attribute__((amdgpu_waves_per_eu(2))) void block_scores_kernel(const void *__restrict__ q,
                                                                   const float *__restrict__ landmarks,
                                                                   const int32_t *__restrict__ seq_lens,
                                                                   int n_h, int n_kv, int d_h, int s_max, int block,
                                                                   int n_keep, int n_blk, double scale,
                                                                   float *__restrict__ scores,
                                                                   int32_t *__restrict__ cand)
{
    extern __shared__ double qs[];                  // the group's queries [r][d_h]
    const int u = kvc_bid_y();
    const int b = u / n_kv, g = u - b * n_kv;
    const int r = n_h / n_kv;
    for (int x = kvc_tid(); x < r * d_h; x += kBlkThreads) {
        const size_t off = ((size_t)b * n_h + g * r) * d_h + x;
        qs[x] = BF16 ? (double)bf16_to_f32(((const uint16_t *)q)[off]) : (double)((const float *)q)[off];
    }
    __syncthreads();
    const int S = clamp_len(seq_lens, b, s_max);
    const int C = S - n_keep > 0 ? S - n_keep : 0;
    const int nc = C / block;
    const int j = kvc_bid_x() * kBlkThreads + kvc_tid();
    if (g == 0 && j == 0) cand[b] = nc;
    if (j >= n_blk) return;
    double s = 0.0;
    if (j < nc) {
        // the landmark row is read once (every load in flight together) and reused for
        // every query head; the sum keeps the h-then-d order
        const float4 *lm = (const float4 *)(landmarks + ((size_t)u * n_blk + j) * D);
        float4 l[D / 4];
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) l[d4] = lm[d4];
        for (int h = 0; h < r; ++h) {
            const double *qh = qs + h * D;
#pragma unroll
            for (int d4 = 0; d4 < D / 4; ++d4) {
                s += qh[4 * d4] * (double)l[d4].x;
                s += qh[4 * d4 + 1] * (double)l[d4].y;
                s += qh[4 * d4 + 2] * (double)l[d4].z;
                s += qh[4 * d4 + 3] * (double)l[d4].w;
            }
        }
    }
    scores[(size_t)u * n_blk + j] = (float)(scale * s);
}

// One thread per output position of a unit: selected block j's tokens at j*block + i,
// then the tail [nc * block, S_b), then -1.
__global__ __launch_bounds__(kBlkThreads) void expand_blocks_kernel(const int32_t *__restrict__ idx_blk,
                                                                    const int32_t *__restrict__ count_blk,
                                                                    const int32_t *__restrict__ seq_lens, int H,
                                                                    int s_max, int block, int n_keep, int cap_blk,
                                                                    int cap, int32_t *__restrict__ idx,
                                                                    int32_t *__restrict__ count)
{
    const int u = kvc_bid_y();
    const int p = kvc_bid_x() * kBlkThreads + kvc_tid();
    const int S = clamp_len(seq_lens, u / H, s_max);
    const int C = S - n_keep > 0 ? S - n_keep : 0;
    const int tail0 = (C / block) * block;
    int kb = count_blk[u];
    kb = kb < 0 ? 0 : (kb > cap_blk ? cap_blk : kb);
    const long body = (long)kb * block;
    const long total = body + (S - tail0);
    const int n = total < cap ? (int)total : cap;
    if (p == 0) count[u] = n;
    if (p >= cap) return;
    int v = -1;
    if (p < n) v = p < body ? idx_blk[(size_t)u * cap_blk + p / block] * block + p % block : tail0 + (int)(p - body);
    idx[(size_t)u * cap + p] = v;
}

}  // namespace

hipError_t launch_block_landmarks(int batch, int n_kv, int s_max, int d_h, bool bf16, const int32_t *seq_lens,
                                  const void *k, int block, float *landmarks, hipStream_t stream)
{
    const int vpr = d_h * (bf16 ? 2 : 4) / 16;
    const int n_blk = (s_max + block - 1) / block;
    const dim3 grid((unsigned)(((long)n_blk * vpr + kBlkThreads - 1) / kBlkThreads), batch * n_kv);
    if (bf16)
        hipLaunchKernelGGL(block_landmarks_kernel<true>, grid, dim3(kBlkThreads), 0, stream, (const u32x4 *)k,
                           seq_lens, n_kv, s_max, vpr, block, n_blk, landmarks);
    else
        hipLaunchKernelGGL(block_landmarks_kernel<false>, grid, dim3(kBlkThreads), 0, stream, (const u32x4 *)k,
                           seq_lens, n_kv, s_max, vpr, block, n_blk, landmarks);
    return hipGetLastError();
}

hipError_t launch_block_scores(int batch, int n_h, int n_kv, int d_h, bool bf16, int s_max, const int32_t *seq_lens,
                               const void *q, const float *landmarks, int block, int n_keep, double scale,
                               float *scores, int32_t *cand, hipStream_t stream)
{
    const int n_blk = (s_max + block - 1) / block;
    const dim3 grid((n_blk + kBlkThreads - 1) / kBlkThreads, batch * n_kv);
    const size_t lds = (size_t)(n_h / n_kv) * d_h * sizeof(double);
    if (bf16 && d_h == 128)
        hipLaunchKernelGGL((block_scores_kernel<true, 128>), grid, dim3(kBlkThreads), lds, stream, q, landmarks,
                           seq_lens, n_h, n_kv, d_h, s_max, block, n_keep, n_blk, scale, scores, cand);
    else if (bf16)
        hipLaunchKernelGGL((block_scores_kernel<true, 64>), grid, dim3(kBlkThreads), lds, stream, q, landmarks,
                           seq_lens, n_h, n_kv, d_h, s_max, block, n_keep, n_blk, scale, scores, cand);
    else if (d_h == 128)
        hipLaunchKernelGGL((block_scores_kernel<false, 128>), grid, dim3(kBlkThreads), lds, stream, q, landmarks,
                           seq_lens, n_h, n_kv, d_h, s_max, block, n_keep, n_blk, scale, scores, cand);
    else
        hipLaunchKernelGGL((block_scores_kernel<false, 64>), grid, dim3(kBlkThreads), lds, stream, q, landmarks,
                           seq_lens, n_h, n_kv, d_h, s_max, block, n_keep, n_blk, scale, scores, cand);
    return hipGetLastError();
}

hipError_t launch_expand_blocks(int batch, int heads, int s_max, const int32_t *seq_lens, int block, int n_keep,
                                const int32_t *idx_blk, const int32_t *count_blk, int cap_blk, int32_t *idx,
                                int32_t *count, int cap, hipStream_t stream)
{
    const dim3 grid((cap + kBlkThreads - 1) / kBlkThreads, batch * heads);
    hipLaunchKernelGGL(expand_blocks_kernel, grid, dim3(kBlkThreads), 0, stream, idx_blk, count_blk, seq_lens,
                       heads, s_max, block, n_keep, cap_blk, cap, idx, count);
    return hipGetLastError();
}

}  // namespace kvc
