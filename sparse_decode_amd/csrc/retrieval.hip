// retrieval.hip -- query similarity of two adjacent decode steps and the KV heads
// whose selection is redone before attention (FreeKV technical summary section 2.A:
// adjacent queries are very similar, so a step can attend over the subset selected
// with the previous query; when a head's two queries fall below a cosine threshold
// tau, selection and retrieval run again for that head first).
//
// Tiny and latency-bound: one wave per (sequence, KV head) walks the group's query
// heads; each lane holds d_h/64 elements of both queries and the three sums are
// reduced in double with a fixed butterfly, so the cosine compared with tau carries
// no fp32 rounding of its own.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

template <bool BF16, int D>
__device__ __forceinline__ double elem(const void *q, size_t off)
{
    if (BF16) return (double)bf16_to_f32(((const uint16_t *)q)[off]);
    return (double)((const float *)q)[off];
}

__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

template <bool BF16, int D>
__global__ __launch_bounds__(kWave) void similarity_kernel(const void *__restrict__ q_cur,
                                                           const void *__restrict__ q_prev, int n_h, int n_kv,
                                                           double tau, float *__restrict__ cos_out,
                                                           int32_t *__restrict__ refresh, int32_t *__restrict__ keep)
{
    constexpr int EPL = D / kWave;          // elements per lane
    const int g = kvc_bid_x();
    const int b = kvc_bid_y();
    const int r = n_h / n_kv;
    const int lane = kvc_tid();
    int drifted = 0;
    for (int j = 0; j < r; ++j) {
        const int h = g * r + j;
        const size_t row = ((size_t)b * n_h + h) * D;
        double xy = 0.0, xx = 0.0, yy = 0.0;
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
            const double x = elem<BF16, D>(q_cur, row + lane + e * kWave);
            const double y = elem<BF16, D>(q_prev, row + lane + e * kWave);
            xy = fma(x, y, xy);
            xx = fma(x, x, xx);
            yy = fma(y, y, yy);
        }
        xy = wave_sum_d(xy);
        xx = wave_sum_d(xx);
        yy = wave_sum_d(yy);
        const double c = (xx > 0.0 && yy > 0.0) ? xy / (sqrt(xx) * sqrt(yy)) : 0.0;
        drifted |= c < tau;
        if (lane == 0 && cos_out) cos_out[(size_t)b * n_h + h] = (float)c;
    }
    if (lane == 0) {
        refresh[(size_t)b * n_kv + g] = drifted;
        if (keep) keep[(size_t)b * n_kv + g] = 1 - drifted;
    }
}

}  // namespace

hipError_t launch_similarity(int batch, int n_h, int n_kv, int d_h, bool bf16, const void *q_cur,
                             const void *q_prev, double tau, float *cos, int32_t *refresh, int32_t *keep,
                             hipStream_t stream)
{
    const dim3 grid(n_kv, batch);
    if (bf16) {
        if (d_h == 128) hipLaunchKernelGGL((similarity_kernel<true, 128>), grid, dim3(kWave), 0, stream, q_cur, q_prev, n_h, n_kv, tau, cos, refresh, keep);
        else hipLaunchKernelGGL((similarity_kernel<true, 64>), grid, dim3(kWave), 0, stream, q_cur, q_prev, n_h, n_kv, tau, cos, refresh, keep);
    } else {
        if (d_h == 128) hipLaunchKernelGGL((similarity_kernel<false, 128>), grid, dim3(kWave), 0, stream, q_cur, q_prev, n_h, n_kv, tau, cos, refresh, keep);
        else hipLaunchKernelGGL((similarity_kernel<false, 64>), grid, dim3(kWave), 0, stream, q_cur, q_prev, n_h, n_kv, tau, cos, refresh, keep);
    }
    return hipGetLastError();
}

}  // namespace kvc
