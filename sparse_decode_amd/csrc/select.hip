// select.hip -- per-KV-head top-k under the retention budget (FastKV section 2.B)
// plus the always-kept trailing window (FastKV section 2.A), emitted in ascending
// original order (Tutorial "Variantes de l'attention et compression du cache KV",
// section "Quand la reutilisation est-elle exacte ?": keep original positions).
//
// One 1024-thread work-group per unit.  Scores become order-preserving uint32 keys
// (-0.0 folded onto +0.0).  Four radix passes of 8 bits over 256-bin LDS histograms
// find the exact k-th largest key T and how many keys equal to T are still needed.
// Window scores cluster in a few exponents, so the lanes of one atomic instruction
// would collide on a handful of bins; each lane adds into one of 16 histogram copies
// (lane & 15), which caps a collision at 4 lanes.  An ordered compaction then writes every key > T and the first
// "needed" keys == T in index order: each wave owns a contiguous slice of the
// candidates, ballots give in-wave prefix counts, and per-wave totals give the
// offsets -- so the indices come out ascending with no sort, and ties resolve to
// the lower index exactly.  When the unit's keys fit in LDS they are read from HBM
// once; otherwise each pass streams them again (from L2/MALL).
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kBins = 256;          // 8-bit digits, four passes
constexpr int kBatch = 8;           // loads in flight per thread

__device__ __forceinline__ uint32_t order_key(float f)
{
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                      // -0.0 == +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kCopies = 16;         // histogram copies, picked by lane & 15

struct SelShared {
    int hist[kCopies][kBins];       // lanes of one instruction spread over 16 copies
    int scan[32];
    int wave_gt[kSelWaves];
    int wave_eq[kSelWaves];
    int wave_eq_base[kSelWaves];
    int wave_sel_base[kSelWaves];
    int digit;
    int above;
};

template <bool RESIDENT>
__device__ __forceinline__ uint32_t load_key(const float *__restrict__ sc, const uint32_t *keys, int t)
{
    if (RESIDENT) return keys[t];
    return order_key(sc[t]);
}

template <bool RESIDENT>
__global__ __launch_bounds__(kSelThreads) void select_topk_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ seq_lens, int s_max, int H, int k,
    int n_keep, int cap, int32_t *__restrict__ idx, int32_t *__restrict__ count)
{
    extern __shared__ uint32_t dyn[];
    __shared__ SelShared sh;
    uint32_t *keys = dyn;

    const int u = blockIdx.x;
    const int b = u / H;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid >> 6;
    const int S = clamp_len(seq_lens, b, s_max);
    const int C = S - n_keep > 0 ? S - n_keep : 0;
    const int k_eff = k < C ? k : C;
    const float *sc = scores + (size_t)u * s_max;
    int32_t *out = idx + (size_t)u * cap;

    if (k_eff == C) {
        for (int t = tid; t < C; t += kSelThreads) out[t] = t;
    } else if (k_eff > 0) {
        if (RESIDENT) {
            for (int t0 = tid; t0 < C; t0 += kBatch * kSelThreads) {
                float v[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int t = t0 + q * kSelThreads;
                    v[q] = t < C ? sc[t] : 0.f;
                }
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int t = t0 + q * kSelThreads;
                    if (t < C) keys[t] = order_key(v[q]);
                }
            }
        }
        uint32_t prefix = 0, pmask = 0;
        int k_rem = k_eff;
#pragma unroll 1
        for (int pass = 0; pass < 4; ++pass) {
            const int shift = 24 - 8 * pass;
            for (int i = tid; i < kCopies * kBins; i += kSelThreads) (&sh.hist[0][0])[i] = 0;
            int *hw = sh.hist[lane & (kCopies - 1)];
            __syncthreads();
            for (int t0 = tid; t0 < C; t0 += kBatch * kSelThreads) {
                uint32_t kk[kBatch];
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int t = t0 + q * kSelThreads;
                    kk[q] = t < C ? load_key<RESIDENT>(sc, keys, t) : 0u;
                }
#pragma unroll
                for (int q = 0; q < kBatch; ++q) {
                    const int t = t0 + q * kSelThreads;
                    if (t < C && (kk[q] & pmask) == prefix) atomicAdd(&hw[(kk[q] >> shift) & 0xffu], 1);
                }
            }
            __syncthreads();
            // thread i < 256 owns digit 255 - i; prefix counts run from the top digit down
            int cnt = 0;
            const int d = kBins - 1 - tid;
            if (tid < kBins)
                for (int c2 = 0; c2 < kCopies; ++c2) cnt += sh.hist[c2][d];
            int tot;
            const int above = block_exclusive_scan(cnt, sh.scan, &tot);
            if (tid < kBins && above < k_rem && above + cnt >= k_rem) {
                sh.digit = d;
                sh.above = above;
            }
            __syncthreads();
            prefix |= (uint32_t)sh.digit << shift;
            pmask |= 0xffu << shift;
            k_rem -= sh.above;
            __syncthreads();
        }
        const uint32_t T = prefix;
        const int ties = k_rem;                       // keys == T to take, lowest index first

        // ordered compaction: wave w owns candidates [w*seg, (w+1)*seg)
        const int seg = (((C + kSelWaves - 1) / kSelWaves) + kWave - 1) / kWave * kWave;
        const int w0 = wid * seg;
        const int w1 = min(C, w0 + seg);
        int gt = 0, eq = 0;
        for (int t0 = w0 + lane; t0 < w1; t0 += kBatch * kWave) {
            uint32_t kk[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int t = t0 + q * kWave;
                kk[q] = t < w1 ? load_key<RESIDENT>(sc, keys, t) : 0u;
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int t = t0 + q * kWave;
                gt += (t < w1) && kk[q] > T;
                eq += (t < w1) && kk[q] == T;
            }
        }
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            gt += shfl_xor_i(gt, o);
            eq += shfl_xor_i(eq, o);
        }
        if (lane == 0) {
            sh.wave_gt[wid] = gt;
            sh.wave_eq[wid] = eq;
        }
        __syncthreads();
        if (tid == 0) {
            int eq_run = 0, sel_run = 0;
            for (int w2 = 0; w2 < kSelWaves; ++w2) {
                int take = ties - eq_run;
                take = take < 0 ? 0 : (take > sh.wave_eq[w2] ? sh.wave_eq[w2] : take);
                sh.wave_eq_base[w2] = eq_run;
                sh.wave_sel_base[w2] = sel_run;
                eq_run += sh.wave_eq[w2];
                sel_run += sh.wave_gt[w2] + take;
            }
        }
        __syncthreads();
        int pos = sh.wave_sel_base[wid];
        int eq_seen = sh.wave_eq_base[wid];
        const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        for (int tb = w0; tb < w1; tb += kBatch * kWave) {
            uint32_t kk[kBatch];
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int t = tb + q * kWave + lane;
                kk[q] = t < w1 ? load_key<RESIDENT>(sc, keys, t) : 0u;
            }
#pragma unroll
            for (int q = 0; q < kBatch; ++q) {
                const int t = tb + q * kWave + lane;
                const bool is_gt = (t < w1) && kk[q] > T;
                const bool is_eq = (t < w1) && kk[q] == T;
                const unsigned long long m_eq = __ballot(is_eq);
                const int rank = eq_seen + __popcll(m_eq & below);
                const bool sel = is_gt || (is_eq && rank < ties);
                const unsigned long long m_sel = __ballot(sel);
                const int p = pos + __popcll(m_sel & below);
                if (sel && p < k_eff) out[p] = t;            // never past the budget
                pos += __popcll(m_sel);
                eq_seen += __popcll(m_eq);
            }
        }
    }
    // the always-kept trailing tokens, the -1 padding and the count
    const int nw = S - C;
    for (int j = tid; j < nw; j += kSelThreads) out[k_eff + j] = C + j;
    for (int j = k_eff + nw + tid; j < cap; j += kSelThreads) out[j] = -1;
    if (tid == 0) count[u] = k_eff + nw;
}

// TSP score: float sum over KV heads in head order (one selection per sequence).
__global__ __launch_bounds__(256) void head_sum_kernel(const float *__restrict__ scores, int n_kv, int s_max,
                                                       float *__restrict__ out)
{
    const int b = blockIdx.y;
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= s_max) return;
    const float *p = scores + (size_t)b * n_kv * s_max + t;
    float s = 0.f;
    for (int g = 0; g < n_kv; ++g) s += p[(size_t)g * s_max];
    out[(size_t)b * s_max + t] = s;
}

}  // namespace

size_t select_ws_bytes(int batch, int n_kv, int s_max, bool shared)
{
    (void)n_kv;
    return shared ? (size_t)batch * s_max * sizeof(float) + 256 : 0;
}

hipError_t launch_select(int batch, int n_kv, int s_max, const int32_t *seq_lens, const float *scores,
                         int k, int n_keep, bool shared, int32_t *idx, int32_t *count, void *ws,
                         const DeviceInfo &dev, hipStream_t stream)
{
    const float *src = scores;
    int H = n_kv;
    if (shared) {
        float *sum = (float *)ws;
        hipLaunchKernelGGL(head_sum_kernel, dim3((s_max + 255) / 256, batch), dim3(256), 0, stream, scores,
                           n_kv, s_max, sum);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        src = sum;
        H = 1;
    }
    const int cap = k + n_keep;
    const size_t static_lds = sizeof(SelShared);
    const size_t need = (size_t)s_max * sizeof(uint32_t);
    const bool resident = static_lds + need + 1024 <= (size_t)dev.max_lds_per_block;
    dim3 grid(batch * H);
    if (resident) {
        hipLaunchKernelGGL(select_topk_kernel<true>, grid, dim3(kSelThreads), need, stream, src, seq_lens,
                           s_max, H, k, n_keep, cap, idx, count);
    } else {
        hipLaunchKernelGGL(select_topk_kernel<false>, grid, dim3(kSelThreads), 0, stream, src, seq_lens, s_max,
                           H, k, n_keep, cap, idx, count);
    }
    return hipGetLastError();
}

}  // namespace kvc
