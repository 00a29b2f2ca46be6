// kvc_api.hip -- the C ABI declared in include/kvc.h: argument validation (every
// host-checkable precondition before any HIP call), workspace sizing and dispatch
// to the gfx950 kernels.  No exception crosses this layer.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "kvc.h"
#include "kvc_launch.h"

#define KVC_EXPORT extern "C" __attribute__((visibility("default")))

namespace kvc {

hipError_t device_info(DeviceInfo *out)
{
    static std::mutex mu;
    static DeviceInfo cache[64];
    static bool have[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (dev >= 0 && dev < 64 && have[dev]) {
        *out = cache[dev];
        return hipSuccess;
    }
    DeviceInfo d;
    int v = 0;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess) return e;
    d.cus = v > 0 ? v : 1;
    if ((e = hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev)) != hipSuccess) return e;
    d.max_lds_per_block = v > 0 ? v : 65536;
    if (dev >= 0 && dev < 64) {
        cache[dev] = d;
        have[dev] = true;
    }
    *out = d;
    return hipSuccess;
}

}  // namespace kvc

namespace {

constexpr int kMaxUnits = 65535;

bool valid_dtype(int32_t dt) { return dt == KVC_F32 || dt == KVC_BF16; }

// Shapes shared by score, select and decode.
kvc_status check_dims(const kvc_dims *d, bool need_s)
{
    if (!d) return KVC_ERR_INVALID_ARG;
    if (d->batch < 1 || d->n_h < 1 || d->n_kv < 1 || d->d_h < 1) return KVC_ERR_INVALID_ARG;
    if (need_s && d->s_max < 1) return KVC_ERR_INVALID_ARG;
    if (d->n_h % d->n_kv != 0) return KVC_ERR_INVALID_ARG;
    if (!valid_dtype(d->dtype)) return KVC_ERR_INVALID_ARG;
    if ((long)d->batch * d->n_kv > kMaxUnits || (long)d->batch * d->n_h > (1L << 30)) return KVC_ERR_INVALID_ARG;
    if (d->d_h != 64 && d->d_h != 128) return KVC_ERR_UNSUPPORTED;
    return KVC_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

KVC_EXPORT int32_t kvc_abi_version(void) { return KVC_ABI_VERSION; }

KVC_EXPORT const char *kvc_status_str(kvc_status s)
{
    switch (s) {
    case KVC_OK: return "ok";
    case KVC_ERR_INVALID_ARG: return "invalid argument";
    case KVC_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case KVC_ERR_WORKSPACE: return "workspace missing or too small";
    case KVC_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

// ---------------------------------------------------------------------------------- score

static kvc_status score_args(const kvc_dims *d, int32_t w, int32_t flags)
{
    kvc_status st = check_dims(d, true);
    if (st != KVC_OK) return st;
    if (w < 1 || w > 1024 || (long)(d->n_h / d->n_kv) * w > 1024) return KVC_ERR_INVALID_ARG;
    if (d->s_max > (1 << 22)) return KVC_ERR_UNSUPPORTED;      // byte offsets within a unit fit 31 bits
    if (flags & ~(KVC_SCORE_GENERIC | KVC_SCORE_DEFER_ALL)) return KVC_ERR_INVALID_ARG;
    return KVC_OK;
}

static size_t score_ws(const kvc_dims *d, int32_t w, int32_t flags, int cus)
{
    kvc::ScorePlan p = kvc::plan_score(d->batch, d->s_max, d->n_h, d->n_kv, d->d_h, d->dtype == KVC_BF16, w,
                                       (flags & KVC_SCORE_GENERIC) != 0, cus);
    return p.ws_bytes;
}

// The workspace size must not depend on the device queried, so plans are sized for
// the largest CU count a gfx950 part has; a smaller part only uses part of it.
static constexpr int kPlanCus = 256;

KVC_EXPORT size_t kvc_score_window_workspace(const kvc_dims *dims, int32_t w, int32_t flags)
{
    if (score_args(dims, w, flags) != KVC_OK) return 0;
    return score_ws(dims, w, flags, kPlanCus);
}

KVC_EXPORT kvc_status kvc_score_window_plan(const kvc_dims *dims, int32_t w, int32_t flags, int32_t *out)
{
    kvc_status st = score_args(dims, w, flags);
    if (st != KVC_OK) return st;
    if (!out) return KVC_ERR_INVALID_ARG;
    const kvc::ScorePlan p = kvc::plan_score(dims->batch, dims->s_max, dims->n_h, dims->n_kv, dims->d_h,
                                             dims->dtype == KVC_BF16, w, (flags & KVC_SCORE_GENERIC) != 0, kPlanCus);
    out[0] = p.mfma ? 1 : 0;
    out[1] = p.mfma ? p.rt : 0;
    out[2] = p.mfma ? (p.single ? p.sp_item : p.chunk_tokens) : 0;
    out[3] = p.mfma ? (p.single ? p.sp_chunks : p.n_chunks) : 0;
    out[4] = p.single ? 1 : 0;
    out[5] = p.mfma && !p.single && p.fold_merge ? 1 : 0;
    return KVC_OK;
}

KVC_EXPORT kvc_status kvc_score_window(const kvc_dims *dims, const void *q_win, const void *k, int32_t w,
                                       int32_t window_in_cache, int32_t n_keep, int32_t pool_kernel,
                                       float scale, float *raw, float *pooled, int32_t flags, void *ws,
                                       size_t ws_bytes, void *stream)
{
    kvc_status st = score_args(dims, w, flags);
    if (st != KVC_OK) return st;
    if (!q_win || !k || !raw || !pooled) return KVC_ERR_INVALID_ARG;
    if (n_keep < 0 || pool_kernel < 1 || pool_kernel > 63 || (pool_kernel & 1) == 0) return KVC_ERR_INVALID_ARG;
    if (!(scale >= 0.f) || scale > 1e30f) return KVC_ERR_INVALID_ARG;
    if (!aligned16(q_win) || !aligned16(k)) return KVC_ERR_INVALID_ARG;
    const size_t need = score_ws(dims, w, flags, kPlanCus);
    if (!ws || ws_bytes < need || !aligned16(ws)) return KVC_ERR_WORKSPACE;
    const float sc = scale == 0.f ? 1.0f / sqrtf((float)dims->d_h) : scale;
    kvc::ScorePlan plan = kvc::plan_score(dims->batch, dims->s_max, dims->n_h, dims->n_kv, dims->d_h,
                                          dims->dtype == KVC_BF16, w, (flags & KVC_SCORE_GENERIC) != 0, kPlanCus);
    if (flags & KVC_SCORE_DEFER_ALL) plan.sp_spin = 0;
    hipError_t e = kvc::launch_score(dims->batch, dims->s_max, dims->seq_lens, dims->n_h, dims->n_kv, dims->d_h,
                                     dims->dtype == KVC_BF16, q_win, k, w, window_in_cache != 0, n_keep,
                                     pool_kernel, sc, raw, pooled, dims->unit_mask, ws, plan, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// --------------------------------------------------------------------------------- select

static kvc_status select_args(const kvc_dims *d, int32_t k, int32_t n_keep, int32_t flags)
{
    if (!d) return KVC_ERR_INVALID_ARG;
    if (d->batch < 1 || d->s_max < 1 || d->n_kv < 1) return KVC_ERR_INVALID_ARG;
    if ((long)d->batch * d->n_kv > kMaxUnits) return KVC_ERR_INVALID_ARG;
    if (k < 0 || n_keep < 0 || (long)k + n_keep < 1 || (long)k + n_keep > (1L << 30)) return KVC_ERR_INVALID_ARG;
    if (flags & ~KVC_SELECT_SHARED_HEADS) return KVC_ERR_INVALID_ARG;
    if ((flags & KVC_SELECT_SHARED_HEADS) && d->unit_mask) return KVC_ERR_INVALID_ARG;
    return KVC_OK;
}

KVC_EXPORT size_t kvc_select_topk_workspace(const kvc_dims *dims, int32_t k, int32_t n_keep, int32_t flags)
{
    if (select_args(dims, k, n_keep, flags) != KVC_OK) return 0;
    return kvc::select_ws_bytes(dims->batch, dims->n_kv, dims->s_max, n_keep, (flags & KVC_SELECT_SHARED_HEADS) != 0);
}

KVC_EXPORT kvc_status kvc_select_topk(const kvc_dims *dims, const float *scores, int32_t k, int32_t n_keep,
                                      int32_t flags, const int32_t *k_per_unit, int32_t *idx, int32_t *count,
                                      void *ws, size_t ws_bytes, void *stream)
{
    kvc_status st = select_args(dims, k, n_keep, flags);
    if (st != KVC_OK) return st;
    if (!scores || !idx || !count) return KVC_ERR_INVALID_ARG;
    const bool shared = (flags & KVC_SELECT_SHARED_HEADS) != 0;
    const size_t need = kvc::select_ws_bytes(dims->batch, dims->n_kv, dims->s_max, n_keep, shared);
    if (need && (!ws || ws_bytes < need || !aligned16(ws))) return KVC_ERR_WORKSPACE;
    kvc::DeviceInfo dev;
    if (kvc::device_info(&dev) != hipSuccess) return KVC_ERR_HIP;
    hipError_t e = kvc::launch_select(dims->batch, dims->n_kv, dims->s_max, dims->seq_lens, scores, k, n_keep,
                                      shared, idx, count, dims->unit_mask, k_per_unit, ws, dev,
                                      (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

KVC_EXPORT size_t kvc_select_core_workspace(const kvc_dims *dims, int32_t n_keep)
{
    if (!dims || dims->batch < 1 || dims->s_max < 1 || dims->n_kv < 1 || n_keep < 0) return 0;
    if ((long)dims->batch * dims->n_kv > kMaxUnits) return 0;
    return kvc::select_core_ws_bytes(dims->batch, dims->n_kv, dims->s_max, n_keep);
}

KVC_EXPORT kvc_status kvc_select_core(const kvc_dims *dims, const float *scores, const uint8_t *core, int32_t k,
                                      int32_t core_cap, int32_t n_keep, int32_t *idx, int32_t *count, void *ws,
                                      size_t ws_bytes, void *stream)
{
    if (k < 0 || core_cap < 0 || (long)k + core_cap > (1L << 29)) return KVC_ERR_INVALID_ARG;
    kvc_status st = select_args(dims, k + core_cap, n_keep, 0);
    if (st != KVC_OK) return st;
    if (!scores || !core || !idx || !count) return KVC_ERR_INVALID_ARG;
    const size_t need = kvc::select_core_ws_bytes(dims->batch, dims->n_kv, dims->s_max, n_keep);
    if (!ws || ws_bytes < need || !aligned16(ws)) return KVC_ERR_WORKSPACE;
    kvc::DeviceInfo dev;
    if (kvc::device_info(&dev) != hipSuccess) return KVC_ERR_HIP;
    hipError_t e = kvc::launch_select_core(dims->batch, dims->n_kv, dims->s_max, dims->seq_lens, scores, core, k,
                                           core_cap, n_keep, idx, count, dims->unit_mask, ws, dev,
                                           (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// --------------------------------------------------------------------------------- gather

KVC_EXPORT kvc_status kvc_gather_compact(int32_t batch, int32_t heads, int32_t s_max, int32_t row_bytes,
                                         const void *src0, const void *src1, const int32_t *src_pos,
                                         const int32_t *idx, const int32_t *count, int32_t idx_heads, int32_t cap,
                                         void *dst0, void *dst1, int32_t *pos_out, const int32_t *unit_mask,
                                         void *stream)
{
    if (batch < 1 || heads < 1 || s_max < 1 || cap < 1 || row_bytes < 16) return KVC_ERR_INVALID_ARG;
    if ((long)batch * heads > kMaxUnits) return KVC_ERR_INVALID_ARG;
    if (idx_heads != 1 && idx_heads != heads) return KVC_ERR_INVALID_ARG;
    if (!src0 || !dst0 || !idx || !count) return KVC_ERR_INVALID_ARG;
    if ((src1 == nullptr) != (dst1 == nullptr)) return KVC_ERR_INVALID_ARG;
    if (row_bytes % 16 != 0) return KVC_ERR_UNSUPPORTED;
    const int vpr = row_bytes / 16;
    const bool pow2 = (vpr & (vpr - 1)) == 0;
    if (!pow2 && vpr % 256 != 0) return KVC_ERR_UNSUPPORTED;
    if (!aligned16(src0) || !aligned16(dst0) || (src1 && (!aligned16(src1) || !aligned16(dst1))))
        return KVC_ERR_UNSUPPORTED;
    kvc::DeviceInfo dev;
    if (kvc::device_info(&dev) != hipSuccess) return KVC_ERR_HIP;
    hipError_t e = kvc::launch_gather(batch, heads, s_max, row_bytes, src0, src1, src_pos, idx, count, idx_heads,
                                      cap, dst0, dst1, pos_out, unit_mask, dev, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// --------------------------------------------------------------------------------- decode

KVC_EXPORT size_t kvc_decode_attn_workspace(const kvc_dims *dims, int32_t cap)
{
    if (check_dims(dims, false) != KVC_OK || cap < 1) return 0;
    return kvc::plan_decode(dims->batch, dims->n_h, dims->n_kv, dims->d_h, cap, kPlanCus).ws_bytes;
}

KVC_EXPORT kvc_status kvc_decode_attn_plan(const kvc_dims *dims, int32_t cap, int32_t *out)
{
    kvc_status st = check_dims(dims, false);
    if (st != KVC_OK) return st;
    if (cap < 1 || cap > (1 << 30) || !out) return KVC_ERR_INVALID_ARG;
    const kvc::DecodePlan p = kvc::plan_decode(dims->batch, dims->n_h, dims->n_kv, dims->d_h, cap, kPlanCus);
    out[0] = p.n_splits;
    out[1] = p.split_tokens;
    out[2] = p.head_chunk;
    out[3] = p.fused ? 1 : 0;
    return KVC_OK;
}

KVC_EXPORT kvc_status kvc_decode_attn(const kvc_dims *dims, const void *q, const void *kc, const void *vc,
                                      const int32_t *count, int32_t cap, float scale, void *out, float *lse,
                                      void *ws, size_t ws_bytes, void *stream)
{
    kvc_status st = check_dims(dims, false);
    if (st != KVC_OK) return st;
    if (cap < 1 || cap > (1 << 30)) return KVC_ERR_INVALID_ARG;
    if (!q || !kc || !vc || !count || !out) return KVC_ERR_INVALID_ARG;
    if (!(scale >= 0.f) || scale > 1e30f) return KVC_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(out)) return KVC_ERR_INVALID_ARG;
    kvc::DecodePlan plan = kvc::plan_decode(dims->batch, dims->n_h, dims->n_kv, dims->d_h, cap, kPlanCus);
    if (!ws || ws_bytes < plan.ws_bytes || !aligned16(ws)) return KVC_ERR_WORKSPACE;
    const float sc = scale == 0.f ? 1.0f / sqrtf((float)dims->d_h) : scale;
    hipError_t e = kvc::launch_decode(dims->batch, dims->n_h, dims->n_kv, dims->d_h, dims->dtype == KVC_BF16, q,
                                      kc, vc, count, cap, sc, out, lse, ws, plan, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// ------------------------------------------------------------ decode without allocation
// The workspace of kvc_decode_attn_noalloc (arrival counters, then split partials)
// lives in this file-scope device array, one copy per GPU, held until the process
// ends.  It is zero when the library loads and every completed call returns the
// counters to zero (the last work-group to arrive resets its own), so no call clears
// it.  Its host-side name is only a stand-in: host code uses the device address
// hipGetSymbolAddress returns for the current device.
static constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

// The device address of `scratch` on the current device (looked up once per device).
static hipError_t scratch_ptr(void **out)
{
    static std::mutex mu;
    static void *addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

KVC_EXPORT kvc_status kvc_decode_attn_noalloc(const kvc_dims *dims, const void *q, const void *kc, const void *vc,
                                              const int32_t *count, int32_t cap, float scale, void *out, float *lse,
                                              void *stream)
{
    kvc_status st = check_dims(dims, false);
    if (st != KVC_OK) return st;
    if (cap < 1 || cap > (1 << 30)) return KVC_ERR_INVALID_ARG;
    if (!q || !kc || !vc || !count || !out) return KVC_ERR_INVALID_ARG;
    if (!(scale >= 0.f) || scale > 1e30f) return KVC_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(kc) || !aligned16(vc) || !aligned16(out)) return KVC_ERR_INVALID_ARG;
    kvc::DecodePlan plan = kvc::plan_decode(dims->batch, dims->n_h, dims->n_kv, dims->d_h, cap, kPlanCus);
    if (plan.ws_bytes > kNoAllocScratchBytes) return KVC_ERR_WORKSPACE;
    void *ws = nullptr;
    if (scratch_ptr(&ws) != hipSuccess) return KVC_ERR_HIP;
    const float sc = scale == 0.f ? 1.0f / sqrtf((float)dims->d_h) : scale;
    hipError_t e = kvc::launch_decode(dims->batch, dims->n_h, dims->n_kv, dims->d_h, dims->dtype == KVC_BF16, q,
                                      kc, vc, count, cap, sc, out, lse, ws, plan, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// ------------------------------------------------------------------------- query similarity

KVC_EXPORT kvc_status kvc_query_similarity(const kvc_dims *dims, const void *q_cur, const void *q_prev, double tau,
                                           float *cos, int32_t *refresh, int32_t *keep, void *stream)
{
    kvc_status st = check_dims(dims, false);
    if (st != KVC_OK) return st;
    if (!q_cur || !q_prev || !refresh) return KVC_ERR_INVALID_ARG;
    uint64_t tau_bits;
    memcpy(&tau_bits, &tau, sizeof tau_bits);
    if (((tau_bits >> 52) & 0x7ff) == 0x7ff) return KVC_ERR_INVALID_ARG;   // inf or NaN (bit test: NaN-free flags)
    if (!aligned16(q_cur) || !aligned16(q_prev)) return KVC_ERR_INVALID_ARG;
    hipError_t e = kvc::launch_similarity(dims->batch, dims->n_h, dims->n_kv, dims->d_h, dims->dtype == KVC_BF16,
                                          q_cur, q_prev, tau, cos, refresh, keep, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

// ------------------------------------------------------------------- block selection

KVC_EXPORT kvc_status kvc_block_landmarks(const kvc_dims *dims, const void *k, int32_t block, float *landmarks,
                                          void *stream)
{
    kvc_status st = check_dims(dims, true);
    if (st != KVC_OK) return st;
    if (!k || !landmarks || block < 1 || block > dims->s_max) return KVC_ERR_INVALID_ARG;
    if (!aligned16(k) || !aligned16(landmarks)) return KVC_ERR_INVALID_ARG;
    hipError_t e = kvc::launch_block_landmarks(dims->batch, dims->n_kv, dims->s_max, dims->d_h,
                                               dims->dtype == KVC_BF16, dims->seq_lens, k, block, landmarks,
                                               (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

KVC_EXPORT kvc_status kvc_block_scores(const kvc_dims *dims, const void *q, const float *landmarks, int32_t block,
                                       int32_t n_keep, float scale, float *scores, int32_t *cand, void *stream)
{
    kvc_status st = check_dims(dims, true);
    if (st != KVC_OK) return st;
    if (!q || !landmarks || !scores || !cand || block < 1 || block > dims->s_max || n_keep < 0)
        return KVC_ERR_INVALID_ARG;
    if (!(scale >= 0.f) || scale > 1e30f) return KVC_ERR_INVALID_ARG;
    if (!aligned16(landmarks)) return KVC_ERR_INVALID_ARG;
    const double sc = scale == 0.f ? 1.0 / sqrt((double)dims->d_h) : (double)scale;
    hipError_t e = kvc::launch_block_scores(dims->batch, dims->n_h, dims->n_kv, dims->d_h, dims->dtype == KVC_BF16,
                                            dims->s_max, dims->seq_lens, q, landmarks, block, n_keep, sc, scores,
                                            cand, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}

KVC_EXPORT kvc_status kvc_expand_blocks(int32_t batch, int32_t heads, int32_t s_max, const int32_t *seq_lens,
                                        int32_t block, int32_t n_keep, const int32_t *idx_blocks,
                                        const int32_t *count_blocks, int32_t cap_blocks, int32_t *idx,
                                        int32_t *count, int32_t cap, void *stream)
{
    if (batch < 1 || heads < 1 || s_max < 1 || block < 1 || n_keep < 0 || cap_blocks < 1 || cap < 1)
        return KVC_ERR_INVALID_ARG;
    if ((long)batch * heads > kMaxUnits || cap > (1 << 30)) return KVC_ERR_INVALID_ARG;
    if (!idx_blocks || !count_blocks || !idx || !count) return KVC_ERR_INVALID_ARG;
    hipError_t e = kvc::launch_expand_blocks(batch, heads, s_max, seq_lens, block, n_keep, idx_blocks, count_blocks,
                                             cap_blocks, idx, count, cap, (hipStream_t)stream);
    return e == hipSuccess ? KVC_OK : KVC_ERR_HIP;
}
