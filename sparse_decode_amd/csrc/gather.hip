// gather.hip -- compacting gather of kept cache rows that keeps their original
// positions (Tutorial "Variantes de l'attention et compression du cache KV",
// section "Quand la reutilisation est-elle exacte ?": keep the original position
// indices after eviction).
//
// Pure data movement, bound by HBM bandwidth: every kept row is read once and
// written once with 16-byte vector accesses.  A row of d_h = 128 bf16 is 256 B =
// 16 lanes; a 4096-wide hidden-state row is 8 KiB = 512 lanes.
#include "kvc_device.h"
#include "kvc_launch.h"

namespace kvc {
namespace {

constexpr int kGatherThreads = 256;
constexpr int kMaxBlockRows = 4096;     // rows per work-group (their indices sit in LDS)

// Work-group (kvc_bid_x(), kvc_bid_y()) copies rows [kvc_bid_x() * rows_per_block, ...)
// of unit kvc_bid_y() = b * heads + h.  The block's source rows are resolved once
// into LDS (one dependent round trip), then every thread keeps U rows of 16-byte
// loads (times two with src1) in flight.  tpr threads share one row (a power of two
// <= 256); a row wider than 256 vectors is walked in strides of 256.
template <int U>
__global__ __launch_bounds__(kGatherThreads) void gather_rows_kernel(
    const u32x4 *__restrict__ src0, const u32x4 *__restrict__ src1,
    const int32_t *__restrict__ src_pos, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ count, int heads, int idx_heads, int s_max, int vpr, int tpr_log2,
    int cap, int rows_per_block, u32x4 *__restrict__ dst0, u32x4 *__restrict__ dst1,
    int32_t *__restrict__ pos_out, const int32_t *__restrict__ mask)
{
    __shared__ int rows[kMaxBlockRows];
    const int unit = kvc_bid_y();
    const int b = unit / heads;
    const int h = unit - b * heads;
    const int list = b * idx_heads + (idx_heads == 1 ? 0 : h);
    if (mask && !ld_uniform(mask, list)) return;
    const int r0 = kvc_bid_x() * rows_per_block;
    const int r1 = min(r0 + rows_per_block, cap);
    const int32_t *lidx = idx + (size_t)list * cap;
    int n = count[list];
    n = n < 0 ? 0 : (n > cap ? cap : n);

    // source row of every output row of the block, -1 where nothing is copied
    for (int j = r0 + (int)kvc_tid(); j < r1; j += kGatherThreads) {
        const int t = lidx[j];
        const bool ok = j < n && t >= 0 && t < s_max;
        rows[j - r0] = ok ? t : -1;
        if (pos_out) pos_out[(size_t)unit * cap + j] = ok ? (src_pos ? src_pos[(size_t)b * s_max + t] : t) : -1;
    }
    __syncthreads();

    const int tpr = 1 << tpr_log2;
    const int rows_per_iter = kGatherThreads >> tpr_log2;
    const int sub = kvc_tid() >> tpr_log2;
    const int col0 = kvc_tid() & (tpr - 1);
    const size_t src_unit = (size_t)unit * s_max * vpr;
    const size_t dst_unit = (size_t)unit * cap * vpr;
    const int m = min(r1, n) - r0;                       // rows of this block that are copied
    for (int j0 = sub; j0 < m; j0 += rows_per_iter * U) {
        int t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u * rows_per_iter;
            t[u] = j < m ? rows[j] : -1;
        }
        for (int c = col0; c < vpr; c += tpr) {
            // every load is unconditional (an absent row reads row 0 of the unit, which
            // exists) so that all of them are in flight before the first store; a load
            // under a branch would be waited for inside it
            u32x4 a[U], bb[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int tr = t[u] >= 0 ? t[u] : 0;
                a[u] = ld_stream(src0 + src_unit + (size_t)tr * vpr + c);
                if (src1) bb[u] = ld_stream(src1 + src_unit + (size_t)tr * vpr + c);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (t[u] >= 0) {
                    const size_t o = dst_unit + (size_t)(r0 + j0 + u * rows_per_iter) * vpr + c;
                    dst0[o] = a[u];
                    if (src1) dst1[o] = bb[u];
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gather(int batch, int heads, int s_max, int row_bytes, const void *src0,
                         const void *src1, const int32_t *src_pos, const int32_t *idx,
                         const int32_t *count, int idx_heads, int cap, void *dst0, void *dst1,
                         int32_t *pos_out, const int32_t *unit_mask, const DeviceInfo &dev,
                         hipStream_t stream)
{
    const int vpr = row_bytes / 16;
    int tpr_log2 = 0;
    while ((1 << (tpr_log2 + 1)) <= vpr && (1 << (tpr_log2 + 1)) <= kGatherThreads) ++tpr_log2;
    const int rows_per_iter = kGatherThreads >> tpr_log2;
    const long units = (long)batch * heads;
    // Enough work-groups to cover every CU several times (a small cache is spread
    // thin: the copy is latency-bound there), at most kMaxBlockRows rows each.
    const long want_blocks = 4L * dev.cus;
    long rpb = (long)cap * units / (want_blocks > 0 ? want_blocks : 1);
    const long min_rows = (long)rows_per_iter * 2;
    if (rpb < min_rows) rpb = min_rows;
    rpb = ((rpb + min_rows - 1) / min_rows) * min_rows;
    if (rpb > kMaxBlockRows) rpb = kMaxBlockRows;
    if (rpb > cap) rpb = cap;
    if (rpb < 1) rpb = 1;
    dim3 grid((unsigned)((cap + rpb - 1) / rpb), (unsigned)units);
    // two loads in flight per thread: one row of K and V, or two rows of one tensor
    // (measured against 4 and 8 rows per thread)
    if (src1)
        hipLaunchKernelGGL(gather_rows_kernel<1>, grid, dim3(kGatherThreads), 0, stream,
                           (const u32x4 *)src0, (const u32x4 *)src1, src_pos, idx, count, heads, idx_heads,
                           s_max, vpr, tpr_log2, cap, (int)rpb, (u32x4 *)dst0, (u32x4 *)dst1, pos_out, unit_mask);
    else
        hipLaunchKernelGGL(gather_rows_kernel<2>, grid, dim3(kGatherThreads), 0, stream,
                           (const u32x4 *)src0, (const u32x4 *)src1, src_pos, idx, count, heads, idx_heads,
                           s_max, vpr, tpr_log2, cap, (int)rpb, (u32x4 *)dst0, (u32x4 *)dst1, pos_out, unit_mask);
    return hipGetLastError();
}

}  // namespace kvc
