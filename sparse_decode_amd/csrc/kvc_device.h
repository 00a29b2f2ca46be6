// kvc_device.h -- device-side helpers shared by the gfx950 kernels of the KV-cache
// compression path: bf16 conversion, 64-lane shuffles, exchange between work-groups
// and work-group scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// Work-item and work-group indices read from the hardware registers.  The kernels are
// built with IEEE mode off and the device library's index functions with it on, so
// the library's versions are not inlined: every kernel would call out for them and
// get per-lane results back, hiding that a work-group index is uniform.
__device__ __forceinline__ unsigned kvc_tid() { return __builtin_amdgcn_workitem_id_x(); }
__device__ __forceinline__ unsigned kvc_bid_x() { return __builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ unsigned kvc_bid_y() { return __builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ unsigned kvc_bid_z() { return __builtin_amdgcn_workgroup_id_z(); }
__device__ __forceinline__ unsigned kvc_bdim_x() { return __builtin_amdgcn_workgroup_size_x(); }

constexpr int kWave = 64;

// Native 16-byte vector (HIP's uint4 is a struct; clang builtins want a vector type).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load hinted as streamed once (non-temporal).
__device__ __forceinline__ u32x4 ld_stream(const u32x4 *p) { return __builtin_nontemporal_load(p); }

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the high half of the float).
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Round to nearest, ties to even; a NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, kWave); }

// Lane exchanges inside a row of 16 lanes, as DPP operand modifiers (plain VALU
// instructions, no LDS crossbar): the mirrors pair lane i with 15 - i (row) or with
// 7 - i inside each half row; the quad permutations pair i with i ^ 2 and i ^ 1.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}
constexpr int kDppRowMirror = 0x140;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppXor2 = 0x4e;     // quad_perm(2, 3, 0, 1)
constexpr int kDppXor1 = 0xb1;     // quad_perm(1, 0, 3, 2)

// Sum over the 16 lanes of a row; every lane receives the total.  The pairings
// (mirror, half mirror, xor 2, xor 1) cover each lane of the row exactly once.
__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_f<kDppRowMirror>(v);
    v += dpp_f<kDppHalfMirror>(v);
    v += dpp_f<kDppXor2>(v);
    v += dpp_f<kDppXor1>(v);
    return v;
}

// p[i] for a wave-uniform i, through the scalar data cache (the constant address
// space): for arrays that no work-group of the running kernel writes (lengths, masks,
// budgets, counts from an earlier kernel), so the load takes no vector memory round
// trip ahead of the kernel's streaming loads.
template <typename T>
__device__ __forceinline__ T ld_uniform(const T *p, int i)
{
    return ((const __attribute__((address_space(4))) T *)p)[i];
}

__device__ __forceinline__ int clamp_len(const int32_t *seq_lens, int b, int s_max)
{
    int s = seq_lens ? ld_uniform(seq_lens, b) : s_max;
    return s < 0 ? 0 : (s > s_max ? s_max : s);
}

// ---- exchange between the work-groups of one running kernel.  Agent-scope relaxed
// atomic loads and stores are coherent across the XCDs (they do not hit a stale line
// of an XCD's own L2); a work-group publishes with st_dev, waits with stores_done()
// until its stores have completed, and only then counts its arrival atomically, so a
// work-group that sees the count complete reads every published value with ld_dev.
__device__ __forceinline__ unsigned long long ld_dev(const unsigned long long *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(unsigned long long *p, unsigned long long v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p)
{
    return __uint_as_float(__hip_atomic_load((const uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_dev(float *p, float v)
{
    __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t ld_dev(const int32_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(int32_t *p, int32_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this thread's earlier memory operations (its stores too) have completed.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ unsigned long long pack2(float a, float b)
{
    return (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32);
}
__device__ __forceinline__ float unpack_lo(unsigned long long v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float unpack_hi(unsigned long long v) { return __uint_as_float((uint32_t)(v >> 32)); }

// v from another lane by a DPP operand modifier, for the rows of 16 lanes in ROW_MASK;
// 0 in lanes with no source lane and in the other rows.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row to the next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 to rows 2 and 3

// Inclusive prefix sum across one 64-lane wave (every lane active), in VALU operand
// modifiers: shifts by 1, 2, 4 and 8 lanes give the scan inside each row of 16; then
// rows 1 and 3 add the last lane of the row before, and rows 2 and 3 add lane 31, by
// then the total of rows 0 and 1.
__device__ __forceinline__ int wave_inclusive_scan(int v)
{
    v += dpp_i<kDppRowShr1, 0xf>(v);
    v += dpp_i<kDppRowShr2, 0xf>(v);
    v += dpp_i<kDppRowShr4, 0xf>(v);
    v += dpp_i<kDppRowShr8, 0xf>(v);
    v += dpp_i<kDppRowBcast15, 0xa>(v);
    v += dpp_i<kDppRowBcast31, 0xc>(v);
    return v;
}

// Exclusive prefix sum across the work-group (kvc_bdim_x() a multiple of 64, at most
// 1024).  `scratch` holds at least 16 ints of LDS.  Returns the exclusive prefix and
// writes the group total to *total.  Every wave adds the wave totals it needs itself
// (broadcast LDS reads), so there is no serial pass.  Contains barriers: call from
// every thread.
__device__ __forceinline__ int block_exclusive_scan(int v, int *scratch, int *total)
{
    const int lane = kvc_tid() & (kWave - 1);
    const int wid = kvc_tid() >> 6;
    const int nw = kvc_bdim_x() >> 6;
    const int inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) scratch[wid] = inc;
    __syncthreads();
    int pre = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int t = i < nw ? scratch[i] : 0;
        pre += i < wid ? t : 0;
        tot += t;
    }
    *total = tot;
    __syncthreads();
    return pre + inc - v;
}

// Exclusive prefix sums of two values across the work-group with the barriers of one
// scan; `scratch` holds at least 32 ints of LDS.  Same conditions as above; the group
// totals go to *total when it is not null.
__device__ __forceinline__ int2 block_exclusive_scan2(int a, int b, int *scratch, int2 *total = nullptr)
{
    const int lane = kvc_tid() & (kWave - 1);
    const int wid = kvc_tid() >> 6;
    const int nw = kvc_bdim_x() >> 6;
    const int ia = wave_inclusive_scan(a);
    const int ib = wave_inclusive_scan(b);
    if (lane == kWave - 1) {
        scratch[wid] = ia;
        scratch[16 + wid] = ib;
    }
    __syncthreads();
    int pa = 0, pb = 0, ta = 0, tb = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (i < nw) {
            const int sa = scratch[i], sb = scratch[16 + i];
            if (i < wid) {
                pa += sa;
                pb += sb;
            }
            ta += sa;
            tb += sb;
        }
    }
    if (total) *total = make_int2(ta, tb);
    __syncthreads();
    return make_int2(pa + ia - a, pb + ib - b);
}

}  // namespace kvc
