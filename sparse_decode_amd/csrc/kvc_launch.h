// kvc_launch.h -- host-side launchers of the gfx950 kernels.  Arguments reaching
// these functions have been validated by the C ABI layer (kvc_api.hip); each
// launcher only sizes grids and enqueues kernels on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvc {

struct DeviceInfo {
    int cus = 256;              // compute units
    int max_lds_per_block = 65536;
};
// Attributes of the current device (cached per device ordinal).
hipError_t device_info(DeviceInfo *out);

// ---- gather -------------------------------------------------------------------------
hipError_t launch_gather(int batch, int heads, int s_max, int row_bytes, const void *src0,
                         const void *src1, const int32_t *src_pos, const int32_t *idx,
                         const int32_t *count, int idx_heads, int cap, void *dst0, void *dst1,
                         int32_t *pos_out, const int32_t *unit_mask, const DeviceInfo &dev,
                         hipStream_t stream);

// ---- decode -------------------------------------------------------------------------
// Decode workspace: kDecCounters arrival counters (zero between calls), then the
// split partial outputs and (max, sum) pairs.
constexpr int kDecCounters = 16384;
struct DecodePlan {
    int n_splits = 1;
    int split_tokens = 0;
    int head_chunk = 1;        // query heads handled per work-group
    int head_chunks = 1;
    bool fused = false;        // the last work-group of a chunk folds its splits
    size_t o_off = 0;          // split partial outputs
    size_t ml_off = 0;         // split (max, sum) pairs
    size_t ws_bytes = 0;
};
DecodePlan plan_decode(int batch, int n_h, int n_kv, int d_h, int cap, int cus);
hipError_t launch_decode(int batch, int n_h, int n_kv, int d_h, bool bf16, const void *q,
                         const void *kc, const void *vc, const int32_t *count, int cap, float scale,
                         void *out, float *lse, void *ws, const DecodePlan &plan, hipStream_t stream);

// ---- select -------------------------------------------------------------------------
size_t select_ws_bytes(int batch, int n_kv, int s_max, int n_keep, bool shared);
hipError_t launch_select(int batch, int n_kv, int s_max, const int32_t *seq_lens, const float *scores,
                         int k, int n_keep, bool shared, int32_t *idx, int32_t *count,
                         const int32_t *unit_mask, const int32_t *k_per_unit, void *ws,
                         const DeviceInfo &dev, hipStream_t stream);

// role-based retention (core tokens always kept, the budget over the others)
size_t select_core_ws_bytes(int batch, int n_kv, int s_max, int n_keep);
hipError_t launch_select_core(int batch, int n_kv, int s_max, const int32_t *seq_lens, const float *scores,
                              const uint8_t *core, int k, int core_cap, int n_keep, int32_t *idx, int32_t *count,
                              const int32_t *unit_mask, void *ws, const DeviceInfo &dev, hipStream_t stream);

// ---- score --------------------------------------------------------------------------
struct ScorePlan {
    bool mfma = false;
    int R = 0;                 // rows per KV head: (n_h / n_kv) * w
    int rt = 0;                // MFMA path: blocks of 16 rows (1, 2, 4 or 8)
    int tiles_per_wave = 1;    // MFMA path: 32-token tiles per wave per chunk
    int chunk_tokens = 0;      // MFMA path: tokens per work-group
    int n_chunks = 0;
    int n_parts = 0;           // MFMA two-pass path: row partials per unit (per chunk, or per
                               // 256-token block with one row block)
    int group_units = 0;       // KV-head units per pass-1/pass-2 launch pair
    int logit_rows = 0;        // MFMA path, R <= 16: logits kept per token between the passes
    bool fold_merge = false;   // two-pass MFMA path: the last pass-1 work-group of a unit merges its
                               // chunks' row statistics (else a merge kernel between the passes)
    size_t logits_off = 0;     // their place in the workspace
    // single-pass MFMA path (16 < R <= 32, S <= 131072): K read once, 1024-token items; its
    // zero-state words open the workspace and the two-pass region (a fallback when too
    // few work-groups fit the device at once) follows at two_pass_off
    bool single = false;
    int sp_chunks = 0;         // items per unit
    int sp_item = 0;           // tokens per item
    int sp_spin = 5000;        // bound of an item's wait (100 MHz ticks: 50 us) before it is deferred
    size_t two_pass_off = 0;
    size_t ws_bytes = 0;
};
ScorePlan plan_score(int batch, int s_max, int n_h, int n_kv, int d_h, bool bf16, int w,
                     bool generic, int cus);
hipError_t launch_score(int batch, int s_max, const int32_t *seq_lens, int n_h, int n_kv, int d_h,
                        bool bf16, const void *q_win, const void *k, int w, bool window_in_cache,
                        int n_keep, int pool, float scale, float *raw, float *pooled,
                        const int32_t *unit_mask, void *ws, const ScorePlan &plan, hipStream_t stream);

// ---- landmark-guided block selection ------------------------------------------------
hipError_t launch_block_landmarks(int batch, int n_kv, int s_max, int d_h, bool bf16, const int32_t *seq_lens,
                                  const void *k, int block, float *landmarks, hipStream_t stream);
hipError_t launch_block_scores(int batch, int n_h, int n_kv, int d_h, bool bf16, int s_max, const int32_t *seq_lens,
                               const void *q, const float *landmarks, int block, int n_keep, double scale,
                               float *scores, int32_t *cand, hipStream_t stream);
hipError_t launch_expand_blocks(int batch, int heads, int s_max, const int32_t *seq_lens, int block, int n_keep,
                                const int32_t *idx_blk, const int32_t *count_blk, int cap_blk, int32_t *idx,
                                int32_t *count, int cap, hipStream_t stream);

// ---- query similarity ---------------------------------------------------------------
hipError_t launch_similarity(int batch, int n_h, int n_kv, int d_h, bool bf16, const void *q_cur,
                             const void *q_prev, double tau, float *cos, int32_t *refresh, int32_t *keep,
                             hipStream_t stream);

}  // namespace kvc
