// Launchers of the gfx950 kernels (defined in fa_kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa_varlen.h"

namespace fa {

// Explicit attention mask as the kernels see it: element (b, n, i, j) at
// amask[b * am_sb + n * am_sn + i * am_sq + j]; amask == nullptr: no explicit mask.
struct MaskArg {
    const uint8_t* amask = nullptr;
    int64_t am_sb = 0;
    int64_t am_sn = 0;
    int32_t am_sq = 0;
};

template <typename A>
inline void set_mask(A& a, const fa_mask_t* m) {
    if (m == nullptr) {
        a.mask = MaskArg{};
        return;
    }
    a.mask.amask = m->data;
    a.mask.am_sb = m->stride_b;
    a.mask.am_sn = m->stride_n;
    a.mask.am_sq = static_cast<int32_t>(m->stride_q);
}

struct TensorArg {
    const void* data;
    int64_t stride_t;
    int64_t stride_h;
};

// Row pass: D[n, t] = sum_d dY * Y (fp32, over V's head dim) and beta[n, t] = max*log2(e) +
// log2(sum).  rowstat holds two planes of heads * tq floats: rowstat[n * tq + t] = -D[n, t]
// and rowstat[heads * tq + n * tq + t] = -beta[n, t] (both negated: the kernels start their dP
// and S accumulators from them).
hipError_t launch_preprocess(int32_t dtype, int head_dim_v, TensorArg dy, TensorArg y,
                             const float* softmax_max, const float* softmax_sum, float* rowstat,
                             int64_t tq, int64_t heads, hipStream_t stream);

struct MainArgs {
    TensorArg q, k, v, dy;
    void* dq;
    int64_t dq_st, dq_sh;
    void* dk;
    int64_t dk_st, dk_sh;
    void* dv;
    int64_t dv_st, dv_sh;
    const float* rowstat;  // planes of -D and -beta (see launch_preprocess)
    const fa_work_item_t* items;    // key-block items (kBlockKv32 keys, kTileQ32 query tiles)
    const fa_work_item_t* items_q;  // query-block items (FA32_FWD_BLOCK queries)
    const uint8_t* drop_mask;
    MaskArg mask;
    int32_t tq;
    int32_t heads;   // query heads
    int32_t group;   // query heads per key/value head
    int32_t mode;
    int32_t pre;     // clamped window bounds
    int32_t nxt;
    float exp_scale;  // scale * log2(e)
    float inv_keep;   // 1 / keep_prob
    float scale;      // folded into dK and dQ
};

constexpr int FA32_FWD_BLOCK = 64;  // queries per fp32 forward / dQ workgroup (one per thread)

// fp32 dK/dV kernel over n_items key-block items x key/value heads.  Head dims (Q/K, V):
// (128, 128), (128, 64) or (64, 64).
hipError_t launch_main(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, const MainArgs& a,
                       int64_t n_items, hipStream_t stream);

// fp32 dQ kernel over n_items query-block items x query heads; the same head dims.
hipError_t launch_dq32(int head_dim_k, int head_dim_v, bool dropout, const MainArgs& a, int64_t n_items,
                       hipStream_t stream);

// ---- 16-bit path: dK/dV and dQ kernels without atomics ----
constexpr int FA16_DKDV_BLOCK = 128;  // keys per dK/dV workgroup
constexpr int FA16_DKDV_TILE_Q = 64;  // query rows per dK/dV step
constexpr int FA16_DQ_BLOCK = 256;    // queries per dQ workgroup
constexpr int FA16_DQ_TILE_K = 64;    // key rows per dQ tile (two steps of 32)

struct Bwd16Args {
    const void* q;
    const void* k;
    const void* v;
    const void* dy;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, dy_st, dy_sh;
    void* dq;
    void* dk;
    void* dv;
    int64_t dq_st, dq_sh, dk_st, dk_sh, dv_st, dv_sh;
    // planes of -D and -beta (layout as in launch_preprocess): written by the dQ kernel, which computes
    // them for its rows from dY, Y and the forward statistics, and read by the dK/dV kernel after it
    float* rowstat;
    const void* y;
    int64_t y_st, y_sh;
    const float* softmax_max;  // [heads, tq, 8]; element 0 of each row is read
    const float* softmax_sum;
    const fa_work_item_t* items_kv;  // key-block items (FA16_DKDV_BLOCK keys, FA16_DKDV_TILE_Q tiles)
    const fa_work_item_t* items_q;   // query-block items (FA16_DQ_BLOCK queries, FA16_DQ_TILE_K tiles)
    const uint8_t* drop_mask;
    int64_t drop_bytes;  // size of the dropout mask in bytes (bounds its reads)
    MaskArg mask;
    int32_t tq, heads, group, mode, pre, nxt;  // heads: query heads; group: query heads per key/value head
    float exp_scale, inv_keep, scale;
    int32_t xcd_group;  // renumber workgroups so each XCD runs whole heads (see wg_unit); set per launch
};

// dK/dV kernel over n_items key-block items x key/value heads (each sums its group of query heads).
// Reads the row statistics planes, so it runs after the dQ kernel.
// Head dims (Q/K, V): (128, 128), (128, 64) or (64, 64).
hipError_t launch_dkdv16(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, bool xmask,
                         const Bwd16Args& a, int64_t n_items, hipStream_t stream);

// dQ kernel over n_items query-block items x query heads; the same head dims.
hipError_t launch_dq16(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, bool xmask,
                       const Bwd16Args& a, int64_t n_items, hipStream_t stream);

// ---- forward ----------------------------------------------------------------------------------
// Y = Dropout(Softmax(Mask(scale Q K^T))) V and the row statistics, over query-block items.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh;
    void* y;
    int64_t y_st, y_sh;
    float* smax;  // [N, Tq, 8]
    float* ssum;  // [N, Tq, 8]
    const fa_work_item_t* items;  // query-block items
    const uint8_t* drop_mask;
    int64_t drop_bytes;  // size of the dropout mask in bytes (bounds its reads)
    MaskArg mask;
    int32_t tq, heads, group, mode, pre, nxt;  // heads: query heads; group: query heads per key/value head
    float scale, exp_scale, inv_keep;
    int32_t xcd_group;  // renumber workgroups so each XCD runs whole heads (see wg_unit); set per launch
};

// bf16 / fp16 forward over n_items query-block items (FA16_DQ_BLOCK queries, FA16_DQ_TILE_K tiles).
// Head dims (Q/K, V): (128, 128), (128, 64) or (64, 64).
hipError_t launch_fwd16(int32_t dtype, int head_dim_k, int head_dim_v, bool dropout, bool xmask,
                        const FwdArgs& a, int64_t n_items, hipStream_t stream);
// fp32 forward over n_items query-block items (FA32_FWD_BLOCK queries); the same head dims.
hipError_t launch_fwd32(int head_dim_k, int head_dim_v, bool dropout, const FwdArgs& a, int64_t n_items,
                        hipStream_t stream);

}  // namespace fa
