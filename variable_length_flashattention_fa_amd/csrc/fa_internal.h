// Internal declarations shared by the host-side sources of libfa_varlen.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "fa_varlen.h"

namespace fa {

// Thread-local error message behind fa_last_error().
void set_error(const std::string& msg);
void clear_error();

// Query tile height of the fp32 kernel (fp32 operands double every staged tile).
constexpr int kTileQ32 = 32;

// Window bounds are clamped to +-2^24: T <= 2^20 on the page, so any wider
// window admits the same keys, and int32 index math in the kernel cannot
// overflow.
constexpr int64_t kWindowClamp = int64_t(1) << 24;
inline int64_t clamp_window(int64_t x) {
    return x > kWindowClamp ? kWindowClamp : (x < -kWindowClamp ? -kWindowClamp : x);
}

// Checks one cu_seqlens array: batch in [1, 2048], cu[0] == 0, non-decreasing.
// Returns FA_OK or an error status (message set).
int check_seqlens(const fa_seqlens_t* s, const char* name);

// Head dims (Q and K, V) the kernels are built for: (128, 128), (128, 64) and (64, 64).
inline bool head_dims_supported(int64_t dk, int64_t dv) {
    return (dk == 128 && (dv == 128 || dv == 64)) || (dk == 64 && dv == 64);
}

// Key rows per workgroup of the fp32 kernel.
constexpr int kBlockKv32 = 128;

// Builds a work list (see fa_varlen_worklist in fa_varlen.h).  Inputs must
// already be validated.  Returns the item count.
int64_t build_worklist(const int64_t* cu_q, const int64_t* cu_kv, int64_t batch, int32_t mode, int64_t pre,
                       int64_t nxt, int64_t heads, int32_t kind, int32_t block_rows, int32_t tile_rows,
                       std::vector<fa_work_item_t>& out);

// A validated backward call: the caller's arguments, with the window bounds clamped.  Pointers
// are borrowed for the duration of the call.
struct BwdPlan {
    const fa_tensor_t* q = nullptr;
    const fa_tensor_t* k = nullptr;
    const fa_tensor_t* v = nullptr;
    const fa_tensor_t* dy = nullptr;
    const fa_tensor_t* y = nullptr;
    const fa_tensor_t* dq = nullptr;
    const fa_tensor_t* dk = nullptr;
    const fa_tensor_t* dv = nullptr;
    const float* softmax_max = nullptr;
    const float* softmax_sum = nullptr;
    const int64_t* cu_q = nullptr;
    const int64_t* cu_kv = nullptr;
    int64_t batch = 0;
    int32_t mode = 0;
    int64_t pre = 0;
    int64_t nxt = 0;
    double keep_prob = 1.0;
    const uint8_t* drop_mask = nullptr;
    const fa_mask_t* atten_mask = nullptr;
    double scale = 1.0;
};

// Every check of fa_varlen_bwd_masked (null pointers, the page's constraints, what is not built);
// FA_OK fills *plan.  No device work.
int plan_bwd(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v, const fa_tensor_t* dy,
             const fa_tensor_t* y, const float* softmax_max, const float* softmax_sum,
             const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv, int32_t atten_mode,
             int64_t pre_tokens, int64_t next_tokens, double keep_prob, const uint8_t* drop_mask,
             const fa_mask_t* atten_mask, double scale, int64_t head_num, const fa_tensor_t* dq,
             const fa_tensor_t* dk, const fa_tensor_t* dv, BwdPlan* plan);

// What identifies the backward's work lists: layout, window, heads and kernel path.
std::vector<int64_t> bwd_list_key(const BwdPlan& p);

// The backward's key-block list (n_first items) followed by its query-block list.
void build_bwd_lists(const BwdPlan& p, std::vector<fa_work_item_t>& items, int64_t& n_first);

// Bytes of the two row-statistics planes (-D and -beta) of a call.
size_t bwd_rowstat_bytes(const BwdPlan& p);

}  // namespace fa
