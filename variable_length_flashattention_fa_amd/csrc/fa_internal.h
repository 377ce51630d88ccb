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

}  // namespace fa
