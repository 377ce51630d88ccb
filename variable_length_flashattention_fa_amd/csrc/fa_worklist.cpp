// Host-side work list for the KV-block-major backward kernel.
//
// Each item is one block of FA_BLOCK_KV keys of one sequence together with the
// contiguous range of query tiles that hold at least one admitted pair with a
// key in that block.  Ranges follow from the mask definitions of the
// "FlashAttention梯度V2" page (parameter table: attenMask with 1 = excluded,
// preTokens / nextTokens as the window's left / right bounds), with the
// causal and band windows aligned to the bottom-right corner.  Blocks and tiles
// that no admitted pair touches are skipped, except that every key block gets
// an item so its dK / dV rows are written.
#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "fa_internal.h"

namespace fa {

static thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }
void clear_error() { g_error.clear(); }
const char* last_error_cstr() { return g_error.c_str(); }

int check_seqlens(const fa_seqlens_t* s, const char* name) {
    if (s == nullptr || s->cu == nullptr) {
        set_error(std::string(name) + " is null");
        return FA_ERR_NULLPTR;
    }
    // the page limits the length arrays to 1..2K entries
    if (s->batch < 1 || s->batch > 2048) {
        set_error(std::string(name) + ": batch must be in [1, 2048], got " + std::to_string(s->batch));
        return FA_ERR_INVALID;
    }
    if (s->cu[0] != 0) {
        set_error(std::string(name) + ": cu[0] must be 0");
        return FA_ERR_INVALID;
    }
    for (int64_t b = 0; b < s->batch; ++b) {
        if (s->cu[b + 1] < s->cu[b]) {
            set_error(std::string(name) + ": prefix sums must be non-decreasing (at " + std::to_string(b) + ")");
            return FA_ERR_INVALID;
        }
    }
    return FA_OK;
}

// Rows [lo, hi] of a sequence (Lq = lq, Lkv = lkv) that admit at least one key
// in [j0, j1].  Returns false when no row does.
static bool admitted_rows(int64_t lq, int64_t lkv, int32_t mode, int64_t pre, int64_t nxt,
                          int64_t j0, int64_t j1, int64_t& lo, int64_t& hi) {
    const int64_t off = lkv - lq;
    lo = 0;
    hi = lq - 1;
    if (mode == FA_MASK_CAUSAL) {
        // j <= i + off for some j >= j0  <=>  i >= j0 - off
        lo = std::max<int64_t>(lo, j0 - off);
    } else if (mode == FA_MASK_BAND) {
        if (pre + nxt < 0) return false;  // every window is empty
        // i + off - pre <= j1  and  i + off + nxt >= j0
        lo = std::max<int64_t>(lo, j0 - off - nxt);
        hi = std::min<int64_t>(hi, j1 - off + pre);
    }
    return lo <= hi;
}

int64_t build_worklist(const int64_t* cu_q, const int64_t* cu_kv, int64_t batch, int32_t mode,
                       int64_t pre, int64_t nxt, int64_t heads, int32_t block_q,
                       std::vector<fa_work_item_t>& out) {
    out.clear();
    pre = clamp_window(pre);
    nxt = clamp_window(nxt);
    int64_t drop_base = 0;
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t lq = cu_q[b + 1] - cu_q[b];
        const int64_t lkv = cu_kv[b + 1] - cu_kv[b];
        const int64_t nblocks = (lkv + FA_BLOCK_KV - 1) / FA_BLOCK_KV;
        for (int64_t jb = 0; jb < nblocks; ++jb) {
            const int64_t j0 = jb * FA_BLOCK_KV;
            const int64_t j1 = std::min<int64_t>(lkv, j0 + FA_BLOCK_KV) - 1;
            fa_work_item_t it;
            std::memset(&it, 0, sizeof(it));
            it.q_start = static_cast<int32_t>(cu_q[b]);
            it.kv_start = static_cast<int32_t>(cu_kv[b]);
            it.len_q = static_cast<int32_t>(lq);
            it.len_kv = static_cast<int32_t>(lkv);
            it.kv_block = static_cast<int32_t>(jb);
            it.seq = static_cast<int32_t>(b);
            it.drop_base = drop_base;
            int64_t lo, hi;
            if (lq > 0 && admitted_rows(lq, lkv, mode, pre, nxt, j0, j1, lo, hi)) {
                it.tile_begin = static_cast<int32_t>(lo / block_q);
                it.tile_end = static_cast<int32_t>(hi / block_q + 1);
            } else {
                it.tile_begin = 0;
                it.tile_end = 0;
            }
            out.push_back(it);
        }
        drop_base += heads * lq * lkv;
    }
    // longest first, so the long causal blocks do not trail at the end of the grid
    std::stable_sort(out.begin(), out.end(), [](const fa_work_item_t& a, const fa_work_item_t& b) {
        return (a.tile_end - a.tile_begin) > (b.tile_end - b.tile_begin);
    });
    return static_cast<int64_t>(out.size());
}

}  // namespace fa

extern "C" int64_t fa_varlen_worklist(const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                                      int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens,
                                      int64_t heads, int32_t block_q, fa_work_item_t* items,
                                      int64_t capacity) {
    fa::clear_error();
    int st = fa::check_seqlens(cu_seqlens_q, "cu_seqlens_q");
    if (st != FA_OK) return -st;
    st = fa::check_seqlens(cu_seqlens_kv, "cu_seqlens_kv");
    if (st != FA_OK) return -st;
    if (cu_seqlens_q->batch != cu_seqlens_kv->batch) {
        fa::set_error("cu_seqlens_q and cu_seqlens_kv have different batch counts");
        return -FA_ERR_INVALID;
    }
    if (atten_mode < FA_MASK_NONE || atten_mode > FA_MASK_BAND) {
        fa::set_error("atten_mode must be 0 (none), 1 (causal) or 2 (band)");
        return -FA_ERR_INVALID;
    }
    if (block_q <= 0 || heads < 1) {
        fa::set_error("block_q and heads must be positive");
        return -FA_ERR_INVALID;
    }
    std::vector<fa_work_item_t> list;
    const int64_t n = fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, cu_seqlens_q->batch,
                                         atten_mode, pre_tokens, next_tokens, heads, block_q, list);
    if (items != nullptr) {
        const int64_t m = std::min(n, capacity);
        if (m > 0) std::memcpy(items, list.data(), static_cast<size_t>(m) * sizeof(fa_work_item_t));
    }
    return n;
}
