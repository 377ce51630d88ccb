// Host-side work lists of the backward kernels.
//
// An item is a block of rows of one sequence that a workgroup keeps resident
// (keys for dK/dV, queries for dQ) together with the contiguous range of
// tiles of the other side that hold at least one admitted (query, key) pair
// with it.  The admitted set follows the mask definitions of the
// "FlashAttention梯度V2" page (parameter table: attenMask with 1 = excluded,
// preTokens / nextTokens as the window's left / right bounds), with the causal
// and band windows aligned to the bottom-right corner: with off = Lkv - Lq,
// query i admits key j iff
//   causal: j <= i + off;   band: i + off - pre <= j <= i + off + next.
// Tiles outside the range are skipped; blocks whose range is empty still get
// an item so their outputs are written as zeros.
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

// Query rows [lo, hi] (clipped to [0, lq)) admitting at least one key of [j0, j1].
static bool rows_for_keys(int64_t lq, int64_t lkv, int32_t mode, int64_t pre, int64_t nxt, int64_t j0,
                          int64_t j1, int64_t& lo, int64_t& hi) {
    const int64_t off = lkv - lq;
    lo = 0;
    hi = lq - 1;
    if (mode == FA_MASK_CAUSAL) {
        lo = std::max<int64_t>(lo, j0 - off);  // some j >= j0 with j <= i + off
    } else if (mode == FA_MASK_BAND) {
        if (pre + nxt < 0) return false;  // every window is empty
        lo = std::max<int64_t>(lo, j0 - off - nxt);
        hi = std::min<int64_t>(hi, j1 - off + pre);
    }
    return lo <= hi;
}

// Keys [lo, hi] (clipped to [0, lkv)) admitted by at least one query of [i0, i1].
static bool keys_for_rows(int64_t lq, int64_t lkv, int32_t mode, int64_t pre, int64_t nxt, int64_t i0,
                          int64_t i1, int64_t& lo, int64_t& hi) {
    const int64_t off = lkv - lq;
    lo = 0;
    hi = lkv - 1;
    if (mode == FA_MASK_CAUSAL) {
        hi = std::min<int64_t>(hi, i1 + off);
    } else if (mode == FA_MASK_BAND) {
        if (pre + nxt < 0) return false;
        lo = std::max<int64_t>(lo, i0 + off - pre);
        hi = std::min<int64_t>(hi, i1 + off + nxt);
    }
    return lo <= hi;
}

int64_t build_worklist(const int64_t* cu_q, const int64_t* cu_kv, int64_t batch, int32_t mode, int64_t pre,
                       int64_t nxt, int64_t heads, int32_t kind, int32_t block_rows, int32_t tile_rows,
                       std::vector<fa_work_item_t>& out) {
    out.clear();
    pre = clamp_window(pre);
    nxt = clamp_window(nxt);
    int64_t drop_base = 0;
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t lq = cu_q[b + 1] - cu_q[b];
        const int64_t lkv = cu_kv[b + 1] - cu_kv[b];
        const int64_t resident = kind == FA_ITEMS_KEY_BLOCKS ? lkv : lq;
        const int64_t walked = kind == FA_ITEMS_KEY_BLOCKS ? lq : lkv;
        const int64_t nblocks = (resident + block_rows - 1) / block_rows;
        for (int64_t blk = 0; blk < nblocks; ++blk) {
            const int64_t r0 = blk * block_rows;
            const int64_t r1 = std::min<int64_t>(resident, r0 + block_rows) - 1;
            fa_work_item_t it;
            std::memset(&it, 0, sizeof(it));
            it.q_start = static_cast<int32_t>(cu_q[b]);
            it.kv_start = static_cast<int32_t>(cu_kv[b]);
            it.len_q = static_cast<int32_t>(lq);
            it.len_kv = static_cast<int32_t>(lkv);
            it.block = static_cast<int32_t>(blk);
            it.seq = static_cast<int32_t>(b);
            it.drop_base = drop_base;
            int64_t lo = 0, hi = -1;
            const bool any = walked > 0 && (kind == FA_ITEMS_KEY_BLOCKS
                                                ? rows_for_keys(lq, lkv, mode, pre, nxt, r0, r1, lo, hi)
                                                : keys_for_rows(lq, lkv, mode, pre, nxt, r0, r1, lo, hi));
            if (any) {
                it.tile_begin = static_cast<int32_t>(lo / tile_rows);
                it.tile_end = static_cast<int32_t>(hi / tile_rows + 1);
            }
            out.push_back(it);
        }
        drop_base += heads * lq * lkv;
    }
    // Sequence by sequence, sequences with the longest item first, and within a sequence longest
    // item first: the long blocks do not trail at the end of the grid, and the workgroups that run
    // together (consecutive items of one head) belong to one sequence, so they walk the same tiles
    // and share an L2.  (A plain longest-first order mixes the sequences' blocks: on 4 x 16384
    // causal the dK/dV kernel then reads 5.2 GB past the L2 per launch instead of 1.8 GB.)
    std::vector<int64_t> longest(static_cast<size_t>(batch), 0);
    for (const fa_work_item_t& it : out)
        longest[it.seq] = std::max<int64_t>(longest[it.seq], it.tile_end - it.tile_begin);
    std::stable_sort(out.begin(), out.end(), [&](const fa_work_item_t& a, const fa_work_item_t& b) {
        if (a.seq != b.seq) {
            if (longest[a.seq] != longest[b.seq]) return longest[a.seq] > longest[b.seq];
            return a.seq < b.seq;
        }
        return (a.tile_end - a.tile_begin) > (b.tile_end - b.tile_begin);
    });
    return static_cast<int64_t>(out.size());
}

}  // namespace fa

extern "C" int64_t fa_varlen_worklist(const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                                      int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens,
                                      int64_t heads, int32_t kind, int32_t block_rows, int32_t tile_rows,
                                      fa_work_item_t* items, int64_t capacity) {
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
    if (kind != FA_ITEMS_KEY_BLOCKS && kind != FA_ITEMS_QUERY_BLOCKS) {
        fa::set_error("kind must be FA_ITEMS_KEY_BLOCKS or FA_ITEMS_QUERY_BLOCKS");
        return -FA_ERR_INVALID;
    }
    if (block_rows <= 0 || tile_rows <= 0 || heads < 1) {
        fa::set_error("block_rows, tile_rows and heads must be positive");
        return -FA_ERR_INVALID;
    }
    std::vector<fa_work_item_t> list;
    const int64_t n = fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, cu_seqlens_q->batch, atten_mode,
                                         pre_tokens, next_tokens, heads, kind, block_rows, tile_rows, list);
    if (items != nullptr) {
        const int64_t m = std::min(n, capacity);
        if (m > 0) std::memcpy(items, list.data(), static_cast<size_t>(m) * sizeof(fa_work_item_t));
    }
    return n;
}
