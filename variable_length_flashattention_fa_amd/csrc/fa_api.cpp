// C ABI entry points: validation, workspace, work list and launch sequence.
//
// Validation follows the constraints and return codes of the
// "FlashAttention梯度V2" page (约束说明 and 返回值 sections): null required
// pointers -> FA_ERR_NULLPTR; dtype / shape / range violations ->
// FA_ERR_INVALID.  Everything is checked before any device work is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "fa_internal.h"
#include "fa_kernels.h"

namespace fa {
const char* last_error_cstr();
}

namespace {

using fa::set_error;

constexpr int64_t kMaxTokens = int64_t(1) << 20;  // T in [1, 1M]
constexpr int64_t kMaxHeads = 256;                 // N in [1, 256]
constexpr int64_t kMaxHeadDim = 768;               // D in [1, 768]

int check_tensor(const fa_tensor_t* t, const char* name) {
    if (t == nullptr || (t->data == nullptr && t->tokens != 0)) {
        set_error(std::string(name) + " is null");
        return FA_ERR_NULLPTR;
    }
    if (t->dtype != FA_F32 && t->dtype != FA_F16 && t->dtype != FA_BF16) {
        set_error(std::string(name) + ": dtype must be FA_F32, FA_F16 or FA_BF16");
        return FA_ERR_INVALID;
    }
    if (t->tokens < 0 || t->tokens > kMaxTokens) {
        set_error(std::string(name) + ": tokens must be in [0, 2^20]");
        return FA_ERR_INVALID;
    }
    if (t->heads < 1 || t->heads > kMaxHeads) {
        set_error(std::string(name) + ": heads must be in [1, 256]");
        return FA_ERR_INVALID;
    }
    if (t->head_dim < 1 || t->head_dim > kMaxHeadDim) {
        set_error(std::string(name) + ": head_dim must be in [1, 768]");
        return FA_ERR_INVALID;
    }
    if (t->stride_t < 0 || t->stride_h < 0) {
        set_error(std::string(name) + ": strides must be non-negative");
        return FA_ERR_INVALID;
    }
    return FA_OK;
}

size_t elem_size(int32_t dtype) { return dtype == FA_F32 ? 4 : 2; }

// 16-byte vector access of rows needs aligned bases and strides.
bool aligned16(const fa_tensor_t* t) {
    const size_t es = elem_size(t->dtype);
    return (reinterpret_cast<uintptr_t>(t->data) % 16 == 0) && ((t->stride_t * es) % 16 == 0) &&
           ((t->stride_h * es) % 16 == 0);
}

struct Workspace {
    float* rowstat = nullptr;  // planes of -D and beta
    size_t rowstat_bytes = 0;
    fa_work_item_t* items = nullptr;
    size_t items_cap = 0;
    // cached work lists: their key and item counts (key-block items, then query-block items)
    std::vector<int64_t> key;
    int64_t n_items = 0;
    int64_t n_q_items = 0;
    // the forward's query-block list, cached the same way
    fa_work_item_t* fwd_items = nullptr;
    size_t fwd_items_cap = 0;
    std::vector<int64_t> fwd_key;
    int64_t n_fwd_items = 0;
};

std::mutex g_mutex;
std::unordered_map<int, Workspace> g_ws;

// ---- optional per-kernel event timing ----
constexpr int kKernels = 5;  // 0 row pass (fp32 path), 1 dK/dV, 2 (unused), 3 dQ, 4 forward
struct EventPair {
    int kernel;
    hipEvent_t start;
    hipEvent_t stop;
};
bool g_profile = false;
std::vector<EventPair> g_events;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Records `start` before and `stop` after the launch made by fn (when profiling).
template <typename F>
hipError_t timed(int kernel, hipStream_t s, F&& fn) {
    if (!g_profile) return fn();
    hipEvent_t a = take_event();
    hipEvent_t b = take_event();
    if (a == nullptr || b == nullptr) return fn();
    (void)hipEventRecord(a, s);
    hipError_t e = fn();
    (void)hipEventRecord(b, s);
    g_events.push_back({kernel, a, b});
    return e;
}

int runtime_error(const char* what, hipError_t e) {
    set_error(std::string(what) + ": " + hipGetErrorString(e));
    return FA_ERR_RUNTIME;
}

int grow(void** ptr, size_t* cap, size_t need, const char* what) {
    if (need <= *cap && *ptr != nullptr) return FA_OK;
    if (*ptr != nullptr) {
        hipError_t e = hipFree(*ptr);  // hipFree synchronises with outstanding work
        *ptr = nullptr;
        *cap = 0;
        if (e != hipSuccess) return runtime_error(what, e);
    }
    size_t bytes = need < 256 ? 256 : need;
    hipError_t e = hipMalloc(ptr, bytes);
    if (e != hipSuccess) return runtime_error(what, e);
    *cap = bytes;
    return FA_OK;
}

// Checks an explicit mask view against the sequence layout (see fa_mask_t in fa_varlen.h).
int check_mask(const fa_mask_t* m, const fa_seqlens_t* cq, const fa_seqlens_t* ck) {
    if (m->stride_b < 0 || m->stride_n < 0 || m->stride_q < 0 || m->rows < 0 || m->cols < 0) {
        set_error("atten_mask: strides and sizes must be non-negative");
        return FA_ERR_INVALID;
    }
    if (m->stride_q < m->cols) {
        set_error("atten_mask: stride_q must be at least cols");
        return FA_ERR_INVALID;
    }
    for (int64_t b = 0; b < cq->batch; ++b) {
        const int64_t lq = cq->cu[b + 1] - cq->cu[b];
        const int64_t lk = ck->cu[b + 1] - ck->cu[b];
        if (lq > m->rows || lk > m->cols) {
            set_error("atten_mask: rows / cols must cover every sequence (Sq >= Lq_b, Skv >= Lkv_b)");
            return FA_ERR_INVALID;
        }
        // the kernels address one (sequence, head) block with 32-bit offsets
        if (lq > 0 && lk > 0 && (lq - 1) * m->stride_q + lk >= (int64_t(1) << 31)) {
            set_error("atten_mask: one (sequence, head) block must span less than 2^31 bytes");
            return FA_ERR_UNSUPPORTED;
        }
    }
    return FA_OK;
}

}  // namespace

extern "C" const char* fa_last_error(void) { return fa::last_error_cstr(); }

extern "C" void fa_release(void) {
    std::lock_guard<std::mutex> lock(g_mutex);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_ws) {
        (void)hipSetDevice(kv.first);
        (void)hipDeviceSynchronize();
        if (kv.second.rowstat) (void)hipFree(kv.second.rowstat);
        if (kv.second.items) (void)hipFree(kv.second.items);
        if (kv.second.fwd_items) (void)hipFree(kv.second.fwd_items);
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
}

extern "C" void fa_profile_enable(int on) {
    std::lock_guard<std::mutex> lock(g_mutex);
    g_profile = on != 0;
}

extern "C" int fa_profile_read(double* ms, int64_t* launches, int capacity) {
    std::lock_guard<std::mutex> lock(g_mutex);
    double sum[kKernels] = {0, 0, 0, 0, 0};
    int64_t cnt[kKernels] = {0, 0, 0, 0, 0};
    int status = kKernels;
    for (auto& ev : g_events) {
        float t = 0.f;
        if (hipEventSynchronize(ev.stop) != hipSuccess || hipEventElapsedTime(&t, ev.start, ev.stop) != hipSuccess) {
            set_error("fa_profile_read: event query failed");
            status = -FA_ERR_RUNTIME;
        } else {
            sum[ev.kernel] += t;
            cnt[ev.kernel] += 1;
        }
        g_event_pool.push_back(ev.start);
        g_event_pool.push_back(ev.stop);
    }
    g_events.clear();
    for (int i = 0; i < kKernels && i < capacity; ++i) {
        if (ms) ms[i] = sum[i];
        if (launches) launches[i] = cnt[i];
    }
    return status;
}

extern "C" int fa_varlen_bwd(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                             const fa_tensor_t* dy, const fa_tensor_t* y, const float* softmax_max,
                             const float* softmax_sum, const fa_seqlens_t* cu_seqlens_q,
                             const fa_seqlens_t* cu_seqlens_kv, int32_t atten_mode, int64_t pre_tokens,
                             int64_t next_tokens, double keep_prob, const uint8_t* drop_mask, double scale,
                             int64_t head_num, const fa_tensor_t* dq, const fa_tensor_t* dk,
                             const fa_tensor_t* dv, void* stream) {
    return fa_varlen_bwd_masked(q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, atten_mode,
                                pre_tokens, next_tokens, keep_prob, drop_mask, nullptr, scale, head_num, dq, dk,
                                dv, stream);
}

extern "C" int fa_varlen_bwd_masked(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                                    const fa_tensor_t* dy, const fa_tensor_t* y, const float* softmax_max,
                                    const float* softmax_sum, const fa_seqlens_t* cu_seqlens_q,
                                    const fa_seqlens_t* cu_seqlens_kv, int32_t atten_mode, int64_t pre_tokens,
                                    int64_t next_tokens, double keep_prob, const uint8_t* drop_mask,
                                    const fa_mask_t* atten_mask, double scale, int64_t head_num,
                                    const fa_tensor_t* dq, const fa_tensor_t* dk, const fa_tensor_t* dv,
                                    void* stream) {
    fa::clear_error();
    // ---- null pointers (page: ACLNN_ERR_PARAM_NULLPTR) ----
    const fa_tensor_t* all[8] = {q, k, v, dy, y, dq, dk, dv};
    const char* names[8] = {"q", "k", "v", "dy", "y", "dq", "dk", "dv"};
    for (int i = 0; i < 8; ++i) {
        // an empty tensor (zero tokens) may carry a null data pointer
        if (all[i] == nullptr || (all[i]->data == nullptr && all[i]->tokens != 0)) {
            set_error(std::string(names[i]) + " is null");
            return FA_ERR_NULLPTR;
        }
    }
    if (softmax_max == nullptr || softmax_sum == nullptr) {
        set_error("softmax_max / softmax_sum is null");
        return FA_ERR_NULLPTR;
    }
    if (cu_seqlens_q == nullptr || cu_seqlens_q->cu == nullptr || cu_seqlens_kv == nullptr ||
        cu_seqlens_kv->cu == nullptr) {
        set_error("cu_seqlens_q / cu_seqlens_kv is null");
        return FA_ERR_NULLPTR;
    }
    if (!(keep_prob > 0.0 && keep_prob <= 1.0)) {
        set_error("keep_prob must be in (0, 1]");
        return FA_ERR_INVALID;
    }
    if (keep_prob < 1.0 && drop_mask == nullptr) {
        set_error("drop_mask is null while keep_prob < 1");
        return FA_ERR_NULLPTR;
    }
    if (atten_mask != nullptr && atten_mask->data == nullptr && q->tokens != 0) {
        set_error("atten_mask->data is null");
        return FA_ERR_NULLPTR;
    }
    // ---- values (page: ACLNN_ERR_PARAM_INVALID) ----
    for (int i = 0; i < 8; ++i) {
        int st = check_tensor(all[i], names[i]);
        if (st != FA_OK) return st;
    }
    for (int i = 1; i < 8; ++i) {
        if (all[i]->dtype != q->dtype) {
            set_error(std::string(names[i]) + ": dtype differs from q (all tensors share one dtype)");
            return FA_ERR_INVALID;
        }
    }
    if (head_num != q->heads) {
        set_error("head_num must equal the N axis of q");
        return FA_ERR_INVALID;
    }
    if (k->heads != v->heads || k->tokens != v->tokens) {
        set_error("k and v must have equal shapes apart from D");
        return FA_ERR_INVALID;
    }
    if (q->heads % k->heads != 0) {
        set_error("q heads must be a multiple of k/v heads");
        return FA_ERR_INVALID;
    }
    if (q->head_dim != k->head_dim || k->head_dim < v->head_dim) {
        set_error("head dims must satisfy qD == kD >= vD");
        return FA_ERR_INVALID;
    }
    if (dy->tokens != q->tokens || dy->heads != q->heads || dy->head_dim != v->head_dim ||
        y->tokens != q->tokens || y->heads != q->heads || y->head_dim != v->head_dim) {
        set_error("dy and y must have q's tokens and heads and v's head_dim");
        return FA_ERR_INVALID;
    }
    if (dq->tokens != q->tokens || dq->heads != q->heads || dq->head_dim != q->head_dim ||
        dk->tokens != k->tokens || dk->heads != k->heads || dk->head_dim != k->head_dim ||
        dv->tokens != v->tokens || dv->heads != v->heads || dv->head_dim != v->head_dim) {
        set_error("dq/dk/dv must have the shapes of q/k/v");
        return FA_ERR_INVALID;
    }
    if (atten_mode < FA_MASK_NONE || atten_mode > FA_MASK_BAND) {
        set_error("atten_mode must be 0 (none), 1 (causal) or 2 (band)");
        return FA_ERR_INVALID;
    }
    if (!std::isfinite(scale)) {
        set_error("scale must be finite");
        return FA_ERR_INVALID;
    }
    int st = fa::check_seqlens(cu_seqlens_q, "cu_seqlens_q");
    if (st != FA_OK) return st;
    st = fa::check_seqlens(cu_seqlens_kv, "cu_seqlens_kv");
    if (st != FA_OK) return st;
    if (cu_seqlens_q->batch != cu_seqlens_kv->batch) {
        set_error("cu_seqlens_q and cu_seqlens_kv must have equal batch counts");
        return FA_ERR_INVALID;
    }
    const int64_t batch = cu_seqlens_q->batch;
    if (cu_seqlens_q->cu[batch] != q->tokens || cu_seqlens_kv->cu[batch] != k->tokens) {
        set_error("cu_seqlens must end at the token counts of q and k");
        return FA_ERR_INVALID;
    }
    if (atten_mask != nullptr) {
        st = check_mask(atten_mask, cu_seqlens_q, cu_seqlens_kv);
        if (st != FA_OK) return st;
    }
    // ---- allowed by the page, not built ----
    if (!fa::head_dims_supported(q->head_dim, v->head_dim)) {
        set_error("head dims (q/k, v) must be (128, 128), (128, 64) or (64, 64)");
        return FA_ERR_UNSUPPORTED;
    }
    for (int i = 0; i < 8; ++i) {
        if (!aligned16(all[i])) {
            set_error(std::string(names[i]) + ": data and strides must be 16-byte aligned");
            return FA_ERR_UNSUPPORTED;
        }
    }

    const int64_t tq = q->tokens;
    const int64_t heads = q->heads;
    const int d = static_cast<int>(q->head_dim);
    const int dv_dim = static_cast<int>(v->head_dim);
    if (tq == 0) return FA_OK;  // empty input: nothing to compute

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t dtype = q->dtype;
    const bool wide = dtype == FA_F32;  // fp32 runs its own dK/dV and dQ kernels
    const int64_t pre = atten_mode == FA_MASK_BAND ? fa::clamp_window(pre_tokens) : 0;
    const int64_t nxt = atten_mode == FA_MASK_BAND ? fa::clamp_window(next_tokens) : 0;

    std::lock_guard<std::mutex> lock(g_mutex);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return runtime_error("hipGetDevice", e);
    Workspace& ws = g_ws[dev];

    // work lists, rebuilt only when the sequence layout, mask or path changes:
    // key-block items first, then (16-bit path) query-block items
    std::vector<int64_t> key;
    key.reserve(2 * (batch + 1) + 5);
    key.push_back(atten_mode);
    key.push_back(pre);
    key.push_back(nxt);
    key.push_back(heads);
    key.push_back(wide ? 1 : 0);
    key.insert(key.end(), cu_seqlens_q->cu, cu_seqlens_q->cu + batch + 1);
    key.insert(key.end(), cu_seqlens_kv->cu, cu_seqlens_kv->cu + batch + 1);
    if (key != ws.key) {
        std::vector<fa_work_item_t> list, qlist;
        if (wide) {
            fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, batch, atten_mode, pre, nxt, heads,
                               FA_ITEMS_KEY_BLOCKS, fa::kBlockKv32, fa::kTileQ32, list);
            fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, batch, atten_mode, pre, nxt, heads,
                               FA_ITEMS_QUERY_BLOCKS, fa::FA32_FWD_BLOCK, fa::FA32_FWD_BLOCK, qlist);
        } else {
            fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, batch, atten_mode, pre, nxt, heads,
                               FA_ITEMS_KEY_BLOCKS, fa::FA16_DKDV_BLOCK, fa::FA16_DKDV_TILE_Q, list);
            fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, batch, atten_mode, pre, nxt, heads,
                               FA_ITEMS_QUERY_BLOCKS, fa::FA16_DQ_BLOCK, fa::FA16_DQ_TILE_K, qlist);
        }
        const int64_t n_kv = static_cast<int64_t>(list.size());
        const int64_t n_q = static_cast<int64_t>(qlist.size());
        list.insert(list.end(), qlist.begin(), qlist.end());
        const int64_t n = n_kv + n_q;
        size_t cap_bytes = ws.items_cap * sizeof(fa_work_item_t);
        void* ptr = ws.items;
        int g = grow(&ptr, &cap_bytes, static_cast<size_t>(n) * sizeof(fa_work_item_t), "work list");
        ws.items = static_cast<fa_work_item_t*>(ptr);
        ws.items_cap = cap_bytes / sizeof(fa_work_item_t);
        if (g != FA_OK) {
            ws.key.clear();
            return g;
        }
        if (n > 0) {
            // The previous list may still be read by kernels queued on this
            // stream; wait for them, then copy synchronously (lists are small
            // and reused by later calls with the same layout).
            e = hipStreamSynchronize(s);
            if (e != hipSuccess) {
                ws.key.clear();
                return runtime_error("stream synchronize", e);
            }
            e = hipMemcpy(ws.items, list.data(), static_cast<size_t>(n) * sizeof(fa_work_item_t),
                          hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                ws.key.clear();
                return runtime_error("work list upload", e);
            }
        }
        ws.key = key;
        ws.n_items = n_kv;
        ws.n_q_items = n_q;
    }

    {
        void* ptr = ws.rowstat;
        int g = grow(&ptr, &ws.rowstat_bytes, static_cast<size_t>(tq * heads) * 2 * sizeof(float), "row statistics");
        ws.rowstat = static_cast<float*>(ptr);
        if (g != FA_OK) return g;
    }

    fa::TensorArg tdy{dy->data, dy->stride_t, dy->stride_h};
    fa::TensorArg ty{y->data, y->stride_t, y->stride_h};

    const float exp_scale = static_cast<float>(scale * 1.4426950408889634);
    const float inv_keep = static_cast<float>(1.0 / keep_prob);
    if (!wide) {
        fa::Bwd16Args a;
        a.q = q->data;
        a.k = k->data;
        a.v = v->data;
        a.dy = dy->data;
        a.q_st = q->stride_t;
        a.q_sh = q->stride_h;
        a.k_st = k->stride_t;
        a.k_sh = k->stride_h;
        a.v_st = v->stride_t;
        a.v_sh = v->stride_h;
        a.dy_st = dy->stride_t;
        a.dy_sh = dy->stride_h;
        a.dq = dq->data;
        a.dk = dk->data;
        a.dv = dv->data;
        a.dq_st = dq->stride_t;
        a.dq_sh = dq->stride_h;
        a.dk_st = dk->stride_t;
        a.dk_sh = dk->stride_h;
        a.dv_st = dv->stride_t;
        a.dv_sh = dv->stride_h;
        a.rowstat = ws.rowstat;
        a.y = y->data;
        a.y_st = y->stride_t;
        a.y_sh = y->stride_h;
        a.softmax_max = softmax_max;
        a.softmax_sum = softmax_sum;
        a.items_kv = ws.items;
        a.items_q = ws.items + ws.n_items;
        a.drop_mask = keep_prob < 1.0 ? drop_mask : nullptr;
        {
            // the bit stream holds heads * Lq_b * Lkv_b bits per sequence
            int64_t bits = 0;
            for (int64_t b = 0; b < batch; ++b)
                bits += heads * (cu_seqlens_q->cu[b + 1] - cu_seqlens_q->cu[b]) *
                        (cu_seqlens_kv->cu[b + 1] - cu_seqlens_kv->cu[b]);
            a.drop_bytes = keep_prob < 1.0 ? (bits + 7) / 8 : 0;
        }
        a.tq = static_cast<int32_t>(tq);
        a.heads = static_cast<int32_t>(heads);
        a.group = static_cast<int32_t>(heads / k->heads);
        a.mode = atten_mode;
        a.pre = static_cast<int32_t>(pre);
        a.nxt = static_cast<int32_t>(nxt);
        a.exp_scale = exp_scale;
        a.inv_keep = inv_keep;
        a.scale = static_cast<float>(scale);
        fa::set_mask(a, atten_mask);
        const bool xm = atten_mask != nullptr;
        // the dQ kernel also writes the row statistics planes (no separate row pass on this path);
        // the dK/dV kernel reads them, so it runs second
        e = timed(3, s, [&] { return fa::launch_dq16(dtype, d, dv_dim, keep_prob < 1.0, xm, a, ws.n_q_items, s); });
        if (e != hipSuccess) return runtime_error("dQ kernel launch", e);
        e = timed(1, s, [&] { return fa::launch_dkdv16(dtype, d, dv_dim, keep_prob < 1.0, xm, a, ws.n_items, s); });
        if (e != hipSuccess) return runtime_error("dK/dV kernel launch", e);
        return FA_OK;
    }

    e = timed(0, s, [&] {
        return fa::launch_preprocess(dtype, dv_dim, tdy, ty, softmax_max, softmax_sum, ws.rowstat, tq, heads, s);
    });
    if (e != hipSuccess) return runtime_error("preprocess launch", e);

    fa::MainArgs a;
    a.q = {q->data, q->stride_t, q->stride_h};
    a.k = {k->data, k->stride_t, k->stride_h};
    a.v = {v->data, v->stride_t, v->stride_h};
    a.dy = tdy;
    a.dq = dq->data;
    a.dq_st = dq->stride_t;
    a.dq_sh = dq->stride_h;
    a.dk = dk->data;
    a.dk_st = dk->stride_t;
    a.dk_sh = dk->stride_h;
    a.dv = dv->data;
    a.dv_st = dv->stride_t;
    a.dv_sh = dv->stride_h;
    a.rowstat = ws.rowstat;
    a.items = ws.items;
    a.items_q = ws.items + ws.n_items;
    a.drop_mask = keep_prob < 1.0 ? drop_mask : nullptr;
    a.tq = static_cast<int32_t>(tq);
    a.heads = static_cast<int32_t>(heads);
    a.group = static_cast<int32_t>(heads / k->heads);
    a.mode = atten_mode;
    a.pre = static_cast<int32_t>(pre);
    a.nxt = static_cast<int32_t>(nxt);
    a.exp_scale = exp_scale;
    a.inv_keep = inv_keep;
    a.scale = static_cast<float>(scale);
    fa::set_mask(a, atten_mask);
    e = timed(1, s, [&] { return fa::launch_main(dtype, d, dv_dim, keep_prob < 1.0, a, ws.n_items, s); });
    if (e != hipSuccess) return runtime_error("dK/dV kernel launch", e);
    e = timed(3, s, [&] { return fa::launch_dq32(d, dv_dim, keep_prob < 1.0, a, ws.n_q_items, s); });
    if (e != hipSuccess) return runtime_error("dQ kernel launch", e);
    return FA_OK;
}

// Forward: validation as in the backward (same page constraints, same codes), then one kernel
// over query-block items.
extern "C" int fa_varlen_fwd(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                             const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                             int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens, double keep_prob,
                             const uint8_t* drop_mask, double scale, int64_t head_num, const fa_tensor_t* y,
                             float* softmax_max, float* softmax_sum, void* stream) {
    return fa_varlen_fwd_masked(q, k, v, cu_seqlens_q, cu_seqlens_kv, atten_mode, pre_tokens, next_tokens,
                                keep_prob, drop_mask, nullptr, scale, head_num, y, softmax_max, softmax_sum, stream);
}

extern "C" int fa_varlen_fwd_masked(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                                    const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv,
                                    int32_t atten_mode, int64_t pre_tokens, int64_t next_tokens, double keep_prob,
                                    const uint8_t* drop_mask, const fa_mask_t* atten_mask, double scale,
                                    int64_t head_num, const fa_tensor_t* y, float* softmax_max,
                                    float* softmax_sum, void* stream) {
    fa::clear_error();
    const fa_tensor_t* all[4] = {q, k, v, y};
    const char* names[4] = {"q", "k", "v", "y"};
    for (int i = 0; i < 4; ++i) {
        if (all[i] == nullptr || (all[i]->data == nullptr && all[i]->tokens != 0)) {
            set_error(std::string(names[i]) + " is null");
            return FA_ERR_NULLPTR;
        }
    }
    if ((softmax_max == nullptr || softmax_sum == nullptr) && q->tokens != 0) {
        set_error("softmax_max / softmax_sum is null");
        return FA_ERR_NULLPTR;
    }
    if (cu_seqlens_q == nullptr || cu_seqlens_q->cu == nullptr || cu_seqlens_kv == nullptr ||
        cu_seqlens_kv->cu == nullptr) {
        set_error("cu_seqlens_q / cu_seqlens_kv is null");
        return FA_ERR_NULLPTR;
    }
    if (!(keep_prob > 0.0 && keep_prob <= 1.0)) {
        set_error("keep_prob must be in (0, 1]");
        return FA_ERR_INVALID;
    }
    if (keep_prob < 1.0 && drop_mask == nullptr) {
        set_error("drop_mask is null while keep_prob < 1");
        return FA_ERR_NULLPTR;
    }
    if (atten_mask != nullptr && atten_mask->data == nullptr && q->tokens != 0) {
        set_error("atten_mask->data is null");
        return FA_ERR_NULLPTR;
    }
    for (int i = 0; i < 4; ++i) {
        int st = check_tensor(all[i], names[i]);
        if (st != FA_OK) return st;
    }
    for (int i = 1; i < 4; ++i) {
        if (all[i]->dtype != q->dtype) {
            set_error(std::string(names[i]) + ": dtype differs from q (all tensors share one dtype)");
            return FA_ERR_INVALID;
        }
    }
    if (head_num != q->heads) {
        set_error("head_num must equal the N axis of q");
        return FA_ERR_INVALID;
    }
    if (k->heads != v->heads || k->tokens != v->tokens) {
        set_error("k and v must have equal shapes apart from D");
        return FA_ERR_INVALID;
    }
    if (q->heads % k->heads != 0) {
        set_error("q heads must be a multiple of k/v heads");
        return FA_ERR_INVALID;
    }
    if (q->head_dim != k->head_dim || k->head_dim < v->head_dim) {
        set_error("head dims must satisfy qD == kD >= vD");
        return FA_ERR_INVALID;
    }
    if (y->tokens != q->tokens || y->heads != q->heads || y->head_dim != v->head_dim) {
        set_error("y must have q's tokens and heads and v's head_dim");
        return FA_ERR_INVALID;
    }
    if (atten_mode < FA_MASK_NONE || atten_mode > FA_MASK_BAND) {
        set_error("atten_mode must be 0 (none), 1 (causal) or 2 (band)");
        return FA_ERR_INVALID;
    }
    if (!std::isfinite(scale)) {
        set_error("scale must be finite");
        return FA_ERR_INVALID;
    }
    int st = fa::check_seqlens(cu_seqlens_q, "cu_seqlens_q");
    if (st != FA_OK) return st;
    st = fa::check_seqlens(cu_seqlens_kv, "cu_seqlens_kv");
    if (st != FA_OK) return st;
    if (cu_seqlens_q->batch != cu_seqlens_kv->batch) {
        set_error("cu_seqlens_q and cu_seqlens_kv must have equal batch counts");
        return FA_ERR_INVALID;
    }
    const int64_t batch = cu_seqlens_q->batch;
    if (cu_seqlens_q->cu[batch] != q->tokens || cu_seqlens_kv->cu[batch] != k->tokens) {
        set_error("cu_seqlens must end at the token counts of q and k");
        return FA_ERR_INVALID;
    }
    if (atten_mask != nullptr) {
        st = check_mask(atten_mask, cu_seqlens_q, cu_seqlens_kv);
        if (st != FA_OK) return st;
    }
    if (!fa::head_dims_supported(q->head_dim, v->head_dim)) {
        set_error("head dims (q/k, v) must be (128, 128), (128, 64) or (64, 64)");
        return FA_ERR_UNSUPPORTED;
    }
    for (int i = 0; i < 4; ++i) {
        if (!aligned16(all[i])) {
            set_error(std::string(names[i]) + ": data and strides must be 16-byte aligned");
            return FA_ERR_UNSUPPORTED;
        }
    }
    if (reinterpret_cast<uintptr_t>(softmax_max) % 16 != 0 || reinterpret_cast<uintptr_t>(softmax_sum) % 16 != 0) {
        set_error("softmax_max / softmax_sum must be 16-byte aligned");
        return FA_ERR_UNSUPPORTED;
    }
    int64_t drop_bits = 0;
    for (int64_t b = 0; b < batch; ++b) {
        const int64_t lq = cu_seqlens_q->cu[b + 1] - cu_seqlens_q->cu[b];
        const int64_t lk = cu_seqlens_kv->cu[b + 1] - cu_seqlens_kv->cu[b];
        // the 16-bit kernel addresses one (sequence, head) region of the bit stream with 32-bit
        // byte offsets
        if (keep_prob < 1.0 && lq * lk >= (int64_t(1) << 34)) {
            set_error("dropout: a sequence's Lq * Lkv must stay below 2^34");
            return FA_ERR_UNSUPPORTED;
        }
        drop_bits += q->heads * lq * lk;
    }

    const int64_t tq = q->tokens;
    const int64_t heads = q->heads;
    const int d = static_cast<int>(q->head_dim);
    const int dv_dim = static_cast<int>(v->head_dim);
    if (tq == 0) return FA_OK;

    hipStream_t s = static_cast<hipStream_t>(stream);
    const int32_t dtype = q->dtype;
    const bool wide = dtype == FA_F32;
    const int64_t pre = atten_mode == FA_MASK_BAND ? fa::clamp_window(pre_tokens) : 0;
    const int64_t nxt = atten_mode == FA_MASK_BAND ? fa::clamp_window(next_tokens) : 0;

    std::lock_guard<std::mutex> lock(g_mutex);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return runtime_error("hipGetDevice", e);
    Workspace& ws = g_ws[dev];

    std::vector<int64_t> key;
    key.reserve(2 * (batch + 1) + 5);
    key.push_back(atten_mode);
    key.push_back(pre);
    key.push_back(nxt);
    key.push_back(heads);
    key.push_back(wide ? 1 : 0);
    key.insert(key.end(), cu_seqlens_q->cu, cu_seqlens_q->cu + batch + 1);
    key.insert(key.end(), cu_seqlens_kv->cu, cu_seqlens_kv->cu + batch + 1);
    if (key != ws.fwd_key) {
        std::vector<fa_work_item_t> list;
        fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, batch, atten_mode, pre, nxt, heads,
                           FA_ITEMS_QUERY_BLOCKS, wide ? fa::FA32_FWD_BLOCK : fa::FA16_DQ_BLOCK,
                           wide ? fa::FA32_FWD_BLOCK : fa::FA16_DQ_TILE_K, list);
        const int64_t n = static_cast<int64_t>(list.size());
        size_t cap_bytes = ws.fwd_items_cap * sizeof(fa_work_item_t);
        void* ptr = ws.fwd_items;
        int g = grow(&ptr, &cap_bytes, static_cast<size_t>(n) * sizeof(fa_work_item_t), "forward work list");
        ws.fwd_items = static_cast<fa_work_item_t*>(ptr);
        ws.fwd_items_cap = cap_bytes / sizeof(fa_work_item_t);
        if (g != FA_OK) {
            ws.fwd_key.clear();
            return g;
        }
        if (n > 0) {
            e = hipStreamSynchronize(s);
            if (e != hipSuccess) {
                ws.fwd_key.clear();
                return runtime_error("stream synchronize", e);
            }
            e = hipMemcpy(ws.fwd_items, list.data(), static_cast<size_t>(n) * sizeof(fa_work_item_t),
                          hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                ws.fwd_key.clear();
                return runtime_error("forward work list upload", e);
            }
        }
        ws.fwd_key = key;
        ws.n_fwd_items = n;
    }

    fa::FwdArgs a;
    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.q_st = q->stride_t;
    a.q_sh = q->stride_h;
    a.k_st = k->stride_t;
    a.k_sh = k->stride_h;
    a.v_st = v->stride_t;
    a.v_sh = v->stride_h;
    a.y = y->data;
    a.y_st = y->stride_t;
    a.y_sh = y->stride_h;
    a.smax = softmax_max;
    a.ssum = softmax_sum;
    a.items = ws.fwd_items;
    a.drop_mask = keep_prob < 1.0 ? drop_mask : nullptr;
    a.drop_bytes = keep_prob < 1.0 ? (drop_bits + 7) / 8 : 0;
    a.tq = static_cast<int32_t>(tq);
    a.heads = static_cast<int32_t>(heads);
    a.group = static_cast<int32_t>(heads / k->heads);
    a.mode = atten_mode;
    a.pre = static_cast<int32_t>(pre);
    a.nxt = static_cast<int32_t>(nxt);
    a.scale = static_cast<float>(scale);
    a.exp_scale = static_cast<float>(scale * 1.4426950408889634);
    a.inv_keep = static_cast<float>(1.0 / keep_prob);
    fa::set_mask(a, atten_mask);
    e = timed(4, s, [&] {
        return wide ? fa::launch_fwd32(d, dv_dim, keep_prob < 1.0, a, ws.n_fwd_items, s)
                    : fa::launch_fwd16(dtype, d, dv_dim, keep_prob < 1.0, atten_mask != nullptr, a,
                                       ws.n_fwd_items, s);
    });
    if (e != hipSuccess) return runtime_error("forward kernel launch", e);
    return FA_OK;
}
