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
#include "fa_workspace.h"

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
    std::lock_guard<std::mutex> lock(fa::state_mutex());
    fa::release_all();
}

extern "C" void fa_profile_enable(int on) {
    std::lock_guard<std::mutex> lock(fa::state_mutex());
    g_profile = on != 0;
}

extern "C" int fa_profile_read(double* ms, int64_t* launches, int capacity) {
    std::lock_guard<std::mutex> lock(fa::state_mutex());
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

namespace fa {

int plan_bwd(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v, const fa_tensor_t* dy,
             const fa_tensor_t* y, const float* softmax_max, const float* softmax_sum,
             const fa_seqlens_t* cu_seqlens_q, const fa_seqlens_t* cu_seqlens_kv, int32_t atten_mode,
             int64_t pre_tokens, int64_t next_tokens, double keep_prob, const uint8_t* drop_mask,
             const fa_mask_t* atten_mask, double scale, int64_t head_num, const fa_tensor_t* dq,
             const fa_tensor_t* dk, const fa_tensor_t* dv, BwdPlan* plan) {
    clear_error();
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

    plan->q = q;
    plan->k = k;
    plan->v = v;
    plan->dy = dy;
    plan->y = y;
    plan->dq = dq;
    plan->dk = dk;
    plan->dv = dv;
    plan->softmax_max = softmax_max;
    plan->softmax_sum = softmax_sum;
    plan->cu_q = cu_seqlens_q->cu;
    plan->cu_kv = cu_seqlens_kv->cu;
    plan->batch = batch;
    plan->mode = atten_mode;
    plan->pre = atten_mode == FA_MASK_BAND ? clamp_window(pre_tokens) : 0;
    plan->nxt = atten_mode == FA_MASK_BAND ? clamp_window(next_tokens) : 0;
    plan->keep_prob = keep_prob;
    plan->drop_mask = drop_mask;
    plan->atten_mask = atten_mask;
    plan->scale = scale;
    return FA_OK;
}

std::vector<int64_t> bwd_list_key(const BwdPlan& p) {
    std::vector<int64_t> key;
    key.reserve(2 * (p.batch + 1) + 6);
    key.push_back(0);  // backward lists
    key.push_back(p.mode);
    key.push_back(p.pre);
    key.push_back(p.nxt);
    key.push_back(p.q->heads);
    key.push_back(p.q->dtype == FA_F32 ? 1 : 0);
    key.insert(key.end(), p.cu_q, p.cu_q + p.batch + 1);
    key.insert(key.end(), p.cu_kv, p.cu_kv + p.batch + 1);
    return key;
}

void build_bwd_lists(const BwdPlan& p, std::vector<fa_work_item_t>& items, int64_t& n_first) {
    const bool wide = p.q->dtype == FA_F32;
    std::vector<fa_work_item_t> qlist;
    if (wide) {
        build_worklist(p.cu_q, p.cu_kv, p.batch, p.mode, p.pre, p.nxt, p.q->heads, FA_ITEMS_KEY_BLOCKS,
                       kBlockKv32, kTileQ32, items);
        build_worklist(p.cu_q, p.cu_kv, p.batch, p.mode, p.pre, p.nxt, p.q->heads, FA_ITEMS_QUERY_BLOCKS,
                       FA32_FWD_BLOCK, FA32_FWD_BLOCK, qlist);
    } else {
        build_worklist(p.cu_q, p.cu_kv, p.batch, p.mode, p.pre, p.nxt, p.q->heads, FA_ITEMS_KEY_BLOCKS,
                       FA16_DKDV_BLOCK, FA16_DKDV_TILE_Q, items);
        build_worklist(p.cu_q, p.cu_kv, p.batch, p.mode, p.pre, p.nxt, p.q->heads, FA_ITEMS_QUERY_BLOCKS,
                       FA16_DQ_BLOCK, FA16_DQ_TILE_K, qlist);
    }
    n_first = static_cast<int64_t>(items.size());
    items.insert(items.end(), qlist.begin(), qlist.end());
}

size_t bwd_rowstat_bytes(const BwdPlan& p) {
    return static_cast<size_t>(p.q->tokens * p.q->heads) * 2 * sizeof(float);
}

}  // namespace fa

namespace fa {

hipError_t launch_bwd(const BwdPlan& p, const fa_work_item_t* items, int64_t n_kv, int64_t n_q, float* rowstat,
                      hipStream_t s, const char** what) {
    const fa_tensor_t *q = p.q, *k = p.k, *v = p.v, *dy = p.dy, *y = p.y, *dq = p.dq, *dk = p.dk, *dv = p.dv;
    const float* softmax_max = p.softmax_max;
    const float* softmax_sum = p.softmax_sum;
    const double keep_prob = p.keep_prob;
    const uint8_t* drop_mask = p.drop_mask;
    const fa_mask_t* atten_mask = p.atten_mask;
    const double scale = p.scale;
    const int64_t batch = p.batch;
    const int64_t pre = p.pre;
    const int64_t nxt = p.nxt;
    const int64_t tq = q->tokens;
    const int64_t heads = q->heads;
    const int d = static_cast<int>(q->head_dim);
    const int dv_dim = static_cast<int>(v->head_dim);
    const int32_t dtype = q->dtype;
    const bool wide = dtype == FA_F32;  // fp32 runs its own dK/dV and dQ kernels
    hipError_t e = hipSuccess;
    TensorArg tdy{dy->data, dy->stride_t, dy->stride_h};
    TensorArg ty{y->data, y->stride_t, y->stride_h};

    const float exp_scale = static_cast<float>(scale * 1.4426950408889634);
    const float inv_keep = static_cast<float>(1.0 / keep_prob);
    if (!wide) {
        Bwd16Args a;
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
        a.rowstat = rowstat;
        a.y = y->data;
        a.y_st = y->stride_t;
        a.y_sh = y->stride_h;
        a.softmax_max = softmax_max;
        a.softmax_sum = softmax_sum;
        a.items_kv = items;
        a.items_q = items + n_kv;
        a.drop_mask = keep_prob < 1.0 ? drop_mask : nullptr;
        {
            // the bit stream holds heads * Lq_b * Lkv_b bits per sequence
            int64_t bits = 0;
            for (int64_t b = 0; b < batch; ++b)
                bits += heads * (p.cu_q[b + 1] - p.cu_q[b]) *
                        (p.cu_kv[b + 1] - p.cu_kv[b]);
            a.drop_bytes = keep_prob < 1.0 ? (bits + 7) / 8 : 0;
        }
        a.tq = static_cast<int32_t>(tq);
        a.heads = static_cast<int32_t>(heads);
        a.group = static_cast<int32_t>(heads / k->heads);
        a.mode = p.mode;
        a.pre = static_cast<int32_t>(pre);
        a.nxt = static_cast<int32_t>(nxt);
        a.exp_scale = exp_scale;
        a.inv_keep = inv_keep;
        a.scale = static_cast<float>(scale);
        set_mask(a, atten_mask);
        const bool xm = atten_mask != nullptr;
        // the dQ kernel also writes the row statistics planes (no separate row pass on this path);
        // the dK/dV kernel reads them, so it runs second
        e = timed(3, s, [&] { return launch_dq16(dtype, d, dv_dim, keep_prob < 1.0, xm, a, n_q, s); });
        if (e != hipSuccess) {
            *what = "dQ kernel launch";
            return e;
        }
        e = timed(1, s, [&] { return launch_dkdv16(dtype, d, dv_dim, keep_prob < 1.0, xm, a, n_kv, s); });
        if (e != hipSuccess) {
            *what = "dK/dV kernel launch";
            return e;
        }
        return hipSuccess;
    }

    e = timed(0, s, [&] {
        return launch_preprocess(dtype, dv_dim, tdy, ty, softmax_max, softmax_sum, rowstat, tq, heads, s);
    });
    if (e != hipSuccess) {
            *what = "preprocess launch";
            return e;
        }

    MainArgs a;
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
    a.rowstat = rowstat;
    a.items = items;
    a.items_q = items + n_kv;
    a.drop_mask = keep_prob < 1.0 ? drop_mask : nullptr;
    a.tq = static_cast<int32_t>(tq);
    a.heads = static_cast<int32_t>(heads);
    a.group = static_cast<int32_t>(heads / k->heads);
    a.mode = p.mode;
    a.pre = static_cast<int32_t>(pre);
    a.nxt = static_cast<int32_t>(nxt);
    a.exp_scale = exp_scale;
    a.inv_keep = inv_keep;
    a.scale = static_cast<float>(scale);
    set_mask(a, atten_mask);
    e = timed(1, s, [&] { return launch_main(dtype, d, dv_dim, keep_prob < 1.0, a, n_kv, s); });
    if (e != hipSuccess) {
            *what = "dK/dV kernel launch";
            return e;
        }
    e = timed(3, s, [&] { return launch_dq32(d, dv_dim, keep_prob < 1.0, a, n_q, s); });
    if (e != hipSuccess) {
            *what = "dQ kernel launch";
            return e;
        }
    return hipSuccess;
}

}  // namespace fa

extern "C" int fa_varlen_bwd_masked(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                                    const fa_tensor_t* dy, const fa_tensor_t* y, const float* softmax_max,
                                    const float* softmax_sum, const fa_seqlens_t* cu_seqlens_q,
                                    const fa_seqlens_t* cu_seqlens_kv, int32_t atten_mode, int64_t pre_tokens,
                                    int64_t next_tokens, double keep_prob, const uint8_t* drop_mask,
                                    const fa_mask_t* atten_mask, double scale, int64_t head_num,
                                    const fa_tensor_t* dq, const fa_tensor_t* dk, const fa_tensor_t* dv,
                                    void* stream) {
    fa::BwdPlan plan;
    int st = fa::plan_bwd(q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, atten_mode,
                          pre_tokens, next_tokens, keep_prob, drop_mask, atten_mask, scale, head_num, dq, dk, dv,
                          &plan);
    if (st != FA_OK) return st;
    if (q->tokens == 0) return FA_OK;  // empty input: nothing to compute

    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(fa::state_mutex());
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return runtime_error("hipGetDevice", e);
    const fa::CaptureInfo ci = fa::capture_info(s);
    fa::ListRef list;
    st = fa::acquire_list(
        dev, fa::bwd_list_key(plan),
        [&](std::vector<fa_work_item_t>& items, int64_t& n_first) { fa::build_bwd_lists(plan, items, n_first); }, s,
        ci, &list);
    if (st != FA_OK) return st;
    float* rowstat = nullptr;
    st = fa::acquire_rowstat(dev, s, fa::bwd_rowstat_bytes(plan), ci, &rowstat);
    if (st != FA_OK) return st;
    const char* what = "";
    e = fa::launch_bwd(plan, list.items, list.n_first, list.n_second, rowstat, s, &what);
    // the list is noted as used even after a failed launch: an earlier kernel may have been enqueued
    st = fa::note_list_use(dev, list, s, ci);
    if (e != hipSuccess) return runtime_error(what, e);
    return st;
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

    std::lock_guard<std::mutex> lock(fa::state_mutex());
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return runtime_error("hipGetDevice", e);
    const fa::CaptureInfo ci = fa::capture_info(s);
    std::vector<int64_t> key;
    key.reserve(2 * (batch + 1) + 6);
    key.push_back(1);  // forward list
    key.push_back(atten_mode);
    key.push_back(pre);
    key.push_back(nxt);
    key.push_back(heads);
    key.push_back(wide ? 1 : 0);
    key.insert(key.end(), cu_seqlens_q->cu, cu_seqlens_q->cu + batch + 1);
    key.insert(key.end(), cu_seqlens_kv->cu, cu_seqlens_kv->cu + batch + 1);
    fa::ListRef list;
    st = fa::acquire_list(
        dev, key,
        [&](std::vector<fa_work_item_t>& items, int64_t& n_first) {
            fa::build_worklist(cu_seqlens_q->cu, cu_seqlens_kv->cu, batch, atten_mode, pre, nxt, heads,
                               FA_ITEMS_QUERY_BLOCKS, wide ? fa::FA32_FWD_BLOCK : fa::FA16_DQ_BLOCK,
                               wide ? fa::FA32_FWD_BLOCK : fa::FA16_DQ_TILE_K, items);
            n_first = static_cast<int64_t>(items.size());
        },
        s, ci, &list);
    if (st != FA_OK) return st;

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
    a.items = list.items;
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
        return wide ? fa::launch_fwd32(d, dv_dim, keep_prob < 1.0, a, list.n_first, s)
                    : fa::launch_fwd16(dtype, d, dv_dim, keep_prob < 1.0, atten_mask != nullptr, a,
                                       list.n_first, s);
    });
    st = fa::note_list_use(dev, list, s, ci);
    if (e != hipSuccess) return runtime_error("forward kernel launch", e);
    return st;
}
