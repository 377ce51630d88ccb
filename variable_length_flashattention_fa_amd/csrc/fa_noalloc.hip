// fa_varlen_bwd_noalloc: the backward for callers that cannot allocate device memory.
//
// The two things the backward keeps beyond its inputs and outputs -- the row statistics (two
// planes of -D and -beta, written by the dQ kernel and read by the dK/dV kernel; on the fp32 path
// by the row pass and both kernels) and the uploaded work lists -- live here in one fixed device
// array per GPU instead of library allocations.  Its device address is looked up once per device
// and only that address is handed to kernels and copies.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "fa_internal.h"
#include "fa_workspace.h"

namespace {

// Row statistics take the first kNoallocRowstatBytes (8 bytes per query token and head: up to
// 6 Mi token-heads, e.g. 2^20 tokens x 6 heads or 65536 tokens x 96 heads); the work lists the
// rest (40-byte items: 52428, more than any layout of up to 2^20 tokens and 2048 sequences needs).
constexpr size_t kNoallocRowstatBytes = size_t(48) << 20;
constexpr size_t kNoallocListBytes = size_t(2) << 20;
constexpr size_t kNoallocBytes = kNoallocRowstatBytes + kNoallocListBytes;

}  // namespace

// The fixed device array.  In host code its name is only a stand-in: kernels and copies get the
// address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNoallocBytes];

namespace {

struct DeviceScratch {
    unsigned char* ptr = nullptr;           // device address of `scratch` on this device
    std::vector<int64_t> key;               // layout of the work lists it holds
    int64_t n_kv = 0;
    int64_t n_q = 0;
    std::vector<fa_work_item_t> host_items;  // source of the last upload
};

std::unordered_map<int, DeviceScratch> g_scratch;

int runtime_error(const std::string& what, hipError_t e) {
    fa::set_error(what + ": " + hipGetErrorString(e));
    return FA_ERR_RUNTIME;
}

}  // namespace

extern "C" int fa_varlen_bwd_noalloc(const fa_tensor_t* q, const fa_tensor_t* k, const fa_tensor_t* v,
                                     const fa_tensor_t* dy, const fa_tensor_t* y, const float* softmax_max,
                                     const float* softmax_sum, const fa_seqlens_t* cu_seqlens_q,
                                     const fa_seqlens_t* cu_seqlens_kv, int32_t atten_mode, int64_t pre_tokens,
                                     int64_t next_tokens, double keep_prob, const uint8_t* drop_mask, double scale,
                                     int64_t head_num, const fa_tensor_t* dq, const fa_tensor_t* dk,
                                     const fa_tensor_t* dv, void* stream) {
    fa::BwdPlan plan;
    int st = fa::plan_bwd(q, k, v, dy, y, softmax_max, softmax_sum, cu_seqlens_q, cu_seqlens_kv, atten_mode,
                          pre_tokens, next_tokens, keep_prob, drop_mask, nullptr, scale, head_num, dq, dk, dv,
                          &plan);
    if (st != FA_OK) return st;
    if (q->tokens == 0) return FA_OK;
    if (fa::bwd_rowstat_bytes(plan) > kNoallocRowstatBytes) {
        fa::set_error("fa_varlen_bwd_noalloc: tokens x heads exceeds its fixed row-statistics space (" +
                      std::to_string(kNoallocRowstatBytes / 8) + " token-heads)");
        return FA_ERR_UNSUPPORTED;
    }
    const std::vector<int64_t> key = fa::bwd_list_key(plan);

    hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(fa::state_mutex());
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return runtime_error("hipGetDevice", e);
    DeviceScratch& ds = g_scratch[dev];
    if (ds.ptr == nullptr) {
        // set-up, once per device with that device current: the array's device address
        e = hipGetSymbolAddress(reinterpret_cast<void**>(&ds.ptr), HIP_SYMBOL(scratch));
        if (e != hipSuccess) {
            ds.ptr = nullptr;
            return runtime_error("fa_varlen_bwd_noalloc: scratch address", e);
        }
    }
    float* rowstat = reinterpret_cast<float*>(ds.ptr);
    fa_work_item_t* dev_items = reinterpret_cast<fa_work_item_t*>(ds.ptr + kNoallocRowstatBytes);
    if (ds.key != key) {
        if (fa::capture_info(s).capturing) {
            fa::set_error("fa_varlen_bwd_noalloc: the stream is being captured and the sequence layout changed: "
                          "make one uncaptured call with this layout first");
            return FA_ERR_UNSUPPORTED;
        }
        std::vector<fa_work_item_t> items;
        int64_t n_first = 0;
        fa::build_bwd_lists(plan, items, n_first);
        if (items.size() * sizeof(fa_work_item_t) > kNoallocListBytes) {
            fa::set_error("fa_varlen_bwd_noalloc: the layout needs " + std::to_string(items.size()) +
                          " work items, more than its fixed space holds (" +
                          std::to_string(kNoallocListBytes / sizeof(fa_work_item_t)) + ")");
            return FA_ERR_UNSUPPORTED;
        }
        ds.key.clear();  // invalid until the copy below has landed
        ds.host_items = std::move(items);
        if (!ds.host_items.empty()) {
            e = hipMemcpyAsync(dev_items, ds.host_items.data(), ds.host_items.size() * sizeof(fa_work_item_t),
                               hipMemcpyHostToDevice, s);
            // the source must outlive the copy, and the next layout change rewrites it: wait here
            if (e == hipSuccess) e = hipStreamSynchronize(s);
            if (e != hipSuccess) return runtime_error("fa_varlen_bwd_noalloc: work list upload", e);
        }
        ds.key = key;
        ds.n_kv = n_first;
        ds.n_q = static_cast<int64_t>(ds.host_items.size()) - n_first;
    }
    const char* what = "";
    e = fa::launch_bwd(plan, dev_items, ds.n_kv, ds.n_q, rowstat, s, &what);
    if (e != hipSuccess) return runtime_error(what, e);
    return FA_OK;
}
