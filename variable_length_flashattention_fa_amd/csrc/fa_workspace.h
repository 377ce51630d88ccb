// Library-owned device memory of the entry points (see fa_workspace.cpp).  Every function here
// must be called with state_mutex() held.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <functional>
#include <mutex>
#include <vector>

#include "fa_internal.h"
#include "fa_varlen.h"

namespace fa {

std::mutex& state_mutex();

struct CaptureInfo {
    bool capturing = false;
    unsigned long long id = 0;
};

// Whether `s` is being captured into a graph (and the capture's id).
CaptureInfo capture_info(hipStream_t s);

// A device work list: n_first items, then n_second items (the backward's key-block list, then its
// query-block list; the forward has only the first).
struct ListRef {
    const fa_work_item_t* items = nullptr;
    int64_t n_first = 0;
    int64_t n_second = 0;
    void* handle = nullptr;
};

// Fills the items of a list and the size of its first part.
using ListBuilder = std::function<void(std::vector<fa_work_item_t>&, int64_t&)>;

// The device list of `key` on device `dev`, built with `build` and uploaded on stream `s` when the
// key is new (FA_ERR_UNSUPPORTED if the key is new while `s` is being captured).
int acquire_list(int dev, const std::vector<int64_t>& key, const ListBuilder& build, hipStream_t s,
                 const CaptureInfo& ci, ListRef* out);

// Records that kernels reading `ref` were enqueued on `s` (call after the launches).
int note_list_use(int dev, const ListRef& ref, hipStream_t s, const CaptureInfo& ci);

// The row-statistics buffer of stream `s`, at least `bytes` long.
int acquire_rowstat(int dev, hipStream_t s, size_t bytes, const CaptureInfo& ci, float** out);

// Enqueues the kernels of a planned backward on `s`: items holds n_kv key-block items then n_q
// query-block items (device memory); rowstat has bwd_rowstat_bytes(p) bytes.  On failure *what
// names the step.
hipError_t launch_bwd(const BwdPlan& p, const fa_work_item_t* items, int64_t n_kv, int64_t n_q, float* rowstat,
                      hipStream_t s, const char** what);

// Waits for every device and frees all of the above.
void release_all();

// Number of work lists cached on device `dev` (tests).
int64_t cached_list_count(int dev);

}  // namespace fa
