// Library-owned device memory of the entry points: uploaded work lists and the per-stream
// row-statistics buffers.
//
// Work lists.  Each sequence layout (with mask window, head count and kernel path) gets its own
// device copy of its work list, uploaded once with an asynchronous copy on the calling stream from
// pinned staging memory, and never written again.  Calls with a cached layout only read it, so a
// new layout never waits for the host or for kernels of another layout, and kernels still in
// flight, or recorded in a graph, keep reading valid items.  The cache holds up to kMaxLists
// layouts; an evicted list's device memory is reused for a new list only after the events
// recorded after its last uses on every stream have completed (reuse, not hipFree, which would
// wait for the whole device).  A list used inside a stream capture is never evicted.
//
// Row statistics.  The two planes of -D and -beta live in a buffer per stream: calls on one stream
// are ordered by the stream, calls on different streams get different buffers.  A buffer grows
// geometrically; the old one is released after its stream has drained.  Inside a stream capture
// the library allocates nothing: the stream's buffer must already be large enough (an uncaptured
// call of at least this size on this stream), and is then reserved for that capture -- later
// uncaptured calls on the stream get a buffer of their own, so replays of the graph never share it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "fa_internal.h"
#include "fa_workspace.h"

namespace fa {
namespace {

constexpr size_t kMaxLists = 64;

struct ListEntry {
    fa_work_item_t* dev = nullptr;
    size_t bytes = 0;
    int64_t n_first = 0;
    int64_t n_second = 0;
    std::vector<std::pair<hipStream_t, hipEvent_t>> uses;  // last eager use per stream
    bool captured = false;
    uint64_t stamp = 0;
};

struct Staging {
    void* host = nullptr;
    size_t bytes = 0;
    hipEvent_t copied = nullptr;  // recorded after the copy out of it
};

struct StreamBuf {
    float* rowstat = nullptr;
    size_t bytes = 0;
    bool captured = false;
    unsigned long long capture_id = 0;
};

struct DeviceState {
    std::map<std::vector<int64_t>, ListEntry> lists;
    std::vector<ListEntry> retired;  // evicted lists waiting for their last uses
    std::vector<std::pair<fa_work_item_t*, size_t>> free_bufs;  // device memory of finished lists
    std::vector<Staging> staging;
    std::unordered_map<hipStream_t, StreamBuf> streams;
    std::vector<float*> graph_owned;  // row statistics buffers reserved by a capture
    std::vector<hipEvent_t> spare_events;
    uint64_t clock = 0;
};

std::unordered_map<int, DeviceState> g_state;

int runtime_error(const std::string& what, hipError_t e) {
    set_error(what + ": " + hipGetErrorString(e));
    return FA_ERR_RUNTIME;
}

int take_event(DeviceState& ds, hipEvent_t* out) {
    if (!ds.spare_events.empty()) {
        *out = ds.spare_events.back();
        ds.spare_events.pop_back();
        return FA_OK;
    }
    hipError_t e = hipEventCreateWithFlags(out, hipEventDisableTiming);
    return e == hipSuccess ? FA_OK : runtime_error("event create", e);
}

// true when every recorded use of the list has completed (or the query failed for good: the
// event is then useless, and waiting would not help)
bool uses_done(const ListEntry& le) {
    for (const auto& u : le.uses) {
        if (hipEventQuery(u.second) == hipErrorNotReady) return false;
    }
    return true;
}

void recycle_events(DeviceState& ds, ListEntry& le) {
    for (auto& u : le.uses) ds.spare_events.push_back(u.second);
    le.uses.clear();
}

// Moves the memory of retired lists whose uses have completed to the free pool.
void reclaim(DeviceState& ds) {
    for (size_t i = 0; i < ds.retired.size();) {
        ListEntry& le = ds.retired[i];
        if (uses_done(le)) {
            ds.free_bufs.emplace_back(le.dev, le.bytes);
            recycle_events(ds, le);
            ds.retired[i] = std::move(ds.retired.back());
            ds.retired.pop_back();
        } else {
            ++i;
        }
    }
    // a bounded pool: past it, drop the smallest (rare; hipFree waits for the device)
    while (ds.free_bufs.size() > kMaxLists) {
        auto small = std::min_element(ds.free_bufs.begin(), ds.free_bufs.end(),
                                      [](const auto& a, const auto& b) { return a.second < b.second; });
        (void)hipFree(small->first);
        ds.free_bufs.erase(small);
    }
}

// Device memory for a list of `bytes`: the smallest free buffer that fits, else a new one.
int take_list_buffer(DeviceState& ds, size_t bytes, fa_work_item_t** dev, size_t* cap) {
    auto best = ds.free_bufs.end();
    for (auto it = ds.free_bufs.begin(); it != ds.free_bufs.end(); ++it) {
        if (it->second >= bytes && (best == ds.free_bufs.end() || it->second < best->second)) best = it;
    }
    if (best != ds.free_bufs.end()) {
        *dev = best->first;
        *cap = best->second;
        ds.free_bufs.erase(best);
        return FA_OK;
    }
    hipError_t e = hipMalloc(reinterpret_cast<void**>(dev), bytes);
    if (e != hipSuccess) return runtime_error("work list allocation", e);
    *cap = bytes;
    return FA_OK;
}

void evict_if_full(DeviceState& ds) {
    while (ds.lists.size() >= kMaxLists) {
        auto victim = ds.lists.end();
        for (auto it = ds.lists.begin(); it != ds.lists.end(); ++it) {
            if (it->second.captured) continue;
            if (victim == ds.lists.end() || it->second.stamp < victim->second.stamp) victim = it;
        }
        if (victim == ds.lists.end()) return;  // everything is held by captured graphs
        ds.retired.push_back(std::move(victim->second));
        ds.lists.erase(victim);
    }
}

// Pinned staging memory of at least `bytes` whose previous copy has completed.
int get_staging(DeviceState& ds, size_t bytes, Staging** out) {
    for (auto& st : ds.staging) {
        if (st.bytes >= bytes && hipEventQuery(st.copied) != hipErrorNotReady) {
            *out = &st;
            return FA_OK;
        }
    }
    Staging st;
    st.bytes = std::max<size_t>(bytes, 4096);
    hipError_t e = hipHostMalloc(&st.host, st.bytes, hipHostMallocDefault);
    if (e != hipSuccess) return runtime_error("work list staging", e);
    e = hipEventCreateWithFlags(&st.copied, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipHostFree(st.host);
        return runtime_error("event create", e);
    }
    ds.staging.push_back(st);
    *out = &ds.staging.back();
    return FA_OK;
}

}  // namespace

std::mutex& state_mutex() {
    static std::mutex m;
    return m;
}

CaptureInfo capture_info(hipStream_t s) {
    CaptureInfo ci;
    if (s == nullptr) return ci;  // the null stream cannot be captured
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    unsigned long long id = 0;
    if (hipStreamGetCaptureInfo(s, &st, &id) == hipSuccess && st != hipStreamCaptureStatusNone) {
        ci.capturing = true;
        ci.id = id;
    }
    return ci;
}

int acquire_list(int dev, const std::vector<int64_t>& key, const ListBuilder& build, hipStream_t s,
                 const CaptureInfo& ci, ListRef* out) {
    DeviceState& ds = g_state[dev];
    auto it = ds.lists.find(key);
    if (it == ds.lists.end()) {
        if (ci.capturing) {
            set_error("this sequence layout has no uploaded work list yet and the stream is being captured: "
                      "make one uncaptured call with this layout first");
            return FA_ERR_UNSUPPORTED;
        }
        std::vector<fa_work_item_t> items;
        int64_t n_first = 0;
        build(items, n_first);
        ListEntry le;
        le.n_first = n_first;
        le.n_second = static_cast<int64_t>(items.size()) - n_first;
        const size_t need = std::max<size_t>(items.size() * sizeof(fa_work_item_t), sizeof(fa_work_item_t));
        evict_if_full(ds);
        reclaim(ds);
        int r = take_list_buffer(ds, need, &le.dev, &le.bytes);
        if (r != FA_OK) return r;
        if (!items.empty()) {
            Staging* st = nullptr;
            r = get_staging(ds, need, &st);
            if (r != FA_OK) {
                ds.free_bufs.emplace_back(le.dev, le.bytes);
                return r;
            }
            std::memcpy(st->host, items.data(), items.size() * sizeof(fa_work_item_t));
            hipError_t e =
                hipMemcpyAsync(le.dev, st->host, items.size() * sizeof(fa_work_item_t), hipMemcpyHostToDevice, s);
            if (e == hipSuccess) e = hipEventRecord(st->copied, s);
            if (e != hipSuccess) {
                // the copy may have been enqueued: wait for it before the memory is handed out again
                (void)hipStreamSynchronize(s);
                ds.free_bufs.emplace_back(le.dev, le.bytes);
                return runtime_error("work list upload", e);
            }
        }
        it = ds.lists.emplace(key, std::move(le)).first;
    }
    ListEntry& le = it->second;
    le.stamp = ++ds.clock;
    out->items = le.dev;
    out->n_first = le.n_first;
    out->n_second = le.n_second;
    out->handle = &le;
    return FA_OK;
}

int note_list_use(int dev, const ListRef& ref, hipStream_t s, const CaptureInfo& ci) {
    DeviceState& ds = g_state[dev];
    ListEntry& le = *static_cast<ListEntry*>(ref.handle);
    if (ci.capturing) {
        le.captured = true;
        return FA_OK;
    }
    hipEvent_t ev = nullptr;
    for (auto& u : le.uses) {
        if (u.first == s) ev = u.second;
    }
    if (ev == nullptr) {
        int r = take_event(ds, &ev);
        if (r != FA_OK) return r;
        le.uses.emplace_back(s, ev);
    }
    hipError_t e = hipEventRecord(ev, s);
    return e == hipSuccess ? FA_OK : runtime_error("event record", e);
}

int acquire_rowstat(int dev, hipStream_t s, size_t bytes, const CaptureInfo& ci, float** out) {
    DeviceState& ds = g_state[dev];
    StreamBuf& sb = ds.streams[s];
    if (ci.capturing) {
        if (sb.rowstat == nullptr || sb.bytes < bytes || (sb.captured && sb.capture_id != ci.id)) {
            set_error("the stream is being captured and has no free row-statistics buffer of this size: make an "
                      "uncaptured call of at least this size on this stream first");
            return FA_ERR_UNSUPPORTED;
        }
        sb.captured = true;
        sb.capture_id = ci.id;
        *out = sb.rowstat;
        return FA_OK;
    }
    if (sb.captured) {
        // reserved for the graph that recorded it: keep it alive, start a new one
        ds.graph_owned.push_back(sb.rowstat);
        sb = StreamBuf{};
    }
    if (sb.rowstat == nullptr || sb.bytes < bytes) {
        if (sb.rowstat != nullptr) {
            // only this stream's calls use it: once they are done it can go
            hipError_t e = hipStreamSynchronize(s);
            if (e != hipSuccess) return runtime_error("stream synchronize", e);
            (void)hipFree(sb.rowstat);
            sb.rowstat = nullptr;
            sb.bytes = 0;
        }
        const size_t grown = std::max<size_t>({bytes, 4096, sb.bytes + sb.bytes / 2});
        hipError_t e = hipMalloc(reinterpret_cast<void**>(&sb.rowstat), grown);
        if (e != hipSuccess) {
            sb.rowstat = nullptr;
            return runtime_error("row statistics allocation", e);
        }
        sb.bytes = grown;
    }
    *out = sb.rowstat;
    return FA_OK;
}

void release_all() {
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_state) {
        (void)hipSetDevice(kv.first);
        (void)hipDeviceSynchronize();
        DeviceState& ds = kv.second;
        for (auto& l : ds.lists) {
            (void)hipFree(l.second.dev);
            for (auto& u : l.second.uses) (void)hipEventDestroy(u.second);
        }
        for (auto& l : ds.retired) {
            (void)hipFree(l.dev);
            for (auto& u : l.uses) (void)hipEventDestroy(u.second);
        }
        for (auto& fb : ds.free_bufs) (void)hipFree(fb.first);
        for (auto& st : ds.staging) {
            (void)hipHostFree(st.host);
            (void)hipEventDestroy(st.copied);
        }
        for (auto& sb : ds.streams) (void)hipFree(sb.second.rowstat);
        for (float* p : ds.graph_owned) (void)hipFree(p);
        for (hipEvent_t e : ds.spare_events) (void)hipEventDestroy(e);
    }
    g_state.clear();
    (void)hipSetDevice(cur);
}

int64_t cached_list_count(int dev) {
    auto it = g_state.find(dev);
    return it == g_state.end() ? 0 : static_cast<int64_t>(it->second.lists.size());
}

}  // namespace fa
