// kmeans_api.hip -- the C ABI: argument validation, dispatch, launches.
// Every check happens on the host before the first HIP call.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <map>
#include <mutex>
#include <functional>
#include <string>
#include <thread>
#include <tuple>
#include <utility>

#include "kmeans_internal.h"
#include "kmeans_mi355x.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

// ---- The fixed device scratch of kmeans_assign_static ----
//
// kmeans_assign_static's split path takes its scratch from this file-scope
// device array instead of the stream's workspace, so that the call allocates
// nothing.  Each device that the library runs on holds its own copy until
// the process ends.  The host-side name `scratch` is only a stand-in for the
// device symbol: its device address, per device, comes from
// hipGetSymbolAddress (static_scratch below) and is the only form ever
// handed to a kernel.
static __device__ __align__(256) uint8_t scratch[KMEANS_STATIC_SCRATCH_BYTES];

namespace kmeans {

kmeans_status_t fail(kmeans_status_t st, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kmeans_status_t ok() {
    g_last_error.clear();
    return KMEANS_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int device_compute_units() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return kDefaultComputeUnits;
    int cus = cache[dev].load(std::memory_order_relaxed);
    if (cus <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            cus <= 0)
            cus = kDefaultComputeUnits;
        cache[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

namespace {
// (device, stream, thread) -> (buffer, bytes).  The thread is part of the key
// only for hipStreamPerThread, one handle that names a different stream in
// every thread.  Never destroyed: at process exit the runtime may be gone
// before static destructors run, and it reclaims device memory itself.
using WsKey = std::tuple<int, uintptr_t, size_t>;
std::mutex g_ws_mutex;
auto *g_ws = new std::map<WsKey, std::pair<void *, size_t>>();
// The persistent path's tile queue per (device, stream, thread): two int32
// counters in a small allocation of their own (the workspace above is
// overwritten by other calls, the queue must stay zero between launches).
auto *g_queues = new std::map<WsKey, int *>();
constexpr size_t kQueueBytes = 256;
constexpr size_t kWorkspaceGranule = size_t(1) << 20;

WsKey ws_key(int dev, hipStream_t stream) {
    const size_t thread = stream == hipStreamPerThread
                              ? std::hash<std::thread::id>()(std::this_thread::get_id())
                              : 0;
    return WsKey{dev, reinterpret_cast<uintptr_t>(stream), thread};
}
}  // namespace

WorkspaceLease::WorkspaceLease(hipStream_t stream, size_t bytes) {
    g_ws_mutex.lock();
    int dev = 0;
    error_ = hipGetDevice(&dev);
    if (error_ != hipSuccess)
        return;
    auto &slot = (*g_ws)[ws_key(dev, stream)];
    if (slot.second < bytes) {
        if (slot.first != nullptr) {
            void *old = slot.first;
            slot = {nullptr, 0};
            error_ = hipFreeAsync(old, stream);
            if (error_ != hipSuccess)
                return;
        }
        const size_t want = (bytes + kWorkspaceGranule - 1) / kWorkspaceGranule * kWorkspaceGranule;
        void *p = nullptr;
        error_ = hipMallocAsync(&p, want, stream);
        if (error_ == hipSuccess && p == nullptr)
            error_ = hipErrorOutOfMemory;
        if (error_ != hipSuccess)
            return;
        slot = {p, want};
    }
    ptr_ = slot.first;
}

WorkspaceLease::~WorkspaceLease() { g_ws_mutex.unlock(); }

QueueLease::QueueLease(hipStream_t stream) {
    g_ws_mutex.lock();
    int dev = 0;
    error_ = hipGetDevice(&dev);
    if (error_ != hipSuccess)
        return;
    int *&q = (*g_queues)[ws_key(dev, stream)];
    if (q == nullptr) {
        void *p = nullptr;
        error_ = hipMallocAsync(&p, kQueueBytes, stream);
        if (error_ == hipSuccess && p == nullptr)
            error_ = hipErrorOutOfMemory;
        if (error_ != hipSuccess)
            return;
        error_ = launch_zero_queue(static_cast<int *>(p), stream);
        if (error_ != hipSuccess) {
            (void)hipFreeAsync(p, stream);
            return;
        }
        q = static_cast<int *>(p);
    }
    ptr_ = q;
}

QueueLease::~QueueLease() { g_ws_mutex.unlock(); }

hipError_t release_workspace(hipStream_t stream) {
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    const WsKey key = ws_key(dev, stream);
    auto qit = g_queues->find(key);
    if (qit != g_queues->end()) {
        int *q = qit->second;
        g_queues->erase(qit);
        if (q != nullptr && (e = hipFreeAsync(q, stream)) != hipSuccess)
            return e;
    }
    auto it = g_ws->find(key);
    if (it == g_ws->end())
        return hipSuccess;
    void *p = it->second.first;
    g_ws->erase(it);
    return p != nullptr ? hipFreeAsync(p, stream) : hipSuccess;
}

kmeans_status_t check_d(int64_t D) {
    if (D < KMEANS_MIN_D || D > KMEANS_MAX_D || D % 16 != 0)
        return fail(KMEANS_ERR_UNSUPPORTED,
                    "D=%lld unsupported: need %d <= D <= %d and D %% 16 == 0",
                    static_cast<long long>(D), KMEANS_MIN_D, KMEANS_MAX_D);
    return KMEANS_OK;
}

}  // namespace kmeans

namespace {

using kmeans::aligned;
using kmeans::check_d;
using kmeans::device_compute_units;
using kmeans::fail;
using kmeans::kMaxRows;
using kmeans::ok;

kmeans_status_t check_shape(int64_t N, int64_t D, int64_t K) {
    if (N < 0)
        return fail(KMEANS_ERR_INVALID_ARG, "N=%lld must be >= 0", static_cast<long long>(N));
    if (K < 1)
        return fail(KMEANS_ERR_INVALID_ARG, "K=%lld must be >= 1", static_cast<long long>(K));
    kmeans_status_t st = check_d(D);
    if (st != KMEANS_OK)
        return st;
    if (N > kMaxRows || K > kMaxRows)
        return fail(KMEANS_ERR_UNSUPPORTED, "N=%lld or K=%lld too large (max %lld)",
                    static_cast<long long>(N), static_cast<long long>(K),
                    static_cast<long long>(kMaxRows));
    if (kmeans::min_k_ranges(D, K) > kmeans::kMaxSplits)
        return fail(KMEANS_ERR_UNSUPPORTED, "K=%lld rows of D=%lld: centroids over %d x 2 GiB",
                    static_cast<long long>(K), static_cast<long long>(D), kmeans::kMaxSplits);
    return KMEANS_OK;
}

constexpr size_t kStaticScratchBytes = KMEANS_STATIC_SCRATCH_BYTES;
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's `scratch`, resolved once per device
// (with that device current) on the first call there.
kmeans_status_t static_scratch(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(KMEANS_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(KMEANS_ERR_UNSUPPORTED, "device %d: the static scratch serves devices "
                    "0..%d", dev, kMaxScratchDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr)
            return fail(KMEANS_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s",
                        dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KMEANS_OK;
}

enum class Scratch { kWorkspace, kStatic };

// The split path's two launches with their scratch at `base`: partial scores
// [splits][N], partial labels [splits][N], ||x||^2 [N].
kmeans_status_t launch_split(const kmeans::Plan &pl, const uint16_t *Xb, const uint16_t *Cb,
                             const float *norms, int n, int d, int k, int32_t *labels,
                             float *min_dist, void *base, hipStream_t stream) {
    const size_t per = static_cast<size_t>(n);
    auto *ws_score = static_cast<float *>(base);
    auto *ws_label = reinterpret_cast<int32_t *>(ws_score + per * pl.splits);
    auto *ws_xx = reinterpret_cast<float *>(ws_label + per * pl.splits);
    hipError_t e = kmeans::launch_assign(pl, Xb, Cb, norms, n, d, k, labels, min_dist, ws_score,
                                         ws_label, ws_xx, stream);
    if (e == hipSuccess)
        e = kmeans::launch_merge(pl, Xb, Cb, norms, n, d, k, labels, min_dist, ws_score,
                                 ws_label, ws_xx, stream);
    if (e != hipSuccess)
        return fail(KMEANS_ERR_HIP, "split-path launch failed: %s", hipGetErrorString(e));
    return ok();
}

kmeans_status_t run_assign(const void *X, const void *C, const float *norms, int64_t N,
                           int64_t D, int64_t K, int32_t *labels, float *min_dist,
                           int path, int count, hipStream_t stream,
                           Scratch scratch_kind = Scratch::kWorkspace) {
    kmeans_status_t st = check_shape(N, D, K);
    if (st != KMEANS_OK)
        return st;
    if (path < KMEANS_PATH_AUTO || path > KMEANS_PATH_PERSISTENT)
        return fail(KMEANS_ERR_INVALID_ARG, "path=%d unknown", path);
    if (count < 0)
        return fail(KMEANS_ERR_INVALID_ARG, "count=%d must be >= 0", count);
    if (kmeans::min_k_ranges(D, K) > 1 &&
        (path == KMEANS_PATH_DIRECT || path == KMEANS_PATH_PERSISTENT))
        return fail(KMEANS_ERR_UNSUPPORTED, "K=%lld rows of D=%lld: centroids over 2 GiB need "
                    "the split path", static_cast<long long>(K), static_cast<long long>(D));
    if (N == 0)
        return ok();
    if (!X || !C || !norms || !labels || !min_dist)
        return fail(KMEANS_ERR_INVALID_ARG, "null pointer argument (X=%p C=%p norms=%p "
                    "labels=%p min_dist=%p)", X, C, static_cast<const void *>(norms),
                    static_cast<void *>(labels), static_cast<void *>(min_dist));
    if (!aligned(X, 16) || !aligned(C, 16))
        return fail(KMEANS_ERR_ALIGNMENT, "X and C must be 16-byte aligned");
    if (!aligned(norms, 4) || !aligned(labels, 4) || !aligned(min_dist, 4))
        return fail(KMEANS_ERR_ALIGNMENT, "norms, labels and min_dist must be 4-byte aligned");

    const kmeans::Plan pl = kmeans::make_plan(N, D, K, path, count, device_compute_units());
    const auto *Xb = static_cast<const uint16_t *>(X);
    const auto *Cb = static_cast<const uint16_t *>(C);
    const int n = static_cast<int>(N), d = static_cast<int>(D), k = static_cast<int>(K);

    if (pl.path == KMEANS_PATH_PERSISTENT) {
        const kmeans::QueueLease queue(stream);
        if (queue.error() != hipSuccess)
            return fail(KMEANS_ERR_NO_MEMORY, "tile queue: %s", hipGetErrorString(queue.error()));
        const hipError_t e = kmeans::launch_assign_queue(pl, Xb, Cb, norms, n, d, k, labels,
                                                         min_dist, queue.ptr(), stream);
        if (e != hipSuccess)
            return fail(KMEANS_ERR_HIP, "assign launch failed: %s", hipGetErrorString(e));
        return ok();
    }
    if (pl.path == KMEANS_PATH_DIRECT) {
        const int head = n - pl.tail_points;
        hipError_t e = kmeans::launch_assign(pl, Xb, Cb, norms, head, d, k, labels, min_dist,
                                             nullptr, nullptr, nullptr, stream);
        if (e == hipSuccess && pl.tail_points > 0) {
            // The last points as narrow tiles: same kernel family on offset
            // pointers, so each point's result is computed exactly as before.
            kmeans::Plan tp = pl;
            tp.pb = 1;
            tp.ppw = pl.ppw / kmeans::wide_point_blocks(pl.ks);
            tp.tiles = tp.wgs = pl.tail_wgs;
            e = kmeans::launch_assign(tp, Xb + static_cast<size_t>(head) * D, Cb, norms,
                                      pl.tail_points, d, k, labels + head, min_dist + head,
                                      nullptr, nullptr, nullptr, stream);
        }
        if (e != hipSuccess)
            return fail(KMEANS_ERR_HIP, "assign launch failed: %s", hipGetErrorString(e));
        return ok();
    }

    // Split path: scratch for the partial winners and ||x||^2, from the
    // stream's workspace or from the fixed device array.  Every element the
    // merge pass reads is written by the assign pass first, so neither needs
    // clearing.
    const size_t per = static_cast<size_t>(N);
    const size_t bytes = per * pl.splits * (sizeof(float) + sizeof(int32_t)) + per * sizeof(float);
    void *base = nullptr;
    if (scratch_kind == Scratch::kStatic) {
        if (bytes > kStaticScratchBytes)
            return fail(KMEANS_ERR_UNSUPPORTED, "N=%lld D=%lld K=%lld plans %d K-ranges, whose "
                        "scratch (%zu bytes) exceeds the static buffer (%zu bytes); use "
                        "kmeans_assign", static_cast<long long>(N), static_cast<long long>(D),
                        static_cast<long long>(K), pl.splits, bytes, kStaticScratchBytes);
        st = static_scratch(&base);
        if (st != KMEANS_OK)
            return st;
        return launch_split(pl, Xb, Cb, norms, n, d, k, labels, min_dist, base, stream);
    }
    const kmeans::WorkspaceLease lease(stream, bytes);
    if (lease.error() != hipSuccess)
        return fail(KMEANS_ERR_NO_MEMORY, "workspace of %zu bytes: %s", bytes,
                    hipGetErrorString(lease.error()));
    return launch_split(pl, Xb, Cb, norms, n, d, k, labels, min_dist, lease.ptr(), stream);
}

}  // namespace

extern "C" {

kmeans_status_t kmeans_centroid_norms(const void *C, int64_t K, int64_t D, float *norms,
                                      hipStream_t stream) {
    if (K < 0)
        return fail(KMEANS_ERR_INVALID_ARG, "K=%lld must be >= 0", static_cast<long long>(K));
    kmeans_status_t st = check_d(D);
    if (st != KMEANS_OK)
        return st;
    if (K > kMaxRows)
        return fail(KMEANS_ERR_UNSUPPORTED, "K=%lld too large", static_cast<long long>(K));
    if (K == 0)
        return ok();
    if (!C || !norms)
        return fail(KMEANS_ERR_INVALID_ARG, "null pointer argument (C=%p norms=%p)", C,
                    static_cast<void *>(norms));
    if (!aligned(C, 16))
        return fail(KMEANS_ERR_ALIGNMENT, "C must be 16-byte aligned");
    if (!aligned(norms, 4))
        return fail(KMEANS_ERR_ALIGNMENT, "norms must be 4-byte aligned");
    hipError_t e = kmeans::launch_norms(static_cast<const uint16_t *>(C), static_cast<int>(K),
                                        static_cast<int>(D), norms, stream);
    if (e != hipSuccess)
        return fail(KMEANS_ERR_HIP, "norms launch failed: %s", hipGetErrorString(e));
    return ok();
}

kmeans_status_t kmeans_assign(const void *X, const void *C, const float *norms, int64_t N,
                              int64_t D, int64_t K, int32_t *labels, float *min_dist,
                              hipStream_t stream) {
    return run_assign(X, C, norms, N, D, K, labels, min_dist, KMEANS_PATH_AUTO, 0, stream);
}

kmeans_status_t kmeans_assign_static(const void *X, const void *C, const float *norms,
                                     int64_t N, int64_t D, int64_t K, int32_t *labels,
                                     float *min_dist, hipStream_t stream) {
    return run_assign(X, C, norms, N, D, K, labels, min_dist, KMEANS_PATH_AUTO, 0, stream,
                      Scratch::kStatic);
}

kmeans_status_t kmeans_assign_path(const void *X, const void *C, const float *norms,
                                   int64_t N, int64_t D, int64_t K, int32_t *labels,
                                   float *min_dist, int32_t path, int32_t count,
                                   hipStream_t stream) {
    return run_assign(X, C, norms, N, D, K, labels, min_dist, path, count, stream);
}

kmeans_status_t kmeans_plan(int64_t N, int64_t D, int64_t K, int32_t compute_units,
                            int32_t *path, int32_t *splits, int32_t *workgroups,
                            int32_t *points_per_wg, int32_t *k_block, int32_t *padded_d) {
    kmeans_status_t st = check_shape(N, D, K);
    if (st != KMEANS_OK)
        return st;
    const kmeans::Plan pl =
        kmeans::make_plan(N > 0 ? N : 1, D, K, KMEANS_PATH_AUTO, 0, compute_units);
    if (path)
        *path = pl.path;
    if (splits)
        *splits = pl.splits;
    if (workgroups)
        *workgroups = N > 0 ? pl.wgs + pl.tail_wgs : 0;
    if (points_per_wg)
        *points_per_wg = pl.ppw;
    if (k_block)
        *k_block = pl.bk;
    if (padded_d)
        *padded_d = pl.ks * 16;
    return ok();
}

kmeans_status_t kmeans_release_workspace(hipStream_t stream) {
    const hipError_t e = kmeans::release_workspace(stream);
    if (e != hipSuccess)
        return fail(KMEANS_ERR_HIP, "releasing the workspace failed: %s", hipGetErrorString(e));
    return ok();
}

const char *kmeans_last_error(void) { return g_last_error.c_str(); }

int kmeans_abi_version(void) { return KMEANS_ABI_VERSION; }

}  // extern "C"
