// kmeans_internal.h -- launch plan and launchers shared by the C ABI layer
// and the kernel translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kmeans_mi355x.h"

namespace kmeans {

constexpr int kThreads = 256;        // norms / merge kernels: 4 wave64s
constexpr int kTileRows = 32;        // centroid rows per MFMA tile (A operand)
constexpr int kTileCols = 32;        // points per MFMA tile (B operand)
constexpr int kMaxSplits = 64;
// Bytes of centroid rows one K-range may span: buffer resources hold a
// 32-bit size, and offsets at or past 2^31 stand for "out of range".
constexpr int64_t kMaxRangeBytes = (int64_t(1) << 31) - (int64_t(1) << 16);
constexpr int32_t kNoLabel = 0x7fffffff;

// Kernel shape for a padded feature width of 16*ks (ks a power of two).
// Point blocks (32 points each) per wave of a wide tile: as many as the
// register budget holds, so each centroid fragment read from LDS feeds that
// many MFMAs.  Narrow tiles (one block per wave) trade that reuse for four
// (D <= 64) or two (D = 128) times as many workgroups when N is small.
constexpr int wide_point_blocks(int ks) { return ks <= 4 ? 4 : (ks == 8 ? 2 : 1); }
// Centroid rows per LDS block (one of two ring stages): whole 32-row tiles,
// at most one norm per thread; 64 KiB of centroid data at D = 128, 256 and
// 512 (where one workgroup holds a CU), 32 KiB at D <= 64.
constexpr int k_block_rows(int ks) { return ks <= 8 ? 256 : (ks == 16 ? 128 : 64); }
// Waves per assign workgroup (two per SIMD when 8).
constexpr int waves_per_wg(int ks) { return ks <= 16 ? 8 : 4; }
constexpr int points_per_wg(int ks, int pb) { return waves_per_wg(ks) * pb * kTileCols; }
// Waves per SIMD the kernel's register budget is sized for.
constexpr int waves_per_simd(int ks) { return ks >= 32 ? 1 : 2; }
// LDS of one assign workgroup: two centroid stages (BK rows of 32*ks
// bytes), two norm stages and a 1 KiB cache warm-up line.
constexpr int assign_lds_bytes(int ks) {
    return 2 * k_block_rows(ks) * 32 * ks + 2 * k_block_rows(ks) * 4 + 1024;
}
constexpr int kLdsPerCu = 160 * 1024;
// Assign workgroups a CU is guaranteed to hold at once (4 SIMDs; waves and
// LDS are the limits; registers may allow more at small D).
constexpr int assign_wgs_per_cu(int ks) {
    return (4 * waves_per_simd(ks) / waves_per_wg(ks)) < (kLdsPerCu / assign_lds_bytes(ks))
               ? (4 * waves_per_simd(ks) / waves_per_wg(ks))
               : (kLdsPerCu / assign_lds_bytes(ks));
}
constexpr int kDefaultComputeUnits = 256;   // MI355X
// Points of one launch beyond this many bytes (the MI355X last-level cache)
// are loaded with the non-temporal hint: they cannot stay in that cache
// anyway, and cached they push the centroid rows out of L2, which then
// refetches them for every round of point tiles.  Smaller launches keep
// cached loads, so repeated calls on the same points can hit that cache.
constexpr int64_t kStreamPointBytes = int64_t(256) << 20;

// MFMA geometry of the assign kernel for a padded width of 16*ks: 16 =
// v_mfma_f32_16x16x32_bf16, 32 = v_mfma_f32_32x32x16_bf16.  Back to back on
// realistic bf16 data the 16x16x32 form sustains about 10% more on MI355X
// (it reads half the accumulator registers per flop), and its half-size
// accumulators leave room for reduction rotation at D >= 256; at D <= 64 a
// 16x16x32 point block holds only two k-steps, too little matrix time to
// hide its reduction behind when a few waves run alone, so the 32x32x16 form
// is the default there (large calls at D = 64 switch, below); at D = 512
// two 16x16x32 point blocks of 16 k-steps spill, and one 32x32x16 block
// does not.  Every launch of one call uses the same form (Plan::geom), so
// the paths' outputs stay bitwise identical.
constexpr int mfma_geometry(int ks) { return ks == 8 || ks == 16 ? 16 : 32; }
// At D = 64 (ks = 4) a call with at least this much work (N K) takes the
// 16x16x32 form after all: with many workgroups per CU its two k-steps per
// B block are hidden by the other waves, and its fragments are read once per
// two B blocks (measured 1.5-6% faster from 65536 x 4096 up); smaller calls,
// where a few waves run alone, keep 32x32x16 (3-16% faster there).  The form
// is chosen per call, so all launches of a call (split ranges, the narrow
// tail) use the same one and agree bitwise.
constexpr int64_t kG16MinWorkAtD64 = int64_t(1) << 28;

struct Plan {
    int path;          // 1 direct, 2 split, 3 persistent (as kmeans_path_t)
    int geom;          // MFMA form: 16 (16x16x32) or 32 (32x32x16)
    int splits;        // K-ranges (grid.y)
    int ks;            // padded D / 16
    int pb;            // point blocks per wave (wide_point_blocks(ks) or 1)
    int tiles;         // point tiles of ppw points
    int wgs;           // workgroups along N (grid.x; path 3: workgroups of the one round)
    int ppw;           // points per workgroup
    int bk;            // centroid rows per LDS block
    int k_chunk;       // centroids per K-range, multiple of bk
    // Direct path only: the last tail_points points run as a second launch of
    // narrow tiles (tail_wgs workgroups) so that a partial last round of wide
    // tiles does not hold the whole GPU; the first launch covers the rest.
    int tail_points;   // 0: one launch
    int tail_wgs;
};

// K-ranges needed so that none spans more than kMaxRangeBytes of centroid
// rows (1 unless C is over 2 GiB); more than kMaxSplits is unsupported.
int min_k_ranges(int64_t D, int64_t K);

// force_path: 0 auto, 1 direct, 2 split, 3 persistent; force_count: K-ranges
// (split), point blocks per wave (direct: 1 narrow, other wide) or
// workgroups (persistent), 0 auto; compute_units: CUs of the GPU.
// Requires 1 <= N < 2^31, valid D, 1 <= K < 2^31 (checked by the caller).
Plan make_plan(int64_t N, int64_t D, int64_t K, int force_path, int force_count,
               int compute_units);

hipError_t launch_norms(const uint16_t *C, int K, int D, float *norms, hipStream_t stream);

// Squared norm of one bf16 row of D values (D % 8 == 0) as a group of 16
// lanes computes it: lane l fma-accumulates the 16-byte chunks l, l + 16, ...
// (low, then high half of each 32-bit word), and the 16 partial sums combine
// over an xor tree, so every lane of the group returns the same value.  The
// norms pre-pass and the centroid update both use it, so a row gets the same
// norm bits from either.  Every lane of the wave must call it (the xor tree
// reads all 16 lanes of each group); a lane with nothing to add passes D = 0.
__device__ __forceinline__ float row_sq_norm16(const uint16_t *row, int D, int l) {
    typedef uint32_t w4 __attribute__((ext_vector_type(4)));
    float acc = 0.0f;
    for (int c = l; c * 8 < D; c += 16) {
        const w4 v = *reinterpret_cast<const w4 *>(row + c * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float lo = __uint_as_float(v[w] << 16);
            const float hi = __uint_as_float(v[w] & 0xffff0000u);
            acc = fmaf(lo, lo, acc);
            acc = fmaf(hi, hi, acc);
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1)
        acc += __shfl_xor(acc, m, 16);
    return acc;
}

// Direct path when ws_score == nullptr, otherwise writes per-split partial
// winners to the workspace and the merge kernel finishes.
hipError_t launch_assign(const Plan &plan, const uint16_t *X, const uint16_t *C,
                         const float *norms, int N, int D, int K, int32_t *labels,
                         float *min_dist, float *ws_score, int32_t *ws_label,
                         float *ws_xx, hipStream_t stream);

// The persistent direct path (plan.path == 3): one round of plan.wgs
// workgroups taking plan.tiles wide point tiles from `queue`, two int32
// counters that are zero at launch and zero again at its end.  Launches that
// share a queue must not overlap.
hipError_t launch_assign_queue(const Plan &plan, const uint16_t *X, const uint16_t *C,
                               const float *norms, int N, int D, int K, int32_t *labels,
                               float *min_dist, int *queue, hipStream_t stream);
// Zeroes a new queue's counters.
hipError_t launch_zero_queue(int *queue, hipStream_t stream);

hipError_t launch_merge(const Plan &plan, const uint16_t *X, const uint16_t *C,
                        const float *norms, int N, int D, int K, int32_t *labels,
                        float *min_dist, const float *ws_score, const int32_t *ws_label,
                        const float *ws_xx, hipStream_t stream);

// ---- C ABI helpers shared by the entry points (kmeans_api.hip) ----

constexpr int64_t kMaxRows = 0x7fffffffLL - 1024;   // int32 indexing headroom

// Record a thread-local message for kmeans_last_error and return st.
kmeans_status_t fail(kmeans_status_t st, const char *fmt, ...);
// Clear the message and return KMEANS_OK.
kmeans_status_t ok();
bool aligned(const void *p, uintptr_t a);
// KMEANS_ERR_UNSUPPORTED unless 16 <= D <= 512 and D % 16 == 0.
kmeans_status_t check_d(int64_t D);
// Compute units of the current device (cached per device), or 256.
int device_compute_units();

// Scratch for one call on `stream`: a buffer of at least `bytes`, kept per
// (device, stream) between calls, since a hipMallocAsync/hipFreeAsync pair
// per call costs ~15 us of host time (more than a small call's kernels).  It
// grows stream-ordered: the old buffer is freed by hipFreeAsync and the new
// one taken from hipMallocAsync, both on `stream`, behind the work already
// queued there.  Calls on one stream run in order, so they can share it;
// another stream gets its own.  The lease holds a process-wide lock until it
// is destroyed, so no other thread can grow the buffer between this call's
// acquisition and its launches.
class WorkspaceLease {
public:
    WorkspaceLease(hipStream_t stream, size_t bytes);
    ~WorkspaceLease();
    WorkspaceLease(const WorkspaceLease &) = delete;
    WorkspaceLease &operator=(const WorkspaceLease &) = delete;
    void *ptr() const { return ptr_; }
    hipError_t error() const { return error_; }

private:
    void *ptr_ = nullptr;
    hipError_t error_ = hipSuccess;
};

// The persistent path's tile queue for `stream` (two int32 counters, zero
// between launches), created and zeroed on first use; like WorkspaceLease it
// holds the process-wide lock until destroyed.
class QueueLease {
public:
    explicit QueueLease(hipStream_t stream);
    ~QueueLease();
    QueueLease(const QueueLease &) = delete;
    QueueLease &operator=(const QueueLease &) = delete;
    int *ptr() const { return ptr_; }
    hipError_t error() const { return error_; }

private:
    int *ptr_ = nullptr;
    hipError_t error_ = hipSuccess;
};

// Frees (stream-ordered) the current device's buffer and tile queue kept for
// `stream`.
hipError_t release_workspace(hipStream_t stream);

}  // namespace kmeans
