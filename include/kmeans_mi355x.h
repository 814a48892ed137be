/*
 * kmeans_mi355x.h -- C ABI of the MI355X (gfx950) k-means assignment library
 * (with the centroid update that follows assignment in a Lloyd iteration).
 *
 * The operation.  flashlib PR #22, "Optimize Blackwell k-means assignment
 * reduction", Summary: the assignment step scores every (point, centroid)
 * pair from the point-centroid product and the centroid norms and keeps the
 * best-scoring centroid per point, the smaller index winning a tie; the
 * "Key ideas and contributions" table (rows "Two-chain argmin" and
 * "Deterministic winner merge") describes the winner search as independent
 * chains merged by (score, index).  The score used here is the squared-
 * Euclidean one,
 *
 *     s_ik = ||c_k||^2 - 2 x_i . c_k ,   label_i = lowest k minimising s_ik,
 *     min_dist_i = ||x_i - c_label_i||^2   (summed directly over the
 *                                          coordinates, in fp32).
 *
 * Non-finite inputs: scores follow IEEE arithmetic and are ranked
 * -inf < finite < +inf < NaN with ties to the lower index, so a NaN score
 * wins only when every score is NaN (label 0).  min_dist is NaN or +inf when
 * x_i or the winning row holds a non-finite value.  Finite inputs must stay
 * below 2^56 in magnitude (no fp32 overflow for D <= 512).
 *
 * Conventions for every entry point:
 *   - All array arguments are DEVICE pointers owned by the caller; the
 *     library keeps no reference after the call returns.
 *   - Calls are asynchronous on `stream` (NULL = the legacy default stream)
 *     and never synchronise.  Execution errors surface at the caller's next
 *     synchronisation on that stream.
 *   - Arguments are validated on the host before any HIP call.  On a non-OK
 *     status nothing was launched (except KMEANS_ERR_HIP, where a launch may
 *     have been attempted) and the outputs are unspecified.
 *   - kmeans_last_error() returns a thread-local message for the last
 *     non-OK status on the calling thread.
 *   - Results are bitwise deterministic for identical inputs and shape; no
 *     floating-point value is accumulated with atomics.
 *   - Outputs must not overlap inputs (not checked).
 */
#ifndef KMEANS_MI355X_H
#define KMEANS_MI355X_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KMEANS_ABI_VERSION 7

/* Supported feature dimension: 16 <= D <= 512 and D % 16 == 0. */
#define KMEANS_MIN_D 16
#define KMEANS_MAX_D 512

typedef enum {
    KMEANS_OK = 0,
    KMEANS_ERR_INVALID_ARG = 1,  /* null pointer, negative size, K < 1 ... */
    KMEANS_ERR_UNSUPPORTED = 2,  /* D outside the supported set; N or K >= 2^31 */
    KMEANS_ERR_ALIGNMENT = 3,    /* X/C not 16-byte or outputs not 4-byte aligned */
    KMEANS_ERR_HIP = 4,          /* a HIP runtime call or launch failed */
    KMEANS_ERR_NO_MEMORY = 5     /* the stream's workspace could not be allocated */
} kmeans_status_t;

typedef enum {
    KMEANS_PATH_AUTO = 0,    /* shape-based choice (what kmeans_assign does) */
    KMEANS_PATH_DIRECT = 1,  /* one pass: every workgroup scans all K centroids */
    KMEANS_PATH_SPLIT = 2,   /* K split over `count` ranges + a merge pass */
    KMEANS_PATH_PERSISTENT = 3  /* direct, one round of workgroups taking point
                                   tiles from a queue (kmeans_assign_path only) */
} kmeans_path_t;

/*
 * Centroid norms, n_k = sum_j c_kj^2 (the "centroid norms" the Summary says
 * the score tile is combined with), one fp32 value per centroid row.
 *
 *   C      bf16 [K][D], row-major, D contiguous, 16-byte aligned.
 *   K      number of centroid rows, 0 <= K < 2^31 (K == 0: no-op, KMEANS_OK).
 *   D      feature dimension (see KMEANS_MIN_D / KMEANS_MAX_D).
 *   norms  fp32 [K], 4-byte aligned, written.
 *
 * Squares of bf16 values are exact in fp32; the sum is fp32 with a fixed
 * order, so bitwise-identical rows get bitwise-identical norms (which the
 * lowest-index rule of kmeans_assign relies on for duplicate rows).
 */
kmeans_status_t kmeans_centroid_norms(const void *C, int64_t K, int64_t D,
                                      float *norms, hipStream_t stream);

/*
 * Nearest-centroid assignment (Summary; "Key ideas and contributions").
 *
 *   X         bf16 [N][D] points, row-major, 16-byte aligned.
 *   C         bf16 [K][D] centroids, row-major, 16-byte aligned.
 *   norms     fp32 [K], ||c_k||^2 as written by kmeans_centroid_norms for
 *             this C (other values give the scores n_k - 2 x.c_k as passed).
 *   N         number of points, 0 <= N < 2^31 (N == 0: no-op, KMEANS_OK).
 *   D         feature dimension, 16 <= D <= 512, D % 16 == 0.
 *   K         number of centroids, 1 <= K < 2^31, with C at most 64 x 2 GiB
 *             (larger: KMEANS_ERR_UNSUPPORTED).  Centroids over 2 GiB always
 *             run the K-split path (kmeans_assign_path with
 *             KMEANS_PATH_DIRECT then returns KMEANS_ERR_UNSUPPORTED).
 *   labels    int32 [N], written: lowest index minimising s_ik.
 *   min_dist  fp32 [N], written: squared distance to the chosen centroid,
 *             sum_j (x_j - c_j)^2 in fp32 (not ||x||^2 + s_best, which
 *             cancels when the data lie far from the origin).
 *
 * Small-N / large-K shapes run a K-split path whose scratch (8 bytes per
 * point per split + 4 bytes per point) is the stream's workspace (see
 * kmeans_release_workspace); KMEANS_ERR_NO_MEMORY if it cannot grow.  All
 * paths give bitwise-identical outputs.
 */
kmeans_status_t kmeans_assign(const void *X, const void *C, const float *norms,
                              int64_t N, int64_t D, int64_t K, int32_t *labels,
                              float *min_dist, hipStream_t stream);

/*
 * Size of the fixed device buffer that kmeans_assign_static uses for the
 * K-split path's scratch (16 MiB, held by every device the library runs on
 * until the process ends).
 */
#define KMEANS_STATIC_SCRATCH_BYTES (16u << 20)

/*
 * kmeans_assign for callers that cannot allocate device memory during the
 * call: code being captured into a HIP graph, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, outputs (bit for bit), dispatch and
 * errors as kmeans_assign, but the K-split path's scratch (8 bytes per point
 * per K-range + 4 per point) comes from a fixed device buffer of
 * KMEANS_STATIC_SCRATCH_BYTES that the library holds per device, so the call
 * makes no hipMalloc/hipFree or other allocating call.  The direct path needs
 * no scratch.  A shape whose split plan needs more than the buffer returns
 * KMEANS_ERR_UNSUPPORTED before any launch (kmeans_assign handles it).
 * Every call on a device shares that device's buffer and leaves its contents
 * behind: calls that overlap in time on one device (different streams or
 * threads, without ordering between them) race and give undefined results;
 * calls ordered on one stream are safe.
 */
kmeans_status_t kmeans_assign_static(const void *X, const void *C, const float *norms,
                                     int64_t N, int64_t D, int64_t K, int32_t *labels,
                                     float *min_dist, hipStream_t stream);

/*
 * kmeans_assign with the dispatch forced: `path` as in kmeans_path_t, and
 * `count` (0 = automatic):
 *   KMEANS_PATH_DIRECT      1: narrow point tiles (32 points per wave), any
 *                           other value: wide tiles (as many points per wave
 *                           as the registers hold; the automatic choice for
 *                           large N)
 *   KMEANS_PATH_SPLIT       number of K-ranges (clamped to 64 and to the
 *                           number of centroid blocks), wide tiles
 *   KMEANS_PATH_PERSISTENT  number of workgroups (0: one per CU), wide
 *                           tiles; each workgroup takes its first tile by
 *                           its index and every later one from a queue of
 *                           two counters that the library keeps per stream
 *                           (created and zeroed on the stream's first such
 *                           call, given back by kmeans_release_workspace),
 *                           so workgroups on faster XCDs take more tiles
 *                           instead of an equal share per XCD.  Centroids
 *                           over 2 GiB: KMEANS_ERR_UNSUPPORTED, as for
 *                           KMEANS_PATH_DIRECT.  Calls on one stream run in
 *                           order and share its queue; another stream has
 *                           its own.
 * Same arguments, outputs and errors as kmeans_assign (count < 0 is
 * KMEANS_ERR_INVALID_ARG); exists so that the paths can be compared bit for
 * bit and timed against each other (the pages' per-shape path table under
 * "Performance").
 */
kmeans_status_t kmeans_assign_path(const void *X, const void *C, const float *norms,
                                   int64_t N, int64_t D, int64_t K, int32_t *labels,
                                   float *min_dist, int32_t path, int32_t count,
                                   hipStream_t stream);

/*
 * The launch plan kmeans_assign would use for a shape on a GPU with
 * `compute_units` CUs (<= 0: 256, an MI355X); host only, makes no HIP call.
 * kmeans_assign itself plans with the current device's CU count.  Any output
 * pointer may be NULL.
 *   path          KMEANS_PATH_DIRECT or KMEANS_PATH_SPLIT
 *   splits        number of K-ranges (1 on the direct path)
 *   workgroups    point-workgroups per K-range, over all launches (when
 *                 the last round of point tiles would be mostly empty, its
 *                 points run as a second launch of narrow tiles)
 *   points_per_wg points owned by one workgroup of the first launch
 *   k_block       centroid rows staged in LDS per block
 *   padded_d      D rounded up to the kernel's k-step multiple
 */
kmeans_status_t kmeans_plan(int64_t N, int64_t D, int64_t K, int32_t compute_units,
                            int32_t *path, int32_t *splits, int32_t *workgroups,
                            int32_t *points_per_wg, int32_t *k_block,
                            int32_t *padded_d);

/*
 * Centroid update: the step that follows assignment in a Lloyd (k-means)
 * iteration.  The pages describe the assignment step only (Summary); this
 * is the plain definition of the update, with the readings noted:
 *
 *     counts[k] = #{ i : labels[i] == k }
 *     means[k]  = (sum of x_i over those i) / counts[k]      (fp32)
 *     C_new[k]  = means[k] rounded to bf16 (nearest, ties to even), or
 *                 C_old[k] bit for bit when counts[k] == 0 (empty cluster)
 *     norms[k]  = ||C_new[k]||^2, the same bits kmeans_centroid_norms gives
 *                 for C_new (so C_new and norms feed kmeans_assign directly)
 *
 *   X       bf16 [N][D] points, row-major, 16-byte aligned.
 *   labels  int32 [N], 4-byte aligned; a label outside [0, K) counts for no
 *           cluster (X and labels may be NULL when N == 0).
 *   C_old   bf16 [K][D] current centroids, 16-byte aligned; read only for
 *           empty clusters.  C_new may be C_old itself (an in-place update);
 *           no other overlap between inputs and outputs is allowed.
 *   N       0 <= N < 2^31 (N == 0: every cluster is empty).
 *   D       16 <= D <= 512, D % 16 == 0.
 *   K       1 <= K < 2^31.
 *   C_new   bf16 [K][D], 16-byte aligned, written.
 *   norms   fp32 [K], written.  counts int32 [K], written.
 *   means   fp32 [K][D] or NULL (then not written); an empty cluster's row
 *           is its old centroid widened to fp32.
 *
 * The sums are fp32, each in an order fixed by the data (see
 * kmeans_update_path for the two orders), so the outputs are bitwise
 * deterministic for a given path; IEEE arithmetic throughout (a NaN
 * coordinate makes that coordinate of the mean NaN).  Scratch of at most
 * about 16 bytes per point plus 8 bytes per cluster is the stream's
 * workspace (see kmeans_release_workspace); KMEANS_ERR_NO_MEMORY if it
 * cannot grow.  The path is chosen from the shape (kmeans_update_path with
 * KMEANS_UPDATE_AUTO): buckets when 256 <= K <= 16384 and N <= 2^24,
 * else the radix sort.
 */
kmeans_status_t kmeans_update(const void *X, const int32_t *labels, const void *C_old,
                              int64_t N, int64_t D, int64_t K, void *C_new, float *norms,
                              int32_t *counts, float *means, hipStream_t stream);

typedef enum {
    KMEANS_UPDATE_AUTO = 0,
    /* Stable LSD radix sort of the labels (8-bit digits or fewer), then
     * fixed chunks of 128 sorted positions (32 KiB of rows) summed per run
     * of equal labels; a cluster cut by chunk edges adds its partial sums in
     * chunk order.  Any N and K; a cluster of any size is spread over many
     * workgroups.  Per radix pass a histogram and a scatter launch (and a
     * scan launch when N is over 2^21), then the reduce and the finish. */
    KMEANS_UPDATE_SORT = 1,
    /* Clusters grouped into at most 1024 buckets of 1, 2, 4, 8 or 16
     * clusters; each tile of 1024 or more points sorts its own points by
     * bucket, stably, and records where each bucket starts in it; then one
     * workgroup per bucket gathers its points tile by tile and sums their
     * rows in index order (buckets of up to 4 clusters: four waves each sum
     * a fixed quarter of every 512 points, added in wave order; of 8 or 16:
     * every 512 points are sorted by cluster, stably, and a cluster's rows
     * are summed by one wave, chunk after chunk).  Two launches.  N <= 2^24
     * and K <= 16384 (else KMEANS_ERR_UNSUPPORTED); a bucket holding a large
     * share of all points runs on one compute unit, far slower than the
     * sort path. */
    KMEANS_UPDATE_BUCKETS = 2
} kmeans_update_path_t;

/*
 * kmeans_update with the path forced (kmeans_update_path_t; any other value
 * is KMEANS_ERR_INVALID_ARG).  Same arguments, outputs and errors
 * otherwise.  The two paths sum in different orders, so their means may
 * differ in the last bits; each is deterministic.
 */
kmeans_status_t kmeans_update_path(const void *X, const int32_t *labels, const void *C_old,
                                   int64_t N, int64_t D, int64_t K, void *C_new, float *norms,
                                   int32_t *counts, float *means, int32_t path,
                                   hipStream_t stream);

/*
 * The workspace of `stream` on the current device.  kmeans_assign's K-split
 * path and kmeans_update take their scratch from one device buffer per
 * (device, stream), kept between calls: a stream-ordered allocation and free
 * on every call costs more host time than a small call's kernels.  It grows
 * in stream order (the old buffer freed by hipFreeAsync and a larger one
 * taken from hipMallocAsync, both on `stream`), so calls on one stream share
 * it safely and calls on different streams never do.  The library never
 * frees it by itself: this call returns it to the device's default memory
 * pool, in stream order, behind the calls already queued on `stream`.  Call
 * it before destroying a stream that was passed to those entry points (a new
 * stream could otherwise inherit the buffer while the old stream's calls
 * still run), or to give the memory back.  hipStreamPerThread gets one
 * buffer per calling thread (release it from that thread).  The same call
 * gives back the stream's tile queue of the persistent path.  No-op when the
 * stream holds none; KMEANS_ERR_HIP if the free fails.
 */
kmeans_status_t kmeans_release_workspace(hipStream_t stream);

/* Thread-local message for the last non-OK status ("" if none). */
const char *kmeans_last_error(void);

/* KMEANS_ABI_VERSION of the built library. */
int kmeans_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KMEANS_MI355X_H */
