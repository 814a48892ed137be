// kmeans_update_internal.h -- launch plan of the centroid update (the step
// after assignment in a Lloyd iteration).  Not part of the public interface.
#pragma once

#include "kmeans_internal.h"

namespace kmeans {

// Workspace layout and launch shape of one kmeans_update call.
struct UpdatePlan {
    int path;          // 1: radix sort + chunked reduce + finish; 2: buckets
    // path 2 (bucket_path_fits): buckets of 2^bucket_log2 clusters, sort
    // tiles of 2^bin_tile_log2 points, workspace offsets of the sorted slot
    // words (point index, cluster in bucket) and the [bin_tiles][buckets + 1]
    // tile directory.
    int bucket_log2, buckets, bin_tile_log2, bin_tiles;
    size_t sidx, dir;
    // path 1
    int passes;        // radix passes over the keys 0..K (K = stray label)
    int digit_bits;    // bits per pass (<= 8): the key bits split evenly
    int tile_log2;     // sort tile of 2^tile_log2 points (>= 1024)
    int tiles;         // sort tiles
    int stride;        // histogram row length: tiles rounded up to 4
    int chunk;         // sorted positions per reduce chunk (32 KiB of rows, <= 240)
    int chunks;        // reduce chunks
    size_t keys[2], vals[2];   // byte offsets of the ping-pong sort buffers
    size_t hist;       // [passes][256][stride] int32
    size_t start, end; // [K] int32 each
    size_t partial;    // [chunks][2][D] fp32
    size_t bytes;      // total workspace (0 when N == 0)
    int compute_units; // reduce workgroups: four per CU
};

// Whether the bucket path supports the shape (N <= 2^24, K <= 16384).
bool bucket_path_fits(int64_t N, int64_t K);

// Requires 0 <= N < 2^31, valid D, 1 <= K < 2^31 (checked by the caller);
// compute_units <= 0 means 256; force_path 0 (automatic), 1 or 2 (2 only
// where bucket_path_fits).
UpdatePlan make_update_plan(int64_t N, int64_t D, int64_t K, int compute_units,
                            int force_path);

// All launches of one update on `stream`; ws holds plan.bytes bytes (may be
// null when N == 0).  means may be null.
hipError_t launch_update(const UpdatePlan &plan, const uint16_t *X, const int32_t *labels,
                         const uint16_t *C_old, int N, int D, int K, uint16_t *C_new,
                         float *norms, int32_t *counts, float *means, void *ws,
                         hipStream_t stream);

}  // namespace kmeans
