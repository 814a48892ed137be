// kmeans_update.hip -- gfx950 kernels of the centroid update, the step that
// follows assignment in a Lloyd (k-means) iteration.
//
// The pages describe the assignment step only (flashlib PR #22, Summary); the
// update is the plain definition: per cluster, the number of its points and
// the mean of their rows, rounded to bf16 (nearest, ties to even); an empty
// cluster keeps its old centroid; a label outside [0, K) belongs to no
// cluster.  The new rows' squared norms come out too, so the next assignment
// needs no separate norms pass.
//
// Design.  The work is a gather and a sum, bound by reading X once (2 D bytes
// per point); nothing here is a contraction, so no MFMA.  No floating-point
// value is ever accumulated with atomics: every sum runs in an order fixed by
// the data, so a call gives the same bits every time.
//
//  1. Points are grouped by label with a stable LSD radix sort of the keys
//     (label, or K for a stray label) carrying the point index, on digits
//     of at most 8 bits, the key's bits split evenly over the passes (7 + 6
//     at K = 4096).  A pass is: a per-tile digit histogram, one exclusive scan over
//     (digit, tile) -- done by every scatter workgroup for its own tile when
//     there are at most 128 tiles, by a scan kernel beyond -- and a scatter
//     in which every tile ranks its keys in index order: wave ballots give
//     the rank among equal digits inside a wave, and a per-wave count table
//     in LDS, tagged with the round so it never needs clearing, the rank
//     across the tile's waves.
//  2. The reduce kernel walks fixed chunks of sorted positions (32 KiB of
//     rows: 128 at D = 128), four persistent workgroups per CU.  A chunk's
//     rows are staged in LDS with all its row loads in flight at once (a
//     gather of whole rows, 16 bytes per load) while the previous chunk is
//     summed; waves sum each run of equal labels from LDS in position order
//     (the lanes share a row, V = 2, 4 or 8 bf16 values each).  A cluster
//     that starts and ends inside the chunk is finished there; a run cut by
//     a chunk boundary leaves its partial sum, and the finish kernel adds a
//     cluster's partials in chunk order.  Work per chunk is bounded whatever
//     the cluster sizes, and the order of every sum is fixed by the sorted
//     order.
//  3. Finishing a cluster: mean = sum / count in fp32, rounded to bf16, and
//     the squared norm of the rounded row computed exactly as the norms
//     pre-pass computes it (row_sq_norm16 over a copy of the row in LDS).
#include <stdint.h>

#include <memory>

#include "kmeans_update_internal.h"

namespace kmeans {
namespace {

constexpr int kSortThreads = 256;    // histogram workgroups: 4 waves
constexpr int kRadix = 256;
constexpr int kScanThreads = 1024;
constexpr int kFusedScanTiles = 128;  // up to this many sort tiles, no scan kernel
constexpr int kScatterThreads = 1024; // 16 waves: 1024 keys per scatter round
constexpr int kBatchRounds = 4;       // scatter rounds whose keys load together
constexpr int kReduceThreads = 256;  // 4 waves
constexpr int kMaxRow = 512;         // bf16 values of the widest supported row
// Rows of one reduce chunk staged in LDS: 32 KiB, so four workgroups share
// a CU (1024 at once on 256 CUs); 8 loads of 16 bytes per thread fill it.
constexpr int kStageBytes = 32768;
constexpr int kStagePieces = kStageBytes / 16 / kReduceThreads;
constexpr int kMaxChunk = 240;        // keeps a reduce workgroup within 40 KiB of LDS

__device__ __forceinline__ int sort_key(int32_t label, int K) {
    return (label < 0 || label >= K) ? K : label;
}

__device__ __forceinline__ float widen(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bits, nearest with ties to even; NaN -> the quiet NaN 0x7FC0
// with the input's sign; values past the largest finite bf16 after rounding
// become infinite (the carry runs into the exponent).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// ---- 1. radix sort -------------------------------------------------------

// Digit histogram of one tile for the pass on (key >> shift) & mask, written
// digit-major ([digit][tile], all 256 rows; rows above mask count zero).
// FIRST: keys come from the labels, and the launch also clears the cluster
// bounds (clear, n_clear entries).
template <bool FIRST>
__global__ __launch_bounds__(kSortThreads)
void upd_hist_kernel(const int32_t *__restrict__ keys_in, int N, int K, int shift, int mask,
                     int tile_log2, int tiles, int stride, int32_t *__restrict__ hist, int32_t *__restrict__ clear,
                     int64_t n_clear) {
    __shared__ int h[kRadix];
    const int tid = threadIdx.x;
    h[tid] = 0;
    __syncthreads();
    const int t = blockIdx.x;
    const int beg = t << tile_log2;
    const int fin = static_cast<int>(min(static_cast<int64_t>(N),
                                         static_cast<int64_t>(beg) + (int64_t(1) << tile_log2)));
    // Eight keys per thread are loaded before any is counted, so their loads
    // are in flight together (a load-then-count loop waits for each load in
    // turn).  The loads are unconditional, clamped to the tile's last key
    // (every launched tile holds at least one), and an empty asm takes all
    // eight values on every lane, so that the compiler cannot sink each load
    // into a branch of its own (where it would wait for it); positions are
    // counted from beg, so none can wrap around 2^31.
    constexpr int kBatch = 8;
    const int len = fin - beg;
    for (int rel0 = 0; rel0 < len; rel0 += kBatch * kSortThreads) {
        int v[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = keys_in[beg + min(rel0 + u * kSortThreads + tid, len - 1)];
#if defined(__HIP_DEVICE_COMPILE__)
        static_assert(kBatch == 8, "the asm below names eight values");
        asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]),
                          "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
#endif
        int key[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int rel = rel0 + u * kSortThreads + tid;
            key[u] = rel < len ? (FIRST ? sort_key(v[u], K) : v[u]) : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (key[u] >= 0)
                atomicAdd(&h[(key[u] >> shift) & mask], 1);
    }
    __syncthreads();
    int32_t *row = hist + static_cast<size_t>(tid) * stride;
    row[t] = h[tid];
    if (t == tiles - 1)                    // rows are padded to a multiple of 4
        for (int p = tiles; p < stride; ++p)
            row[p] = 0;
    if (FIRST) {
        const int64_t step = static_cast<int64_t>(gridDim.x) * kSortThreads;
        for (int64_t j = static_cast<int64_t>(t) * kSortThreads + tid; j < n_clear; j += step)
            clear[j] = 0;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave by DPP: shifts right by
// 1, 2, 4 and 8 lanes within each row of 16 (lanes shifted in from outside
// the row read 0), then each row adds the last lane of the rows before it
// (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2 and 3).
__device__ __forceinline__ int wave_inclusive_sum(int x) {
    constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 1, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 2, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 4, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowShr + 8, 0xf, 0xf, true);
    x += __builtin_amdgcn_update_dpp(0, x, kRowBcast15, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kRowBcast31, 0xc, 0xf, false);
    return x;
}

// Exclusive scan of h[0..M) in place (M a multiple of 4), one workgroup:
// each thread owns a contiguous run of 16-byte groups, loaded eight at a
// time into registers so the loads overlap (one batch when M <= 32768, and
// then the values stay in registers for the write-back).
__global__ __launch_bounds__(kScanThreads)
void upd_scan_kernel(int32_t *__restrict__ h, int M) {
    typedef int32_t i4 __attribute__((ext_vector_type(4)));
    constexpr int kBatch = 8;
    __shared__ int wtot[kScanThreads / 64];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int groups = M >> 2;
    const int per = (groups + kScanThreads - 1) / kScanThreads;
    const int b = min(groups, tid * per);
    const int e = min(groups, b + per);
    i4 *hv = reinterpret_cast<i4 *>(h);
    i4 keep[kBatch];
    int sum = 0;
    for (int j0 = b; j0 < e; j0 += kBatch) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            keep[u] = j0 + u < e ? hv[j0 + u] : i4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            sum += keep[u][0] + keep[u][1] + keep[u][2] + keep[u][3];
    }
    // Block-wide exclusive prefix of the per-thread sums: within each wave,
    // then across the 16 wave totals.
    const int x = wave_inclusive_sum(sum);
    if (lane == 63)
        wtot[w] = x;
    __syncthreads();
    if (w == 0) {
        const int t = wave_inclusive_sum(lane < kScanThreads / 64 ? wtot[lane] : 0);
        if (lane < kScanThreads / 64)     // same wave: its reads came first
            wtot[lane] = t;
    }
    __syncthreads();
    int run = x - sum + (w > 0 ? wtot[w - 1] : 0);
    auto put = [&](int j, const i4 &v) __attribute__((always_inline)) {
        i4 o;
        o[0] = run;
        o[1] = run + v[0];
        o[2] = o[1] + v[1];
        o[3] = o[2] + v[2];
        run = o[3] + v[3];
        hv[j] = o;
    };
    if (per <= kBatch) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (b + u < e)
                put(b + u, keep[u]);
    } else {
        for (int j0 = b; j0 < e; j0 += kBatch) {
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                keep[u] = j0 + u < e ? hv[j0 + u] : i4{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < kBatch; ++u)
                if (j0 + u < e)
                    put(j0 + u, keep[u]);
        }
    }
}

// One stable scatter pass on digit (key >> shift) & mask.  hist is this
// pass's histogram ([digit][stride]); SCANNED: it holds exclusive offsets
// already (the scan kernel ran), else each workgroup derives its own 256
// offsets from the raw counts (four threads sum each digit's row, the
// digits' totals are prefix-summed across the first four waves).  FIRST: keys come
// from the labels and the values are the point indices.
//
// A round places 1024 keys (16 waves): each wave finds the lanes sharing
// its digit with one ballot per digit bit (rank = earlier such lanes) and the group's last
// lane records the count, tagged with the round, in wcnt[wave][digit]; the
// owner thread of each digit then turns the 16 counts into per-wave starts
// (its running position plus the counts of earlier waves).
template <bool FIRST, bool SCANNED>
__global__ __launch_bounds__(kScatterThreads)
void upd_scatter_kernel(const int32_t *__restrict__ keys_in, const int32_t *__restrict__ vals_in,
                        int N, int K, int shift, int mask, int tile_log2, int tiles,
                        int stride, const int32_t *__restrict__ hist, int32_t *__restrict__ keys_out,
                        int32_t *__restrict__ vals_out) {
    typedef int32_t i4 __attribute__((ext_vector_type(4)));
    constexpr int kWaves = kScatterThreads / 64;
    __shared__ int wcnt[kWaves][kRadix];   // (round tag << 8) | count
    __shared__ int wpos[kWaves][kRadix];   // first position of (wave, digit) this round
    __shared__ int wsum[4];
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int t = blockIdx.x;
    const int beg = t << tile_log2;
    const int fin = static_cast<int>(min(static_cast<int64_t>(N),
                                         static_cast<int64_t>(beg) + (int64_t(1) << tile_log2)));
    // Positions inside the tile are counted from beg (at most 2^19 plus a
    // batch), so that no index past the tile can wrap around 2^31.
    const int len = fin - beg;
    // Keys and values are loaded kBatchRounds rounds at a time, all loads of
    // a batch in flight together; the first batch is issued before the
    // offsets are worked out, so the two sets of loads overlap.  The loads
    // are unconditional (clamped to the tile's last position) and their
    // values are taken by an empty asm only where they are first needed, so
    // that the compiler cannot sink each load into a branch of its own and
    // wait for it there.
    int bkey[kBatchRounds], bval[kBatchRounds];
    auto load_batch = [&](int rel0) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < kBatchRounds; ++r) {
            const int i = beg + min(rel0 + r * kScatterThreads + tid, len - 1);
            bkey[r] = keys_in[i];
            bval[r] = FIRST ? i : vals_in[i];
        }
    };
    auto ready_batch = [&](int rel0) __attribute__((always_inline)) {
#if defined(__HIP_DEVICE_COMPILE__)
        static_assert(kBatchRounds == 4, "the asm below names four values");
        asm volatile("" : "+v"(bkey[0]), "+v"(bkey[1]), "+v"(bkey[2]), "+v"(bkey[3]));
        if constexpr (!FIRST)
            asm volatile("" : "+v"(bval[0]), "+v"(bval[1]), "+v"(bval[2]), "+v"(bval[3]));
#endif
#pragma unroll
        for (int r = 0; r < kBatchRounds; ++r) {
            const bool in = rel0 + r * kScatterThreads + tid < len;
            const int key = FIRST ? sort_key(bkey[r], K) : bkey[r];
            bkey[r] = in ? key : 0;
            bval[r] = in ? bval[r] : 0;
        }
    };
    load_batch(0);
    const bool owner = tid < kRadix;       // thread d < 256 owns digit d
    int run = 0;                           // owner: next position of its digit
    if (SCANNED) {
        if (owner)
            run = hist[static_cast<size_t>(tid) * stride + t];
    } else {
        // Digit d's counts in earlier tiles and in all tiles (stride <= 128):
        // four threads per digit each sum a quarter of its row.  Digits above
        // the mask, and above K >> shift (keys are at most K), never occur:
        // their rows hold zeros and are not read (at K = 4096, 128 of the
        // 256 rows in the first pass and 223 in the second).
        const int d = tid & (kRadix - 1);
        const int qq = tid >> 8;
        const bool live = d <= min(mask, K >> shift);
        constexpr int kG = kFusedScanTiles / 16;        // 16-byte groups per quarter
        // One branch around all of a thread's loads (a dead row, or a quarter
        // wholly past the row's end, loads nothing), none inside it, so that
        // they stay in flight together: a group past the end of a partly
        // filled quarter re-reads the row's last group and counts as zero.
        const i4 *rv = reinterpret_cast<const i4 *>(hist + static_cast<size_t>(d) * stride);
        i4 v[kG];
#pragma unroll
        for (int g = 0; g < kG; ++g)
            v[g] = i4{0, 0, 0, 0};
        if (live && qq * kG * 4 < stride) {
#pragma unroll
            for (int g = 0; g < kG; ++g)
                v[g] = rv[min(qq * kG + g, stride / 4 - 1)];
        }
#if defined(__HIP_DEVICE_COMPILE__)
        static_assert(kG == 8, "the asm below names eight values");
        asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]),
                          "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
#endif
#pragma unroll
        for (int g = 0; g < kG; ++g)
            v[g] = live && (qq * kG + g) * 4 < stride ? v[g] : i4{0, 0, 0, 0};
        int pre = 0, tot = 0;
#pragma unroll
        for (int g = 0; g < kG; ++g) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                tot += v[g][c];
                pre += (qq * kG + g) * 4 + c < t ? v[g][c] : 0;
            }
        }
        wpos[qq][d] = pre;
        wcnt[qq][d] = tot;
        __syncthreads();
        int x = 0;
        if (owner) {
            pre = wpos[0][tid] + wpos[1][tid] + wpos[2][tid] + wpos[3][tid];
            tot = wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
            x = tot;                       // inclusive prefix over digits
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int y = __shfl_up(x, off);
                if (lane >= off)
                    x += y;
            }
            if (lane == 63)
                wsum[w] = x;
        }
        __syncthreads();
        if (owner) {
            run = x - tot + pre;
            for (int v2 = 0; v2 < w; ++v2)
                run += wsum[v2];
        }
    }
#pragma unroll
    for (int i = 0; i < kWaves * kRadix / kScatterThreads; ++i)
        (&wcnt[0][0])[tid + i * kScatterThreads] = 0;
    __syncthreads();
    const uint64_t below = (uint64_t(1) << lane) - 1;
    int tag = 0;
    for (int rel0 = 0; rel0 < len; rel0 += kBatchRounds * kScatterThreads) {
        if (rel0 != 0)
            load_batch(rel0);
        ready_batch(rel0);
#pragma unroll
        for (int r = 0; r < kBatchRounds; ++r) {
            const int base = rel0 + r * kScatterThreads;
            if (base >= len)
                break;                         // uniform: the tile ends here
            ++tag;
            const bool valid = base + tid < len;
            const int key = bkey[r];
            const int d = (key >> shift) & mask;
            uint64_t same = __ballot(valid);
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                if ((mask >> b) == 0)
                    break;                     // uniform: no digit bit b
                const bool bit = (d >> b) & 1;
                const uint64_t m = __ballot(valid && bit);
                same &= bit ? m : ~m;
            }
            if (valid && (same >> lane) == 1)          // last lane of its group
                wcnt[w][d] = (tag << 8) | __popcll(same);
            __syncthreads();
            if (owner) {
#pragma unroll
                for (int v = 0; v < kWaves; ++v) {
                    const int e = wcnt[v][tid];
                    wpos[v][tid] = run;
                    run += (e >> 8) == tag ? (e & 255) : 0;
                }
            }
            __syncthreads();
            if (valid) {
                const int pos = wpos[w][d] + __popcll(same & below);
                keys_out[pos] = key;
                vals_out[pos] = bval[r];
            }
        }
    }
}

// ---- 2./3. per-cluster sums ----------------------------------------------

// V bf16 values of one row per lane (lane l holds columns l*V .. l*V+V-1).
template <int V>
struct RowBits {
    static_assert(V == 2 || V == 4 || V == 8, "two, four or eight columns per lane");
    uint32_t w[V / 2];
};

template <int V>
__device__ __forceinline__ RowBits<V> load_row(const uint16_t *p) {
    RowBits<V> r;
    if constexpr (V == 2) {
        r.w[0] = *reinterpret_cast<const uint32_t *>(p);
    } else if constexpr (V == 4) {
        typedef uint32_t w2 __attribute__((ext_vector_type(2)));
        const w2 v = *reinterpret_cast<const w2 *>(p);
        r.w[0] = v[0];
        r.w[1] = v[1];
    } else {
        typedef uint32_t w4 __attribute__((ext_vector_type(4)));
        const w4 v = *reinterpret_cast<const w4 *>(p);
        r.w[0] = v[0];
        r.w[1] = v[1];
        r.w[2] = v[2];
        r.w[3] = v[3];
    }
    return r;
}

template <int V>
__device__ __forceinline__ float row_value(const RowBits<V> &r, int v) {
    return (v & 1) ? __uint_as_float(r.w[v >> 1] & 0xffff0000u) : widen(r.w[v >> 1] & 0xffffu);
}

template <int V>
__device__ __forceinline__ void store_bits(uint16_t *p, const uint32_t (&b)[V]) {
    if constexpr (V == 2) {
        *reinterpret_cast<uint32_t *>(p) = b[0] | (b[1] << 16);
    } else if constexpr (V == 4) {
        typedef uint32_t w2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<w2 *>(p) = w2{b[0] | (b[1] << 16), b[2] | (b[3] << 16)};
    } else {
        typedef uint32_t w4 __attribute__((ext_vector_type(4)));
        *reinterpret_cast<w4 *>(p) = w4{b[0] | (b[1] << 16), b[2] | (b[3] << 16),
                                        b[4] | (b[5] << 16), b[6] | (b[7] << 16)};
    }
}

template <int V>
__device__ __forceinline__ void store_f32(float *p, const float (&f)[V]) {
#pragma unroll
    for (int v = 0; v < V; ++v)
        p[v] = f[v];
}

// Write the outputs of cluster k from its new row's bits: the row, its fp32
// mean (optional), its norm (via the wave's LDS row copy) and its count.
// Called by all 64 lanes of a wave together.
template <int V>
__device__ __forceinline__ void emit_cluster(int k, const uint32_t (&bits)[V], const float (&mean)[V],
                                             int count, int D, int lane, uint16_t *lds_row,
                                             uint16_t *__restrict__ C_new, float *__restrict__ means,
                                             float *__restrict__ norms, int32_t *__restrict__ counts) {
    const bool on = lane * V < D;
    const size_t row = static_cast<size_t>(k) * D + lane * V;
    if (on) {
        store_bits<V>(C_new + row, bits);
        if (means)
            store_f32<V>(means + row, mean);
#pragma unroll
        for (int v = 0; v < V; ++v)
            lds_row[lane * V + v] = static_cast<uint16_t>(bits[v]);
    }
    // The wave's own LDS writes are seen by its later LDS reads (LDS runs a
    // wave's operations in order); the barrier keeps the compiler from
    // moving the reads above the writes.
    __builtin_amdgcn_wave_barrier();
    const float n = row_sq_norm16(lds_row, D, lane & 15);
    if (lane == 0) {
        norms[k] = n;
        counts[k] = count;
    }
    __builtin_amdgcn_wave_barrier();
}

template <int V>
__device__ __forceinline__ void emit_mean(int k, const float (&sum)[V], int count, int D, int lane,
                                          uint16_t *lds_row, uint16_t *__restrict__ C_new,
                                          float *__restrict__ means, float *__restrict__ norms,
                                          int32_t *__restrict__ counts) {
    const float c = static_cast<float>(count);
    float mean[V];
    uint32_t bits[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        mean[v] = sum[v] / c;
        bits[v] = bf16_rne(mean[v]);
    }
    emit_cluster<V>(k, bits, mean, count, D, lane, lds_row, C_new, means, norms, counts);
}

template <int V>
__device__ __forceinline__ RowBits<V> lds_row_bits(const uint16_t *p) {
    RowBits<V> r;
    if constexpr (V == 2) {
        r.w[0] = *reinterpret_cast<const uint32_t *>(p);
    } else if constexpr (V == 4) {
        typedef uint32_t w2 __attribute__((ext_vector_type(2)));
        const w2 v = *reinterpret_cast<const w2 *>(p);
        r.w[0] = v[0];
        r.w[1] = v[1];
    } else {
        typedef uint32_t w4 __attribute__((ext_vector_type(4)));
        const w4 v = *reinterpret_cast<const w4 *>(p);
        r.w[0] = v[0];
        r.w[1] = v[1];
        r.w[2] = v[2];
        r.w[3] = v[3];
    }
    return r;
}

// Chunks of P sorted positions; workgroup b takes chunks b, b + G, ... (G
// workgroups, four per CU).  A chunk's keys, point indices and rows are
// staged in LDS (all row loads of a chunk in flight at once), then each
// wave takes every fourth run of equal keys (in position order: runs w, w +
// 4, ... go to wave w) and sums each run's rows from LDS in position
// order.  Loads run ahead of the sums: while chunk c is summed, the rows of
// the next chunk are on their way into registers and the keys of the one
// after into registers too.
//
// For a run [a, b) of cluster k: a is k's first position unless the run
// starts the chunk and the position before holds k too; b is its end unless
// the run ends the chunk and the position after holds k too.  A run that is
// the whole cluster is finished here; otherwise its sum goes to partial slot
// 0 (the run began before this chunk) or 1 (it began here and continues).
template <int V>
__global__ __launch_bounds__(kReduceThreads, 4)
void upd_reduce_kernel(const uint16_t *__restrict__ X, const int32_t *__restrict__ keys,
                       const int32_t *__restrict__ vals, int N, int D, int K, int P, int chunks,
                       int cpr_inv, int32_t *__restrict__ start, int32_t *__restrict__ end,
                       float *__restrict__ partial, uint16_t *__restrict__ C_new,
                       float *__restrict__ means, float *__restrict__ norms,
                       int32_t *__restrict__ counts) {
    typedef uint32_t w4 __attribute__((ext_vector_type(4)));
    constexpr int kKeysPerThread = (kMaxChunk + kReduceThreads - 1) / kReduceThreads;
    __shared__ __attribute__((aligned(16))) uint16_t rows[kStageBytes / 2];
    __shared__ int skey[2][kMaxChunk];
    __shared__ int sval[2][kMaxChunk];
    __shared__ int edge[2][2];
    __shared__ __attribute__((aligned(16))) uint16_t nrow[kReduceThreads / 64][kMaxRow];
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int G = gridDim.x;
    const int cpr = D >> 3;
    const bool on = lane * V < D;
    uint16_t *lds_row = nrow[wave];

    int kr[kKeysPerThread], vr[kKeysPerThread], er[2] = {-1, -1};
    auto load_keys = [&](int c) __attribute__((always_inline)) {
        const int c0 = c * P;
        const int n = min(N - c0, P);
#pragma unroll
        for (int u = 0; u < kKeysPerThread; ++u) {
            const int j = tid + u * kReduceThreads;
            kr[u] = j < n ? keys[c0 + j] : 0;
            vr[u] = j < n ? vals[c0 + j] : 0;
        }
        if (tid == 0) {
            er[0] = c0 > 0 ? keys[c0 - 1] : -1;
            er[1] = c0 + n < N ? keys[c0 + n] : -1;
        }
    };
    auto store_keys = [&](int b, int c) __attribute__((always_inline)) {
        const int n = min(N - c * P, P);
#pragma unroll
        for (int u = 0; u < kKeysPerThread; ++u) {
            const int j = tid + u * kReduceThreads;
            if (j < n) {
                skey[b][j] = kr[u];
                sval[b][j] = vr[u];
            }
        }
        if (tid == 0) {
            edge[b][0] = er[0];
            edge[b][1] = er[1];
        }
    };
    // 16-byte piece q of a chunk is column (q % cpr) * 8 of its row q / cpr
    // (q / cpr as (q * cpr_inv) >> 20, exact for q < 4096 and cpr <= 64).
    // Rows of stray labels are staged too (they are point rows all the
    // same) and never read.
    w4 buf[kStagePieces];
    auto load_rows = [&](int b, int c) __attribute__((always_inline)) {
        const int pieces = min(N - c * P, P) * cpr;
#pragma unroll
        for (int i = 0; i < kStagePieces; ++i) {
            const int q = tid + i * kReduceThreads;
            buf[i] = w4{0u, 0u, 0u, 0u};
            if (q < pieces) {
                const int r = (q * cpr_inv) >> 20;
                buf[i] = *reinterpret_cast<const w4 *>(X + static_cast<size_t>(sval[b][r]) * D +
                                                       (q - r * cpr) * 8);
            }
        }
    };
    auto store_rows = [&](int c) __attribute__((always_inline)) {
        const int pieces = min(N - c * P, P) * cpr;
#pragma unroll
        for (int i = 0; i < kStagePieces; ++i) {
            const int q = tid + i * kReduceThreads;
            if (q < pieces)
                *reinterpret_cast<w4 *>(rows + q * 8) = buf[i];
        }
    };

    int c = blockIdx.x;
    if (c >= chunks)
        return;
    load_keys(c);
    store_keys(0, c);
    __syncthreads();
    if (c + G < chunks)
        load_keys(c + G);
    load_rows(0, c);
    for (int b = 0; c < chunks; c += G, b ^= 1) {
        const int cn = c + G;
        store_rows(c);
        if (cn < chunks)
            store_keys(b ^ 1, cn);
        __syncthreads();
        if (cn + G < chunks)
            load_keys(cn + G);
        if (cn < chunks)
            load_rows(b ^ 1, cn);

        const int c0 = c * P;
        const int n = min(N - c0, P);
        const int *sk = skey[b];
        // Every wave walks all run starts of the chunk in order and takes
        // runs 0, 4, 8, ... (wave 0), 1, 5, ... (wave 1) and so on.
        static_assert(((kReduceThreads / 64) & (kReduceThreads / 64 - 1)) == 0,
                      "wave count must be a power of two");
        int run = 0;
        for (int base = 0; base < n; base += 64) {
            const int j = base + lane;
            const int kj = j < n ? sk[j] : K;
            uint64_t starts = __ballot(j < n && kj < K && (j == 0 || sk[j - 1] != kj));
            while (starts) {
                const int a = base + __builtin_ctzll(starts);
                starts &= starts - 1;
                if ((run++ & (kReduceThreads / 64 - 1)) != wave)
                    continue;
                const int k = __builtin_amdgcn_readfirstlane(sk[a]);
                int e = n;
                for (int base = a + 1; base < n; base += 64) {
                    const int q = base + lane;
                    const uint64_t diff = __ballot(q < n && sk[q] != k);
                    if (diff) {
                        e = base + __builtin_ctzll(diff);
                        break;
                    }
                }
                float acc[V];
#pragma unroll
                for (int v = 0; v < V; ++v)
                    acc[v] = 0.0f;
                if (on) {
                    const uint16_t *src = rows + lane * V;
#pragma unroll 8
                    for (int p = a; p < e; ++p) {
                        const RowBits<V> r = lds_row_bits<V>(src + p * D);
#pragma unroll
                        for (int v = 0; v < V; ++v)
                            acc[v] += row_value<V>(r, v);
                    }
                }
                const bool before = a == 0 && edge[b][0] == k;
                const bool after = e == n && edge[b][1] == k;
                if (lane == 0) {
                    if (!before)
                        start[k] = c0 + a;
                    if (!after)
                        end[k] = c0 + e;
                }
                if (!before && !after) {
                    emit_mean<V>(k, acc, e - a, D, lane, lds_row, C_new, means, norms, counts);
                } else if (on) {
                    float *dst = partial + (static_cast<size_t>(c) * 2 + (before ? 0 : 1)) * D +
                                 lane * V;
                    store_f32<V>(dst, acc);
                }
            }
        }
        __syncthreads();
    }
}

// Clusters the reduce kernel did not finish: empty ones (old row kept) and
// those spanning several chunks (partials added in chunk order).
template <int V>
__global__ __launch_bounds__(kReduceThreads)
void upd_finish_kernel(const uint16_t *__restrict__ C_old, const int32_t *__restrict__ start,
                       const int32_t *__restrict__ end, const float *__restrict__ partial,
                       int N, int D, int K, int P, uint16_t *__restrict__ C_new,
                       float *__restrict__ means, float *__restrict__ norms,
                       int32_t *__restrict__ counts) {
    __shared__ __attribute__((aligned(16))) uint16_t nrow[kReduceThreads / 64][kMaxRow];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const bool on = lane * V < D;
    uint16_t *lds_row = nrow[wave];
    const int64_t nwaves = static_cast<int64_t>(gridDim.x) * (kReduceThreads / 64);
    // 64-bit stride: K may lie within one stride of 2^31.
    for (int64_t kk = static_cast<int64_t>(blockIdx.x) * (kReduceThreads / 64) + wave; kk < K;
         kk += nwaves) {
        const int k = static_cast<int>(kk);
        const int s = N > 0 ? start[k] : 0;
        const int e = N > 0 ? end[k] : 0;
        const int count = e - s;
        if (count == 0) {
            uint32_t bits[V];
            float mean[V];
            RowBits<V> r = on ? load_row<V>(C_old + static_cast<size_t>(k) * D + lane * V)
                              : RowBits<V>{};
#pragma unroll
            for (int v = 0; v < V; ++v) {
                mean[v] = row_value<V>(r, v);
                bits[v] = __float_as_uint(mean[v]) >> 16;
            }
            emit_cluster<V>(k, bits, mean, 0, D, lane, lds_row, C_new, means, norms, counts);
            continue;
        }
        const int cf = s / P;
        const int cl = (e - 1) / P;
        if (cf == cl)
            continue;                   // finished by the reduce kernel
        float sum[V];
        const float *pf = partial + (static_cast<size_t>(cf) * 2 + 1) * D + lane * V;
#pragma unroll
        for (int v = 0; v < V; ++v)
            sum[v] = on ? pf[v] : 0.0f;
        for (int c = cf + 1; c <= cl; ++c) {
            const float *pc = partial + static_cast<size_t>(c) * 2 * D + lane * V;
#pragma unroll
            for (int v = 0; v < V; ++v)
                sum[v] += on ? pc[v] : 0.0f;
        }
        emit_mean<V>(k, sum, count, D, lane, lds_row, C_new, means, norms, counts);
    }
}

// ---- 4. bucket path: a tile-local sort and one workgroup per bucket ------
//
// For K up to 16384 and N up to 2^24 (the common Lloyd shapes), two launches
// replace the radix passes, the reduce and the finish kernels.  Clusters are
// grouped into nb <= 1024 buckets of S = 2^s <= 16 clusters (bucket k >> s).
//
//  a. upd_bin_kernel: every tile of 2^tl points sorts its own points by
//     bucket, stably (index order inside a bucket), and records where each
//     bucket starts in the tile (dir[tile][bucket]).  No global offsets: a
//     bucket's points are the concatenation, over tiles in order, of one
//     segment per tile, which is already index order.
//  b. upd_bucket_kernel: one workgroup per bucket gathers those segments'
//     slot words (point index, cluster in bucket) in tile order into LDS and
//     walks them in chunks of 512 slots; each of its four waves sums a fixed
//     quarter of every chunk's slots in order into per-cluster registers, the
//     four partials are added in wave order, and the workgroup finishes its S
//     clusters (empty ones keep their rows).  Buckets of 8 or 16 clusters
//     take upd_bucket_runs_kernel instead, which sorts the words by cluster
//     first.  The order of every sum depends only on the data, so a call
//     gives the same bits every time.
//
// A bucket is summed by one workgroup, so a bucket holding a large share of
// all points runs on one CU (correct, but far slower than the radix path,
// whose reduce spreads any cluster over fixed chunks).

constexpr int kBinWaves = 8;         // each owns a contiguous eighth of the tile
constexpr int kBinThreads = 64 * kBinWaves;
constexpr int kMinBinTileLog2 = 10;
constexpr int kMaxBuckets = 1024;
constexpr int kScanThreads2 = 256;   // threads of the bin scan: 4 buckets each
constexpr int kBinDigitsPerThread = kMaxBuckets / kScanThreads2;   // one 16-byte group
constexpr int kMaxBinTiles = 512;
constexpr int64_t kMaxBinPoints = int64_t(1) << 24;
constexpr int kMaxBucketLog2 = 4;    // S <= 16
constexpr int64_t kMaxBinClusters = int64_t(kMaxBuckets) << kMaxBucketLog2;
constexpr int kBucketThreads = 256;  // 4 waves
constexpr int kBucketWaves = kBucketThreads / 64;
constexpr int kBucketChunk = 512;    // slots summed per round
constexpr int kBucketSlots = 2048;   // a bucket up to this size has all its slot words in LDS
constexpr int kSlotIdxBits = 24;     // a slot word: point index | cluster in bucket << 24
static_assert(kMaxBinPoints <= (int64_t(1) << kSlotIdxBits), "point indices fit the slot word");
static_assert(kSlotIdxBits + kMaxBucketLog2 <= 31, "the cluster in its bucket fits the slot word");


// Tile t: positions [t << tl, min(N, (t + 1) << tl)).  Wave w owns the
// contiguous eighth [w q, (w + 1) q) of the tile (q = 2^tl / 8), so the
// stable order is: bucket, then wave, then position inside the wave.
//  1. per-wave bucket counts (LDS atomics on the wave's own row; stray
//     labels are not counted);
//  2. one exclusive scan over (bucket, wave), bucket-major: cnt[w][d]
//     becomes the first slot of (w, d), and dir[t][d] the first slot of
//     bucket d, dir[t][nb] the number of points with a real label.  Thread
//     r < 256 owns buckets 4r .. 4r + 3 (one 16-byte group per row);
//  3. each wave ranks its points 64 at a time in position order: lanes with
//     the same bucket are found with one ballot per bucket bit, a lane's
//     slot is the running slot of its bucket plus the earlier such lanes, and
//     the group's last lane advances the running slot.  Every point with a
//     real label writes one word at its slot: its index (below 2^24) in the
//     low 24 bits, its cluster within the bucket (label mod S) above them.
// Labels are loaded eight chunks (512 points) per wave at a time, all in
// flight together (unconditional loads clamped to the wave's last point,
// taken by an empty asm); a wave holding one batch (tiles up to 4096) keeps
// it in registers from the counts to the ranks.
__global__ __launch_bounds__(kBinThreads)
void upd_bin_kernel(const int32_t *__restrict__ labels, int N, int K, int s_log2, int nb,
                    int tl, int32_t *__restrict__ sidx, int32_t *__restrict__ dir) {
    typedef int32_t i4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(16))) int cnt[kBinWaves * kMaxBuckets];
    __shared__ int wtot[kBinWaves];
    constexpr int kBatch = 8;
    constexpr int NR = kMaxBuckets;                // row length of cnt
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int t = blockIdx.x;
    const int beg = t << tl;                       // N <= 2^24: no overflow
    const int len = min(N - beg, 1 << tl);
    const int q = (1 << tl) / kBinWaves;
    const int wb = min(len, w * q);
    const int we = min(len, wb + q);
    i4 *cv = reinterpret_cast<i4 *>(cnt);
#pragma unroll
    for (int i = tid; i < kBinWaves * NR / 4; i += kBinThreads)
        cv[i] = i4{0, 0, 0, 0};
    int v[kBatch];
    auto load_batch = [&](int i0) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            v[u] = labels[beg + min(i0 + u * 64 + lane, we - 1)];
#if defined(__HIP_DEVICE_COMPILE__)
        static_assert(kBatch == 8, "the asm below names eight values");
        asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]),
                          "+v"(v[5]), "+v"(v[6]), "+v"(v[7]));
#endif
    };
    // Bucket of a label, nb for a stray one.
    auto bucket = [&](int32_t l) __attribute__((always_inline)) {
        return (l < 0 || l >= K) ? nb : (l >> s_log2);
    };
    const bool one_batch = we - wb <= kBatch * 64;
    if (wb < we)
        load_batch(wb);
    __syncthreads();                               // cnt cleared
    int *mine = cnt + w * NR;

    // 1. Counts.
    for (int i0 = wb; i0 < we; i0 += kBatch * 64) {
        if (i0 != wb)
            load_batch(i0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int d = bucket(v[u]);
            if (i0 + u * 64 + lane < we && d < nb)
                atomicAdd(&mine[d], 1);
        }
    }
    __syncthreads();

    // 2. Scan: the first 256 threads own 4 buckets each (whole waves, so the
    // shuffles below see full waves); every wave reaches both barriers.
    {
        const bool scanner = tid < kScanThreads2;
        i4 c[kBinWaves];
        int tot[kBinDigitsPerThread];
        int sum = 0;
        if (scanner) {
#pragma unroll
            for (int r = 0; r < kBinWaves; ++r)
                c[r] = cv[r * (NR / 4) + tid];
#pragma unroll
            for (int j = 0; j < kBinDigitsPerThread; ++j) {
                tot[j] = 0;
#pragma unroll
                for (int r = 0; r < kBinWaves; ++r)
                    tot[j] += c[r][j];
                sum += tot[j];
            }
        }
        const int x = wave_inclusive_sum(sum);
        if (lane == 63)
            wtot[w] = x;
        __syncthreads();
        if (scanner) {
            int ex = x - sum;
            for (int v2 = 0; v2 < w; ++v2)
                ex += wtot[v2];
            int32_t *drow = dir + static_cast<size_t>(t) * (nb + 1);
            i4 o[kBinWaves];
#pragma unroll
            for (int j = 0; j < kBinDigitsPerThread; ++j) {
                const int d = tid * kBinDigitsPerThread + j;
                if (d <= nb)
                    drow[d] = ex;
                int run = ex;
#pragma unroll
                for (int r = 0; r < kBinWaves; ++r) {
                    o[r][j] = run;
                    run += c[r][j];
                }
                ex += tot[j];
            }
            if (tid == kScanThreads2 - 1 && nb == kMaxBuckets)
                drow[nb] = ex;                     // the total (no owner at index 1024)
#pragma unroll
            for (int r = 0; r < kBinWaves; ++r)
                cv[r * (NR / 4) + tid] = o[r];
        }
    }
    __syncthreads();

    // 3. Ranks and placement.  Every lane of the wave reads its bucket's
    // running slot before the group's last lane writes it back (LDS runs a
    // wave's operations in order, and the leader's own read precedes its
    // write in program order).
    const uint64_t below = (uint64_t(1) << lane) - 1;
    const int nbits = 32 - __clz(nb);              // buckets 0..nb
    for (int i0 = wb; i0 < we; i0 += kBatch * 64) {
        if (!one_batch)
            load_batch(i0);
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int c0 = i0 + u * 64;
            if (c0 >= we)
                break;                             // uniform
            const int i = c0 + lane;
            const int d = bucket(v[u]);
            const bool valid = i < we && d < nb;
            uint64_t same = __ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = (d >> b) & 1;
                const uint64_t m = __ballot(valid && bit);
                same &= bit ? m : ~m;
            }
            if (valid) {
                const int pos = mine[d] + __popcll(same & below);
                if ((same >> lane) == 1)           // last lane of its group
                    mine[d] = pos + 1;
                sidx[beg + pos] = (beg + i) | ((v[u] & ((1 << s_log2) - 1)) << kSlotIdxBits);
            }
        }
    }
}

// Workgroups are dispatched to the eight XCDs in turn (workgroup i to XCD
// i mod 8), and each XCD has its own L2.  Mapping workgroup i to item
// start(x) + i / 8 (x = i mod 8, XCD x owning the contiguous items
// [start(x), start(x + 1))) gives each XCD a contiguous range of buckets, so
// the directory lines and sorted-index lines it reads are its own eighth of
// them instead of lines shared with every other XCD.  A bijection on
// [0, n) for any n.
__device__ __forceinline__ int xcd_contiguous(int i, int n) {
    constexpr int kXcds = 8;
    const int x = i % kXcds;
    const int q = n / kXcds;
    const int r = n % kXcds;
    return x * q + min(x, r) + i / kXcds;
}

// Bucket b's slot words (point index, cluster in bucket) in slot order,
// i.e. tile order, for a workgroup of kBucketThreads threads; every thread
// calls it.  A bucket of at most kBucketSlots points gets all its words in
// ci; a larger one gets off[0..T] (first slot of each tile's segment) and
// src[0..T) (its first sorted position) for chunk_words.  Ends with a
// barrier.
struct SlotWords {
    int n_pts;     // points in the bucket
    bool whole;    // all their words are in ci (the same on every thread)
};

__device__ __forceinline__ SlotWords gather_slot_words(const int32_t *__restrict__ sidx,
                                                       const int32_t *__restrict__ dir, int N,
                                                       int nb, int T, int tl, int b, int *ci,
                                                       int (*wtot)[kBucketWaves], int *off,
                                                       int *src) {
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int ND = nb + 1;
    // Thread r owns tiles r and r + 256 (T <= 512), so that
    // every wave holds tiles when T <= 256; the directory loads are
    // unconditional (clamped to tile T - 1) so they are in flight together,
    // and each takes a tile's two adjacent entries at once (8 bytes, 4-byte
    // aligned, which global loads allow).  The thread's own points (its two
    // segments) are then loaded kPre at a time, so that their latency
    // overlaps the scan; once the scan gives each segment its first slot
    // they are placed in ci (when the whole bucket fits there).  Slots run in
    // tile order: tiles 0..255 first, then 256..511, so the two halves are
    // scanned side by side and the second is offset by the first's total.
    typedef int32_t i2 __attribute__((ext_vector_type(2)));
    constexpr int kTilesPerThread = kMaxBinTiles / kBucketThreads;
    static_assert(kTilesPerThread == 2, "two segments per thread");
    constexpr int kPre = 8;
    int seg[kTilesPerThread] = {0, 0}, base[kTilesPerThread];
    int wv[kPre];
    // Sorted position of this thread's p-th point, p < seg[0] + seg[1].
    auto word_pos = [&](int p) __attribute__((always_inline)) {
        return p < seg[0] ? base[0] + p : base[1] + (p - seg[0]);
    };
    // Position read by a lane without a p-th point, the same on every lane
    // of the wave (so a load costs one line request per real point plus at
    // most one): the first point of the wave's lowest lane that has one, a
    // line the wave reads anyway; in a wave with no points, a position that
    // differs by wave and bucket, so that no one line is read by all waves.
    int stand_in = 0;
    if (T > 0) {
#pragma unroll
        for (int u = 0; u < kTilesPerThread; ++u) {
            const int tt = min(tid + u * kBucketThreads, T - 1);
            i2 pr;
            __builtin_memcpy(&pr, dir + static_cast<size_t>(tt) * ND + b, sizeof(pr));
            seg[u] = tid + u * kBucketThreads < T ? pr.y - pr.x : 0;
            base[u] = (tt << tl) + pr.x;
        }
        // Unconditional loads (no branch to wait in).
        const int sum = seg[0] + seg[1];
        const uint64_t have = __ballot(sum > 0);
        stand_in = have != 0 ? __builtin_amdgcn_readlane(word_pos(0), __builtin_ctzll(have))
                             : min(b * 64 + w * 16, N - 1);
#pragma unroll
        for (int p = 0; p < kPre; ++p)
            wv[p] = sidx[p < sum ? word_pos(p) : stand_in];
    }
    const int sum = seg[0] + seg[1];
    const int x[kTilesPerThread] = {wave_inclusive_sum(seg[0]), wave_inclusive_sum(seg[1])};
    if (lane == 63) {
        wtot[0][w] = x[0];
        wtot[1][w] = x[1];
    }
    __syncthreads();
    int ex[kTilesPerThread], tot[kTilesPerThread];
#pragma unroll
    for (int u = 0; u < kTilesPerThread; ++u) {
        ex[u] = x[u] - seg[u];
        tot[u] = 0;
#pragma unroll
        for (int v2 = 0; v2 < kBucketWaves; ++v2) {
            ex[u] += v2 < w ? wtot[u][v2] : 0;
            tot[u] += wtot[u][v2];
        }
    }
    ex[1] += tot[0];
    const int n_pts = tot[0] + tot[1];
    // Slot of this thread's p-th point.
    auto slot_of = [&](int p) __attribute__((always_inline)) {
        return p < seg[0] ? ex[0] + p : ex[1] + (p - seg[0]);
    };
    // Same for every thread of the workgroup (so are the barriers below that
    // depend on it): the bucket's slot words all fit in ci.
    const bool whole = n_pts <= kBucketSlots;
    if (whole) {
#pragma unroll
        for (int p = 0; p < kPre; ++p)
            if (p < sum)
                ci[slot_of(p)] = wv[p];
        for (int p0 = kPre; p0 < sum; p0 += kPre) {    // a thread with more points
            int more[kPre];
#pragma unroll
            for (int p = 0; p < kPre; ++p)
                more[p] = sidx[p0 + p < sum ? word_pos(p0 + p) : stand_in];
#pragma unroll
            for (int p = 0; p < kPre; ++p)
                if (p0 + p < sum)
                    ci[slot_of(p0 + p)] = more[p];
        }
    } else {
        // Larger buckets resolve one chunk of slots at a time below: each
        // slot finds its tile by binary search over the segments' first slots.
#pragma unroll
        for (int u = 0; u < kTilesPerThread; ++u) {
            const int tt = tid + u * kBucketThreads;
            if (tt < T) {
                off[tt] = ex[u];
                src[tt] = base[u];
            }
        }
        if (tid == 0)
            off[T] = n_pts;
    }
    __syncthreads();
    return SlotWords{n_pts, whole};
}

// Words of slots [c0, c0 + nc) of a gathered bucket: in place in ci when the
// whole bucket is there, else resolved into ci[0, nc) (each slot finds its
// tile by binary search over the segments' first slots).  Every thread
// calls it; the second case ends with a barrier, and the caller must reach
// one more before ci is resolved again.
__device__ __forceinline__ const int *chunk_words(const SlotWords &sw, int c0, int nc, int T,
                                                  const int *off, const int *src,
                                                  const int32_t *__restrict__ sidx, int *ci) {
    if (sw.whole)
        return ci + c0;
    constexpr int kSlotsPerThread = kBucketChunk / kBucketThreads;
    const int tid = threadIdx.x;
    int sp[kSlotsPerThread];
#pragma unroll
    for (int u = 0; u < kSlotsPerThread; ++u) {
        const int slot = c0 + min(tid + u * kBucketThreads, nc - 1);
        int lo = 0, hi = T - 1;                    // last tile whose segment starts <= slot
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (off[mid] <= slot)
                lo = mid;
            else
                hi = mid - 1;
        }
        sp[u] = src[lo] + (slot - off[lo]);
    }
    int li[kSlotsPerThread];
#pragma unroll
    for (int u = 0; u < kSlotsPerThread; ++u)
        li[u] = sidx[sp[u]];
#pragma unroll
    for (int u = 0; u < kSlotsPerThread; ++u) {
        const int j = tid + u * kBucketThreads;
        if (j < nc)
            ci[j] = li[u];
    }
    __syncthreads();
    return ci;
}

// One workgroup per bucket b (clusters b S .. b S + S - 1).  Dynamic LDS:
// the four waves' S x D partial sums, then, for a bucket of more than 2048
// points, off[T + 1] (first slot of each tile's segment) and src[T] (its
// first sorted position).
template <int V, int S>
__global__ __launch_bounds__(kBucketThreads)
void upd_bucket_kernel(const uint16_t *__restrict__ X, const int32_t *__restrict__ sidx,
                       const int32_t *__restrict__ dir,
                       const uint16_t *__restrict__ C_old, int N, int D, int K, int nb, int T,
                       int tl,
                       uint16_t *__restrict__ C_new, float *__restrict__ means,
                       float *__restrict__ norms, int32_t *__restrict__ counts) {
    extern __shared__ __attribute__((aligned(16))) int bdyn[];
    __shared__ int ci[kBucketSlots];
    __shared__ int wtot[2][kBucketWaves];
    __shared__ int bcnt[kBucketWaves][S];
    __shared__ __attribute__((aligned(16))) uint16_t nrow[kBucketWaves][kMaxRow];
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int b = xcd_contiguous(blockIdx.x, nb);
    const bool on = lane * V < D;
    const int col = on ? lane * V : 0;             // idle lanes load column 0
    float *part = reinterpret_cast<float *>(bdyn);         // [4][S][D]
    int *off = bdyn + kBucketWaves * S * D;                // [T + 1]
    int *src = off + T + 1;                                // [T]

    // 1. The bucket's slot words.
    const SlotWords sw = gather_slot_words(sidx, dir, N, nb, T, tl, b, ci, wtot, off, src);
    const int n_pts = sw.n_pts;

    // 2. Sums, over chunks of 512 slots.  A wave takes kRows slots at a
    // time: lane u reads slot u's word (point index, cluster) from LDS, the
    // row loads take them by readlane as scalar bases, all kRows loads in
    // flight together.
    constexpr int kRows = V == 2 ? 32 : (V == 4 ? 16 : 8);
    float acc[S][V];
    int cw[S];
#pragma unroll
    for (int c = 0; c < S; ++c) {
        cw[c] = 0;
#pragma unroll
        for (int v = 0; v < V; ++v)
            acc[c][v] = 0.0f;
    }
    for (int c0 = 0; c0 < n_pts; c0 += kBucketChunk) {
        const int nc = min(kBucketChunk, n_pts - c0);
        const int *words = chunk_words(sw, c0, nc, T, off, src, sidx, ci);
        const int j0 = nc * w / kBucketWaves;
        const int j1 = nc * (w + 1) / kBucketWaves;
        for (int jb = j0; jb < j1; jb += kRows) {
            const int jj = min(jb + (kRows == 64 ? lane : lane % kRows), j1 - 1);
            const int word = words[jj];
            const int my_i = word & ((1 << kSlotIdxBits) - 1);
            const int my_c = S > 1 ? word >> kSlotIdxBits : 0;
            RowBits<V> r[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                const int i = __builtin_amdgcn_readlane(my_i, u);
                r[u] = load_row<V>(X + static_cast<size_t>(i) * D + col);
            }
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                if (jb + u < j1) {                 // uniform
                    const int c = S > 1 ? __builtin_amdgcn_readlane(my_c, u) : 0;
#pragma unroll
                    for (int cc = 0; cc < S; ++cc) {
                        if (S == 1 || c == cc) {
                            ++cw[cc];
#pragma unroll
                            for (int v = 0; v < V; ++v)
                                acc[cc][v] += row_value<V>(r[u], v);
                        }
                    }
                }
            }
        }
        if (!sw.whole)
            __syncthreads();                       // ci is refilled for the next chunk
    }

    // 3. Partials of the four waves to LDS; cluster c's sum adds them in
    // wave order.
#pragma unroll
    for (int c = 0; c < S; ++c) {
        if (on) {
#pragma unroll
            for (int v = 0; v < V; ++v)
                part[(w * S + c) * D + lane * V + v] = acc[c][v];
        }
        if (lane == 0)
            bcnt[w][c] = cw[c];
    }
    __syncthreads();

    // 4. Outputs: wave w finishes clusters b S + w, b S + w + 4, ...
    for (int c = w; c < S; c += kBucketWaves) {
        const int64_t kk = static_cast<int64_t>(b) * S + c;
        if (kk >= K)
            break;
        const int k = static_cast<int>(kk);
        const int count = bcnt[0][c] + bcnt[1][c] + bcnt[2][c] + bcnt[3][c];
        if (count == 0) {
            uint32_t bits[V];
            float mean[V];
            RowBits<V> r = on ? load_row<V>(C_old + static_cast<size_t>(k) * D + lane * V)
                              : RowBits<V>{};
#pragma unroll
            for (int v = 0; v < V; ++v) {
                mean[v] = row_value<V>(r, v);
                bits[v] = __float_as_uint(mean[v]) >> 16;
            }
            emit_cluster<V>(k, bits, mean, 0, D, lane, nrow[w], C_new, means, norms, counts);
        } else {
            float s2[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                s2[v] = 0.0f;
                if (on) {
                    const int e = c * D + lane * V + v;
                    s2[v] = ((part[e] + part[S * D + e]) + part[2 * S * D + e]) +
                            part[3 * S * D + e];
                }
            }
            emit_mean<V>(k, s2, count, D, lane, nrow[w], C_new, means, norms, counts);
        }
    }
}

// Buckets of S = 8 or 16 clusters (K up to 16384).  Choosing each row's
// cluster among S register accumulators would cost an S-way choice per row,
// so the bucket's slot words are first sorted by cluster in LDS (stably, so
// a cluster's slots keep index order; a bucket of more than 2048 points
// chunk by chunk, 512 slots at a time) and each wave walks a fixed quarter
// of the sorted piece with one accumulator, closing a run when the cluster
// changes.  A run inside the wave's quarter goes straight to its cluster's
// LDS sum (no other wave has that cluster in the piece); the quarter's first
// and last runs, which may continue in the neighbouring quarters, go to
// edge rows that wave 0 adds in slot order once all waves are done.  A
// cluster's sum is thus its run pieces added left to right in slot order,
// piece after piece, each summed in index order: the same bits on every
// call, whatever the cluster sizes.  Dynamic LDS: the S x D sums, the 4 x 2
// x D edge rows, then, for a bucket of more than 2048 points, off[T + 1]
// and src[T] (as in upd_bucket_kernel).
template <int V, int S>
__global__ __launch_bounds__(kBucketThreads)
__attribute__((amdgpu_waves_per_eu(kBucketWaves, kBucketWaves)))   // four workgroups per CU
void upd_bucket_runs_kernel(const uint16_t *__restrict__ X, const int32_t *__restrict__ sidx,
                            const int32_t *__restrict__ dir, const uint16_t *__restrict__ C_old,
                            int N, int D, int K, int nb, int T, int tl,
                            uint16_t *__restrict__ C_new, float *__restrict__ means,
                            float *__restrict__ norms, int32_t *__restrict__ counts) {
    static_assert(S == 8 || S == 16, "buckets of eight or sixteen clusters");
    constexpr int kKeyBits = S == 8 ? 3 : 4;
    constexpr int kWordsPerThread = kBucketSlots / kBucketThreads;
    constexpr int kGroups = kWordsPerThread * kBucketWaves;   // 64-slot groups of a sort
    constexpr int kRows = V == 2 ? 32 : (V == 4 ? 16 : 8);
    extern __shared__ __attribute__((aligned(16))) int bdyn[];
    __shared__ int ci[kBucketSlots];
    __shared__ int sorted[kBucketSlots];
    __shared__ int wtot[2][kBucketWaves];
    __shared__ int grp[kGroups][S];                // per (group, key): count, then first position
    __shared__ int ccount[S];                      // points of each cluster, all chunks
    __shared__ int edge_c[kBucketWaves][2];        // cluster of each edge row, -1 if none
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int b = xcd_contiguous(blockIdx.x, nb);
    const bool on = lane * V < D;
    const int col = on ? lane * V : 0;             // idle lanes load column 0
    float *sums = reinterpret_cast<float *>(bdyn);         // [S][D]
    float *edge = sums + S * D;                            // [4][2][D]
    // The outputs' row copies (one row of D bf16 per wave) reuse the edge
    // rows, which are done with by then.
    uint16_t *nrow = reinterpret_cast<uint16_t *>(edge);
    int *off = bdyn + (S + 2 * kBucketWaves) * D;          // [T + 1]
    int *src = off + T + 1;                                // [T]
    // Cleared here; the barrier that ends the gather orders this before use.
    for (int i = tid; i < S * D; i += kBucketThreads)
        sums[i] = 0.0f;
    if (tid < S)
        ccount[tid] = 0;

    // 1. The bucket's slot words.
    const SlotWords sw = gather_slot_words(sidx, dir, N, nb, T, tl, b, ci, wtot, off, src);

    const uint64_t below = (uint64_t(1) << lane) - 1;
    // A bucket whose words are all in ci is sorted and summed in one piece;
    // a larger one in chunks of 512 slots.
    const int piece = sw.whole ? max(sw.n_pts, 1) : kBucketChunk;
    for (int c0 = 0; c0 < sw.n_pts; c0 += piece) {
        const int nc = min(piece, sw.n_pts - c0);
        const int *words = chunk_words(sw, c0, nc, T, off, src, sidx, ci);

        // 2. Stable counting sort of the piece by key (the cluster in the
        // bucket).  Slot u * 256 + tid lies in group u * 4 + w, groups in
        // slot order; inside a group a slot's rank among its key's slots
        // comes from one ballot per key bit, and the key's last lane
        // records the group's count.
        const int ng = (nc + 63) / 64;             // groups holding slots
        for (int i = tid; i < ng * S; i += kBucketThreads)
            (&grp[0][0])[i] = 0;
        __syncthreads();
        // Key of a slot word: its cluster in the bucket.
        auto key_of = [](int word) __attribute__((always_inline)) {
            return static_cast<int>(static_cast<uint32_t>(word) >> kSlotIdxBits);
        };
        int wd[kWordsPerThread], rank[kWordsPerThread];
#pragma unroll
        for (int u = 0; u < kWordsPerThread; ++u) {
            if (u * kBucketThreads >= nc)
                break;                             // uniform
            const int j = u * kBucketThreads + tid;
            const bool valid = j < nc;
            wd[u] = valid ? words[j] : 0;
            const int key = key_of(wd[u]);
            uint64_t same = __ballot(valid);
#pragma unroll
            for (int bit = 0; bit < kKeyBits; ++bit) {
                const bool one = (key >> bit) & 1;
                const uint64_t m = __ballot(valid && one);
                same &= one ? m : ~m;
            }
            rank[u] = __popcll(same & below);
            if (valid && (same >> lane) == 1)
                grp[u * kBucketWaves + w][key] = rank[u] + 1;
        }
        __syncthreads();
        // Exclusive scan over (key, group), key-major: lane k of wave 0 owns
        // key (cluster) k; the piece's cluster counts are added to the
        // totals.
        if (w == 0) {
            int t = 0;
            if (lane < S)
                for (int g = 0; g < ng; ++g)
                    t += grp[g][lane];
            const int x = wave_inclusive_sum(t);
            if (lane < S) {
                int st = x - t;
                for (int g = 0; g < ng; ++g) {
                    const int cnt = grp[g][lane];
                    grp[g][lane] = st;
                    st += cnt;
                }
                ccount[lane] += t;
            }
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kWordsPerThread; ++u) {
            if (u * kBucketThreads >= nc)
                break;                             // uniform
            if (u * kBucketThreads + tid < nc)
                sorted[grp[u * kBucketWaves + w][key_of(wd[u])] + rank[u]] = wd[u];
        }
        __syncthreads();

        // 3. Sums: wave w walks sorted positions [j0, j1), kRows rows at a
        // time, rows loaded by readlane of the point index.
        const int j0 = nc * w / kBucketWaves;
        const int j1 = nc * (w + 1) / kBucketWaves;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; ++v)
            acc[v] = 0.0f;
        int cur = -1;                              // cluster of the open run (uniform)
        int runs = 0;                              // runs closed so far (uniform)
        // Closes the open run: the quarter's first run to edge row 0, any
        // later one to its cluster's sum; the last run is closed after the
        // loop, to edge row 1.
        auto close_run = [&](bool last) __attribute__((always_inline)) {
            const int e = runs == 0 ? 0 : (last ? 1 : -1);
            if (on) {
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    if (e >= 0)
                        edge[(w * 2 + e) * D + lane * V + v] = acc[v];
                    else
                        sums[cur * D + lane * V + v] += acc[v];
                }
            }
            if (e >= 0 && lane == 0)
                edge_c[w][e] = cur;
#pragma unroll
            for (int v = 0; v < V; ++v)
                acc[v] = 0.0f;
            ++runs;
        };
        if (lane == 0) {
            edge_c[w][0] = -1;
            edge_c[w][1] = -1;
        }
        for (int jb = j0; jb < j1; jb += kRows) {
            const int jj = min(jb + lane % kRows, j1 - 1);
            const int word = sorted[jj];
            const int my_i = word & ((1 << kSlotIdxBits) - 1);
            const int my_c = static_cast<int>(static_cast<uint32_t>(word) >> kSlotIdxBits);
            RowBits<V> r[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                const int i = __builtin_amdgcn_readlane(my_i, u);
                r[u] = load_row<V>(X + static_cast<size_t>(i) * D + col);
            }
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                if (jb + u < j1) {                 // uniform
                    const int c = __builtin_amdgcn_readlane(my_c, u);
                    if (c != cur) {                // uniform
                        if (cur >= 0)
                            close_run(false);
                        cur = c;
                    }
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        acc[v] += row_value<V>(r[u], v);
                }
            }
        }
        if (cur >= 0)
            close_run(true);
        __syncthreads();
        // Edge rows in slot order: wave by wave, its first run then its last.
        if (w == 0 && on) {
            for (int q = 0; q < kBucketWaves * 2; ++q) {
                const int c = edge_c[q >> 1][q & 1];
                if (c >= 0) {
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        sums[c * D + lane * V + v] += edge[q * D + lane * V + v];
                }
            }
        }
        // sorted, grp, the edge rows and their clusters are rewritten by the
        // next chunk; the sums are read below.
        __syncthreads();
    }

    // 4. Outputs: wave w finishes clusters b S + w, b S + w + 4, ...
    for (int c = w; c < S; c += kBucketWaves) {
        const int64_t kk = static_cast<int64_t>(b) * S + c;
        if (kk >= K)
            break;
        const int k = static_cast<int>(kk);
        const int count = ccount[c];
        if (count == 0) {
            uint32_t bits[V];
            float mean[V];
            RowBits<V> r = on ? load_row<V>(C_old + static_cast<size_t>(k) * D + lane * V)
                              : RowBits<V>{};
#pragma unroll
            for (int v = 0; v < V; ++v) {
                mean[v] = row_value<V>(r, v);
                bits[v] = __float_as_uint(mean[v]) >> 16;
            }
            emit_cluster<V>(k, bits, mean, 0, D, lane, nrow + w * D, C_new, means, norms, counts);
        } else {
            float s2[V];
#pragma unroll
            for (int v = 0; v < V; ++v)
                s2[v] = on ? sums[c * D + lane * V + v] : 0.0f;
            emit_mean<V>(k, s2, count, D, lane, nrow + w * D, C_new, means, norms, counts);
        }
    }
}

template <int V, int S>
hipError_t launch_bucket_sums(const UpdatePlan &pl, const uint16_t *X, const int32_t *sidx,
                              const int32_t *dir, const uint16_t *C_old, int N, int D, int K,
                              uint16_t *C_new, float *norms, int32_t *counts, float *means,
                              hipStream_t stream) {
    if constexpr (S <= 4) {
        const size_t lds = (static_cast<size_t>(kBucketWaves) * S * D +
                            2 * static_cast<size_t>(pl.bin_tiles) + 1) * 4;
        hipLaunchKernelGGL((upd_bucket_kernel<V, S>), dim3(pl.buckets), dim3(kBucketThreads),
                           lds, stream, X, sidx, dir, C_old, N, D, K, pl.buckets, pl.bin_tiles,
                           pl.bin_tile_log2, C_new, means, norms, counts);
    } else {
        const size_t lds = ((static_cast<size_t>(S) + 2 * kBucketWaves) * D +
                            2 * static_cast<size_t>(pl.bin_tiles) + 1) * 4;
        hipLaunchKernelGGL((upd_bucket_runs_kernel<V, S>), dim3(pl.buckets),
                           dim3(kBucketThreads), lds, stream, X, sidx, dir, C_old, N, D, K,
                           pl.buckets, pl.bin_tiles, pl.bin_tile_log2, C_new, means, norms,
                           counts);
    }
    return hipGetLastError();
}

template <int V>
hipError_t launch_bucket_v(const UpdatePlan &pl, const uint16_t *X, const int32_t *sidx,
                           const int32_t *dir, const uint16_t *C_old, int N, int D, int K,
                           uint16_t *C_new, float *norms, int32_t *counts, float *means,
                           hipStream_t stream) {
    if (pl.bucket_log2 == 0)
        return launch_bucket_sums<V, 1>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                        means, stream);
    if (pl.bucket_log2 == 1)
        return launch_bucket_sums<V, 2>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                        means, stream);
    if (pl.bucket_log2 == 2)
        return launch_bucket_sums<V, 4>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                        means, stream);
    if (pl.bucket_log2 == 3)
        return launch_bucket_sums<V, 8>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                        means, stream);
    return launch_bucket_sums<V, 16>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                     means, stream);
}

size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

template <int V>
hipError_t launch_sums(const UpdatePlan &pl, const uint16_t *X, const int32_t *keys,
                       const int32_t *vals, const uint16_t *C_old, int N, int D, int K,
                       int32_t *start, int32_t *end, float *partial, uint16_t *C_new,
                       float *norms, int32_t *counts, float *means, hipStream_t stream) {
    const dim3 block(kReduceThreads);
    if (N > 0) {
        const int cpr_inv = ((1 << 20) + D / 8 - 1) / (D / 8);
        const int wgs = min(pl.chunks, 4 * pl.compute_units);
        hipLaunchKernelGGL(upd_reduce_kernel<V>, dim3(wgs), block, 0, stream, X, keys, vals, N,
                           D, K, pl.chunk, pl.chunks, cpr_inv, start, end, partial, C_new, means,
                           norms, counts);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int fin_wgs = min((K + 3) / 4, 8192);
    hipLaunchKernelGGL(upd_finish_kernel<V>, dim3(fin_wgs), block, 0, stream, C_old, start, end,
                       partial, N, D, K, pl.chunk, C_new, means, norms, counts);
    return hipGetLastError();
}

}  // namespace

// Below this many clusters there are too few buckets to fill the GPU (one
// workgroup each), and the radix path is used.
constexpr int64_t kMinBucketPathK = 256;

bool bucket_path_fits(int64_t N, int64_t K) {
    return N <= kMaxBinPoints && K <= kMaxBinClusters;
}

UpdatePlan make_update_plan(int64_t N, int64_t D, int64_t K, int compute_units, int force_path) {
    UpdatePlan p{};
    p.compute_units = compute_units > 0 ? compute_units : kDefaultComputeUnits;
    p.path = force_path != 0 ? force_path
                             : (K >= kMinBucketPathK && bucket_path_fits(N, K) ? 2 : 1);
    if (p.path == 2) {
        // Buckets of S = 2^s clusters, at most 1024 of them (one round of
        // bucket workgroups on 256 CUs); tiles of 2^tl >= 1024 points, at
        // most 512 of them (each bucket workgroup reads two directory
        // entries per tile).
        int sl = 0;
        while ((K + (int64_t(1) << sl) - 1) >> sl > kMaxBuckets)
            ++sl;
        p.bucket_log2 = sl;
        p.buckets = static_cast<int>((K + (int64_t(1) << sl) - 1) >> sl);
        int tl = kMinBinTileLog2;
        while (((N + (int64_t(1) << tl) - 1) >> tl) > kMaxBinTiles)
            ++tl;
        p.bin_tile_log2 = tl;
        p.bin_tiles = static_cast<int>((N + (int64_t(1) << tl) - 1) >> tl);
        size_t off = 0;
        if (N > 0) {
            const size_t n4 = align_up(static_cast<size_t>(N) * 4);
            p.sidx = off;
            off += n4;
            p.dir = off;
            off += align_up(static_cast<size_t>(p.buckets + 1) * p.bin_tiles * 4);
        }
        p.bytes = off;
        return p;
    }
    int bits = 0;
    while ((int64_t(1) << bits) <= K)
        ++bits;                                   // keys run 0..K
    p.passes = (bits + 7) / 8;
    // Even digits (K = 4096: 7 + 6 bits, not 8 + 5) halve the histogram rows
    // the first pass's scatter reads and cost the second pass little.
    p.digit_bits = (bits + p.passes - 1) / p.passes;
    // Sort tiles of 2^tl >= 1024 points: at most 128 tiles while tiles stay
    // <= 16384 points (the scan then holds its histogram in registers), at
    // most 4096 beyond.
    int tl = 10;
    while (tl < 14 && (int64_t(1) << tl) * 128 < N)
        ++tl;
    while ((int64_t(1) << tl) * 4096 < N)
        ++tl;
    p.tile_log2 = tl;
    p.tiles = static_cast<int>((N + (int64_t(1) << tl) - 1) >> tl);
    p.stride = (p.tiles + 3) & ~3;
    p.chunk = static_cast<int>(min(static_cast<int64_t>(kMaxChunk), kStageBytes / (2 * D)));
    p.chunks = static_cast<int>((N + p.chunk - 1) / p.chunk);
    if (N == 0)
        return p;
    size_t off = 0;
    const size_t n4 = align_up(static_cast<size_t>(N) * 4);
    for (int i = 0; i < 2; ++i) {
        p.keys[i] = off;
        off += n4;
        p.vals[i] = off;
        off += n4;
    }
    p.hist = off;
    off += align_up(static_cast<size_t>(p.passes) * kRadix * p.stride * 4);
    p.start = off;
    off += align_up(static_cast<size_t>(K) * 4);
    p.end = off;
    off += align_up(static_cast<size_t>(K) * 4);
    p.partial = off;
    off += align_up(static_cast<size_t>(p.chunks) * 2 * D * 4);
    p.bytes = off;
    return p;
}

hipError_t launch_update(const UpdatePlan &pl, const uint16_t *X, const int32_t *labels,
                         const uint16_t *C_old, int N, int D, int K, uint16_t *C_new,
                         float *norms, int32_t *counts, float *means, void *ws,
                         hipStream_t stream) {
    auto *base = static_cast<char *>(ws);
    if (pl.path == 2) {
        int32_t *sidx = nullptr, *dir = nullptr;
        if (N > 0) {
            sidx = reinterpret_cast<int32_t *>(base + pl.sidx);
            dir = reinterpret_cast<int32_t *>(base + pl.dir);
            hipLaunchKernelGGL(upd_bin_kernel, dim3(pl.bin_tiles), dim3(kBinThreads), 0, stream,
                               labels, N, K, pl.bucket_log2, pl.buckets, pl.bin_tile_log2, sidx,
                               dir);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        if (D <= 128)
            return launch_bucket_v<2>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                      means, stream);
        if (D <= 256)
            return launch_bucket_v<4>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                      means, stream);
        return launch_bucket_v<8>(pl, X, sidx, dir, C_old, N, D, K, C_new, norms, counts,
                                  means, stream);
    }
    int32_t *start = nullptr, *end = nullptr, *keys = nullptr, *vals = nullptr;
    float *partial = nullptr;
    if (N > 0) {
        start = reinterpret_cast<int32_t *>(base + pl.start);
        end = reinterpret_cast<int32_t *>(base + pl.end);
        partial = reinterpret_cast<float *>(base + pl.partial);
        auto *hist = reinterpret_cast<int32_t *>(base + pl.hist);
        const size_t hsz = static_cast<size_t>(kRadix) * pl.stride;
        const bool scan = pl.tiles > kFusedScanTiles;
        const dim3 grid(pl.tiles), block(kSortThreads);
        hipError_t e = hipSuccess;
        const int mask = (1 << pl.digit_bits) - 1;
        for (int q = 0; q < pl.passes && e == hipSuccess; ++q) {
            const int sh = pl.digit_bits * q;
            int32_t *h = hist + hsz * q;
            const int32_t *kin = q == 0 ? labels : reinterpret_cast<int32_t *>(base + pl.keys[(q - 1) & 1]);
            const int32_t *vin = q == 0 ? nullptr : reinterpret_cast<int32_t *>(base + pl.vals[(q - 1) & 1]);
            keys = reinterpret_cast<int32_t *>(base + pl.keys[q & 1]);
            vals = reinterpret_cast<int32_t *>(base + pl.vals[q & 1]);
            if (q == 0)   // also clears start and end (adjacent in the workspace)
                hipLaunchKernelGGL(upd_hist_kernel<true>, grid, block, 0, stream, kin, N, K, 0,
                                   mask, pl.tile_log2, pl.tiles, pl.stride, h, start,
                                   static_cast<int64_t>((pl.partial - pl.start) / 4));
            else
                hipLaunchKernelGGL(upd_hist_kernel<false>, grid, block, 0, stream, kin, N, K, sh,
                                   mask, pl.tile_log2, pl.tiles, pl.stride, h, nullptr, int64_t(0));
            if (scan)
                hipLaunchKernelGGL(upd_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, h,
                                   static_cast<int>(hsz));
            const dim3 sblock(kScatterThreads);
            if (q == 0 && scan)
                hipLaunchKernelGGL((upd_scatter_kernel<true, true>), grid, sblock, 0, stream, kin,
                                   vin, N, K, sh, mask, pl.tile_log2, pl.tiles, pl.stride, h, keys, vals);
            else if (q == 0)
                hipLaunchKernelGGL((upd_scatter_kernel<true, false>), grid, sblock, 0, stream, kin,
                                   vin, N, K, sh, mask, pl.tile_log2, pl.tiles, pl.stride, h, keys, vals);
            else if (scan)
                hipLaunchKernelGGL((upd_scatter_kernel<false, true>), grid, sblock, 0, stream, kin,
                                   vin, N, K, sh, mask, pl.tile_log2, pl.tiles, pl.stride, h, keys, vals);
            else
                hipLaunchKernelGGL((upd_scatter_kernel<false, false>), grid, sblock, 0, stream, kin,
                                   vin, N, K, sh, mask, pl.tile_log2, pl.tiles, pl.stride, h, keys, vals);
            e = hipGetLastError();
        }
        if (e != hipSuccess)
            return e;
    }
    // Two columns per lane up to D = 128 (D / 2 lanes active below 128): a
    // one-column variant needs several times the registers for no gain.
    if (D <= 128)
        return launch_sums<2>(pl, X, keys, vals, C_old, N, D, K, start, end, partial, C_new, norms,
                              counts, means, stream);
    if (D <= 256)
        return launch_sums<4>(pl, X, keys, vals, C_old, N, D, K, start, end, partial, C_new, norms,
                              counts, means, stream);
    return launch_sums<8>(pl, X, keys, vals, C_old, N, D, K, start, end, partial, C_new, norms,
                          counts, means, stream);
}

}  // namespace kmeans

// ---- C entry point ---------------------------------------------------------

extern "C" kmeans_status_t kmeans_update_path(const void *X, const int32_t *labels,
                                              const void *C_old, int64_t N, int64_t D, int64_t K,
                                              void *C_new, float *norms, int32_t *counts,
                                              float *means, int32_t path, hipStream_t stream) {
    using namespace kmeans;
    if (path < KMEANS_UPDATE_AUTO || path > KMEANS_UPDATE_BUCKETS)
        return fail(KMEANS_ERR_INVALID_ARG, "path=%d is not a kmeans_update_path_t", path);
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
    if (!C_old || !C_new || !norms || !counts || (N > 0 && (!X || !labels)))
        return fail(KMEANS_ERR_INVALID_ARG, "null pointer argument (X=%p labels=%p C_old=%p "
                    "C_new=%p norms=%p counts=%p)", X, static_cast<const void *>(labels), C_old,
                    C_new, static_cast<void *>(norms), static_cast<void *>(counts));
    if ((N > 0 && !aligned(X, 16)) || !aligned(C_old, 16) || !aligned(C_new, 16))
        return fail(KMEANS_ERR_ALIGNMENT, "X, C_old and C_new must be 16-byte aligned");
    if ((N > 0 && !aligned(labels, 4)) || !aligned(norms, 4) || !aligned(counts, 4) ||
        !aligned(means, 4))
        return fail(KMEANS_ERR_ALIGNMENT, "labels, norms, counts and means must be 4-byte aligned");

    if (path == KMEANS_UPDATE_BUCKETS && !bucket_path_fits(N, K))
        return fail(KMEANS_ERR_UNSUPPORTED, "the bucket path needs N <= %lld and K <= %lld "
                    "(N=%lld, K=%lld)", static_cast<long long>(kMaxBinPoints),
                    static_cast<long long>(kMaxBinClusters), static_cast<long long>(N),
                    static_cast<long long>(K));
    const UpdatePlan pl = make_update_plan(N, D, K, device_compute_units(), path);
    // The stream's scratch (none when N == 0), held until the launches are queued.
    std::unique_ptr<WorkspaceLease> lease;
    void *ws = nullptr;
    if (pl.bytes > 0) {
        lease = std::make_unique<WorkspaceLease>(stream, pl.bytes);
        if (lease->error() != hipSuccess)
            return fail(KMEANS_ERR_NO_MEMORY, "workspace of %zu bytes: %s", pl.bytes,
                        hipGetErrorString(lease->error()));
        ws = lease->ptr();
    }
    hipError_t e = launch_update(pl, static_cast<const uint16_t *>(X), labels,
                                         static_cast<const uint16_t *>(C_old),
                                         static_cast<int>(N), static_cast<int>(D),
                                         static_cast<int>(K), static_cast<uint16_t *>(C_new),
                                         norms, counts, means, ws, stream);
    if (e != hipSuccess)
        return fail(KMEANS_ERR_HIP, "update launch failed: %s", hipGetErrorString(e));
    return ok();
}

extern "C" kmeans_status_t kmeans_update(const void *X, const int32_t *labels, const void *C_old,
                                         int64_t N, int64_t D, int64_t K, void *C_new,
                                         float *norms, int32_t *counts, float *means,
                                         hipStream_t stream) {
    return kmeans_update_path(X, labels, C_old, N, D, K, C_new, norms, counts, means,
                              KMEANS_UPDATE_AUTO, stream);
}
