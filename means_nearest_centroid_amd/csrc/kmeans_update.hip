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
//     (label, or K for a stray label) carrying the point index, on 8-bit
//     digits.  A pass is: a per-tile digit histogram, one exclusive scan over
//     (digit, tile), and a scatter in which every tile ranks its keys in
//     index order -- wave ballots give the rank among equal digits inside a
//     wave, and a per-wave count table in LDS, tagged with the round so it
//     never needs clearing, the rank across the tile's waves.  The scatter of
//     one pass also counts the next pass's digits per destination tile
//     (integer atomics), so only the first pass has a histogram kernel.
//  2. The reduce kernel gives each wave a fixed chunk of sorted positions.  A
//     wave walks its chunk in order, gathering one row per position (all 64
//     lanes share the row, V bf16 values each) and adding it to the running
//     sum of the current run of equal labels.  A cluster that starts and ends
//     inside the chunk is finished there; a run cut by a chunk boundary
//     leaves its partial sum, and the finish kernel adds a cluster's partials
//     in chunk order.  Work per wave is bounded by the chunk, whatever the
//     cluster sizes, and the order of every sum is fixed by the sorted order.
//  3. Finishing a cluster: mean = sum / count in fp32, rounded to bf16, and
//     the squared norm of the rounded row computed exactly as the norms
//     pre-pass computes it (row_sq_norm16 over a copy of the row in LDS).
#include <stdint.h>

#include "kmeans_internal.h"

namespace kmeans {
namespace {

constexpr int kSortThreads = 256;    // 4 waves; one key per thread per round
constexpr int kRadix = 256;
constexpr int kScanThreads = 1024;
constexpr int kReduceWaves = 4;
constexpr int kPrefetch = 16;        // rows in flight per wave in the reduce
constexpr int kMaxRow = 512;         // bf16 values of the widest supported row

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

// Pass-0 digit histogram of one tile, written digit-major ([digit][tile]).
// The same launch clears the cluster bounds and the histograms the later
// passes accumulate into.
__global__ __launch_bounds__(kSortThreads)
void upd_hist_kernel(const int32_t *__restrict__ labels, int N, int K, int tile_log2, int tiles,
                     int32_t *__restrict__ hist0, int32_t *__restrict__ clear_a, int64_t n_a,
                     int32_t *__restrict__ clear_b, int64_t n_b) {
    __shared__ int h[kRadix];
    const int tid = threadIdx.x;
    h[tid] = 0;
    __syncthreads();
    const int t = blockIdx.x;
    const int beg = t << tile_log2;
    const int fin = static_cast<int>(min(static_cast<int64_t>(N),
                                         static_cast<int64_t>(beg) + (int64_t(1) << tile_log2)));
    for (int i = beg + tid; i < fin; i += kSortThreads)
        atomicAdd(&h[sort_key(labels[i], K) & (kRadix - 1)], 1);
    __syncthreads();
    hist0[static_cast<size_t>(tid) * tiles + t] = h[tid];
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kSortThreads;
    for (int64_t j = static_cast<int64_t>(t) * kSortThreads + tid; j < n_a; j += stride)
        clear_a[j] = 0;
    for (int64_t j = static_cast<int64_t>(t) * kSortThreads + tid; j < n_b; j += stride)
        clear_b[j] = 0;
}

// Exclusive scan of h[0..M) in place, one workgroup: each thread owns a
// contiguous run of entries.
__global__ __launch_bounds__(kScanThreads)
void upd_scan_kernel(int32_t *__restrict__ h, int M) {
    __shared__ int part[kScanThreads];
    const int tid = threadIdx.x;
    const int per = (M + kScanThreads - 1) / kScanThreads;
    const int b = min(M, tid * per);
    const int e = min(M, b + per);
    int sum = 0;
    for (int j = b; j < e; ++j)
        sum += h[j];
    part[tid] = sum;
    __syncthreads();
    for (int off = 1; off < kScanThreads; off <<= 1) {
        const int v = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - sum;
    for (int j = b; j < e; ++j) {
        const int v = h[j];
        h[j] = run;
        run += v;
    }
}

// One stable scatter pass on digit (key >> shift) & 255.  FIRST: keys come
// from the labels and values are the point indices.  hist_next (null on the
// last pass) collects the next digit per destination tile.
template <bool FIRST>
__global__ __launch_bounds__(kSortThreads)
void upd_scatter_kernel(const int32_t *__restrict__ keys_in, const int32_t *__restrict__ vals_in,
                        int N, int K, int shift, int tile_log2, int tiles,
                        const int32_t *__restrict__ offs, int32_t *__restrict__ keys_out,
                        int32_t *__restrict__ vals_out, int32_t *__restrict__ hist_next) {
    __shared__ int running[kRadix];
    __shared__ int wcnt[kSortThreads / 64][kRadix];   // (round tag << 8) | count
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int t = blockIdx.x;
    running[tid] = offs[static_cast<size_t>(tid) * tiles + t];
#pragma unroll
    for (int i = 0; i < kSortThreads / 64; ++i)
        wcnt[i][tid] = 0;
    __syncthreads();
    const int beg = t << tile_log2;
    const int fin = static_cast<int>(min(static_cast<int64_t>(N),
                                         static_cast<int64_t>(beg) + (int64_t(1) << tile_log2)));
    const uint64_t below = (uint64_t(1) << lane) - 1;
    int tag = 0;
    for (int base = beg; base < fin; base += kSortThreads) {
        ++tag;
        const int i = base + tid;
        const bool valid = i < fin;
        int key = 0, val = 0;
        if (valid) {
            key = FIRST ? sort_key(keys_in[i], K) : keys_in[i];
            val = FIRST ? i : vals_in[i];
        }
        const int d = (key >> shift) & (kRadix - 1);
        // Lanes of this wave holding the same digit.
        uint64_t same = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const bool bit = (d >> b) & 1;
            const uint64_t m = __ballot(valid && bit);
            same &= bit ? m : ~m;
        }
        if (valid && (same >> lane) == 1)              // last lane of its group
            wcnt[w][d] = (tag << 8) | __popcll(same);
        __syncthreads();
        if (valid) {
            int pos = running[d] + __popcll(same & below);
            for (int v = 0; v < w; ++v) {
                const int e = wcnt[v][d];
                pos += (e >> 8) == tag ? (e & 255) : 0;
            }
            keys_out[pos] = key;
            vals_out[pos] = val;
            if (hist_next)
                atomicAdd(&hist_next[static_cast<size_t>((key >> (shift + 8)) & (kRadix - 1)) *
                                         tiles + (pos >> tile_log2)], 1);
        }
        int tot = 0;
#pragma unroll
        for (int v = 0; v < kSortThreads / 64; ++v) {
            const int e = wcnt[v][tid];
            tot += (e >> 8) == tag ? (e & 255) : 0;
        }
        __syncthreads();
        running[tid] += tot;
    }
}

// ---- 2./3. per-cluster sums ----------------------------------------------

// V bf16 values of one row per lane (lane l holds columns l*V .. l*V+V-1).
template <int V>
struct RowBits {
    uint32_t w[(V + 1) / 2];
};

template <int V>
__device__ __forceinline__ RowBits<V> load_row(const uint16_t *p) {
    RowBits<V> r;
    if constexpr (V == 1) {
        r.w[0] = *p;
    } else if constexpr (V == 2) {
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
    if constexpr (V == 1)
        return widen(r.w[0]);
    else
        return (v & 1) ? __uint_as_float(r.w[v >> 1] & 0xffff0000u) : widen(r.w[v >> 1] & 0xffffu);
}

template <int V>
__device__ __forceinline__ void store_bits(uint16_t *p, const uint32_t (&b)[V]) {
    if constexpr (V == 1) {
        *p = static_cast<uint16_t>(b[0]);
    } else if constexpr (V == 2) {
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
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");   // row copy visible to the wave
    const float n = row_sq_norm16(lds_row, D, lane & 15);
    if (lane == 0) {
        norms[k] = n;
        counts[k] = count;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");   // reads done before the next copy
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

// Runs of equal keys over one chunk of sorted positions per wave.  For a run
// [a, b) of cluster k: a is k's first position unless the run starts the
// chunk and the previous position holds k too; b is its end unless the run
// ends the chunk and the next position holds k too.  A run that is the whole
// cluster is finished here; otherwise its sum goes to partial slot 0 (the run
// began before this chunk) or 1 (it began here and continues past it).
template <int V>
__global__ __launch_bounds__(64 * kReduceWaves)
void upd_reduce_kernel(const uint16_t *__restrict__ X, const int32_t *__restrict__ keys,
                       const int32_t *__restrict__ vals, int N, int D, int K,
                       int32_t *__restrict__ start, int32_t *__restrict__ end,
                       float *__restrict__ partial, uint16_t *__restrict__ C_new,
                       float *__restrict__ means, float *__restrict__ norms,
                       int32_t *__restrict__ counts) {
    __shared__ uint16_t lds[kReduceWaves][kMaxRow];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int chunk = blockIdx.x * kReduceWaves + wave;
    const int c0 = chunk * kUpdateChunk;
    if (c0 >= N)
        return;
    const int c1 = min(N, c0 + kUpdateChunk);
    const bool on = lane * V < D;
    const uint16_t *xl = X + lane * V;
    uint16_t *lds_row = lds[wave];

    int cur = keys[c0];
    if (cur >= K)
        return;                         // only stray labels from here on
    int run_start = c0;
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v)
        acc[v] = 0.0f;

    auto flush = [&](int b) __attribute__((always_inline)) {
        const bool before = run_start == c0 && c0 > 0 && keys[c0 - 1] == cur;
        const bool after = b == c1 && c1 < N && keys[c1] == cur;
        if (lane == 0) {
            if (!before)
                start[cur] = run_start;
            if (!after)
                end[cur] = b;
        }
        if (!before && !after) {
            emit_mean<V>(cur, acc, b - run_start, D, lane, lds_row, C_new, means, norms, counts);
        } else if (on) {
            float *dst = partial + (static_cast<size_t>(chunk) * 2 + (before ? 0 : 1)) * D + lane * V;
            store_f32<V>(dst, acc);
        }
    };

    // Positions past the chunk read as key K, like stray labels: either ends
    // the walk.  Keys and indices are wave-uniform (scalar registers).
    bool done = false;
    for (int p = c0; p < c1 && !done; p += kPrefetch) {
        int kk[kPrefetch];
        RowBits<V> rb[kPrefetch];
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) {
            const int q = p + u;
            kk[u] = q < c1 ? __builtin_amdgcn_readfirstlane(keys[q]) : K;
            const int idx = kk[u] < K ? __builtin_amdgcn_readfirstlane(vals[q]) : -1;
            rb[u] = (on && idx >= 0) ? load_row<V>(xl + static_cast<size_t>(idx) * D)
                                     : RowBits<V>{};
        }
#pragma unroll
        for (int u = 0; u < kPrefetch; ++u) {
            if (!done && kk[u] != cur) {
                flush(p + u);
                if (kk[u] >= K) {
                    done = true;
                } else {
                    cur = kk[u];
                    run_start = p + u;
#pragma unroll
                    for (int v = 0; v < V; ++v)
                        acc[v] = 0.0f;
                }
            }
            if (!done) {
#pragma unroll
                for (int v = 0; v < V; ++v)
                    acc[v] += row_value<V>(rb[u], v);
            }
        }
    }
    if (!done)
        flush(c1);
}

// Clusters the reduce kernel did not finish: empty ones (old row kept) and
// those spanning several chunks (partials added in chunk order).
template <int V>
__global__ __launch_bounds__(64 * kReduceWaves)
void upd_finish_kernel(const uint16_t *__restrict__ C_old, const int32_t *__restrict__ start,
                       const int32_t *__restrict__ end, const float *__restrict__ partial,
                       int N, int D, int K, uint16_t *__restrict__ C_new,
                       float *__restrict__ means, float *__restrict__ norms,
                       int32_t *__restrict__ counts) {
    __shared__ uint16_t lds[kReduceWaves][kMaxRow];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const bool on = lane * V < D;
    uint16_t *lds_row = lds[wave];
    const int nwaves = gridDim.x * kReduceWaves;
    for (int k = blockIdx.x * kReduceWaves + wave; k < K; k += nwaves) {
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
        const int cf = s / kUpdateChunk;
        const int cl = (e - 1) / kUpdateChunk;
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

size_t align_up(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

template <int V>
hipError_t launch_sums(const UpdatePlan &pl, const uint16_t *X, const int32_t *keys,
                       const int32_t *vals, const uint16_t *C_old, int N, int D, int K,
                       int32_t *start, int32_t *end, float *partial, uint16_t *C_new,
                       float *norms, int32_t *counts, float *means, hipStream_t stream) {
    const dim3 block(64 * kReduceWaves);
    if (N > 0) {
        const int wgs = (pl.chunks + kReduceWaves - 1) / kReduceWaves;
        hipLaunchKernelGGL(upd_reduce_kernel<V>, dim3(wgs), block, 0, stream, X, keys, vals, N, D,
                           K, start, end, partial, C_new, means, norms, counts);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int fin_wgs = min((K + kReduceWaves - 1) / kReduceWaves, 8192);
    hipLaunchKernelGGL(upd_finish_kernel<V>, dim3(fin_wgs), block, 0, stream, C_old, start, end,
                       partial, N, D, K, C_new, means, norms, counts);
    return hipGetLastError();
}

}  // namespace

UpdatePlan make_update_plan(int64_t N, int64_t D, int64_t K) {
    UpdatePlan p{};
    int bits = 0;
    while ((int64_t(1) << bits) <= K)
        ++bits;                                   // keys run 0..K
    p.passes = (bits + 7) / 8;
    int tl = 10;                                  // tiles of >= 1024 points,
    while ((int64_t(1) << tl) * 4096 < N)         // at most 4096 tiles
        ++tl;
    p.tile_log2 = tl;
    p.tiles = static_cast<int>((N + (int64_t(1) << tl) - 1) >> tl);
    p.chunks = static_cast<int>((N + kUpdateChunk - 1) / kUpdateChunk);
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
    off += align_up(static_cast<size_t>(p.passes) * kRadix * p.tiles * 4);
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
    int32_t *start = nullptr, *end = nullptr, *keys = nullptr, *vals = nullptr;
    float *partial = nullptr;
    if (N > 0) {
        start = reinterpret_cast<int32_t *>(base + pl.start);
        end = reinterpret_cast<int32_t *>(base + pl.end);
        partial = reinterpret_cast<float *>(base + pl.partial);
        auto *hist = reinterpret_cast<int32_t *>(base + pl.hist);
        const size_t hsz = static_cast<size_t>(kRadix) * pl.tiles;
        // start and end are adjacent in the workspace; clear both at once.
        hipLaunchKernelGGL(upd_hist_kernel, dim3(pl.tiles), dim3(kSortThreads), 0, stream, labels,
                           N, K, pl.tile_log2, pl.tiles, hist, start,
                           static_cast<int64_t>((pl.partial - pl.start) / 4), hist + hsz,
                           static_cast<int64_t>(hsz * (pl.passes - 1)));
        hipError_t e = hipGetLastError();
        for (int q = 0; q < pl.passes && e == hipSuccess; ++q) {
            int32_t *h = hist + hsz * q;
            hipLaunchKernelGGL(upd_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, h,
                               static_cast<int>(hsz));
            e = hipGetLastError();
            if (e != hipSuccess)
                break;
            const int32_t *kin = q == 0 ? labels : reinterpret_cast<int32_t *>(base + pl.keys[(q - 1) & 1]);
            const int32_t *vin = q == 0 ? nullptr : reinterpret_cast<int32_t *>(base + pl.vals[(q - 1) & 1]);
            keys = reinterpret_cast<int32_t *>(base + pl.keys[q & 1]);
            vals = reinterpret_cast<int32_t *>(base + pl.vals[q & 1]);
            int32_t *hn = q + 1 < pl.passes ? h + hsz : nullptr;
            if (q == 0)
                hipLaunchKernelGGL(upd_scatter_kernel<true>, dim3(pl.tiles), dim3(kSortThreads), 0,
                                   stream, kin, vin, N, K, 8 * q, pl.tile_log2, pl.tiles, h, keys,
                                   vals, hn);
            else
                hipLaunchKernelGGL(upd_scatter_kernel<false>, dim3(pl.tiles), dim3(kSortThreads), 0,
                                   stream, kin, vin, N, K, 8 * q, pl.tile_log2, pl.tiles, h, keys,
                                   vals, hn);
            e = hipGetLastError();
        }
        if (e != hipSuccess)
            return e;
    }
    if (D <= 64)
        return launch_sums<1>(pl, X, keys, vals, C_old, N, D, K, start, end, partial, C_new, norms,
                              counts, means, stream);
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
