// kmeans_kernels.hip -- gfx950 (CDNA4) kernels of the k-means assignment step.
//
// Operation (flashlib PR #22, "Optimize Blackwell k-means assignment
// reduction", Summary and "Key ideas and contributions" table): per point,
// score every centroid by s = ||c||^2 - 2 x.c and keep the lowest-index
// minimum.  Design for CDNA4, not a translation of the pages' Blackwell
// kernel:
//
//  * The x.c contraction runs on bf16 MFMA (v_mfma_f32_32x32x16_bf16): the
//    centroid tile is the A operand (32 rows), 32 points are the B operand.
//    Each lane then owns 16 scores of ONE point, so the argmin needs no
//    cross-lane traffic inside the hot loop.
//  * The norm is folded into the accumulator: the points are held as -2x
//    (exact in bf16) and the MFMA's C input is the norm tile, so the MFMA
//    result is the score s itself -- no epilogue op applies the norms and no
//    LDS round trip or barrier is spent on them (the pages' "Register-staged
//    norms" / "Barrier elimination" rows reach the same goal on Blackwell).
//  * Points stay resident in VGPRs for the whole K loop; centroid blocks are
//    double-buffered through LDS with an XOR swizzle so the A-operand reads
//    (ds_read_b128, 32 rows at one column) hit distinct banks.
//  * The epilogue keeps two running (score, index) chains per point (even and
//    odd accumulator slots, the pages' "Two-chain argmin"), each scanned in
//    increasing index with a strict '<', merged by (score, index) at the end,
//    then across the two lanes that share a point ("Deterministic winner
//    merge").  The N x K score matrix never leaves registers.
//  * A point whose every score is +inf or NaN, or whose result is not finite,
//    takes a cold per-lane path after the loop (rule: -inf < finite < +inf <
//    NaN, ties to the lower index).
#include <math.h>
#include <stdint.h>

#include "kmeans_internal.h"

namespace kmeans {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float widen(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Scale the 8 bf16 values of v by -2 (exact: a sign flip and an exponent
// step) and accumulate their squares (fp32) into xx.
__device__ __forceinline__ u32x4 neg2_and_square(u32x4 v, float &xx) {
    u32x4 r;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float lo = __uint_as_float(v[w] << 16);
        const float hi = __uint_as_float(v[w] & 0xffff0000u);
        xx = fmaf(lo, lo, xx);
        xx = fmaf(hi, hi, xx);
        const uint32_t lo2 = __float_as_uint(lo * -2.0f);
        const uint32_t hi2 = __float_as_uint(hi * -2.0f);
        r[w] = (hi2 & 0xffff0000u) | (lo2 >> 16);
    }
    return r;
}

// Physical 16-byte slot of logical chunk c in row `row` of an LDS block with
// S chunks per row.  Keeps 16 consecutive rows at one logical chunk in 16
// distinct 16-byte bank groups of a 256-byte line.
template <int S>
__device__ __forceinline__ int swz(int row, int c) {
    if constexpr (S >= 16)
        return c ^ (row & 15);
    else
        return c ^ ((row / (16 / S)) & (S - 1));
}

// (s, i) strictly before (so, io) under score-then-index order.
__device__ __forceinline__ bool pair_before(float s, int32_t i, float so, int32_t io) {
    return s < so || (s == so && i < io);
}

// Final label and min_dist of point n from its merged winner (s, lab) and
// ||x||^2.  Hot case: finite result, min_dist = max(0, xx + s).  Cold cases
// (non-finite data) recompute on the VALU in IEEE fp32; only the class of
// each score matters there and it does not depend on summation order.
__device__ void finalize_point(int n, float s, int32_t lab, float xx,
                               const uint16_t *__restrict__ X,
                               const uint16_t *__restrict__ C,
                               const float *__restrict__ norms, int D, int K,
                               int32_t *__restrict__ labels,
                               float *__restrict__ min_dist) {
    float md;
    if (lab == kNoLabel || !isfinite(xx) || !isfinite(s)) {
        const uint16_t *xr = X + static_cast<size_t>(n) * D;
        if (lab == kNoLabel) {
            // Every score is +inf or NaN: lowest +inf index, else 0.  A NaN
            // coordinate makes every score NaN.
            lab = 0;
            if (!isnan(xx)) {
                for (int k = 0; k < K; ++k) {
                    const uint16_t *cr = C + static_cast<size_t>(k) * D;
                    float sk = norms[k];
                    for (int j = 0; j < D; ++j)
                        sk = fmaf(-2.0f * widen(xr[j]), widen(cr[j]), sk);
                    if (sk == INFINITY) {
                        lab = k;
                        break;
                    }
                }
            }
        }
        const uint16_t *cr = C + static_cast<size_t>(lab) * D;
        float d = 0.0f;
        for (int j = 0; j < D; ++j) {
            const float e = widen(xr[j]) - widen(cr[j]);
            d = fmaf(e, e, d);
        }
        md = d;
    } else {
        md = fmaxf(0.0f, xx + s);
    }
    labels[n] = lab;
    min_dist[n] = md;
}

// One workgroup = 4 waves; wave w owns P blocks of 32 points.  Grid:
// x = point workgroups, y = K-ranges of k_chunk centroids.
template <int KS, int P, int BK, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(WPE, WPE)))
void assign_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ C,
                   const float *__restrict__ norms, int N, int D, int K, int k_chunk,
                   int write_partials, int32_t *__restrict__ labels,
                   float *__restrict__ min_dist, float *__restrict__ ws_score,
                   int32_t *__restrict__ ws_label, float *__restrict__ ws_xx) {
    constexpr int S = 2 * KS;                  // 16-byte chunks per centroid row
    constexpr int ROW_BYTES = 16 * S;
    constexpr int LOADS = BK * S / kThreads;   // chunks each thread stages per block
    constexpr int NLOADS = (BK + kThreads - 1) / kThreads;
    static_assert((BK * S) % kThreads == 0, "block must split evenly");
    static_assert(BK % kTileRows == 0, "block is whole tiles");

    __shared__ __attribute__((aligned(16))) uint8_t lds_c[2][BK * ROW_BYTES];
    __shared__ __attribute__((aligned(16))) float lds_n[2][BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int col = lane & 31;   // point column of the B tile; row of the A tile
    const int half = lane >> 5;  // which 8-element half of a 16-wide k-step

    const int split = blockIdx.y;
    const int k_begin = split * k_chunk;
    const int k_end = min(K, k_begin + k_chunk);
    const int point0 = blockIdx.x * (kWavesPerWg * P * kTileCols) + wave * (P * kTileCols);

    // ---- resident points: -2x as MFMA B fragments, and ||x||^2 ----
    u32x4 xb[P][KS];
    float xx[P];
#pragma unroll
    for (int p = 0; p < P; ++p) {
        xx[p] = 0.0f;
        const int row = point0 + p * kTileCols + col;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int c0 = ks * 16 + half * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row < N && c0 < D)
                v = *reinterpret_cast<const u32x4 *>(X + static_cast<size_t>(row) * D + c0);
            xb[p][ks] = neg2_and_square(v, xx[p]);
        }
        xx[p] += __shfl_xor(xx[p], 32);
    }

    float bs[P][2];
    int32_t bi[P][2];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
            bs[p][ch] = INFINITY;
            bi[p][ch] = kNoLabel;
        }

    // ---- centroid blocks: global -> registers -> LDS, double-buffered ----
    u32x4 stage[LOADS];
    float nstage[NLOADS];
    auto fetch = [&](int kb) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int q = tid + i * kThreads;
            const int r = q / S, c = q % S;
            const int k = kb + r;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (k < k_end && c * 8 < D)
                v = *reinterpret_cast<const u32x4 *>(C + static_cast<size_t>(k) * D + c * 8);
            stage[i] = v;
        }
#pragma unroll
        for (int i = 0; i < NLOADS; ++i) {
            const int r = tid + i * kThreads;
            // Rows past the range score NaN, which never wins.
            nstage[i] = (r < BK && kb + r < k_end) ? norms[kb + r] : __builtin_nanf("");
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int q = tid + i * kThreads;
            const int r = q / S, c = q % S;
            *reinterpret_cast<u32x4 *>(&lds_c[buf][r * ROW_BYTES + swz<S>(r, c) * 16]) = stage[i];
        }
#pragma unroll
        for (int i = 0; i < NLOADS; ++i) {
            const int r = tid + i * kThreads;
            if (r < BK)
                lds_n[buf][r] = nstage[i];
        }
    };

    const int nblocks = (k_end - k_begin + BK - 1) / BK;
    fetch(k_begin);
    store(0);
    __syncthreads();

    for (int b = 0; b < nblocks; ++b) {
        const int buf = b & 1;
        const int kb = k_begin + b * BK;
        if (b + 1 < nblocks)
            fetch(kb + BK);

#pragma unroll
        for (int tt = 0; tt < BK / kTileRows; ++tt) {
            const int r0 = tt * kTileRows;
            if (kb + r0 >= k_end)
                break;
            // Norm tile as the MFMA C input: slot r of this lane is row
            // 8*(r/4) + 4*half + r%4 of the tile.
            f32x16 ninit;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(&lds_n[buf][r0 + 8 * q + 4 * half]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ninit[4 * q + e] = v[e];
            }
            bf16x8 a[KS];
            const int arow = r0 + col;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a[ks] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(
                                &lds_c[buf][arow * ROW_BYTES + swz<S>(arow, 2 * ks + half) * 16]));

            const int kt = kb + r0;   // wave-uniform index base of this tile
#pragma unroll
            for (int p = 0; p < P; ++p) {
                f32x16 acc = ninit;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        a[ks], __builtin_bit_cast(bf16x8, xb[p][ks]), acc, 0, 0, 0);
                // acc[r] = s for centroid kt + 8*(r/4) + 4*half + r%4 (the
                // lane term 4*half is added once after the loop).
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int ch = r & 1;
                    const int32_t idx = kt + 8 * (r >> 2) + (r & 3);
                    const float s = acc[r];
                    const bool lt = s < bs[p][ch];
                    bs[p][ch] = lt ? s : bs[p][ch];
                    bi[p][ch] = lt ? idx : bi[p][ch];
                }
            }
        }

        if (b + 1 < nblocks)
            store(buf ^ 1);
        __syncthreads();
    }

    // ---- merge chains, then the two lanes that hold the same point ----
#pragma unroll
    for (int p = 0; p < P; ++p) {
        float s = bs[p][0];
        int32_t i = bi[p][0];
        if (pair_before(bs[p][1], bi[p][1], s, i)) {
            s = bs[p][1];
            i = bi[p][1];
        }
        if (i != kNoLabel)
            i += 4 * half;
        const float so = __shfl_xor(s, 32);
        const int32_t io = __shfl_xor(i, 32);
        if (pair_before(so, io, s, i)) {
            s = so;
            i = io;
        }
        const int n = point0 + p * kTileCols + col;
        if (half == 0 && n < N) {
            if (write_partials) {
                ws_score[static_cast<size_t>(split) * N + n] = s;
                ws_label[static_cast<size_t>(split) * N + n] = i;
                if (split == 0)
                    ws_xx[n] = xx[p];
            } else {
                finalize_point(n, s, i, xx[p], X, C, norms, D, K, labels, min_dist);
            }
        }
    }
}

// Second pass of the K-split path: (score, index) minimum over the splits.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void merge_kernel(const float *__restrict__ ws_score, const int32_t *__restrict__ ws_label,
                  const float *__restrict__ ws_xx, int splits,
                  const uint16_t *__restrict__ X, const uint16_t *__restrict__ C,
                  const float *__restrict__ norms, int N, int D, int K,
                  int32_t *__restrict__ labels, float *__restrict__ min_dist) {
    const int n = blockIdx.x * kThreads + threadIdx.x;
    if (n >= N)
        return;
    float s = ws_score[n];
    int32_t i = ws_label[n];
    for (int sp = 1; sp < splits; ++sp) {
        const float so = ws_score[static_cast<size_t>(sp) * N + n];
        const int32_t io = ws_label[static_cast<size_t>(sp) * N + n];
        if (pair_before(so, io, s, i)) {
            s = so;
            i = io;
        }
    }
    finalize_point(n, s, i, ws_xx[n], X, C, norms, D, K, labels, min_dist);
}

// ||c_k||^2: 16 lanes per row, 16 rows per workgroup, 16-byte loads.  Every
// row is reduced with the same lane pattern, so identical rows get identical
// bits.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void norms_kernel(const uint16_t *__restrict__ C, int K, int D, float *__restrict__ norms) {
    const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    float acc = 0.0f;
    if (row < K) {
        const uint16_t *cr = C + static_cast<size_t>(row) * D;
        for (int c = l; c * 8 < D; c += 16) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(cr + c * 8);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float lo = __uint_as_float(v[w] << 16);
                const float hi = __uint_as_float(v[w] & 0xffff0000u);
                acc = fmaf(lo, lo, acc);
                acc = fmaf(hi, hi, acc);
            }
        }
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1)
        acc += __shfl_xor(acc, m, 16);
    if (row < K && l == 0)
        norms[row] = acc;
}

template <int KS>
hipError_t launch_assign_ks(const Plan &pl, const uint16_t *X, const uint16_t *C,
                            const float *norms, int N, int D, int K, int32_t *labels,
                            float *min_dist, float *ws_score, int32_t *ws_label,
                            float *ws_xx, hipStream_t stream) {
    constexpr int P = point_blocks_per_wave(KS);
    constexpr int BK = k_block_rows(KS);
    constexpr int WPE = KS >= 32 ? 1 : 2;
    const int partial = ws_score != nullptr ? 1 : 0;
    hipLaunchKernelGGL((assign_kernel<KS, P, BK, WPE>), dim3(pl.wgs, pl.splits), dim3(kThreads),
                       0, stream, X, C, norms, N, D, K, pl.k_chunk, partial, labels, min_dist,
                       ws_score, ws_label, ws_xx);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_norms(const uint16_t *C, int K, int D, float *norms, hipStream_t stream) {
    const int blocks = (K + 15) / 16;
    hipLaunchKernelGGL(norms_kernel, dim3(blocks), dim3(kThreads), 0, stream, C, K, D, norms);
    return hipGetLastError();
}

hipError_t launch_assign(const Plan &pl, const uint16_t *X, const uint16_t *C,
                         const float *norms, int N, int D, int K, int32_t *labels,
                         float *min_dist, float *ws_score, int32_t *ws_label,
                         float *ws_xx, hipStream_t stream) {
    switch (pl.ks) {
    case 1: return launch_assign_ks<1>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, stream);
    case 2: return launch_assign_ks<2>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, stream);
    case 4: return launch_assign_ks<4>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, stream);
    case 8: return launch_assign_ks<8>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, stream);
    case 16: return launch_assign_ks<16>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, stream);
    case 32: return launch_assign_ks<32>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_merge(const Plan &pl, const uint16_t *X, const uint16_t *C,
                        const float *norms, int N, int D, int K, int32_t *labels,
                        float *min_dist, const float *ws_score, const int32_t *ws_label,
                        const float *ws_xx, hipStream_t stream) {
    const int blocks = (N + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(kThreads), 0, stream, ws_score,
                       ws_label, ws_xx, pl.splits, X, C, norms, N, D, K, labels, min_dist);
    return hipGetLastError();
}

Plan make_plan(int64_t N, int64_t D, int64_t K, int force_path, int force_splits) {
    Plan pl{};
    int ks_needed = static_cast<int>((D + 15) / 16);
    int ks = 1;
    while (ks < ks_needed)
        ks <<= 1;
    pl.ks = ks;
    pl.ppw = points_per_wg(ks);
    pl.bk = k_block_rows(ks);
    pl.wgs = static_cast<int>((N + pl.ppw - 1) / pl.ppw);
    const int nkb = static_cast<int>((K + pl.bk - 1) / pl.bk);   // centroid blocks

    int splits = 1;
    if (force_path == 2) {
        splits = force_splits > 0 ? force_splits : (1024 + pl.wgs - 1) / pl.wgs;
        if (splits < 1)
            splits = 1;
    } else if (force_path == 0 && pl.wgs < 512) {
        // Too few point-workgroups to give every CU two: split K as well.
        splits = (1024 + pl.wgs - 1) / pl.wgs;
    }
    if (splits > kMaxSplits)
        splits = kMaxSplits;
    if (splits > nkb)
        splits = nkb;
    const int blocks_per_split = (nkb + splits - 1) / splits;
    pl.k_chunk = blocks_per_split * pl.bk;
    pl.splits = static_cast<int>((K + pl.k_chunk - 1) / pl.k_chunk);
    pl.path = (force_path == 2 || (force_path == 0 && pl.splits > 1)) ? 2 : 1;
    if (pl.path == 1) {
        pl.splits = 1;
        pl.k_chunk = nkb * pl.bk;
    }
    return pl;
}

}  // namespace kmeans
