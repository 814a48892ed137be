// kmeans_kernels.hip -- gfx950 (CDNA4) kernels of the k-means assignment step.
//
// Operation (flashlib PR #22, "Optimize Blackwell k-means assignment
// reduction", Summary and "Key ideas and contributions" table): per point,
// score every centroid by s = ||c||^2 - 2 x.c and keep the lowest-index
// minimum.  Design for CDNA4, not a translation of the pages' Blackwell
// kernel:
//
//  * The x.c contraction runs on bf16 MFMA: the centroid tile (32 rows) is
//    the A operand, the points the B operand.  At D = 128 and 256 it is
//    v_mfma_f32_16x16x32_bf16 on two 16-row A blocks and 16-point B blocks
//    (8 scores per lane per point block), elsewhere v_mfma_f32_32x32x16_bf16
//    on one 32-row A block and 32-point B blocks (16 scores per lane).  Each
//    lane owns scores of ONE point per block, so the argmin needs no
//    cross-lane traffic inside the hot loop.
//  * The norm is folded into the accumulator: the points are held as -2x
//    (exact in bf16) and the MFMA's C input is the norm tile, so the MFMA
//    result is the score s itself -- no epilogue op applies the norms and no
//    LDS round trip or barrier is spent on them (the pages' "Register-staged
//    norms" / "Barrier elimination" rows reach the same goal on Blackwell).
//  * Points stay resident in VGPRs for the whole K loop; centroid blocks are
//    double-buffered through LDS with an XOR swizzle so the A-operand reads
//    (ds_read_b128, 16 or 32 rows at one column) hit distinct banks.  Buffer loads
//    return zero past the end, so ragged N, K and D need no branches.
//  * Reductions never wait on the matrix pipe: a point block's scores are
//    reduced only after the MFMAs of the next point block (or tile) have
//    been issued, so the VALU work runs while those MFMAs execute.
//  * The epilogue does not run one compare-select chain per score (the
//    pages' serial scan and its "Two-chain argmin" ILP fix): on CDNA4 an
//    index can only enter a v_cndmask as a VGPR or an inline constant, so a
//    per-score (score, index) update costs 3+ VALU ops.  Instead each tile is
//    reduced to its minimum with v_min3 (half an op per score) and the exact
//    slot is searched only when that minimum beats the running best: about
//    ln(K) times per point over a scan, though a wave (64 lanes) still takes
//    that branch on most tiles early in K and fewer later.  The lanes that
//    share a point (four, or two with 32x32x16) exchange their bests every
//    few tiles and compare against the point's best, which halves the
//    searches; where the registers allow (one point block per wave, or a
//    whole SIMD at D = 512) an improving lane only copies the tile's scores
//    and searches them once after the loop.  Ties keep the lower index at
//    every level; the lanes of a point merge by (score, index)
//    ("Deterministic winner merge").  The N x K score matrix never leaves
//    registers.
//  * min_dist is ||x||^2 + s for the winner while that expansion is
//    accurate for the wave's points, else the direct sum of (x - c)^2 over
//    the winner's row.
//  * A launch whose points exceed the last-level cache streams them past L2
//    (non-temporal loads), so they do not evict the centroid rows.
//  * A point whose every score is +inf or NaN takes a cold per-lane path
//    after the loop (rule: -inf < finite < +inf < NaN, ties to the lower
//    index).
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kmeans_internal.h"

namespace kmeans {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
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

// The values of lane l and lane l ^ OFF (OFF = 16 or 32), in registers:
// v_permlane16_swap / v_permlane32_swap of a value with its own copy leave
// the lower lane's value in one result and the upper lane's in the other,
// in both lanes of the pair (no LDS round trip, unlike ds_bpermute).
// Callers combine the two symmetrically, so which is which does not matter.
template <int OFF>
__device__ __forceinline__ void lane_pair(uint32_t x, uint32_t &u, uint32_t &w) {
    static_assert(OFF == 16 || OFF == 32, "pairs 16 or 32 lanes apart");
    if constexpr (OFF == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        u = r[0];
        w = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        u = r[0];
        w = r[1];
    }
}

// Sum of x over the lanes l, l ^ G, ... that hold one point (G = 16: four
// lanes, G = 32: two); every one of them gets the same bits.
template <int G>
__device__ __forceinline__ float point_lane_sum(float x) {
    uint32_t u, w;
    if constexpr (G == 16) {
        lane_pair<16>(__float_as_uint(x), u, w);
        x = __uint_as_float(u) + __uint_as_float(w);
    }
    lane_pair<32>(__float_as_uint(x), u, w);
    return __uint_as_float(u) + __uint_as_float(w);
}

// min(a, b) of two running bests (never NaN: they start at +inf and take
// only NaN-ignoring minima) as one v_min_f32; fminf would first quiet each
// operand with a v_max, which values that come from a lane exchange need.
__device__ __forceinline__ float min_of_finite_or_inf(uint32_t a, uint32_t b) {
    float r;
    asm volatile("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// (s, i) strictly before (so, io) under score-then-index order.
__device__ __forceinline__ bool pair_before(float s, int32_t i, float so, int32_t io) {
    return s < so || (s == so && i < io);
}

// Final label and min_dist of point n from its merged winner `lab` and the
// squared distance d to that centroid, which the caller sums directly from
// the point's and the centroid's coordinates (||x||^2 + s would cancel badly
// when ||x||^2 is much larger than the distance, e.g. for data far from the
// origin).  Cold case: no finite or -inf score won (every score +inf or NaN):
// lowest +inf index, else 0 -- found by a VALU rescan in IEEE fp32, where only
// each score's class matters, which does not depend on summation order.
__device__ void finalize_point(int n, int32_t lab, float xx, float d,
                               const uint16_t *__restrict__ X,
                               const uint16_t *__restrict__ C,
                               const float *__restrict__ norms, int D, int K,
                               int32_t *__restrict__ labels,
                               float *__restrict__ min_dist) {
    if (lab == kNoLabel) {
        const uint16_t *xr = X + static_cast<size_t>(n) * D;
        // A NaN coordinate (NaN ||x||^2) makes every score NaN: label 0.
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
        const uint16_t *cr = C + static_cast<size_t>(lab) * D;
        d = 0.0f;
        for (int j = 0; j < D; ++j) {
            const float e = widen(xr[j]) - widen(cr[j]);
            d = fmaf(e, e, d);
        }
    }
    labels[n] = lab;
    min_dist[n] = d;
}

// Whether the winner's squared distance may be taken as the expansion
// d = max(0, ||x||^2 + s) for a point with squared norm xx, at padded width
// 16 * ks.  Its fp32 rounding error grows with ||x||^2 (and ||c||^2, which
// is close to it for a point near its centroid) while the tolerance on d is
// 2e-3 (d + 1): with a typical error of about 2^-24 sqrt(D + 40) (||x||^2 +
// ||c||^2) for the D-term sums behind xx and s, the expansion is used while
// ||x||^2 <= R (d + 1), R = 2e-3 / (4 * 4 * 2^-24 * sqrt(D + 40)) (a quarter
// of the tolerance at ||c||^2 up to 3 ||x||^2), so it stays about 8x inside
// the tolerance (R = 162 at D = 128; points of zero-mean data sit near 50).
// Beyond it (data far from the origin) the distance is summed directly.
// NaN or infinite xx or d fail the test and take the direct sum too.  R per
// padded width (2097.152 / sqrt(16 ks + 40), rounded down), a compile-time
// constant shared by the assign and merge kernels, so both decide alike.
constexpr float expansion_ratio(int ks) {
    return ks <= 1 ? 280.0f : ks == 2 ? 247.0f : ks == 4 ? 205.0f
         : ks == 8 ? 161.0f : ks == 16 ? 121.0f : 89.0f;
}
__device__ __forceinline__ bool expansion_accurate(float xx, float d, int ks) {
    return xx <= expansion_ratio(ks) * (d + 1.0f);
}

// d + sum (x_e - c_e)^2 over the 8 coordinates of one 16-byte chunk, the
// point held as -2x (so x = -0.5 * that, exactly, and the fma below is the
// correctly rounded x - c), in coordinate order.
__device__ __forceinline__ float sqdiff_chunk(u32x4 xneg2, u32x4 c, float d) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const float xl = __uint_as_float(xneg2[w] << 16);
        const float xh = __uint_as_float(xneg2[w] & 0xffff0000u);
        const float cl = __uint_as_float(c[w] << 16);
        const float ch = __uint_as_float(c[w] & 0xffff0000u);
        const float el = fmaf(-0.5f, xl, -cl);
        const float eh = fmaf(-0.5f, xh, -ch);
        d = fmaf(el, el, d);
        d = fmaf(eh, eh, d);
    }
    return d;
}

// Raw buffer resource over `bytes` bytes at `base`: loads past the end
// return zero, which pads ragged N, K and D without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The same with the non-temporal hint (cache policy NT on gfx950).
__device__ __forceinline__ u32x4 load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2));
}

// An offset past every buffer's num_records: point tiles span at most 512
// KiB and a K-range at most kMaxRangeBytes (< 2^31) of centroid rows.
constexpr uint32_t kOutOfRange = 0x80000000u;
static_assert(kMaxRangeBytes < kOutOfRange, "K-range cap must leave the marker out of range");

#define KM_LDS __attribute__((address_space(3)))
// The assign kernel's lambdas must be inlined before its arrays (resident
// points, fragments, accumulators) are promoted to registers; left to the
// inliner, a late inline can leave such an array in scratch memory.
#define KM_INLINE __attribute__((always_inline))

// s_waitcnt vmcnt(0): every vector-memory load this wave issued, LDS DMAs
// included, has landed.  A workgroup barrier does not imply it on CDNA, and
// the compiler only adds it where this wave itself reads the data.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// 16 bytes per lane from a buffer straight into LDS (buffer_load_dwordx4 ...
// lds): lane i writes dst + 16*i.  The builtin exists only for the device
// target; clang's host pass (which emits the launch stubs and never runs
// this body) drops the whole kernel if it sees it, hence the guard.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, KM_LDS void *dst, uint32_t off) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, off, 0, 0, 0);
#endif
}

// Lowest row, among the rows one lane holds in a tile, whose score equals m
// (the minimum of those scores and of the running best, which m beats).
// The scores come in pairs, in the order the running minimum took them: t[k]
// is that minimum after pair k, so the first k with t[k] == m names the
// first pair holding m (the last pair if none does), and one more compare
// tells whether it is the pair's first score.  v_cmp_eq_f32 treats -0 and +0
// as equal, as '==' does; a NaN score never equals m.  Written as assembly:
// the compares go to separate SGPR pairs, each read two or more
// instructions after it is written, so no wait states are needed (the
// compiler's form sends every compare through VCC and waits two cycles
// before each select).  Runs only on lanes whose best improved (under the
// exec mask of the caller's branch).
//
// 16x16x32 layout: scores a[0..3] are tile rows 0..3, b[0..3] rows 16..19
// (plus the lane's 4 * (lane / 16), added by the caller); pairs (a0, a1),
// (a2, a3), (b0, b1), (b2, b3).
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ int lowest_row_of_min_16x16(const f32x4 &a, const f32x4 &b,
                                                       const float (&t)[4], float m) {
    int row = 0;
#if defined(__HIP_DEVICE_COMPILE__)
    int e, r;
    uint64_t k1, k2, k3, kd, kc;
    asm volatile(
        "v_cmp_eq_f32_e64 %[k3], %[t3], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k2], %[t2], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k1], %[t1], %[m]\n\t"
        "v_cndmask_b32_e64 %[e], %[b2], %[b0], %[k3]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[a2], %[k2]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[a0], %[k1]\n\t"
        "v_cmp_neq_f32_e64 %[kd], %[e], %[m]\n\t"
        "v_cndmask_b32_e64 %[r], 18, 16, %[k3]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 2, %[k2]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 0, %[k1]\n\t"
        "v_addc_co_u32_e64 %[row], %[kc], %[r], 0, %[kd]"
        : [row] "=&v"(row), [e] "=&v"(e), [r] "=&v"(r), [k1] "=&s"(k1), [k2] "=&s"(k2),
          [k3] "=&s"(k3), [kd] "=&s"(kd), [kc] "=&s"(kc)
        : [m] "v"(m), [t1] "v"(t[0]), [t2] "v"(t[1]), [t3] "v"(t[2]), [a0] "v"(a[0]),
          [a2] "v"(a[2]), [b0] "v"(b[0]), [b2] "v"(b[2]));
#endif
    return row;
}

// 32x32x16 layout: score e (0..15) is tile row 8 * (e / 4) + e % 4 (plus the
// lane's 4 * (lane / 32)); pairs (s0, s1), (s2, s3), ..., (s14, s15).
__device__ __forceinline__ int lowest_row_of_min_32x32(const f32x16 &s, const float (&t)[8],
                                                       float m) {
    int row = 0;
#if defined(__HIP_DEVICE_COMPILE__)
    int e, r;
    uint64_t k1, k2, k3, k4, k5, k6, k7, kd, kc;
    asm volatile(
        "v_cmp_eq_f32_e64 %[k7], %[t7], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k6], %[t6], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k5], %[t5], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k4], %[t4], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k3], %[t3], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k2], %[t2], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[k1], %[t1], %[m]\n\t"
        "v_cndmask_b32_e64 %[e], %[s14], %[s12], %[k7]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[s10], %[k6]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[s8], %[k5]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[s6], %[k4]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[s4], %[k3]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[s2], %[k2]\n\t"
        "v_cndmask_b32_e64 %[e], %[e], %[s0], %[k1]\n\t"
        "v_cmp_neq_f32_e64 %[kd], %[e], %[m]\n\t"
        "v_cndmask_b32_e64 %[r], 26, 24, %[k7]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 18, %[k6]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 16, %[k5]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 10, %[k4]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 8, %[k3]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 2, %[k2]\n\t"
        "v_cndmask_b32_e64 %[r], %[r], 0, %[k1]\n\t"
        "v_addc_co_u32_e64 %[row], %[kc], %[r], 0, %[kd]"
        : [row] "=&v"(row), [e] "=&v"(e), [r] "=&v"(r), [k1] "=&s"(k1), [k2] "=&s"(k2),
          [k3] "=&s"(k3), [k4] "=&s"(k4), [k5] "=&s"(k5), [k6] "=&s"(k6), [k7] "=&s"(k7),
          [kd] "=&s"(kd), [kc] "=&s"(kc)
        : [m] "v"(m), [t1] "v"(t[0]), [t2] "v"(t[1]), [t3] "v"(t[2]), [t4] "v"(t[3]),
          [t5] "v"(t[4]), [t6] "v"(t[5]), [t7] "v"(t[6]), [s0] "v"(s[0]), [s2] "v"(s[2]),
          [s4] "v"(s[4]), [s6] "v"(s[6]), [s8] "v"(s[8]), [s10] "v"(s[10]),
          [s12] "v"(s[12]), [s14] "v"(s[14]));
#endif
    return row;
}

// The same without the running minima (fewer live registers, where the
// register budget has no room for them): one compare/select per score,
// from the last score to the first, through three rotating SGPR pairs.
__device__ __forceinline__ int lowest_row_of_min_32x32_chain(const f32x16 &s, float m) {
    int row = 0;
#if defined(__HIP_DEVICE_COMPILE__)
    uint64_t ka, kb, kc;
    asm volatile(
        "v_cmp_eq_f32_e64 %[ka], %[s15], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[kb], %[s14], %[m]\n\t"
        "v_cmp_eq_f32_e64 %[kc], %[s13], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], 0, 27, %[ka]\n\t"
        "v_cmp_eq_f32_e64 %[ka], %[s12], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 26, %[kb]\n\t"
        "v_cmp_eq_f32_e64 %[kb], %[s11], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 25, %[kc]\n\t"
        "v_cmp_eq_f32_e64 %[kc], %[s10], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 24, %[ka]\n\t"
        "v_cmp_eq_f32_e64 %[ka], %[s9], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 19, %[kb]\n\t"
        "v_cmp_eq_f32_e64 %[kb], %[s8], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 18, %[kc]\n\t"
        "v_cmp_eq_f32_e64 %[kc], %[s7], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 17, %[ka]\n\t"
        "v_cmp_eq_f32_e64 %[ka], %[s6], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 16, %[kb]\n\t"
        "v_cmp_eq_f32_e64 %[kb], %[s5], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 11, %[kc]\n\t"
        "v_cmp_eq_f32_e64 %[kc], %[s4], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 10, %[ka]\n\t"
        "v_cmp_eq_f32_e64 %[ka], %[s3], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 9, %[kb]\n\t"
        "v_cmp_eq_f32_e64 %[kb], %[s2], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 8, %[kc]\n\t"
        "v_cmp_eq_f32_e64 %[kc], %[s1], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 3, %[ka]\n\t"
        "v_cmp_eq_f32_e64 %[ka], %[s0], %[m]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 2, %[kb]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 1, %[kc]\n\t"
        "v_cndmask_b32_e64 %[row], %[row], 0, %[ka]"
        : [row] "=&v"(row), [ka] "=&s"(ka), [kb] "=&s"(kb), [kc] "=&s"(kc)
        : [m] "v"(m), [s0] "v"(s[0]), [s1] "v"(s[1]), [s2] "v"(s[2]), [s3] "v"(s[3]),
          [s4] "v"(s[4]), [s5] "v"(s[5]), [s6] "v"(s[6]), [s7] "v"(s[7]), [s8] "v"(s[8]),
          [s9] "v"(s[9]), [s10] "v"(s[10]), [s11] "v"(s[11]), [s12] "v"(s[12]),
          [s13] "v"(s[13]), [s14] "v"(s[14]), [s15] "v"(s[15]));
#endif
    return row;
}

// One workgroup = WAVES waves (8 up to D = 256, so that one centroid stream
// per CU feeds two waves per SIMD; 4 at D = 512, one wave per SIMD); wave w owns P blocks of
// 32 points.  assign_tile is the whole computation for one point tile (the
// workgroup's WAVES * P * 32 points) against one K-range; assign_kernel runs
// it for tile x = blockIdx.x and K-range y = blockIdx.y, assign_queue_kernel
// for a sequence of tiles taken from a queue.
//
// Data movement.  Centroid rows stream through two LDS stages in blocks of
// BK rows.  Each block is copied global -> LDS by buffer_load ... lds (no
// staging registers); its norms go through one register per thread.  One
// barrier per block, at the start of the block's last tile, publishes the
// next block (each wave first waits for its own DMAs); by then every wave
// has also finished reading the current block's stage (the last tile's
// fragments were read one tile earlier), so the DMA for the block after next
// goes into that stage right behind the barrier and has a whole block of
// compute to land.  The two stages are distinct arrays and the block loop is
// unrolled by two, so the compiler can tell a ds_read of one stage from a
// DMA into the other and does not wait on the DMA.
//
// Per tile (32 centroid rows) a wave issues P*KS MFMAs; right after the last
// MFMA that reads A fragment ks, the fragment of the NEXT tile is read into
// the same registers, so LDS latency hides behind the MFMA chain.
//
// Reduction per (tile, point block), per lane (16 scores of one point):
//   m = min(best, s_0..s_15)           8 v_min3 (NaN inputs are ignored)
//   if m < best (strict; taken less and less often as K advances):
//       slot = lowest r with s_r == m  (compare/select pairs, no stalls)
//       best = m, best_tile = tile, best_slot = slot
// m is always one of its inputs, so the winner is exact; a strict '<' keeps
// the earlier tile on equal scores, and the slot search keeps the lower row.
template <int G, int KS, int P, int BK, int WAVES>
__device__ KM_INLINE inline void assign_tile(
    int tile_x, int tid, const uint16_t *__restrict__ X, const uint16_t *__restrict__ C,
    const float *__restrict__ norms, int N, int D, int K, int k_chunk, int write_partials,
    int x_stream, int32_t *__restrict__ labels, float *__restrict__ min_dist,
    float *__restrict__ ws_score, int32_t *__restrict__ ws_label, float *__restrict__ ws_xx) {
    // MFMA geometry.  G = 32: v_mfma_f32_32x32x16_bf16, one 32-row A block
    // per tile, 32-point B blocks, k-steps of 16; lane = (pcol = lane % 32,
    // kq = lane / 32); accumulator element e is tile row 8(e/4) + 4kq + e%4.
    // G = 16: v_mfma_f32_16x16x32_bf16, two 16-row A blocks per tile, each
    // 32-point block split into two 16-point B blocks, k-steps of 32; lane =
    // (pcol = lane % 16, kq = lane / 16); element e of A block m is tile row
    // 16m + 4kq + e.  Either way a lane holds scores of one point only, and
    // the 64 / G lanes with the same pcol share that point.
    constexpr int KSTEP = G == 32 ? 16 : 32;
    constexpr int NKS = KS * 16 / KSTEP;       // MFMA k-steps over the padded row
    static_assert(NKS >= 1 && NKS * KSTEP == KS * 16, "padded D must cover whole k-steps");
    constexpr int MB = 32 / G;                 // A row blocks per 32-row tile
    constexpr int PB = P * (32 / G);           // B point blocks per wave
    constexpr int AV = G * G / 64;             // accumulator floats per lane per MFMA
    typedef float accv __attribute__((ext_vector_type(AV)));
    constexpr int S = 2 * KS;                  // 16-byte chunks per centroid row
    constexpr int ROW_BYTES = 16 * S;
    constexpr int TB = BK / kTileRows;         // tiles per block
    constexpr int STAGE_BYTES = BK * ROW_BYTES;
    constexpr int DMA_PER_WAVE = STAGE_BYTES / (1024 * WAVES);
    static_assert(STAGE_BYTES % (1024 * WAVES) == 0, "block must split into 1 KiB DMAs");
    static_assert(BK % kTileRows == 0 && BK <= 64 * WAVES, "block shape");
    // Centroid blocks per best-sharing period: about 8 tiles (256 rows).  A
    // CPU count over the headline workload's scores puts the search branch
    // at 0.64 of (point block, tile) steps without sharing, 0.32 with a share
    // every 8 tiles and 0.30 with one every tile.
    constexpr int SHARE_BLOCKS = TB >= 8 ? 1 : 8 / TB;

    __shared__ __attribute__((aligned(16))) uint8_t c_st0[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t c_st1[STAGE_BYTES];
    __shared__ __attribute__((aligned(16))) float n_st0[BK];
    __shared__ __attribute__((aligned(16))) float n_st1[BK];

    const int lane = tid & 63;
    // Wave-uniform, and said so: the LDS addresses of the DMAs below (M0)
    // and the wave's branches are then scalar arithmetic.
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pcol = lane % G;   // point column of a B block; row of an A block
    const int kq = lane / G;     // which 8-element group of a k-step

    const int split = blockIdx.y;
    const int k_begin = split * k_chunk;
    const int k_rows = min(K, k_begin + k_chunk) - k_begin;
    const int wg_point0 = tile_x * (WAVES * P * kTileCols);
    const int wg_points = min(N - wg_point0, WAVES * P * kTileCols);
    const uint32_t row_bytes = static_cast<uint32_t>(D) * 2u;

    u32x4 xb[PB][NKS];   // resident points (-2x), loaded below
    float xx[PB];

    // ---- centroid blocks: DMA into the LDS ring, norms via one register ----
    const uint16_t *c_range = C + static_cast<size_t>(k_begin) * D;
    const __amdgpu_buffer_rsrc_t nr = make_rsrc(norms + k_begin, static_cast<uint32_t>(k_rows) * 4u);
    // Lane `lane` of DMA i writes LDS bytes [o, o+16) of the stage; fetch the
    // global chunk that the swizzled layout puts there (XOR is its own inverse).
    uint32_t dma_src[DMA_PER_WAVE];
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int o = (wave * DMA_PER_WAVE + i) * 1024 + lane * 16;
        const int r = o / ROW_BYTES, c = swz<S>(r, (o % ROW_BYTES) / 16);
        dma_src[i] = c * 8 < D ? static_cast<uint32_t>(r) * row_bytes + c * 16 : kOutOfRange;
    }
    // One buffer resource per block (blk < the range's block count, so its
    // size is positive), built with scalar arithmetic: each lane's offset
    // is then dma_src as it stands, where an offset into one resource for
    // the whole range cost an add, a compare and a select per DMA.  Rows
    // past the range and the padding chunks stay out of range and land as
    // zeros, as before.
    auto dma = [&](int blk, uint8_t *stage) KM_INLINE {
        const __amdgpu_buffer_rsrc_t rb =
            make_rsrc(c_range + static_cast<size_t>(blk) * BK * D,
                      __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(k_rows - blk * BK) * row_bytes));
#pragma unroll
        for (int i = 0; i < DMA_PER_WAVE; ++i)
            dma16(rb, (KM_LDS void *)(stage + (wave * DMA_PER_WAVE + i) * 1024), dma_src[i]);
    };
    uint32_t nbits = 0;
    bool nvalid = false;
    auto load_norm = [&](int blk) KM_INLINE {
        if (tid < BK) {
            const int r = blk * BK + tid;
            nbits = static_cast<uint32_t>(
                __builtin_amdgcn_raw_buffer_load_b32(nr, static_cast<uint32_t>(r) * 4u, 0, 0));
            nvalid = r < k_rows;
        }
    };
    auto write_norm = [&](float *stage) KM_INLINE {
        // Rows past the range score NaN, which never wins.
        if (tid < BK)
            stage[tid] = nvalid ? __uint_as_float(nbits) : __builtin_nanf("");
    };

    // Per-lane LDS read offsets inside a tile (tiles start at multiples of 32
    // rows, where the swizzle pattern repeats): A block m, k-step ks.
    int a_off[MB][NKS];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int row = m * G + pcol;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            a_off[m][ks] = row * ROW_BYTES + swz<S>(row, ks * (KSTEP / 8) + kq) * 16;
    }
    // Where two stages span more than 64 KiB of LDS, stage 1's reads lie
    // beyond a ds_read's 16-bit offset, so its per-lane offsets are kept with
    // the stage's address added (opaque to the compiler, which would
    // otherwise fold the stage address into each read's constant and add it
    // on the VALU; the low 32 bits of a flat LDS address are its LDS
    // offset): every fragment read is then one base register plus the tile's
    // row offset as the immediate.  Smaller stages need no such
    // registers; at D = 512 the 32 registers they take cost more than the
    // adds they save (3% slower at 262144 x 512 x 4096; +0.9% at D = 128,
    // 8 registers, and part of the D = 256 gain below, 16 registers).
    constexpr bool ST1_BASE = 2 * STAGE_BYTES > 65536 && MB * NKS <= 16;
    uint32_t a_off1[ST1_BASE ? MB : 1][ST1_BASE ? NKS : 1];
#pragma unroll
    for (int m = 0; m < (ST1_BASE ? MB : 0); ++m)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            a_off1[m][ks] = static_cast<uint32_t>(a_off[m][ks]) +
                            static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
                                static_cast<const uint8_t *>(c_st1)));
            asm volatile("" : "+v"(a_off1[m][ks]));
        }
    auto read_a = [&](const uint8_t *stage, int r0, int m, int ks) KM_INLINE {
        if constexpr (ST1_BASE) {
            if (stage == c_st1) {
                const uint32_t addr = a_off1[m][ks] + static_cast<uint32_t>(r0 * ROW_BYTES);
                return __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<KM_LDS const u32x4 *>(static_cast<uintptr_t>(addr)));
            }
        }
        return __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4 *>(&stage[r0 * ROW_BYTES + a_off[m][ks]]));
    };
    // Norm tile as the MFMA C input, element e of A block m at its tile row.
    auto read_n = [&](const float *stage, int r0, accv (&v)[MB]) KM_INLINE {
        if constexpr (G == 32) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 t = *reinterpret_cast<const f32x4 *>(&stage[r0 + 8 * q + 4 * kq]);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[0][4 * q + e] = t[e];
            }
        } else {
#pragma unroll
            for (int m = 0; m < MB; ++m)
                v[m] = *reinterpret_cast<const f32x4 *>(&stage[r0 + 16 * m + 4 * kq]);
        }
    };
    bf16x8 a[MB][NKS];
    accv ninit[MB];

    // Where the registers allow it (one point block per wave, or the D = 512
    // shape with a whole SIMD's registers), a lane whose best improves only
    // saves that tile's scores and the exact slot is searched in them once,
    // after the loop (DEFER); elsewhere the slot is searched on the spot.
    // Either way it is the lowest row holding the best score, so the outputs
    // are the same bits.
    constexpr bool DEFER = (P == 1 && KS <= 8) || KS >= 32;
    float bs[PB];
    int32_t bt[PB], bo[PB];
    accv sv[DEFER ? PB : 1][MB];
#pragma unroll
    for (int p = 0; p < PB; ++p) {
        bs[p] = INFINITY;
        bt[p] = kNoLabel;
        bo[p] = 0;
    }
    if constexpr (DEFER) {
#pragma unroll
        for (int p = 0; p < PB; ++p)
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int r = 0; r < AV; ++r)
                    sv[p][m][r] = INFINITY;
    }
    // The lanes that hold one point (64 / G of them, each seeing a quarter or
    // a half of every tile's rows) take the point's running best as their own
    // threshold.  A lane whose best is beaten by another lane's drops its
    // record (tile kNoLabel, which loses every tie in the final merge) and
    // keeps only the threshold, so it searches for a slot only when it finds
    // a score below the point's best, not merely below its own: the search
    // branch is taken about half as often.  Exact and tie-safe: a lane
    // holding the point's best keeps its record, and everything found after
    // the exchange lies in later tiles (higher indices), where a strict '<'
    // against an equal threshold leaves the earlier record in place.
    auto share_best = [&](int p) KM_INLINE {
        float pb = bs[p];
        uint32_t u, w;
        if constexpr (G == 16) {
            lane_pair<16>(__float_as_uint(pb), u, w);
            pb = min_of_finite_or_inf(u, w);
        }
        lane_pair<32>(__float_as_uint(pb), u, w);
        pb = min_of_finite_or_inf(u, w);
        bt[p] = pb < bs[p] ? kNoLabel : bt[p];
        bs[p] = pb;
    };
    // Fold the scores of point block p in v (centroid kt + the element's tile
    // row, as the lowest_row_of_min_* helpers map it, + 4*kq) into that
    // block's running best; first share the best between the point's lanes
    // when `share` (wave-uniform).
    auto reduce = [&](int p, const accv (&v)[MB], int kt, bool share) KM_INLINE {
        if (share)
            share_best(p);
        // Running minimum over the scores in pairs; t[k] after pair k.
        float t[MB * AV / 2];
        float mn = bs[p];
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < AV; r += 2) {
                mn = __builtin_fminf(__builtin_fminf(mn, v[m][r]), v[m][r + 1]);
                t[(m * AV + r) / 2] = mn;
            }
        const bool improved = mn < bs[p];
        bs[p] = mn;                // mn <= bs[p]: the same value when not improved
        // 16x16x32 tiles at D = 128 and 256: the scheduler otherwise issues
        // this block's dependent v_min3 chain as a burst after six of the
        // next block's MFMAs; one VALU op after each of the first five
        // MFMAs, then the block's other MFMAs (3 of 8 at D = 128, 11 of 16
        // at D = 256), measured faster: wide D = 128 0.5-0.7% (with the
        // priority split below), narrow D = 128 1.2-2.8%, D = 256 0.5-1.4%;
        // at D = 64 (4 MFMAs per block) 1-2.5% slower, so not there.
        if constexpr (G == 16 && KS >= 8) {
#pragma unroll
            for (int i = 0; i < 5; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // one VALU op
            }
            __builtin_amdgcn_sched_group_barrier(0x008, MB * NKS - 5, 0);
        }
        if (improved) {
            bt[p] = kt;
            if constexpr (DEFER) {
                // Only the improving lanes (exec mask) copy the tile's
                // scores, two per v_mov_b64, where the search costs a compare
                // and a select per pair of scores.  As assembly, so that the
                // compiler keeps the copies inside the branch rather than
                // turning them into a select per score on every step.
#pragma unroll
                for (int m = 0; m < MB; ++m)
#pragma unroll
                    for (int r = 0; r < AV; r += 2) {
                        f32x2 d;
                        const f32x2 src = {v[m][r], v[m][r + 1]};
                        asm volatile("v_mov_b64 %0, %1" : "=v"(d) : "v"(src));
                        sv[p][m][r] = d[0];
                        sv[p][m][r + 1] = d[1];
                    }
            } else {
                int slot;
                if constexpr (G == 16)
                    slot = lowest_row_of_min_16x16(v[0], v[1], t, mn);
                else
                    slot = lowest_row_of_min_32x32(v[0], t, mn);
                bo[p] = slot;
            }
        }
    };
    // Lowest row of the saved tile whose score equals the block's best (the
    // minimum of the saved scores whenever the record is valid).
    auto saved_slot = [&](int p) KM_INLINE {
        if constexpr (!DEFER) {
            return bo[p];
        } else if constexpr (G == 32 && KS >= 32) {
            return lowest_row_of_min_32x32_chain(sv[p][0], bs[p]);
        } else {
            float t[MB * AV / 2];
            float mn = INFINITY;
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int r = 0; r < AV; r += 2) {
                    mn = __builtin_fminf(__builtin_fminf(mn, sv[p][m][r]), sv[p][m][r + 1]);
                    t[(m * AV + r) / 2] = mn;
                }
            if constexpr (G == 16)
                return lowest_row_of_min_16x16(sv[p][0], sv[p][1], t, bs[p]);
            else
                return lowest_row_of_min_32x32(sv[p][0], t, bs[p]);
        }
    };

    // Every reduction reads MFMA results issued a whole chain earlier.  With
    // several point blocks per wave, point block p's MFMAs are issued, then
    // block p-1 is reduced while they run (the previous tile's last block
    // after the first block of this tile).  With one block per wave, two
    // accumulator sets alternate between tiles and the previous tile is
    // reduced while this one's MFMAs run.  The set read first holds +inf.
    // At D >= 256 with G = 32 the second set does not fit the register
    // budget: a tile is reduced right after its own MFMAs and the other wave
    // of the SIMD keeps the matrix pipe busy meanwhile.
    constexpr int NACC = PB > 1 ? PB : (KS <= 8 ? 2 : 1);
    static_assert(NACC != 2 || PB > 1 || TB % 2 == 0, "tile parity must repeat in every block");
    accv acc[NACC][MB];
    if constexpr (NACC > 1) {
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int r = 0; r < AV; ++r)
                acc[NACC - 1][m][r] = INFINITY;
    }
    auto mfma = [](const bf16x8 &x, const bf16x8 &y, const accv &c) KM_INLINE {
        if constexpr (G == 32)
            return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c, 0, 0, 0);
        else
            return __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, y, c, 0, 0, 0);
    };
    // One tile (j-th of its block, first centroid kt): MFMAs with the
    // current operands (a, ninit), whose registers are refilled with the next
    // tile's fragments right after their last use, interleaved with the
    // reductions.
    // `share`: wave-uniform, true when this tile's block starts a sharing
    // period; the best is shared right before each point block folds the
    // period's first tile.
    auto tile = [&](const uint8_t *next_c, const float *next_n, int next_r0, int kt, int j,
                    bool share) KM_INLINE {
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            accv (&dst)[MB] = acc[PB > 1 ? p : (NACC == 2 ? (j & 1) : 0)];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
                for (int m = 0; m < MB; ++m)
                    dst[m] = mfma(a[m][ks], __builtin_bit_cast(bf16x8, xb[p][ks]),
                                  ks == 0 ? ninit[m] : dst[m]);
                if (p == PB - 1) {
#pragma unroll
                    for (int m = 0; m < MB; ++m)
                        a[m][ks] = read_a(next_c, next_r0, m, ks);
                    if (ks == 0)
                        read_n(next_n, next_r0, ninit);
                }
            }
            if (NACC == 1)
                reduce(0, acc[0], kt, share && j == 0);
            else if (PB == 1)
                reduce(0, acc[(j + 1) & 1], kt - kTileRows, share && j == 1);
            else if (p == 0)
                reduce(PB - 1, acc[PB - 1], kt - kTileRows, share && j == 1);
            else
                reduce(p - 1, acc[p - 1], kt, share && j == 0);
        }
    };

    const int nblocks = (k_rows + BK - 1) / BK;
    dma(0, c_st0);
    load_norm(0);

    // ---- resident points: -2x as MFMA B fragments, and ||x||^2 ----
    // Loaded after block 0's DMA is issued, so that the conversion below,
    // which waits for the points, does not hold the DMA back.
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(X + static_cast<size_t>(wg_point0) * D,
                                                static_cast<uint32_t>(wg_points) * row_bytes);
    // x_stream (wave-uniform): the launch's points are larger than the
    // last-level cache, so they are loaded with the non-temporal hint and do
    // not push the centroid rows out of L2.
    auto load_points = [&](auto nt) KM_INLINE {
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            const uint32_t prow = static_cast<uint32_t>(wave * P * kTileCols + p * G + pcol);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c0 = ks * KSTEP + kq * 8;
                const uint32_t off = c0 < D ? prow * row_bytes + c0 * 2 : kOutOfRange;
                xb[p][ks] = decltype(nt)::value ? load16_nt(xr, off) : load16(xr, off);
            }
        }
    };
    if (x_stream)
        load_points(std::true_type{});
    else
        load_points(std::false_type{});
    // Keep the conversion below the loads: pulled up between them, each of its
    // waits would also wait for block 0's DMA (loads complete in order).
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < PB; ++p) {
        xx[p] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            xb[p][ks] = neg2_and_square(xb[p][ks], xx[p]);
        xx[p] = point_lane_sum<G>(xx[p]);
    }

    wait_vmem();      // block 0, its norms and the points, in one round trip
    write_norm(n_st0);
    __syncthreads();
    // Block 1 is first read after block 0's barrier, a whole block later.
    if (nblocks > 1) {
        dma(1, c_st1);
        load_norm(1);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            a[m][ks] = read_a(c_st0, 0, m, ks);
    read_n(n_st0, 0, ninit);

    // Block b lives in stage cc/nc, block b+1 in cn/nn; block b+2 is fetched
    // into cc/nc once the barrier shows nobody reads block b any more.
    // Alternating wave priority pays where blocks hold eight tiles (D = 128)
    // or four (D = 256: with 128-row blocks and the stage-1 base registers,
    // 2.4-3.0% faster than 64-row blocks without them; with two tiles per
    // block it measured 0.7% slower).  With four-wave workgroups the waves
    // sharing a SIMD belong to different workgroups.
    constexpr bool kAlternatePriority = WAVES == 8 && (TB == 8 || TB == 4);
    auto do_block = [&](int b, uint8_t *cc, float *nc, uint8_t *cn, float *nn) KM_INLINE {
        const int kb = k_begin + b * BK;
        const bool share = b % SHARE_BLOCKS == 0;
#pragma unroll
        for (int j = 0; j < TB; ++j) {
            // Waves w and w + 4 of an eight-wave workgroup share a SIMD, and
            // when both can issue the older one goes first: it reaches the
            // block's barrier early and waits there (29% of the K loop for
            // waves 0-3 against 2% for waves 4-7, D = 128) while its partner
            // runs alone.  Giving each wave of the pair the higher priority
            // for alternate pairs of tiles keeps them level (10% and 2% with
            // a switch every tile; every two tiles measured 0.3-0.5% faster
            // than every tile or every four).  On the wide D = 128 tile the
            // older wave leads on 3 of the 8 tiles (0, 1 and 4; bit j of
            // kOlderLeads), which measured 0.1-0.3% faster again there and
            // 2% slower on narrow tiles.
            if constexpr (kAlternatePriority) {
                if constexpr (KS == 8 && P > 1) {
                    constexpr unsigned kOlderLeads = 0x13u;
                    if (wave < WAVES / 2) {
                        if ((kOlderLeads >> j) & 1u) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
                    } else {
                        if ((kOlderLeads >> j) & 1u) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1);
                    }
                } else if (wave < WAVES / 2) {
                    if (j & 2) __builtin_amdgcn_s_setprio(0); else __builtin_amdgcn_s_setprio(1);
                } else {
                    if (j & 2) __builtin_amdgcn_s_setprio(1); else __builtin_amdgcn_s_setprio(0);
                }
            }
            if (j + 1 < TB) {
                tile(cc, nc, (j + 1) * kTileRows, kb + j * kTileRows, j, share);
            } else {
                if (b + 1 < nblocks) {
                    write_norm(nn);
                    wait_vmem();              // this wave's DMA of block b+1 ...
                    __syncthreads();          // ... and everybody else's
                    if (b + 2 < nblocks) {
                        dma(b + 2, cc);
                        load_norm(b + 2);
                    }
                }
                tile(cn, nn, 0, kb + j * kTileRows, j, share);
            }
        }
    };
    for (int b = 0; b < nblocks; b += 2) {
        do_block(b, c_st0, n_st0, c_st1, n_st1);
        if (b + 1 >= nblocks)
            break;
        do_block(b + 1, c_st1, n_st1, c_st0, n_st0);
    }
    if constexpr (NACC > 1)   // the last tile's last point block
        reduce(PB - 1, acc[PB > 1 ? PB - 1 : ((TB - 1) & 1)],
               k_begin + (nblocks - 1) * BK + (TB - 1) * kTileRows, false);
    if constexpr (kAlternatePriority)
        __builtin_amdgcn_s_setprio(0);

    // ---- merge the lanes that hold the same point ----
    int32_t lab[PB];
    float win[PB];
#pragma unroll
    for (int p = 0; p < PB; ++p) {
        float s = bs[p];
        int32_t i = bt[p] == kNoLabel ? kNoLabel : bt[p] + saved_slot(p) + 4 * kq;
        auto merge = [&](auto off) KM_INLINE {
            uint32_t su, sw, iu, iw;
            lane_pair<decltype(off)::value>(__float_as_uint(s), su, sw);
            lane_pair<decltype(off)::value>(static_cast<uint32_t>(i), iu, iw);
            const bool w_first = pair_before(__uint_as_float(sw), static_cast<int32_t>(iw),
                                             __uint_as_float(su), static_cast<int32_t>(iu));
            s = __uint_as_float(w_first ? sw : su);
            i = static_cast<int32_t>(w_first ? iw : iu);
        };
        if constexpr (G == 16)
            merge(std::integral_constant<int, 16>{});
        merge(std::integral_constant<int, 32>{});
        win[p] = s;
        lab[p] = i;
    }
    if (write_partials) {
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            const int n = wg_point0 + wave * P * kTileCols + p * G + pcol;
            if (kq == 0 && n < N) {
                ws_score[static_cast<size_t>(split) * N + n] = win[p];
                ws_label[static_cast<size_t>(split) * N + n] = lab[p];
                if (split == 0)
                    ws_xx[n] = xx[p];
            }
        }
        return;
    }
    // ---- min_dist ----
    // The expansion ||x||^2 + s where it is accurate; otherwise (data far
    // from the origin, or non-finite) the sum of (x - c)^2 over the winner's
    // row, for every point of the wave if any of them needs it.
    float dist[PB];
    bool need_any = false;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
        dist[p] = fmaxf(0.0f, xx[p] + win[p]);
        need_any |= lab[p] != kNoLabel && !expansion_accurate(xx[p], dist[p], KS);
    }
    if (__any(need_any)) {
        // The packed -2x registers are read again here; made opaque, so
        // that the compiler does not keep their unpacked fp32 halves (which
        // it can see are the prologue's products) alive through the K loop.
#pragma unroll
        for (int p = 0; p < PB; ++p)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                asm volatile("" : "+v"(xb[p][ks]));
        // The winners' rows, all loads in flight together (global loads:
        // each lane has its own row, which a buffer resource, being
        // wave-uniform, cannot address without a loop over the distinct
        // rows).  kNoLabel reads row 0 (the cold path recomputes);
        // padding columns are zero.
        u32x4 cw[PB][NKS];
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            const uint16_t *row = C + static_cast<size_t>(lab[p] == kNoLabel ? 0 : lab[p]) * D;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int c0 = ks * KSTEP + kq * 8;
                cw[p][ks] = c0 < D ? *reinterpret_cast<const u32x4 *>(row + c0)
                                   : u32x4{0u, 0u, 0u, 0u};
            }
        }
        // Each lane of a point adds up the coordinates it holds (its 8-wide
        // chunk of every k-step, in order), then the point's lanes combine
        // as point_lane_sum does; merge_kernel repeats exactly this order
        // and this choice, so the direct and split paths give the same bits.
#pragma unroll
        for (int p = 0; p < PB; ++p) {
            float d = 0.0f;
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                d = sqdiff_chunk(xb[p][ks], cw[p][ks], d);
            d = point_lane_sum<G>(d);
            if (!expansion_accurate(xx[p], dist[p], KS))
                dist[p] = d;
        }
    }
#pragma unroll
    for (int p = 0; p < PB; ++p) {
        const int n = wg_point0 + wave * P * kTileCols + p * G + pcol;
        if (kq == 0 && n < N)
            finalize_point(n, lab[p], xx[p], dist[p], X, C, norms, D, K, labels, min_dist);
    }
}

template <int G, int KS, int P, int BK, int WAVES, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(WPE, WPE)))
void assign_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ C,
                   const float *__restrict__ norms, int N, int D, int K, int k_chunk,
                   int write_partials, int x_stream, int32_t *__restrict__ labels,
                   float *__restrict__ min_dist, float *__restrict__ ws_score,
                   int32_t *__restrict__ ws_label, float *__restrict__ ws_xx) {
    assign_tile<G, KS, P, BK, WAVES>(blockIdx.x, threadIdx.x, X, C, norms, N, D, K, k_chunk,
                                     write_partials, x_stream, labels, min_dist, ws_score,
                                     ws_label, ws_xx);
}

// Persistent form of the direct path: one round of workgroups that take point
// tiles from a queue until none is left.  A workgroup's first tile is its
// blockIdx.x; every later one is a ticket from queue[0] (an atomic add) plus
// gridDim.x.  The hardware hands workgroups to the eight XCDs in turn, an
// equal share each, whatever their clocks; with the queue a workgroup on a
// faster XCD simply takes more tiles.  Each tile is assign_tile, so every
// point's outputs are bitwise those of assign_kernel.  The queue counters
// (queue[0], queue[1]) must be zero at launch and are zero again when the
// launch ends: a workgroup that draws a ticket past the last tile counts
// itself out in queue[1], and the last one out resets both.  Launches that
// share a queue must not overlap (the caller keeps one queue per stream).
template <int G, int KS, int P, int BK, int WAVES, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WAVES, 64 * WAVES),
                          amdgpu_waves_per_eu(WPE, WPE)))
void assign_queue_kernel(const uint16_t *__restrict__ X, const uint16_t *__restrict__ C,
                         const float *__restrict__ norms, int N, int D, int K, int k_chunk,
                         int x_stream, int tiles, int32_t *__restrict__ labels,
                         float *__restrict__ min_dist, int *__restrict__ queue) {
    __shared__ int next_tile;
    int t = blockIdx.x;
    while (t < tiles) {
        // The thread index, opaque on every tile: otherwise the compiler
        // hoists the per-lane offsets of the tile's prologue and epilogue out
        // of this loop and holds them through the K loop, where the
        // registers are all taken.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        assign_tile<G, KS, P, BK, WAVES>(t, tid, X, C, norms, N, D, K, k_chunk, 0, x_stream,
                                         labels, min_dist, nullptr, nullptr, nullptr);
        // Every wave is done with the tile's LDS stages and with the last
        // ticket before the next one is drawn and the stages refilled.  (A
        // ticket drawn earlier, when the tile's last centroid block starts,
        // measured 1.5-3% slower: it reserves a tile ahead and so gives up
        // most of the balancing.)
        __syncthreads();
        if (tid == 0)
            next_tile = __hip_atomic_fetch_add(&queue[0], 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) + static_cast<int>(gridDim.x);
        __syncthreads();
        t = next_tile;
    }
    if (threadIdx.x == 0) {
        // Release: this workgroup's last ticket precedes its count; the
        // workgroup that brings the count to gridDim.x sees every ticket
        // drawn and leaves both counters at zero for the next launch.
        const int out = __hip_atomic_fetch_add(&queue[1], 1, __ATOMIC_ACQ_REL,
                                               __HIP_MEMORY_SCOPE_AGENT);
        if (out == static_cast<int>(gridDim.x) - 1) {
            __hip_atomic_store(&queue[0], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&queue[1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Zeroes a queue's two counters (once, when the queue is created).
__global__ void zero_queue_kernel(int *queue) {
    if (threadIdx.x < 2)
        queue[threadIdx.x] = 0;
}

// Second pass of the K-split path: (score, index) minimum over the splits,
// then the winner's squared distance summed in the order the assign kernel
// uses for the geometry G of this D (lane q of a point adds its 8-wide
// chunks q*8, q*8 + KSTEP, ...; the lanes' sums combine pairwise), so split
// and direct outputs are bitwise equal.
template <int KS, int G>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void merge_kernel(const float *__restrict__ ws_score, const int32_t *__restrict__ ws_label,
                  const float *__restrict__ ws_xx, int splits,
                  const uint16_t *__restrict__ X, const uint16_t *__restrict__ C,
                  const float *__restrict__ norms, int N, int D, int K,
                  int32_t *__restrict__ labels, float *__restrict__ min_dist) {
    constexpr int KSTEP = G == 32 ? 16 : 32;
    constexpr int LANES = 64 / G;
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
    const float xx = ws_xx[n];
    float d = fmaxf(0.0f, xx + s);
    if (i != kNoLabel && !expansion_accurate(xx, d, KS)) {
        const uint16_t *xr = X + static_cast<size_t>(n) * D;
        const uint16_t *cr = C + static_cast<size_t>(i) * D;
        float part[LANES];
#pragma unroll
        for (int q = 0; q < LANES; ++q) {
            part[q] = 0.0f;
            for (int c0 = q * 8; c0 < D; c0 += KSTEP)
                for (int e = 0; e < 8; ++e) {
                    const float diff = widen(xr[c0 + e]) - widen(cr[c0 + e]);
                    part[q] = fmaf(diff, diff, part[q]);
                }
        }
        if constexpr (LANES == 4)
            d = (part[0] + part[1]) + (part[2] + part[3]);
        else
            d = part[0] + part[1];
    }
    finalize_point(n, i, xx, d, X, C, norms, D, K, labels, min_dist);
}

// ||c_k||^2: 16 lanes per row, 16 rows per workgroup, 16-byte loads.  Every
// row is reduced with the same lane pattern, so identical rows get identical
// bits.
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void norms_kernel(const uint16_t *__restrict__ C, int K, int D, float *__restrict__ norms) {
    const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
    const int l = threadIdx.x & 15;
    const bool live = row < K;
    const float n = row_sq_norm16(C + static_cast<size_t>(live ? row : 0) * D, live ? D : 0, l);
    if (live && l == 0)
        norms[row] = n;
}

template <int KS, int G, int P>
hipError_t launch_assign_kp(const Plan &pl, const uint16_t *X, const uint16_t *C,
                            const float *norms, int N, int D, int K, int32_t *labels,
                            float *min_dist, float *ws_score, int32_t *ws_label,
                            float *ws_xx, int *queue, hipStream_t stream) {
    constexpr int BK = k_block_rows(KS);
    constexpr int WAVES = waves_per_wg(KS);
    constexpr int WPE = waves_per_simd(KS);
    static_assert(assign_wgs_per_cu(KS) >= 1, "workgroup must fit a CU");
    const int partial = ws_score != nullptr ? 1 : 0;
    const int x_stream = static_cast<int64_t>(N) * D * 2 > kStreamPointBytes ? 1 : 0;
    if (queue != nullptr) {
        // The queue path takes wide tiles only (make_plan); not instantiated
        // for narrow ones.
        if constexpr (P == wide_point_blocks(KS)) {
            hipLaunchKernelGGL((assign_queue_kernel<G, KS, P, BK, WAVES, WPE>), dim3(pl.wgs),
                               dim3(64 * WAVES), 0, stream, X, C, norms, N, D, K, pl.k_chunk,
                               x_stream, pl.tiles, labels, min_dist, queue);
            return hipGetLastError();
        }
        return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((assign_kernel<G, KS, P, BK, WAVES, WPE>), dim3(pl.wgs, pl.splits), dim3(64 * WAVES),
                       0, stream, X, C, norms, N, D, K, pl.k_chunk, partial, x_stream, labels,
                       min_dist, ws_score, ws_label, ws_xx);
    return hipGetLastError();
}

template <int KS, int G>
hipError_t launch_assign_kg(const Plan &pl, const uint16_t *X, const uint16_t *C,
                            const float *norms, int N, int D, int K, int32_t *labels,
                            float *min_dist, float *ws_score, int32_t *ws_label,
                            float *ws_xx, int *queue, hipStream_t stream) {
    constexpr int WIDE = wide_point_blocks(KS);
    if (WIDE > 1 && pl.pb == 1)
        return launch_assign_kp<KS, G, 1>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score,
                                          ws_label, ws_xx, queue, stream);
    return launch_assign_kp<KS, G, WIDE>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score,
                                         ws_label, ws_xx, queue, stream);
}

template <int KS>
hipError_t launch_assign_ks(const Plan &pl, const uint16_t *X, const uint16_t *C,
                            const float *norms, int N, int D, int K, int32_t *labels,
                            float *min_dist, float *ws_score, int32_t *ws_label,
                            float *ws_xx, int *queue, hipStream_t stream) {
    if constexpr (KS == 4) {
        if (pl.geom == 16)
            return launch_assign_kg<KS, 16>(pl, X, C, norms, N, D, K, labels, min_dist,
                                            ws_score, ws_label, ws_xx, queue, stream);
    }
    return launch_assign_kg<KS, mfma_geometry(KS)>(pl, X, C, norms, N, D, K, labels, min_dist,
                                                   ws_score, ws_label, ws_xx, queue, stream);
}

}  // namespace

hipError_t launch_norms(const uint16_t *C, int K, int D, float *norms, hipStream_t stream) {
    const int blocks = (K + 15) / 16;
    hipLaunchKernelGGL(norms_kernel, dim3(blocks), dim3(kThreads), 0, stream, C, K, D, norms);
    return hipGetLastError();
}

namespace {
hipError_t launch_assign_any(const Plan &pl, const uint16_t *X, const uint16_t *C,
                             const float *norms, int N, int D, int K, int32_t *labels,
                             float *min_dist, float *ws_score, int32_t *ws_label,
                             float *ws_xx, int *queue, hipStream_t stream) {
    switch (pl.ks) {
    case 1: return launch_assign_ks<1>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, queue, stream);
    case 2: return launch_assign_ks<2>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, queue, stream);
    case 4: return launch_assign_ks<4>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, queue, stream);
    case 8: return launch_assign_ks<8>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, queue, stream);
    case 16: return launch_assign_ks<16>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, queue, stream);
    case 32: return launch_assign_ks<32>(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label, ws_xx, queue, stream);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_assign(const Plan &pl, const uint16_t *X, const uint16_t *C,
                         const float *norms, int N, int D, int K, int32_t *labels,
                         float *min_dist, float *ws_score, int32_t *ws_label,
                         float *ws_xx, hipStream_t stream) {
    return launch_assign_any(pl, X, C, norms, N, D, K, labels, min_dist, ws_score, ws_label,
                             ws_xx, nullptr, stream);
}

hipError_t launch_assign_queue(const Plan &pl, const uint16_t *X, const uint16_t *C,
                               const float *norms, int N, int D, int K, int32_t *labels,
                               float *min_dist, int *queue, hipStream_t stream) {
    return launch_assign_any(pl, X, C, norms, N, D, K, labels, min_dist, nullptr, nullptr,
                             nullptr, queue, stream);
}

hipError_t launch_zero_queue(int *queue, hipStream_t stream) {
    hipLaunchKernelGGL(zero_queue_kernel, dim3(1), dim3(64), 0, stream, queue);
    return hipGetLastError();
}

hipError_t launch_merge(const Plan &pl, const uint16_t *X, const uint16_t *C,
                        const float *norms, int N, int D, int K, int32_t *labels,
                        float *min_dist, const float *ws_score, const int32_t *ws_label,
                        const float *ws_xx, hipStream_t stream) {
    const int blocks = (N + kThreads - 1) / kThreads;
#define KM_MERGE(KSV, GV)                                                                   \
    hipLaunchKernelGGL((merge_kernel<KSV, GV>), dim3(blocks), dim3(kThreads), 0, stream,     \
                       ws_score, ws_label, ws_xx, pl.splits, X, C, norms, N, D, K, labels,    \
                       min_dist)
    switch (pl.ks) {
    case 1: KM_MERGE(1, mfma_geometry(1)); break;
    case 2: KM_MERGE(2, mfma_geometry(2)); break;
    case 4:
        if (pl.geom == 16)
            KM_MERGE(4, 16);
        else
            KM_MERGE(4, mfma_geometry(4));
        break;
    case 8: KM_MERGE(8, mfma_geometry(8)); break;
    case 16: KM_MERGE(16, mfma_geometry(16)); break;
    case 32: KM_MERGE(32, mfma_geometry(32)); break;
    default: return hipErrorInvalidValue;
    }
#undef KM_MERGE
    return hipGetLastError();
}

int min_k_ranges(int64_t D, int64_t K) {
    int ks = 1;
    while (ks * 16 < D)
        ks <<= 1;
    const int64_t bk = k_block_rows(ks);
    const int64_t cap_blocks = kMaxRangeBytes / (D * 2) / bk;   // whole blocks per range
    const int64_t nkb = (K + bk - 1) / bk;
    const int64_t r = (nkb + cap_blocks - 1) / cap_blocks;
    return r > kMaxSplits ? kMaxSplits + 1 : static_cast<int>(r);
}

Plan make_plan(int64_t N, int64_t D, int64_t K, int force_path, int force_count,
               int compute_units) {
    Plan pl{};
    int ks_needed = static_cast<int>((D + 15) / 16);
    int ks = 1;
    while (ks < ks_needed)
        ks <<= 1;
    pl.ks = ks;
    pl.geom = ks == 4 && N * K >= kG16MinWorkAtD64 ? 16 : mfma_geometry(ks);
    pl.bk = k_block_rows(ks);
    const int nkb = static_cast<int>((K + pl.bk - 1) / pl.bk);   // centroid blocks
    const int cus = compute_units > 0 ? compute_units : kDefaultComputeUnits;
    const int resident = cus * assign_wgs_per_cu(ks);            // workgroups held at once
    const int wide = wide_point_blocks(ks);
    auto tiles_for = [&](int pb) {
        return static_cast<int>((N + points_per_wg(ks, pb) - 1) / points_per_wg(ks, pb));
    };

    // Too few wide point tiles to fill the GPU: either narrow tiles (one
    // point block per wave; only while they fit in one round and K is at
    // most 16 centroid blocks) or K split into ranges of wide tiles, as many
    // as one round holds (rounded down: a second, nearly empty round costs
    // a whole range's time) with at least two centroid blocks per range
    // (every range pays the point prologue, and the merge pass a launch).
    // The split is taken when it gives at least twice the narrow tiles'
    // workgroups, i.e. when narrow tiles would leave half the CUs idle.
    // Measured (median us, settled, scratch kept per stream; narrow / split
    // s / direct wide):
    //   N = 65536: D=64 K=4096 35.5 / s=4 39.6; D=64 K=2048 18.2 / s=4 24.5;
    //     D=64 K=16384 126.9 / s=4 109.4; D=128 K=1024 18.5 / s=2 22.4;
    //     D=128 K=2048 29.7 / 32.1; D=128 K=3072 42.2 / 43.2; D=128
    //     K=4096 54.3 / 52.7; D=128 K=512 11.6 / 15.9.
    //   smaller N: 49152 x 128 x 4096 49.0 / s=2 48.9 (s=3: 58.3);
    //     40960 x 64 x 4096 27.9 / s=6 30.5; 32768 x 128 x 4096 48.9 /
    //     s=4 33.8; 32768 x 64 x 4096 28.0 / s=8 26.0; 24576 x 128 x 4096
    //     48.0 / s=5 32.8; 16384 x 128 x 4096 47.9 / s=8 25.1; 16384 x 32 x
    //     4096 21.5 / s=8 18.7.
    //   wide tiles only: 49152 x 128 x 16384 s=2 165.6 (s=3: 212.6, direct
    //     285.6); 98304 x 128 x 4096 direct 82.3 (s=2, two rounds: 97.6).
    const int target_wgs = resident;
    int pb = wide;
    int splits = 1;
    const int wide_tiles = tiles_for(wide);
    if (force_path == 1 && force_count == 1) {
        pb = 1;
    } else if (force_path == 0 && wide_tiles < target_wgs) {
        int s = target_wgs / wide_tiles;
        if (s > nkb / 2)
            s = nkb / 2;
        if (s < 1)
            s = 1;
        const bool narrow_ok = wide > 1 && nkb <= 16 && tiles_for(1) <= resident;
        if (narrow_ok && static_cast<int64_t>(wide_tiles) * s < 2 * static_cast<int64_t>(tiles_for(1)))
            pb = 1;
        else
            splits = s;
    }
    pl.pb = pb;
    pl.ppw = points_per_wg(ks, pb);
    pl.tiles = tiles_for(pb);
    pl.wgs = pl.tiles;

    if (force_path == 2) {
        splits = force_count > 0 ? force_count : (target_wgs + pl.tiles - 1) / pl.tiles;
        if (splits < 1)
            splits = 1;
    }
    const int need = min_k_ranges(D, K);   // C over 2 GiB: split regardless
    if (splits < need)
        splits = need;
    if (splits > kMaxSplits)
        splits = kMaxSplits;
    if (splits > nkb)
        splits = nkb;
    const int blocks_per_split = (nkb + splits - 1) / splits;
    pl.k_chunk = blocks_per_split * pl.bk;
    pl.splits = static_cast<int>((K + pl.k_chunk - 1) / pl.k_chunk);
    pl.path = (force_path == 2 || (force_path == 0 && pl.splits > 1) || need > 1) ? 2 : 1;
    if (pl.path == 1) {
        pl.splits = 1;
        pl.k_chunk = nkb * pl.bk;
    }
    if (force_path == 3 && pl.path == 1) {
        // Persistent: wide tiles, one round of workgroups (one per CU unless
        // force_count names another count), never more than the tiles.
        pl.path = 3;
        const int round = force_count > 0 ? force_count : resident;
        pl.wgs = round < pl.tiles ? round : pl.tiles;
        return pl;
    }

    // Wave tail: wide tiles that fill only part of their last round (at most
    // half of it at D = 128, a quarter at D <= 64) take as long as a full
    // round.  Their points run instead as one round of narrow tiles, each
    // about half as long, in a second launch (measured: N = 300000 and
    // 600000 at D = 128, K = 4096).
    pl.tail_points = 0;
    pl.tail_wgs = 0;
    if (force_path == 0 && pl.path == 1 && pb == wide && wide > 1 && pl.tiles > resident) {
        const int rem = pl.tiles % resident;
        const int64_t tail = N - static_cast<int64_t>(pl.tiles - rem) * pl.ppw;
        const int64_t narrow_tiles = (tail + points_per_wg(ks, 1) - 1) / points_per_wg(ks, 1);
        if (rem > 0 && narrow_tiles <= resident) {
            pl.tail_points = static_cast<int>(tail);
            pl.tail_wgs = static_cast<int>(narrow_tiles);
            pl.tiles -= rem;
            pl.wgs = pl.tiles;
        }
    }
    return pl;
}

}  // namespace kmeans
