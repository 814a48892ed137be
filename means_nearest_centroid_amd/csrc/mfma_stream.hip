// mfma_stream.hip -- measurement probe, not part of the assignment path.
//
// Runs the assign kernel's matrix instruction at the headline width D = 128
// (v_mfma_f32_16x16x32_bf16, fp32 accumulate) back to back with nothing else
// in the loop: no LDS, no VALU epilogue, no global traffic.  Each wave holds
// two 16-row A blocks and four 16-column B blocks of D = 128 in VGPRs and
// issues 32 MFMAs per tile in eight chains that restart from a fixed C tile
// every tile, as the assign kernel's do.  Two waves per SIMD.
//
// The rate it reaches is the ceiling of the matrix pipe for those operand
// bit patterns on the running part: with zero operands it is close to the
// spec rate, with realistic bf16 data the part lowers its clock under this
// load, and the assign kernel cannot beat that.
#include <stdint.h>

#include "kmeans_mfma_stream.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // columns of every operand row
constexpr int kKs = kD / 32;     // k-steps per tile
constexpr int kThreads = 256;    // 4 waves

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void mfma_stream_kernel(const uint16_t *__restrict__ a_rows, const uint16_t *__restrict__ b_rows,
                        int rows, int tiles, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r16 = lane & 15, quad = lane >> 4;
    const int w = blockIdx.x * (kThreads / 64) + wave;

    // Operand fragments: A row = 16m + lane % 16, B column = 16n + lane % 16,
    // k-steps of 32 with this lane's 8-element quarter.  Rows wrap inside
    // [0, rows).
    bf16x8 a[2][kKs], b[4][kKs];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const int ar = (w * 32 + m * 16 + r16) % rows;
#pragma unroll
        for (int k = 0; k < kKs; ++k)
            a[m][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                     a_rows + static_cast<size_t>(ar) * kD + k * 32 + quad * 8));
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) {
        const int br = (w * 64 + n * 16 + r16) % rows;
#pragma unroll
        for (int k = 0; k < kKs; ++k)
            b[n][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                     b_rows + static_cast<size_t>(br) * kD + k * 32 + quad * 8));
    }
    f32x4 c0;
#pragma unroll
    for (int r = 0; r < 4; ++r)
        c0[r] = static_cast<float>(r + 4 * quad);
    // Two accumulator sets: while one tile's chains run, the previous tile's
    // results are read (one VALU op per 4 MFMAs), so no read waits on an MFMA
    // in flight.  Every chain is read, so none is optimised away.
    f32x4 acc[2][8];
    auto tile = [&](f32x4 (&out)[8]) {
        c0[0] += 0.5f;   // a different C tile each time, as the assign kernel's norm tiles
#pragma unroll
        for (int k = 0; k < kKs; ++k) {
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n)
                    out[m * 4 + n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a[m][k], b[n][k], k == 0 ? c0 : out[m * 4 + n], 0, 0, 0);
        }
    };
    float keep = 0.0f;
    tile(acc[0]);
    for (int t = 1; t < tiles; t += 2) {
        tile(acc[1]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            keep += acc[0][j][1 + j % 3];
        tile(acc[0]);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            keep += acc[1][j][1 + (j + 1) % 3];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
        keep += acc[0][j][1 + (j + 2) % 3];
    sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = keep;
}

}  // namespace

extern "C" int32_t kmeans_mfma_stream(const void *a_rows, const void *b_rows, int32_t rows,
                                      int32_t tiles, int32_t workgroups, float *sink,
                                      hipStream_t stream) {
    if (!a_rows || !b_rows || !sink || rows < 1 || tiles < 1 || workgroups < 1 ||
        workgroups > 65536)
        return 1;
    if ((reinterpret_cast<uintptr_t>(a_rows) | reinterpret_cast<uintptr_t>(b_rows)) % 16 != 0 ||
        reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return 1;
    hipLaunchKernelGGL(mfma_stream_kernel, dim3(workgroups), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t *>(a_rows), static_cast<const uint16_t *>(b_rows),
                       rows, tiles, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int32_t kmeans_mfma_stream_threads(void) { return kThreads; }

// Shader clock sampler (measurement only).  Each workgroup is one wave that
// records the shader-clock counter (s_memtime) and the constant 100 MHz
// counter (s_memrealtime) at its start and again once `ticks` 100 MHz ticks
// have passed, sleeping in between (s_sleep: it takes almost no issue slots
// from kernels that share its SIMD).  Run beside another kernel, it gives the
// clock that kernel ran at; workgroup w lands on XCD w % 8 under the default
// round-robin dispatch, and its XCD id is recorded too.
namespace {

__global__ __attribute__((amdgpu_flat_work_group_size(64, 64)))
void clock_sampler_kernel(uint64_t *__restrict__ out, uint64_t ticks) {
    const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
    const uint64_t c0 = __builtin_amdgcn_s_memtime();
    uint64_t r = r0;
    // Bounded: at most ~2^20 sleeps of ~8k cycles whatever the counters do.
    for (int i = 0; i < (1 << 20) && r - r0 < ticks; ++i) {
        __builtin_amdgcn_s_sleep(127);
        r = __builtin_amdgcn_s_memrealtime();
    }
    const uint64_t c1 = __builtin_amdgcn_s_memtime();
    if (threadIdx.x == 0) {
        uint64_t *o = out + static_cast<size_t>(blockIdx.x) * 4;
        o[0] = r - r0;
        o[1] = c1 - c0;
        o[2] = static_cast<uint64_t>(__builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)));
        o[3] = 0;
    }
}

}  // namespace

extern "C" int32_t kmeans_clock_sampler(uint64_t *out, int32_t workgroups, int32_t duration_us,
                                        hipStream_t stream) {
    if (!out || workgroups < 1 || workgroups > 1024 || duration_us < 1 || duration_us > 10000000)
        return 1;
    if (reinterpret_cast<uintptr_t>(out) % 8 != 0)
        return 1;
    hipLaunchKernelGGL(clock_sampler_kernel, dim3(workgroups), dim3(64), 0, stream, out,
                       static_cast<uint64_t>(duration_us) * 100u);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
