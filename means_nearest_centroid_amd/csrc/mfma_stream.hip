// mfma_stream.hip -- measurement probe, not part of the assignment path.
//
// Runs the assign kernel's matrix instruction (v_mfma_f32_32x32x16_bf16,
// fp32 accumulate) back to back with nothing else in the loop: no LDS, no
// VALU epilogue, no global traffic.  Each wave holds one 32-row A operand
// and two 32-column B operands of D = 128 (the headline shape's tile) in
// VGPRs and issues 16 MFMAs per tile in two chains that restart from a
// fixed C tile every tile, as the assign kernel's do.  Two waves per SIMD.
//
// The rate it reaches is the ceiling of the matrix pipe for those operand
// bit patterns on the running part: with zero operands it is close to the
// spec rate, with realistic bf16 data the part lowers its clock under this
// load, and the assign kernel cannot beat that.
#include <stdint.h>

#include "kmeans_mfma_stream.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;          // columns of every operand row
constexpr int kKs = kD / 16;     // k-steps per tile
constexpr int kThreads = 256;    // 4 waves

__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads),
                          amdgpu_waves_per_eu(2, 2)))
void mfma_stream_kernel(const uint16_t *__restrict__ a_rows, const uint16_t *__restrict__ b_rows,
                        int rows, int tiles, float *__restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 31, half = lane >> 5;
    const int w = blockIdx.x * (kThreads / 64) + wave;

    // Operand fragments: A row = lane % 32, B column = lane % 32, k-steps
    // of 16 with this lane's 8-element half.  Rows wrap inside [0, rows).
    bf16x8 a[kKs], b[2][kKs];
    const int ar = (w * 32 + col) % rows;
#pragma unroll
    for (int k = 0; k < kKs; ++k)
        a[k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                              a_rows + static_cast<size_t>(ar) * kD + k * 16 + half * 8));
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int br = (w * 64 + p * 32 + col) % rows;
#pragma unroll
        for (int k = 0; k < kKs; ++k)
            b[p][k] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(
                                                     b_rows + static_cast<size_t>(br) * kD + k * 16 + half * 8));
    }
    f32x16 c0;
#pragma unroll
    for (int r = 0; r < 16; ++r)
        c0[r] = static_cast<float>(r + 8 * half);
    // Two accumulator sets: while one tile's chains run, the previous tile's
    // results are read (one VALU op per 8 MFMAs), so no read waits on an
    // MFMA in flight.
    f32x16 acc[2][2];
    auto tile = [&](f32x16 (&out)[2]) {
        c0[0] += 0.5f;   // a different C tile each time, as the assign kernel's norm tiles
#pragma unroll
        for (int k = 0; k < kKs; ++k) {
#pragma unroll
            for (int p = 0; p < 2; ++p)
                out[p] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[p][k], k == 0 ? c0 : out[p],
                                                                 0, 0, 0);
        }
    };
    float keep = 0.0f;
    tile(acc[0]);
    for (int t = 1; t < tiles; t += 2) {
        tile(acc[1]);
        keep += acc[0][0][3] + acc[0][1][11];
        tile(acc[0]);
        keep += acc[1][0][5] + acc[1][1][13];
    }
    keep += acc[0][0][1] + acc[0][1][9];
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
