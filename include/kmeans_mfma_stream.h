/*
 * kmeans_mfma_stream.h -- measurement probe shipped beside the assignment
 * library (libkmeans_mfma_stream.so); not part of the assignment path.
 *
 * A back-to-back stream of the assign kernel's MFMA at D = 128 (bf16 x bf16
 * -> fp32, 16x16x32) on operands the caller supplies, with no memory traffic or
 * epilogue in the loop.  Its flop rate is the ceiling of the matrix pipe for
 * those bit patterns on the running GPU (the part lowers its clock under
 * dense bf16 MFMA with realistic data), against which the assign kernel's
 * rate can be read.
 */
#ifndef KMEANS_MFMA_STREAM_H
#define KMEANS_MFMA_STREAM_H

#include <stdint.h>
#include <hip/hip_runtime.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Launch `workgroups` workgroups of kmeans_mfma_stream_threads() threads
 * (4 waves, 2 waves per SIMD); each wave issues 32 * (1 + 2 * floor(tiles / 2))
 * MFMAs of 16*16*32*2 flop (32 * tiles for odd `tiles`).  Asynchronous on
 * `stream`; time it with events.
 *
 *   a_rows, b_rows  bf16 [rows][128], device, 16-byte aligned: the A
 *                   (centroid-like) and B (point-like) operand rows; wave w
 *                   uses A rows 32w.. and B rows 64w.. modulo `rows`.
 *   rows            >= 1
 *   tiles           >= 1
 *   workgroups      1..65536 (two per CU fill the GPU at 2 waves per SIMD)
 *   sink            fp32 [workgroups * kmeans_mfma_stream_threads()], device,
 *                   written (keeps the results alive).
 *
 * Returns 0, 1 for an invalid argument (nothing launched), 2 if the launch
 * failed.
 */
int32_t kmeans_mfma_stream(const void *a_rows, const void *b_rows, int32_t rows,
                           int32_t tiles, int32_t workgroups, float *sink,
                           hipStream_t stream);

/* Threads per workgroup of kmeans_mfma_stream. */
int32_t kmeans_mfma_stream_threads(void);

/*
 * Shader clock sampler, to run beside another kernel (on another stream) and
 * read the clock it ran at.  Launches `workgroups` one-wave workgroups; each
 * sleeps (s_sleep) for `duration_us` microseconds of the constant 100 MHz
 * counter and writes to out[4w .. 4w+3]: the 100 MHz ticks elapsed, the
 * shader-clock ticks elapsed over the same interval (clock in MHz = 100 *
 * out[4w+1] / out[4w]), the XCD id it ran on, 0.  With the default
 * round-robin dispatch, workgroup w runs on XCD w % 8.  Asynchronous on
 * `stream`.
 *
 *   out          uint64 [4 * workgroups], device, 8-byte aligned, written
 *   workgroups   1..1024
 *   duration_us  1..10^7
 *
 * Returns 0, 1 for an invalid argument (nothing launched), 2 if the launch
 * failed.
 */
int32_t kmeans_clock_sampler(uint64_t *out, int32_t workgroups, int32_t duration_us,
                             hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KMEANS_MFMA_STREAM_H */
