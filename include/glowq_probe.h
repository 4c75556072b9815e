/*
 * glowq_probe.h -- measurement probes shipped as a separate library (libglowq_probe.so) next to
 * libglowq.so.  They are not part of the forward path: the benchmark uses them to measure, on
 * the GPU it runs on, the achievable peaks its kernels are compared against (an HBM streaming
 * read and a matrix-core-only loop), next to the vendor peaks, and the floor that a sequence of
 * separate launches of given sizes allows.
 *
 * All launch asynchronously on `stream` and return 0, or -1 for an invalid argument (checked on
 * the host before any HIP call), or -6 for a launch failure.  All pointers are device pointers
 * owned by the caller, 16-byte aligned.
 */
#ifndef GLOWQ_PROBE_H
#define GLOWQ_PROBE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read `bytes` (a multiple of 16) at src_dev with `blocks` workgroups of 256 threads; sink_dev
 * receives blocks * 256 16-byte words (the xor of what each thread read). */
int glowq_probe_read(const void* src_dev, size_t bytes, void* sink_dev, int32_t blocks, hipStream_t stream);

/* `blocks` workgroups of 4 wavefronts, each wavefront running `iters` rounds of 4 independent
 * v_mfma_f32_32x32x16_f16 on register operands; sink_dev receives blocks * 256 x 16 fp32 (each
 * lane's 16 outputs summed over the 4 chains). */
int glowq_probe_mfma_f16(int64_t iters, void* sink_dev, int32_t blocks, hipStream_t stream);

/* n streaming reads launched back to back: read i covers bytes[i] (host array; each a multiple of
 * 16, at most 256 MiB) starting where read i - 1 ended (read 0 at src_dev), with one workgroup of
 * 256 threads per 32 KiB -- the floor that n separate launches of these sizes allow, launch ramp
 * and tail included.  sink_dev receives at least max_i(bytes[i] / 32 KiB rounded up) * 256
 * 16-byte words. */
int glowq_probe_read_sequence(const void* src_dev, const int64_t* bytes, int32_t n, void* sink_dev,
                              hipStream_t stream);

/* Dense fp16 floating-point operations one glowq_probe_mfma_f16 call performs. */
double glowq_probe_mfma_f16_flops(int64_t iters, int32_t blocks);

/* Matrix-core issue rate of one fp16 instruction shape: shape 0 = v_mfma_f32_32x32x16_f16,
 * 1 = v_mfma_f32_16x16x32_f16; chains = 4, 8 or 16 independent accumulators per wave, iters
 * iterations, blocks workgroups of 4 waves; sink_dev takes blocks * 256 * 16 bytes.  Asynchronous. */
int glowq_probe_mfma_shape(int32_t shape, int32_t chains, int64_t iters, void* sink_dev, int32_t blocks,
                           hipStream_t stream);
double glowq_probe_mfma_shape_flops(int32_t shape, int32_t chains, int64_t iters, int32_t blocks);

#ifdef __cplusplus
}
#endif

#endif /* GLOWQ_PROBE_H */
