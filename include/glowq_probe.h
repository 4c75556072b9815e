/*
 * glowq_probe.h -- measurement probes shipped as a separate library (libglowq_probe.so) next to
 * libglowq.so.  They are not part of the forward path: the benchmark uses them to measure, on
 * the GPU it runs on, the achievable peaks its kernels are compared against (an HBM streaming
 * read and a matrix-core-only loop), next to the vendor peaks, and the floor that a sequence of
 * separate launches of given sizes allows; and a check of the decode projection hand-off.
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

/* The decode path's projection hand-off (epoch, arrivals, tagged pairs with their bounded wait;
 * the same device routines as the forward kernels) on its own, with producers the caller slows
 * down or silences.  Not a measurement: a check of the protocol that the forward kernels rely on.
 * One launch of n_prod producer and n_cons consumer workgroups (256 threads) on the workspace of
 * glowq.h (zero-filled once by glowq_workspace_init; the epoch and counters in its header, the
 * pairs after it):
 *   producer p  : reads the epoch, sleeps delay * (p + 1) / n_prod times ~8128 clocks, arrives,
 *                 then (publish == 1) writes pairs [p c, (p + 1) c) of the n_pairs (c =
 *                 ceil(n_pairs / n_prod)) with value salt + k, tagged epoch + 1
 *   consumer    : reads the epoch, arrives, then reads all n_pairs pairs through the bounded wait
 *                 and adds to counts_dev[0] the values that differ from salt + k and to
 *                 counts_dev[1] the pairs it read
 * The launch's last arrival advances the epoch by one (skipping 2^32 - 1).  An expired wait sets
 * the workspace error word (glowq_workspace_status reports GLOWQ_ERR_HANDOFF).
 *   workspace_bytes >= 8192 + 8 n_pairs; workspace 256-byte aligned; counts_dev int32 [2],
 *   16-byte aligned, accumulated into (not cleared)
 *   1 <= n_prod <= 1024, 1 <= n_cons <= 65536, 1 <= n_pairs <= 65536, 0 <= delay <= 4096
 *   publish 0 or 1; publish == 0 (every consumer thread waits out one full bounded wait, about a
 *   second) needs n_pairs <= 256 and n_cons <= 64
 * Returns -1 for an invalid argument (before any HIP call), -6 for a launch failure, else 0.
 * Asynchronous on `stream`. */
int glowq_probe_handoff(void* workspace, size_t workspace_bytes, int32_t n_prod, int32_t n_cons, int32_t n_pairs,
                        int64_t delay, int32_t publish, float salt, int32_t* counts_dev, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* GLOWQ_PROBE_H */
