// Measurement probes (libglowq_probe.so): the achievable peaks that the forward kernels are
// compared against, measured on the same GPU in the same process.
//
//   * a streaming read: 16-byte nontemporal loads over a buffer much larger than the last-level
//     cache, eight per thread in flight, grid-stride, folded into a per-thread xor (the only
//     store) -- the HBM read rate a kernel with a perfect access pattern reaches;
//   * a matrix-core loop: v_mfma_f32_32x32x16_f16 on register operands, four independent
//     accumulators per wave, no memory traffic in the loop -- the dense fp16 rate the matrix
//     cores sustain (including any clock reduction under that load).  The 32x32x16 form is used
//     because it is the fastest fp16 matrix step here: 16x16x32 sustains about half its rate;
//   * a sequence of streaming reads, one launch per region with one workgroup per 32 KiB -- what
//     back-to-back launches of given sizes allow, launch ramp and tail included.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "glowq_probe.h"

namespace {

constexpr int64_t kSequenceMaxBlocks = 8192;  // workgroups of one read of a sequence (256 MiB)

typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f16x __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void read_kernel(const u4* __restrict__ p, uint64_t n16, u4* __restrict__ sink) {
    const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    u4 acc = {0u, 0u, 0u, 0u};
    for (uint64_t i = tid; i < n16; i += 8 * stride) {
        u4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint64_t j = i + (uint64_t)u * stride;
            v[u] = j < n16 ? __builtin_nontemporal_load(p + j) : u4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u];
    }
    sink[tid] = acc;
}

__global__ __launch_bounds__(256) void mfma_kernel(int64_t iters, f4* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    // small exact operands (no overflow over any number of iterations of a fixed sum)
    h8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)((float)((lane + e) & 3) * 0.25f);
        b[e] = (_Float16)((float)((lane * 3 + e) & 3) * 0.125f);
    }
    f16x acc[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
    }
    // lane l: the 16 outputs it holds, summed over the chains, as four f4
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        f4 v = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k = 0; k < 4; ++k) v += f4{acc[k][4 * q], acc[k][4 * q + 1], acc[k][4 * q + 2], acc[k][4 * q + 3]};
        sink[((uint64_t)blockIdx.x * 256 + threadIdx.x) * 4 + q] = v;
    }
}

// Matrix-core rate of one fp16 instruction shape with C independent accumulation chains per wave:
// SHAPE 0 = v_mfma_f32_32x32x16_f16 (16 outputs per lane), 1 = v_mfma_f32_16x16x32_f16 (4 outputs
// per lane).  Enough chains hide each instruction's latency, so the loop measures issue rate.
typedef float f4x __attribute__((ext_vector_type(4)));

template <int SHAPE, int C>
__global__ __launch_bounds__(256) void mfma_shape_kernel(int64_t iters, f4* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    h8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (_Float16)((float)((lane + e) & 3) * 0.25f);
        b[e] = (_Float16)((float)((lane * 3 + e) & 3) * 0.125f);
    }
    f4 out = {0.f, 0.f, 0.f, 0.f};
    if constexpr (SHAPE == 0) {
        f16x acc[C];
#pragma unroll
        for (int k = 0; k < C; ++k)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[k][i] = 0.f;
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < C; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < C; ++k)
#pragma unroll
            for (int i = 0; i < 16; ++i) out[i & 3] += acc[k][i];
    } else {
        f4x acc[C];
#pragma unroll
        for (int k = 0; k < C; ++k) acc[k] = f4x{0.f, 0.f, 0.f, 0.f};
        for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
            for (int k = 0; k < C; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[k], 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < C; ++k) out += acc[k];
    }
    sink[(uint64_t)blockIdx.x * 256 + threadIdx.x] = out;
}

}  // namespace

extern "C" {

int glowq_probe_mfma_shape(int32_t shape, int32_t chains, int64_t iters, void* sink_dev, int32_t blocks,
                           hipStream_t stream) {
    if (sink_dev == nullptr || blocks < 1 || iters < 0 || (shape != 0 && shape != 1)) return -1;
    if (chains != 4 && chains != 8 && chains != 16) return -1;
    if ((reinterpret_cast<uintptr_t>(sink_dev) & 15) != 0) return -1;
    const dim3 grid((unsigned)blocks), block(256);
    f4* sk = static_cast<f4*>(sink_dev);
    if (shape == 0) {
        if (chains == 4) hipLaunchKernelGGL((mfma_shape_kernel<0, 4>), grid, block, 0, stream, iters, sk);
        else if (chains == 8) hipLaunchKernelGGL((mfma_shape_kernel<0, 8>), grid, block, 0, stream, iters, sk);
        else hipLaunchKernelGGL((mfma_shape_kernel<0, 16>), grid, block, 0, stream, iters, sk);
    } else {
        if (chains == 4) hipLaunchKernelGGL((mfma_shape_kernel<1, 4>), grid, block, 0, stream, iters, sk);
        else if (chains == 8) hipLaunchKernelGGL((mfma_shape_kernel<1, 8>), grid, block, 0, stream, iters, sk);
        else hipLaunchKernelGGL((mfma_shape_kernel<1, 16>), grid, block, 0, stream, iters, sk);
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

double glowq_probe_mfma_shape_flops(int32_t shape, int32_t chains, int64_t iters, int32_t blocks) {
    // 32 x 32 x 16 = 16384 multiply-adds per instruction, 16 x 16 x 32 = 8192
    return (double)blocks * 4.0 * (double)iters * (double)chains * 32.0 * 32.0 * 16.0 * 2.0 / (shape == 0 ? 1.0 : 2.0);
}

int glowq_probe_read(const void* src_dev, size_t bytes, void* sink_dev, int32_t blocks, hipStream_t stream) {
    if (src_dev == nullptr || sink_dev == nullptr || blocks < 1 || bytes % 16 != 0) return -1;
    if ((reinterpret_cast<uintptr_t>(src_dev) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink_dev) & 15) != 0)
        return -1;
    hipLaunchKernelGGL(read_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<const u4*>(src_dev), (uint64_t)(bytes / 16), static_cast<u4*>(sink_dev));
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int glowq_probe_mfma_f16(int64_t iters, void* sink_dev, int32_t blocks, hipStream_t stream) {
    if (sink_dev == nullptr || blocks < 1 || iters < 0) return -1;
    if ((reinterpret_cast<uintptr_t>(sink_dev) & 15) != 0) return -1;
    hipLaunchKernelGGL(mfma_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters, static_cast<f4*>(sink_dev));
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int glowq_probe_read_sequence(const void* src_dev, const int64_t* bytes, int32_t n, void* sink_dev,
                              hipStream_t stream) {
    if (src_dev == nullptr || bytes == nullptr || sink_dev == nullptr || n < 1) return -1;
    if ((reinterpret_cast<uintptr_t>(src_dev) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink_dev) & 15) != 0)
        return -1;
    for (int32_t i = 0; i < n; ++i)
        if (bytes[i] < 16 || bytes[i] % 16 != 0 || (bytes[i] + 32767) / 32768 > kSequenceMaxBlocks) return -1;
    const char* p = static_cast<const char*>(src_dev);
    for (int32_t i = 0; i < n; ++i) {
        const unsigned blocks = (unsigned)((bytes[i] + 32767) / 32768);
        hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, stream, reinterpret_cast<const u4*>(p),
                           (uint64_t)(bytes[i] / 16), static_cast<u4*>(sink_dev));
        if (hipGetLastError() != hipSuccess) return -6;
        p += bytes[i];
    }
    return 0;
}

double glowq_probe_mfma_f16_flops(int64_t iters, int32_t blocks) {
    return (double)blocks * 4.0 * (double)iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
}

}  // extern "C"
