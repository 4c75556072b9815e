// INT4-g128 weight format: canonical -> device layout repack, and the dequantisation export.
//
// The dequantised weight of the W4A16 format is (q - z) * s per 128-input group (GlowQ paper
// note, "Experimental setup"; arXiv page, Table 1 header "INT4, g128").  The export runs the
// same in-register routine (nib8_minus_z) as the forward kernels, so a bit-exact export checks
// the arithmetic the forward kernels feed to the matrix cores.
#include "glowq_internal.h"

namespace glowq {

// One thread per 32-bit word of the device layout.  Word (rt, g, lane l, slice j) takes the
// canonical word holding inputs k0 .. k0+7, k0 = 128 g + 32 j + 8 (l / 16), of row 16 rt + l % 16,
// and moves input e from nibble slot e to slot e/2 (even e) or 4 + e/2 (odd e).
__global__ __launch_bounds__(256) void repack_q_kernel(const uint32_t* __restrict__ qc, int64_t n_out,
                                                       int64_t k_in, int64_t n_words,
                                                       uint32_t* __restrict__ qd) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_words) return;
    const int64_t NT = ceil_div(n_out, 16);
    const int64_t blk = idx >> 8;  // block g * NT + rt
    const int within = (int)(idx & 255);
    const int l = within >> 2, j = within & 3;
    const int64_t g = blk / NT, rt = blk - g * NT;
    const int64_t row = rt * 16 + (l & 15);
    const int64_t k0 = g * kGroup + 32 * j + 8 * (l >> 4);
    uint32_t v = 0;
    if (row < n_out) v = qc[row * (k_in / 8) + k0 / 8];
    uint32_t o = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        o |= ((v >> (8 * p)) & 0xFu) << (4 * p);
        o |= ((v >> (8 * p + 4)) & 0xFu) << (4 * (p + 4));
    }
    qd[idx] = o;
}

// One thread per (row tile, group, row-in-tile): the (z, s) pair word, with range checks.
__global__ __launch_bounds__(256) void repack_sz_kernel(const _Float16* __restrict__ s,
                                                        const _Float16* __restrict__ z, int64_t n_out,
                                                        int64_t G, int64_t n_pairs,
                                                        uint32_t* __restrict__ szd,
                                                        int32_t* __restrict__ flag) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_pairs) return;
    const int64_t NT = ceil_div(n_out, 16);
    const int64_t blk = idx >> 4;  // block g * NT + rt
    const int i = (int)(idx & 15);
    const int64_t g = blk / NT, rt = blk - g * NT;
    const int64_t row = rt * 16 + i;
    h2 pair = {(_Float16)0.0f, (_Float16)0.0f};
    if (row < n_out) {
        const _Float16 zz = z[row * G + g];
        const _Float16 ss = s[row * G + g];
        const float zf = (float)zz, sf = (float)ss;
        const bool ok = (zf == rintf(zf)) && (fabsf(zf) <= 1024.0f) && isfinite(sf);
        if (!ok) atomicOr(flag, 1);
        pair = h2{zz, ss};
    }
    szd[idx] = as_u32(pair);
}

__global__ void flag_clear_kernel(int32_t* flag) { *flag = 0; }

// One thread per device-layout word: eight consecutive inputs of one row.
template <int DTYPE>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t* __restrict__ qd,
                                                      const uint32_t* __restrict__ szd, int64_t n_out,
                                                      int64_t k_in, int64_t n_words, void* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_words) return;
    const int64_t NT = ceil_div(n_out, 16);
    const int64_t blk = idx >> 8;  // block g * NT + rt
    const int within = (int)(idx & 255);
    const int l = within >> 2, j = within & 3;
    const int64_t g = blk / NT, rt = blk - g * NT;
    const int64_t row = rt * 16 + (l & 15);
    if (row >= n_out) return;
    const int64_t k0 = g * kGroup + 32 * j + 8 * (l >> 4);
    const uint32_t zs = szd[blk * 16 + (l & 15)];
    h2 c1024, c64;
    zero_consts(zs, c1024, c64);
    const h8 dq = nib8_minus_z(qd[idx], c1024, c64, nib_consts());
    const _Float16 s = as_h2(zs)[1];
    if (DTYPE == 0) {
        float* o = reinterpret_cast<float*>(out) + row * k_in + k0;
        const float sf = (float)s;
        f4 v0 = {(float)dq[0] * sf, (float)dq[1] * sf, (float)dq[2] * sf, (float)dq[3] * sf};
        f4 v1 = {(float)dq[4] * sf, (float)dq[5] * sf, (float)dq[6] * sf, (float)dq[7] * sf};
        reinterpret_cast<f4*>(o)[0] = v0;
        reinterpret_cast<f4*>(o)[1] = v1;
    } else {
        const h8 s8 = {s, s, s, s, s, s, s, s};
        const h8 w = dq * s8;
        *reinterpret_cast<u4*>(reinterpret_cast<_Float16*>(out) + row * k_in + k0) =
            __builtin_bit_cast(u4, w);
    }
}

hipError_t launch_flag_clear(int32_t* flag, hipStream_t stream) {
    hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(1), 0, stream, flag);
    return hipGetLastError();
}

hipError_t launch_repack(const uint32_t* qc, const _Float16* s, const _Float16* z, int64_t n_out,
                         int64_t k_in, uint8_t* q_dev, uint8_t* sz_dev, int32_t* flag,
                         hipStream_t stream) {
    const int64_t NT = ceil_div(n_out, 16), G = k_in / kGroup;
    const int64_t n_words = NT * G * 256;
    const int64_t n_pairs = NT * G * 16;
    hipLaunchKernelGGL(repack_q_kernel, dim3((unsigned)ceil_div(n_words, 256)), dim3(256), 0, stream,
                       qc, n_out, k_in, n_words, reinterpret_cast<uint32_t*>(q_dev));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(repack_sz_kernel, dim3((unsigned)ceil_div(n_pairs, 256)), dim3(256), 0, stream,
                       s, z, n_out, G, n_pairs, reinterpret_cast<uint32_t*>(sz_dev), flag);
    return hipGetLastError();
}

hipError_t launch_dequant(const uint8_t* q, const uint8_t* sz, int64_t n_out, int64_t k_in, void* out,
                          int dtype, hipStream_t stream) {
    const int64_t NT = ceil_div(n_out, 16), G = k_in / kGroup;
    const int64_t n_words = NT * G * 256;
    const dim3 grid((unsigned)ceil_div(n_words, 256));
    if (dtype == 0)
        hipLaunchKernelGGL(dequant_kernel<0>, grid, dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t*>(q), reinterpret_cast<const uint32_t*>(sz),
                           n_out, k_in, n_words, out);
    else
        hipLaunchKernelGGL(dequant_kernel<1>, grid, dim3(256), 0, stream,
                           reinterpret_cast<const uint32_t*>(q), reinterpret_cast<const uint32_t*>(sz),
                           n_out, k_in, n_words, out);
    return hipGetLastError();
}

}  // namespace glowq
