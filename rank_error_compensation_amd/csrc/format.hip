// Weight formats: canonical -> device layout repack, and the dequantisation export.
//
// The dequantised weight of the W4A16 format is (q - z) * s per 128-input group (GlowQ paper
// note, "Experimental setup"; arXiv page, Table 1 header "INT4, g128").  MX modules (the MXFP4 /
// MXFP6 datatypes of the arXiv page's Table 13) dequantise to element * 2^(S - 127) per 32-input
// block.  The export runs the same in-register routines (nib8_minus_z, mx4_h8, mx6_h32) as the
// forward kernels, so a bit-exact export checks the operands the forward kernels feed to the
// matrix cores.
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

// Zero-fill of n bytes: 16-byte stores in a grid-stride loop, the last n % 16 bytes by thread 0.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t* __restrict__ p, size_t n) {
    const size_t n16 = n / 16;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
        reinterpret_cast<u4*>(p)[i] = u4{0u, 0u, 0u, 0u};
    if (blockIdx.x == 0 && threadIdx.x == 0)
        for (size_t i = n16 * 16; i < n; ++i) p[i] = 0;
}

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

// MX codes: one thread per lane record (row tile, group, lane l) of the device layout: the 32
// codes of row 16 rt + l % 16 at inputs 128 g + 32 (l / 16) + n (one MX block), code n packed at
// bit NB n (NB = 4 or 6); codes wider than NB bits set bit 0 of the flag.
template <int NB>
__global__ __launch_bounds__(256) void repack_mx_q_kernel(const uint8_t* __restrict__ codes, int64_t n_out,
                                                          int64_t k_in, int64_t n_lanes, uint8_t* __restrict__ qd,
                                                          int32_t* __restrict__ flag) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_lanes) return;
    const int64_t NT = ceil_div(n_out, 16);
    const int64_t blk = idx >> 6;  // block g * NT + rt
    const int l = (int)(idx & 63);
    const int64_t g = blk / NT, rt = blk - g * NT;
    const int64_t row = rt * 16 + (l & 15);
    uint32_t w[NB] = {};
    bool bad = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u2 c8 = {0u, 0u};
        if (row < n_out)
            c8 = *reinterpret_cast<const u2*>(codes + row * k_in + g * kGroup + 32 * (l >> 4) + 8 * j);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t c = (c8[e >> 2] >> (8 * (e & 3))) & 0xFFu;
            bad |= c >= (1u << NB);
            const int bit = NB * (8 * j + e);
            w[bit >> 5] |= (c & ((1u << NB) - 1)) << (bit & 31);
            if ((bit & 31) + NB > 32) w[(bit >> 5) + 1] |= (c & ((1u << NB) - 1)) >> (32 - (bit & 31));
        }
    }
    if (bad) atomicOr(flag, 1);
    uint8_t* base = qd + blk * Fmt<NB == 4 ? kFmtMxfp4 : kFmtMxfp6E2M3>::qblock;
    *reinterpret_cast<u4*>(base + 16 * l) = u4{w[0], w[1], w[2], w[3]};
    if constexpr (NB == 6) *reinterpret_cast<u2*>(base + 1024 + 8 * l) = u2{w[4], w[5]};
}

// MX scales: one thread per (row tile, group, row-in-tile): the four block scales of the group as
// one word; a scale outside [lo, hi] (biased) sets bit 0 of the flag.  Rows past n_out get 127.
__global__ __launch_bounds__(256) void repack_mx_s_kernel(const uint8_t* __restrict__ scales, int64_t n_out,
                                                          int64_t G, int64_t n_words, uint32_t lo, uint32_t hi,
                                                          uint32_t* __restrict__ szd, int32_t* __restrict__ flag) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_words) return;
    const int64_t NT = ceil_div(n_out, 16);
    const int64_t blk = idx >> 4;
    const int i = (int)(idx & 15);
    const int64_t g = blk / NT, rt = blk - g * NT;
    const int64_t row = rt * 16 + i;
    uint32_t w = 0x7F7F7F7Fu;
    if (row < n_out) {
        w = *reinterpret_cast<const uint32_t*>(scales + row * G * 4 + 4 * g);
        bool ok = true;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t b = (w >> (8 * j)) & 0xFFu;
            ok &= b >= lo && b <= hi;
        }
        if (!ok) atomicOr(flag, 1);
    }
    szd[idx] = w;
}

// MX export: one thread per lane record, 32 values of one row.
template <int F, int DTYPE>
__global__ __launch_bounds__(256) void dequant_mx_kernel(const uint8_t* __restrict__ qd, const uint32_t* __restrict__ szd,
                                                         int64_t n_out, int64_t k_in, int64_t n_lanes,
                                                         void* __restrict__ out) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= n_lanes) return;
    const int64_t NT = ceil_div(n_out, 16);
    const int64_t blk = idx >> 6;
    const int l = (int)(idx & 63);
    const int64_t g = blk / NT, rt = blk - g * NT;
    const int64_t row = rt * 16 + (l & 15);
    if (row >= n_out) return;
    const uint8_t* base = qd + blk * Fmt<F>::qblock;
    const u4 q = *reinterpret_cast<const u4*>(base + 16 * l);
    const float sc = mx_scale(szd[blk * 16 + (l & 15)], l >> 4);  // the lane's block
    h8 v[4];
    if constexpr (Fmt<F>::six) {
        const h32 e = mx6_h32<F>(q, *reinterpret_cast<const u2*>(base + 1024 + 8 * l), sc);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = mx6_slice(e, j);
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = mx4_h8(q[j], sc);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t k0 = g * kGroup + 32 * (l >> 4) + 8 * j;
        if (DTYPE == 0) {
            float* o = reinterpret_cast<float*>(out) + row * k_in + k0;
            reinterpret_cast<f4*>(o)[0] = f4{(float)v[j][0], (float)v[j][1], (float)v[j][2], (float)v[j][3]};
            reinterpret_cast<f4*>(o)[1] = f4{(float)v[j][4], (float)v[j][5], (float)v[j][6], (float)v[j][7]};
        } else {
            *reinterpret_cast<u4*>(reinterpret_cast<_Float16*>(out) + row * k_in + k0) = __builtin_bit_cast(u4, v[j]);
        }
    }
}

hipError_t launch_flag_clear(int32_t* flag, hipStream_t stream) {
    hipLaunchKernelGGL(flag_clear_kernel, dim3(1), dim3(1), 0, stream, flag);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t stream) {
    const size_t n16 = bytes / 16;
    const size_t want = (n16 + 255) / 256;
    const unsigned grid = (unsigned)(want < 1 ? 1 : (want > 2048 ? 2048 : want));
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint8_t*>(p), bytes);
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

hipError_t launch_repack_mx(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t n_out, int64_t k_in,
                            uint8_t* q_dev, uint8_t* sz_dev, int32_t* flag, hipStream_t stream) {
    const int64_t NT = ceil_div(n_out, 16), G = k_in / kGroup;
    const int64_t n_lanes = NT * G * 64, n_words = NT * G * 16;
    const dim3 gq((unsigned)ceil_div(n_lanes, 256));
    if (fmt == kFmtMxfp4)
        hipLaunchKernelGGL(repack_mx_q_kernel<4>, gq, dim3(256), 0, stream, codes, n_out, k_in, n_lanes, q_dev, flag);
    else
        hipLaunchKernelGGL(repack_mx_q_kernel<6>, gq, dim3(256), 0, stream, codes, n_out, k_in, n_lanes, q_dev, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // admitted block exponents: every element times 2^X an fp16 value (finest element step times
    // 2^X at least 2^-24, largest element times 2^X at most 65504)
    const int lo = fmt == kFmtMxfp4 ? -23 : (fmt == kFmtMxfp6E2M3 ? -21 : -20);
    const int hi = fmt == kFmtMxfp6E3M2 ? 11 : 13;
    hipLaunchKernelGGL(repack_mx_s_kernel, dim3((unsigned)ceil_div(n_words, 256)), dim3(256), 0, stream, scales,
                       n_out, G, n_words, (uint32_t)(lo + 127), (uint32_t)(hi + 127),
                       reinterpret_cast<uint32_t*>(sz_dev), flag);
    return hipGetLastError();
}

template <int F>
static void launch_dequant_mx(const uint8_t* q, const uint8_t* sz, int64_t n_out, int64_t k_in, void* out,
                              int dtype, hipStream_t stream) {
    const int64_t n_lanes = ceil_div(n_out, 16) * (k_in / kGroup) * 64;
    const dim3 grid((unsigned)ceil_div(n_lanes, 256));
    const uint32_t* szw = reinterpret_cast<const uint32_t*>(sz);
    if (dtype == 0)
        hipLaunchKernelGGL((dequant_mx_kernel<F, 0>), grid, dim3(256), 0, stream, q, szw, n_out, k_in, n_lanes, out);
    else
        hipLaunchKernelGGL((dequant_mx_kernel<F, 1>), grid, dim3(256), 0, stream, q, szw, n_out, k_in, n_lanes, out);
}

hipError_t launch_dequant(int fmt, const uint8_t* q, const uint8_t* sz, int64_t n_out, int64_t k_in, void* out,
                          int dtype, hipStream_t stream) {
    if (fmt != kFmtInt4) {
        switch (fmt) {
            case kFmtMxfp4: launch_dequant_mx<kFmtMxfp4>(q, sz, n_out, k_in, out, dtype, stream); break;
            case kFmtMxfp6E2M3: launch_dequant_mx<kFmtMxfp6E2M3>(q, sz, n_out, k_in, out, dtype, stream); break;
            case kFmtMxfp6E3M2: launch_dequant_mx<kFmtMxfp6E3M2>(q, sz, n_out, k_in, out, dtype, stream); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
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
