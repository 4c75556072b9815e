// Decode path (T <= 64 tokens): dequant-in-register INT4 GEMV/skinny GEMM on the matrix cores,
// with the low-rank correction epilogue fused.
//
// For an input-sharing group every module's rows are one launch; module i's output is
//   y_i = X W_hat_i^T + R_p A_i^T,   R_p = X B_p^T  (p = 0 for the shared factor)
// (GlowQ paper note, key design 4 and the flowchart's last node).  R is formed once per call
// by the projection kernel and read here from the workspace in fp32.
//
// Work decomposition: one workgroup (4 wavefronts) per 16-row tile; the K dimension (input
// groups of 128) is split across the 4 wavefronts (group g goes to wave g % 4), so that every
// CU keeps many independent 128-bit weight loads in flight.  Each wave streams its groups:
// one 16-byte load per lane brings a full group (16 rows x 128 inputs) in matrix-core operand
// order; nibbles become exact fp16 (q - z) values in registers; four v_mfma_f32_16x16x32_f16
// accumulate the group's partial sums against the tokens (padded to 16 per tile); the
// per-(row, group) scale is applied once per group in fp32.  The partial sums of the four
// waves, each with its share of the correction terms, are reduced in LDS in a fixed order
// (deterministic) and rounded once to fp16.
#include "glowq_internal.h"

namespace glowq {

__device__ __forceinline__ void pick_module(const ForwardArgs& a, int tile, ModuleArgs& m) {
    m = a.mod[0];
#pragma unroll
    for (int i = 1; i < kMaxModules; ++i)
        if (i < a.n_mod && tile >= a.mod[i].tile_begin) m = a.mod[i];
}

template <int NTT>
__global__ __launch_bounds__(256) void decode_kernel(const ForwardArgs args) {
    constexpr int U = 4;  // groups per wave in flight
    __shared__ f4 red[4][NTT][64];

    ModuleArgs M;
    pick_module(args, blockIdx.x, M);
    const int rt = blockIdx.x - M.tile_begin;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = args.G, T = args.T, d = args.d;
    const uint8_t* qbase = M.q + (size_t)rt * G * 1024 + lane * 16;
    const uint8_t* szbase = M.sz + (size_t)rt * G * 64;
    const int kofs = 8 * (lane >> 4);

    // token rows this lane feeds into the B operand
    const _Float16* xrow[NTT];
    bool tok_ok[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const int t = 16 * tt + (lane & 15);
        tok_ok[tt] = t < T;
        xrow[tt] = args.x + (size_t)(tok_ok[tt] ? t : 0) * d + kofs;
    }

    f4 acc[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[tt] = f4{0.f, 0.f, 0.f, 0.f};

    for (int g0 = wave; g0 < G; g0 += 4 * U) {
        u4 qv[U];
        uint32_t zso[U];
        u4 zs4[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + 4 * u;
            if (g < G) {
                qv[u] = *reinterpret_cast<const u4*>(qbase + (size_t)g * 1024);
                zso[u] = *reinterpret_cast<const uint32_t*>(szbase + (size_t)g * 64 + (lane & 15) * 4);
                zs4[u] = *reinterpret_cast<const u4*>(szbase + (size_t)g * 64 + (lane >> 4) * 16);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int g = g0 + 4 * u;
            if (g < G) {
                h2 c1024, c64;
                zero_consts(zso[u], c1024, c64);
                h8 aop[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) aop[j] = nib8_minus_z(qv[u][j], c1024, c64);
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    h8 bop[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (tok_ok[tt])
                            bop[j] = load_h8(xrow[tt] + (size_t)g * kGroup + 32 * j);
                        else
                            bop[j] = h8{0, 0, 0, 0, 0, 0, 0, 0};
                    }
                    f4 part = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < 4; ++j) part = mfma16(aop[j], bop[j], part);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[tt][i] += (float)as_h2(zs4[u][i])[1] * part[i];
                }
            }
        }
    }

    // correction epilogue: this wave adds R[t][8c..8c+8) . A[row][8c..8c+8) for chunks c = wave mod 4
    if (args.r > 0 && M.a != nullptr) {
        const int r = args.r;
        const float* R = reinterpret_cast<const float*>(args.R) + (size_t)M.proj * T * r;
        const int row0 = rt * 16 + 4 * (lane >> 4);
        for (int c = wave; c < r / 8; c += 4) {
            h8 a8[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = row0 + i;
                if (row < M.n_out)
                    a8[i] = load_h8(M.a + (size_t)row * r + 8 * c);
                else
                    a8[i] = h8{0, 0, 0, 0, 0, 0, 0, 0};
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                const int t = 16 * tt + (lane & 15);
                if (t < T) {
                    const f4* rp = reinterpret_cast<const f4*>(R + (size_t)t * r + 8 * c);
                    const f4 r0 = rp[0], r1 = rp[1];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float s = acc[tt][i];
                        s = fmaf((float)a8[i][0], r0[0], s);
                        s = fmaf((float)a8[i][1], r0[1], s);
                        s = fmaf((float)a8[i][2], r0[2], s);
                        s = fmaf((float)a8[i][3], r0[3], s);
                        s = fmaf((float)a8[i][4], r1[0], s);
                        s = fmaf((float)a8[i][5], r1[1], s);
                        s = fmaf((float)a8[i][6], r1[2], s);
                        s = fmaf((float)a8[i][7], r1[3], s);
                        acc[tt][i] = s;
                    }
                }
            }
        }
    }

#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) red[wave][tt][lane] = acc[tt];
    __syncthreads();
    if (wave < NTT) {  // wave w stores token tile w
        const int tt = wave;
        const f4 v0 = red[0][tt][lane], v1 = red[1][tt][lane], v2 = red[2][tt][lane], v3 = red[3][tt][lane];
        const int t = 16 * tt + (lane & 15);
        const int row0 = rt * 16 + 4 * (lane >> 4);
        if (t < T) {
            _Float16 o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (_Float16)(((v0[i] + v1[i]) + v2[i]) + v3[i]);
            _Float16* yp = M.y + (size_t)t * M.n_out + row0;
            if ((M.n_out & 3) == 0 && row0 + 3 < M.n_out) {
                h2 lo = {o[0], o[1]}, hi = {o[2], o[3]};
                *reinterpret_cast<u2*>(yp) = u2{as_u32(lo), as_u32(hi)};
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (row0 + i < M.n_out) yp[i] = o[i];
            }
        }
    }
}

hipError_t launch_decode(const ForwardArgs& a, hipStream_t stream) {
    const int ntt = (int)ceil_div(a.T, 16);
    const dim3 grid(a.n_tiles), block(256);
    switch (ntt) {
        case 1: hipLaunchKernelGGL(decode_kernel<1>, grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace glowq
