// MX (OCP microscaling) quantisation on gfx950: whole matrices (the experts'
// weights, offline) and the encode step's token rows (MXFP8, fused into the
// copy into the flat expert buffer). Four lanes take a 32-value block, eight
// values each: the block's amax is a two-step shuffle max, the shared exponent
// comes from frexp, values are scaled by an exact power of two and converted
// (E4M3 by the hardware conversion, which rounds to nearest even; E2M1 by
// comparison with the rounding midpoints).
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ void load8(const void *src, int dtype, int64_t off, float *f) {
    if (dtype == MOE_DT_BF16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(src) + off);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(src) + off);
        const float4 a = p[0], b = p[1];
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    }
}

// The lane's eight values of a block whose four lanes are consecutive -> its codes
// (fp8: 8 bytes, fp4: 4 bytes, in .x) and the block's scale byte (same in all four).
template <int FMT>
__device__ __forceinline__ uint2 mx_block8(const float *f, uint32_t &scale) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 4));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 4));
    const int e = mx_shared_exp(amax, FMT == kMxFp8 ? 8 : 2);
    scale = static_cast<uint32_t>(e + 127);
    uint2 out = make_uint2(0u, 0u);
    if constexpr (FMT == kMxFp8) {
        const uint32_t c01 = mx_fp8x2(ldexpf(f[0], -e), ldexpf(f[1], -e));
        const uint32_t c23 = mx_fp8x2(ldexpf(f[2], -e), ldexpf(f[3], -e));
        const uint32_t c45 = mx_fp8x2(ldexpf(f[4], -e), ldexpf(f[5], -e));
        const uint32_t c67 = mx_fp8x2(ldexpf(f[6], -e), ldexpf(f[7], -e));
        out.x = c01 | (c23 << 16);
        out.y = c45 | (c67 << 16);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) out.x |= mx_fp4(ldexpf(f[i], -e)) << (4 * i);
    }
    return out;
}

// grid-stride over the rows*K/32 blocks; a wavefront takes 16 blocks at a time.
template <int FMT>
__global__ __launch_bounds__(kThreads) void mx_quantize_kernel(const void *__restrict__ src, int dtype, int64_t rows,
                                                               int32_t K, uint8_t *__restrict__ codes,
                                                               uint8_t *__restrict__ scales) {
    const int64_t nblk = rows * (K / 32);
    const int sub = threadIdx.x & 3;
    for (int64_t b = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / 4; b < nblk;
         b += static_cast<int64_t>(gridDim.x) * (kThreads / 4)) {
        const int64_t r = b / (K / 32), kb = b - r * (K / 32);
        float f[8];
        load8(src, dtype, r * K + kb * 32 + sub * 8, f);
        uint32_t sc;
        const uint2 c = mx_block8<FMT>(f, sc);
        if constexpr (FMT == kMxFp8)
            *reinterpret_cast<uint2 *>(codes + r * K + kb * 32 + sub * 8) = c;
        else
            *reinterpret_cast<uint32_t *>(codes + r * (K / 2) + kb * 16 + sub * 4) = c.x;
        if (sub == 0) scales[b] = static_cast<uint8_t>(sc);
    }
}

// One wavefront per token: the row is quantised once (16 blocks = 512 values per
// pass) and its codes and scales are written to every kept slot; then the
// padding rows of every expert are zero-filled (codes 0, scale byte 0).
__global__ __launch_bounds__(kThreads) void encode_mx_kernel(const bf16_t *__restrict__ x,
                                                             const int32_t *__restrict__ idx,
                                                             const int32_t *__restrict__ loc,
                                                             const int32_t *__restrict__ fill,
                                                             const int32_t *__restrict__ cap,
                                                             uint8_t *__restrict__ codes,
                                                             uint8_t *__restrict__ scales, int S, int M, int E, int k) {
    const int C = *cap;
    const int lane = threadIdx.x & 63;
    const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
    const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / 64;
    const int sub = lane & 3;
    for (int64_t s = w0; s < S; s += nw) {
        int slot = -1;
        if (lane < k) {
            const int64_t q = static_cast<int64_t>(lane) * S + s;
            const int l = loc[q];
            if (l < C) slot = idx[q] * C + l;
        }
        for (int m0 = 0; m0 < M; m0 += 512) {
            const int kb = (m0 + lane * 8) / 32;  // this lane's block
            const bool in = m0 + lane * 8 < M;    // M is a multiple of 64: whole blocks
            float f[8];
            if (in) load8(x, MOE_DT_BF16, s * M + m0 + lane * 8, f);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] = 0.f;
            uint32_t sc;
            const uint2 c = mx_block8<kMxFp8>(f, sc);
            for (int r = 0; r < k; ++r) {
                const int sl = __builtin_amdgcn_readlane(slot, r);
                if (sl < 0 || !in) continue;
                *reinterpret_cast<uint2 *>(codes + static_cast<int64_t>(sl) * M + m0 + lane * 8) = c;
                if (sub == 0) scales[static_cast<int64_t>(sl) * (M / 32) + kb] = static_cast<uint8_t>(sc);
            }
        }
    }
    const int64_t rows = static_cast<int64_t>(E) * C;
    for (int64_t row = w0; row < rows; row += nw) {
        const int e = static_cast<int>(row / C);
        const int j = static_cast<int>(row - static_cast<int64_t>(e) * C);
        if (j < fill[e]) continue;
        for (int m = lane * 16; m < M; m += 64 * 16)
            *reinterpret_cast<uint4 *>(codes + row * M + m) = make_uint4(0u, 0u, 0u, 0u);
        for (int b = lane; b < M / 32; b += 64) scales[row * (M / 32) + b] = 0;
    }
}

int grid_blocks(int64_t threads) {
    const int64_t b = (threads + kThreads - 1) / kThreads;
    return static_cast<int>(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

}  // namespace

hipError_t launch_mx_quantize(int fmt, int64_t rows, int32_t K, int dtype, const void *src, uint8_t *codes,
                              uint8_t *scales, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    const int grid = grid_blocks(rows * (K / 32) * 4);
    if (fmt == kMxFp8)
        hipLaunchKernelGGL(mx_quantize_kernel<kMxFp8>, dim3(grid), dim3(kThreads), 0, st, src, dtype, rows, K, codes,
                           scales);
    else
        hipLaunchKernelGGL(mx_quantize_kernel<kMxFp4>, dim3(grid), dim3(kThreads), 0, st, src, dtype, rows, K, codes,
                           scales);
    return hipGetLastError();
}

hipError_t launch_encode_mx(const moe_shape &s, const void *x, const int32_t *idx, const int32_t *loc,
                            const int32_t *fill, const int32_t *cap, uint8_t *buf_codes, uint8_t *buf_scales,
                            int32_t cmax, hipStream_t st) {
    const int grid = grid_blocks((static_cast<int64_t>(s.S) + static_cast<int64_t>(s.E) * cmax) * 64);
    hipLaunchKernelGGL(encode_mx_kernel, dim3(grid), dim3(kThreads), 0, st, static_cast<const bf16_t *>(x), idx, loc,
                       fill, cap, buf_codes, buf_scales, s.S, s.M, s.E, s.k);
    return hipGetLastError();
}

}  // namespace moe
