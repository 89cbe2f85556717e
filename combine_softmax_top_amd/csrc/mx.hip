// MX (OCP microscaling) and block-wise FP8 quantisation on gfx950: whole
// matrices (the experts' weights, offline) and the encode step's token rows
// (fused into the copy into the flat expert buffer). MX: four lanes take a
// 32-value block, eight values each: the block's amax is a two-step shuffle max,
// the shared exponent comes from frexp, values are scaled by an exact power of
// two and converted (E4M3 by the hardware conversion, which rounds to nearest
// even; E2M1 by comparison with the rounding midpoints). Block-wise FP8: sixteen
// lanes take a 1 x 128 block, a workgroup a 128 x 128 one, and the values are
// divided by the block's fp32 scale before the same E4M3 conversion.
// NVFP4 (weights only): workgroups over stretches of each tensor combine its amax by
// an atomic max, then two lanes per 16-value block round the block scale to E4M3 and
// the values to E2M1.
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

// ---------------------------------------------------------------- block-wise FP8
// E4M3 codes with one fp32 scale s = amax / 448 per block (1 x 128 for activations,
// 128 x 128 for weights); code = v / s (fp32 division) converted to nearest even and
// saturated like the MX elements; an all-zero block has s = 0 and codes 0.

// Eight values of a block with scale s -> eight E4M3 codes.
__device__ __forceinline__ uint2 blk_codes8(const float *f, float s) {
    return make_uint2(blk_fp8x2(f[0], f[1], s) | (blk_fp8x2(f[2], f[3], s) << 16),
                      blk_fp8x2(f[4], f[5], s) | (blk_fp8x2(f[6], f[7], s) << 16));
}

// Amax of a 128-value block held by 16 consecutive lanes, eight values each.
__device__ __forceinline__ float blk_amax16(const float *f) {
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 16));
    return amax;
}

// 1 x 128 blocks: sixteen lanes per block, grid-stride over the rows * K/128 blocks.
__global__ __launch_bounds__(kThreads) void blk_quantize_rows_kernel(const void *__restrict__ src, int dtype,
                                                                     int64_t rows, int32_t K,
                                                                     uint8_t *__restrict__ codes,
                                                                     float *__restrict__ scales) {
    const int KB = K / 128;
    const int64_t nblk = rows * KB;
    const int sub = threadIdx.x & 15;
    for (int64_t b = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / 16; b < nblk;
         b += static_cast<int64_t>(gridDim.x) * (kThreads / 16)) {
        const int64_t r = b / KB, kb = b - r * KB;
        const int64_t at = r * K + kb * 128 + sub * 8;
        float f[8];
        load8(src, dtype, at, f);
        const float sc = blk_amax16(f) / 448.f;
        *reinterpret_cast<uint2 *>(codes + at) = blk_codes8(f, sc);
        if (sub == 0) scales[b] = sc;
    }
}

// 128 x 128 blocks: a workgroup per block, each thread 64 values of one row (two per row).
__global__ __launch_bounds__(kThreads) void blk_quantize_tiles_kernel(const void *__restrict__ src, int dtype,
                                                                      int64_t rows, int32_t K,
                                                                      uint8_t *__restrict__ codes,
                                                                      float *__restrict__ scales) {
    static_assert(kThreads == 256, "two threads per row of a 128-row block");
    __shared__ float wmax[kThreads / 64];
    const int KB = K / 128;
    const int64_t nblk = (rows / 128) * KB;
    const int row = threadIdx.x >> 1, half = threadIdx.x & 1, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    for (int64_t b = blockIdx.x; b < nblk; b += gridDim.x) {
        const int64_t rb = b / KB, kb = b - rb * KB;
        const int64_t at = (rb * 128 + row) * K + kb * 128 + half * 64;
        float f[64];
#pragma unroll
        for (int u = 0; u < 8; ++u) load8(src, dtype, at + 8 * u, f + 8 * u);
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 64; ++i) amax = fmaxf(amax, fabsf(f[i]));
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
        if (lane == 0) wmax[wave] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        const float sc = amax / 448.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint2 lo = blk_codes8(f + 16 * u, sc), hi = blk_codes8(f + 16 * u + 8, sc);
            *reinterpret_cast<uint4 *>(codes + at + 16 * u) = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        if (threadIdx.x == 0) scales[b] = sc;
        __syncthreads();  // wmax is read before the next block overwrites it
    }
}

// NVFP4 weights: E2M1 codes in 16-value blocks along K with E4M3 block scales and one
// fp32 scale g per tensor (rows / ntensor consecutive rows). g = amax / 2688 needs the
// whole tensor's amax first: one workgroup per tensor (offline weight preparation).
__global__ __launch_bounds__(kThreads) void nvfp4_amax_kernel(const void *__restrict__ src, int dtype,
                                                              int64_t per_elems, int64_t span,
                                                              uint32_t *__restrict__ amax_bits) {
    // blockIdx.y: the tensor; blockIdx.x: its span-th stretch of elements (span a multiple of 8)
    __shared__ float wmax[kThreads / 64];
    const int64_t base = static_cast<int64_t>(blockIdx.y) * per_elems;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * span, hi = min(per_elems, lo + span);
    float amax = 0.f;
    for (int64_t i = lo + static_cast<int64_t>(threadIdx.x) * 8; i < hi; i += kThreads * 8) {
        float f[8];
        load8(src, dtype, base + i, f);
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(f[j]));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
    __syncthreads();
    // non-negative floats order as their bit patterns
    if (threadIdx.x == 0)
        atomicMax(amax_bits + blockIdx.y, __float_as_uint(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]))));
}

__global__ void nvfp4_amax_zero_kernel(uint32_t *__restrict__ amax_bits, int n) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) amax_bits[t] = 0u;
}

// g = amax / 2688 (448 * 6), in place, once the quantiser has read the maxima
__global__ void nvfp4_g_kernel(float *__restrict__ g, int n) {
    const int t = blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n) g[t] = g[t] / 2688.f;
}

// Two lanes per 16-value block, eight values each: d = (amax_b / 6) / g rounded to the
// E4M3 code q (the hardware conversion: nearest even, clamped to 448), then each value
// divided by the fp32 product e4m3(q) * g and rounded to E2M1 (codes 0 when that
// product is 0, as for an all-zero tensor).
__global__ __launch_bounds__(kThreads) void nvfp4_quantize_kernel(const void *__restrict__ src, int dtype,
                                                                  int64_t rows, int32_t K, int64_t per,
                                                                  const float *__restrict__ amax_t,
                                                                  uint8_t *__restrict__ codes,
                                                                  uint8_t *__restrict__ scales) {
    const int KB = K / 16;
    const int64_t nblk = rows * KB;
    const int sub = threadIdx.x & 1;
    for (int64_t b = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / 2; b < nblk;
         b += static_cast<int64_t>(gridDim.x) * (kThreads / 2)) {
        const int64_t r = b / KB;
        const int64_t at = b * 16 + sub * 8;  // = r * K + (b - r * KB) * 16 + sub * 8
        float f[8];
        load8(src, dtype, at, f);
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(f[i]));
        amax = fmaxf(amax, __shfl_xor(amax, 1, 2));
        const float gt = amax_t[r / per] / 2688.f;  // the tensor's g, as nvfp4_g_kernel computes it
        uint32_t q = 0u;
        if (gt > 0.f) q = mx_fp8x2((amax / 6.f) / gt, 0.f) & 0xFFu;
        const float den = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(q), 0) * gt;
        uint32_t c = 0u;
        if (den > 0.f) {
#pragma unroll
            for (int i = 0; i < 8; ++i) c |= mx_fp4(f[i] / den) << (4 * i);
        }
        *reinterpret_cast<uint32_t *>(codes + at / 2) = c;
        if (sub == 0) scales[b] = static_cast<uint8_t>(q);
    }
}

// One wavefront per token, as encode_mx_kernel: the row is quantised once in 1 x 128 blocks
// (four per pass of 512 values) and its codes and scales go to every kept slot; then the
// padding rows of every expert get codes 0 and scale 0.
__global__ __launch_bounds__(kThreads) void encode_blk_kernel(const bf16_t *__restrict__ x,
                                                              const int32_t *__restrict__ idx,
                                                              const int32_t *__restrict__ loc,
                                                              const int32_t *__restrict__ fill,
                                                              const int32_t *__restrict__ cap,
                                                              uint8_t *__restrict__ codes, float *__restrict__ scales,
                                                              int S, int M, int E, int k) {
    const int C = *cap;
    const int lane = threadIdx.x & 63;
    const int64_t nw = static_cast<int64_t>(gridDim.x) * (kThreads / 64);
    const int64_t w0 = (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / 64;
    for (int64_t s = w0; s < S; s += nw) {
        int slot = -1;
        if (lane < k) {
            const int64_t q = static_cast<int64_t>(lane) * S + s;
            const int l = loc[q];
            if (l < C) slot = idx[q] * C + l;
        }
        for (int m0 = 0; m0 < M; m0 += 512) {
            const bool in = m0 + lane * 8 < M;  // M is a multiple of 128: whole blocks of 16 lanes
            float f[8];
            if (in) load8(x, MOE_DT_BF16, s * M + m0 + lane * 8, f);
            else
#pragma unroll
                for (int i = 0; i < 8; ++i) f[i] = 0.f;
            const float sc = blk_amax16(f) / 448.f;
            const uint2 c = blk_codes8(f, sc);
            for (int r = 0; r < k; ++r) {
                const int sl = __builtin_amdgcn_readlane(slot, r);
                if (sl < 0 || !in) continue;
                *reinterpret_cast<uint2 *>(codes + static_cast<int64_t>(sl) * M + m0 + lane * 8) = c;
                if ((lane & 15) == 0) scales[static_cast<int64_t>(sl) * (M / 128) + (m0 + lane * 8) / 128] = sc;
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
        for (int b = lane; b < M / 128; b += 64) scales[row * (M / 128) + b] = 0.f;
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

hipError_t launch_blk_quantize(int brows, int64_t rows, int32_t K, int dtype, const void *src, uint8_t *codes,
                               float *scales, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    if (brows == 1) {
        hipLaunchKernelGGL(blk_quantize_rows_kernel, dim3(grid_blocks(rows * (K / 128) * 16)), dim3(kThreads), 0, st,
                           src, dtype, rows, K, codes, scales);
    } else {
        const int64_t nblk = (rows / 128) * (K / 128);
        const int grid = static_cast<int>(nblk < 8192 ? nblk : 8192);
        hipLaunchKernelGGL(blk_quantize_tiles_kernel, dim3(grid), dim3(kThreads), 0, st, src, dtype, rows, K, codes,
                           scales);
    }
    return hipGetLastError();
}

hipError_t launch_nvfp4_quantize(int64_t rows, int32_t K, int32_t ntensor, int dtype, const void *src,
                                 uint8_t *codes, uint8_t *scales, float *g, hipStream_t st) {
    if (rows == 0) return hipSuccess;
    // g holds each tensor's amax (as bits) until the codes are written: a fill, the
    // maxima over stretches of 32 K values (one atomic max per workgroup), the
    // quantiser, then g = amax / 2688 in place
    const int64_t per = rows / ntensor, per_elems = per * K;
    const int64_t span = static_cast<int64_t>(kThreads) * 8 * 16;
    const int64_t nspan = (per_elems + span - 1) / span;
    if (nspan > 0x7FFFFFFF) return hipErrorInvalidValue;
    uint32_t *bits = reinterpret_cast<uint32_t *>(g);
    const int small = (ntensor + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(nvfp4_amax_zero_kernel, dim3(small), dim3(kThreads), 0, st, bits, ntensor);
    hipLaunchKernelGGL(nvfp4_amax_kernel, dim3(static_cast<uint32_t>(nspan), ntensor), dim3(kThreads), 0, st, src,
                       dtype, per_elems, span, bits);
    hipLaunchKernelGGL(nvfp4_quantize_kernel, dim3(grid_blocks(rows * (K / 16) * 2)), dim3(kThreads), 0, st, src,
                       dtype, rows, K, per, static_cast<const float *>(g), codes, scales);
    hipLaunchKernelGGL(nvfp4_g_kernel, dim3(small), dim3(kThreads), 0, st, g, ntensor);
    return hipGetLastError();
}

hipError_t launch_encode_blk(const moe_shape &s, const void *x, const int32_t *idx, const int32_t *loc,
                             const int32_t *fill, const int32_t *cap, uint8_t *buf_codes, float *buf_scales,
                             int32_t cmax, hipStream_t st) {
    const int grid = grid_blocks((static_cast<int64_t>(s.S) + static_cast<int64_t>(s.E) * cmax) * 64);
    hipLaunchKernelGGL(encode_blk_kernel, dim3(grid), dim3(kThreads), 0, st, static_cast<const bf16_t *>(x), idx, loc,
                       fill, cap, buf_codes, buf_scales, s.S, s.M, s.E, s.k);
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
