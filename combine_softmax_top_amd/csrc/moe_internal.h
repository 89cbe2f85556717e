// Internal declarations of the gfx950 MoE library: device helpers shared by the
// kernels and the host launchers that the C ABI (moe_api.hip) calls.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront
constexpr int kRouteTile = 64;     // tokens per routing tile: one wavefront, one lane per token
constexpr int kMaxK = 32;
constexpr int kMaxE = 512;

typedef uint16_t bf16_t;           // bf16 bit pattern

// ------------------------------------------------------------- device helpers

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (finite values), the rounding of every bf16 store.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// GELU in its exact erf form and its derivative, fp32.
__device__ __forceinline__ float gelu_f(float v) {
    return 0.5f * v * (1.0f + erff(v * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_grad_f(float v) {
    const float cdf = 0.5f * (1.0f + erff(v * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * __expf(-0.5f * v * v);
    return cdf + v * pdf;
}

// erf by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erf(x) = 1 - t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-x^2),
// t = 1 / (1 + p x) for x >= 0, odd extension; absolute error <= 1.5e-7.
// Used by the activation-gradient epilogue, where it costs about half the
// instructions of erff. *ex receives exp(-x^2), which the formula computes anyway.
__device__ __forceinline__ float erf_as(float x, float *ex = nullptr) {
    const float ax = fabsf(x);
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
    float y = fmaf(1.061405429f, t, -1.453152027f);
    y = fmaf(y, t, 1.421413741f);
    y = fmaf(y, t, -0.284496736f);
    y = fmaf(y, t, 0.254829592f);
    y *= t;
    const float e = __expf(-ax * ax);
    if (ex != nullptr) *ex = e;
    const float r = 1.0f - y * e;
    return copysignf(r, x);
}
// GELU for the GEMM epilogues, where it is VALU-bound (one evaluation per output):
// gelu(v) = v Phi(v), and with a = min(|v|, 6) and q = Phi(-a) = 2^P(a), where P is
// the degree-7 least-squares fit (Chebyshev basis on [0, 6], then expanded in a) of
// log2 Phi(-a), gelu = v q for v < 0 and v - v q for v >= 0, i.e. max(v, 0) - |v| q.
// One exp2, no reciprocal, and no cancellation on the negative side (1 + erf there
// loses the small values):
// |error| <= 5e-7, relative error <= 9e-6 where |gelu| > 1e-3; past |v| = 6 the
// error is below 2e-8. combine_softmax_top_amd/gelu_fit.py recomputes the coefficients.
__device__ __forceinline__ float gelu_fast(float v) {
    const float a = fabsf(__builtin_amdgcn_fmed3f(v, -6.0f, 6.0f));
    float p = -1.9449178e-06f;
    p = fmaf(p, a, 6.3860469e-05f);
    p = fmaf(p, a, -9.4887050e-04f);
    p = fmaf(p, a, 8.5823713e-03f);
    p = fmaf(p, a, -5.4118313e-02f);
    p = fmaf(p, a, -4.5829743e-01f);
    p = fmaf(p, a, -1.1513246e+00f);
    p = fmaf(p, a, -9.9998695e-01f);
    // max(v, 0) in one instruction: fmaxf would first canonicalize v (NaN quieting)
    float m;
    asm("v_max_f32 %0, 0, %1" : "=v"(m) : "v"(v));
    return fmaf(-fabsf(v), __builtin_amdgcn_exp2f(p), m);
}
// d/dv of 0.5 v (1 + erf(v / sqrt 2)) = Phi(v) + v phi(v), phi(v) = exp(-v^2/2) / sqrt(2 pi);
// exp(-v^2/2) is the exp(-x^2) of erf_as at x = v / sqrt 2.
__device__ __forceinline__ float gelu_grad_fast(float v) {
    float e;
    const float erf = erf_as(v * 0.70710678118654752f, &e);
    return fmaf(v * 0.39894228040143268f, e, 0.5f * (1.0f + erf));
}

template <int ACT>
__device__ __forceinline__ float act_fast(float v) {
    if constexpr (ACT == MOE_ACT_RELU) return v > 0.f ? v : 0.f;
    else return gelu_fast(v);
}

template <int ACT>
__device__ __forceinline__ float act_grad_fast(float v) {
    if constexpr (ACT == MOE_ACT_RELU) return v > 0.f ? 1.f : 0.f;
    else return gelu_grad_fast(v);
}

template <int ACT>
__device__ __forceinline__ float act_f(float v) {
    if constexpr (ACT == MOE_ACT_RELU) return v > 0.f ? v : 0.f;
    else return gelu_f(v);
}
template <int ACT>
__device__ __forceinline__ float act_grad_f(float v) {
    if constexpr (ACT == MOE_ACT_RELU) return v > 0.f ? 1.f : 0.f;
    else return gelu_grad_f(v);
}

// ------------------------------------------------------------- MX (OCP microscaling) elements
// Blocks of 32 values along the reduction dimension share an E8M0 scale 2^(b - 127);
// MXFP8 elements are E4M3 (max 448), MXFP4 elements E2M1 (max 6), two per byte (even
// index in the low nibble). A block's shared exponent is floor(log2 amax) - emax_elem
// (8 for E4M3, 2 for E2M1), clamped to [-127, 127], and -127 for an all-zero block.
constexpr int kMxFp8 = 0, kMxFp4 = 1;
// The expert GEMMs' third operand scheme: block-wise FP8 (E4M3, fp32 scales per 1 x 128
// token block and 128 x 128 weight block), passed where the MX weight format goes.
constexpr int kBlkFp8 = 2;

__device__ __forceinline__ int mx_shared_exp(float amax, int emax) {
    if (!(amax > 0.f)) return -127;
    int ex;
    (void)frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1)
    const int e = ex - 1 - emax;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// Two values (already divided by the block scale) -> two E4M3 codes in the low 16
// bits: the conversion rounds to nearest even; values beyond 448 are clamped first
// (the conversion itself would give NaN above 464). The sign of zero is kept.
__device__ __forceinline__ uint32_t mx_fp8x2(float a, float b) {
    a = fminf(fmaxf(a, -448.f), 448.f);
    b = fminf(fmaxf(b, -448.f), 448.f);
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}
// Block-wise FP8: two values of a block with fp32 scale s -> two E4M3 codes of v / s
// (fp32 division), both 0 when s is 0 (an all-zero block).
__device__ __forceinline__ uint32_t blk_fp8x2(float a, float b, float s) {
    return s > 0.f ? mx_fp8x2(a / s, b / s) : 0u;
}
// One value (already divided by the block scale) -> E2M1 code: nearest of 0, 0.5, 1,
// 1.5, 2, 3, 4, 6, ties to the even code, saturating at 6, sign bit 8.
__device__ __forceinline__ uint32_t mx_fp4(float q) {
    const float a = fabsf(q);
    const uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) + (a >= 3.5f) + (a > 5.0f);
    return c | (signbit(q) ? 8u : 0u);
}

// ------------------------------------------------------------- host launchers
// Each returns hipSuccess or the launch error; arguments were validated by the
// caller. `cap` and `fill` are device pointers written by the routing step.

struct RouteWs {
    int32_t *counts;  // [E][k][nblk] per-tile route counts, scanned in place to offsets
    int32_t nblk;
};

hipError_t launch_gate_project(const moe_shape &s, const void *x, const float *Wg, float *logits,
                               hipStream_t st);
// Whether the gate projection's LDS tiles fit for this model dim / expert count.
bool gate_supported(int M, int E, int dtype);
// Routing phase 2 inside the assignment launch of moe_route when the per-tile count
// table is small (E * k * nblk <= kScanInBlock, 8 KiB): each of its few workgroups
// (one per four routing tiles) reads the raw counts [E][k][nblk] and scans them itself,
// which saves the scan's own launch (S = 4096, E = 8, k = 2: 13.2 -> 10.7 us). Not in
// the fused forward's encode launch, whose many workgroups would each re-read the table
// (measured: slower, and 15% slower at S = 8192, E = 16, k = 3).
constexpr int kScanInBlock = 2048;
inline bool scan_in_assign(int E, int k, int nblk) {
    return static_cast<int64_t>(E) * k * nblk <= kScanInBlock;
}
// The scan: off[] (same layout as counts) gets each expert's exclusive prefix in (route,
// tile) order, need[e] the expert's total. The table is first copied into off[] with
// every thread's loads in flight together (the loads are independent; a loop-carried
// scan over global memory would wait for one load latency per 64 counts), then one
// wavefront per expert scans its counts in place, 64 a step.
__device__ __forceinline__ void block_scan_counts(const int32_t *__restrict__ counts, int E, int L,
                                                  int32_t *off, int32_t *need) {
    const int T = E * L, nt = blockDim.x;
    constexpr int U = 8;
    for (int b = threadIdx.x; b < T; b += nt * U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = b + u * nt < T ? counts[b + u * nt] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (b + u * nt < T) off[b + u * nt] = v[u];
    }
    __syncthreads();
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = nt >> 6;
    for (int e = w; e < E; e += nw) {
        int run = 0;
        for (int b = 0; b < L; b += 64) {
            const int i = e * L + b + lane;
            const bool in = b + lane < L;
            const int v = in ? off[i] : 0;
            int inc = v;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(inc, o, 64);
                if (lane >= o) inc += t;
            }
            if (in) off[i] = run + inc - v;
            run += __shfl(inc, 63, 64);
        }
        if (lane == 0) need[e] = run;
    }
    __syncthreads();
}

// Capacity C from the per-expert route counts, in every thread of a 256-thread
// block: mode +1 the factor's bound (cap_by_factor), 0 the largest count, -1 the
// smaller of the two; at least 1. sh: 4 ints of LDS.
__device__ __forceinline__ int block_capacity(const int32_t *needed, int E, int mode, int64_t cap_by_factor,
                                              int *sh) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    int mx = 0;
    for (int e = tid; e < E; e += 256) mx = max(mx, needed[e]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
    if (lane == 0) sh[wv] = mx;
    __syncthreads();
    mx = max(max(sh[0], sh[1]), max(sh[2], sh[3]));
    const int64_t c = mode > 0 ? cap_by_factor : (mode == 0 ? mx : min<int64_t>(cap_by_factor, mx));
    return static_cast<int>(c < 1 ? 1 : c);
}
inline int capacity_mode(const moe_shape &s) {
    return s.capacity_factor > 0 ? 1 : (s.capacity_factor == 0 ? 0 : -1);
}

// Routing phases 1 and 2 (top-k, gates, per-tile counts scanned to offsets, needed;
// with scan = false phase 1 only, the counts left raw); launch_assign_encode then
// places every route and encodes.
hipError_t launch_route_counts(const moe_shape &s, const float *logits, int32_t *idx, float *gates,
                               int32_t *needed, RouteWs ws, hipStream_t st, bool scan = true);
// Phase 3 of routing fused with encode: loc, fill, capacity and slot_route as
// launch_route's, and buf as launch_encode's, in one launch.
hipError_t launch_assign_encode(const moe_shape &s, const void *x, const int32_t *idx, RouteWs ws,
                                const int32_t *needed, int64_t cap_by_factor, int32_t *loc, int32_t *fill,
                                int32_t *cap, int32_t *slot_route, void *buf, int32_t cmax, hipStream_t st);
hipError_t launch_route(const moe_shape &s, const float *logits, int32_t *idx, int32_t *loc,
                        float *gates, int32_t *needed, int32_t *fill, int32_t *cap, int32_t *slot_route,
                        RouteWs ws, int64_t cap_by_factor, hipStream_t st);
hipError_t launch_encode(const moe_shape &s, const void *x, const int32_t *idx, const int32_t *loc,
                         const int32_t *fill, const int32_t *cap, void *buf, int32_t cmax,
                         hipStream_t st);
// Gate-weighted combine (unit_gates = false) or plain gather-sum (gates ignored);
// yres: Residual-MoE's dense-branch rows (y_r, or dx_r in the encode backward),
// added after the routes, before the rounding.
hipError_t launch_decode(const moe_shape &s, const void *y, const float *gates, const int32_t *idx,
                         const int32_t *loc, const int32_t *cap, void *out, bool unit_gates,
                         hipStream_t st, const void *yres = nullptr);
// Residual-MoE dense branch: pre_r = x W1r^T + b1r (stored when pre_r is non-NULL),
// h_r = act(pre_r), y_r = h_r W2r^T + b2r over all S tokens; dense_rows is 2 int32 of
// device scratch (the branch's row count and "capacity").
hipError_t launch_residual_ffn(const moe_shape &s, const void *x, const void *W1r, const void *b1r,
                               const void *W2r, const void *b2r, void *pre_r, void *h_r, void *y_r,
                               int32_t *dense_rows, hipStream_t st);
// Its backward for upstream gradient dout [S, M]: dpre_r, dx_r = dpre_r W1r (stored),
// dW1r, db1r, dW2r, db2r (fp32; the bias gradients may be NULL).
hipError_t launch_residual_bwd(const moe_shape &s, const void *dout, const void *x, const void *pre_r,
                               const void *h_r, const void *W1r, const void *W2r, void *dpre_r, void *dx_r,
                               float *dW1r, float *db1r, float *dW2r, float *db2r, int32_t *dense_rows,
                               hipStream_t st);
hipError_t launch_decode_bwd(const moe_shape &s, const void *dout, const void *y, const float *gates,
                             const int32_t *idx, const int32_t *loc, const int32_t *cap, void *dy,
                             float *dgates, hipStream_t st);
hipError_t launch_fc1(const moe_shape &s, const void *buf, const void *W1, const void *b1, const int32_t *fill,
                      const int32_t *cap, void *pre, void *h, int32_t cmax, hipStream_t st);
hipError_t launch_fc2(const moe_shape &s, const void *h, const void *W2, const void *b2, const int32_t *fill,
                      const int32_t *cap, void *y, int32_t cmax, hipStream_t st);
// fc1 and fc2 on the capacity slots [s0, s1) of every expert only (bf16 data).
hipError_t launch_ffn_window(const moe_shape &s, const void *buf, const void *W1, const void *b1, const void *W2,
                             const void *b2, const int32_t *fill, const int32_t *cap, void *pre, void *h, void *y,
                             int32_t cmax, int32_t s0, int32_t s1, hipStream_t st);
// Gate backward: dlogits (and, with needed, the auxiliary-loss partials in ws
// and aux_loss if non-NULL); dWg = x^T dlogits; dx = kept dbuf rows + dlogits Wg^T.
size_t gate_grad_ws_bytes(int S, int M, int E);
hipError_t launch_gate_backward(const moe_shape &s, const float *logits, const int32_t *idx, const float *dgates,
                                const int32_t *needed, double aux_coef, float *dlogits, float *aux_loss, void *ws,
                                hipStream_t st);
hipError_t launch_gate_weight_grad(const moe_shape &s, const void *x, const float *dlogits, float *dWg, void *ws,
                                   hipStream_t st);
// dxres (may be NULL): Residual-MoE's dense-branch dx_r rows, added last before the rounding.
hipError_t launch_gate_dx(const moe_shape &s, const void *dbuf, const int32_t *idx, const int32_t *loc,
                          const int32_t *cap, const float *dlogits, const float *Wg, void *dx, hipStream_t st,
                          const void *dxres = nullptr);
// MX: quantise a row-major [rows, K] matrix (K a multiple of 32) of the data type;
// encode with the token rows quantised to MXFP8; the expert FFN on MX operands.
hipError_t launch_mx_quantize(int fmt, int64_t rows, int32_t K, int dtype, const void *src, uint8_t *codes,
                              uint8_t *scales, hipStream_t st);
hipError_t launch_encode_mx(const moe_shape &s, const void *x, const int32_t *idx, const int32_t *loc,
                            const int32_t *fill, const int32_t *cap, uint8_t *buf_codes, uint8_t *buf_scales,
                            int32_t cmax, hipStream_t st);
// Block-wise FP8: quantise a row-major [rows, K] matrix (K a multiple of 128) in blocks of
// brows (1 or 128; rows a multiple of it) x 128; encode with the token rows quantised in
// 1 x 128 blocks. The FFN launchers below take wfmt = kBlkFp8 for this scheme (scales fp32).
hipError_t launch_blk_quantize(int brows, int64_t rows, int32_t K, int dtype, const void *src, uint8_t *codes,
                               float *scales, hipStream_t st);
// Expert fc1 / fc2 with NVFP4 weights (codes [E*N][K/2], E4M3 block scales [E*N][K/16],
// fp32 g [E]) and bf16 tokens: the bf16 products' definitions on the weights' values.
hipError_t launch_fc1_nvfp4(const moe_shape &s, const void *buf, const uint8_t *w1_codes, const uint8_t *w1_scales,
                            const float *w1_g, const void *b1, const int32_t *fill, const int32_t *cap, void *pre,
                            void *h, int32_t cmax, hipStream_t st);
hipError_t launch_fc2_nvfp4(const moe_shape &s, const void *h, const uint8_t *w2_codes, const uint8_t *w2_scales,
                            const float *w2_g, const void *b2, const int32_t *fill, const int32_t *cap, void *y,
                            int32_t cmax, hipStream_t st);
// NVFP4 weights: rows / ntensor rows per tensor, K a multiple of 16; g [ntensor].
hipError_t launch_nvfp4_quantize(int64_t rows, int32_t K, int32_t ntensor, int dtype, const void *src,
                                 uint8_t *codes, uint8_t *scales, float *g, hipStream_t st);
hipError_t launch_encode_blk(const moe_shape &s, const void *x, const int32_t *idx, const int32_t *loc,
                             const int32_t *fill, const int32_t *cap, uint8_t *buf_codes, float *buf_scales,
                             int32_t cmax, hipStream_t st);
hipError_t launch_fc1_mx(const moe_shape &s, int wfmt, const uint8_t *buf_codes, const uint8_t *buf_scales,
                         const uint8_t *w1_codes, const uint8_t *w1_scales, const void *b1, const int32_t *fill,
                         const int32_t *cap, uint8_t *h_codes, uint8_t *h_scales, int32_t cmax, hipStream_t st);
hipError_t launch_fc2_mx(const moe_shape &s, int wfmt, const uint8_t *h_codes, const uint8_t *h_scales,
                         const uint8_t *w2_codes, const uint8_t *w2_scales, const void *b2, const int32_t *fill,
                         const int32_t *cap, void *y, int32_t cmax, hipStream_t st);
hipError_t launch_expert_ffn_mx(const moe_shape &s, int wfmt, const uint8_t *buf_codes, const uint8_t *buf_scales,
                                const uint8_t *w1_codes, const uint8_t *w1_scales, const void *b1,
                                const uint8_t *w2_codes, const uint8_t *w2_scales, const void *b2,
                                const int32_t *fill, const int32_t *cap, uint8_t *h_codes, uint8_t *h_scales, void *y,
                                int32_t cmax, hipStream_t st);
// The FFN backward's four products (one kernel each), then all four in order.
hipError_t launch_fc2_bwd_data(const moe_shape &s, const void *dy, const void *W2, const void *pre,
                               const int32_t *fill, const int32_t *cap, void *dpre, int32_t cmax, hipStream_t st);
hipError_t launch_fc2_wgrad(const moe_shape &s, const void *dy, const void *h, const int32_t *fill, const int32_t *cap,
                            float *dW2, float *db2, int32_t cmax, hipStream_t st);
hipError_t launch_fc1_bwd_data(const moe_shape &s, const void *dpre, const void *W1, const int32_t *fill,
                               const int32_t *cap, void *dbuf, int32_t cmax, hipStream_t st);
hipError_t launch_fc1_wgrad(const moe_shape &s, const void *dpre, const void *buf, const int32_t *fill,
                            const int32_t *cap, float *dW1, float *db1, int32_t cmax, hipStream_t st);
hipError_t launch_expert_ffn_bwd(const moe_shape &s, const void *buf, const void *pre, const void *h,
                                 const void *W1, const void *W2, const int32_t *fill,
                                 const int32_t *cap, const void *dy, void *dpre, void *dbuf, float *dW1,
                                 float *db1, float *dW2, float *db2, int32_t cmax, hipStream_t st);

}  // namespace moe
