// Gate backward on gfx950: the softmax top-k gate's gradient and the
// auxiliary load-balance loss (MoE training blog, part 2 section 2.1: the
// auxiliary loss coefficient 0.01), all fp32, all deterministic (fixed
// reduction orders, no floating-point atomics).
//
//  - gate_bwd_kernel: one group of G lanes per token (EPL experts per lane, as
//    in routing) recomputes p = softmax(logits[s]), forms the gradient reaching
//    p -- dgates at each route's expert plus c * needed[e] from the auxiliary
//    loss -- and writes dlogits = p * (g - <p, g>). For the loss it also sums
//    q_s = sum_e needed[e] p[s][e] over the block's tokens into one fp64
//    partial per block; aux_finish_kernel adds the partials in a fixed order:
//    l_aux = alpha * E / (k S^2) * sum_s q_s.
//  - gate_wgrad_kernel: dWg[m][e] = sum_s x[s][m] dlogits[s][e]. A block owns
//    64*VM columns of x, ET experts and one slice of the tokens; wavefront w
//    takes tokens 16w .. 16w+15 of each 64-token chunk (the chunk's dlogits
//    staged in LDS), then the four add their sums in wavefront order. With
//    more than one slice, each writes a partial [M, E] and wgrad_reduce_kernel
//    adds them in a fixed order.
//  - gate_dx_kernel: dx[s] = sum of the kept dbuf rows (route order, fp32) +
//    dlogits[s] . Wg^T (+ the Residual-MoE dense branch's dx_r[s]), rounded once
//    to the data type: the encode backward with the gate projection's share fused in. A block takes 32 tokens x 256
//    columns; the dlogits . Wg^T product runs over E in chunks of 16 staged in
//    LDS (a small-K outer-product GEMM in fp32 FMA).
#include <algorithm>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kGbTile = 64;  // tokens per gate-backward block (one aux partial each)

template <int G>
__device__ __forceinline__ float group_max_f32(float v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, G));
    return v;
}
template <int G>
__device__ __forceinline__ float group_sum_f32(float v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
    return v;
}

// Value of lane r of the calling lane's group of G lanes.
template <int G, class T>
__device__ __forceinline__ T group_bcast(T v, int r) {
    if constexpr (G == 64) {
        if constexpr (sizeof(T) == 4 && !__is_same(T, int)) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), r));
        else return __builtin_amdgcn_readlane(v, r);
    } else {
        return __shfl(v, r, G);
    }
}

// Block = 256 threads, tokens [blockIdx.x * 64, +64); G lanes per token, expert
// e = lane_in_group + G * j for j < EPL. Group grp takes tokens grp, grp +
// groups, ... of the tile, B at a time, and runs every step of the B tokens
// side by side (all loads first, then each cross-lane reduction stage for all B
// tokens), so that B independent shuffles or loads are in flight where one
// token alone would wait on each. caux = alpha * E / (k S^2) (0: no auxiliary
// term; needed may then be NULL). partial[blockIdx.x] = sum of q_s over the tile.
template <int G, int EPL, int B>
__global__ __launch_bounds__(256) void gate_bwd_kernel(const float *__restrict__ logits,
                                                       const int32_t *__restrict__ idx,
                                                       const float *__restrict__ dgates,
                                                       const int32_t *__restrict__ needed, float caux, int S,
                                                       int E, int k, float *__restrict__ dlogits,
                                                       double *__restrict__ partial) {
    constexpr int groups = 256 / G;
    constexpr int NT = (kGbTile + groups - 1) / groups;  // tile tokens per group (the last may be absent)
    __shared__ double wsum[groups];
    const int tid = threadIdx.x, gl = tid % G, grp = tid / G;
    float nd[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = gl + G * j;
        nd[j] = (needed != nullptr && e < E) ? static_cast<float>(needed[e]) : 0.f;
    }
    double qsum = 0.0;  // this group's tokens, in token order
    for (int i0 = 0; i0 < NT; i0 += B) {
        float v[B][EPL], p[B][EPL], g[B][EPL], mx[B], sm[B], dot[B], q[B];
        int re[B];
        float rdg[B];
        bool ok[B];
        int srow[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int t = grp + groups * (i0 + b);
            const int s = blockIdx.x * kGbTile + t;
            ok[b] = i0 + b < NT && t < kGbTile && s < S;  // uniform across the G lanes of a group
            srow[b] = ok[b] ? s : 0;  // absent tokens compute on row 0 and store nothing
            const float *row = logits + static_cast<int64_t>(srow[b]) * E;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = gl + G * j;
                v[b][j] = e < E ? row[e] : -INFINITY;
            }
            // route r's (expert, dgate) is read by lane r of the group (k <= E <= G * EPL, and G >= k)
            re[b] = -1;
            rdg[b] = 0.f;
            if (gl < k) {
                const int64_t qi = static_cast<int64_t>(gl) * S + srow[b];
                re[b] = idx[qi];
                rdg[b] = dgates[qi];
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            mx[b] = v[b][0];
#pragma unroll
            for (int j = 1; j < EPL; ++j) mx[b] = fmaxf(mx[b], v[b][j]);
        }
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1)
#pragma unroll
            for (int b = 0; b < B; ++b) mx[b] = fmaxf(mx[b], __shfl_xor(mx[b], off, G));
#pragma unroll
        for (int b = 0; b < B; ++b) {
            sm[b] = 0.f;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                p[b][j] = gl + G * j < E ? expf(v[b][j] - mx[b]) : 0.f;
                sm[b] += p[b][j];
            }
        }
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1)
#pragma unroll
            for (int b = 0; b < B; ++b) sm[b] += __shfl_xor(sm[b], off, G);
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const float inv = 1.0f / sm[b];
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                p[b][j] *= inv;
                g[b][j] = caux * nd[j];
            }
        }
        for (int r = 0; r < k; ++r) {
#pragma unroll
            for (int b = 0; b < B; ++b) {
                const int er = group_bcast<G>(re[b], r);
                const float dgr = group_bcast<G>(rdg[b], r);
#pragma unroll
                for (int j = 0; j < EPL; ++j)
                    if (er == gl + G * j) g[b][j] += dgr;
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            dot[b] = 0.f;
            q[b] = 0.f;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                dot[b] += p[b][j] * g[b][j];
                q[b] += nd[j] * p[b][j];
            }
        }
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1)
#pragma unroll
            for (int b = 0; b < B; ++b) {
                dot[b] += __shfl_xor(dot[b], off, G);
                q[b] += __shfl_xor(q[b], off, G);
            }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (!ok[b]) continue;
            float *drow = dlogits + static_cast<int64_t>(srow[b]) * E;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = gl + G * j;
                if (e < E) drow[e] = p[b][j] * (g[b][j] - dot[b]);
            }
            qsum += static_cast<double>(q[b]);
        }
    }
    if (partial == nullptr) return;
    if (gl == 0) wsum[grp] = qsum;
    __syncthreads();
    if (tid == 0) {
        double tot = 0.0;
        for (int i = 0; i < groups; ++i) tot += wsum[i];
        partial[blockIdx.x] = tot;
    }
}

// One block: aux_loss[0] = coef * sum of the n partials (0 when n == 0).
__global__ __launch_bounds__(256) void aux_finish_kernel(const double *__restrict__ partial, int n, double coef,
                                                         float *__restrict__ aux_loss) {
    __shared__ double sh[256];
    const int tid = threadIdx.x;
    double acc = 0.0;
    for (int i = tid; i < n; i += 256) acc += partial[i];
    sh[tid] = acc;
    __syncthreads();
    for (int st = 128; st > 0; st >>= 1) {
        if (tid < st) sh[tid] += sh[tid + st];
        __syncthreads();
    }
    if (tid == 0) aux_loss[0] = static_cast<float>(coef * sh[0]);
}

// ------------------------------------------------------------- dWg

constexpr int kWgChunk = 64;  // tokens per LDS chunk (16 per wavefront)

template <bool BF16, int VM>
__device__ __forceinline__ void load_x(const void *x, int64_t off, float *f) {
    if constexpr (BF16) {
        const bf16_t *p = static_cast<const bf16_t *>(x) + off;
        if constexpr (VM == 4) {
            const uint2 u = *reinterpret_cast<const uint2 *>(p);
            f[0] = __uint_as_float(u.x << 16);
            f[1] = __uint_as_float(u.x & 0xFFFF0000u);
            f[2] = __uint_as_float(u.y << 16);
            f[3] = __uint_as_float(u.y & 0xFFFF0000u);
        } else {
            f[0] = bf16_to_f32(*p);
        }
    } else {
        const float *p = static_cast<const float *>(x) + off;
        if constexpr (VM == 4) {
            const float4 u = *reinterpret_cast<const float4 *>(p);
            f[0] = u.x;
            f[1] = u.y;
            f[2] = u.z;
            f[3] = u.w;
        } else {
            f[0] = *p;
        }
    }
}

// grid = (M / (64 VM), ceil(E / ET), nsplit); slice sp takes tokens
// [sp * per, min(S, (sp + 1) * per)), per a multiple of 64. out is dWg when
// nsplit == 1, else the partial [nsplit][M][E].
template <bool BF16, int VM, int ET>
__global__ __launch_bounds__(256) void gate_wgrad_kernel(const void *__restrict__ x,
                                                         const float *__restrict__ dlogits, int S, int M, int E,
                                                         int per, float *__restrict__ out) {
    __shared__ __align__(16) float sdl[kWgChunk * ET];
    __shared__ float sred[3][64 * VM * ET];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m0 = blockIdx.x * 64 * VM + lane * VM;
    const int e0 = blockIdx.y * ET;
    const int t_begin = blockIdx.z * per, t_end = min(S, t_begin + per);
    float acc[VM][ET];
#pragma unroll
    for (int v = 0; v < VM; ++v)
#pragma unroll
        for (int j = 0; j < ET; ++j) acc[v][j] = 0.f;
    for (int c0 = t_begin; c0 < t_end; c0 += kWgChunk) {
        const int n = min(kWgChunk, t_end - c0);
        for (int i = tid; i < kWgChunk * ET; i += 256) {
            const int t = i / ET, j = i - t * ET;
            sdl[i] = (t < n && e0 + j < E) ? dlogits[static_cast<int64_t>(c0 + t) * E + e0 + j] : 0.f;
        }
        __syncthreads();
        // wavefront w takes tokens 16w .. 16w+15 of the chunk, XB rows of x in flight at a time
        constexpr int XB = VM * ET <= 32 ? 16 : 8;
        const int tb = wave * (kWgChunk / 4), te = min(n, tb + kWgChunk / 4);
        for (int t0 = tb; t0 < te; t0 += XB) {
            float xv[XB][VM];
#pragma unroll
            for (int u = 0; u < XB; ++u) {
                const int t = min(t0 + u, te - 1);  // clamped: a repeated row is loaded, not used
                load_x<BF16, VM>(x, static_cast<int64_t>(c0 + t) * M + m0, xv[u]);
            }
#pragma unroll
            for (int u = 0; u < XB; ++u) {
                if (t0 + u >= te) break;
                const float4 *d4 = reinterpret_cast<const float4 *>(sdl + (t0 + u) * ET);
#pragma unroll
                for (int j4 = 0; j4 < ET / 4; ++j4) {
                    const float4 d = d4[j4];
#pragma unroll
                    for (int v = 0; v < VM; ++v) {
                        acc[v][4 * j4 + 0] = fmaf(xv[u][v], d.x, acc[v][4 * j4 + 0]);
                        acc[v][4 * j4 + 1] = fmaf(xv[u][v], d.y, acc[v][4 * j4 + 1]);
                        acc[v][4 * j4 + 2] = fmaf(xv[u][v], d.z, acc[v][4 * j4 + 2]);
                        acc[v][4 * j4 + 3] = fmaf(xv[u][v], d.w, acc[v][4 * j4 + 3]);
                    }
                }
            }
        }
        __syncthreads();
    }
    // wavefronts 1..3 hand their sums to wavefront 0, which adds them in order
    if (wave > 0) {
#pragma unroll
        for (int v = 0; v < VM; ++v)
#pragma unroll
            for (int j = 0; j < ET; ++j) sred[wave - 1][(v * ET + j) * 64 + lane] = acc[v][j];
    }
    __syncthreads();
    if (wave != 0) return;
    float *dst = out + static_cast<int64_t>(blockIdx.z) * M * E;
#pragma unroll
    for (int v = 0; v < VM; ++v)
#pragma unroll
        for (int j = 0; j < ET; ++j) {
            float a = acc[v][j];
#pragma unroll
            for (int w = 0; w < 3; ++w) a += sred[w][(v * ET + j) * 64 + lane];
            if (e0 + j < E) dst[static_cast<int64_t>(m0 + v) * E + e0 + j] = a;
        }
}

// dWg[i] = sum over the n slice partials partial[sp][i]. A block takes 64
// consecutive outputs; wavefront w adds slices w, w + 4, w + 8, ... (8 loads
// in flight), then wavefront 0 adds the four sums in wavefront order: a fixed
// order for a given n.
__global__ __launch_bounds__(256) void wgrad_reduce_kernel(const float *__restrict__ partial, int64_t count, int n,
                                                           float *__restrict__ dWg) {
    __shared__ float sh[3][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t i = static_cast<int64_t>(blockIdx.x) * 64 + lane;
    const bool in = i < count;
    float a = 0.f;
    for (int sp0 = wave; sp0 < n; sp0 += 32) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sp = sp0 + 4 * u;
            v[u] = (in && sp < n) ? partial[sp * count + i] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) a += v[u];
    }
    if (wave > 0) sh[wave - 1][lane] = a;
    __syncthreads();
    if (wave == 0 && in) dWg[i] = ((a + sh[0][lane]) + sh[1][lane]) + sh[2][lane];
}

// ------------------------------------------------------------- dx with the gate share

constexpr int kDxTok = 32, kDxCols = 256, kDxEK = 16;

// grid = (ceil(S / 32), ceil(M / 256)). Thread (tg = tid / 32, cg = tid % 32)
// owns columns c0 + 8 cg .. +8 of tokens t0 + tg + 8 i, i < 4.
template <bool BF16>
__global__ __launch_bounds__(256) void gate_dx_kernel(const void *__restrict__ dbuf, const int32_t *__restrict__ idx,
                                                      const int32_t *__restrict__ loc,
                                                      const int32_t *__restrict__ cap,
                                                      const float *__restrict__ dlogits,
                                                      const float *__restrict__ Wg, int S, int M, int E, int k,
                                                      const void *__restrict__ dxres, void *__restrict__ dx) {
#pragma clang fp contract(off)
    __shared__ __align__(16) float swg[kDxEK][kDxCols];
    __shared__ float sdl[kDxTok][kDxEK + 1];
    __shared__ int sslot[kDxTok * kMaxK];
    const int tid = threadIdx.x, cg = tid & 31, tg = tid >> 5;
    const int t0 = blockIdx.x * kDxTok, c0 = blockIdx.y * kDxCols;
    const int C = *cap;
    for (int i = tid; i < kDxTok * k; i += 256) {
        const int t = i / k, r = i - t * k, s = t0 + t;
        int sl = -1;
        if (s < S) {
            const int64_t q = static_cast<int64_t>(r) * S + s;
            const int l = loc[q];
            if (l < C) sl = idx[q] * C + l;
        }
        sslot[i] = sl;
    }
    float acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[i][c] = 0.f;
    for (int e0 = 0; e0 < E; e0 += kDxEK) {
        __syncthreads();  // sslot published (first chunk), previous chunk consumed
        for (int i = tid; i < kDxEK * kDxCols; i += 256) {  // Wg is L2-resident; LDS writes stay conflict-free
            const int j = i / kDxCols, m = i - j * kDxCols;
            swg[j][m] = (c0 + m < M && e0 + j < E) ? Wg[static_cast<int64_t>(c0 + m) * E + e0 + j] : 0.f;
        }
        for (int i = tid; i < kDxTok * kDxEK; i += 256) {
            const int t = i / kDxEK, j = i - t * kDxEK;
            sdl[t][j] = (t0 + t < S && e0 + j < E) ? dlogits[static_cast<int64_t>(t0 + t) * E + e0 + j] : 0.f;
        }
        __syncthreads();
        const int ej = min(kDxEK, E - e0);
        for (int j = 0; j < ej; ++j) {
            const float4 w0 = *reinterpret_cast<const float4 *>(&swg[j][8 * cg]);
            const float4 w1 = *reinterpret_cast<const float4 *>(&swg[j][8 * cg + 4]);
            const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float d = sdl[tg + 8 * i][j];
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[i][c] = fmaf(d, w[c], acc[i][c]);
            }
        }
    }
    const int m = c0 + 8 * cg;
    if (m >= M) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = tg + 8 * i, s = t0 + t;
        if (s >= S) break;
        float sum[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) sum[c] = 0.f;
        for (int r = 0; r < k; ++r) {
            const int sl = sslot[t * k + r];
            if (sl < 0) continue;
            if constexpr (BF16) {
                const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(dbuf) +
                                                                 static_cast<int64_t>(sl) * M + m);
                const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    sum[2 * h] = sum[2 * h] + __uint_as_float(wv[h] << 16);
                    sum[2 * h + 1] = sum[2 * h + 1] + __uint_as_float(wv[h] & 0xFFFF0000u);
                }
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(dbuf) +
                                                                   static_cast<int64_t>(sl) * M + m);
                const float4 a = p[0], b = p[1];
                const float f[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
                for (int c = 0; c < 8; ++c) sum[c] = sum[c] + f[c];
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c) sum[c] = sum[c] + acc[i][c];
        if (dxres != nullptr) {
            float f[8];
            if constexpr (BF16) {
                const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const bf16_t *>(dxres) +
                                                                 static_cast<int64_t>(s) * M + m);
                const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    f[2 * h] = __uint_as_float(wv[h] << 16);
                    f[2 * h + 1] = __uint_as_float(wv[h] & 0xFFFF0000u);
                }
            } else {
                const float4 *p = reinterpret_cast<const float4 *>(static_cast<const float *>(dxres) +
                                                                   static_cast<int64_t>(s) * M + m);
                const float4 a = p[0], b = p[1];
                f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
                f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) sum[c] = sum[c] + f[c];
        }
        if constexpr (BF16) {
            uint4 o;
            o.x = pack_bf16x2(sum[0], sum[1]);
            o.y = pack_bf16x2(sum[2], sum[3]);
            o.z = pack_bf16x2(sum[4], sum[5]);
            o.w = pack_bf16x2(sum[6], sum[7]);
            *reinterpret_cast<uint4 *>(static_cast<bf16_t *>(dx) + static_cast<int64_t>(s) * M + m) = o;
        } else {
            float4 *p = reinterpret_cast<float4 *>(static_cast<float *>(dx) + static_cast<int64_t>(s) * M + m);
            p[0] = make_float4(sum[0], sum[1], sum[2], sum[3]);
            p[1] = make_float4(sum[4], sum[5], sum[6], sum[7]);
        }
    }
}

template <int G, int EPL>
hipError_t gb_launch(const float *logits, const int32_t *idx, const float *dgates, const int32_t *needed, float caux,
                     int S, int E, int k, float *dlogits, double *partial, hipStream_t st) {
    const int nblk = (S + kGbTile - 1) / kGbTile;
    // rows in flight per group: all of the group's tile tokens, at most 32 logits per lane
    constexpr int NT = (kGbTile + 256 / G - 1) / (256 / G);
    constexpr int B = NT < 32 / EPL ? NT : 32 / EPL;
    hipLaunchKernelGGL((gate_bwd_kernel<G, EPL, B>), dim3(nblk), dim3(256), 0, st, logits, idx, dgates, needed, caux,
                       S, E, k, dlogits, partial);
    return hipGetLastError();
}

// Slices of the token range for dWg: enough blocks to fill the chip, 64-token multiples.
struct WgradPlan {
    int vm, et, mt, etiles, nsplit, per;
};
WgradPlan wgrad_plan(int S, int M, int E) {
    WgradPlan p;
    p.vm = M % 256 == 0 ? 4 : 1;
    p.et = E <= 8 ? 8 : 16;
    p.mt = M / (64 * p.vm);
    p.etiles = (E + p.et - 1) / p.et;
    const int tiles = p.mt * p.etiles;
    const int chunks = (S + kWgChunk - 1) / kWgChunk;
    int n = (512 + tiles - 1) / tiles;
    n = std::max(1, std::min(n, chunks));
    p.per = ((chunks + n - 1) / n) * kWgChunk;
    p.nsplit = S > 0 ? (S + p.per - 1) / p.per : 0;
    return p;
}

template <bool BF16, int VM, int ET>
hipError_t wgrad_launch(const WgradPlan &p, const void *x, const float *dlogits, int S, int M, int E, float *out,
                        hipStream_t st) {
    hipLaunchKernelGGL((gate_wgrad_kernel<BF16, VM, ET>), dim3(p.mt, p.etiles, p.nsplit), dim3(256), 0, st, x,
                       dlogits, S, M, E, p.per, out);
    return hipGetLastError();
}

}  // namespace

size_t gate_grad_ws_bytes(int S, int M, int E) {
    const size_t aux = ((static_cast<size_t>((S + kGbTile - 1) / kGbTile) * sizeof(double)) + 255) & ~size_t(255);
    const WgradPlan p = wgrad_plan(S, M, E);
    const size_t wg = p.nsplit > 1 ? static_cast<size_t>(p.nsplit) * M * E * sizeof(float) : 0;
    return aux + ((wg + 255) & ~size_t(255));
}

hipError_t launch_gate_backward(const moe_shape &s, const float *logits, const int32_t *idx, const float *dgates,
                                const int32_t *needed, double aux_coef, float *dlogits, float *aux_loss, void *ws,
                                hipStream_t st) {
    const int S = s.S, E = s.E, k = s.k;
    const int nblk = (S + kGbTile - 1) / kGbTile;
    const bool aux = needed != nullptr;
    double *partial = aux ? static_cast<double *>(ws) : nullptr;
    const float caux = aux && S > 0
                           ? static_cast<float>(aux_coef * E / (static_cast<double>(k) * S * static_cast<double>(S)))
                           : 0.f;
    hipError_t err = hipSuccess;
    if (nblk > 0) {
        if (E <= 64) {
            int G = 1;
            while (G < E) G <<= 1;
            switch (G) {
            case 1: err = gb_launch<1, 1>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st); break;
            case 2: err = gb_launch<2, 1>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st); break;
            case 4: err = gb_launch<4, 1>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st); break;
            case 8: err = gb_launch<8, 1>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st); break;
            case 16: err = gb_launch<16, 1>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st); break;
            case 32: err = gb_launch<32, 1>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st); break;
            default: err = gb_launch<64, 1>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st); break;
            }
        } else if (E <= 128) {
            err = gb_launch<64, 2>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st);
        } else if (E <= 256) {
            err = gb_launch<64, 4>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st);
        } else {
            err = gb_launch<64, 8>(logits, idx, dgates, needed, caux, S, E, k, dlogits, partial, st);
        }
        if (err != hipSuccess) return err;
    }
    if (aux_loss != nullptr) {
        const double coef = aux && S > 0 ? aux_coef * E / (static_cast<double>(k) * S * static_cast<double>(S)) : 0.0;
        hipLaunchKernelGGL(aux_finish_kernel, dim3(1), dim3(256), 0, st, partial, aux ? nblk : 0, coef, aux_loss);
        err = hipGetLastError();
    }
    return err;
}

hipError_t launch_gate_weight_grad(const moe_shape &s, const void *x, const float *dlogits, float *dWg, void *ws,
                                   hipStream_t st) {
    const int S = s.S, M = s.M, E = s.E;
    const WgradPlan p = wgrad_plan(S, M, E);
    const size_t aux = ((static_cast<size_t>((S + kGbTile - 1) / kGbTile) * sizeof(double)) + 255) & ~size_t(255);
    float *out = p.nsplit > 1 ? reinterpret_cast<float *>(static_cast<char *>(ws) + aux) : dWg;
    hipError_t err = hipSuccess;
    if (p.nsplit > 0) {
        const bool bf = s.dtype == MOE_DT_BF16;
        if (p.vm == 4) {
            if (p.et == 8) err = bf ? wgrad_launch<true, 4, 8>(p, x, dlogits, S, M, E, out, st)
                                    : wgrad_launch<false, 4, 8>(p, x, dlogits, S, M, E, out, st);
            else err = bf ? wgrad_launch<true, 4, 16>(p, x, dlogits, S, M, E, out, st)
                          : wgrad_launch<false, 4, 16>(p, x, dlogits, S, M, E, out, st);
        } else {
            if (p.et == 8) err = bf ? wgrad_launch<true, 1, 8>(p, x, dlogits, S, M, E, out, st)
                                    : wgrad_launch<false, 1, 8>(p, x, dlogits, S, M, E, out, st);
            else err = bf ? wgrad_launch<true, 1, 16>(p, x, dlogits, S, M, E, out, st)
                          : wgrad_launch<false, 1, 16>(p, x, dlogits, S, M, E, out, st);
        }
        if (err != hipSuccess) return err;
    }
    if (p.nsplit != 1) {  // several slices to add, or no token: dWg = 0
        const int64_t count = static_cast<int64_t>(M) * E;
        hipLaunchKernelGGL(wgrad_reduce_kernel, dim3(static_cast<unsigned>((count + 63) / 64)), dim3(256), 0, st, out,
                           count, p.nsplit, dWg);
        err = hipGetLastError();
    }
    return err;
}

hipError_t launch_gate_dx(const moe_shape &s, const void *dbuf, const int32_t *idx, const int32_t *loc,
                          const int32_t *cap, const float *dlogits, const float *Wg, void *dx, hipStream_t st,
                          const void *dxres) {
    const int S = s.S, M = s.M;
    if (S == 0) return hipSuccess;
    const dim3 grid((S + kDxTok - 1) / kDxTok, (M + kDxCols - 1) / kDxCols);
    if (s.dtype == MOE_DT_BF16)
        hipLaunchKernelGGL(gate_dx_kernel<true>, grid, dim3(256), 0, st, dbuf, idx, loc, cap, dlogits, Wg, S, M, s.E,
                           s.k, dxres, dx);
    else
        hipLaunchKernelGGL(gate_dx_kernel<false>, grid, dim3(256), 0, st, dbuf, idx, loc, cap, dlogits, Wg, S, M, s.E,
                           s.k, dxres, dx);
    return hipGetLastError();
}

}  // namespace moe
