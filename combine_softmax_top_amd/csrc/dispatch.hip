// Index-based dispatch and combine on gfx950 (HBM-bound row copies):
//  - encode (kernel K1 forward of the MoE training blog, part 3 section 3.5):
//    one wavefront per token reads the token's row once with 16-byte loads and
//    writes it to each kept slot; the same launch zero-fills padding rows;
//  - decode (K0 forward) and the encode backward (K0 on dbuf): one wavefront
//    per token gathers the token's kept rows and accumulates in fp32;
//  - decode backward (K1 backward + K2): dy rows = gate * dout, and the gate
//    gradient <dout, y[slot]>;
//  - the gate projection x . Wg with fp64 accumulation.
// Rows are moved as uint4 (8 bf16 or 4 fp32). Grids are sized to fill the
// chip and loop over tokens/rows (grid-stride), reading C from the device.
#include <algorithm>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

__device__ __forceinline__ int64_t global_wave() {
    return (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
}
__device__ __forceinline__ int64_t num_waves() { return static_cast<int64_t>(gridDim.x) * kWavesPerBlock; }

// Slot of route `lane` of token s (lanes < k), -1 when dropped or lane >= k.
__device__ __forceinline__ int lane_slot(const int32_t *idx, const int32_t *loc, int64_t s, int S, int k, int C,
                                         int lane) {
    if (lane >= k) return -1;
    const int64_t q = static_cast<int64_t>(lane) * S + s;
    const int l = loc[q];
    return l < C ? idx[q] * C + l : -1;
}

__device__ __forceinline__ int wave_read(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float wave_read(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// ---------------------------------------------------------------- encode

__global__ __launch_bounds__(kThreads) void encode_kernel(const uint4 *__restrict__ x, const int32_t *__restrict__ idx,
                                                          const int32_t *__restrict__ loc,
                                                          const int32_t *__restrict__ fill,
                                                          const int32_t *__restrict__ cap, uint4 *__restrict__ buf,
                                                          int S, int E, int k, int V) {
    const int C = *cap;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = num_waves();
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t s = global_wave(); s < S; s += nw) {
        const int slot = lane_slot(idx, loc, s, S, k, C, lane);
        const uint4 *src = x + s * V;
        int v = lane;
        for (; v + 3 * kWave < V; v += 4 * kWave) {
            uint4 a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) a[u] = src[v + u * kWave];
            for (int r = 0; r < k; ++r) {
                const int sl = wave_read(slot, r);
                if (sl < 0) continue;
                uint4 *dst = buf + static_cast<int64_t>(sl) * V + v;
#pragma unroll
                for (int u = 0; u < 4; ++u) dst[u * kWave] = a[u];
            }
        }
        for (; v < V; v += kWave) {
            const uint4 a = src[v];
            for (int r = 0; r < k; ++r) {
                const int sl = wave_read(slot, r);
                if (sl >= 0) buf[static_cast<int64_t>(sl) * V + v] = a;
            }
        }
    }
    // Padding rows j in [fill[e], C) of every expert are +0.
    const int64_t rows = static_cast<int64_t>(E) * C;
    for (int64_t row = global_wave(); row < rows; row += nw) {
        const int e = static_cast<int>(row / C);
        const int j = static_cast<int>(row - static_cast<int64_t>(e) * C);
        if (j < fill[e]) continue;
        uint4 *dst = buf + row * V;
        for (int v = lane; v < V; v += kWave) dst[v] = zero;
    }
}

// ---------------------------------------------------------------- decode / gather-sum

template <bool BF16>
struct Vec;
template <>
struct Vec<true> {  // 8 bf16 in a uint4
    static constexpr int N = 8;
    __device__ static void unpack(const uint4 &u, float *f) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f[2 * i] = __uint_as_float(w[i] << 16);
            f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
    __device__ static uint4 pack(const float *f) {
        return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                          pack_bf16x2(f[6], f[7]));
    }
};
template <>
struct Vec<false> {  // 4 fp32 in a uint4
    static constexpr int N = 4;
    __device__ static void unpack(const uint4 &u, float *f) {
        f[0] = __uint_as_float(u.x);
        f[1] = __uint_as_float(u.y);
        f[2] = __uint_as_float(u.z);
        f[3] = __uint_as_float(u.w);
    }
    __device__ static uint4 pack(const float *f) {
        return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
    }
};

// out[s] = sum over kept routes r (in order) of g_r * rows[slot_r], fp32 from +0,
// multiply and add separately rounded. UNIT: g_r = 1 and the multiply is
// skipped (encode backward: dx = sum of dbuf rows).
template <bool BF16, bool UNIT>
__global__ __launch_bounds__(kThreads) void gather_sum_kernel(const uint4 *__restrict__ rows,
                                                              const float *__restrict__ gates,
                                                              const int32_t *__restrict__ idx,
                                                              const int32_t *__restrict__ loc,
                                                              const int32_t *__restrict__ cap,
                                                              uint4 *__restrict__ out, int S, int k, int V) {
#pragma clang fp contract(off)
    using VT = Vec<BF16>;
    constexpr int N = VT::N;
    constexpr int RB = 8;  // routes whose loads are issued together
    const int C = *cap;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = num_waves();
    for (int64_t s = global_wave(); s < S; s += nw) {
        const int slot = lane_slot(idx, loc, s, S, k, C, lane);
        float g = 0.f;
        if (!UNIT && slot >= 0) g = gates[static_cast<int64_t>(lane) * S + s];
        for (int v = lane; v < V; v += kWave) {
            float acc[N];
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] = 0.f;
            for (int r0 = 0; r0 < k; r0 += RB) {
                uint4 val[RB];
                float gr[RB];
                int sls[RB];
#pragma unroll
                for (int u = 0; u < RB; ++u) {
                    const int r = r0 + u;
                    sls[u] = r < k ? wave_read(slot, r) : -1;
                    gr[u] = (UNIT || sls[u] < 0) ? 0.f : wave_read(g, r);
                    val[u] = make_uint4(0u, 0u, 0u, 0u);
                    if (sls[u] >= 0) val[u] = rows[static_cast<int64_t>(sls[u]) * V + v];
                }
#pragma unroll
                for (int u = 0; u < RB; ++u) {
                    if (sls[u] < 0) continue;
                    float f[N];
                    VT::unpack(val[u], f);
#pragma unroll
                    for (int i = 0; i < N; ++i) acc[i] = UNIT ? acc[i] + f[i] : acc[i] + gr[u] * f[i];
                }
            }
            out[s * V + v] = VT::pack(acc);
        }
    }
}

// ---------------------------------------------------------------- decode backward (K1' + K2)

// dy[slot_r] = round(g_r * dout[s]) for every kept route, and
// dgates[r][s] = <dout[s], y[slot_r]> (fp32), 0 for dropped routes.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void decode_bwd_kernel(const uint4 *__restrict__ dout,
                                                              const uint4 *__restrict__ y,
                                                              const float *__restrict__ gates,
                                                              const int32_t *__restrict__ idx,
                                                              const int32_t *__restrict__ loc,
                                                              const int32_t *__restrict__ cap,
                                                              uint4 *__restrict__ dy, float *__restrict__ dgates,
                                                              int S, int k, int V) {
    using VT = Vec<BF16>;
    constexpr int N = VT::N;
    const int C = *cap;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = num_waves();
    for (int64_t s = global_wave(); s < S; s += nw) {
        const int slot = lane_slot(idx, loc, s, S, k, C, lane);
        float g = 0.f;
        if (slot >= 0) g = gates[static_cast<int64_t>(lane) * S + s];
        const uint4 *drow = dout + s * V;
        for (int r = 0; r < k; ++r) {
            const int sl = wave_read(slot, r);
            float dot = 0.f;
            if (sl >= 0) {
                const float gr = wave_read(g, r);
                const uint4 *yrow = y + static_cast<int64_t>(sl) * V;
                uint4 *dyrow = dy + static_cast<int64_t>(sl) * V;
                for (int v = lane; v < V; v += kWave) {
                    float d[N], yy[N], o[N];
                    VT::unpack(drow[v], d);
                    VT::unpack(yrow[v], yy);
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        o[i] = gr * d[i];
                        dot += d[i] * yy[i];
                    }
                    dyrow[v] = VT::pack(o);
                }
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, kWave);
            }
            if (lane == 0) dgates[static_cast<int64_t>(r) * S + s] = dot;
        }
    }
}

// ---------------------------------------------------------------- gate projection

// logits[s][e] = fp32(sum_m x[s][m] * Wg[m][e]): one thread per output, an fp64
// accumulator updated in increasing m. Each product of a bf16/fp32 input and an
// fp32 weight is exact in fp64, so fma(x, w, acc) rounds exactly like acc + x*w
// and the fp32 logit is the fp64 sequential sum rounded once. A block covers TT
// tokens and all E experts (IPT experts per thread when E > 256). Per chunk of
// MC rows of Wg, the block first copies the chunk of Wg and its TT rows of x
// into LDS with all loads in flight at once (the chains are short, so load
// latency, not arithmetic, bounds this kernel), then runs the chains from LDS.
constexpr int GP_W_FLOATS = 8192;  // Wg rows of one chunk: 32 KiB
constexpr int GP_X_BYTES = 32768;  // the block's x rows of one chunk: 32 KiB
constexpr int GP_MAX_TT = 16;
constexpr int GP_UNROLL = 8;       // 16-byte loads in flight per thread

template <bool BF16>
__global__ __launch_bounds__(kThreads) void gate_project_kernel(const void *__restrict__ xv,
                                                                const float *__restrict__ Wg,
                                                                float *__restrict__ logits, int S, int M, int E,
                                                                int TT, int MC) {
    __shared__ float4 ws[GP_W_FLOATS / 4];
    // row t of the x chunk starts at xs[t * xstride]; the one-vector pad puts
    // consecutive tokens' vectors on different banks
    __shared__ uint4 xs[GP_X_BYTES / 16 + GP_MAX_TT];
    constexpr int EPV = BF16 ? 8 : 4;  // x elements per 16-byte vector
    const int tid = threadIdx.x, nt = blockDim.x;
    const int64_t s0 = static_cast<int64_t>(blockIdx.x) * TT;
    const int ntok = static_cast<int>(min<int64_t>(TT, S - s0));
    const int items = TT * E;
    const int xstride = MC / EPV + 1;
    const uint4 *xg = reinterpret_cast<const uint4 *>(xv);  // row s, vector v at xg[s * (M / EPV) + v]
    const float4 *wg = reinterpret_cast<const float4 *>(Wg);
    const float *wsf = reinterpret_cast<const float *>(ws);
    constexpr int IPT = kMaxE / 256;
    double acc[IPT];
    int tok[IPT], ex[IPT];
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
        acc[j] = 0.0;
        const int it = tid + j * nt;
        tok[j] = it < items ? it / E : -1;
        ex[j] = it < items ? it - (it / E) * E : 0;
        if (tok[j] >= ntok) tok[j] = -1;
    }
    for (int m0 = 0; m0 < M; m0 += MC) {
        const int mc = min(MC, M - m0);
        const int nv = mc / EPV;
        __syncthreads();
        // Wg rows m0 .. m0+mc-1 are mc*E contiguous floats (a multiple of 8)
        const int nw = mc * E / 4;
        const float4 *wsrc = wg + static_cast<int64_t>(m0) * E / 4;
        // loads are unconditional (index clamped to the last element) so that the
        // staging registers stay registers; only the LDS stores are guarded
        for (int i0 = tid; i0 < nw; i0 += GP_UNROLL * nt) {
            float4 r[GP_UNROLL];
#pragma unroll
            for (int u = 0; u < GP_UNROLL; ++u) r[u] = wsrc[min(i0 + u * nt, nw - 1)];
#pragma unroll
            for (int u = 0; u < GP_UNROLL; ++u)
                if (i0 + u * nt < nw) ws[i0 + u * nt] = r[u];
        }
        const int nx = ntok * nv;
        for (int i0 = tid; i0 < nx; i0 += GP_UNROLL * nt) {
            uint4 r[GP_UNROLL];
            int dst[GP_UNROLL];
#pragma unroll
            for (int u = 0; u < GP_UNROLL; ++u) {
                const int i = min(i0 + u * nt, nx - 1);
                const int t = i / nv, v = i - t * nv;
                r[u] = xg[(s0 + t) * (M / EPV) + m0 / EPV + v];
                dst[u] = t * xstride + v;
            }
#pragma unroll
            for (int u = 0; u < GP_UNROLL; ++u)
                if (i0 + u * nt < nx) xs[dst[u]] = r[u];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < IPT; ++j) {
            if (tok[j] < 0) continue;
            const uint4 *xr = xs + tok[j] * xstride;
            const float *wcol = wsf + ex[j];
#pragma unroll 2
            for (int v = 0; v < nv; ++v) {
                const uint4 u = xr[v];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
                float xf[EPV];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (BF16) {
                        xf[2 * q] = __uint_as_float(w4[q] << 16);
                        xf[2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
                    } else {
                        xf[q] = __uint_as_float(w4[q]);
                    }
                }
#pragma unroll
                for (int q = 0; q < EPV; ++q)
                    acc[j] = fma(static_cast<double>(xf[q]), static_cast<double>(wcol[(v * EPV + q) * E]), acc[j]);
            }
        }
    }
#pragma unroll
    for (int j = 0; j < IPT; ++j)
        if (tok[j] >= 0) logits[(s0 + tok[j]) * E + ex[j]] = static_cast<float>(acc[j]);
}

int grid_for(int64_t waves) {
    // enough waves to cover the work, capped at 32 waves per CU on 256 CUs
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    return static_cast<int>(blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks));
}

}  // namespace

hipError_t launch_gate_project(const moe_shape &s, const void *x, const float *Wg, float *logits, hipStream_t st) {
    if (s.S == 0) return hipSuccess;
    // tokens per block: up to 256 outputs per block, at most 16 tokens so that
    // small-E layers still spread over many workgroups
    const int TT = s.E >= 256 ? 1 : std::min(GP_MAX_TT, 256 / s.E);
    const int threads = s.E > 256 ? 256 : std::max(64, ((TT * s.E + 63) / 64) * 64);
    const int esz = s.dtype == MOE_DT_BF16 ? 2 : 4;
    // chunk rows: Wg chunk and x chunk each fit their LDS area; a multiple of 8
    // (>= 16 for E <= 512), so every chunk is whole 16-byte vectors
    const int MC = std::min(GP_W_FLOATS / s.E, GP_X_BYTES / (esz * TT)) & ~7;
    const int grid = (s.S + TT - 1) / TT;
    if (s.dtype == MOE_DT_BF16)
        hipLaunchKernelGGL(gate_project_kernel<true>, dim3(grid), dim3(threads), 0, st, x, Wg, logits, s.S, s.M, s.E,
                           TT, MC);
    else
        hipLaunchKernelGGL(gate_project_kernel<false>, dim3(grid), dim3(threads), 0, st, x, Wg, logits, s.S, s.M,
                           s.E, TT, MC);
    return hipGetLastError();
}

hipError_t launch_encode(const moe_shape &s, const void *x, const int32_t *idx, const int32_t *loc,
                         const int32_t *fill, const int32_t *cap, void *buf, int32_t cmax, hipStream_t st) {
    const int eb = s.dtype == MOE_DT_BF16 ? 2 : 4;
    const int V = s.M * eb / 16;
    const int grid = grid_for(static_cast<int64_t>(s.S) + static_cast<int64_t>(s.E) * cmax);
    hipLaunchKernelGGL(encode_kernel, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint4 *>(x), idx, loc, fill,
                       cap, static_cast<uint4 *>(buf), s.S, s.E, s.k, V);
    return hipGetLastError();
}

hipError_t launch_decode(const moe_shape &s, const void *y, const float *gates, const int32_t *idx,
                         const int32_t *loc, const int32_t *cap, void *out, bool unit_gates, hipStream_t st) {
    if (s.S == 0) return hipSuccess;
    const int eb = s.dtype == MOE_DT_BF16 ? 2 : 4;
    const int V = s.M * eb / 16;
    const int grid = grid_for(s.S);
    auto Y = static_cast<const uint4 *>(y);
    auto O = static_cast<uint4 *>(out);
    if (s.dtype == MOE_DT_BF16) {
        if (unit_gates)
            hipLaunchKernelGGL((gather_sum_kernel<true, true>), dim3(grid), dim3(kThreads), 0, st, Y, gates, idx, loc,
                               cap, O, s.S, s.k, V);
        else
            hipLaunchKernelGGL((gather_sum_kernel<true, false>), dim3(grid), dim3(kThreads), 0, st, Y, gates, idx, loc,
                               cap, O, s.S, s.k, V);
    } else {
        if (unit_gates)
            hipLaunchKernelGGL((gather_sum_kernel<false, true>), dim3(grid), dim3(kThreads), 0, st, Y, gates, idx, loc,
                               cap, O, s.S, s.k, V);
        else
            hipLaunchKernelGGL((gather_sum_kernel<false, false>), dim3(grid), dim3(kThreads), 0, st, Y, gates, idx,
                               loc, cap, O, s.S, s.k, V);
    }
    return hipGetLastError();
}

hipError_t launch_decode_bwd(const moe_shape &s, const void *dout, const void *y, const float *gates,
                             const int32_t *idx, const int32_t *loc, const int32_t *cap, void *dy, float *dgates,
                             hipStream_t st) {
    if (s.S == 0) return hipSuccess;
    const int eb = s.dtype == MOE_DT_BF16 ? 2 : 4;
    const int V = s.M * eb / 16;
    const int grid = grid_for(s.S);
    auto D = static_cast<const uint4 *>(dout);
    auto Y = static_cast<const uint4 *>(y);
    auto DY = static_cast<uint4 *>(dy);
    if (s.dtype == MOE_DT_BF16)
        hipLaunchKernelGGL(decode_bwd_kernel<true>, dim3(grid), dim3(kThreads), 0, st, D, Y, gates, idx, loc, cap, DY,
                           dgates, s.S, s.k, V);
    else
        hipLaunchKernelGGL(decode_bwd_kernel<false>, dim3(grid), dim3(kThreads), 0, st, D, Y, gates, idx, loc, cap,
                           DY, dgates, s.S, s.k, V);
    return hipGetLastError();
}

}  // namespace moe
