// Index-based dispatch and combine on gfx950 (HBM-bound row copies):
//  - encode (kernel K1 forward of the MoE training blog, part 3 section 3.5):
//    one wavefront per token reads the token's row once with 16-byte loads and
//    writes it to each kept slot; the same launch zero-fills padding rows;
//  - decode (K0 forward) and the encode backward (K0 on dbuf): one wavefront
//    per token gathers the token's kept rows and accumulates in fp32;
//  - decode backward (K1 backward + K2): dy rows = gate * dout, and the gate
//    gradient <dout, y[slot]>;
//  - the gate projection x . Wg (fp32 accumulation).
// Rows are moved as uint4 (8 bf16 or 4 fp32). Grids are sized to fill the
// chip and loop over tokens/rows (grid-stride), reading C from the device.
#include <algorithm>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Streaming 16-byte accesses for rows that a launch reads or writes once
// (non-temporal: they are not kept in L2 / the Infinity Cache). Measured at
// S=32768, M=4096, E=128, k=8: decode and the encode backward 0.50 -> 0.43 ms,
// the decode backward 0.96 -> 0.86 ms (with its dout chunk read once per route
// batch); encode's row stores were slower this way (0.90 -> 0.94 ms) and stay
// ordinary stores.
__device__ __forceinline__ uint4 ld_nt(const uint4 *p) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4 *p, const uint4 &u) {
    const u32x4_t v = {u.x, u.y, u.z, u.w};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(p));
}

__device__ __forceinline__ int64_t global_wave() {
    return (static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x) / kWave;
}
__device__ __forceinline__ int64_t num_waves() { return static_cast<int64_t>(gridDim.x) * kWavesPerBlock; }

__device__ __forceinline__ int wave_read(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float wave_read(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Lane r < k of a token's wavefront: the slot e * C + loc of route r (-1 when
// the route was dropped) and, with gates given, its gate. The loads (loc, idx
// and the gate, read whether or not the route was kept) all go out together and
// are waited for once, here: the values pass through one empty asm statement.
// Without it the compiler moves each read-only load into the branch that uses
// it (one memory round trip after another), and its wait counting, which is
// conservative where branches join, would wait for every load in flight
// (vmcnt(0)) before each read of the slot or gate inside the per-route loops
// that follow, one round trip per route row.
__device__ __forceinline__ int lane_slot(const int32_t *idx, const int32_t *loc, const float *gates, int64_t s,
                                         int S, int k, int C, int lane, float &g) {
    int l = C, e = 0;
    g = 0.f;
    if (lane < k) {
        const int64_t q = static_cast<int64_t>(lane) * S + s;
        l = loc[q];
        e = idx[q];
        if (gates != nullptr) g = gates[q];
    }
    asm volatile("" : "+v"(l), "+v"(e), "+v"(g));
    return l < C ? e * C + l : -1;
}

// ---------------------------------------------------------------- encode

// Padding rows j in [min(filled[e], C), C) of every expert are +0. A wavefront
// takes rows in grid-stride order; the row index is scalar, so filled[e] is a
// scalar load and no vector-memory wait sits between one row's stores and the
// next's. At S=32768, M=4096, E=128, k=8 the clearing (2.3 GB) takes 0.43 ms on
// its own, 5.3 TB/s, against 0.34 ms for a plain fill of as many bytes; neither
// this form nor the whole grid clearing each expert's padding as one range
// (0.46 ms) closes that gap.
__device__ __forceinline__ void clear_padding(const int32_t *__restrict__ filled, uint4 *__restrict__ buf, int E,
                                              int C, int V, int lane) {
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const int64_t rows = static_cast<int64_t>(E) * C;  // below 2^31 (checked on the host)
    const int64_t nw = num_waves();
    for (int64_t row = __builtin_amdgcn_readfirstlane(static_cast<int>(global_wave())); row < rows; row += nw) {
        const int r = static_cast<int>(row);  // 32-bit division: row < rows < 2^31
        const int e = r / C;
        if (r - e * C < min(filled[e], C)) continue;
        uint4 *dst = buf + row * V;
        for (int v = lane; v < V; v += kWave) dst[v] = zero;
    }
}

__global__ __launch_bounds__(kThreads) void encode_kernel(const uint4 *__restrict__ x, const int32_t *__restrict__ idx,
                                                          const int32_t *__restrict__ loc,
                                                          const int32_t *__restrict__ fill,
                                                          const int32_t *__restrict__ cap, uint4 *__restrict__ buf,
                                                          int S, int E, int k, int V) {
    const int C = *cap;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = num_waves();
    for (int64_t s = global_wave(); s < S; s += nw) {
        float g_unused;
        const int slot = lane_slot(idx, loc, nullptr, s, S, k, C, lane, g_unused);
        const uint4 *src = x + s * V;
        // four vectors per lane at a time, the last batch masked: all loads of a
        // batch are in flight before its stores
        for (int v = lane; v < V; v += 4 * kWave) {
            uint4 a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                a[u] = v + u * kWave < V ? src[v + u * kWave] : make_uint4(0u, 0u, 0u, 0u);
            for (int r = 0; r < k; ++r) {
                const int sl = wave_read(slot, r);
                if (sl < 0) continue;
                uint4 *dst = buf + static_cast<int64_t>(sl) * V + v;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (v + u * kWave < V) dst[u * kWave] = a[u];
            }
        }
    }
    // Padding rows j in [fill[e], C) of every expert are +0.
    clear_padding(fill, buf, E, C, V, lane);
}

// Routing's phase 3 fused with encode. The wavefront of token s places each of
// its routes r as the route assignment does: rank = the number of lower tokens
// of its 64-token tile whose route r goes to the same expert (one ballot over
// the tile), loc = the tile's scanned offset for (expert, r) + rank; then the
// row is copied to the kept slots. Every block derives C from needed[]; fill is
// min(needed, C), computed where the padding rows are cleared.
__global__ __launch_bounds__(kThreads) void assign_encode_kernel(
    const uint4 *__restrict__ x, const int32_t *__restrict__ idx, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ needed, int S, int E, int k, int nblk, int mode, int64_t cap_by_factor,
    int32_t *__restrict__ loc, int32_t *__restrict__ fill, int32_t *__restrict__ cap_out,
    int32_t *__restrict__ slot_route, uint4 *__restrict__ buf, int V) {
    __shared__ int sh[4];
    const int C = block_capacity(needed, E, mode, cap_by_factor, sh);
    const int lane = threadIdx.x & (kWave - 1);
    if (blockIdx.x == 0) {
        if (threadIdx.x == 0) cap_out[0] = C;
        for (int e = threadIdx.x; e < E; e += kThreads) fill[e] = min(needed[e], C);
    }
    const int64_t nw = num_waves();
    for (int64_t s = global_wave(); s < S; s += nw) {
        const int tile = static_cast<int>(s / kRouteTile);
        const int64_t t0 = static_cast<int64_t>(tile) * kRouteTile;
        const int j = static_cast<int>(s - t0);
        const uint64_t below = j == 0 ? 0ull : (~0ull >> (64 - j));
        const bool in = t0 + lane < S;
        int slot = -1;
        for (int r = 0; r < k; ++r) {
            const int64_t q = static_cast<int64_t>(r) * S + s;
            const int e = idx[q];
            const int te = in ? idx[static_cast<int64_t>(r) * S + t0 + lane] : -1;
            const int rank = __popcll(__ballot(te == e) & below);
            const int l = offsets[(static_cast<int64_t>(e) * k + r) * nblk + tile] + rank;
            if (lane == 0) {
                loc[q] = l;
                if (slot_route != nullptr && l < C) slot_route[static_cast<int64_t>(e) * C + l] = static_cast<int32_t>(q);
            }
            if (lane == r) slot = l < C ? e * C + l : -1;
        }
        const uint4 *src = x + s * V;
        // four vectors per lane at a time, the last batch masked: all loads of a
        // batch are in flight before its stores
        for (int v = lane; v < V; v += 4 * kWave) {
            uint4 a[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                a[u] = v + u * kWave < V ? src[v + u * kWave] : make_uint4(0u, 0u, 0u, 0u);
            for (int r = 0; r < k; ++r) {
                const int sl = wave_read(slot, r);
                if (sl < 0) continue;
                uint4 *dst = buf + static_cast<int64_t>(sl) * V + v;
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (v + u * kWave < V) dst[u * kWave] = a[u];
            }
        }
    }
    // Padding rows j in [min(needed[e], C), C) of every expert are +0.
    clear_padding(needed, buf, E, C, V, lane);
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
// skipped (encode backward: dx = sum of dbuf rows). RES: Residual-MoE, the
// dense branch's row yres[s] is added after the routes, before the rounding.
template <bool BF16, bool UNIT, bool RES, int NV>
__global__ __launch_bounds__(kThreads) void gather_sum_kernel(const uint4 *__restrict__ rows,
                                                              const float *__restrict__ gates,
                                                              const int32_t *__restrict__ idx,
                                                              const int32_t *__restrict__ loc,
                                                              const int32_t *__restrict__ cap,
                                                              const uint4 *__restrict__ yres,
                                                              uint4 *__restrict__ out, int S, int k, int V) {
#pragma clang fp contract(off)
    using VT = Vec<BF16>;
    constexpr int N = VT::N;
    constexpr int RB = 8;  // routes whose loads are issued together
    const int C = *cap;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = num_waves();
    for (int64_t s = global_wave(); s < S; s += nw) {
        float g;
        const int slot = lane_slot(idx, loc, UNIT ? nullptr : gates, s, S, k, C, lane, g);
        // NV vectors per lane at a time (v, v + 64, ...): the loads of a batch of
        // routes for all of them are in flight together; each output still sums
        // its routes in route order. NV = 4 for rows of more than 128 vectors
        // (M = 4096: 0.50 -> 0.43 ms with streaming loads); shorter rows keep 2,
        // where the masked-off half would only cost registers (occupancy)
        for (int v = lane; v < V; v += NV * kWave) {
            float acc[NV][N];
#pragma unroll
            for (int h = 0; h < NV; ++h)
#pragma unroll
                for (int i = 0; i < N; ++i) acc[h][i] = 0.f;
            for (int r0 = 0; r0 < k; r0 += RB) {
                uint4 val[NV][RB];
                float gr[RB];
                int sls[RB];
#pragma unroll
                for (int u = 0; u < RB; ++u) {
                    const int r = r0 + u;
                    sls[u] = r < k ? wave_read(slot, r) : -1;
                    gr[u] = (UNIT || sls[u] < 0) ? 0.f : wave_read(g, r);
#pragma unroll
                    for (int h = 0; h < NV; ++h) val[h][u] = make_uint4(0u, 0u, 0u, 0u);
                    if (sls[u] >= 0) {
                        const uint4 *row = rows + static_cast<int64_t>(sls[u]) * V;
#pragma unroll
                        for (int h = 0; h < NV; ++h)
                            if (v + h * kWave < V) val[h][u] = ld_nt(row + v + h * kWave);
                    }
                }
#pragma unroll
                for (int u = 0; u < RB; ++u) {
                    if (sls[u] < 0) continue;
#pragma unroll
                    for (int h = 0; h < NV; ++h) {
                        float f[N];
                        VT::unpack(val[h][u], f);
#pragma unroll
                        for (int i = 0; i < N; ++i) acc[h][i] = UNIT ? acc[h][i] + f[i] : acc[h][i] + gr[u] * f[i];
                    }
                }
            }
#pragma unroll
            for (int h = 0; h < NV; ++h) {
                if (v + h * kWave >= V) break;
                const int vv = v + h * kWave;
                if constexpr (RES) {
                    float f[N];
                    VT::unpack(yres[s * V + vv], f);
#pragma unroll
                    for (int i = 0; i < N; ++i) acc[h][i] = acc[h][i] + f[i];
                }
                st_nt(out + s * V + vv, VT::pack(acc[h]));
            }
        }
    }
}

// ---------------------------------------------------------------- decode backward (K1' + K2)

// dy[slot_r] = round(g_r * dout[s]) for every kept route, and
// dgates[r][s] = <dout[s], y[slot_r]> (fp32), 0 for dropped routes. Routes go in
// batches of eight: a lane reads its chunk of dout once per batch and the
// chunks of the batch's y rows together, keeping one partial dot product per
// route (each summed over the lane's chunks in order, then across the wavefront).
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
    constexpr int RB = 8;  // routes per batch: the token's dout chunk is read once per batch
    const int C = *cap;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t nw = num_waves();
    for (int64_t s = global_wave(); s < S; s += nw) {
        float g;
        const int slot = lane_slot(idx, loc, gates, s, S, k, C, lane, g);
        const uint4 *drow = dout + s * V;
        for (int r0 = 0; r0 < k; r0 += RB) {
            int sls[RB];
            float gr[RB], dot[RB];
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                sls[u] = r0 + u < k ? wave_read(slot, r0 + u) : -1;
                gr[u] = sls[u] >= 0 ? wave_read(g, r0 + u) : 0.f;
                dot[u] = 0.f;
            }
            for (int v = lane; v < V; v += kWave) {
                float d[N];
                VT::unpack(ld_nt(drow + v), d);
                uint4 yv[RB];
#pragma unroll
                for (int u = 0; u < RB; ++u)
                    yv[u] = sls[u] >= 0 ? ld_nt(y + static_cast<int64_t>(sls[u]) * V + v) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
                for (int u = 0; u < RB; ++u) {
                    if (sls[u] < 0) continue;
                    float yy[N], o[N];
                    VT::unpack(yv[u], yy);
#pragma unroll
                    for (int i = 0; i < N; ++i) {
                        o[i] = gr[u] * d[i];
                        dot[u] += d[i] * yy[i];
                    }
                    uint4 *dst = dy + static_cast<int64_t>(sls[u]) * V + v;
                    st_nt(dst, VT::pack(o));
                }
            }
#pragma unroll
            for (int u = 0; u < RB; ++u) {
                if (r0 + u >= k) break;
                float t = dot[u];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, kWave);
                if (lane == 0) dgates[static_cast<int64_t>(r0 + u) * S + s] = sls[u] >= 0 ? t : 0.f;
            }
        }
    }
}

// ---------------------------------------------------------------- gate projection

// logits[s][e] = sum_m x[s][m] * Wg[m][e] in fp32 (Tutel catalogue page, "key
// configuration": the gate scores each token against the E experts). An
// HBM-bound product: x is read once; the small Wg is staged in LDS.
// A workgroup takes 16 tokens (TPW per wavefront) and one chunk of 8 experts.
// It stages Wg's rows for those experts, kGateRows rows at a time, in LDS (every load
// of a pass issued together); lane l owns the 16-byte chunks c = l, l + 64, ...
// of its tokens' rows (VE elements each) and keeps TPW * 8 fp32 sums, each taken
// over its chunks in increasing m with fused multiply-adds; the wavefront then
// adds the 64 lanes' sums in a fixed butterfly (reduce-scatter: at step b, lanes
// with bit b set keep the upper half of their values and add their partner's),
// after which lanes 2i and 2i + 1 both hold value i. The summation order is
// fixed: results are reproducible run to run.
// LDS layout: Wg row m of the pass (8 fp32) is two 16-byte units u = 2m, 2m + 1;
// a lane's chunk c covers UPC = 2 VE consecutive units, and unit u sits at slot
// u ^ ((u / UPC) mod UPC), so the 16 lanes of a read pass (consecutive chunks,
// same unit within the chunk) hit different banks.
constexpr int kGateRows = 2048;  // Wg rows per LDS pass (64 KiB)

template <bool BF16, int TPW>
__global__ __launch_bounds__(kThreads) void gate_project_kernel(const uint4 *__restrict__ x,
                                                                const float *__restrict__ Wg,
                                                                float *__restrict__ logits, int S, int M, int E) {
    constexpr int EC = 8, NV = TPW * EC, VE = BF16 ? 8 : 4, UPC = 2 * VE;
    static_assert(NV == 32, "the butterfly below reduces 32 values per lane");
    __shared__ __align__(16) f32x4_t wl[2 * kGateRows];
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t tok0 = (static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6)) * TPW;
    const int e0 = blockIdx.y * EC;
    const int ne = min(EC, E - e0);
    const bool wg4 = (E & 3) == 0;  // rows' 8-expert slices are two aligned 16-byte loads
    const int nchunks = M / VE;      // M is a multiple of 64
    float acc[TPW][EC];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int e = 0; e < EC; ++e) acc[t][e] = 0.f;
    // the token rows this wave reads: chunk c of token t, or zeros past the last token
    auto load_x = [&](uint4 (&xv)[TPW], int c) {
#pragma unroll
        for (int t = 0; t < TPW; ++t)
            xv[t] = tok0 + t < S ? x[(tok0 + t) * nchunks + c] : make_uint4(0u, 0u, 0u, 0u);
    };
    for (int m0 = 0; m0 < M; m0 += kGateRows) {
        const int rows = min(kGateRows, M - m0);
        const int c0 = m0 / VE, c1 = c0 + rows / VE;
        // the pass's first chunk of x is in flight while the expert columns are staged
        uint4 xn[TPW];
        if (tok0 < S && c0 + lane < c1) load_x(xn, c0 + lane);
        if (m0 > 0) __syncthreads();  // the previous pass is read
        // eight units per thread at a time, all eight loads issued before the stores
        for (int ub = 0; ub < 2 * rows; ub += 8 * kThreads) {
            f32x4_t v[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int u = ub + threadIdx.x + i * kThreads;
                const int64_t m = m0 + (u >> 1);
                const int eh = e0 + 4 * (u & 1);
                v[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if (u < 2 * rows) {
                    if (wg4) {
                        if (eh < E) v[i] = *reinterpret_cast<const f32x4_t *>(Wg + m * E + eh);
                    } else {
                        v[i].x = eh < E ? Wg[m * E + eh] : 0.f;
                        v[i].y = eh + 1 < E ? Wg[m * E + eh + 1] : 0.f;
                        v[i].z = eh + 2 < E ? Wg[m * E + eh + 2] : 0.f;
                        v[i].w = eh + 3 < E ? Wg[m * E + eh + 3] : 0.f;
                    }
                }
            }
            asm volatile("" : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]), "+v"(v[6]),
                         "+v"(v[7]));
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int u = ub + threadIdx.x + i * kThreads;
                if (u < 2 * rows) wl[u ^ ((u / UPC) & (UPC - 1))] = v[i];  // (the LDS tile holds f32x4_t)
            }
        }
        __syncthreads();
        if (tok0 < S) {
            for (int c = c0 + lane; c < c1; c += kWave) {
                uint4 xv[TPW];
#pragma unroll
                for (int t = 0; t < TPW; ++t) xv[t] = xn[t];
                if (c + kWave < c1) load_x(xn, c + kWave);  // the next chunk loads under this one's FMAs
                const int cl = c - c0;  // chunk within the pass
#pragma unroll
                for (int j = 0; j < VE; ++j) {
                    const int u = cl * UPC + 2 * j;
                    const f32x4_t lo = wl[u ^ (cl & (UPC - 1))];
                    const f32x4_t hi = wl[(u + 1) ^ (cl & (UPC - 1))];
                    const float w[EC] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                    for (int t = 0; t < TPW; ++t) {
                        const uint32_t word = j / (VE / 4) == 0 ? xv[t].x
                                            : j / (VE / 4) == 1 ? xv[t].y
                                            : j / (VE / 4) == 2 ? xv[t].z : xv[t].w;
                        const float xf = BF16 ? __uint_as_float((j & 1) ? (word & 0xFFFF0000u) : (word << 16))
                                              : __uint_as_float(word);
#pragma unroll
                        for (int e = 0; e < EC; ++e) acc[t][e] = fmaf(xf, w[e], acc[t][e]);
                    }
                }
            }
        }
    }
    if (tok0 >= S) return;
    float v[NV];
#pragma unroll
    for (int t = 0; t < TPW; ++t)
#pragma unroll
        for (int e = 0; e < EC; ++e) v[t * EC + e] = acc[t][e];
#pragma unroll
    for (int half = NV / 2, bit = 32; half >= 1; half >>= 1, bit >>= 1) {
        const bool upper = (lane & bit) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            // selects on values: a conditional on the two array elements themselves
            // would read the array at a lane-dependent index
            const float lo = v[i], hi = v[i + half];
            const float send = upper ? lo : hi;
            const float keep = upper ? hi : lo;
            v[i] = keep + __shfl_xor(send, bit, kWave);
        }
    }
    v[0] = v[0] + __shfl_xor(v[0], 1, kWave);
    const int idx = (lane >> 1) & (NV - 1);
    const int t = idx / EC, e = idx % EC;
    if ((lane & 1) == 0 && tok0 + t < S && e < ne) logits[(tok0 + t) * E + e0 + e] = v[0];
}

int grid_for(int64_t waves, int64_t max_blocks = 2048) {
    // enough waves to cover the work, by default capped at 32 waves per CU on 256 CUs
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    return static_cast<int>(blocks < 1 ? 1 : (blocks > max_blocks ? max_blocks : blocks));
}
// Encode (row copies and the padding clear, almost all writes) runs its grid-stride
// loops on up to 32768 workgroups: at S=32768, M=4096, E=128, k=8 the launch takes
// 0.86 ms against 0.90 ms on 2048 and 0.88 ms with one wavefront per item.
constexpr int64_t kEncodeMaxBlocks = 32768;

}  // namespace

template <bool BF16>
static hipError_t gate_launch(const moe_shape &s, const void *x, const float *Wg, float *logits, hipStream_t st) {
    constexpr int TPW = 4;
    const dim3 grid(static_cast<unsigned>((s.S + TPW * kWavesPerBlock - 1) / (TPW * kWavesPerBlock)),
                    static_cast<unsigned>((s.E + 7) / 8));
    hipLaunchKernelGGL((gate_project_kernel<BF16, TPW>), grid, dim3(kThreads), 0, st, static_cast<const uint4 *>(x),
                       Wg, logits, s.S, s.M, s.E);
    return hipGetLastError();
}

bool gate_supported(int M, int E, int dtype) {
    (void)M; (void)E; (void)dtype;  // any shape the layer supports
    return true;
}

hipError_t launch_gate_project(const moe_shape &s, const void *x, const float *Wg, float *logits, hipStream_t st) {
    if (s.S == 0) return hipSuccess;
    return s.dtype == MOE_DT_BF16 ? gate_launch<true>(s, x, Wg, logits, st) : gate_launch<false>(s, x, Wg, logits, st);
}

hipError_t launch_encode(const moe_shape &s, const void *x, const int32_t *idx, const int32_t *loc,
                         const int32_t *fill, const int32_t *cap, void *buf, int32_t cmax, hipStream_t st) {
    const int eb = s.dtype == MOE_DT_BF16 ? 2 : 4;
    const int V = s.M * eb / 16;
    const int grid = grid_for(static_cast<int64_t>(s.S) + static_cast<int64_t>(s.E) * cmax, kEncodeMaxBlocks);
    hipLaunchKernelGGL(encode_kernel, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint4 *>(x), idx, loc, fill,
                       cap, static_cast<uint4 *>(buf), s.S, s.E, s.k, V);
    return hipGetLastError();
}

hipError_t launch_assign_encode(const moe_shape &s, const void *x, const int32_t *idx, RouteWs ws,
                                const int32_t *needed, int64_t cap_by_factor, int32_t *loc, int32_t *fill,
                                int32_t *cap, int32_t *slot_route, void *buf, int32_t cmax, hipStream_t st) {
    const int eb = s.dtype == MOE_DT_BF16 ? 2 : 4;
    const int V = s.M * eb / 16;
    const int grid = grid_for(static_cast<int64_t>(s.S) + static_cast<int64_t>(s.E) * cmax, kEncodeMaxBlocks);
    hipLaunchKernelGGL(assign_encode_kernel, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint4 *>(x), idx,
                       ws.counts, needed, s.S, s.E, s.k, ws.nblk, capacity_mode(s), cap_by_factor, loc, fill, cap,
                       slot_route, static_cast<uint4 *>(buf), V);
    return hipGetLastError();
}

template <bool BF16, int NV>
static void decode_dispatch_nv(bool unit, bool res, int grid, hipStream_t st, const uint4 *Y, const float *gates,
                               const int32_t *idx, const int32_t *loc, const int32_t *cap, const uint4 *R, uint4 *O,
                               int S, int k, int V) {
    if (unit && res)
        hipLaunchKernelGGL((gather_sum_kernel<BF16, true, true, NV>), dim3(grid), dim3(kThreads), 0, st, Y, gates,
                           idx, loc, cap, R, O, S, k, V);
    else if (unit)
        hipLaunchKernelGGL((gather_sum_kernel<BF16, true, false, NV>), dim3(grid), dim3(kThreads), 0, st, Y, gates,
                           idx, loc, cap, R, O, S, k, V);
    else if (res)
        hipLaunchKernelGGL((gather_sum_kernel<BF16, false, true, NV>), dim3(grid), dim3(kThreads), 0, st, Y, gates,
                           idx, loc, cap, R, O, S, k, V);
    else
        hipLaunchKernelGGL((gather_sum_kernel<BF16, false, false, NV>), dim3(grid), dim3(kThreads), 0, st, Y, gates,
                           idx, loc, cap, R, O, S, k, V);
}
template <bool BF16>
static void decode_dispatch(bool unit, bool res, int grid, hipStream_t st, const uint4 *Y, const float *gates,
                            const int32_t *idx, const int32_t *loc, const int32_t *cap, const uint4 *R, uint4 *O, int S,
                            int k, int V) {
    if (V > 2 * kWave)
        decode_dispatch_nv<BF16, 4>(unit, res, grid, st, Y, gates, idx, loc, cap, R, O, S, k, V);
    else
        decode_dispatch_nv<BF16, 2>(unit, res, grid, st, Y, gates, idx, loc, cap, R, O, S, k, V);
}

hipError_t launch_decode(const moe_shape &s, const void *y, const float *gates, const int32_t *idx,
                         const int32_t *loc, const int32_t *cap, void *out, bool unit_gates, hipStream_t st,
                         const void *yres) {
    if (s.S == 0) return hipSuccess;
    const int eb = s.dtype == MOE_DT_BF16 ? 2 : 4;
    const int V = s.M * eb / 16;
    const int grid = grid_for(s.S);
    auto Y = static_cast<const uint4 *>(y);
    auto R = static_cast<const uint4 *>(yres);
    auto O = static_cast<uint4 *>(out);
    const bool res = yres != nullptr;
    if (s.dtype == MOE_DT_BF16)
        decode_dispatch<true>(unit_gates, res, grid, st, Y, gates, idx, loc, cap, R, O, s.S, s.k, V);
    else
        decode_dispatch<false>(unit_gates, res, grid, st, Y, gates, idx, loc, cap, R, O, s.S, s.k, V);
    return hipGetLastError();
}

// ---------------------------------------------------------------- Residual-MoE dense branch

// The grouped GEMMs read an expert's row count and the capacity from device
// memory; the dense branch is one "expert" whose rows are all S tokens (the
// capacity, a row stride only, is kept at least 1).
__global__ void set_dense_rows_kernel(int32_t *rows, int S) {
    if (threadIdx.x == 0) {
        rows[0] = S;             // fill[0]
        rows[1] = S > 0 ? S : 1;  // capacity
    }
}

hipError_t launch_residual_ffn(const moe_shape &s, const void *x, const void *W1r, const void *b1r, const void *W2r,
                               const void *b2r, void *pre_r, void *h_r, void *y_r, int32_t *dense_rows,
                               hipStream_t st) {
    if (s.S == 0) return hipSuccess;
    hipLaunchKernelGGL(set_dense_rows_kernel, dim3(1), dim3(64), 0, st, dense_rows, s.S);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    moe_shape d = s;
    d.E = 1;
    if ((err = launch_fc1(d, x, W1r, b1r, dense_rows, dense_rows + 1, pre_r, h_r, s.S, st)) != hipSuccess)
        return err;
    return launch_fc2(d, h_r, W2r, b2r, dense_rows, dense_rows + 1, y_r, s.S, st);
}

// The dense branch's backward: the expert FFN backward's four products with the
// branch as one expert over all S rows (dy = dout, buf = x). With S = 0 the
// weight-gradient products still run, over no rows, and write zeros.
hipError_t launch_residual_bwd(const moe_shape &s, const void *dout, const void *x, const void *pre_r,
                               const void *h_r, const void *W1r, const void *W2r, void *dpre_r, void *dx_r,
                               float *dW1r, float *db1r, float *dW2r, float *db2r, int32_t *dense_rows,
                               hipStream_t st) {
    hipLaunchKernelGGL(set_dense_rows_kernel, dim3(1), dim3(64), 0, st, dense_rows, s.S);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    moe_shape d = s;
    d.E = 1;
    return launch_expert_ffn_bwd(d, x, pre_r, h_r, W1r, W2r, dense_rows, dense_rows + 1, dout,
                                 dpre_r, dx_r, dW1r, db1r, dW2r, db2r, s.S > 0 ? s.S : 1, st);
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
