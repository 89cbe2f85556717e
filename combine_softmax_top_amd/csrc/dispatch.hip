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

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
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
    const int64_t rows = static_cast<int64_t>(E) * C;
    for (int64_t row = global_wave(); row < rows; row += nw) {
        const int e = static_cast<int>(row / C);
        const int j = static_cast<int>(row - static_cast<int64_t>(e) * C);
        if (j < fill[e]) continue;
        uint4 *dst = buf + row * V;
        for (int v = lane; v < V; v += kWave) dst[v] = zero;
    }
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
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    const int64_t rows = static_cast<int64_t>(E) * C;
    for (int64_t row = global_wave(); row < rows; row += nw) {
        const int e = static_cast<int>(row / C);
        const int j = static_cast<int>(row - static_cast<int64_t>(e) * C);
        if (j < min(needed[e], C)) continue;
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
// skipped (encode backward: dx = sum of dbuf rows). RES: Residual-MoE, the
// dense branch's row yres[s] is added after the routes, before the rounding.
template <bool BF16, bool UNIT, bool RES>
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
        // four vectors per lane at a time (v, v + 64, ...): the loads of a batch
        // of routes for all four are in flight together; each output still sums
        // its routes in route order
        constexpr int NV = 4;
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

// logits[s][e] = fp32(sum_m x[s][m] * Wg[m][e]), the sum in fp64 in a fixed
// order: m is cut into n chunks of L = 64 * ceil(M / 4096) (n <= 64, the last
// may be shorter), each chunk is summed from 0 in increasing m, and the chunk
// sums are combined level by level, neighbours 2i and 2i+1 added, an unpaired
// last sum carried up; the root is rounded once to fp32. Each product of a
// bf16/fp32 input and an fp32 weight is exact in fp64, so fma(x, w, acc)
// rounds exactly like acc + x*w.
//
// A block takes a tile of TT tokens and ET experts. It stages in LDS the
// tile's x rows and the Wg columns of its experts, every load in flight at
// once, both cut into the summation chunks with a 16-byte pad per chunk so
// that lanes on different chunks read different banks. Lane (c, e, u) then
// runs the L-long chains of chunk c, expert e for tokens u, u + TS, ... (TPL of
// them, TS = 256 / (G * ET)) from LDS. The G = pow2ceil(n) lanes of a
// (token, expert) are consecutive, so the tree runs on shuffles: at stride s,
// lane c (a multiple of 2s) adds lane c + s when c + s < n -- the element at
// lane j * 2^l of level l exists iff j * 2^l < n, which is the level-by-level
// pairing above. Lanes c >= n hold empty chains that are never added.
// Division by a run-time invariant d >= 1 for 0 <= x < 2^31 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1,
// x / d = (mulhi(x, m) + x) >> s.
struct FastDiv {
    uint32_t d, m, s;
    __host__ static FastDiv make(uint32_t dv) {
        FastDiv f{dv, 0u, 0u};
        while ((1ull << f.s) < dv) ++f.s;
        f.m = static_cast<uint32_t>(((1ull << 32) * ((1ull << f.s) - dv)) / dv + 1);
        return f;
    }
    __device__ __forceinline__ int div(int x) const {
        const uint32_t hi = __umulhi(static_cast<uint32_t>(x), m);
        return static_cast<int>((static_cast<uint64_t>(hi) + static_cast<uint32_t>(x)) >> s);
    }
};

struct GateTile {
    FastDiv dne, dvpr, dvpc, dL, dLE4;  // by experts in the tile, x vectors per row / per chunk,
                                        // chunk length, float4s per chunk of all experts
    int L, n, G;     // chunk length, chunk count, lanes per (token, expert)
    int ET, TS, TPL; // experts per block, token lanes, tokens per lane
    int wpitch;      // floats per Wg chunk in LDS: L * ET + 4
    int xpitch;      // bytes per x chunk in LDS: L * esz + 16
    size_t lds;      // bytes
};

constexpr int kGateLdsMax = 160 * 1024;

__host__ GateTile gate_tile(int S, int M, int E, int esz) {
    GateTile t{};
    t.L = 64 * ((M + 4095) / 4096);
    t.n = (M + t.L - 1) / t.L;
    t.G = 1;
    while (t.G < t.n) t.G <<= 1;
    t.ET = std::min(E, 256 / t.G);
    t.wpitch = t.L * t.ET + 4;
    while (t.ET > 1 && static_cast<size_t>(t.n) * (t.L * t.ET + 4) * 4 > 64 * 1024) {
        --t.ET;
        t.wpitch = t.L * t.ET + 4;
    }
    t.TS = 256 / (t.G * t.ET);
    t.xpitch = t.L * esz + 16;
    const size_t wbytes = static_cast<size_t>(t.n) * t.wpitch * 4;
    const size_t xrow = static_cast<size_t>(t.n) * t.xpitch;
    // tokens per lane: up to 8 while the LDS tiles fit and the grid keeps at
    // least two blocks per CU (512) along the tokens
    t.TPL = 1;
    while (t.TPL < 8 && wbytes + xrow * t.TS * (t.TPL * 2) <= static_cast<size_t>(kGateLdsMax) &&
           (S + t.TS * t.TPL * 2 - 1) / (t.TS * t.TPL * 2) >= 512)
        t.TPL *= 2;
    t.lds = wbytes + xrow * t.TS * t.TPL;
    t.dne = FastDiv::make(static_cast<uint32_t>(t.ET));
    t.dvpr = FastDiv::make(static_cast<uint32_t>(M / (16 / esz)));
    t.dvpc = FastDiv::make(static_cast<uint32_t>(t.L / (16 / esz)));
    t.dL = FastDiv::make(static_cast<uint32_t>(t.L));
    t.dLE4 = FastDiv::make(static_cast<uint32_t>(t.L * E / 4));
    return t;
}

// The eight loaded values of a staging batch pass through one empty asm
// statement, so every load of the batch is issued (and waited for once) before
// the first of the conditional LDS stores that consume them. Without it the
// compiler sinks each load into its store's branch (the inputs are read-only,
// so nothing pins the loads), and the batch costs one memory round trip per load.
typedef float gate_f4 __attribute__((ext_vector_type(4)));
typedef uint32_t gate_u4 __attribute__((ext_vector_type(4)));
template <class V>
__device__ __forceinline__ void issue_together(V (&r)[8]) {
    asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]), "+v"(r[4]), "+v"(r[5]), "+v"(r[6]),
                 "+v"(r[7]));
}

template <bool BF16, int TPL>
__global__ __launch_bounds__(kThreads) void gate_project_kernel(const void *__restrict__ xv,
                                                                const float *__restrict__ Wg,
                                                                float *__restrict__ logits, int S, int M, int E,
                                                                GateTile tl) {
    extern __shared__ __align__(16) unsigned char gsm[];
    constexpr int ESZ = BF16 ? 2 : 4;
    constexpr int EPV = 16 / ESZ;  // x elements per 16-byte vector
    const int L = tl.L, n = tl.n, G = tl.G, ET = tl.ET, TS = tl.TS;
    const int TT = TS * TPL;
    float *wl = reinterpret_cast<float *>(gsm);
    unsigned char *xl = gsm + static_cast<size_t>(n) * tl.wpitch * 4;
    const int tid = threadIdx.x;
    const int64_t s0 = static_cast<int64_t>(blockIdx.x) * TT;
    const int e0 = blockIdx.y * ET;
    const int ne = min(ET, E - e0);
    const int nt = static_cast<int>(min<int64_t>(TT, S - s0));

    // stage Wg[m][e0 .. e0+ne) at wl[c * wpitch + (m - c*L) * ET + (e - e0)]
    // (the tile's last expert block may hold ne < ET experts: its divisor is
    // ne, not the one precomputed for ET)
    if (ET == E) {
        // every expert: Wg is M*E contiguous floats; a chunk's L*E of them are
        // contiguous in LDS too (L*E is a multiple of 4)
        const int total4 = M * E / 4;
        const gate_f4 *w4 = reinterpret_cast<const gate_f4 *>(Wg);
        for (int i0 = tid; i0 < total4; i0 += 8 * kThreads) {
            gate_f4 r[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = min(i0 + u * kThreads, total4 - 1);
                const int c = tl.dLE4.div(i);
                r[u] = w4[i];
                dst[u] = c * tl.wpitch + (i - c * (L * E / 4)) * 4;
            }
            issue_together(r);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u * kThreads < total4) *reinterpret_cast<gate_f4 *>(wl + dst[u]) = r[u];
        }
    } else {
        const FastDiv dne = ne == ET ? tl.dne : FastDiv{static_cast<uint32_t>(ne), 0u, 0u};
        const bool fast = ne == ET;
        const int total = M * ne;
        for (int i0 = tid; i0 < total; i0 += 8 * kThreads) {
            float r[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = min(i0 + u * kThreads, total - 1);
                const int m = fast ? dne.div(i) : i / ne, e = i - m * ne, c = tl.dL.div(m);
                r[u] = Wg[static_cast<int64_t>(m) * E + e0 + e];
                dst[u] = c * tl.wpitch + (m - c * L) * ET + e;
            }
            issue_together(r);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u * kThreads < total) wl[dst[u]] = r[u];
        }
    }
    // stage x rows s0 .. s0+nt, 16-byte vectors, at xl[(t * n + c) * xpitch + (m - c*L) * ESZ]
    {
        const int vpr = M / EPV;  // vectors per row
        const int vpc = L / EPV;  // vectors per chunk
        const int total = nt * vpr;
        const gate_u4 *xg = reinterpret_cast<const gate_u4 *>(xv);
        for (int i0 = tid; i0 < total; i0 += 8 * kThreads) {
            gate_u4 r[8];
            int dst[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = min(i0 + u * kThreads, total - 1);
                const int t = tl.dvpr.div(i), v = i - t * vpr, c = tl.dvpc.div(v);
                r[u] = xg[(s0 + t) * vpr + v];
                dst[u] = (t * n + c) * tl.xpitch + (v - c * vpc) * 16;
            }
            issue_together(r);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i0 + u * kThreads < total) *reinterpret_cast<gate_u4 *>(xl + dst[u]) = r[u];
        }
    }
    __syncthreads();

    const int c = tid & (G - 1);
    const int el = (tid / G) % ET;
    const int u = tid / (G * ET);
    const bool live = u < TS && el < ne;
    const int m0 = c * L, len = max(0, min(M, m0 + L) - m0);
    double acc[TPL];
#pragma unroll
    for (int j = 0; j < TPL; ++j) acc[j] = 0.0;
    if (live) {
        const float *wc = wl + c * tl.wpitch + el;
        const unsigned char *xc[TPL];
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const int t = min(u + j * TS, nt - 1);  // tokens past the tile re-read the last one, never stored
            xc[j] = xl + static_cast<size_t>(t * n + c) * tl.xpitch;
        }
        for (int i = 0; i < len; i += EPV) {
            // all reads of the step first, then the TPL independent chains
            // interleaved (each chain still takes its products in increasing m)
            double w[EPV];
#pragma unroll
            for (int q = 0; q < EPV; ++q) w[q] = static_cast<double>(wc[(i + q) * ET]);
            uint4 xv4[TPL];
#pragma unroll
            for (int j = 0; j < TPL; ++j) xv4[j] = *reinterpret_cast<const uint4 *>(xc[j] + i * ESZ);
#pragma unroll
            for (int q = 0; q < EPV; ++q) {
#pragma unroll
                for (int j = 0; j < TPL; ++j) {
                    const uint32_t word = q / (EPV / 4) == 0 ? xv4[j].x
                                        : q / (EPV / 4) == 1 ? xv4[j].y
                                        : q / (EPV / 4) == 2 ? xv4[j].z : xv4[j].w;
                    float xf;
                    if (BF16) xf = __uint_as_float((q & 1) ? (word & 0xFFFF0000u) : (word << 16));
                    else xf = __uint_as_float(word);
                    acc[j] = fma(static_cast<double>(xf), w[q], acc[j]);
                }
            }
        }
    }
    for (int st = 1; st < G; st <<= 1) {
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const double o = __shfl_down(acc[j], st, 64);
            if ((c & (2 * st - 1)) == 0 && c + st < n) acc[j] += o;
        }
    }
    if (live && c == 0) {
#pragma unroll
        for (int j = 0; j < TPL; ++j) {
            const int t = u + j * TS;
            if (t < nt) logits[(s0 + t) * E + e0 + el] = static_cast<float>(acc[j]);
        }
    }
}

int grid_for(int64_t waves) {
    // enough waves to cover the work, capped at 32 waves per CU on 256 CUs
    const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    return static_cast<int>(blocks < 1 ? 1 : (blocks > 2048 ? 2048 : blocks));
}

}  // namespace

template <bool BF16, int TPL>
static hipError_t gate_launch(const moe_shape &s, const void *x, const float *Wg, float *logits, const GateTile &t,
                              hipStream_t st) {
    auto k = gate_project_kernel<BF16, TPL>;
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGateLdsMax);
    if (attr != hipSuccess) return attr;
    const int TT = t.TS * TPL;
    const dim3 grid((s.S + TT - 1) / TT, (s.E + t.ET - 1) / t.ET);
    hipLaunchKernelGGL(k, grid, dim3(kThreads), t.lds, st, x, Wg, logits, s.S, s.M, s.E, t);
    return hipGetLastError();
}

template <bool BF16>
static hipError_t gate_dispatch(const moe_shape &s, const void *x, const float *Wg, float *logits, hipStream_t st) {
    const GateTile t = gate_tile(s.S, s.M, s.E, BF16 ? 2 : 4);
    if (t.lds > static_cast<size_t>(kGateLdsMax)) return hipErrorInvalidValue;
    switch (t.TPL) {
    case 8: return gate_launch<BF16, 8>(s, x, Wg, logits, t, st);
    case 4: return gate_launch<BF16, 4>(s, x, Wg, logits, t, st);
    case 2: return gate_launch<BF16, 2>(s, x, Wg, logits, t, st);
    default: return gate_launch<BF16, 1>(s, x, Wg, logits, t, st);
    }
}

bool gate_supported(int M, int E, int dtype) {
    // the token count only lowers tokens per lane, never below the one-token tile checked here
    return gate_tile(0, M, E, dtype == MOE_DT_BF16 ? 2 : 4).lds <= static_cast<size_t>(kGateLdsMax);
}

hipError_t launch_gate_project(const moe_shape &s, const void *x, const float *Wg, float *logits, hipStream_t st) {
    if (s.S == 0) return hipSuccess;
    return s.dtype == MOE_DT_BF16 ? gate_dispatch<true>(s, x, Wg, logits, st)
                                  : gate_dispatch<false>(s, x, Wg, logits, st);
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

hipError_t launch_assign_encode(const moe_shape &s, const void *x, const int32_t *idx, RouteWs ws,
                                const int32_t *needed, int64_t cap_by_factor, int32_t *loc, int32_t *fill,
                                int32_t *cap, int32_t *slot_route, void *buf, int32_t cmax, hipStream_t st) {
    const int eb = s.dtype == MOE_DT_BF16 ? 2 : 4;
    const int V = s.M * eb / 16;
    const int grid = grid_for(static_cast<int64_t>(s.S) + static_cast<int64_t>(s.E) * cmax);
    hipLaunchKernelGGL(assign_encode_kernel, dim3(grid), dim3(kThreads), 0, st, static_cast<const uint4 *>(x), idx,
                       ws.counts, needed, s.S, s.E, s.k, ws.nblk, capacity_mode(s), cap_by_factor, loc, fill, cap,
                       slot_route, static_cast<uint4 *>(buf), V);
    return hipGetLastError();
}

template <bool BF16>
static void decode_dispatch(bool unit, bool res, int grid, hipStream_t st, const uint4 *Y, const float *gates,
                            const int32_t *idx, const int32_t *loc, const int32_t *cap, const uint4 *R, uint4 *O, int S,
                            int k, int V) {
    if (unit)
        hipLaunchKernelGGL((gather_sum_kernel<BF16, true, false>), dim3(grid), dim3(kThreads), 0, st, Y, gates, idx,
                           loc, cap, R, O, S, k, V);
    else if (res)
        hipLaunchKernelGGL((gather_sum_kernel<BF16, false, true>), dim3(grid), dim3(kThreads), 0, st, Y, gates, idx,
                           loc, cap, R, O, S, k, V);
    else
        hipLaunchKernelGGL((gather_sum_kernel<BF16, false, false>), dim3(grid), dim3(kThreads), 0, st, Y, gates, idx,
                           loc, cap, R, O, S, k, V);
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
// memory; the dense branch is one "expert" whose rows are all S tokens.
__global__ void set_dense_rows_kernel(int32_t *rows, int S) {
    if (threadIdx.x == 0) {
        rows[0] = S;  // fill[0]
        rows[1] = S;  // capacity
    }
}

hipError_t launch_residual_ffn(const moe_shape &s, const void *x, const void *W1r, const void *b1r, const void *W2r,
                               const void *b2r, void *h_r, void *y_r, int32_t *dense_rows, hipStream_t st) {
    if (s.S == 0) return hipSuccess;
    hipLaunchKernelGGL(set_dense_rows_kernel, dim3(1), dim3(64), 0, st, dense_rows, s.S);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    moe_shape d = s;
    d.E = 1;
    if ((err = launch_fc1(d, x, W1r, b1r, dense_rows, dense_rows + 1, nullptr, h_r, s.S, st)) != hipSuccess)
        return err;
    return launch_fc2(d, h_r, W2r, b2r, dense_rows, dense_rows + 1, y_r, s.S, st);
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
