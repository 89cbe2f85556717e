// Routing on gfx950: softmax top-k gate, ordered per-expert slot count, capacity.
//
// The pages (MoE training blog, part 1 section 1.4 "kernel optimisation", and
// part 3 section 3.5) describe one fused top-k + cumsum (Blelloch scan) +
// scatter kernel. Here the work is split in three short launches so that the
// location of every route is exact and deterministic without atomics deciding
// order:
//   phase 1 (topk):   one group of G lanes per token keeps the token's E logits
//                     in registers, selects the k largest with k group-wide
//                     max-reductions of a 64-bit (logit, index) key, computes
//                     the fp64 softmax, and counts routes per (route rank,
//                     expert) for its 64-token tile in LDS;
//   phase 2 (scan):   one workgroup per expert scans that expert's tile counts
//                     in (route rank, tile) order: the exclusive prefix is the
//                     first location of each tile, the total is needed[e];
//   phase 3 (assign): one wavefront per (route rank, tile); a lane per token
//                     ranks itself among lanes with the same expert using nine
//                     ballots (a match over the expert id's bits), adds the
//                     tile's offset, and compares with C, which every
//                     workgroup derives from needed[] and capacity_factor.
// The fused layer forward runs phase 3 inside the encode launch instead
// (assign_encode_kernel: the same ranks and offsets, one wavefront per token),
// so routing and encode there take three launches, not four. In moe_route, when
// the count table is small (E * k * tiles <= kScanInBlock) phase 2 moves into
// phase 3's launch: each of its workgroups scans the raw counts in LDS
// (block_scan_counts), and routing takes two launches.
#include "moe_internal.h"

namespace moe {

// Total order on fp32 as unsigned integers (finite inputs), with -0 == +0.
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_order_key(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Larger logit wins; among equal logits the lower expert index wins.
__device__ __forceinline__ uint64_t route_key(float logit, int e) {
    return (static_cast<uint64_t>(order_key(logit)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) {
        const uint64_t o = __shfl_xor(v, off, G);
        v = o > v ? o : v;
    }
    return v;
}

template <int G>
__device__ __forceinline__ double group_sum_f64(double v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, G);
    return v;
}

// Phase 1. Block = one 64-token tile, NT = 64 * G threads up to 1024 (every token's
// group at once when G <= 16); G lanes per token, EPL experts per lane (expert
// e = lane_in_group + G * j). counts is [E][k][nblk].
template <int G>
constexpr int topk_threads() {
    return kRouteTile * G < 256 ? 256 : (kRouteTile * G > 1024 ? 1024 : kRouteTile * G);
}

template <int G, int EPL>
__global__ __launch_bounds__(topk_threads<G>()) void route_topk_kernel(const float *__restrict__ logits, int S,
                                                                       int E, int k, int nblk,
                                                                       int32_t *__restrict__ idx,
                                                                       float *__restrict__ gates,
                                                                       int32_t *__restrict__ counts) {
    constexpr int NT = topk_threads<G>();
    extern __shared__ int32_t tile_count[];  // [k][E]
    const int tid = threadIdx.x;
    const int tile = blockIdx.x;
    for (int i = tid; i < k * E; i += NT) tile_count[i] = 0;
    __syncthreads();

    const int gl = tid % G;
    constexpr int groups = NT / G;
    for (int t = tid / G; t < kRouteTile; t += groups) {
        const int s = tile * kRouteTile + t;
        if (s >= S) break;  // uniform across the G lanes of a group
        const float *row = logits + static_cast<int64_t>(s) * E;
        float v[EPL];
        uint64_t key[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = gl + G * j;
            v[j] = e < E ? row[e] : 0.f;
            key[j] = e < E ? route_key(v[j], e) : 0ull;  // a real key is never 0
        }
        int my_e = 0;
        float my_l = 0.f, top = 0.f;
        for (int r = 0; r < k; ++r) {
            uint64_t best = key[0];
#pragma unroll
            for (int j = 1; j < EPL; ++j) best = key[j] > best ? key[j] : best;
            best = group_max_u64<G>(best);
            const float l = from_order_key(static_cast<uint32_t>(best >> 32));
            if (r == 0) top = l;
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                if (key[j] == best) key[j] = 0ull;
            if (gl == r) {
                my_e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
                my_l = l;
            }
        }
        // Softmax over all E logits in fp64; `top` is the largest logit.
        double sum = 0.0;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (gl + G * j < E) sum += exp(static_cast<double>(v[j]) - static_cast<double>(top));
        sum = group_sum_f64<G>(sum);
        if (gl < k) {
            const int64_t q = static_cast<int64_t>(gl) * S + s;
            idx[q] = my_e;
            gates[q] = static_cast<float>(exp(static_cast<double>(my_l) - static_cast<double>(top)) / sum);
            atomicAdd(&tile_count[gl * E + my_e], 1);  // integer counts: order-free
        }
    }
    __syncthreads();
    for (int i = tid; i < k * E; i += NT) {
        const int r = i / E, e = i - r * E;
        counts[(static_cast<int64_t>(e) * k + r) * nblk + tile] = tile_count[i];
    }
}

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ __forceinline__ int block_exclusive_scan(int v, int *total, int *sh) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int inc = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(inc, off, 64);
        if (lane >= off) inc += o;
    }
    if (lane == 63) sh[w] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        base += i < w ? sh[i] : 0;
        tot += sh[i];
    }
    *total = tot;
    return base + inc - v;
}

// Phase 2. One block per expert: counts[e] (k*nblk entries, route-major then
// tile order) becomes its exclusive prefix; needed[e] is the total.
__global__ __launch_bounds__(256) void route_scan_kernel(int32_t *__restrict__ counts, int L,
                                                         int32_t *__restrict__ needed) {
    __shared__ int sh[4];
    int32_t *c = counts + static_cast<int64_t>(blockIdx.x) * L;
    const int per = (L + 255) / 256;
    const int b = threadIdx.x * per, e = min(L, b + per);
    int local = 0;
    for (int i = b; i < e; ++i) local += c[i];
    int total;
    int run = block_exclusive_scan(local, &total, sh);
    for (int i = b; i < e; ++i) {
        const int v = c[i];
        c[i] = run;
        run += v;
    }
    if (threadIdx.x == 0) needed[blockIdx.x] = total;
}

// Phase 3. Four (route rank, tile) wavefronts per block. mode: +1 fixed factor,
// 0 max needed, -1 min(factor bound, max needed); cap_by_factor is
// ceil(k*S*|f|/E) computed on the host. SCAN: offsets holds phase 1's raw counts,
// which every block scans in LDS (phase 2 folded in); block 0 writes needed.
template <bool SCAN>
__global__ __launch_bounds__(256) void route_assign_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ offsets, int32_t *__restrict__ needed,
    int S, int E, int k, int nblk, int ebits, int mode, int64_t cap_by_factor, int32_t *__restrict__ loc,
    int32_t *__restrict__ fill, int32_t *__restrict__ cap_out, int32_t *__restrict__ slot_route) {
    __shared__ int sh[4];
    extern __shared__ int32_t scan_lds[];  // SCAN: offsets [E*k*nblk], then needed [E]
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int32_t *offs = offsets, *need = needed;
    if constexpr (SCAN) {
        int32_t *o = scan_lds, *nd = scan_lds + E * k * nblk;
        block_scan_counts(offsets, E, k * nblk, o, nd);
        if (blockIdx.x == 0)
            for (int e = tid; e < E; e += 256) needed[e] = nd[e];
        offs = o;
        need = nd;
    }
    const int C = block_capacity(need, E, mode, cap_by_factor, sh);
    if (blockIdx.x == 0) {
        if (tid == 0) cap_out[0] = C;
        for (int e = tid; e < E; e += 256) fill[e] = min(need[e], C);
    }
    const int w = blockIdx.x * 4 + wv;
    if (w >= k * nblk) return;
    const int r = w / nblk, b = w - r * nblk;
    const int s = b * kRouteTile + lane;
    const bool active = s < S;
    const int e = active ? idx[static_cast<int64_t>(r) * S + s] : 0;
    uint64_t same = __ballot(active);
    for (int bit = 0; bit < ebits; ++bit) {
        const bool one = (e >> bit) & 1;
        const uint64_t ones = __ballot(active && one);
        same &= one ? ones : ~ones;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(same & below);
    if (active) {
        const int64_t q = static_cast<int64_t>(r) * S + s;
        const int l = offs[(static_cast<int64_t>(e) * k + r) * nblk + b] + rank;
        loc[q] = l;
        if (slot_route != nullptr && l < C) slot_route[static_cast<int64_t>(e) * C + l] = static_cast<int32_t>(q);
    }
}

template <int G, int EPL>
static hipError_t launch_topk(const float *logits, int S, int E, int k, int nblk, int32_t *idx, float *gates,
                              int32_t *counts, hipStream_t st) {
    const size_t lds = sizeof(int32_t) * static_cast<size_t>(k) * E;
    hipLaunchKernelGGL((route_topk_kernel<G, EPL>), dim3(nblk), dim3(topk_threads<G>()), lds, st, logits, S, E, k,
                       nblk, idx, gates, counts);
    return hipGetLastError();
}

hipError_t launch_route_counts(const moe_shape &s, const float *logits, int32_t *idx, float *gates,
                               int32_t *needed, RouteWs ws, hipStream_t st, bool scan) {
    const int S = s.S, E = s.E, k = s.k, nblk = ws.nblk;
    hipError_t err = hipSuccess;
    if (nblk > 0) {
        if (E <= 64) {
            int G = 1;
            while (G < E) G <<= 1;
            switch (G) {
                case 1: err = launch_topk<1, 1>(logits, S, E, k, nblk, idx, gates, ws.counts, st); break;
                case 2: err = launch_topk<2, 1>(logits, S, E, k, nblk, idx, gates, ws.counts, st); break;
                case 4: err = launch_topk<4, 1>(logits, S, E, k, nblk, idx, gates, ws.counts, st); break;
                case 8: err = launch_topk<8, 1>(logits, S, E, k, nblk, idx, gates, ws.counts, st); break;
                case 16: err = launch_topk<16, 1>(logits, S, E, k, nblk, idx, gates, ws.counts, st); break;
                case 32: err = launch_topk<32, 1>(logits, S, E, k, nblk, idx, gates, ws.counts, st); break;
                default: err = launch_topk<64, 1>(logits, S, E, k, nblk, idx, gates, ws.counts, st); break;
            }
        } else if (E <= 128) {
            err = launch_topk<64, 2>(logits, S, E, k, nblk, idx, gates, ws.counts, st);
        } else if (E <= 256) {
            err = launch_topk<64, 4>(logits, S, E, k, nblk, idx, gates, ws.counts, st);
        } else {
            err = launch_topk<64, 8>(logits, S, E, k, nblk, idx, gates, ws.counts, st);
        }
        if (err != hipSuccess) return err;
    }
    const int L = k * nblk;
    if (scan) hipLaunchKernelGGL(route_scan_kernel, dim3(E), dim3(256), 0, st, ws.counts, L, needed);
    return hipGetLastError();
}

hipError_t launch_route(const moe_shape &s, const float *logits, int32_t *idx, int32_t *loc, float *gates,
                        int32_t *needed, int32_t *fill, int32_t *cap, int32_t *slot_route, RouteWs ws,
                        int64_t cap_by_factor, hipStream_t st) {
    const int S = s.S, E = s.E, k = s.k, nblk = ws.nblk;
    const bool fold = scan_in_assign(E, k, nblk);  // the assignment scans the counts itself
    hipError_t err = launch_route_counts(s, logits, idx, gates, needed, ws, st, !fold);
    if (err != hipSuccess) return err;
    const int L = k * nblk;
    int ebits = 0;
    while ((1 << ebits) < E) ++ebits;
    const int mode = capacity_mode(s);
    const int blocks = L > 0 ? (L + 3) / 4 : 1;
    if (fold) {
        const size_t lds = sizeof(int32_t) * (static_cast<size_t>(E) * L + E);
        hipLaunchKernelGGL(route_assign_kernel<true>, dim3(blocks), dim3(256), lds, st, idx, ws.counts, needed, S, E,
                           k, nblk, ebits, mode, cap_by_factor, loc, fill, cap, slot_route);
    } else {
        hipLaunchKernelGGL(route_assign_kernel<false>, dim3(blocks), dim3(256), 0, st, idx, ws.counts, needed, S, E,
                           k, nblk, ebits, mode, cap_by_factor, loc, fill, cap, slot_route);
    }
    return hipGetLastError();
}

}  // namespace moe
