// Expert FFN on gfx950: grouped GEMMs over the experts' filled slots.
//
// The blog (part 3 section 3.5, Flexible All-to-All) keeps each expert's
// tokens contiguous as [E, C, M] so that the experts run as a batched matrix
// multiply whose shape does not depend on the GPU count. Here every expert e
// owns rows [e*C, e*C + fill[e]) of the flat buffer, and two kernel families
// cover the forward and backward products:
//
//  rows-grouped:  D[e*C + i][n] = sum_k A[e*C + i][k] * B_e(k, n),  i < fill[e]
//                 (fc1, fc2, and the backward data products dh, dbuf); A is
//                 k-contiguous; B_e is [N][K] (forward, nn.Linear weights) or
//                 [K][N] (backward, the same weights read transposed);
//  K-grouped:     D_e[i][n] = sum_{j < fill[e]} A[e*C + j][i] * B[e*C + j][n]
//                 (weight gradients dW2 = dy^T h, dW1 = dpre^T buf), fp32, with
//                 the column sums of A (bias gradients) taken on the way.
//
// bf16 kernels: 128x128 output tile per 256-thread workgroup, four wavefronts
// of 64x64, each a 2x2 grid of v_mfma_f32_32x32x16_bf16 (fp32 accumulation);
// K steps of 64 staged through LDS in two buffers (the next step's global
// loads are in flight while the current step is multiplied); the LDS tile is
// [rows][64] with 16-byte chunks XOR-swizzled by row so that the fragment
// reads (8 consecutive k of one row per lane) are bank-conflict free.
// Operands that are k-strided in memory (MN-major) are transposed while being
// written to LDS. Results are staged through LDS so that bias, activation and
// stores run on 16-byte row chunks. Row tiles past fill[e] exit at once.
// fp32 (MOE_DT_F32) uses a plain LDS-tiled SIMT kernel with the same maths.
#include <cstdlib>

#include <algorithm>

#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 128, BN = 128, BK = 64, NT = 256;
constexpr int kTileElems = 128 * BK;  // one operand tile, bf16 elements

enum Epi { EPI_FC1 = 0, EPI_FC2 = 1, EPI_DACT = 2, EPI_PLAIN = 3 };

__device__ __forceinline__ int swz(int row, int k) { return row * BK + ((((k >> 3) ^ (row & 7))) << 3) + (k & 7); }

// A 128-row tile whose rows are k-contiguous in memory: 16-byte chunks copied
// as they are (4 per thread).
struct KMajorTile {
    uint4 r[4];
    __device__ __forceinline__ void load(const bf16_t *base, int64_t ld, int rows_valid, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + NT * i, row = c >> 3, kc = c & 7;
            r[i] = row < rows_valid ? *reinterpret_cast<const uint4 *>(base + static_cast<int64_t>(row) * ld + k0 + kc * 8)
                                    : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ __forceinline__ void store(bf16_t *s, int tid) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + NT * i, row = c >> 3, kc = c & 7;
            *reinterpret_cast<uint4 *>(s + row * BK + ((kc ^ (row & 7)) << 3)) = r[i];
        }
    }
};

// A 128-column tile stored k-major in memory ([K][ld], the 128 columns
// contiguous): each thread loads 8 columns of one k and writes them to LDS
// transposed (one lane per k in a wavefront, so the 2-byte LDS writes of a
// wavefront cover 64 distinct k of one row).
struct MNMajorTile {
    uint4 r[4];
    __device__ __forceinline__ void load(const bf16_t *base, int64_t ld, int mn_valid, int k_valid, int k0, int tid) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + NT * i, kk = c & 63, mc = c >> 6;
            const bool ok = (k0 + kk < k_valid) && (mc * 8 < mn_valid);
            r[i] = ok ? *reinterpret_cast<const uint4 *>(base + static_cast<int64_t>(k0 + kk) * ld + mc * 8)
                      : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    __device__ __forceinline__ void store(bf16_t *s, int tid) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = tid + NT * i, kk = c & 63, mc = c >> 6;
            const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const bf16_t v = static_cast<bf16_t>((jj & 1) ? (w[jj >> 1] >> 16) : (w[jj >> 1] & 0xFFFFu));
                s[swz(mc * 8 + jj, kk)] = v;
            }
        }
    }
};

// One K step of 64 on the LDS tiles: each wavefront multiplies its 64x64 block.
__device__ __forceinline__ void mma_step(const bf16_t *sA, const bf16_t *sB, f32x16 (&acc)[2][2], int wm, int wn,
                                         int lane) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8 a[2], b[2];
        const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int row = wm * 64 + i * 32 + (lane & 31);
            a[i] = *reinterpret_cast<const bf16x8 *>(sA + row * BK + ((chunk ^ (row & 7)) << 3));
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int col = wn * 64 + j * 32 + (lane & 31);
            b[j] = *reinterpret_cast<const bf16x8 *>(sB + col * BK + ((chunk ^ (col & 7)) << 3));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
}

// Accumulators -> LDS as fp32 [wave][64][64]. Output element (row, col) of a
// 32x32 block sits in lane (col + 32 * ((row / 4) % 2)), register
// 4 * (row / 8) + row % 4.
__device__ __forceinline__ void stage_acc(float *st, const f32x16 (&acc)[2][2], int lane) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                const int col = j * 32 + (lane & 31);
                st[row * 64 + col] = acc[i][j][v];
            }
}

__device__ __forceinline__ void load8_bf16(const bf16_t *p, float *f) {
    const uint4 u = *reinterpret_cast<const uint4 *>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __uint_as_float(w[i] << 16);
        f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void store8_bf16(bf16_t *p, const float *f) {
    *reinterpret_cast<uint4 *>(p) =
        make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

// ------------------------------------------------------------------ rows-grouped bf16 GEMM

template <bool B_KMAJ, int EPI, int ACT>
__global__ __launch_bounds__(NT) void rows_gemm_bf16(const bf16_t *__restrict__ A, const bf16_t *__restrict__ B,
                                                     bf16_t *__restrict__ D, int N, int K,
                                                     const int32_t *__restrict__ fill, const int32_t *__restrict__ cap,
                                                     const bf16_t *__restrict__ bias, const bf16_t *__restrict__ aux,
                                                     bf16_t *__restrict__ pre_out) {
    __shared__ __align__(16) bf16_t smem[4 * kTileElems];  // 64 KiB: A,B x 2 buffers; reused for staging
    const int g = blockIdx.z;
    const int rows_g = fill[g];
    const int row0 = blockIdx.y * BM;
    if (row0 >= rows_g) return;
    const int C = *cap;
    const int col0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int rows_valid = min(BM, rows_g - row0);
    const int cols_valid = min(BN, N - col0);
    const int64_t grow0 = static_cast<int64_t>(g) * C + row0;  // first buffer row of this tile
    const bf16_t *Ab = A + grow0 * K;
    const bf16_t *Bb = B_KMAJ ? B + static_cast<int64_t>(g) * N * K + static_cast<int64_t>(col0) * K
                              : B + static_cast<int64_t>(g) * K * N + col0;
    // buffer b of operand A at smem + b * kTileElems, of operand B at smem + (2 + b) * kTileElems
#define SA(b) (smem + (b) * kTileElems)
#define SB(b) (smem + (2 + (b)) * kTileElems)

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    KMajorTile ta;
    typename std::conditional<B_KMAJ, KMajorTile, MNMajorTile>::type tb;
    const int nk = K / BK;
    ta.load(Ab, K, rows_valid, 0, tid);
    if constexpr (B_KMAJ) tb.load(Bb, K, cols_valid, 0, tid);
    else tb.load(Bb, N, cols_valid, K, 0, tid);
    ta.store(SA(0), tid);
    tb.store(SB(0), tid);
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < nk;
        if (more) {
            const int k0 = (t + 1) * BK;
            ta.load(Ab, K, rows_valid, k0, tid);
            if constexpr (B_KMAJ) tb.load(Bb, K, cols_valid, k0, tid);
            else tb.load(Bb, N, cols_valid, K, k0, tid);
        }
        mma_step(SA(cur), SB(cur), acc, wm, wn, lane);
        if (more) {
            ta.store(SA(cur ^ 1), tid);
            tb.store(SB(cur ^ 1), tid);
        }
        __syncthreads();
    }

    float *st = reinterpret_cast<float *>(smem) + wave * 64 * 64;
    stage_acc(st, acc, lane);
    __syncthreads();
#pragma unroll 2
    for (int i = 0; i < 8; ++i) {
        const int c = lane + 64 * i, r = c >> 3, cc = c & 7;
        const int trow = wm * 64 + r, tcol = wn * 64 + cc * 8;
        if (trow >= rows_valid || tcol >= cols_valid) continue;
        float v[8];
        const float4 lo = *reinterpret_cast<const float4 *>(st + r * 64 + cc * 8);
        const float4 hi = *reinterpret_cast<const float4 *>(st + r * 64 + cc * 8 + 4);
        v[0] = lo.x; v[1] = lo.y; v[2] = lo.z; v[3] = lo.w;
        v[4] = hi.x; v[5] = hi.y; v[6] = hi.z; v[7] = hi.w;
        const int64_t off = (grow0 + trow) * N + col0 + tcol;
        if constexpr (EPI == EPI_FC1 || EPI == EPI_FC2) {
            if (bias != nullptr) {
                float b[8];
                load8_bf16(bias + static_cast<int64_t>(g) * N + col0 + tcol, b);
#pragma unroll
                for (int u = 0; u < 8; ++u) v[u] += b[u];
            }
        }
        if constexpr (EPI == EPI_FC1) {
            if (pre_out != nullptr) store8_bf16(pre_out + off, v);
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = act_f<ACT>(v[u]);
        }
        if constexpr (EPI == EPI_DACT) {
            float p[8];
            load8_bf16(aux + off, p);
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] *= act_grad_f<ACT>(p[u]);
        }
        store8_bf16(D + off, v);
    }
}

// ------------------------------------------------------------------ rows-grouped bf16 GEMM, large tiles

// Forward products (A and B both k-contiguous) with BM x BN tiles (128 or 256
// each), NTH/64 wavefronts in a 2 x (NTH/128) grid, a two-stage LDS ring of
// 64-wide K steps filled by direct global->LDS 16-byte loads (no register
// staging), persistent workgroups walking an XCD-aware tile order. A
// wavefront's load writes 64 consecutive 16-byte LDS slots (8 rows of 64 k);
// each lane fetches the global chunk that belongs at its slot under the row
// XOR swizzle, so fragment reads are free of bank conflicts. Rows past the
// valid range are clamped to the last valid row: they only feed output rows
// or columns that are never stored.

typedef __attribute__((address_space(3))) void lds_void_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Direct global->LDS loads, 16 bytes per lane (lane l's chunk lands at LDS byte
// M0 + 16 l), issued from inline asm rather than through the compiler's
// builtins. After a builtin direct load the compiler cannot tell that a
// transposing LDS read (ds_read_b64_tr_b16) does not touch the LDS being
// filled, and makes that read wait for every outstanding vector-memory
// operation: the loads of the next ring stage, meant to stay in flight for a
// whole stage, were waited for at every K step of the products that read an
// operand n-contiguous (plain 16-byte LDS reads get no such wait). The kernels
// order every stage themselves (each wavefront waits for its own loads, then a
// workgroup barrier, before a stage is read), so the compiler need not see
// these loads. The LDS destination goes to M0; gfx9-family parts need one
// wait state between an M0 write and a direct load reading it (s_nop 0). Every
// direct load in this file goes through these two helpers, so no M0 value the
// compiler sets is live across them.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is a reserved register; the clobber is declared anyway
__device__ __forceinline__ uint32_t lds_m0(const void *lds_dst) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void_t *)lds_dst)));
}
// global_load_lds_dwordx4 from base (uniform) + voff_bytes (per lane)
__device__ __forceinline__ void dma16(const void *base, uint32_t voff_bytes, const void *lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_m0(lds_dst)), "v"(voff_bytes), "s"(base)
                 : "memory", "m0");
}
// global_load_lds_dword: 4 bytes per lane, lane l's word at LDS byte M0 + 4 l
__device__ __forceinline__ void dma4(const void *base, uint32_t voff_bytes, const void *lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(lds_m0(lds_dst)), "v"(voff_bytes), "s"(base)
                 : "memory", "m0");
}
// buffer_load_dwordx4 ... lds through a raw buffer resource (loads past its range return zero)
__device__ __forceinline__ void dma16_buf(i32x4_t rsrc, uint32_t voff_bytes, const void *lds_dst) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_m0(lds_dst)), "v"(voff_bytes), "s"(rsrc)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// 16-byte chunk slot of logical chunk c of row r in a tile whose rows hold KB
// bf16 (KB/8 chunks). The LDS serves 16 lanes of a 16-byte read per cycle over
// 64 four-byte banks (256 bytes, 16 chunk slots); row r starts at slot
// (r * KB/8) mod 16, so rows r and r + 16/(KB/8) start on the same slot. XOR-ing
// the chunk index with (r / (16/(KB/8))) mod (KB/8) spreads the 16 consecutive
// rows a fragment read touches (same logical chunk) over all 16 slots.
template <int KB>
__device__ __forceinline__ int swz_chunk(int row, int c) {
    constexpr int CPR = KB / 8, RPB = 16 / CPR;
    return c ^ ((row / RPB) & (CPR - 1));
}

template <int R, int KB, int NW>
__device__ __forceinline__ void dma_tile(const bf16_t *base, int64_t ld, int rows_valid, int k0, bf16_t *lds,
                                         int wave, int lane) {
    constexpr int CPR = KB / 8;          // chunks per row
    constexpr int RPI = 64 / CPR;        // rows per wavefront instruction
    static_assert(R % (NW * RPI) == 0, "tile rows must split evenly over the wavefronts");
#pragma unroll
    for (int j = 0; j < R / (NW * RPI); ++j) {
        const int rb = (j * NW + wave) * RPI;
        const int row = rb + lane / CPR;
        const int kc = swz_chunk<KB>(row, lane % CPR);  // the logical chunk stored at slot lane % CPR
        const int src_row = row < rows_valid ? row : rows_valid - 1;
        // uniform base + 32-bit lane offset (a tile spans well under 2^31 elements)
        const uint32_t off = static_cast<uint32_t>(src_row * static_cast<int>(ld) + kc * 8);
        dma16(base + k0, off * 2, lds + rb * KB);
    }
}

// A B tile stored n-contiguous in memory (B[k][n], as the weights are read by
// the backward data products): KB rows of k, each BN values of n. It lands in
// LDS as [KB][BN] with 16-byte chunk c of row k at slot c ^ 4(k mod 4). The
// transposing fragment reads below take a 4 (k) x 16 (n) block per 16 lanes;
// with this swizzle the 32 lanes of a half-wave touch each of the 64 banks once.
template <int BN, int KB, int NW>
__device__ __forceinline__ void dma_tile_mn(const bf16_t *base, int64_t ld, int cols_valid, int k0, bf16_t *lds,
                                            int wave, int lane) {
    constexpr int CPR = BN / 8;   // chunks per k row
    constexpr int RPI = 64 / CPR; // k rows per wavefront instruction
    static_assert(CPR >= 16 && KB % (NW * RPI) == 0, "n-contiguous tile shape");
#pragma unroll
    for (int j = 0; j < KB / (NW * RPI); ++j) {
        const int rb = (j * NW + wave) * RPI;
        const int row = rb + lane / CPR;
        const int c = min((lane % CPR) ^ (4 * (row & 3)), cols_valid / 8 - 1);  // chunk stored at this slot
        const uint32_t off = static_cast<uint32_t>(row * static_cast<int>(ld) + c * 8);
        dma16(base + static_cast<int64_t>(k0) * ld, off * 2, lds + rb * BN);
    }
}

typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef short v8s16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4s16 lds_v4s16_t;

// Weight fragments (the 32-row MFMA operand) of k slice kk from an n-contiguous
// tile. ds_read_b64_tr_b16 gives lane i of each 16-lane group, for q = 0..3,
// element (i mod 4) of the 8 bytes read by lane 4q + i/4 of the group; when
// that lane addresses (k0 + q', n0 + 4 (lane mod 4)) for q' = lane / 4, lane i
// receives column n0 + i at rows k0 .. k0+3. Two reads (k0 and k0 + 4) make the
// eight k values of the operand: lane l holds n = l mod 32 of the block and
// k = 8 (l / 32) .. +7 of the slice.
// The lane's offset (elements) in the tile for block j at kk = 0: k mod 4 is
// the same for every slice and both halves, so the other reads add constants.
template <int BN>
__device__ __forceinline__ int frag_b_mn_offset(int j, int wc0, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const int k = (g >> 1) * 8 + (i >> 2);
    const int n = wc0 + j * 32 + (g & 1) * 16 + 4 * (i & 3);
    return k * BN + (((n >> 3) ^ (4 * (k & 3))) << 3) + (n & 7);
}

template <int TN, int BN>
__device__ __forceinline__ void frag_b_mn(const bf16_t *sB, int kk, bf16x8 (&bx)[TN], int wc0, int lane) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const bf16_t *p = sB + frag_b_mn_offset<BN>(j, wc0, lane) + kk * 16 * BN;
        const v4s16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16_t *)p);
        const v4s16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16_t *)(p + 4 * BN));
        const v8s16 w = __builtin_shufflevector(r0, r1, 0, 1, 2, 3, 4, 5, 6, 7);
        bx[j] = __builtin_bit_cast(bf16x8, w);
    }
}

// s_waitcnt with only the vector-memory counter constrained (vmcnt <= N).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that leaves direct-to-LDS loads in flight. __syncthreads()
// is a release/acquire fence plus s_barrier, and the fence makes the compiler
// wait for every outstanding vector-memory operation (vmcnt(0)), which would
// drain the loads of later ring stages at every K step. Here each wavefront
// waits for its own loads of the stage about to be read (wait_vmcnt) before
// the barrier; the memory clobber keeps the compiler from moving LDS accesses
// across it. LDS reads of the stage being recycled have completed before the
// barrier because their fragments were consumed by MFMAs.
__device__ __forceinline__ void barrier_keep_loads() { asm volatile("s_barrier" ::: "memory"); }
// The same after this wavefront's outstanding LDS reads have completed, for a
// barrier after which other wavefronts overwrite the LDS just read.
__device__ __forceinline__ void barrier_keep_loads_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Fragments of one 16-wide k slice (kk) of the LDS tiles. The MFMA operands
// are swapped: the weight (output-feature) fragment is the 32-row operand and
// the token fragment the 32-column one, so lane l ends up holding, for each
// 32x32 block, token (l % 32) and features 8q + 4(l / 32) + r at accumulator
// register 4q + r: four consecutive features per q, stored as one 8-byte chunk.
template <int TM, int TN, int KB, bool BMN = false, int BN = 0>
__device__ __forceinline__ void frag_load(const bf16_t *sA, const bf16_t *sB, int kk, bf16x8 (&ax)[TM],
                                          bf16x8 (&bx)[TN], int wr0, int wc0, int lane) {
    const int chunk = kk * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int row = wr0 + i * 32 + (lane & 31);
        ax[i] = *reinterpret_cast<const bf16x8 *>(sA + row * KB + (swz_chunk<KB>(row, chunk) << 3));
    }
    if constexpr (BMN) {
        frag_b_mn<TN, BN>(sB, kk, bx, wc0, lane);
    } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int col = wc0 + j * 32 + (lane & 31);
            bx[j] = *reinterpret_cast<const bf16x8 *>(sB + col * KB + (swz_chunk<KB>(col, chunk) << 3));
        }
    }
}

template <int TM, int TN>
__device__ __forceinline__ void mfma_slice(const bf16x8 (&ax)[TM], const bf16x8 (&bx)[TN], f32x16 (&acc)[TM][TN]) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bx[j], ax[i], acc[i][j], 0, 0, 0);
}

// Instruction order of one slice: its MFMAs interleaved one-to-one with the
// fragment reads of the following slice, then the remaining MFMAs.
template <int TM, int TN>
__device__ __forceinline__ void slice_schedule() {
    constexpr int FR = TM + TN, MF = TM * TN;
    static_assert(MF >= FR, "a slice needs at least as many MFMAs as fragment reads");
#pragma unroll
    for (int f = 0; f < FR; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MF - FR, 0);
}

// The same order for FR fragment reads (LDS instructions) and MF MFMAs in any ratio:
// pairs while both last, then the rest of either.
template <int FR, int MF>
__device__ __forceinline__ void slice_schedule_n() {
    constexpr int P = FR < MF ? FR : MF;
#pragma unroll
    for (int f = 0; f < P; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    if constexpr (MF > P) __builtin_amdgcn_sched_group_barrier(0x008, MF - P, 0);
    if constexpr (FR > P) __builtin_amdgcn_sched_group_barrier(0x100, FR - P, 0);
}

// NVFP4 weights in the bf16 kernel: eight E2M1 codes (one dword, element i in nibble
// i) of a 16-value block with E4M3 scale byte sb -> their exact values as bf16 (an
// E2M1 value has two significant bits and an E4M3 scale four, so each product is a
// bf16 number). The codes' magnitudes index a byte table of the E4M3 encodings of
// 0, 0.5, 1, 1.5, 2, 3, 4, 6 (v_perm_b32 picks four bytes at once), the sign bits
// move to bit 7, and the hardware's E4M3 -> fp32 conversion gives the values.
__device__ __forceinline__ bf16x8 nvfp4_expand(uint32_t w, uint32_t sb) {
    constexpr uint32_t kLo = 0x3C383000u, kHi = 0x4C484440u;  // E4M3 of 0, .5, 1, 1.5 | 2, 3, 4, 6
    const float s = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sb), 0);
    const uint32_t even = __builtin_amdgcn_perm(kHi, kLo, w & 0x07070707u) | ((w & 0x08080808u) << 4);
    const uint32_t odd = __builtin_amdgcn_perm(kHi, kLo, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
    const f32x2 e02 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(even), false);  // elements 0, 2
    const f32x2 e46 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(even), true);   // 4, 6
    const f32x2 e13 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(odd), false);   // 1, 3
    const f32x2 e57 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(odd), true);    // 5, 7
    const f32x2 p0 = {e02[0] * s, e13[0] * s}, p1 = {e02[1] * s, e13[1] * s};
    const f32x2 p2 = {e46[0] * s, e57[0] * s}, p3 = {e46[1] * s, e57[1] * s};
    const bf16x2 b0 = __builtin_convertvector(p0, bf16x2), b1 = __builtin_convertvector(p1, bf16x2);
    const bf16x2 b2 = __builtin_convertvector(p2, bf16x2), b3 = __builtin_convertvector(p3, bf16x2);
    return bf16x8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
}

// Bytes per weight row of an NVFP4 ring stage (64 k): 32 of codes, then 4 E4M3 scales.
constexpr int kNvRowCodes = 32, kNvRowBytes = 36;

__device__ __forceinline__ void load4_bf16(const bf16_t *p, float *f) {
    const uint2 u = *reinterpret_cast<const uint2 *>(p);
    f[0] = __uint_as_float(u.x << 16);
    f[1] = __uint_as_float(u.x & 0xFFFF0000u);
    f[2] = __uint_as_float(u.y << 16);
    f[3] = __uint_as_float(u.y & 0xFFFF0000u);
}
__device__ __forceinline__ void store4_bf16(bf16_t *p, const float *f) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
}


// 16-byte chunk slot of chunk c of row r in the epilogue tile (CH chunks per
// row, a power of two): XOR with the row spreads the 32 rows that one
// fragment store touches over the chunk slots, and a row read stays a
// permutation of the row's chunks.
template <int CH>
__device__ __forceinline__ int epi_swz(int r, int c) {
    return c ^ (r & (CH - 1));
}

constexpr int kBigKB = 64;  // k per ring stage of the large-tile GEMM
// LDS of the MX GEMM after its ring: the tile prefix table (kMaxE + 1 ints,
// padded to 16 bytes), then the tile's BN bias values.
constexpr int kBigPrefixBytes = ((kMaxE + 1) * 4 + 15) / 16 * 16;
// LDS of the large-tile bf16 GEMM: the two ring stages only (its tile schedule
// lives in registers and its bias is read from global memory), so a 192 x 128
// tile (80 KiB) runs two workgroups per CU.
// With NVFP4 weights (WQ) the ring is followed by two slots of the weights' codes and
// scales (kNvRowBytes per row), which the ring's bf16 weight tiles are expanded from.
template <int BM, int BN, bool WQ = false>
constexpr int big_lds_bytes() {
    return 2 * (BM + BN) * kBigKB * 2 + (WQ ? 2 * BN * kNvRowBytes : 0);
}

// Tile schedule of a persistent rows-grouped GEMM. Expert e has
// rt_e = ceil(fill[e] / BM) row tiles and nx column tiles; tiles are numbered
// expert by expert, and inside an expert in groups of GM row tiles walked
// column by column, so that a window of consecutive tiles shares few A row
// tiles and few B column tiles. Workgroups are dispatched to the 8 XCDs round
// robin (workgroup b on XCD b % 8), so XCD x takes the x-th eighth of the tile
// numbers and its workgroups walk that range together: the tiles in flight on
// one XCD share their operands in that XCD's L2.
constexpr int kXcds = 8;
constexpr int kGroupM = 4;
// Weight gradients with 256 x 256 tiles walk output tiles in groups of
// kGroupKgrad row tiles (128 x 128 tiles keep kGroupM). Measured at S=32768,
// M=4096, E=128, k=8 (256 x 256 tiles, ms): dW2 (16 x 6 tiles per expert) 3.49 /
// 3.51 / 3.41 / 3.50 / 3.64 / 3.55 / 3.63 for groups of 1 / 2 / 3 / 4 / 6 / 8 / 16,
// dW1 (6 x 16) 3.98 / 3.99 / 3.18 / 3.36 / 3.14 / 3.11 / 3.10: a group of 3
// keeps the first and splits the second's 6 row tiles evenly. The row-grouped
// products change by under 2% with group sizes 2 to 8.
constexpr int kGroupKgrad = 3;

struct TileSched {
    int T;        // total tiles
    int first;    // first tile of this workgroup
    int stride;   // workgroups on this XCD
    int end;      // end of this XCD's range
};

// Rows of expert e inside the slot window [s0, s1) of its capacity.
__device__ __forceinline__ int window_rows(const int32_t *fill, int e, int s0, int s1) {
    return max(0, min(fill[e], s1) - s0);
}

// prefix[e] = sum over e' < e of row tiles (LDS, E + 1 entries); returns the schedule.
// Only the slots [s0, s1) of every expert are walked (the whole capacity by default).
template <int NTH>
__device__ __forceinline__ TileSched make_sched(const int32_t *fill, int E, int BMv, int nx, int *prefix, int s0 = 0,
                                                int s1 = 0x7FFFFFFF) {
    __shared__ int wsum[NTH / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += NTH) {
        const int e = e0 + tid;
        const int rt = e < E ? (window_rows(fill, e, s0, s1) + BMv - 1) / BMv : 0;
        int inc = rt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(inc, off, 64);
            if (lane >= off) inc += o;
        }
        if (lane == 63) wsum[w] = inc;
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int q = 0; q < NTH / 64; ++q) {
            before += q < w ? wsum[q] : 0;
            total += wsum[q];
        }
        if (e < E) prefix[e] = base + before + inc - rt;
        base += total;
        __syncthreads();
    }
    if (tid == 0) prefix[E] = base;
    __syncthreads();
    TileSched sc;
    sc.T = base * nx;
    const int x = blockIdx.x % kXcds, nb = gridDim.x / kXcds;  // gridDim.x is a multiple of 8
    const int per = (sc.T + kXcds - 1) / kXcds;
    const int start = min(sc.T, x * per);
    sc.end = min(sc.T, start + per);
    sc.first = start + static_cast<int>(blockIdx.x) / kXcds;
    sc.stride = nb;
    return sc;
}

// tile number -> (expert, row tile, column tile)
__device__ __forceinline__ void decode_tile(int L, const int *prefix, int E, int nx, int &e, int &rtile, int &ctile) {
    const int r = L / nx;  // global row-tile index
    int lo = 0, hi = E - 1;
    while (lo < hi) {  // last e with prefix[e] <= r
        const int mid = (lo + hi + 1) >> 1;
        if (prefix[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    e = __builtin_amdgcn_readfirstlane(lo);  // wavefront-uniform: scalar registers
    const int pe = __builtin_amdgcn_readfirstlane(prefix[e]);
    const int rt_e = __builtin_amdgcn_readfirstlane(prefix[e + 1]) - pe;
    const int u = L - pe * nx;  // tile within the expert
    const int g = u / (kGroupM * nx);
    const int gm = min(kGroupM, rt_e - g * kGroupM);
    const int within = u - g * kGroupM * nx;
    rtile = g * kGroupM + within % gm;
    ctile = within / gm;
}

// The same tile schedule without LDS, computed by every wavefront for itself:
// lane l of a 64-expert chunk holds expert e0 + l's row tiles, a wavefront scan
// gives the prefix, and a ballot finds the tile's expert. Every lane returns
// the same values.
__device__ __forceinline__ int wave_row_tiles(const int32_t *fill, int e, int E, int BMv, int s0, int s1) {
    return e < E ? (window_rows(fill, e, s0, s1) + BMv - 1) / BMv : 0;
}

__device__ __forceinline__ TileSched wave_sched(const int32_t *fill, int E, int BMv, int nx, int s0, int s1) {
    const int lane = threadIdx.x & 63;
    int total = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        int v = wave_row_tiles(fill, e0 + lane, E, BMv, s0, s1);
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        total += v;
    }
    TileSched sc;
    sc.T = __builtin_amdgcn_readfirstlane(total) * nx;
    const int x = blockIdx.x % kXcds, nb = gridDim.x / kXcds;  // gridDim.x is a multiple of 8
    const int per = (sc.T + kXcds - 1) / kXcds;
    const int start = min(sc.T, x * per);
    sc.end = min(sc.T, start + per);
    sc.first = start + static_cast<int>(blockIdx.x) / kXcds;
    sc.stride = nb;
    return sc;
}

// tile number -> (expert, row tile, column tile), as decode_tile
__device__ __forceinline__ void wave_decode_tile(int L, const int32_t *fill, int E, int BMv, int nx, int s0, int s1,
                                                 int &e, int &rtile, int &ctile) {
    const int lane = threadIdx.x & 63;
    const int r = L / nx;  // global row-tile index
    int base = 0, before = 0, rt_e = 1;
    e = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int rt = wave_row_tiles(fill, e0 + lane, E, BMv, s0, s1);
        int inc = rt;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int o = __shfl_up(inc, off, 64);
            if (lane >= off) inc += o;
        }
        const uint64_t hit = __ballot(base + inc > r);  // experts whose tiles end past r
        if (hit != 0ull) {
            const int l = __ffsll(static_cast<long long>(hit)) - 1;
            e = e0 + l;
            rt_e = __shfl(rt, l, 64);
            before = base + __shfl(inc, l, 64) - rt_e;
            break;
        }
        base += __shfl(inc, 63, 64);
    }
    // wavefront-uniform: kept in scalar registers (so are the addresses derived from them)
    e = __builtin_amdgcn_readfirstlane(e);
    before = __builtin_amdgcn_readfirstlane(before);
    rt_e = __builtin_amdgcn_readfirstlane(rt_e);
    const int u = L - before * nx;  // tile within the expert
    const int g = u / (kGroupM * nx);
    const int gm = min(kGroupM, rt_e - g * kGroupM);
    const int within = u - g * kGroupM * nx;
    rtile = g * kGroupM + within % gm;
    ctile = within / gm;
}

// K loop ("ping-pong"): two LDS stages of 64 k. The workgroup barrier of stage
// t sits before its last 16-wide slice: by then every wavefront has read all of
// stage t's fragments (waited with lgkmcnt(0)) and has waited for its own loads
// of stage t+1; after it, the loads of stage t+2 go into stage t's buffer and
// the first fragments of stage t+1 are read while the last slice of stage t
// multiplies. The barrier does not wait for vector memory (barrier_keep_loads),
// so a stage's loads have one full stage of MFMA work to land.
//
// B is read k-contiguous (B[e][n][k], the forward weights) or, with BMN,
// n-contiguous (B[e][k][n], the weights as the backward data products read
// them). Epilogues: fc1 (bias, optional pre-activation output, activation),
// fc2 (bias), plain, and the activation gradient (D = acc * act'(aux), aux the
// saved pre-activation, staged through LDS so that the product is rounded once).
//
// WQ: NVFP4 weights (B = their codes [E*N][K/2], Bsc the E4M3 block scales
// [E*N][K/16], Bg the fp32 scale per expert). The direct loads bring a stage's
// codes ([BN][32] bytes, then the scales [BN][4]) into one of two slots behind the
// ring, one stage earlier than its tokens; the workgroup expands them once
// (nvfp4_expand: a dword of codes and its block's scale byte -> one 16-byte chunk of
// exact bf16 values) into the ring's weight tile, in the layout the bf16 loads give,
// one chunk per thread per slice: stage t+2's expansion starts after stage t's
// barrier, in the buffer that barrier releases, and runs beside stage t+1's MFMAs
// until stage t+1's barrier publishes it. Fragments are then read as for bf16
// weights. The accumulators start at 0; the epilogue multiplies them by the expert's
// g and then adds the bias.
template <int BM, int BN, int NTH, int EPI, int ACT, bool BMN, int WR = 2, bool WQ = false>
__global__ __launch_bounds__(NTH, (big_lds_bytes<BM, BN, WQ>() * 2 <= 160 * 1024 ? 2 : 1)) void rows_gemm_big(const bf16_t *__restrict__ A, const bf16_t *__restrict__ B,
                                                      bf16_t *__restrict__ D, int N, int K, int E,
                                                      const int32_t *__restrict__ fill,
                                                      const int32_t *__restrict__ cap,
                                                      const bf16_t *__restrict__ bias, bf16_t *__restrict__ pre_out,
                                                      const bf16_t *__restrict__ aux, int s0, int s1,
                                                      const uint8_t *__restrict__ Bsc, const float *__restrict__ Bg) {
    extern __shared__ __align__(16) bf16_t lds[];
    constexpr int KB = kBigKB, S = KB / 16;
    // NW wavefronts in 2 rows x NW/2 columns, each owning a (BM/2) x (BN/(NW/2)) block
    constexpr int NW = NTH / 64, WGC = NW / WR;  // WR rows x WGC columns of wavefronts
    constexpr int TM = BM / (32 * WR), TN = BN / (32 * WGC);
    static_assert(TN >= 1 && BN % (32 * WGC) == 0, "wavefront columns must be whole 32-wide blocks");
    static_assert(!WQ || (!BMN && EPI <= EPI_FC2 && BN % (32 * NW) == 0), "NVFP4 weights: forward products");
    constexpr int STAGE = (BM + BN) * KB;                // bf16 units
    constexpr int LPS = (BM + BN) * KB / 8 / NTH;        // direct-load instructions per stage per thread
    constexpr int SLOT = BN * kNvRowBytes;               // bytes of an NVFP4 code slot
    static_assert(BM * BN <= 2 * STAGE, "the epilogue tile must fit in the ring");
    static_assert(!WQ || BN * KB / 8 == S * NTH, "NVFP4: one weight chunk per thread per slice");
    static_assert(BM * (BN / 8) % NTH == 0, "epilogue chunks must split evenly over the threads");
    const int nx = (N + BN - 1) / BN;
    const TileSched sc = wave_sched(fill, E, BM, nx, s0, s1);
    const int C = *cap;
    // the wavefront index as a scalar: the tile offsets and LDS addresses derived
    // from it stay in SGPRs rather than taking VGPRs from the accumulators
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr0 = (wave / WGC) * (BM / WR), wc0 = (wave % WGC) * (BN / WGC);
    const int nk = K / KB;
    for (int L = sc.first; L < sc.end; L += sc.stride) {
        int g, rtile, ctile;
        wave_decode_tile(L, fill, E, BM, nx, s0, s1, g, rtile, ctile);
        const int row0 = rtile * BM, col0 = ctile * BN;
        const int rows_valid = min(BM, window_rows(fill, g, s0, s1) - row0);
        const int cols_valid = min(BN, N - col0);
        const int64_t grow0 = static_cast<int64_t>(g) * C + s0 + row0;
        const bf16_t *Ab = A + grow0 * K;
        const bf16_t *Bb = BMN ? B + static_cast<int64_t>(g) * K * N + col0
                               : B + static_cast<int64_t>(g) * N * K + static_cast<int64_t>(col0) * K;
        const uint8_t *Bq = WQ ? reinterpret_cast<const uint8_t *>(B) + (static_cast<int64_t>(g) * N + col0) * (K / 2)
                               : nullptr;
        const uint8_t *Bsq = WQ ? Bsc + (static_cast<int64_t>(g) * N + col0) * (K / 16) : nullptr;
        auto load_b = [&](int k0, bf16_t *dst) {
            if constexpr (BMN) {
                dma_tile_mn<BN, KB, NW>(Bb, N, cols_valid, k0, dst, wave, lane);
            } else {
                dma_tile<BN, KB, NW>(Bb, K, cols_valid, k0, dst, wave, lane);
            }
        };
        uint8_t *const cslot = reinterpret_cast<uint8_t *>(lds + 2 * STAGE);
        // NVFP4: a stage's codes into a slot: the scale words first (BN / 64 wavefronts,
        // a dword per row), then the codes, 32 rows of 32 bytes per wavefront
        // instruction; rows past the matrix clamped (their columns are never stored)
        auto load_codes = [&](int k0, uint8_t *dq) {
            if (wave < BN / 64) {
                const int row = min(wave * 64 + lane, cols_valid - 1);
                dma4(Bsq, static_cast<uint32_t>(row * (K / 16) + k0 / 16), dq + BN * kNvRowCodes + wave * 256);
            }
#pragma unroll
            for (int j = 0; j < BN / (32 * NW); ++j) {
                const int rb = (j * NW + wave) * 32;
                const int row = min(rb + (lane >> 1), cols_valid - 1);
                dma16(Bq, static_cast<uint32_t>(row * (K / 2) + k0 / 2 + (lane & 1) * 16), dq + rb * kNvRowCodes);
            }
        };
        // NVFP4: chunk j of a slot (row n, eight k from 8c) to the weight tile's bf16 chunk;
        // a wavefront covers eight whole rows, so its code reads are one contiguous block.
        // A chunk's codes are read one slice before its expansion where they can be.
        auto read_chunk = [&](const uint8_t *sq, int j, uint32_t &w, uint32_t &sb) {
            const int idx = j * NTH + tid, n = idx >> 3, c = idx & 7;
            w = *reinterpret_cast<const uint32_t *>(sq + n * kNvRowCodes + c * 4);
            sb = sq[BN * kNvRowCodes + n * 4 + (c >> 1)];
        };
        auto write_chunk = [&](bf16_t *dB, int j, uint32_t w, uint32_t sb) {
            const int idx = j * NTH + tid, n = idx >> 3, c = idx & 7;
            *reinterpret_cast<bf16x8 *>(dB + n * KB + (swz_chunk<KB>(n, c) << 3)) = nvfp4_expand(w, sb);
        };
        auto expand_chunk = [&](const uint8_t *sq, bf16_t *dB, int j) {
            uint32_t w, sb;
            read_chunk(sq, j, w, sb);
            write_chunk(dB, j, w, sb);
        };
        uint32_t pw = 0, psb = 0;  // NVFP4: the codes of the next chunk to expand
        auto load_frags = [&](const bf16_t *st, int kk, bf16x8(&ax)[TM], bf16x8(&bx)[TN]) {
            frag_load<TM, TN, KB, BMN, BN>(st, st + BM * KB, kk, ax, bx, wr0, wc0, lane);
        };
        auto schedule = [&]() {
            // NVFP4: the expansion's two LDS reads go with the fragment reads
            if constexpr (WQ) slice_schedule_n<TM + TN + 2, TM * TN>();
            else slice_schedule<TM, TN>();
        };

        // Only the forward products have a bias: the accumulators start at it (read
        // from global memory, L2-resident; columns past the matrix read the last
        // valid chunk and are never stored), so the epilogue only applies the
        // activation. Its loads go out ahead of the prologue's stage loads: loads
        // complete in order, so the wait for stage 0 covers them as well, where
        // loads issued after stage 1 would hold the first MFMA until stage 1 lands.
        // Tiles with 128 accumulators per lane at eight wavefronts (256 x 256) have
        // no registers to spare across the prologue and read it after the prologue.
        constexpr bool kBias = EPI <= EPI_FC2;
        constexpr bool kEarlyBias = !WQ && kBias && TM * TN * 16 < 128;
        const bool with_bias = kBias && bias != nullptr;
        const bf16_t *bt = with_bias ? bias + static_cast<int64_t>(g) * N + col0 : nullptr;
        uint2 bq[kEarlyBias ? TN : 1][4];
        if (kEarlyBias && with_bias) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    bq[kEarlyBias ? j : 0][q] = *reinterpret_cast<const uint2 *>(
                        bt + min(wc0 + j * 32 + 8 * q + 4 * (lane >> 5), cols_valid - 4));
        }
        f32x16 acc[TM][TN];
        if constexpr (!kEarlyBias) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        }

        // The previous tile's LDS reads (epilogue) are complete in every
        // wavefront; its global stores may still be in flight.
        barrier_keep_loads_lds();
        if constexpr (WQ) {
            // stage 0's weights expanded whole, stage 1's first chunk (the rest during
            // stage 0); stage 2's codes go out once every wavefront has read slot 0
            // (stage 1's tokens go last, so that the expansion need not wait for them)
            dma_tile<BM, KB, NW>(Ab, K, rows_valid, 0, lds, wave, lane);
            load_codes(0, cslot);
            if (nk > 1) {
                load_codes(KB, cslot + SLOT);
                dma_tile<BM, KB, NW>(Ab, K, rows_valid, KB, lds + STAGE, wave, lane);
                wait_vmcnt<BM * KB / 8 / NTH>();
            } else {
                wait_vmcnt<0>();
            }
            barrier_keep_loads();
#pragma unroll
            for (int j = 0; j < S; ++j) expand_chunk(cslot, lds + BM * KB, j);
            expand_chunk(cslot + SLOT, lds + STAGE + BM * KB, 0);
            read_chunk(cslot + SLOT, 1, pw, psb);
            barrier_keep_loads_lds();
            if (nk > 2) load_codes(2 * KB, cslot);
        } else {
            dma_tile<BM, KB, NW>(Ab, K, rows_valid, 0, lds, wave, lane);
            load_b(0, lds + BM * KB);
            if (nk > 1) {
                dma_tile<BM, KB, NW>(Ab, K, rows_valid, KB, lds + STAGE, wave, lane);
                load_b(KB, lds + STAGE + BM * KB);
                wait_vmcnt<LPS>();
            } else {
                wait_vmcnt<0>();
            }
            barrier_keep_loads();
        }
        if constexpr (kEarlyBias) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float b4[4] = {0.f, 0.f, 0.f, 0.f};
                    if (with_bias) {
                        const uint2 u = bq[kEarlyBias ? j : 0][q];
                        b4[0] = __uint_as_float(u.x << 16);
                        b4[1] = __uint_as_float(u.x & 0xFFFF0000u);
                        b4[2] = __uint_as_float(u.y << 16);
                        b4[3] = __uint_as_float(u.y & 0xFFFF0000u);
                    }
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] = b4[r];
                }
        } else if (!WQ && kBias && with_bias) {
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float b4[4];
                    load4_bf16(bt + min(wc0 + j * 32 + 8 * q + 4 * (lane >> 5), cols_valid - 4), b4);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] = b4[r];
                }
        }
        bf16x8 fa[2][TM], fb[2][TN];
        load_frags(lds, 0, fa[0], fb[0]);
        for (int t = 0; t < nk; ++t) {
            const bf16_t *scur = lds + (t & 1) * STAGE;
            bf16_t *const onext = lds + ((t + 1) & 1) * STAGE;
#pragma unroll
            for (int kk = 0; kk < S - 1; ++kk) {
                load_frags(scur, kk + 1, fa[(kk + 1) & 1], fb[(kk + 1) & 1]);
                // NVFP4: the rest of stage t+1's weights. Branch-free: at the last step it
                // rewrites the other buffer's weight tile, which nothing reads any more.
                if constexpr (WQ) {
                    uint32_t nw = 0, nsb = 0;
                    if (kk + 2 < S) read_chunk(cslot + ((t + 1) & 1) * SLOT, kk + 2, nw, nsb);
                    write_chunk(onext + BM * KB, kk + 1, pw, psb);
                    pw = nw;
                    psb = nsb;
                }
                mfma_slice<TM, TN>(fa[kk & 1], fb[kk & 1], acc);
                schedule();
            }
            // At the last step this also runs, uniformly: there is no load to wait
            // for, and the fragments read from the other buffer are not used.
            wait_vmcnt<0>();  // this wavefront's loads of stage t+1 have landed
            barrier_keep_loads_lds();
            bf16_t *const sn = lds + (t & 1) * STAGE;
            if (t + 2 < nk) {
                dma_tile<BM, KB, NW>(Ab, K, rows_valid, (t + 2) * KB, sn, wave, lane);
                if constexpr (WQ) {
                    if (t + 3 < nk) load_codes((t + 3) * KB, cslot + ((t + 1) & 1) * SLOT);
                } else {
                    load_b((t + 2) * KB, sn + BM * KB);
                }
            }
            // NVFP4: the first chunk of stage t+2's weights (from the last two steps on,
            // into a buffer that nothing reads any more); its codes are read ahead of the
            // fragments, so that their wait does not take in the fragment reads
            uint32_t w0 = 0, s0b = 0;
            if constexpr (WQ) {
                read_chunk(cslot + (t & 1) * SLOT, 0, w0, s0b);
                read_chunk(cslot + (t & 1) * SLOT, 1, pw, psb);
            }
            load_frags(onext, 0, fa[S & 1], fb[S & 1]);
            if constexpr (WQ) write_chunk(sn + BM * KB, 0, w0, s0b);
            mfma_slice<TM, TN>(fa[(S - 1) & 1], fb[(S - 1) & 1], acc);
            schedule();
        }
        if constexpr (WQ) {
            // the expert's fp32 scale, then the bias: acc = g * acc + b
            const float gs = Bg[g];
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float b4[4] = {0.f, 0.f, 0.f, 0.f};
                    if (with_bias) load4_bf16(bt + min(wc0 + j * 32 + 8 * q + 4 * (lane >> 5), cols_valid - 4), b4);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[i][j][4 * q + r] = fmaf(acc[i][j][4 * q + r], gs, b4[r]);
                }
        }

        // Epilogue through LDS. Per 32x32 block, lane l owns token row (l % 32)
        // and, for q = 0..3, features 8q + 4(l / 32) .. +3 (the bias is already in
        // the accumulators): written (activation applied, rounded to bf16) into
        // the free ring as a row-major
        // BM x BN tile whose 16-byte chunks are XOR-swizzled by row, then read
        // back a row at a time so that every global store is whole 16-byte
        // chunks of contiguous rows (full cache lines), not 32 rows x 16 bytes.
        // fc1 with a pre-activation output makes two passes (pre, then h).
        barrier_keep_loads_lds();  // every wavefront is done with the ring
        if constexpr (EPI == EPI_DACT) {
            // the tile's saved pre-activations, in the epilogue tile's layout
            constexpr int CH = BN / 8, RPI = 64 / CH;
            static_assert(BM % (NW * RPI) == 0, "pre-activation tile rows must split over the wavefronts");
#pragma unroll
            for (int j = 0; j < BM / (NW * RPI); ++j) {
                const int rb = (j * NW + wave) * RPI;
                const int r = rb + lane / CH;
                const int c = min(epi_swz<CH>(r, lane % CH), cols_valid / 8 - 1);  // chunk stored at this slot
                const int rr = min(r, rows_valid - 1);
                const uint32_t off = static_cast<uint32_t>(rr * N + c * 8);
                dma16(aux + grow0 * N + col0, off * 2, lds + rb * BN);
            }
            wait_vmcnt<0>();
            barrier_keep_loads();
        }
        constexpr int NPASS = EPI == EPI_FC1 ? 2 : 1;
#pragma unroll
        for (int pass = 0; pass < NPASS; ++pass) {
            // fc1: pass 0 = pre-activation (only when requested), pass 1 = h
            if (NPASS == 2 && pass == 0 && pre_out == nullptr) continue;
            const bool act = EPI == EPI_FC1 && pass == NPASS - 1;
            bf16_t *dst = (NPASS == 2 && pass == 0) ? pre_out : D;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int trow = wr0 + i * 32 + (lane & 31);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int tcol = wc0 + j * 32 + 8 * q + 4 * (lane >> 5);
                        f32x2 lo = {acc[i][j][4 * q], acc[i][j][4 * q + 1]};
                        f32x2 hi = {acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                        if (act) {
                            lo[0] = act_fast<ACT>(lo[0]);
                            lo[1] = act_fast<ACT>(lo[1]);
                            hi[0] = act_fast<ACT>(hi[0]);
                            hi[1] = act_fast<ACT>(hi[1]);
                        }
                        const int c = tcol >> 3;
                        uint2 *slot = reinterpret_cast<uint2 *>(lds + trow * BN + (epi_swz<BN / 8>(trow, c) << 3) +
                                                                ((lane >> 5) << 2));
                        if constexpr (EPI == EPI_DACT) {
                            const uint2 p = *slot;  // the pre-activations of these four outputs
                            lo[0] *= act_grad_fast<ACT>(__uint_as_float(p.x << 16));
                            lo[1] *= act_grad_fast<ACT>(__uint_as_float(p.x & 0xFFFF0000u));
                            hi[0] *= act_grad_fast<ACT>(__uint_as_float(p.y << 16));
                            hi[1] *= act_grad_fast<ACT>(__uint_as_float(p.y & 0xFFFF0000u));
                        }
                        const bf16x2 plo = __builtin_convertvector(lo, bf16x2);
                        const bf16x2 phi = __builtin_convertvector(hi, bf16x2);
                        uint2 w;
                        w.x = *reinterpret_cast<const uint32_t *>(&plo);
                        w.y = *reinterpret_cast<const uint32_t *>(&phi);
                        *slot = w;
                    }
                    // one 32 x 32 block at a time: keeps the activation math of
                    // different blocks from being interleaved (register pressure)
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            barrier_keep_loads_lds();
            constexpr int CH = BN / 8;
#pragma unroll 4
            for (int u = 0; u < BM * CH / NTH; ++u) {
                const int idx = tid + u * NTH, r = idx / CH, c = idx % CH;
                const uint4 v = *reinterpret_cast<const uint4 *>(lds + r * BN + (epi_swz<CH>(r, c) << 3));
                if (r < rows_valid && c * 8 < cols_valid)
                    *reinterpret_cast<uint4 *>(dst + (grow0 + r) * N + col0 + c * 8) = v;
            }
            if (pass + 1 < NPASS) barrier_keep_loads_lds();  // the tile is read before the next pass rewrites it
        }
        // The next tile's barrier (below the loop head) orders these LDS reads
        // before its loads refill the ring; the global stores drain meanwhile.
    }
    wait_vmcnt<0>();  // no direct-to-LDS write may land after the workgroup's LDS is released
}

// ------------------------------------------------------------------ rows-grouped MX GEMM (MXFP8 / MXFP4)

// The expert FFN on MX operands (OCP microscaling: 32-value blocks along K share
// an E8M0 scale) with gfx950's scaled MFMA v_mfma_scale_f32_32x32x64_f8f6f4:
// A = the tokens (MXFP8), B = the weights (MXFP8 or MXFP4), both k-contiguous
// codes with per-row scale bytes [rows][K/32]. Same persistent, XCD-aware tile
// walk and ping-pong ring of direct loads as the bf16 kernel; a ring stage
// holds 128 k (128 bytes per token row, 128 or 64 per weight row) and feeds two
// 64-wide MFMA slices. Operand layout of the scaled MFMA (checked on the GPU):
// lane l holds row l % 32; with 8-bit elements lane half h = l / 32 holds the
// slice's bytes [16h, 16h+16) and [32+16h, 32+16h+16) (two 16-byte LDS reads),
// with 4-bit elements bytes [16h, 16h+16) (32 values); the scale of k-block h of
// the slice comes from lane half h, byte 2 * slice + h of the row's dword for the
// stage. The scale dwords travel through LDS with the ring: the stage that opens a
// group of four stages (one stage when K is not a multiple of 512) also loads the
// group's dwords of every tile row, 16 (or 4) bytes per row, into one of two group
// buffers, and each wavefront reads its rows' dwords after the end-of-stage barrier.
// Loading them into registers instead would make the compiler, which does not see
// the ring's direct loads, wait at their first use for every load in flight, the
// next ring stage included. The hardware's fp8 accumulation drops low-order bits of products
// far below the largest one in a group of eight (about 1e-4 of the sum of
// magnitudes), so results match an exact sum within that, not bit for bit.
// Epilogues: fc1 adds the bias, applies the activation and quantises h to MXFP8
// per (token, 32 features): the two lanes l, l ^ 32 holding a token's 32
// features of a block exchange their amax, codes and scales go through LDS to
// whole-row stores; fc2 adds the bias and stores bf16 as the bf16 kernel does.
//
// BLK: block-wise FP8 instead (E4M3 codes; one fp32 scale per 1 x 128 block of a
// token row, s = amax / 448, and per 128 x 128 block of the weights). A ring stage
// is exactly one 128-deep block of both operands, so its two MFMAs run with unit
// scales into a fresh partial P, and acc += P * (s_token * s_weight): the token's
// scale is per lane (its row), the weight's per 32-column MFMA block (uniform).
// The scale words have the MX layout's stride (one 32-bit word per row and stage),
// so they travel the same way. fc1 quantises h per (token, 128 features): a
// wavefront holds 64 of a block's features, so the two wavefronts of a block
// exchange their amax through LDS before dividing by s.
typedef int mx_v8i __attribute__((ext_vector_type(8)));

constexpr int kMxStageK = 128;  // k per ring stage

// Bytes of the LDS region shared by the two ring stages and the epilogue tile
// (bf16 y of fc2, or fc1's h codes and scales), then the tile prefix and bias.
template <int BM, int BN, int WFMT, int EPI, bool BLK = false>
constexpr int mx_region_bytes() {
    constexpr int ring = 2 * (BM * kMxStageK + BN * (WFMT == kMxFp8 ? kMxStageK : kMxStageK / 2));
    // fc1's h tile: codes, then the scales (BLK: fp32 per 128 features, and each wavefront's
    // per-row amax, BN / 64 of them per row)
    constexpr int epi = EPI == EPI_FC1 ? (BLK ? BM * BN + BM * (BN / 128) * 4 + BM * (BN / 64) * 4
                                              : BM * BN + BM * BN / 32)
                                       : BM * BN * 2;
    return ring > epi ? ring : epi;
}
// Bytes of one scale group buffer: four stages' dwords of every tile row.
template <int BM, int BN>
constexpr int mx_scale_buf_bytes() {
    return (BM + BN) * 16;
}
template <int BM, int BN, int WFMT, int EPI, bool BLK = false>
constexpr int mx_lds_bytes() {
    return mx_region_bytes<BM, BN, WFMT, EPI, BLK>() + kBigPrefixBytes + BN * 2 + 2 * mx_scale_buf_bytes<BM, BN>();
}

// MFMA operand of one row (the lane's) for slice s from an LDS tile of rows of
// RB bytes (CPR = RB / 16 chunks, swizzled by swz_chunk on bf16 units).
template <int RB, bool FP4>
__device__ __forceinline__ mx_v8i mx_frag(const bf16_t *tile, int row, int s, int h) {
    constexpr int KBU = RB / 2;  // row length in bf16 units
    const bf16_t *base = tile + row * KBU;
    mx_v8i v;
    if constexpr (FP4) {
        const uint4 a = *reinterpret_cast<const uint4 *>(base + (swz_chunk<KBU>(row, 2 * s + h) << 3));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = 0; v[5] = 0; v[6] = 0; v[7] = 0;
    } else {
        const uint4 a = *reinterpret_cast<const uint4 *>(base + (swz_chunk<KBU>(row, 4 * s + h) << 3));
        const uint4 b = *reinterpret_cast<const uint4 *>(base + (swz_chunk<KBU>(row, 4 * s + 2 + h) << 3));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    return v;
}

template <int BM, int BN, int NTH, int EPI, int ACT, int WFMT, bool BLK = false>
__global__ __launch_bounds__(NTH, (BLK && BM * BN <= 128 * 128) ? 2 : 1) void rows_gemm_mx(const uint8_t *__restrict__ A, const uint8_t *__restrict__ As,
                                                     const uint8_t *__restrict__ B, const uint8_t *__restrict__ Bs,
                                                     void *__restrict__ D, uint8_t *__restrict__ Dsc, int N, int K,
                                                     int E, const int32_t *__restrict__ fill,
                                                     const int32_t *__restrict__ cap,
                                                     const bf16_t *__restrict__ bias) {
    extern __shared__ __align__(16) bf16_t lds[];
    constexpr bool FP4 = WFMT == kMxFp4;
    constexpr int RA = kMxStageK, RBW = FP4 ? kMxStageK / 2 : kMxStageK;  // bytes per row per stage
    constexpr int KA = RA / 2, KW = RBW / 2;                              // ... in bf16 units
    constexpr int NW = NTH / 64, WGC = NW / 2;
    constexpr int TM = BM / 64, TN = BN / (32 * WGC);
    static_assert(TN >= 1 && BN % (32 * WGC) == 0, "wavefront columns must be whole 32-wide blocks");
    static_assert(!BLK || (WFMT == kMxFp8 && BN / WGC == 64), "block FP8: E4M3 weights, 64 columns a wavefront");
    constexpr int STAGE = BM * KA + BN * KW;  // bf16 units
    constexpr int REGION = mx_region_bytes<BM, BN, WFMT, EPI, BLK>() / 2;
    int *prefix = reinterpret_cast<int *>(lds + REGION);
    bf16_t *sbias = lds + REGION + kBigPrefixBytes / 2;
    // two scale group buffers, each [BM][GS] token dwords then [BN][GS] weight dwords
    uint32_t *ssc = reinterpret_cast<uint32_t *>(sbias + BN);
    constexpr int SCB = mx_scale_buf_bytes<BM, BN>() / 4;  // dwords per buffer
    const int nx = (N + BN - 1) / BN;
    const TileSched sc = make_sched<NTH>(fill, E, BM, nx, prefix);
    const int C = *cap;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), h = lane >> 5;
    const int wr0 = (wave / WGC) * (BM / 2), wc0 = (wave % WGC) * (BN / WGC);
    const int nk = K / kMxStageK, KS = K / 32;  // stages, scale bytes per row
    const int ldA = K / 2, ldB = FP4 ? K / 4 : K / 2;   // row length in bf16 units
    constexpr int WCODE = FP4 ? 4 : 0;                  // scaled-MFMA operand formats: 4 = E2M1, 0 = E4M3
    for (int L = sc.first; L < sc.end; L += sc.stride) {
        int g, rtile, ctile;
        decode_tile(L, prefix, E, nx, g, rtile, ctile);
        const int row0 = rtile * BM, col0 = ctile * BN;
        const int rows_valid = min(BM, fill[g] - row0);
        const int cols_valid = min(BN, N - col0);
        const int64_t grow0 = static_cast<int64_t>(g) * C + row0;
        const bf16_t *Ab = reinterpret_cast<const bf16_t *>(A + grow0 * K);
        const int64_t wrow0 = static_cast<int64_t>(g) * N + col0;  // first weight row of the tile
        const bf16_t *Bb = reinterpret_cast<const bf16_t *>(B + wrow0 * (FP4 ? K / 2 : K));
        // scale rows: the tile's tokens; the weights' rows (BLK: their 128-row blocks, the
        // tile's first one at wrow0 / 128 as N is a multiple of 128)
        const uint8_t *sa_base = As + grow0 * KS;
        const uint8_t *sb_base = Bs + (BLK ? wrow0 / 128 : wrow0) * KS;

        f32x16 acc[TM][TN], part[TM][TN];  // part: BLK's per-stage partial sums
        f32x16 zero;
#pragma unroll
        for (int v = 0; v < 16; ++v) zero[v] = 0.f;
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = zero;

        barrier_keep_loads_lds();  // the previous tile's epilogue reads of LDS are complete
        if (bias != nullptr && wave == 0 && lane < BN / 8) {
            const int c = min(lane * 8, cols_valid - 8);
            dma16(bias + wrow0, static_cast<uint32_t>(c) * 2, sbias);
        }
        // Scale groups of GS stages: 16-byte loads of four stages' dwords when the rows are
        // 16-byte aligned (K a multiple of 512), else one stage's dword. Each wavefront loads
        // 64 rows per instruction (rows clamped into the valid range, as for the ring), the
        // group of stages [s, s + GS) going to buffer (s / GS) & 1.
        const int GS = (K % 512) == 0 ? 4 : 1;
        auto dma_scales = [&](int s) {
            uint32_t *buf = ssc + ((s / GS) & 1) * SCB;
            for (int q = wave; q < (BM + BN) / 64; q += NW) {
                const bool tok = q < BM / 64;
                const int r0 = (tok ? q : q - BM / 64) * 64;
                uint32_t off;
                if (tok) {
                    off = static_cast<uint32_t>(min(r0 + lane, rows_valid - 1) * KS + s * 4);
                } else {
                    const int c = min(r0 + lane, cols_valid - 1);
                    off = static_cast<uint32_t>((BLK ? c / 128 : c) * KS + s * 4);
                }
                uint32_t *dst = buf + (tok ? 0 : BM * 4) + r0 * GS;
                if (GS == 4)
                    dma16(tok ? sa_base : sb_base, off, dst);
                else
                    dma4(tok ? sa_base : sb_base, off, dst);
            }
        };
        // stage s's dwords of the wavefront's rows (the group was loaded with stage s - s % GS,
        // which has passed an end-of-stage barrier)
        auto read_scales = [&](int s, uint32_t(&ca)[TM], uint32_t(&cb)[TN]) {
            const uint32_t *buf = ssc + ((s / GS) & 1) * SCB;
            const int slot = s & (GS - 1);
#pragma unroll
            for (int i = 0; i < TM; ++i) ca[i] = buf[(wr0 + i * 32 + (lane & 31)) * GS + slot];
#pragma unroll
            for (int j = 0; j < TN; ++j) cb[j] = buf[BM * 4 + (wc0 + j * 32 + (lane & 31)) * GS + slot];
        };
        // stage t's ring loads, after its scale group when t opens one
        auto dma_stage = [&](int t) {
            if (t % GS == 0) dma_scales(t);
            bf16_t *sn = lds + (t & 1) * STAGE;
            dma_tile<BM, KA, NW>(Ab, ldA, rows_valid, t * KA, sn, wave, lane);
            dma_tile<BN, KW, NW>(Bb, ldB, cols_valid, t * KW, sn + BM * KA, wave, lane);
        };
        uint32_t sa_cur[TM], sb_cur[TN];
        dma_stage(0);
        if (nk > 1) {
            // stage 1's scale dwords (GS = 1) are requested before its ring loads, so this count
            // of stage 1's ring loads still covers them
            if (GS == 1) dma_scales(1);
            bf16_t *sn = lds + STAGE;
            dma_tile<BM, KA, NW>(Ab, ldA, rows_valid, KA, sn, wave, lane);
            dma_tile<BN, KW, NW>(Bb, ldB, cols_valid, KW, sn + BM * KA, wave, lane);
            wait_vmcnt<(BM * KA + BN * KW) / 8 / NTH>();
        } else {
            wait_vmcnt<0>();
        }
        barrier_keep_loads();
        read_scales(0, sa_cur, sb_cur);
        if constexpr (BLK) {
            // One set of fragments: a stage's slice 0 is read and multiplied, then slice 1,
            // into the partial P; then acc += P * (s_token * s_weight) and the end-of-stage
            // barrier, after which stage t+2's loads refill the buffer just read. Without the
            // ping-pong's second set of fragments the kernel fits two workgroups per CU, whose
            // MFMAs cover each other's LDS reads.
            for (int t = 0; t < nk; ++t) {
                const bf16_t *scur = lds + (t & 1) * STAGE;
#pragma unroll
                for (int sl = 0; sl < 2; ++sl) {
                    mx_v8i fa[TM], fb[TN];
#pragma unroll
                    for (int i = 0; i < TM; ++i) fa[i] = mx_frag<RA, false>(scur, wr0 + i * 32 + (lane & 31), sl, h);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        fb[j] = mx_frag<RBW, false>(scur + BM * KA, wc0 + j * 32 + (lane & 31), sl, h);
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fb[j], fa[i], sl == 0 ? zero : part[i][j], 0, 0, 0, 127, 0, 127);
                }
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const float f = __uint_as_float(sa_cur[i]) * __uint_as_float(sb_cur[j]);
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[i][j][v] = fmaf(part[i][j][v], f, acc[i][j][v]);
                    }
                wait_vmcnt<0>();  // stage t+1's ring loads and scales have landed
                barrier_keep_loads_lds();
                if (t + 1 < nk) read_scales(t + 1, sa_cur, sb_cur);
                if (t + 2 < nk) dma_stage(t + 2);
            }
        } else {
            // Ping-pong over the two 64-wide slices of a stage: slice 1's fragments are read
            // while slice 0 multiplies; the barrier sits before slice 1's MFMAs, after which
            // stage t+2's loads refill the buffer just read and stage t+1's first fragments are
            // read while slice 1 multiplies.
            mx_v8i fa0[TM], fb0[TN], fa1[TM], fb1[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa0[i] = mx_frag<RA, false>(lds, wr0 + i * 32 + (lane & 31), 0, h);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb0[j] = mx_frag<RBW, FP4>(lds + BM * KA, wc0 + j * 32 + (lane & 31), 0, h);
            for (int t = 0; t < nk; ++t) {
                const bf16_t *scur = lds + (t & 1) * STAGE;
#pragma unroll
                for (int i = 0; i < TM; ++i) fa1[i] = mx_frag<RA, false>(scur, wr0 + i * 32 + (lane & 31), 1, h);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    fb1[j] = mx_frag<RBW, FP4>(scur + BM * KA, wc0 + j * 32 + (lane & 31), 1, h);
                {
                    const int sh = 8 * h;  // slice 0: k-blocks 0 (half 0) and 1 (half 1) of the stage
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fb0[j], fa0[i], acc[i][j], WCODE, 0, 0, static_cast<int>((sb_cur[j] >> sh) & 0xFFu), 0,
                                static_cast<int>((sa_cur[i] >> sh) & 0xFFu));
                }
                wait_vmcnt<0>();  // stage t+1's ring loads and scales have landed
                barrier_keep_loads_lds();
                uint32_t sa_nxt[TM], sb_nxt[TN];
                if (t + 1 < nk) read_scales(t + 1, sa_nxt, sb_nxt);
                if (t + 2 < nk) dma_stage(t + 2);
                // at the last stage these reads are from the other buffer and unused
                const bf16_t *snext = lds + ((t + 1) & 1) * STAGE;
#pragma unroll
                for (int i = 0; i < TM; ++i) fa0[i] = mx_frag<RA, false>(snext, wr0 + i * 32 + (lane & 31), 0, h);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    fb0[j] = mx_frag<RBW, FP4>(snext + BM * KA, wc0 + j * 32 + (lane & 31), 0, h);
                {
                    const int sh = 8 * (2 + h);  // slice 1: k-blocks 2 and 3
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                                fb1[j], fa1[i], acc[i][j], WCODE, 0, 0, static_cast<int>((sb_cur[j] >> sh) & 0xFFu), 0,
                                static_cast<int>((sa_cur[i] >> sh) & 0xFFu));
                }
                if (t + 1 < nk) {
#pragma unroll
                    for (int i = 0; i < TM; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
                    for (int j = 0; j < TN; ++j) sb_cur[j] = sb_nxt[j];
                }
            }
        }
        wait_vmcnt<0>();
        barrier_keep_loads_lds();  // every wavefront is done with the ring

        if constexpr (EPI == EPI_FC1 && BLK) {
            // h = act(acc + b1) quantised per (token, 128 features): codes staged as below, the
            // fp32 scales as [BM][BN/128]; each wavefront first posts its rows' amax over its 64
            // columns ([BM][BN/64]), and a block's two wavefronts combine them
            constexpr int CH = BN / 16, NB = BN / 128, WPR = BN / 64;
            uint8_t *scodes = reinterpret_cast<uint8_t *>(lds);
            float *sscale = reinterpret_cast<float *>(scodes + BM * BN);
            float *samax = sscale + BM * NB;
            const int wq = wave % WGC;  // the wavefront's 64-column slab; block wq / 2
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int trow = wr0 + i * 32 + (lane & 31);
                float am = 0.f;
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int tcol = wc0 + j * 32 + 8 * q + 4 * h;
                        float b4[4] = {0.f, 0.f, 0.f, 0.f};
                        if (bias != nullptr) {
                            const uint2 u2 = *reinterpret_cast<const uint2 *>(sbias + tcol);
                            b4[0] = __uint_as_float(u2.x << 16);
                            b4[1] = __uint_as_float(u2.x & 0xFFFF0000u);
                            b4[2] = __uint_as_float(u2.y << 16);
                            b4[3] = __uint_as_float(u2.y & 0xFFFF0000u);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const float v = act_fast<ACT>(acc[i][j][4 * q + r] + b4[r]);
                            acc[i][j][4 * q + r] = v;
                            am = fmaxf(am, fabsf(v));
                        }
                    }
                am = fmaxf(am, __shfl_xor(am, 32, 64));
                if (h == 0) samax[trow * WPR + wq] = am;
            }
            barrier_keep_loads_lds();
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int trow = wr0 + i * 32 + (lane & 31);
                const float sc = fmaxf(samax[trow * WPR + (wq & ~1)], samax[trow * WPR + (wq | 1)]) / 448.f;
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = blk_fp8x2(acc[i][j][4 * q], acc[i][j][4 * q + 1], sc);
                        const uint32_t hi = blk_fp8x2(acc[i][j][4 * q + 2], acc[i][j][4 * q + 3], sc);
                        const int tcol = wc0 + j * 32 + 8 * q + 4 * h;
                        *reinterpret_cast<uint32_t *>(scodes + trow * BN + (epi_swz<CH>(trow, tcol >> 4) << 4) +
                                                      (tcol & 15)) = lo | (hi << 16);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (h == 0 && (wq & 1) == 0) sscale[trow * NB + wq / 2] = sc;
            }
            barrier_keep_loads_lds();
            uint8_t *Dc = static_cast<uint8_t *>(D);
#pragma unroll 4
            for (int u = 0; u < BM * CH / NTH; ++u) {
                const int idx = tid + u * NTH, r = idx / CH, c = idx % CH;
                const uint4 v = *reinterpret_cast<const uint4 *>(scodes + r * BN + (epi_swz<CH>(r, c) << 4));
                if (r < rows_valid && c * 16 < cols_valid)
                    *reinterpret_cast<uint4 *>(Dc + (grow0 + r) * N + col0 + c * 16) = v;
            }
            float *Ds = reinterpret_cast<float *>(Dsc);
            for (int idx = tid; idx < BM * NB; idx += NTH) {
                const int r = idx / NB, c = idx % NB;
                if (r < rows_valid && c * 128 < cols_valid) Ds[(grow0 + r) * (N / 128) + col0 / 128 + c] = sscale[idx];
            }
        } else if constexpr (EPI == EPI_FC1) {
            // h = act(acc + b1) quantised to MXFP8 per (token, 32-feature block); codes staged as a
            // row-major BM x BN byte tile (16-byte chunks XOR-swizzled by row), scales as [BM][BN/32]
            constexpr int CH = BN / 16;
            uint8_t *scodes = reinterpret_cast<uint8_t *>(lds);
            uint8_t *sscale = scodes + BM * BN;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int trow = wr0 + i * 32 + (lane & 31);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    float v[16];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int tcol = wc0 + j * 32 + 8 * q + 4 * h;
                        float b4[4] = {0.f, 0.f, 0.f, 0.f};
                        if (bias != nullptr) {
                            const uint2 u2 = *reinterpret_cast<const uint2 *>(sbias + tcol);
                            b4[0] = __uint_as_float(u2.x << 16);
                            b4[1] = __uint_as_float(u2.x & 0xFFFF0000u);
                            b4[2] = __uint_as_float(u2.y << 16);
                            b4[3] = __uint_as_float(u2.y & 0xFFFF0000u);
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) v[4 * q + r] = act_fast<ACT>(acc[i][j][4 * q + r] + b4[r]);
                    }
                    float amax = 0.f;
#pragma unroll
                    for (int u = 0; u < 16; ++u) amax = fmaxf(amax, fabsf(v[u]));
                    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
                    const int e = mx_shared_exp(amax, 8);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = mx_fp8x2(ldexpf(v[4 * q], -e), ldexpf(v[4 * q + 1], -e));
                        const uint32_t hi = mx_fp8x2(ldexpf(v[4 * q + 2], -e), ldexpf(v[4 * q + 3], -e));
                        const int tcol = wc0 + j * 32 + 8 * q + 4 * h;
                        *reinterpret_cast<uint32_t *>(scodes + trow * BN + (epi_swz<CH>(trow, tcol >> 4) << 4) +
                                                      (tcol & 15)) = lo | (hi << 16);
                    }
                    if (h == 0) sscale[trow * (BN / 32) + (wc0 + j * 32) / 32] = static_cast<uint8_t>(e + 127);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            barrier_keep_loads_lds();
            uint8_t *Dc = static_cast<uint8_t *>(D);
#pragma unroll 4
            for (int u = 0; u < BM * CH / NTH; ++u) {
                const int idx = tid + u * NTH, r = idx / CH, c = idx % CH;
                const uint4 v = *reinterpret_cast<const uint4 *>(scodes + r * BN + (epi_swz<CH>(r, c) << 4));
                if (r < rows_valid && c * 16 < cols_valid)
                    *reinterpret_cast<uint4 *>(Dc + (grow0 + r) * N + col0 + c * 16) = v;
            }
            for (int idx = tid; idx < BM * (BN / 128); idx += NTH) {  // four scale bytes (128 features) per store
                const int r = idx / (BN / 128), c = idx % (BN / 128);
                if (r < rows_valid && c * 128 < cols_valid)
                    *reinterpret_cast<uint32_t *>(Dsc + (grow0 + r) * (N / 32) + col0 / 32 + c * 4) =
                        *reinterpret_cast<const uint32_t *>(sscale + r * (BN / 32) + c * 4);
            }
        } else {
            // y = acc + b2, bf16, staged like the bf16 kernel's epilogue
            constexpr int CH = BN / 8;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int trow = wr0 + i * 32 + (lane & 31);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int tcol = wc0 + j * 32 + 8 * q + 4 * h;
                        f32x2 lo = {acc[i][j][4 * q], acc[i][j][4 * q + 1]};
                        f32x2 hi = {acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                        if (bias != nullptr) {
                            const uint2 u2 = *reinterpret_cast<const uint2 *>(sbias + tcol);
                            lo[0] += __uint_as_float(u2.x << 16);
                            lo[1] += __uint_as_float(u2.x & 0xFFFF0000u);
                            hi[0] += __uint_as_float(u2.y << 16);
                            hi[1] += __uint_as_float(u2.y & 0xFFFF0000u);
                        }
                        const bf16x2 plo = __builtin_convertvector(lo, bf16x2);
                        const bf16x2 phi = __builtin_convertvector(hi, bf16x2);
                        uint2 w;
                        w.x = *reinterpret_cast<const uint32_t *>(&plo);
                        w.y = *reinterpret_cast<const uint32_t *>(&phi);
                        *reinterpret_cast<uint2 *>(lds + trow * BN + (epi_swz<CH>(trow, tcol >> 3) << 3) + (4 * h)) = w;
                    }
                }
            }
            barrier_keep_loads_lds();
            bf16_t *Dy = static_cast<bf16_t *>(D);
#pragma unroll 4
            for (int u = 0; u < BM * CH / NTH; ++u) {
                const int idx = tid + u * NTH, r = idx / CH, c = idx % CH;
                const uint4 v = *reinterpret_cast<const uint4 *>(lds + r * BN + (epi_swz<CH>(r, c) << 3));
                if (r < rows_valid && c * 8 < cols_valid)
                    *reinterpret_cast<uint4 *>(Dy + (grow0 + r) * N + col0 + c * 8) = v;
            }
        }
    }
    wait_vmcnt<0>();
}

// ------------------------------------------------------------------ weight gradients, large tiles

// D[e][p][q] = sum over the filled rows r < fill[e] of X[e*C + r][p] * Y[e*C + r][q]
// (fp32), and with colsum also colsum[e][p] = sum_r X[e*C + r][p]: the weight
// and bias gradients of one expert layer (X = the layer's output gradient, Y =
// its input). Both operands are read n-contiguous, so their tiles land in LDS
// as [64 rows][BM or BN] in the transposed swizzle and every MFMA operand comes
// from transposing reads. Loads are raw-buffer direct loads whose range ends at
// the expert's last filled row: rows past it read as zero, so the last, partial
// K step needs no masking. Same ping-pong K loop as the row-grouped kernel;
// persistent workgroups over the E * ceil(P/BM) * ceil(Q/BN) tiles, in
// XCD-contiguous ranges. The bias gradient is summed from the X fragments of
// the first column tile.
template <int BN, int KB, int NW>
__device__ __forceinline__ void buf_tile_mn(i32x4_t rs, int ld, int cols_valid, int k0, bf16_t *lds,
                                            int wave, int lane) {
    constexpr int CPR = BN / 8;   // chunks per k row
    constexpr int RPI = 64 / CPR; // k rows per wavefront instruction
    static_assert(CPR >= 16 && KB % (NW * RPI) == 0, "n-contiguous tile shape");
#pragma unroll
    for (int j = 0; j < KB / (NW * RPI); ++j) {
        const int rb = (j * NW + wave) * RPI;
        const int row = rb + lane / CPR;
        const int c = min((lane % CPR) ^ (4 * (row & 3)), cols_valid / 8 - 1);  // chunk stored at this slot
        const int voff = ((k0 + row) * ld + c * 8) * 2;
        dma16_buf(rs, static_cast<uint32_t>(voff), lds + rb * BN);
    }
}

// Raw buffer resource over [base, base + bytes): loads past the end return zero.
// Words: base address (low 32 bits; high 16 bits with stride 0), the range in
// bytes, and the flags word 0x00020000.
__device__ __forceinline__ i32x4_t raw_rsrc(const bf16_t *base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4_t{static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>(static_cast<uint32_t>(a >> 32) & 0xFFFFu),
                   static_cast<int>(bytes), 0x00020000};
}

// First tile of the weight-gradient tile list (expert-major, per_e tiles per
// expert) at which cumulative work reaches t. A tile of expert e costs
// w_e = ceil(fill[e] / KB) + 1 units (its K steps and its store); cw_e is the
// work of the experts before e. The list is cut at work t, so that the 8 XCDs
// get equal work rather than equal tile counts: with uneven fills (a skewed
// router) equal tile counts leave one XCD with half again the mean work.
// Computed by every wavefront for itself; every lane returns the same value.
__device__ __forceinline__ int kgrad_cut(const int32_t *fill, int E, int per_e, int KB, int64_t t) {
    const int lane = threadIdx.x & 63;
    int64_t base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        const int64_t w = e < E ? static_cast<int64_t>((fill[e] + KB - 1) / KB + 1) : 0;
        int64_t inc = w * per_e;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int64_t o = __shfl_up(inc, off, 64);
            if (lane >= off) inc += o;
        }
        // the expert whose work range [cw_e, cw_e + W_e) holds t
        const uint64_t hit = __ballot(e < E && base + inc > t);
        if (hit != 0ull) {
            const int l = __ffsll(static_cast<long long>(hit)) - 1;
            const int64_t we = __shfl(w, l, 64);
            const int64_t cw = base + __shfl(inc, l, 64) - we * per_e;
            const int u = static_cast<int>(min<int64_t>((t - cw + we - 1) / we, per_e));
            // a cut within an eighth of an expert's tiles of the expert's first or last
            // tile moves to that boundary: with even fills every XCD then keeps whole
            // experts (their operands shared in its L2), as an equal count would
            const int snap = u * 8 <= per_e ? 0 : ((per_e - u) * 8 <= per_e ? per_e : u);
            return __builtin_amdgcn_readfirstlane((e0 + l) * per_e + snap);
        }
        base += __shfl(inc, 63, 64);
    }
    return E * per_e;  // t at or past the total work
}

// Total work of the weight-gradient tile list (units as kgrad_cut), in every lane.
__device__ __forceinline__ int64_t kgrad_work(const int32_t *fill, int E, int per_e, int KB) {
    const int lane = threadIdx.x & 63;
    int64_t total = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
        const int e = e0 + lane;
        int64_t v = e < E ? static_cast<int64_t>((fill[e] + KB - 1) / KB + 1) * per_e : 0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
        total += v;
    }
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(total));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(total >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int BM, int BN, int NTH>
__global__ __launch_bounds__(NTH, (4 * (BM + BN) * kBigKB * 2 <= 160 * 1024 ? 2 : 1)) void kgrad_gemm_big(const bf16_t *__restrict__ X, const bf16_t *__restrict__ Y,
                                                       float *__restrict__ D, int P, int Q, int E,
                                                       const int32_t *__restrict__ fill,
                                                       const int32_t *__restrict__ cap,
                                                       float *__restrict__ colsum) {
    extern __shared__ __align__(16) bf16_t lds[];
    constexpr int KB = kBigKB, S = KB / 16;
    constexpr int NW = NTH / 64, WGC = NW / 2;
    constexpr int TM = BM / 64, TN = BN / (32 * WGC);
    static_assert(TN >= 1 && BN % (32 * WGC) == 0, "wavefront columns must be whole 32-wide blocks");
    constexpr int STAGE = (BM + BN) * KB;
    const int tp = (P + BM - 1) / BM, tq = (Q + BN - 1) / BN;
    const int per_e = tp * tq;
    const int x = blockIdx.x % kXcds, nb = gridDim.x / kXcds;
    // XCD x takes the tiles of the x-th eighth of the work (see kgrad_cut)
    const int64_t work = kgrad_work(fill, E, per_e, KB);
    const int start = kgrad_cut(fill, E, per_e, KB, work * x / kXcds);
    const int end = kgrad_cut(fill, E, per_e, KB, work * (x + 1) / kXcds);
    const int C = *cap;
    // the wavefront index as a scalar: the tile offsets and LDS addresses derived
    // from it stay in SGPRs rather than taking VGPRs from the accumulators
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wr0 = (wave / WGC) * (BM / 2), wc0 = (wave % WGC) * (BN / WGC);
    for (int L = start + static_cast<int>(blockIdx.x) / kXcds; L < end; L += nb) {
        const int e = L / per_e, u = L - e * per_e;
        constexpr int GK = BM >= 256 ? kGroupKgrad : kGroupM;  // the size measured for each tile shape
        const int grp = u / (GK * tq);
        const int gm = min(GK, tp - grp * GK);
        const int within = u - grp * GK * tq;
        const int pt = grp * GK + within % gm, qt = within / gm;
        const int p0 = pt * BM, q0 = qt * BN;
        const int pv = min(BM, P - p0), qv = min(BN, Q - q0);
        const int rows = fill[e];
        const int nk = (rows + KB - 1) / KB;
        const int64_t r0 = static_cast<int64_t>(e) * C;
        const i32x4_t rx = raw_rsrc(X + r0 * P + p0, static_cast<uint32_t>((rows * P - p0) * 2));
        const i32x4_t ry = raw_rsrc(Y + r0 * Q + q0, static_cast<uint32_t>((rows * Q - q0) * 2));
        const bool col_sums = colsum != nullptr && qt == 0 && (wave % WGC) == 0;

        f32x16 acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        float csum[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) csum[i] = 0.f;

        barrier_keep_loads_lds();  // the previous tile's LDS reads are complete in every wavefront
        if (nk > 0) {
            buf_tile_mn<BM, KB, NW>(rx, P, pv, 0, lds, wave, lane);
            buf_tile_mn<BN, KB, NW>(ry, Q, qv, 0, lds + BM * KB, wave, lane);
            if (nk > 1) {
                buf_tile_mn<BM, KB, NW>(rx, P, pv, KB, lds + STAGE, wave, lane);
                buf_tile_mn<BN, KB, NW>(ry, Q, qv, KB, lds + STAGE + BM * KB, wave, lane);
                wait_vmcnt<(BM + BN) * KB / 8 / NTH>();
            } else {
                wait_vmcnt<0>();
            }
            barrier_keep_loads();
            bf16x8 fx[2][TM], fy[2][TN];
            frag_b_mn<TM, BM>(lds, 0, fx[0], wr0, lane);
            frag_b_mn<TN, BN>(lds + BM * KB, 0, fy[0], wc0, lane);
            auto colsum_add = [&](const bf16x8 (&f)[TM]) {
                if (!col_sums) return;
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int v = 0; v < 8; ++v) csum[i] += static_cast<float>(f[i][v]);
            };
            for (int t = 0; t < nk; ++t) {
                const bf16_t *scur = lds + (t & 1) * STAGE;
#pragma unroll
                for (int kk = 0; kk < S - 1; ++kk) {
                    const int nx = (kk + 1) & 1;
                    frag_b_mn<TM, BM>(scur, kk + 1, fx[nx], wr0, lane);
                    frag_b_mn<TN, BN>(scur + BM * KB, kk + 1, fy[nx], wc0, lane);
                    mfma_slice<TM, TN>(fx[kk & 1], fy[kk & 1], acc);
                    slice_schedule<TM, TN>();
                    colsum_add(fx[kk & 1]);
                }
                wait_vmcnt<0>();  // this wavefront's loads of stage t+1 have landed
                barrier_keep_loads_lds();
                if (t + 2 < nk) {
                    bf16_t *sn = lds + (t & 1) * STAGE;
                    buf_tile_mn<BM, KB, NW>(rx, P, pv, (t + 2) * KB, sn, wave, lane);
                    buf_tile_mn<BN, KB, NW>(ry, Q, qv, (t + 2) * KB, sn + BM * KB, wave, lane);
                }
                const bf16_t *snext = lds + ((t + 1) & 1) * STAGE;
                frag_b_mn<TM, BM>(snext, 0, fx[S & 1], wr0, lane);
                frag_b_mn<TN, BN>(snext + BM * KB, 0, fy[S & 1], wc0, lane);
                mfma_slice<TM, TN>(fx[(S - 1) & 1], fy[(S - 1) & 1], acc);
                slice_schedule<TM, TN>();
                colsum_add(fx[(S - 1) & 1]);
            }
        }
        // Output through LDS, in two halves of BM/2 rows (the fp32 tile is twice
        // the ring): the wavefronts owning the half write their accumulators as
        // a row-major [BM/2][BN] fp32 tile, 16-byte chunk c of row r at slot
        // c ^ (r mod CH), and every thread then stores whole rows. Lane l holds,
        // per 32 x 32 block, p = wr0 + 32 i + (l mod 32) and q = wc0 + 32 j +
        // 8 q' + 4 (l / 32) .. +3 (one chunk).
        float *De = D + static_cast<int64_t>(e) * P * Q;
        float *tile = reinterpret_cast<float *>(lds);
        constexpr int CH = BN / 4;  // 16-byte chunks per fp32 row
        static_assert((BM / 2) * BN * 4 <= 2 * STAGE * 2, "half the fp32 tile must fit in the ring");
        static_assert((BM / 2) * CH % NTH == 0, "output chunks must split evenly over the threads");
        barrier_keep_loads_lds();  // every wavefront is done with the ring
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            if (wr0 / (BM / 2) == half) {
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int r = wr0 - half * (BM / 2) + i * 32 + (lane & 31);
#pragma unroll
                    for (int j = 0; j < TN; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int c = (wc0 + j * 32 + 8 * q + 4 * (lane >> 5)) >> 2;
                            *reinterpret_cast<float4 *>(tile + r * BN + ((c ^ (r & (CH - 1))) << 2)) =
                                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                            acc[i][j][4 * q + 3]);
                        }
                }
            }
            barrier_keep_loads_lds();
#pragma unroll 4
            for (int u = 0; u < (BM / 2) * CH / NTH; ++u) {
                const int idx = tid + u * NTH, r = idx / CH, c = idx % CH;
                const float4 v = *reinterpret_cast<const float4 *>(tile + r * BN + ((c ^ (r & (CH - 1))) << 2));
                const int p = half * (BM / 2) + r;
                if (p < pv && c * 4 < qv)
                    *reinterpret_cast<float4 *>(De + static_cast<int64_t>(p0 + p) * Q + q0 + c * 4) = v;
            }
            if (half == 0) barrier_keep_loads_lds();  // read before the second half overwrites it
        }
        if (col_sums) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const float v = csum[i] + __shfl_down(csum[i], 32, 64);  // k 0-7 and 8-15 of each slice
                const int p = wr0 + i * 32 + lane;
                if (lane < 32 && p < pv) colsum[static_cast<int64_t>(e) * P + p0 + p] = v;
            }
        }
    }
    wait_vmcnt<0>();  // no direct-to-LDS write may land after the workgroup's LDS is released
}

// ------------------------------------------------------------------ K-grouped bf16 GEMM (weight gradients)

__global__ __launch_bounds__(NT) void kgroup_gemm_bf16(const bf16_t *__restrict__ A, const bf16_t *__restrict__ B,
                                                       float *__restrict__ D, int Mo, int No,
                                                       const int32_t *__restrict__ fill,
                                                       const int32_t *__restrict__ cap, float *__restrict__ colsum) {
    __shared__ __align__(16) bf16_t smem[4 * kTileElems];
    const int g = blockIdx.z;
    const int C = *cap;
    const int kv = fill[g];
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, wm = wave >> 1, wn = wave & 1;
    const int m_valid = min(BM, Mo - m0), n_valid = min(BN, No - n0);
    const bf16_t *Ab = A + static_cast<int64_t>(g) * C * Mo + m0;
    const bf16_t *Bb = B + static_cast<int64_t>(g) * C * No + n0;
    const bool do_colsum = colsum != nullptr && blockIdx.x == 0;

    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    float cs = 0.f;

    const int nk = (kv + BK - 1) / BK;
    MNMajorTile ta, tb;
    if (nk > 0) {
        ta.load(Ab, Mo, m_valid, kv, 0, tid);
        tb.load(Bb, No, n_valid, kv, 0, tid);
        ta.store(SA(0), tid);
        tb.store(SB(0), tid);
    }
    __syncthreads();
    for (int t = 0; t < nk; ++t) {
        const int cur = t & 1;
        const bool more = t + 1 < nk;
        if (more) {
            ta.load(Ab, Mo, m_valid, kv, (t + 1) * BK, tid);
            tb.load(Bb, No, n_valid, kv, (t + 1) * BK, tid);
        }
        mma_step(SA(cur), SB(cur), acc, wm, wn, lane);
        if (do_colsum && tid < BM) {
#pragma unroll 8
            for (int kk = 0; kk < BK; ++kk) cs += bf16_to_f32(SA(cur)[swz(tid, kk)]);
        }
        if (more) {
            ta.store(SA(cur ^ 1), tid);
            tb.store(SB(cur ^ 1), tid);
        }
        __syncthreads();
    }

    float *st = reinterpret_cast<float *>(smem) + wave * 64 * 64;
    stage_acc(st, acc, lane);
    __syncthreads();
    for (int i = 0; i < 8; ++i) {
        const int c = lane + 64 * i, r = c >> 3, cc = c & 7;
        const int trow = wm * 64 + r, tcol = wn * 64 + cc * 8;
        if (trow >= m_valid || tcol >= n_valid) continue;
        float *dst = D + (static_cast<int64_t>(g) * Mo + m0 + trow) * No + n0 + tcol;
        *reinterpret_cast<float4 *>(dst) = *reinterpret_cast<const float4 *>(st + r * 64 + cc * 8);
        *reinterpret_cast<float4 *>(dst + 4) = *reinterpret_cast<const float4 *>(st + r * 64 + cc * 8 + 4);
    }
    if (do_colsum && tid < m_valid) colsum[static_cast<int64_t>(g) * Mo + m0 + tid] = cs;
}

#undef SA
#undef SB

// ------------------------------------------------------------------ fp32 SIMT GEMM

// Generic strided grouped GEMM in fp32 for MOE_DT_F32:
//   D[g](i, n) = sum_kk A[g](i, kk) * B[g](n, kk),
// group g's base offsets are g * (gfix + C * gcap) elements. Row-grouped mode:
// i < fill[g], kk < K. K-grouped mode: i < rows, kk < fill[g].
struct SimtArgs {
    const float *A; int64_t a_si, a_sk, a_gfix, a_gcap;
    const float *B; int64_t b_sn, b_sk, b_gfix, b_gcap;
    float *D; int64_t d_si, d_gfix, d_gcap;
    int rows, N, K, kgrouped;
    const int32_t *fill; const int32_t *cap;
    const float *bias;       // [g*N + n] or null
    const float *aux;        // DACT: pre, indexed like D
    float *pre_out;          // FC1: pre, indexed like D
    float *colsum;           // K-grouped: sum_kk A(i, kk) -> colsum[g*rows + i]
};

template <int EPI, int ACT>
__global__ __launch_bounds__(256) void simt_gemm_f32(SimtArgs p) {
    constexpr int T = 64, TK = 16;
    __shared__ float As[TK][T + 1], Bs[TK][T + 1];
    const int g = blockIdx.z;
    const int C = *p.cap;
    const int rows = p.kgrouped ? p.rows : p.fill[g];
    const int K = p.kgrouped ? p.fill[g] : p.K;
    const int i0 = blockIdx.y * T, n0 = blockIdx.x * T;
    if (i0 >= rows) return;
    const float *A = p.A + g * (p.a_gfix + static_cast<int64_t>(C) * p.a_gcap);
    const float *B = p.B + g * (p.b_gfix + static_cast<int64_t>(C) * p.b_gcap);
    const int64_t dbase = g * (p.d_gfix + static_cast<int64_t>(C) * p.d_gcap);
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
    float acc[4][4] = {};
    float cs = 0.f;
    const bool do_colsum = p.colsum != nullptr && blockIdx.x == 0;
    for (int k0 = 0; k0 < K; k0 += TK) {
        for (int e = threadIdx.x; e < TK * T; e += 256) {
            const int kk = e / T, r = e % T;
            const bool ka = k0 + kk < K;
            As[kk][r] = (ka && i0 + r < rows) ? A[(i0 + r) * p.a_si + static_cast<int64_t>(k0 + kk) * p.a_sk] : 0.f;
            Bs[kk][r] = (ka && n0 + r < p.N) ? B[(n0 + r) * p.b_sn + static_cast<int64_t>(k0 + kk) * p.b_sk] : 0.f;
        }
        __syncthreads();
        if (do_colsum && threadIdx.x < T)
            for (int kk = 0; kk < TK; ++kk) cs += As[kk][threadIdx.x];
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], b[4];
            for (int u = 0; u < 4; ++u) { a[u] = As[kk][ty * 4 + u]; b[u] = Bs[kk][tx * 4 + u]; }
            for (int u = 0; u < 4; ++u)
                for (int w = 0; w < 4; ++w) acc[u][w] = fmaf(a[u], b[w], acc[u][w]);
        }
        __syncthreads();
    }
    if (do_colsum && threadIdx.x < T && i0 + threadIdx.x < rows) p.colsum[static_cast<int64_t>(g) * p.rows + i0 + threadIdx.x] = cs;
    for (int u = 0; u < 4; ++u) {
        const int i = i0 + ty * 4 + u;
        if (i >= rows) continue;
        for (int w = 0; w < 4; ++w) {
            const int n = n0 + tx * 4 + w;
            if (n >= p.N) continue;
            float v = acc[u][w];
            const int64_t off = dbase + static_cast<int64_t>(i) * p.d_si + n;
            if constexpr (EPI == EPI_FC1 || EPI == EPI_FC2)
                if (p.bias != nullptr) v += p.bias[static_cast<int64_t>(g) * p.N + n];
            if constexpr (EPI == EPI_FC1) {
                if (p.pre_out != nullptr) p.pre_out[off] = v;
                v = act_f<ACT>(v);
            }
            if constexpr (EPI == EPI_DACT) v *= act_grad_f<ACT>(p.aux[off]);
            p.D[off] = v;
        }
    }
}

template <int EPI>
hipError_t simt_launch(const SimtArgs &a, int act, int rows_bound, int E, hipStream_t st) {
    const dim3 grid((a.N + 63) / 64, (rows_bound + 63) / 64, E);
    if (act == MOE_ACT_GELU) hipLaunchKernelGGL((simt_gemm_f32<EPI, MOE_ACT_GELU>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((simt_gemm_f32<EPI, MOE_ACT_RELU>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <bool B_KMAJ, int EPI>
hipError_t rows_launch(int act, const void *A, const void *B, void *D, int N, int K, int cmax, int E,
                       const int32_t *fill, const int32_t *cap, const void *bias, const void *aux, void *pre_out,
                       hipStream_t st) {
    const dim3 grid((N + BN - 1) / BN, (cmax + BM - 1) / BM, E);
    auto a = static_cast<const bf16_t *>(A);
    auto b = static_cast<const bf16_t *>(B);
    auto d = static_cast<bf16_t *>(D);
    auto bi = static_cast<const bf16_t *>(bias);
    auto ax = static_cast<const bf16_t *>(aux);
    auto po = static_cast<bf16_t *>(pre_out);
    if (act == MOE_ACT_GELU)
        hipLaunchKernelGGL((rows_gemm_bf16<B_KMAJ, EPI, MOE_ACT_GELU>), grid, dim3(NT), 0, st, a, b, d, N, K, fill,
                           cap, bi, ax, po);
    else
        hipLaunchKernelGGL((rows_gemm_bf16<B_KMAJ, EPI, MOE_ACT_RELU>), grid, dim3(NT), 0, st, a, b, d, N, K, fill,
                           cap, bi, ax, po);
    return hipGetLastError();
}

// Workgroups that fit on the device at once (a multiple of the XCD count).
static int resident_blocks(int per_cu) {
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev] = n;
    }
    return ((cus[dev] * per_cu + kXcds - 1) / kXcds) * kXcds;
}

template <int BM, int BN, int NTH, int EPI, bool BMN = false, int WR = 2, bool WQ = false>
hipError_t big_launch(int act, const void *A, const void *B, void *D, int N, int K, int E, const int32_t *fill,
                      const int32_t *cap, const void *bias, void *pre_out, hipStream_t st,
                      const void *aux = nullptr, int s0 = 0, int s1 = 0x7FFFFFFF, const uint8_t *Bsc = nullptr,
                      const float *Bg = nullptr) {
    constexpr int lds = big_lds_bytes<BM, BN, WQ>();
    constexpr int per_cu = (160 * 1024) / lds >= 2 ? 2 : 1;  // the kernel's launch bounds match
    const dim3 grid(resident_blocks(per_cu));
    auto a = static_cast<const bf16_t *>(A);
    auto b = static_cast<const bf16_t *>(B);
    auto d = static_cast<bf16_t *>(D);
    auto bi = static_cast<const bf16_t *>(bias);
    auto po = static_cast<bf16_t *>(pre_out);
    auto ax = static_cast<const bf16_t *>(aux);
    if (act == MOE_ACT_GELU) {
        auto k = rows_gemm_big<BM, BN, NTH, EPI, MOE_ACT_GELU, BMN, WR, WQ>;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k, grid, dim3(NTH), lds, st, a, b, d, N, K, E, fill, cap, bi, po, ax, s0, s1, Bsc, Bg);
    } else {
        auto k = rows_gemm_big<BM, BN, NTH, EPI, MOE_ACT_RELU, BMN, WR, WQ>;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k, grid, dim3(NTH), lds, st, a, b, d, N, K, E, fill, cap, bi, po, ax, s0, s1, Bsc, Bg);
    }
    return hipGetLastError();
}

// Forward-product tile configuration. 256 x 256 tiles (eight wavefronts, one
// workgroup per CU) halve the operand traffic per flop of 128 x 128 tiles (four
// wavefronts, two workgroups per CU), and win where there are enough of them:
// short-K products (K <= 1024) lose, because a tile's fixed cost (prologue
// loads and the epilogue) is a large share of its time and two independent
// workgroups per CU overlap one's epilogue with the other's MFMAs; and so do
// products with fewer than 128 large tiles (half the CUs), where 128 x 128
// tiles keep four times as many workgroups busy (measured: top-1 fc2 at S=4096,
// M=1024, E=8, H=4096, 64 large tiles, 86 -> 55 us; the top-2 layer's 128 large
// tiles still favour 256 x 256, 96 vs 105 us). Between 256 x 256 and 192 x 256
// tiles (eight wavefronts of 96 x 64) the choice counts the rounds of the
// persistent grid each needs at an even fill per expert: a tile is computed for
// all its rows, filled or not, and the last round runs on part of the CUs, so
// where 192-row tiles take as many rounds they finish sooner (a round costs
// about 192/256 of the time at ~8% lower throughput per flop; measured: fc2 of
// the top-2 layer above, 144 large tiles or 192 of 192 rows, 95 -> 82 us).
// rows_hint bounds the filled rows over all experts (k*S, or S for a dense
// product). MOE_GEMM_CFG overrides the choice for tuning (1 = 256 x 256,
// 2 = 256 x 128, 3 = 128 x 128, 4 = 192 x 256).
static int gemm_cfg_override() {
    static const int v = [] {
        const char *e = getenv("MOE_GEMM_CFG");
        return e ? atoi(e) : 0;
    }();
    return v;
}

// Rounds of a persistent grid of `slots` workgroups over E experts' row tiles of
// BMv rows and nx column tiles, at an even fill f per expert; fills vary around
// f, so an expert is taken to need f / BMv + 1/2 row tiles, rounded up.
static int64_t tile_rounds(int64_t f, int BMv, int64_t nx, int E, int64_t slots) {
    const int64_t rt = (2 * f + BMv + 2 * BMv - 1) / (2 * BMv);
    return (E * rt * nx + slots - 1) / slots;
}

// one workgroup per CU: 256 x 256 tiles, or 192 x 256 where their rounds cost less
static int wide_cfg(int N, int64_t rows_hint, int E) {
    const int64_t f = (rows_hint + E - 1) / E, cus = resident_blocks(1);
    const int64_t nx = (N + 255) / 256;
    const int64_t r256 = tile_rounds(f, 256, nx, E, cus), r192 = tile_rounds(f, 192, nx, E, cus);
    return r192 * 192 * 100 < r256 * 256 * 92 ? 4 : 1;
}

static int default_cfg(int N, int K, int64_t rows_hint, int E) {
    const int64_t big_tiles = ((rows_hint + 255) / 256) * ((N + 255) / 256);
    const int64_t f = (rows_hint + E - 1) / E, cus = resident_blocks(1);
    if (K <= 1024 || big_tiles < 128) {
        // two workgroups per CU: 128 x 128 tiles, or 192 x 128 where they take
        // fewer rounds (each costs about 1.5 of a 128-row round)
        const int64_t n128 = (N + 127) / 128;
        const int64_t r128 = tile_rounds(f, 128, n128, E, 2 * cus), r192 = tile_rounds(f, 192, n128, E, 2 * cus);
        return r192 * 3 < r128 * 2 ? 5 : 3;
    }
    return wide_cfg(N, rows_hint, E);
}

// Backward data products, weights read n-contiguous: same tile choice as the
// forward products.
template <int EPI>
hipError_t bwd_data_launch(int act, const void *A, const void *B, void *D, int N, int K, int E, const int32_t *fill,
                           const int32_t *cap, const void *aux, int64_t rows_hint, hipStream_t st) {
    int cfg = gemm_cfg_override();
    if (cfg < 1 || cfg > 5) cfg = default_cfg(N, K, rows_hint, E);
    switch (cfg) {
    case 1: return big_launch<256, 256, 512, EPI, true>(act, A, B, D, N, K, E, fill, cap, nullptr, nullptr, st, aux);
    case 2: return big_launch<256, 128, 256, EPI, true>(act, A, B, D, N, K, E, fill, cap, nullptr, nullptr, st, aux);
    case 4: return big_launch<192, 256, 512, EPI, true>(act, A, B, D, N, K, E, fill, cap, nullptr, nullptr, st, aux);
    case 5: return big_launch<192, 128, 256, EPI, true>(act, A, B, D, N, K, E, fill, cap, nullptr, nullptr, st, aux);

    default: return big_launch<128, 128, 256, EPI, true>(act, A, B, D, N, K, E, fill, cap, nullptr, nullptr, st, aux);
    }
}

template <int EPI>
hipError_t fwd_launch(int act, const void *A, const void *B, void *D, int N, int K, int64_t rows_hint, int E,
                      const int32_t *fill, const int32_t *cap, const void *bias, void *pre_out, hipStream_t st,
                      int s0 = 0, int s1 = 0x7FFFFFFF) {
    int cfg = gemm_cfg_override();
    if (cfg < 1 || cfg > 5) cfg = default_cfg(N, K, rows_hint, E);
    switch (cfg) {
    case 1: return big_launch<256, 256, 512, EPI>(act, A, B, D, N, K, E, fill, cap, bias, pre_out, st, nullptr, s0, s1);
    case 2: return big_launch<256, 128, 256, EPI>(act, A, B, D, N, K, E, fill, cap, bias, pre_out, st, nullptr, s0, s1);
    case 4: return big_launch<192, 256, 512, EPI>(act, A, B, D, N, K, E, fill, cap, bias, pre_out, st, nullptr, s0, s1);
    case 5: return big_launch<192, 128, 256, EPI>(act, A, B, D, N, K, E, fill, cap, bias, pre_out, st, nullptr, s0, s1);

    default:
        return big_launch<128, 128, 256, EPI>(act, A, B, D, N, K, E, fill, cap, bias, pre_out, st, nullptr, s0, s1);
    }
}

// Forward products with NVFP4 weights: eight-wavefront tiles 256 wide at every
// size. Their code slots keep the smaller tiles to one workgroup per CU, and the
// expansion (one chunk per thread per slice) costs least per MFMA on the wide
// tiles (gated S=4096 fc1 / fc2: 192 x 256 106 / 95 us, 128 x 128 118 / 131,
// 192 x 128 139 / 131). Of MOE_GEMM_CFG, 1 and 4 are honoured.
template <int EPI>
hipError_t fwd_launch_nvfp4(int act, const void *A, const uint8_t *Bcodes, const uint8_t *Bsc, const float *Bg,
                            void *D, int N, int K, int64_t rows_hint, int E, const int32_t *fill, const int32_t *cap,
                            const void *bias, void *pre_out, hipStream_t st) {
    int cfg = gemm_cfg_override();
    if (cfg != 1 && cfg != 4) cfg = wide_cfg(N, rows_hint, E);
    const int s0 = 0, s1 = 0x7FFFFFFF;
    if (cfg == 4)
        return big_launch<192, 256, 512, EPI, false, 2, true>(act, A, Bcodes, D, N, K, E, fill, cap, bias, pre_out, st,
                                                              nullptr, s0, s1, Bsc, Bg);
    return big_launch<256, 256, 512, EPI, false, 2, true>(act, A, Bcodes, D, N, K, E, fill, cap, bias, pre_out, st,
                                                          nullptr, s0, s1, Bsc, Bg);
}

// Weight gradients: the large-tile kernel when one expert's rows of either
// operand span less than 2 GiB (its raw-buffer offsets are 32-bit), else the
// register-staged kernel below. The reduction runs over an expert's rows: up to
// about 1024 of them (16 K steps) the fp32 tile's store is a large share of a
// tile, and 128 x 128 tiles at two workgroups per CU overlap one's stores with
// the other's MFMAs (the bench layer's backward: 500 -> 488 us); with more rows
// 256 x 256 tiles win (S=32768, E=128, k=8: 19.5 vs 20.7 ms), unless there are
// fewer of them than CUs (one expert's gradients, as Residual-MoE's dense
// branch: four times as many 128 x 128 tiles). MOE_KGRAD_CFG (1 = 256 x 256,
// 2 = 128 x 128) overrides the choice for tuning.
hipError_t kgroup_launch(const void *A, const void *B, float *D, int Mo, int No, int E, const int32_t *fill,
                         const int32_t *cap, float *colsum, int32_t cmax, int64_t rows_hint, hipStream_t st) {
    // the last K step reads up to 63 rows past the expert's fill (they read as zero)
    if (static_cast<int64_t>(cmax + 64) * std::max(Mo, No) * 2 < (int64_t(1) << 31)) {
        static const int kc = [] {
            const char *v = getenv("MOE_KGRAD_CFG");
            return v ? atoi(v) : 0;
        }();
        const int64_t big_tiles = static_cast<int64_t>(E) * ((Mo + 255) / 256) * ((No + 255) / 256);
        const bool small = kc == 2 || (kc != 1 && (rows_hint <= 1024LL * E || big_tiles < resident_blocks(1)));
        if (small) {
            constexpr int lds = 2 * (128 + 128) * kBigKB * 2;
            auto k = kgrad_gemm_big<128, 128, 256>;
            static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                               hipFuncAttributeMaxDynamicSharedMemorySize, lds);
            if (attr != hipSuccess) return attr;
            hipLaunchKernelGGL(k, dim3(resident_blocks(2)), dim3(256), lds, st, static_cast<const bf16_t *>(A),
                               static_cast<const bf16_t *>(B), D, Mo, No, E, fill, cap, colsum);
            return hipGetLastError();
        }
        constexpr int lds = 2 * (256 + 256) * kBigKB * 2;
        auto k = kgrad_gemm_big<256, 256, 512>;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k, dim3(resident_blocks(1)), dim3(512), lds, st, static_cast<const bf16_t *>(A),
                           static_cast<const bf16_t *>(B), D, Mo, No, E, fill, cap, colsum);
        return hipGetLastError();
    }
    const dim3 grid((No + BN - 1) / BN, (Mo + BM - 1) / BM, E);
    hipLaunchKernelGGL(kgroup_gemm_bf16, grid, dim3(NT), 0, st, static_cast<const bf16_t *>(A),
                       static_cast<const bf16_t *>(B), D, Mo, No, fill, cap, colsum);
    return hipGetLastError();
}

}  // namespace

// Upper bound of the filled rows over all experts: every route kept, at most E*cmax.
static int64_t rows_hint(const moe_shape &s, int32_t cmax) {
    return std::min<int64_t>(static_cast<int64_t>(s.k) * s.S, static_cast<int64_t>(s.E) * cmax);
}

hipError_t launch_fc1(const moe_shape &s, const void *buf, const void *W1, const void *b1, const int32_t *fill,
                      const int32_t *cap, void *pre, void *h, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16)
        return fwd_launch<EPI_FC1>(s.act, buf, W1, h, H, M, rows_hint(s, cmax), E, fill, cap, b1, pre, st);
    SimtArgs a{};
    a.A = static_cast<const float *>(buf); a.a_si = M; a.a_sk = 1; a.a_gfix = 0; a.a_gcap = M;
    a.B = static_cast<const float *>(W1); a.b_sn = M; a.b_sk = 1; a.b_gfix = static_cast<int64_t>(H) * M; a.b_gcap = 0;
    a.D = static_cast<float *>(h); a.d_si = H; a.d_gfix = 0; a.d_gcap = H;
    a.N = H; a.K = M; a.kgrouped = 0; a.fill = fill; a.cap = cap;
    a.bias = static_cast<const float *>(b1); a.pre_out = static_cast<float *>(pre);
    return simt_launch<EPI_FC1>(a, s.act, cmax, E, st);
}

// The expert FFN on the capacity slots [s0, s1) of every expert (bf16 data).
hipError_t launch_ffn_window(const moe_shape &s, const void *buf, const void *W1, const void *b1, const void *W2,
                             const void *b2, const int32_t *fill, const int32_t *cap, void *pre, void *h, void *y,
                             int32_t cmax, int32_t s0, int32_t s1, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    const int64_t win = std::max<int64_t>(0, std::min<int64_t>(s1, cmax) - s0);
    const int64_t rh = std::min<int64_t>(static_cast<int64_t>(s.k) * s.S, static_cast<int64_t>(E) * win);
    hipError_t err = fwd_launch<EPI_FC1>(s.act, buf, W1, h, H, M, rh, E, fill, cap, b1, pre, st, s0, s1);
    if (err != hipSuccess) return err;
    return fwd_launch<EPI_FC2>(s.act, h, W2, y, M, H, rh, E, fill, cap, b2, nullptr, st, s0, s1);
}

hipError_t launch_fc2(const moe_shape &s, const void *h, const void *W2, const void *b2, const int32_t *fill,
                      const int32_t *cap, void *y, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16)
        return fwd_launch<EPI_FC2>(s.act, h, W2, y, M, H, rows_hint(s, cmax), E, fill, cap, b2, nullptr, st);
    SimtArgs b{};
    b.A = static_cast<const float *>(h); b.a_si = H; b.a_sk = 1; b.a_gfix = 0; b.a_gcap = H;
    b.B = static_cast<const float *>(W2); b.b_sn = H; b.b_sk = 1; b.b_gfix = static_cast<int64_t>(M) * H; b.b_gcap = 0;
    b.D = static_cast<float *>(y); b.d_si = M; b.d_gfix = 0; b.d_gcap = M;
    b.N = M; b.K = H; b.kgrouped = 0; b.fill = fill; b.cap = cap;
    b.bias = static_cast<const float *>(b2);
    return simt_launch<EPI_FC2>(b, s.act, cmax, E, st);
}

hipError_t launch_fc1_nvfp4(const moe_shape &s, const void *buf, const uint8_t *w1_codes, const uint8_t *w1_scales,
                            const float *w1_g, const void *b1, const int32_t *fill, const int32_t *cap, void *pre,
                            void *h, int32_t cmax, hipStream_t st) {
    return fwd_launch_nvfp4<EPI_FC1>(s.act, buf, w1_codes, w1_scales, w1_g, h, s.H, s.M, rows_hint(s, cmax), s.E, fill,
                                     cap, b1, pre, st);
}

hipError_t launch_fc2_nvfp4(const moe_shape &s, const void *h, const uint8_t *w2_codes, const uint8_t *w2_scales,
                            const float *w2_g, const void *b2, const int32_t *fill, const int32_t *cap, void *y,
                            int32_t cmax, hipStream_t st) {
    return fwd_launch_nvfp4<EPI_FC2>(s.act, h, w2_codes, w2_scales, w2_g, y, s.M, s.H, rows_hint(s, cmax), s.E, fill,
                                     cap, b2, nullptr, st);
}

template <int BM, int BN, int NTH, int EPI, int WFMT, bool BLK = false>
hipError_t mx_launch(int act, const uint8_t *A, const uint8_t *As, const uint8_t *B, const uint8_t *Bs, void *D,
                     uint8_t *Dsc, int N, int K, int E, const int32_t *fill, const int32_t *cap, const void *bias,
                     hipStream_t st) {
    constexpr int lds = mx_lds_bytes<BM, BN, WFMT, EPI, BLK>();
    // BLK's 256-row tiles need every register of a SIMD for one wavefront (their per-stage
    // partial sums); the 128 x 128 tiles fit two workgroups per CU
    constexpr int per_cu = ((!BLK || BM * BN <= 128 * 128) && (160 * 1024) / lds >= 2) ? 2 : 1;
    const dim3 grid(resident_blocks(per_cu));
    auto bi = static_cast<const bf16_t *>(bias);
    if (act == MOE_ACT_GELU) {
        auto k = rows_gemm_mx<BM, BN, NTH, EPI, MOE_ACT_GELU, WFMT, BLK>;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k, grid, dim3(NTH), lds, st, A, As, B, Bs, D, Dsc, N, K, E, fill, cap, bi);
    } else {
        auto k = rows_gemm_mx<BM, BN, NTH, EPI, MOE_ACT_RELU, WFMT, BLK>;
        static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void *>(k),
                                                           hipFuncAttributeMaxDynamicSharedMemorySize, lds);
        if (attr != hipSuccess) return attr;
        hipLaunchKernelGGL(k, grid, dim3(NTH), lds, st, A, As, B, Bs, D, Dsc, N, K, E, fill, cap, bi);
    }
    return hipGetLastError();
}

template <int EPI, int WFMT, bool BLK = false>
hipError_t mx_product(int act, const uint8_t *A, const uint8_t *As, const uint8_t *B, const uint8_t *Bs, void *D,
                      uint8_t *Dsc, int N, int K, int E, const int32_t *fill, const int32_t *cap, const void *bias,
                      int64_t rows_hint, hipStream_t st) {
    // 128 x 128 tiles by default: with 8-bit operands a tile moves half the LDS bytes per
    // flop of a bf16 one, and the 256 x 256 layout runs out of registers (MOE_GEMM_CFG
    // selects the others for measurement)
    (void)rows_hint;
    const int cfg = gemm_cfg_override();
    switch (cfg) {
    case 1: return mx_launch<256, 256, 512, EPI, WFMT, BLK>(act, A, As, B, Bs, D, Dsc, N, K, E, fill, cap, bias, st);
    case 2: return mx_launch<256, 128, 256, EPI, WFMT, BLK>(act, A, As, B, Bs, D, Dsc, N, K, E, fill, cap, bias, st);
    default: return mx_launch<128, 128, 256, EPI, WFMT, BLK>(act, A, As, B, Bs, D, Dsc, N, K, E, fill, cap, bias, st);
    }
}

hipError_t launch_fc1_mx(const moe_shape &s, int wfmt, const uint8_t *buf_codes, const uint8_t *buf_scales,
                         const uint8_t *w1_codes, const uint8_t *w1_scales, const void *b1, const int32_t *fill,
                         const int32_t *cap, uint8_t *h_codes, uint8_t *h_scales, int32_t cmax, hipStream_t st) {
    const int64_t rh = rows_hint(s, cmax);
    if (wfmt == kBlkFp8)
        return mx_product<EPI_FC1, kMxFp8, true>(s.act, buf_codes, buf_scales, w1_codes, w1_scales, h_codes, h_scales,
                                                 s.H, s.M, s.E, fill, cap, b1, rh, st);
    if (wfmt == kMxFp8)
        return mx_product<EPI_FC1, kMxFp8>(s.act, buf_codes, buf_scales, w1_codes, w1_scales, h_codes, h_scales, s.H,
                                           s.M, s.E, fill, cap, b1, rh, st);
    return mx_product<EPI_FC1, kMxFp4>(s.act, buf_codes, buf_scales, w1_codes, w1_scales, h_codes, h_scales, s.H, s.M,
                                       s.E, fill, cap, b1, rh, st);
}

hipError_t launch_fc2_mx(const moe_shape &s, int wfmt, const uint8_t *h_codes, const uint8_t *h_scales,
                         const uint8_t *w2_codes, const uint8_t *w2_scales, const void *b2, const int32_t *fill,
                         const int32_t *cap, void *y, int32_t cmax, hipStream_t st) {
    const int64_t rh = rows_hint(s, cmax);
    if (wfmt == kBlkFp8)
        return mx_product<EPI_FC2, kMxFp8, true>(s.act, h_codes, h_scales, w2_codes, w2_scales, y, nullptr, s.M, s.H,
                                                 s.E, fill, cap, b2, rh, st);
    if (wfmt == kMxFp8)
        return mx_product<EPI_FC2, kMxFp8>(s.act, h_codes, h_scales, w2_codes, w2_scales, y, nullptr, s.M, s.H, s.E,
                                           fill, cap, b2, rh, st);
    return mx_product<EPI_FC2, kMxFp4>(s.act, h_codes, h_scales, w2_codes, w2_scales, y, nullptr, s.M, s.H, s.E, fill,
                                       cap, b2, rh, st);
}

hipError_t launch_expert_ffn_mx(const moe_shape &s, int wfmt, const uint8_t *buf_codes, const uint8_t *buf_scales,
                                const uint8_t *w1_codes, const uint8_t *w1_scales, const void *b1,
                                const uint8_t *w2_codes, const uint8_t *w2_scales, const void *b2,
                                const int32_t *fill, const int32_t *cap, uint8_t *h_codes, uint8_t *h_scales, void *y,
                                int32_t cmax, hipStream_t st) {
    hipError_t err = launch_fc1_mx(s, wfmt, buf_codes, buf_scales, w1_codes, w1_scales, b1, fill, cap, h_codes,
                                   h_scales, cmax, st);
    if (err != hipSuccess) return err;
    return launch_fc2_mx(s, wfmt, h_codes, h_scales, w2_codes, w2_scales, b2, fill, cap, y, cmax, st);
}

// The four products of the FFN backward, one kernel each.
// dpre = (dy . W2[e]) * act'(pre): A = dy [rows][M], B = W2[e] read as [K=M][N=H]
hipError_t launch_fc2_bwd_data(const moe_shape &s, const void *dy, const void *W2, const void *pre,
                               const int32_t *fill, const int32_t *cap, void *dpre, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16)
        return bwd_data_launch<EPI_DACT>(s.act, dy, W2, dpre, H, M, E, fill, cap, pre, rows_hint(s, cmax), st);
    SimtArgs a{};  // B(n=h, kk=m) = W2[e][m][h]
    a.A = static_cast<const float *>(dy); a.a_si = M; a.a_sk = 1; a.a_gfix = 0; a.a_gcap = M;
    a.B = static_cast<const float *>(W2); a.b_sn = 1; a.b_sk = H; a.b_gfix = static_cast<int64_t>(M) * H; a.b_gcap = 0;
    a.D = static_cast<float *>(dpre); a.d_si = H; a.d_gfix = 0; a.d_gcap = H;
    a.N = H; a.K = M; a.kgrouped = 0; a.fill = fill; a.cap = cap; a.aux = static_cast<const float *>(pre);
    return simt_launch<EPI_DACT>(a, s.act, cmax, E, st);
}

// dW2[e] = dy^T h (+ db2 = column sums of dy)
hipError_t launch_fc2_wgrad(const moe_shape &s, const void *dy, const void *h, const int32_t *fill, const int32_t *cap,
                            float *dW2, float *db2, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16) return kgroup_launch(dy, h, dW2, M, H, E, fill, cap, db2, cmax, rows_hint(s, cmax), st);
    SimtArgs b{};  // dW2[e](m, h) = sum_j dy[j][m] h[j][h]
    b.A = static_cast<const float *>(dy); b.a_si = 1; b.a_sk = M; b.a_gfix = 0; b.a_gcap = M;
    b.B = static_cast<const float *>(h); b.b_sn = 1; b.b_sk = H; b.b_gfix = 0; b.b_gcap = H;
    b.D = dW2; b.d_si = H; b.d_gfix = static_cast<int64_t>(M) * H; b.d_gcap = 0;
    b.rows = M; b.N = H; b.kgrouped = 1; b.fill = fill; b.cap = cap; b.colsum = db2;
    return simt_launch<EPI_PLAIN>(b, s.act, M, E, st);
}

// dbuf = dpre . W1[e]: B = W1[e] read as [K=H][N=M]
hipError_t launch_fc1_bwd_data(const moe_shape &s, const void *dpre, const void *W1, const int32_t *fill,
                               const int32_t *cap, void *dbuf, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16)
        return bwd_data_launch<EPI_PLAIN>(s.act, dpre, W1, dbuf, M, H, E, fill, cap, nullptr, rows_hint(s, cmax), st);
    SimtArgs c{};  // B(n=m, kk=h) = W1[e][h][m]
    c.A = static_cast<const float *>(dpre); c.a_si = H; c.a_sk = 1; c.a_gfix = 0; c.a_gcap = H;
    c.B = static_cast<const float *>(W1); c.b_sn = 1; c.b_sk = M; c.b_gfix = static_cast<int64_t>(H) * M; c.b_gcap = 0;
    c.D = static_cast<float *>(dbuf); c.d_si = M; c.d_gfix = 0; c.d_gcap = M;
    c.N = M; c.K = H; c.kgrouped = 0; c.fill = fill; c.cap = cap;
    return simt_launch<EPI_PLAIN>(c, s.act, cmax, E, st);
}

// dW1[e] = dpre^T buf (+ db1 = column sums of dpre)
hipError_t launch_fc1_wgrad(const moe_shape &s, const void *dpre, const void *buf, const int32_t *fill,
                            const int32_t *cap, float *dW1, float *db1, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16)
        return kgroup_launch(dpre, buf, dW1, H, M, E, fill, cap, db1, cmax, rows_hint(s, cmax), st);
    SimtArgs d{};  // dW1[e](h, m) = sum_j dpre[j][h] buf[j][m]
    d.A = static_cast<const float *>(dpre); d.a_si = 1; d.a_sk = H; d.a_gfix = 0; d.a_gcap = H;
    d.B = static_cast<const float *>(buf); d.b_sn = 1; d.b_sk = M; d.b_gfix = 0; d.b_gcap = M;
    d.D = dW1; d.d_si = M; d.d_gfix = static_cast<int64_t>(H) * M; d.d_gcap = 0;
    d.rows = H; d.N = M; d.kgrouped = 1; d.fill = fill; d.cap = cap; d.colsum = db1;
    return simt_launch<EPI_PLAIN>(d, s.act, H, E, st);
}

// The FFN backward in the order that keeps operands cached: dW2 first, so that
// dbuf runs right after dpre is written (dpre's rows are still in the last-level
// cache); dbuf may alias dy, which is consumed by then.
hipError_t launch_expert_ffn_bwd(const moe_shape &s, const void *buf, const void *pre, const void *h, const void *W1,
                                 const void *W2, const int32_t *fill, const int32_t *cap, const void *dy, void *dpre,
                                 void *dbuf, float *dW1, float *db1, float *dW2, float *db2, int32_t cmax,
                                 hipStream_t st) {
    hipError_t err;
    if ((err = launch_fc2_wgrad(s, dy, h, fill, cap, dW2, db2, cmax, st)) != hipSuccess) return err;
    if ((err = launch_fc2_bwd_data(s, dy, W2, pre, fill, cap, dpre, cmax, st)) != hipSuccess) return err;
    if ((err = launch_fc1_bwd_data(s, dpre, W1, fill, cap, dbuf, cmax, st)) != hipSuccess) return err;
    return launch_fc1_wgrad(s, dpre, buf, fill, cap, dW1, db1, cmax, st);
}

}  // namespace moe
