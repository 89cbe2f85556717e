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
#include "moe_internal.h"

namespace moe {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

hipError_t kgroup_launch(const void *A, const void *B, float *D, int Mo, int No, int E, const int32_t *fill,
                         const int32_t *cap, float *colsum, hipStream_t st) {
    const dim3 grid((No + BN - 1) / BN, (Mo + BM - 1) / BM, E);
    hipLaunchKernelGGL(kgroup_gemm_bf16, grid, dim3(NT), 0, st, static_cast<const bf16_t *>(A),
                       static_cast<const bf16_t *>(B), D, Mo, No, fill, cap, colsum);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fc1(const moe_shape &s, const void *buf, const void *W1, const void *b1, const int32_t *fill,
                      const int32_t *cap, void *pre, void *h, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16)
        return rows_launch<true, EPI_FC1>(s.act, buf, W1, h, H, M, cmax, E, fill, cap, b1, nullptr, pre, st);
    SimtArgs a{};
    a.A = static_cast<const float *>(buf); a.a_si = M; a.a_sk = 1; a.a_gfix = 0; a.a_gcap = M;
    a.B = static_cast<const float *>(W1); a.b_sn = M; a.b_sk = 1; a.b_gfix = static_cast<int64_t>(H) * M; a.b_gcap = 0;
    a.D = static_cast<float *>(h); a.d_si = H; a.d_gfix = 0; a.d_gcap = H;
    a.N = H; a.K = M; a.kgrouped = 0; a.fill = fill; a.cap = cap;
    a.bias = static_cast<const float *>(b1); a.pre_out = static_cast<float *>(pre);
    return simt_launch<EPI_FC1>(a, s.act, cmax, E, st);
}

hipError_t launch_fc2(const moe_shape &s, const void *h, const void *W2, const void *b2, const int32_t *fill,
                      const int32_t *cap, void *y, int32_t cmax, hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    if (s.dtype == MOE_DT_BF16)
        return rows_launch<true, EPI_FC2>(s.act, h, W2, y, M, H, cmax, E, fill, cap, b2, nullptr, nullptr, st);
    SimtArgs b{};
    b.A = static_cast<const float *>(h); b.a_si = H; b.a_sk = 1; b.a_gfix = 0; b.a_gcap = H;
    b.B = static_cast<const float *>(W2); b.b_sn = H; b.b_sk = 1; b.b_gfix = static_cast<int64_t>(M) * H; b.b_gcap = 0;
    b.D = static_cast<float *>(y); b.d_si = M; b.d_gfix = 0; b.d_gcap = M;
    b.N = M; b.K = H; b.kgrouped = 0; b.fill = fill; b.cap = cap;
    b.bias = static_cast<const float *>(b2);
    return simt_launch<EPI_FC2>(b, s.act, cmax, E, st);
}

hipError_t launch_expert_ffn_bwd(const moe_shape &s, const void *buf, const void *pre, const void *h, const void *W1,
                                 const void *W2, const int32_t *fill, const int32_t *cap, void *dy, void *dpre,
                                 void *dbuf, float *dW1, float *db1, float *dW2, float *db2, int32_t cmax,
                                 hipStream_t st) {
    const int M = s.M, H = s.H, E = s.E;
    hipError_t err;
    if (s.dtype == MOE_DT_BF16) {
        // dpre = (dy . W2[e]) * act'(pre): A = dy [rows][M], B = W2[e] read as [K=M][N=H]
        if ((err = rows_launch<false, EPI_DACT>(s.act, dy, W2, dpre, H, M, cmax, E, fill, cap, nullptr, pre, nullptr,
                                                st)) != hipSuccess)
            return err;
        // dW2[e] = dy^T h (+ db2 = column sums of dy)
        if ((err = kgroup_launch(dy, h, dW2, M, H, E, fill, cap, db2, st)) != hipSuccess) return err;
        // dbuf = dpre . W1[e]: B = W1[e] read as [K=H][N=M]   (dbuf may alias dy: dy is consumed above)
        if ((err = rows_launch<false, EPI_PLAIN>(s.act, dpre, W1, dbuf, M, H, cmax, E, fill, cap, nullptr, nullptr,
                                                 nullptr, st)) != hipSuccess)
            return err;
        // dW1[e] = dpre^T buf (+ db1 = column sums of dpre)
        return kgroup_launch(dpre, buf, dW1, H, M, E, fill, cap, db1, st);
    }
    SimtArgs a{};  // dpre = (dy . W2) * act'(pre); B(n=h, kk=m) = W2[e][m][h]
    a.A = static_cast<const float *>(dy); a.a_si = M; a.a_sk = 1; a.a_gfix = 0; a.a_gcap = M;
    a.B = static_cast<const float *>(W2); a.b_sn = 1; a.b_sk = H; a.b_gfix = static_cast<int64_t>(M) * H; a.b_gcap = 0;
    a.D = static_cast<float *>(dpre); a.d_si = H; a.d_gfix = 0; a.d_gcap = H;
    a.N = H; a.K = M; a.kgrouped = 0; a.fill = fill; a.cap = cap; a.aux = static_cast<const float *>(pre);
    if ((err = simt_launch<EPI_DACT>(a, s.act, cmax, E, st)) != hipSuccess) return err;
    SimtArgs b{};  // dW2[e](m, h) = sum_j dy[j][m] h[j][h]
    b.A = static_cast<const float *>(dy); b.a_si = 1; b.a_sk = M; b.a_gfix = 0; b.a_gcap = M;
    b.B = static_cast<const float *>(h); b.b_sn = 1; b.b_sk = H; b.b_gfix = 0; b.b_gcap = H;
    b.D = dW2; b.d_si = H; b.d_gfix = static_cast<int64_t>(M) * H; b.d_gcap = 0;
    b.rows = M; b.N = H; b.kgrouped = 1; b.fill = fill; b.cap = cap; b.colsum = db2;
    if ((err = simt_launch<EPI_PLAIN>(b, s.act, M, E, st)) != hipSuccess) return err;
    SimtArgs c{};  // dbuf = dpre . W1; B(n=m, kk=h) = W1[e][h][m]
    c.A = static_cast<const float *>(dpre); c.a_si = H; c.a_sk = 1; c.a_gfix = 0; c.a_gcap = H;
    c.B = static_cast<const float *>(W1); c.b_sn = 1; c.b_sk = M; c.b_gfix = static_cast<int64_t>(H) * M; c.b_gcap = 0;
    c.D = static_cast<float *>(dbuf); c.d_si = M; c.d_gfix = 0; c.d_gcap = M;
    c.N = M; c.K = H; c.kgrouped = 0; c.fill = fill; c.cap = cap;
    if ((err = simt_launch<EPI_PLAIN>(c, s.act, cmax, E, st)) != hipSuccess) return err;
    SimtArgs d{};  // dW1[e](h, m) = sum_j dpre[j][h] buf[j][m]
    d.A = static_cast<const float *>(dpre); d.a_si = 1; d.a_sk = H; d.a_gfix = 0; d.a_gcap = H;
    d.B = static_cast<const float *>(buf); d.b_sn = 1; d.b_sk = M; d.b_gfix = 0; d.b_gcap = M;
    d.D = dW1; d.d_si = M; d.d_gfix = static_cast<int64_t>(H) * M; d.d_gcap = 0;
    d.rows = H; d.N = M; d.kgrouped = 1; d.fill = fill; d.cap = cap; d.colsum = db1;
    return simt_launch<EPI_PLAIN>(d, s.act, H, E, st);
}

}  // namespace moe
