// bf16 MFMA GEMM path for prefill-sized M (gfx950).
//
// At prefill the two phases of y = (x . U) . V are dense contractions with M = B*S in the
// thousands (about M flop per factor byte, far above the MFMA ridge), so each phase runs as an
// NT GEMM C[M, N] = A[M, K] . B[N, K]^T on the matrix cores with a fused epilogue:
//   - tiles of BM x BN (256 or 128 x 256 or 128), BK = 64, four waves as 2 x 2, each wave a grid
//     of 32 x 32 blocks computed with v_mfma_f32_32x32x16_bf16 (fp32 accumulation);
//   - operands staged global -> registers -> LDS, double buffered, in an XOR-swizzled layout
//     (16-byte chunk c of row r stored at chunk c ^ (r & 7)) so the 32-row fragment reads of one
//     MFMA hit distinct banks; M/N/K tails are zero-filled;
//   - tiles are handed out XCD by XCD (workgroup i runs on XCD i mod 8) so the WGs that share an
//     XCD's L2 work on neighbouring M tiles of one N tile and reuse its B operand.
// Epilogues: per-row scale (RMSNorm folded after the product), bias + residual, Q/K/V with
// rotate-half RoPE (the partner column of a pair sits in the same lane) and the dense KV-cache
// append, SwiGLU (two accumulators, gate and up, with their own A column ranges), GELU.
//
// Sources: fused low-rank projections ("FlashSVD: Memory-Efficient Inference with Streaming for
// Low-Rank Models", abstract); prefill kernels shared by every checkpoint family, the packed
// gate|up projection ("FlashSVD v1.5" explainer, Methodology 1 and 3).
#include "kernels.h"

namespace fsvd {

namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 64;          // k per LDS stage (8 chunks of 16 bytes per row)
constexpr int kThreads = 256;   // 4 waves, arranged 2 x 2

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

// global -> register staging of one operand tile (ROWS x BK); zero outside [0,rows) x [0,K)
template <int ROWS>
struct Stage {
    static constexpr int N = ROWS * 8 / kThreads;  // 16-byte chunks per thread
    u32x4 v[N];
    __device__ __forceinline__ void load(const bf16_t* base, int64_t ld, int row0, int rows, int k0, int K, int tid) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + i * kThreads;
            const int r = q >> 3, c = q & 7;
            const int gr = row0 + r, gk = k0 + c * 8;
            if (gr < rows && gk < K)
                v[i] = *reinterpret_cast<const u32x4*>(base + (int64_t)gr * ld + gk);
            else
                v[i] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(u32x4* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int q = tid + i * kThreads;
            lds[swz(q >> 3, q & 7)] = v[i];
        }
    }
};

__device__ __forceinline__ bf16x8_v frag(const u32x4* lds, int row, int chunk) {
    return __builtin_bit_cast(bf16x8_v, lds[swz(row, chunk)]);
}

// C tile accumulation over k in [0, K): acc[i][j] += A[wm + 32 i + .., k] . B[wn + 32 j + .., k]
template <int BM, int BN>
struct Tile {
    static constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
    static constexpr int FI = WM / 32, FJ = WN / 32;    // 32x32 blocks per wave
    f32x16 acc[FI][FJ];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    }

    __device__ __forceinline__ void run(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, int m0, int n0,
                                        int M, int N, int K, u32x4* smem, int tid) {
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
        u32x4* la[2] = {smem, smem + BM * 8 + BN * 8};
        u32x4* lb[2] = {smem + BM * 8, smem + 2 * BM * 8 + BN * 8};
        Stage<BM> sa;
        Stage<BN> sb;
        const int nk = (K + BK - 1) / BK;
        sa.load(A, lda, m0, M, 0, K, tid);
        sb.load(B, ldb, n0, N, 0, K, tid);
        sa.store(la[0], tid);
        sb.store(lb[0], tid);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) {
                sa.load(A, lda, m0, M, (kt + 1) * BK, K, tid);
                sb.load(B, ldb, n0, N, (kt + 1) * BK, K, tid);
            }
            const u32x4* pa = la[cur];
            const u32x4* pb = lb[cur];
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int ch = kk * 2 + (lane >> 5);
                bf16x8_v af[FI], bfr[FJ];
#pragma unroll
                for (int i = 0; i < FI; ++i) af[i] = frag(pa, wm + i * 32 + (lane & 31), ch);
#pragma unroll
                for (int j = 0; j < FJ; ++j) bfr[j] = frag(pb, wn + j * 32 + (lane & 31), ch);
#pragma unroll
                for (int i = 0; i < FI; ++i)
#pragma unroll
                    for (int j = 0; j < FJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nk) {
                sa.store(la[cur ^ 1], tid);
                sb.store(lb[cur ^ 1], tid);
            }
            __syncthreads();
        }
    }
};

// tile index -> (m tile, n tile), XCD-grouped: workgroup i runs on XCD i % 8
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int* tm, int* tn) {
    const int nt = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int per = (nt + 7) / 8;
    const int full = nt - 8 * (per - 1);  // XCDs that receive 'per' tiles (the rest get per - 1)
    const int x = bid & 7, local = bid >> 3;
    const int logical = (x < full) ? x * per + local : full * per + (x - full) * (per - 1) + local;
    *tn = logical / tiles_m;
    *tm = logical - *tn * tiles_m;
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs g) {
    extern __shared__ u32x4 smem[];
    using T = Tile<BM, BN>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, &tm, &tn);
    const int m0 = tm * BM, n0 = tn * BN;

    T t;
    t.zero();
    t.run(g.A + g.a_col_off, g.lda, g.Bm, g.ldb, m0, n0, g.M, g.N, g.K, smem, tid);
    T t2;  // up accumulator (SwiGLU only)
    if constexpr (EPI == GEPI_SWIGLU) {
        t2.zero();
        t2.run(g.A + g.a_col_off2, g.lda, g.B2, g.ldb2, m0, n0, g.M, g.N, g.K2, smem, tid);
    }

    const int wm = m0 + (wave >> 1) * T::WM, wn = n0 + (wave & 1) * T::WN;
    const int col_in = lane & 31, rsub = (lane >> 5) * 4;

    if constexpr (EPI == GEPI_QKV) {
        // Pairs (c, c + D/2) of a head: the wave's column range is 128-aligned and holds whole
        // heads, so the partner of block j is block j + D/64 in the same lane.
        const int halfD = g.D >> 1, pb = halfD / 32;
        const bool rope = g.seg != 2 && g.rope_theta > 0.f;
        double rev[T::FJ];  // revolutions per position for the pair index of block j
#pragma unroll
        for (int j = 0; j < T::FJ; ++j) {
            const int ip = ((wn + j * 32 + col_in) % g.D) % halfD;
            rev[j] = exp2(-2.0 * (double)ip / (double)g.D * log2((double)g.rope_theta)) *
                     0.15915494309189533576888376337251;  // 1 / (2 pi)
        }
#pragma unroll
        for (int i = 0; i < T::FI; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm + i * 32 + (e >> 2) * 8 + rsub + (e & 3);
                if (row >= g.M) continue;
                const int b = row / g.S, s = row - b * g.S;
                const int64_t p = (int64_t)g.seqlens[b] + s;
                const bool in_cache = p >= 0 && p < g.L_max;
                bf16_t* dst = g.seg == 0 ? g.q_out : (g.seg == 1 ? g.k_cache : g.v_cache);
                bf16_t* dbg = g.seg == 1 ? g.k_out : (g.seg == 2 ? g.v_out : nullptr);
                const int64_t drow = g.seg == 0 ? (int64_t)row * g.N : ((int64_t)b * g.L_max + p) * g.N;
                const bool write = g.seg == 0 || in_cache;
                if (!write) set_dev_error(g.err, FSVD_DEVERR_KV_OVERFLOW);
#pragma unroll
                for (int j = 0; j < T::FJ; ++j) {
                    const int col = wn + j * 32 + col_in;
                    if (col >= g.N) continue;
                    if (rope) {
                        if ((j / pb) & 1) continue;  // second half: written with its partner
                        const double tr = (double)p * rev[j];
                        const float ang = (float)((tr - floor(tr)) * 6.283185307179586476925286766559);
                        float c, sn;
                        sincosf(ang, &sn, &c);
                        // partner block j + pb, selected with constant indices only
                        const float x1 = t.acc[i][j][e];
                        float x2 = 0.f;
#pragma unroll
                        for (int jj = 0; jj < T::FJ; ++jj)
                            if (jj == j + pb) x2 = t.acc[i][jj][e];
                        const bf16_t v1 = f2bf(x1 * c - x2 * sn), v2 = f2bf(x2 * c + x1 * sn);
                        if (write) {
                            dst[drow + col] = v1;
                            dst[drow + col + halfD] = v2;
                        }
                        if (dbg) {
                            dbg[(int64_t)row * g.N + col] = v1;
                            dbg[(int64_t)row * g.N + col + halfD] = v2;
                        }
                    } else {
                        const bf16_t v = f2bf(t.acc[i][j][e]);
                        if (write) dst[drow + col] = v;
                        if (dbg) dbg[(int64_t)row * g.N + col] = v;
                    }
                }
            }
        }
        return;
    }

#pragma unroll
    for (int i = 0; i < T::FI; ++i) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = wm + i * 32 + (e >> 2) * 8 + rsub + (e & 3);
            if (row >= g.M) continue;
            const float rs = g.rstd ? g.rstd[row] : 1.0f;
#pragma unroll
            for (int j = 0; j < T::FJ; ++j) {
                const int col = wn + j * 32 + col_in;
                if (col >= g.N) continue;
                float y = t.acc[i][j][e] * rs;
                if constexpr (EPI == GEPI_LINEAR) {
                    if (g.bias) y += bf2f(g.bias[col]);
                    if (g.residual) y += bf2f(g.residual[(int64_t)row * g.ldr + col]);
                } else if constexpr (EPI == GEPI_SWIGLU) {
                    y = silu_f(y) * t2.acc[i][j][e];
                } else if constexpr (EPI == GEPI_GELU) {
                    y = gelu_f(y);
                }
                g.C[(int64_t)row * g.ldc + col] = f2bf(y);
            }
        }
    }
}

template <int BM, int BN, int EPI>
fsvd_status_t launch_t(const GemmArgs& g, hipStream_t st) {
    const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN);
    const size_t lds = (size_t)2 * (BM + BN) * BK * 2;
    static bool attr_set = false;
    if (!attr_set) {
        (void)hipFuncSetAttribute((const void*)gemm_kernel<BM, BN, EPI>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)lds);
        attr_set = true;
    }
    gemm_kernel<BM, BN, EPI><<<tiles, kThreads, lds, st>>>(g);
    return check_launch("gemm");
}

}  // namespace

fsvd_status_t launch_gemm(const GemmArgs& g, int epi, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0) return FSVD_OK;
    if (g.K <= 0 || (epi == GEPI_SWIGLU && g.K2 <= 0)) return fail(FSVD_ERR_INVALID_ARG, "gemm: empty reduction");
    if (epi == GEPI_QKV && (g.D != 64 && g.D != 128)) return fail(FSVD_ERR_UNSUPPORTED, "RoPE epilogue needs D in {64,128}");
    // tile choice: 256 x 256 when the grid still covers the chip, else 128 x 256
    const int t256 = ((g.M + 255) / 256) * ((g.N + 255) / 256);
    switch (epi) {
        case GEPI_STORE:
            return t256 >= 512 ? launch_t<256, 256, GEPI_STORE>(g, st) : launch_t<128, 256, GEPI_STORE>(g, st);
        case GEPI_LINEAR:
            return t256 >= 512 ? launch_t<256, 256, GEPI_LINEAR>(g, st) : launch_t<128, 256, GEPI_LINEAR>(g, st);
        case GEPI_QKV:
            return t256 >= 512 ? launch_t<256, 256, GEPI_QKV>(g, st) : launch_t<128, 256, GEPI_QKV>(g, st);
        case GEPI_SWIGLU: return launch_t<256, 128, GEPI_SWIGLU>(g, st);
        case GEPI_GELU:
            return t256 >= 512 ? launch_t<256, 256, GEPI_GELU>(g, st) : launch_t<128, 256, GEPI_GELU>(g, st);
    }
    return fail(FSVD_ERR_UNSUPPORTED, "unknown gemm epilogue %d", epi);
}

}  // namespace fsvd
