// bf16 MFMA GEMM path for prefill-sized M (gfx950).
//
// At prefill the two phases of y = (x . U) . V are dense contractions with M = B*S in the
// thousands (about M flop per factor byte, far above the MFMA ridge), so each phase runs as an
// NT GEMM C[M, N] = A[M, K] . B[N, K]^T on the matrix cores with a fused epilogue:
//   - tiles of BM x BN (256 or 128 x 256 or 128), BK = 64, four waves as 2 x 2, each wave a grid
//     of 32 x 32 blocks computed with v_mfma_f32_32x32x16_bf16 (fp32 accumulation);
//   - operands move global -> LDS directly (global_load_lds_dwordx4, no staging registers) through
//     a 4-stage pipeline of BK = 32 slices, each lane choosing the global chunk whose XOR-swizzled
//     LDS home is its slot, so the 32-row fragment reads of one MFMA hit distinct banks; M/N tails
//     re-read the last row (never stored), the K tail is zeroed in LDS;
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

constexpr int BK = 32;          // k per LDS stage: 4 chunks of 16 bytes per row
constexpr int kStages = 4;      // LDS pipeline depth
constexpr int kThreads = 256;   // 4 waves, arranged 2 x 2

typedef __attribute__((address_space(3))) void lds_void;

// chunk c of row r of a stage buffer sits at chunk slot r * 4 + (c ^ ((r >> 2) & 3)): the 16 rows
// read by one quarter-wave for an MFMA fragment then fall in 16 distinct 16-byte bank groups
__device__ __forceinline__ int swz(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

// Issue the direct global -> LDS loads of one operand tile (ROWS x BK) into stage buffer 'dst'.
// A wave instruction writes 64 consecutive 16-byte slots; each lane picks the global chunk whose
// swizzled home is its slot.  Rows past 'rows' re-read the last row (their products are never
// stored); chunks past K are clamped inside the row and zeroed by zero_k_tail() before use.
template <int ROWS>
__device__ __forceinline__ void issue_tile(const bf16_t* base, int64_t ld, int row0, int rows, int k0, int K,
                                           u32x4* dst, int wave, int lane) {
    constexpr int PER_WAVE = ROWS * 4 / 64 / 4;  // instructions per wave
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int slot0 = (wave * PER_WAVE + i) * 64;
        const int slot = slot0 + lane;
        const int r = slot >> 2, phys = slot & 3;
        const int c = phys ^ ((r >> 2) & 3);
        const int gr = min(row0 + r, rows - 1);
        const int gk = min(k0 + c * 8, K - 8);
        __builtin_amdgcn_global_load_lds((const void*)(base + (int64_t)gr * ld + gk), (lds_void*)(dst + slot0), 16, 0, 0);
    }
}

// zero the chunks of a stage whose k index is >= K (only the last k tile can have them)
template <int ROWS>
__device__ __forceinline__ void zero_k_tail(u32x4* dst, int k0, int K, int tid) {
    for (int q = tid; q < ROWS * 4; q += kThreads) {
        const int r = q >> 2, c = q & 3;
        if (k0 + c * 8 >= K) dst[swz(r, c)] = u32x4{0u, 0u, 0u, 0u};
    }
}

__device__ __forceinline__ bf16x8_v frag(const u32x4* lds, int row, int chunk) {
    return __builtin_bit_cast(bf16x8_v, lds[swz(row, chunk)]);
}

// s_waitcnt on the vector-memory counter only: vmcnt in bits [3:0] and [15:14], expcnt (bits 6:4)
// and lgkmcnt (bits 11:8) left at their maxima so they do not wait
#define FSVD_VMCNT(n) (0x0F70 | ((n) & 0xF) | ((((n) >> 4) & 3) << 14))
__device__ __forceinline__ void wait_vm(int n) {
    // wait until at most n vector-memory operations of this wave are outstanding (n rounded down)
    if (n >= 16) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(16));
    else if (n >= 12) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(12));
    else if (n >= 8) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(8));
    else if (n >= 6) __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(6));
    else __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(0));
}

// Workgroup barrier that waits for this wave's LDS operations only.  __syncthreads() would also
// drain every outstanding global load (vmcnt(0)), i.e. the prefetches of later stages, which is
// exactly what the pipeline must keep in flight; stage arrival is ordered by wait_vm() instead.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt/expcnt unchanged
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Instruction order for one pipeline phase of NM MFMAs: the NR LDS reads and the NG global loads
// issued in that phase are spread evenly between the MFMAs (reads first), so they issue in the
// shadow of the matrix cores instead of in a burst that stalls them.
template <int NR, int NG, int NM, int Q = 0>
__device__ __forceinline__ void sched_interleave() {
    constexpr int NX = NG + NR;
    constexpr int per = NX ? (NM + NX - 1) / NX : NM;  // MFMAs between two memory instructions
    constexpr int left = NM - Q * per > 0 ? NM - Q * per : 0;
    constexpr int m = left < per ? left : per;
    if constexpr (Q < NX) {
        if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        __builtin_amdgcn_sched_group_barrier(Q < NR ? 0x100 : 0x020, 1, 0);
        sched_interleave<NR, NG, NM, Q + 1>();
    } else if constexpr (left > 0) {
        __builtin_amdgcn_sched_group_barrier(0x008, left, 0);
    }
}

// C tile accumulation over k in [0, K): acc[i][j] += A[wm + 32 i + .., k] . B[wn + 32 j + .., k]
template <int BM, int BN>
struct Tile {
    static constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
    static constexpr int FI = WM / 32, FJ = WN / 32;    // 32x32 blocks per wave
    static constexpr int STAGE = (BM + BN) * 4;         // 16-byte slots per stage
    static constexpr int LOADS = (BM + BN) * 4 / 64 / 4;  // load instructions per wave per stage
    f32x16 acc[FI][FJ];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    }

    // fragments of one 16-wide k step (substep kk of a BK = 32 stage) for this wave
    __device__ __forceinline__ void read_frags(const u32x4* st, int kk, int wm, int wn, int lane, bf16x8_v (&af)[FI],
                                               bf16x8_v (&bf)[FJ]) {
        const u32x4* pa = st;
        const u32x4* pb = st + BM * 4;
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FI; ++i) af[i] = frag(pa, wm + i * 32 + (lane & 31), ch);
#pragma unroll
        for (int j = 0; j < FJ; ++j) bf[j] = frag(pb, wn + j * 32 + (lane & 31), ch);
    }

    __device__ __forceinline__ void mfmas(const bf16x8_v (&af)[FI], const bf16x8_v (&bf)[FJ]) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }

    // Software pipeline over k tiles, two 16-wide substeps per tile.  Global -> LDS loads run
    // three tiles ahead; within a tile, the fragments of the next substep are read from LDS while
    // the MFMAs of the current one run, so the matrix cores wait neither for LDS nor at the single
    // barrier per tile, which sits between the two substeps:
    //   [loads of tile kt+3] [reads F1(kt)] [MFMA F0(kt)] wait tile kt+1, barrier
    //   [reads F0(kt+1)] [MFMA F1(kt)]
    // The barrier makes tile kt+1 visible and retires every wave's reads of tile kt, whose stage
    // the next iteration's loads (tile kt+4) overwrite.
    __device__ __forceinline__ void run(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, int m0, int n0,
                                        int M, int N, int K, u32x4* smem, int tid) {
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
        const int nk = (K + BK - 1) / BK;
        auto issue = [&](int t) {
            u32x4* st = smem + (t % kStages) * STAGE;
            issue_tile<BM>(A, lda, m0, M, t * BK, K, st, wave, lane);
            issue_tile<BN>(B, ldb, n0, N, t * BK, K, st + BM * 4, wave, lane);
        };
        // the last tile's chunks past K are zeroed once it has landed (all waves), before any read
        auto k_tail = [&](int t) {
            if (t == nk - 1 && K % BK) {
                lds_barrier();
                u32x4* st = smem + (t % kStages) * STAGE;
                zero_k_tail<BM>(st, t * BK, K, tid);
                zero_k_tail<BN>(st + BM * 4, t * BK, K, tid);
            }
        };
        bf16x8_v a0[FI], b0[FJ], a1[FI], b1[FJ];
        // prologue: tiles 0 .. 2 in flight, tile 0 landed, F0(0) read
        const int pro = min(nk, kStages - 1);
        for (int t = 0; t < pro; ++t) issue(t);
        wait_vm((pro - 1) * LOADS);
        k_tail(0);
        lds_barrier();
        read_frags(smem, 0, wm, wn, lane, a0, b0);

        // steady state: every iteration issues tile kt + 3, so tiles kt+2 and kt+3 may still be
        // in flight when tile kt+1 must have landed
        int kt = 0;
        for (; kt + kStages - 1 < nk; ++kt) {
            // phase A: loads of tile kt+3 and reads of F1(kt) interleaved with the MFMAs of F0(kt)
            __builtin_amdgcn_sched_barrier(0);
            const u32x4* st = smem + (kt % kStages) * STAGE;
            read_frags(st, 1, wm, wn, lane, a1, b1);
            issue(kt + kStages - 1);
            mfmas(a0, b0);
            sched_interleave<FI + FJ, 2 * LOADS, FI * FJ>();
            __builtin_amdgcn_sched_barrier(0);
            wait_vm((kStages - 2) * LOADS);
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            // phase B: reads of F0(kt+1) interleaved with the MFMAs of F1(kt)
            read_frags(smem + ((kt + 1) % kStages) * STAGE, 0, wm, wn, lane, a0, b0);
            mfmas(a1, b1);
            sched_interleave<FI + FJ, 0, FI * FJ>();
            __builtin_amdgcn_sched_barrier(0);
        }
        // drain: no more loads to issue
        for (; kt < nk; ++kt) {
            const u32x4* st = smem + (kt % kStages) * STAGE;
            read_frags(st, 1, wm, wn, lane, a1, b1);
            mfmas(a0, b0);
            if (kt + 1 < nk) {
                wait_vm((nk - 2 - kt) * LOADS);
                k_tail(kt + 1);
                lds_barrier();
                read_frags(smem + ((kt + 1) % kStages) * STAGE, 0, wm, wn, lane, a0, b0);
            }
            mfmas(a1, b1);
        }
        __syncthreads();  // the caller may reuse the stage buffers
    }
};

// workgroup -> (m tile, n tile).  Workgroup i runs on XCD i % 8; each XCD receives a contiguous
// range of logical tiles, and logical tiles are ordered in groups of GM m-tiles walked column by
// column, so the ~32 workgroups an XCD runs at once cover a GM x (32 / GM) patch of C and share
// GM A panels and 32 / GM B panels through that XCD's L2.
template <int GM>
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int* tm, int* tn) {
    const int nt = tiles_m * tiles_n;
    const int bid = blockIdx.x;
    const int per = (nt + 7) / 8;
    const int full = nt - 8 * (per - 1);  // XCDs that receive 'per' tiles (the rest get per - 1)
    const int x = bid & 7, local = bid >> 3;
    const int L = (x < full) ? x * per + local : full * per + (x - full) * (per - 1) + local;
    const int in_group = GM * tiles_n;
    const int group = L / in_group;
    const int first_m = group * GM;
    const int gsize = min(tiles_m - first_m, GM);
    const int r = L - group * in_group;
    *tm = first_m + r % gsize;
    *tn = r / gsize;
}

template <int BM, int BN, int EPI>
__global__ __launch_bounds__(kThreads, 1)
#if defined(FSVD_GEMM_WPE)
__attribute__((amdgpu_waves_per_eu(1, 1)))
#endif
void gemm_kernel(const GemmArgs g) {
    extern __shared__ u32x4 smem[];
    using T = Tile<BM, BN>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
    int tm, tn;
    tile_coords<(BM >= 256 ? 4 : 8)>(tiles_m, tiles_n, &tm, &tn);
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
    const size_t lds = (size_t)kStages * (BM + BN) * BK * 2;
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
