// bf16 MFMA GEMM path for prefill-sized M (gfx950).
//
// At prefill the two phases of y = (x . U) . V are dense contractions with M = B*S in the
// thousands (about M flop per factor byte, far above the MFMA ridge), so each phase runs as an
// NT GEMM C[M, N] = A[M, K] . B[N, K]^T on the matrix cores with a fused epilogue:
//   - tiles of BM x BN (256 x 256 down to 64 x 128, the largest that still fills the chip; short
//     reductions take 128 x 192 or 64 x 128), four waves as 2 x 2, each wave a grid of 32 x 32
//     blocks computed with
//     v_mfma_f32_32x32x16_bf16 (fp32 accumulation);
//   - operands move global -> LDS directly (global_load_lds_dwordx4, no staging registers) through
//     a 3- or 4-stage pipeline of BK = 64 or 32 slices (BK = 64: one whole 128-byte line per row
//     and stage), each lane choosing the global chunk
//     whose XOR-swizzled LDS home is its slot, so the fragment reads of one MFMA hit distinct
//     banks; M/N tails re-read the last row (never stored), the K tail is zeroed in LDS;
//   - tiles are handed out XCD by XCD (workgroup i runs on XCD i mod 8) so the WGs that share an
//     XCD's L2 work on neighbouring M tiles of one N tile and reuse its B operand.
// Epilogues: per-row scale (RMSNorm folded after the product), bias + residual, Q/K/V with
// rotate-half RoPE (the partner column of a pair sits in the same lane) and the dense KV-cache
// append, SwiGLU (two accumulators, gate and up, with their own A column ranges), GELU, and an
// fp32 accumulation into C for symmetric products (tiles below the diagonal skipped).
//
// Sources: fused low-rank projections ("FlashSVD: Memory-Efficient Inference with Streaming for
// Low-Rank Models", abstract); prefill kernels shared by every checkpoint family, the packed
// gate|up projection ("FlashSVD v1.5" explainer, Methodology 1 and 3).
#include "kernels.h"

namespace fsvd {

namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;   // 4 waves, arranged 2 x 2

// Per tile shape: k per LDS stage (KB) and pipeline depth.  256 x 256 tiles stage BK = 32 slices
// four deep (4 x 32 KiB); the smaller tiles (128 x 256, 256 x 128, 128 x 128, 64 x 128) stage
// BK = 64 slices, one whole 128-byte line per row (the load path serves whole lines about 1.4x
// faster than half lines), three deep (3 x 48 KiB for 128 x 256).  Measured on MI355X, the deeper
// pipeline matters more for the big tile.
#ifndef FSVD_GEMM_SPLITB
#define FSVD_GEMM_SPLITB 1  // 256 x 256 tiles: B loads of a tile in its second k step
#endif
template <int BM, int BN>
constexpr int kb_for() { return BM + BN > 384 ? 32 : 64; }
template <int BM, int BN>
constexpr int stages_for() { return kb_for<BM, BN>() == 32 ? 4 : 3; }

typedef __attribute__((address_space(3))) void lds_void;

// Swizzled home of chunk c (16 bytes) of row r in a stage buffer.  KB = 64: rows of 8 chunks
// (128 bytes, half the 64 x 4-byte banks), slot r * 8 + (c ^ ((r >> 1) & 7)); KB = 32: rows of 4
// chunks, slot r * 4 + (c ^ ((r >> 2) & 3)).  Either way the 16 rows read by one quarter-wave for
// an MFMA fragment cover 16 distinct 16-byte bank groups.
template <int KB>
__device__ __forceinline__ int swz(int row, int chunk) {
    if constexpr (KB == 64) return row * 8 + (chunk ^ ((row >> 1) & 7));
    else return row * 4 + (chunk ^ ((row >> 2) & 3));
}

// Issue the direct global -> LDS loads of one operand tile (ROWS x KB) into stage buffer 'dst'.
// A wave instruction writes 64 consecutive 16-byte slots; each lane picks the global chunk whose
// swizzled home is its slot.  Rows past 'rows' re-read the last row (their products are never
// stored); chunks past K are clamped inside the row and zeroed by zero_k_tail() before use.
template <int ROWS, int KB>
__device__ __forceinline__ void issue_tile(const bf16_t* base, int64_t ld, int row0, int rows, int k0, int K,
                                           u32x4* dst, int wave, int lane) {
    constexpr int CPR = KB / 8;
    constexpr int PER_WAVE = ROWS * CPR / kThreads;  // instructions per wave
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
        const int slot0 = (wave * PER_WAVE + i) * 64;
        const int slot = slot0 + lane;
        const int r = slot / CPR, phys = slot % CPR;
        const int c = KB == 64 ? (phys ^ ((r >> 1) & 7)) : (phys ^ ((r >> 2) & 3));
        const int gr = min(row0 + r, rows - 1);
        const int gk = min(k0 + c * 8, K - 8);
        __builtin_amdgcn_global_load_lds((const void*)(base + (int64_t)gr * ld + gk), (lds_void*)(dst + slot0), 16, 0, 0);
    }
}

// zero the chunks of a stage whose k index is >= K (only the last k tile can have them)
template <int ROWS, int KB>
__device__ __forceinline__ void zero_k_tail(u32x4* dst, int k0, int K, int tid) {
    constexpr int CPR = KB / 8;
    for (int q = tid; q < ROWS * CPR; q += kThreads) {
        const int r = q / CPR, c = q % CPR;
        if (k0 + c * 8 >= K) dst[swz<KB>(r, c)] = u32x4{0u, 0u, 0u, 0u};
    }
}

// Instruction order for one pipeline step of NM MFMAs: one memory instruction after each of the
// first MFMAs, the NR LDS reads (fragments of the next k step) first so they land well before
// the step ends, then the NG global loads, then the remaining MFMAs.
template <int NR, int NG, int NM, int Q = 0>
__device__ __forceinline__ void sched_interleave() {
    constexpr int NX = NR + NG;
    if constexpr (Q < NX) {
        if constexpr (Q < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(Q < NR ? 0x100 : 0x020, 1, 0);
        sched_interleave<NR, NG, NM, Q + 1>();
    } else if constexpr (NM > NX) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM - NX, 0);
    }
}

// C tile accumulation over k in [0, K): acc[i][j] += A[wm + 32 i + .., k] . B[wn + 32 j + .., k]
template <int BM, int BN>
struct Tile {
    static constexpr int KB = kb_for<BM, BN>();          // k per stage
    static constexpr int CPR = KB / 8;                   // 16-byte chunks per row and stage
    static constexpr int S = stages_for<BM, BN>();       // LDS stages
    static constexpr int WM = BM / 2, WN = BN / 2;      // wave tile
    static constexpr int FI = WM / 32, FJ = WN / 32;    // 32x32 blocks per wave
    static constexpr int STAGE = (BM + BN) * CPR;       // 16-byte slots per stage
    static constexpr int LOADS = STAGE / kThreads;      // load instructions per wave per stage
    static constexpr int KSUB = KB / 16;                // 16-wide MFMA k steps per stage
    static constexpr size_t LDS_BYTES = (size_t)S * STAGE * 16;
    f32x16 acc[FI][FJ];

    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    }

    // fragments of k step kk (0 .. KSUB-1) of a stage for this wave
    __device__ __forceinline__ void read_frags(const u32x4* st, int kk, int wm, int wn, int lane, bf16x8_v (&af)[FI],
                                               bf16x8_v (&bf)[FJ]) {
        const u32x4* pa = st;
        const u32x4* pb = st + BM * CPR;
        const int ch = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FI; ++i) af[i] = __builtin_bit_cast(bf16x8_v, pa[swz<KB>(wm + i * 32 + (lane & 31), ch)]);
#pragma unroll
        for (int j = 0; j < FJ; ++j) bf[j] = __builtin_bit_cast(bf16x8_v, pb[swz<KB>(wn + j * 32 + (lane & 31), ch)]);
    }

    __device__ __forceinline__ void mfmas(const bf16x8_v (&af)[FI], const bf16x8_v (&bf)[FJ]) {
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }

    // Software pipeline over k tiles (S LDS stages, KSUB MFMA k steps per tile).  Global -> LDS
    // loads run S - 1 tiles ahead; within a tile the fragments of the next k step are read from LDS
    // while the MFMAs of the current one run, so the matrix cores wait neither for LDS nor at the
    // single barrier per tile, which sits before the last k step (KSUB = 4 shown):
    //   [reads F1, loads A of tile kt+S-1, MFMA F0] [reads F2, loads B, MFMA F1] [reads F3, MFMA F2]
    //   wait for tile kt+1, barrier, [reads F0 of tile kt+1, MFMA F3]
    // The barrier makes tile kt+1 visible and retires every wave's reads of tile kt, whose stage
    // the next iteration's loads (tile kt+S) overwrite.
    template <bool ISSUE>
    __device__ __forceinline__ void step(int kt, int nk, const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb,
                                         int m0, int n0, int M, int N, int K, u32x4* smem, int tid, int wm, int wn,
                                         bf16x8_v (&af)[2][FI], bf16x8_v (&bf)[2][FJ]) {
        const int lane = tid & 63, wave = tid >> 6;
        constexpr int LA = BM * CPR / kThreads, LB = BN * CPR / kThreads;  // loads per operand
        // k step issuing the B loads; with two k steps per tile (KSUB = 2) they go into the last
        // one, after the barrier, so each k step carries half of the tile's loads
        constexpr bool B_LAST = KSUB == 2 && FSVD_GEMM_SPLITB;
        constexpr int KB_B = KSUB > 2 ? 1 : 0;
        const u32x4* st = smem + (kt % S) * STAGE;
        u32x4* dst = smem + ((kt + S - 1) % S) * STAGE;
#pragma unroll
        for (int kk = 0; kk + 1 < KSUB; ++kk) {
            __builtin_amdgcn_sched_barrier(0);
            read_frags(st, kk + 1, wm, wn, lane, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
            if constexpr (ISSUE) {
                if (kk == 0) issue_tile<BM, KB>(A, lda, m0, M, (kt + S - 1) * KB, K, dst, wave, lane);
                if (!B_LAST && kk == KB_B) issue_tile<BN, KB>(B, ldb, n0, N, (kt + S - 1) * KB, K, dst + BM * CPR, wave, lane);
            }
            mfmas(af[kk & 1], bf[kk & 1]);
            constexpr int ng0 = ISSUE ? ((KB_B == 0 && !B_LAST) ? LA + LB : LA) : 0;
            constexpr int ng1 = ISSUE ? LB : 0;
            if (kk == 0) sched_interleave<FI + FJ, ng0, FI * FJ>();
            else if (kk == KB_B) sched_interleave<FI + FJ, ng1, FI * FJ>();
            else sched_interleave<FI + FJ, 0, FI * FJ>();
        }
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < nk) {
            // tile kt + 1 must have landed; issued after it so far: the whole tiles up to
            // min(kt + S - 1, nk - 1), or with B_LAST up to kt + S - 2 plus the A part of kt + S - 1
            if constexpr (B_LAST)
                wait_vm(max(0, min(kt + S - 2, nk - 1) - (kt + 1)) * LOADS + (ISSUE ? LA : 0));
            else
                wait_vm((min(kt + S - 1, nk - 1) - (kt + 1)) * LOADS);
            if (kt + 1 == nk - 1 && K % KB) {
                lds_barrier();
                u32x4* last = smem + ((kt + 1) % S) * STAGE;
                zero_k_tail<BM, KB>(last, (kt + 1) * KB, K, tid);
                zero_k_tail<BN, KB>(last + BM * CPR, (kt + 1) * KB, K, tid);
            }
            lds_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_frags(smem + ((kt + 1) % S) * STAGE, 0, wm, wn, lane, af[0], bf[0]);
        }
        if constexpr (ISSUE && B_LAST) issue_tile<BN, KB>(B, ldb, n0, N, (kt + S - 1) * KB, K, dst + BM * CPR, wave, lane);
        mfmas(af[(KSUB - 1) & 1], bf[(KSUB - 1) & 1]);
        sched_interleave<FI + FJ, (ISSUE && B_LAST) ? LB : 0, FI * FJ>();
        __builtin_amdgcn_sched_barrier(0);
    }

    __device__ __forceinline__ void run(const bf16_t* A, int64_t lda, const bf16_t* B, int64_t ldb, int m0, int n0,
                                        int M, int N, int K, u32x4* smem, int tid) {
        const int lane = tid & 63, wave = tid >> 6;
        const int wm = (wave >> 1) * WM, wn = (wave & 1) * WN;
        const int nk = (K + KB - 1) / KB;
        bf16x8_v af[2][FI], bf[2][FJ];
        // prologue: tiles 0 .. S-2 in flight, tile 0 landed (and K-tail zeroed), F0(0) read
        const int pro = min(nk, S - 1);
        for (int t = 0; t < pro; ++t) {
            u32x4* dst = smem + (t % S) * STAGE;
            issue_tile<BM, KB>(A, lda, m0, M, t * KB, K, dst, wave, lane);
            issue_tile<BN, KB>(B, ldb, n0, N, t * KB, K, dst + BM * CPR, wave, lane);
        }
        wait_vm((pro - 1) * LOADS);
        if (nk == 1 && K % KB) {
            lds_barrier();
            zero_k_tail<BM, KB>(smem, 0, K, tid);
            zero_k_tail<BN, KB>(smem + BM * CPR, 0, K, tid);
        }
        lds_barrier();
        read_frags(smem, 0, wm, wn, lane, af[0], bf[0]);
        int kt = 0;
        for (; kt + S - 1 < nk; ++kt) step<true>(kt, nk, A, lda, B, ldb, m0, n0, M, N, K, smem, tid, wm, wn, af, bf);
        for (; kt < nk; ++kt) step<false>(kt, nk, A, lda, B, ldb, m0, n0, M, N, K, smem, tid, wm, wn, af, bf);
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
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(const GemmArgs g) {
    extern __shared__ u32x4 smem[];
    using T = Tile<BM, BN>;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the problem of this workgroup: the launch's, or one column segment of a grouped launch
    const bf16_t* Bm = g.Bm;
    int64_t ldb = g.ldb;
    int K = g.K, N = g.N, acol = g.a_col_off, seg = g.seg;
    const int tiles_m = (g.M + BM - 1) / BM;
    int tiles_n = (g.N + BN - 1) / BN;
    if constexpr (EPI == GEPI_QKV) {
        if (g.nseg > 1) {
            tiles_n = 0;
            for (int s = 0; s < g.nseg; ++s) tiles_n += (g.segs[s].N + BN - 1) / BN;
        }
    }
    int tm, tn;
    tile_coords<(BM >= 256 ? 4 : 8)>(tiles_m, tiles_n, &tm, &tn);
    if constexpr (EPI == GEPI_QKV) {
        if (g.nseg > 1) {  // segment of column tile tn, and tn within it
            int s = 0;
            while (s + 1 < g.nseg && tn >= (g.segs[s].N + BN - 1) / BN) tn -= (g.segs[s++].N + BN - 1) / BN;
            Bm = g.segs[s].Bm; ldb = g.segs[s].ldb; K = g.segs[s].K; acol = g.segs[s].a_col_off; N = g.segs[s].N;
            seg = s;
        }
    }
    const int m0 = tm * BM, n0 = tn * BN;
    if constexpr (EPI == GEPI_ACC32) {
        if (m0 >= n0 + BN) return;  // wholly below the diagonal of a symmetric product (whole workgroup)
    }

    T t;
    t.zero();
    t.run(g.A + acol, g.lda, Bm, ldb, m0, n0, g.M, N, K, smem, tid);
    T t2;  // up accumulator (SwiGLU only)
    if constexpr (EPI == GEPI_SWIGLU) {
        t2.zero();
        t2.run(g.A + g.a_col_off2, g.lda, g.B2, g.ldb2, m0, n0, g.M, g.N, g.K2, smem, tid);
    }

    const int wm = m0 + (wave >> 1) * T::WM, wn = n0 + (wave & 1) * T::WN;
    const int col_in = lane & 31, rsub = (lane >> 5) * 4;

    // Staging buffer of the row epilogues: each wave stages one 32-row block of its fp32 tile at a
    // time (the MFMA layout gives a lane one column of 16 rows) and reads it back by rows.
    constexpr int SROW = T::WN + 8;        // staged row stride in floats (rows 4 apart: 32 banks apart)
    float* stg = reinterpret_cast<float*>(smem) + wave * 32 * SROW;
    // block i is selected with constant indices only (a runtime index into the accumulators
    // would move them to scratch memory when the caller's loop over i is not unrolled)
    auto stage = [&](int i) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int ii = 0; ii < T::FI; ++ii) {
            if (ii != i) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int r = (e >> 2) * 8 + rsub + (e & 3);
#pragma unroll
                for (int j = 0; j < T::FJ; ++j) {
                    float v = t.acc[ii][j][e];
                    if constexpr (EPI == GEPI_SWIGLU) {
                        const int row = wm + ii * 32 + r;
                        const float rs = (g.rstd && row < g.M) ? g.rstd[row] : 1.0f;
                        v = silu_f(v * rs) * t2.acc[ii][j][e];
                    }
                    stg[r * SROW + j * 32 + col_in] = v;
                }
            }
        }
        asm volatile("" ::: "memory");
    };
    auto ld8 = [&](int r, int c, float (&y)[8]) {
        const u32x4 lo = *reinterpret_cast<const u32x4*>(stg + r * SROW + c);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(stg + r * SROW + c + 4);
        y[0] = __uint_as_float(lo.x); y[1] = __uint_as_float(lo.y); y[2] = __uint_as_float(lo.z); y[3] = __uint_as_float(lo.w);
        y[4] = __uint_as_float(hi.x); y[5] = __uint_as_float(hi.y); y[6] = __uint_as_float(hi.z); y[7] = __uint_as_float(hi.w);
    };
    auto pack8 = [](const float (&y)[8]) {
        return u32x4{pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]), pack_bf2(y[4], y[5]), pack_bf2(y[6], y[7])};
    };

    if constexpr (EPI == GEPI_QKV) {
        // Row layout by RoPE pairs: a wave tile row holds whole heads (its 128 columns are
        // 128-aligned), i.e. 64 pairs (c, c + D/2); a lane owns 8 consecutive pairs of a row,
        // rotates them (sin/cos once per pair) and writes the two 16-byte halves, to the Q
        // output or to the cache row of the token's position (and the optional K/V copies).
        constexpr int LPR = T::WN / 16;    // lanes per row
        constexpr int RP = 64 / LPR;       // rows per pass
        const int halfD = g.D >> 1;
        const bool rope = seg != 2 && g.rope_theta > 0.f;
        const int pr0 = (lane % LPR) * 8;             // first pair slot of the lane in the row
        const int h = pr0 / halfD, i0 = pr0 % halfD;  // head within the wave tile, pair index
        const int c1 = h * g.D + i0, c2 = c1 + halfD;  // staged columns of the two halves
        // revolutions per position of each pair index, computed once per workgroup into LDS past
        // the staging buffers (after the k loop, so nothing of it is live across that loop)
        double* rev = reinterpret_cast<double*>(reinterpret_cast<float*>(smem) + 4 * 32 * SROW);
        if (tid < halfD)
            rev[tid] = rope ? exp2(-2.0 * (double)tid / (double)g.D * log2((double)g.rope_theta)) *
                                  0.15915494309189533576888376337251  // 1 / (2 pi)
                            : 0.0;
        // per tile row, once: its token position (RoPE) and its destination row offset (-1: the
        // position is past the cache, nothing is written), so the passes below need no global
        // load of cache_seqlens and no division
        int64_t* rpos = reinterpret_cast<int64_t*>(rev + 64);
        int64_t* rdst = rpos + BM;
        for (int r = tid; r < BM; r += kThreads) {
            const int row = m0 + r;
            int64_t pp = 0, dr = -1;
            if (row < g.M) {
                const int grow = g.row_off + row;  // token index within the call
                const int b = grow / g.S, s = grow - b * g.S;
                pp = (g.seqlens ? (int64_t)g.seqlens[b] : 0) + s;
                if (seg == 0) dr = (int64_t)row * N;
                else if (pp >= 0 && pp < g.L_max) dr = ((int64_t)b * g.L_max + pp) * N;
                else set_dev_error(g.err, FSVD_DEVERR_KV_OVERFLOW);
            }
            rpos[r] = pp;
            rdst[r] = dr;
        }
        __syncthreads();
        bf16_t* dst = seg == 0 ? g.q_out : (seg == 1 ? g.k_cache : g.v_cache);
        bf16_t* dbg = seg == 1 ? g.k_out : (seg == 2 ? g.v_out : nullptr);
#pragma unroll 1
        for (int i = 0; i < T::FI; ++i) {
            stage(i);
#pragma unroll
            for (int pass = 0; pass < 32 / RP; ++pass) {
                const int r = pass * RP + lane / LPR;
                const int row = wm + i * 32 + r;
                if (row >= g.M || wn + c2 >= N) continue;
                const int tr_ = row - m0;  // row within the tile
                const int64_t p = rpos[tr_];
                const int64_t drow = rdst[tr_];
                const bool write = drow >= 0;
                float x1[8], x2[8];
                ld8(r, c1, x1);
                ld8(r, c2, x2);
                if (rope) {
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const double tr = (double)p * rev[i0 + q];
                        const float fr = (float)(tr - floor(tr));  // angle in revolutions, [0, 1)
                        // v_sin_f32 / v_cos_f32 take revolutions (error <= 1.3e-7 on [0, 1), measured)
                        const float sn = __builtin_amdgcn_sinf(fr), c = __builtin_amdgcn_cosf(fr);
                        const float a = x1[q], bb = x2[q];
                        x1[q] = a * c - bb * sn;
                        x2[q] = bb * c + a * sn;
                    }
                }
                const u32x4 v1 = pack8(x1), v2 = pack8(x2);
                if (write) {
                    __builtin_nontemporal_store(v1, reinterpret_cast<u32x4*>(dst + drow + wn + c1));
                    __builtin_nontemporal_store(v2, reinterpret_cast<u32x4*>(dst + drow + wn + c2));
                }
                if (dbg) {
                    *reinterpret_cast<u32x4*>(dbg + (int64_t)row * N + wn + c1) = v1;
                    *reinterpret_cast<u32x4*>(dbg + (int64_t)row * N + wn + c2) = v2;
                }
            }
        }
        return;
    }

    // Row epilogue: a lane owns 8 consecutive columns of a row; the per-row scale, bias, residual
    // and activation are applied there and the result leaves as one 16-byte store (bias and
    // residual arrive as 16-byte loads), instead of 2-byte stores scattered over the tile.  The
    // residual rows and row scales of the next 32-row block are loaded while the current block is
    // processed, so the passes do not wait on them one by one.
    constexpr int LPR = T::WN / 8;         // lanes per row
    constexpr int RP = 64 / LPR;           // rows per pass
    constexpr int NP = (32 + RP - 1) / RP; // passes per 32-row block
    // with 96-wide wave tiles 12 lanes cover a row: 5 rows per pass, lanes 60-63 idle, and the
    // seventh pass covers the last 2 rows
    const bool lane_on = lane < RP * LPR;
    const int c8 = (lane % LPR) * 8;
    const int col = wn + c8;
    const bool full = col + 8 <= g.N;
    float bias8[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) bias8[q] = 0.f;
    if constexpr (EPI == GEPI_LINEAR) {
        if (g.bias && col < g.N) {
            if (full) {
                const u32x4 bv = *reinterpret_cast<const u32x4*>(g.bias + col);
                const uint32_t w[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bias8[2 * q] = bf_lo(w[q]);
                    bias8[2 * q + 1] = bf_hi(w[q]);
                }
            } else {
                for (int q = 0; q < 8 && col + q < g.N; ++q) bias8[q] = bf2f(g.bias[col + q]);
            }
        }
    }
    u32x4 resv[2][NP];
    float rsv[2][NP];
    auto prefetch = [&](int i, u32x4 (&rv)[NP], float (&rs)[NP]) {
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int r = pass * RP + lane / LPR;
            const int row = wm + i * 32 + r;
            const bool ok = lane_on && r < 32 && row < g.M && col < g.N;
            rs[pass] = (EPI != GEPI_SWIGLU && g.rstd && ok) ? g.rstd[row] : 1.0f;
            rv[pass] = u32x4{0u, 0u, 0u, 0u};
            if constexpr (EPI == GEPI_LINEAR) {
                if (g.residual && ok && full)
                    rv[pass] = *reinterpret_cast<const u32x4*>(g.residual + (int64_t)row * g.ldr + col);
            }
        }
    };
    prefetch(0, resv[0], rsv[0]);
#pragma unroll
    for (int i = 0; i < T::FI; ++i) {
        if (i + 1 < T::FI) prefetch(i + 1, resv[(i + 1) & 1], rsv[(i + 1) & 1]);
        stage(i);
#pragma unroll
        for (int pass = 0; pass < NP; ++pass) {
            const int r = pass * RP + lane / LPR;
            const int row = wm + i * 32 + r;
            if (!lane_on || r >= 32 || row >= g.M || col >= g.N) continue;
            float y[8];
            ld8(r, c8, y);
            if constexpr (EPI != GEPI_SWIGLU) {
                const float rs = rsv[i & 1][pass];
#pragma unroll
                for (int q = 0; q < 8; ++q) y[q] *= rs;
            }
            if constexpr (EPI == GEPI_LINEAR) {
#pragma unroll
                for (int q = 0; q < 8; ++q) y[q] += bias8[q];
                if (g.residual) {
                    if (full) {
                        const u32x4 rv = resv[i & 1][pass];
                        const uint32_t w[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            y[2 * q] += bf_lo(w[q]);
                            y[2 * q + 1] += bf_hi(w[q]);
                        }
                    } else {
                        const bf16_t* rp = g.residual + (int64_t)row * g.ldr + col;
                        for (int q = 0; q < 8 && col + q < g.N; ++q) y[q] += bf2f(rp[q]);
                    }
                }
            } else if constexpr (EPI == GEPI_GELU) {
#pragma unroll
                for (int q = 0; q < 8; ++q) y[q] = gelu_f(y[q]);
            }
            if constexpr (EPI == GEPI_ACC32) {
                float* cp = g.C32 + (int64_t)row * g.ldc + col;
                if (full) {
                    u32x4 lo = *reinterpret_cast<const u32x4*>(cp), hi = *reinterpret_cast<const u32x4*>(cp + 4);
                    lo.x = __float_as_uint(__uint_as_float(lo.x) + y[0]); lo.y = __float_as_uint(__uint_as_float(lo.y) + y[1]);
                    lo.z = __float_as_uint(__uint_as_float(lo.z) + y[2]); lo.w = __float_as_uint(__uint_as_float(lo.w) + y[3]);
                    hi.x = __float_as_uint(__uint_as_float(hi.x) + y[4]); hi.y = __float_as_uint(__uint_as_float(hi.y) + y[5]);
                    hi.z = __float_as_uint(__uint_as_float(hi.z) + y[6]); hi.w = __float_as_uint(__uint_as_float(hi.w) + y[7]);
                    *reinterpret_cast<u32x4*>(cp) = lo;
                    *reinterpret_cast<u32x4*>(cp + 4) = hi;
                } else {
                    for (int q = 0; q < 8 && col + q < g.N; ++q) cp[q] += y[q];
                }
            } else {
                bf16_t* cp = g.C + (int64_t)row * g.ldc + col;
                if (full) {
                    // written once, read by the next kernel: past the caches, so the operand panels
                    // other tiles still reuse stay in L2 (BERT-Base layer 0.1456 -> 0.1426 ms on MI355X)
                    __builtin_nontemporal_store(pack8(y), reinterpret_cast<u32x4*>(cp));
                } else {
                    for (int q = 0; q < 8 && col + q < g.N; ++q) cp[q] = f2bf(y[q]);
                }
            }
        }
    }
}

// column tiles of width bn: of the single problem, or summed over the segments of a grouped launch
int col_tiles(const GemmArgs& g, int bn) {
    if (g.nseg <= 1) return (g.N + bn - 1) / bn;
    int t = 0;
    for (int s = 0; s < g.nseg; ++s) t += (g.segs[s].N + bn - 1) / bn;
    return t;
}

template <int BM, int BN, int EPI>
fsvd_status_t launch_t(const GemmArgs& g, hipStream_t st) {
    const int tiles = ((g.M + BM - 1) / BM) * col_tiles(g, BN);
    const size_t lds = Tile<BM, BN>::LDS_BYTES;
    if (const fsvd_status_t s = allow_dynamic_lds((const void*)gemm_kernel<BM, BN, EPI>, lds, "gemm")) return s;
    gemm_kernel<BM, BN, EPI><<<tiles, kThreads, lds, st>>>(g);
    return check_launch("gemm");
}

// Tile choice: the largest tile whose grid still covers most of the 256 CUs (256 x 256 from 200
// tiles: one round on 200-256 CUs beats 1.75-3.25 rounds of 128 x 256 tiles, measured on MI355X
// for N = 1640 and 3280 at M = 8192), down to 64 x 128 for small M x N, where a big tile would leave
// most CUs idle.  The Q/K/V epilogue rotates RoPE pairs (c, c + D/2) inside one wave tile, so with
// D = 128 it needs the 128-wide wave tiles of BN = 256.
template <int EPI>
fsvd_status_t launch_epi(const GemmArgs& g, hipStream_t st) {
    auto tiles = [&](int bm, int bn) { return ((g.M + bm - 1) / bm) * col_tiles(g, bn); };
    if constexpr (EPI == GEPI_ACC32) {
        // square tiles; about half of them (below the diagonal) exit at once
        if (tiles(256, 256) >= 1024) return launch_t<256, 256, EPI>(g, st);
        return launch_t<128, 128, EPI>(g, st);
    } else {
        if constexpr (EPI == GEPI_SWIGLU) {
            if (tiles(256, 128) >= 256) return launch_t<256, 128, EPI>(g, st);
        } else if constexpr (EPI == GEPI_GELU) {
            // the exact-erf activation is a long epilogue: below 1024 tiles of 128 x 256 the smaller
            // tiles spread it over more workgroups (BERT-Base up projection, M = 4096, N = 3072,
            // K = 384: 49 -> 33.5 us on MI355X)
            if (tiles(128, 256) >= 1024) return launch_t<128, 256, EPI>(g, st);
            return launch_t<64, 128, EPI>(g, st);
        } else {
            if (tiles(256, 256) >= 200) return launch_t<256, 256, EPI>(g, st);
            // Short reductions (K <= 1024, the BERT-Base-sized projections): a tile's prologue and
            // epilogue are a large share of its time, so the tiles that win either let two
            // workgroups share a CU (64 x 128, 72 KiB of LDS), each hiding the other's, or fill
            // the CUs in one round (128 x 192).  Measured on MI355X at M = 4096: Q/K/V phase 1
            // (N 1152, K 768) 16.7 us on 128 x 192 against 21.7 on 128 x 128 and 17.7 on
            // 64 x 128; the grouped Q/K/V phase 2 (3 x N 768, K 384, D 64) 19.3 us on 64 x 128
            // against 24.0 on 128 x 256; N 384 and 768 fastest on 64 x 128.
            if (g.K <= 1024 && !(EPI == GEPI_QKV && g.D > 64)) {
                if constexpr (EPI == GEPI_STORE || EPI == GEPI_LINEAR) {
                    if (g.N % 192 == 0 && tiles(128, 192) >= 160 && tiles(128, 192) <= 256)
                        return launch_t<128, 192, EPI>(g, st);
                }
                return launch_t<64, 128, EPI>(g, st);
            }
            if (tiles(128, 256) >= 256 || (EPI == GEPI_QKV && g.D > 64)) return launch_t<128, 256, EPI>(g, st);
        }
        if (tiles(128, 128) >= 256) return launch_t<128, 128, EPI>(g, st);
        return launch_t<64, 128, EPI>(g, st);
    }
}

}  // namespace

fsvd_status_t launch_gemm(const GemmArgs& g, int epi, hipStream_t st) {
    if (g.M <= 0 || g.N <= 0) return FSVD_OK;
    if (g.K <= 0 || (epi == GEPI_SWIGLU && g.K2 <= 0)) return fail(FSVD_ERR_INVALID_ARG, "gemm: empty reduction");
    if (epi == GEPI_QKV && (g.D != 64 && g.D != 128)) return fail(FSVD_ERR_UNSUPPORTED, "RoPE epilogue needs D in {64,128}");
    if (g.nseg > 1) {
        if (epi != GEPI_QKV || g.nseg > 3) return fail(FSVD_ERR_UNSUPPORTED, "gemm: grouped launches are Q/K/V, 2-3 segments");
        for (int s = 0; s < g.nseg; ++s)
            if (g.segs[s].K <= 0 || g.segs[s].N <= 0) return fail(FSVD_ERR_INVALID_ARG, "gemm: empty segment %d", s);
    }
    switch (epi) {
        case GEPI_STORE: return launch_epi<GEPI_STORE>(g, st);
        case GEPI_LINEAR: return launch_epi<GEPI_LINEAR>(g, st);
        case GEPI_QKV: return launch_epi<GEPI_QKV>(g, st);
        case GEPI_SWIGLU: return launch_epi<GEPI_SWIGLU>(g, st);
        case GEPI_GELU: return launch_epi<GEPI_GELU>(g, st);
        case GEPI_ACC32:
            if (g.M != g.N) return fail(FSVD_ERR_INVALID_ARG, "gemm: the symmetric accumulation needs M == N");
            return launch_epi<GEPI_ACC32>(g, st);
    }
    return fail(FSVD_ERR_UNSUPPORTED, "unknown gemm epilogue %d", epi);
}

}  // namespace fsvd
