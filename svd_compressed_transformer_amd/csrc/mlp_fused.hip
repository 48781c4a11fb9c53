// Fused MLP middle for prefill (bf16 MFMA, gfx950): the up (and gate) phase 2, the activation and
// the down phase 1 in one kernel, so the d_ff-wide t never leaves the compute unit.
//
//   t   = GELU(z_u . Vt_u^T)            or  SiLU(z_g . Vt_g^T) * (z_u . Vt_u^T)
//   z_d = t . Ut_d^T
//
// A workgroup of 8 waves owns 128 token rows (16 per wave) and a slice of the d_ff columns.  Each
// wave keeps its rows' z_u (and z_g) in registers for the whole slice and walks the slice in
// chunks of 32 columns; per chunk:
//   1. t^T[32 columns, 16 rows] = Vt_u[chunk] . z_u^T on v_mfma_f32_16x16x32_bf16 (the factor chunk
//      is the A operand, read from LDS with its rows permuted so that each lane ends with 8
//      consecutive columns of one token row; z is the B operand, from registers);
//   2. the activation in fp32, rounded to bf16: those 8 values are the B-operand fragment of the
//      next product as they stand;
//   3. z_d^T[r_d, 16 rows] += Ut_d[:, chunk] . t^T, accumulated in registers over the slice (one
//      16-byte LDS read per Ut_d fragment).
// The factor chunks (Vt_u rows j0 .. j0 + 31, whole; Ut_d columns j0 .. j0 + 31 of every row) move
// global -> LDS with direct loads into three stage buffers, XOR-swizzled so the 16 rows one
// quarter-wave reads land in distinct bank groups.  Two waves share each SIMD (about 230 registers
// each), so one wave's activation and address work overlaps the other's matrix products.
//
// Parallelism: a BERT-Base-sized pass (4096 rows) has only 32 row blocks, so the d_ff columns are
// split into S slices and each (row block, slice) pair is a workgroup; every slice writes its
// partial z_d in bf16 and a small kernel sums the S partials (fp32) into z_d.  With S = 1 the
// kernel writes z_d itself.  Per row block the factors stream through L2 once per slice instead of
// once per output tile of two separate products, and t costs no HBM traffic at all.
//
// Sources: rank-aware streaming of the low-rank factors, no full-size activation buffer ("FlashSVD:
// Memory-Efficient Inference with Streaming for Low-Rank Models", abstract); the packed gate|up
// MLP feeding the down projection ("FlashSVD v1.5" explainer, Methodology 3).
#include "kernels.h"

namespace fsvd {

namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kChunk = 32;      // d_ff columns per pipeline step

// Compile-time shape of one instantiation: KU k steps of 32 for each of z_u and z_g (rank KU*32),
// ND tiles of 16 down-rank columns (r_d = ND*16), NW waves with QW sets of 16 token rows each
// (BM = 16 * NW * QW rows per workgroup).
template <bool GATE, int KU, int ND, int QW, int NW>
struct FusedShape {
    static constexpr int THREADS = 64 * NW;
    static constexpr int BM = 16 * NW * QW;
    static constexpr int CV = KU * 4;                       // 16-byte chunks per Vt row (rank KU*32)
    static constexpr int NV = GATE ? 2 : 1;                 // Vt operands (up, gate)
    static constexpr int V_SLOTS = kChunk * CV;             // per Vt operand and stage
    static constexpr int U_ROWS = ND * 16;
    static constexpr int U_SLOTS = U_ROWS * 4;              // 64 bytes (32 columns) per Ut_d row
    static constexpr int STAGE = NV * V_SLOTS + U_SLOTS;    // 16-byte slots per stage
    static constexpr int LOADS = STAGE / 64;                // wave-wide load instructions per stage
    static constexpr int LOADS_W = LOADS / NW;              // per wave
    static constexpr int NS = 3;                            // stages lc, lc + 1 in use, lc + 2 loading
    static constexpr size_t LDS = (size_t)NS * STAGE * 16;
    static_assert(CV % 16 == 0, "ranks are multiples of 128 (the Vt swizzle spans 16 chunks)");
    static_assert(LOADS % NW == 0, "each wave issues the same number of loads per stage");
    static_assert(LDS <= 160 * 1024, "stages must fit the 160 KiB of LDS");
};

// Swizzled homes of 16-byte chunk c of row r.  Vt rows (CV chunks, CV a multiple of 16): the chunk
// index is XORed with vf(r), which is distinct over the 16 rows 8a + 4jt + b (a, b < 4) that one
// quarter-wave reads for a fragment (see step 1), so they hit 16 distinct bank groups.  Ut_d rows
// (4 chunks): XOR with (r >> 2) & 3, distinct over any 16 consecutive rows' (r mod 4, r >> 2 mod 4).
__device__ __forceinline__ int vf(int r) { return (r & 3) | ((r >> 1) & 12); }
template <int CV>
__device__ __forceinline__ int v_slot(int row, int c) { return row * CV + (c ^ vf(row)); }
__device__ __forceinline__ int u_slot(int row, int c) { return row * 4 + (c ^ ((row >> 2) & 3)); }

struct FusedArgsDev {
    const bf16_t* z; int64_t ldz; int zu_off;     // z_u = z[:, zu_off : zu_off + ru], z_g = z[:, 0 : rg]
    const bf16_t* Vg; const bf16_t* Vu;           // [d_ff, rank]
    const bf16_t* Ud; int64_t ldu;                // [rd, ldu >= d_ff]
    int M, d_ff, nb, S, cps;
    bf16_t* part;                                 // [S, M, rd]
};

template <bool GATE, int KU, int ND, int QW, int NW>
__global__ __launch_bounds__(64 * NW, 1) void mlp_fused_kernel(const FusedArgsDev a) {
    using F = FusedShape<GATE, KU, ND, QW, NW>;
    constexpr int CV = F::CV, NS = F::NS, RANK = KU * 32, RD = ND * 16;
    extern __shared__ u32x4 smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: load regions are chosen per wave
    const int li = lane & 15, lg = lane >> 4;

    // workgroup -> (slice, row block): workgroup i runs on XCD i % 8 and each XCD takes a
    // contiguous range of logical items, slice-major, so an XCD's workgroups share one slice's
    // factor chunks through its L2
    const int W = a.nb * a.S;
    const int per = (W + 7) / 8, full = W - 8 * (per - 1);
    const int x = blockIdx.x & 7, local = blockIdx.x >> 3;
    const int L = (x < full) ? x * per + local : full * per + (x - full) * (per - 1) + local;
    const int slice = L / a.nb, rb = L - slice * a.nb;
    const int m0 = rb * F::BM;
    const int nch = (a.d_ff + kChunk - 1) / kChunk;
    const int c_begin = slice * a.cps, nloc = min(a.cps, nch - c_begin);

    // this wave's token rows (set q: m0 + q*16*NW + wave*16 + li) as B-operand fragments of z_u
    // (and z_g): lane (li, lg) holds z[row][kk*32 + 8*lg .. +7]
    bf16x8_v zu[QW][KU], zg[GATE ? QW : 1][GATE ? KU : 1];
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int row = min(m0 + q * 16 * NW + wave * 16 + li, a.M - 1);
        const bf16_t* zr = a.z + (int64_t)row * a.ldz;
#pragma unroll
        for (int kk = 0; kk < KU; ++kk) {
            zu[q][kk] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4*>(zr + a.zu_off + kk * 32 + lg * 8));
            if constexpr (GATE)
                zg[q][kk] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4*>(zr + kk * 32 + lg * 8));
        }
    }

    // Loads of one stage: LOADS instructions of 64 slots over [Vt_u | Vt_g | Ut_d]; wave w issues
    // instructions w * LOADS_W .. +LOADS_W - 1, each lane the global chunk whose home is its slot.
    // A lane's element offset from the chunk's first row (Vt) or column (Ut_d) is the same for every
    // chunk (loff); the chunk adds a wave-uniform base.  In a chunk that reaches past d_ff, rows past
    // it (Vt) and columns past it (Ut_d) re-read the last valid ones; the t values of those columns
    // are zeroed, so they add nothing.
    auto lane_load = [&](int i, int* r, int* c) {  // (row, column) of this lane's chunk in instruction i
        const int slot0 = (wave * F::LOADS_W + i) * 64;
        const int s = slot0 + lane;
        if (slot0 < F::NV * F::V_SLOTS) {
            const int sv = s % F::V_SLOTS;
            *r = sv / CV;
            *c = ((sv - *r * CV) ^ vf(*r)) * 8;
        } else {
            const int su = s - F::NV * F::V_SLOTS;
            *r = su >> 2;
            *c = ((su & 3) ^ ((*r >> 2) & 3)) * 8;
        }
    };
    int loff[F::LOADS_W];  // < 2^31: ranks <= 512 rows of Vt; r_d * ldu < 2^31 is checked by the planner
#pragma unroll
    for (int i = 0; i < F::LOADS_W; ++i) {
        int r, c;
        lane_load(i, &r, &c);
        loff[i] = (wave * F::LOADS_W + i) * 64 < F::NV * F::V_SLOTS ? r * RANK + c : r * (int)a.ldu + c;
    }
    auto issue = [&](int chunk, int buf) {
        const int j0 = chunk * kChunk;
        u32x4* st = smem + buf * F::STAGE;
        if (j0 + kChunk <= a.d_ff) {
#pragma unroll
            for (int i = 0; i < F::LOADS_W; ++i) {
                const int slot0 = (wave * F::LOADS_W + i) * 64;
                const bool vt = slot0 < F::NV * F::V_SLOTS;
                const bf16_t* base = vt ? (slot0 < F::V_SLOTS ? a.Vu : a.Vg) + (int64_t)j0 * RANK : a.Ud + j0;
                __builtin_amdgcn_global_load_lds((const void*)(base + loff[i]), (lds_void*)(st + slot0), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < F::LOADS_W; ++i) {
                const int slot0 = (wave * F::LOADS_W + i) * 64;
                const bool vt = slot0 < F::NV * F::V_SLOTS;
                int r, c;
                lane_load(i, &r, &c);
                const bf16_t* src = vt ? (slot0 < F::V_SLOTS ? a.Vu : a.Vg) + (int64_t)min(j0 + r, a.d_ff - 1) * RANK + c
                                       : a.Ud + (int64_t)r * a.ldu + min(j0 + c, a.d_ff - 8);
                __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(st + slot0), 16, 0, 0);
            }
        }
    };

    f32x4 acc[QW][ND];
#pragma unroll
    for (int q = 0; q < QW; ++q)
#pragma unroll
        for (int n = 0; n < ND; ++n) acc[q][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    constexpr int RING = 4;  // LDS fragment reads run RING - 1 steps ahead of the products using them
    const int pro = min(NS - 1, nloc);
    for (int c = 0; c < pro; ++c) issue(c_begin + c, c);

    for (int lc = 0; lc < nloc; ++lc) {
        // this wave's loads of stage lc have landed once at most the later stages' are in flight;
        // after the barrier every wave's have, and every wave is done with stage lc - 1, whose
        // buffer stage lc + NS - 1 takes
        wait_vm((min(lc + NS - 2, nloc - 1) - lc) * F::LOADS_W);
        lds_barrier();
        if (lc + NS - 1 < nloc) issue(c_begin + lc + NS - 1, (lc + NS - 1) % NS);
        const u32x4* st = smem + (lc % NS) * F::STAGE;
        const u32x4* sv_u = st;
        const u32x4* sv_g = st + F::V_SLOTS;
        const u32x4* su = st + F::NV * F::V_SLOTS;
        const int j0 = (c_begin + lc) * kChunk;

        // 1. t^T (and g^T) for the 32 columns.  Output row m of tile jt is column 8*(m/4) + 4*jt + m%4
        //    of the chunk (the A fragment reads that Vt row), so lane (li, lg) ends with columns
        //    8*lg + 4*jt + i of token row li: 8 consecutive columns, in order, over (jt, i)
        f32x4 tu[QW][2], tg[GATE ? QW : 1][2];
#pragma unroll
        for (int q = 0; q < QW; ++q)
#pragma unroll
            for (int jt = 0; jt < 2; ++jt) {
                tu[q][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
                if constexpr (GATE) tg[q][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        {
            bf16x8_v ru[RING][2], rg[GATE ? RING : 1][2];
            auto read_v = [&](int kk, int slotr) {
#pragma unroll
                for (int jt = 0; jt < 2; ++jt) {
                    const int vs = v_slot<CV>(8 * (li >> 2) + 4 * jt + (li & 3), kk * 4 + lg);
                    ru[slotr][jt] = __builtin_bit_cast(bf16x8_v, sv_u[vs]);
                    if constexpr (GATE) rg[slotr][jt] = __builtin_bit_cast(bf16x8_v, sv_g[vs]);
                }
            };
#pragma unroll
            for (int kk = 0; kk < RING - 1 && kk < KU; ++kk) read_v(kk, kk);
#pragma unroll
            for (int kk = 0; kk < KU; ++kk) {
                if (kk + RING - 1 < KU) read_v(kk + RING - 1, (kk + RING - 1) % RING);
#pragma unroll
                for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                    for (int q = 0; q < QW; ++q) {
                        tu[q][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ru[kk % RING][jt], zu[q][kk], tu[q][jt], 0, 0, 0);
                        if constexpr (GATE)
                            tg[q][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(rg[kk % RING][jt], zg[q][kk], tg[q][jt], 0, 0, 0);
                    }
                __builtin_amdgcn_sched_barrier(0);  // keep the read-ahead distance
            }
        }

        // 2. activation in fp32, columns past d_ff zeroed (only in the last chunk of d_ff), rounded
        //    to bf16: the B-operand fragment of step 3, k slot 8*lg + e holding column 8*lg + e
        const bool ragged = j0 + kChunk > a.d_ff;
        bf16x8_v pf[QW];
#pragma unroll
        for (int q = 0; q < QW; ++q) {
            float t[2][4];
#pragma unroll
            for (int jt = 0; jt < 2; ++jt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float u = tu[q][jt][i];
                    float v;
                    if constexpr (GATE) v = silu_f(tg[q][jt][i]) * u;
                    else v = gelu_f(u);
                    t[jt][i] = (!ragged || j0 + lg * 8 + jt * 4 + i < a.d_ff) ? v : 0.f;
                }
            pf[q] = __builtin_bit_cast(bf16x8_v, u32x4{pack_bf2(t[0][0], t[0][1]), pack_bf2(t[0][2], t[0][3]),
                                                       pack_bf2(t[1][0], t[1][1]), pack_bf2(t[1][2], t[1][3])});
        }

        // 3. z_d^T += Ut_d[:, chunk] . t^T; the Ut_d fragment of lane (li, lg) for tile n is row
        //    n*16 + li at columns 8*lg .. +7: one 16-byte chunk
        {
            bf16x8_v uf[RING];
            auto read_u = [&](int n, int slotr) { uf[slotr] = __builtin_bit_cast(bf16x8_v, su[u_slot(n * 16 + li, lg)]); };
#pragma unroll
            for (int n = 0; n < RING - 1 && n < ND; ++n) read_u(n, n);
#pragma unroll
            for (int n = 0; n < ND; ++n) {
                if (n + RING - 1 < ND) read_u(n + RING - 1, (n + RING - 1) % RING);
#pragma unroll
                for (int q = 0; q < QW; ++q)
                    acc[q][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(uf[n % RING], pf[q], acc[q][n], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // partial z_d of this slice: lane (li, lg) holds z_d[row li][n*16 + 4*lg .. +3] of tile n
    bf16_t* out = a.part + (int64_t)slice * a.M * RD;
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int row = m0 + q * 16 * NW + wave * 16 + li;
        if (row < a.M) {
            bf16_t* orow = out + (int64_t)row * RD + lg * 4;
#pragma unroll
            for (int n = 0; n < ND; ++n)
                *reinterpret_cast<uint2*>(orow + n * 16) =
                    uint2{pack_bf2(acc[q][n][0], acc[q][n][1]), pack_bf2(acc[q][n][2], acc[q][n][3])};
        }
    }
}

// z_d[m, c] = bf16(sum over s of part[s, m, c]) in fp32, 8 columns per thread
__global__ __launch_bounds__(256) void part_sum_kernel(const bf16_t* __restrict__ part, int S, int64_t n8,
                                                       bf16_t* __restrict__ out) {
    const int64_t stride8 = n8;  // slices are n8 16-byte vectors apart
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8; i += (int64_t)gridDim.x * blockDim.x) {
        float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int k = 0; k < S; ++k) {
            const u32x4 v = reinterpret_cast<const u32x4*>(part)[k * stride8 + i];
            const uint32_t e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                s[2 * j] += bf_lo(e[j]);
                s[2 * j + 1] += bf_hi(e[j]);
            }
        }
        reinterpret_cast<u32x4*>(out)[i] =
            u32x4{pack_bf2(s[0], s[1]), pack_bf2(s[2], s[3]), pack_bf2(s[4], s[5]), pack_bf2(s[6], s[7])};
    }
}

template <bool GATE, int KU, int ND, int QW, int NW>
fsvd_status_t launch_fused_t(const FusedArgsDev& d, hipStream_t st) {
    using F = FusedShape<GATE, KU, ND, QW, NW>;
    if (const fsvd_status_t s =
            allow_dynamic_lds((const void*)mlp_fused_kernel<GATE, KU, ND, QW, NW>, F::LDS, "mlp_fused"))
        return s;
    mlp_fused_kernel<GATE, KU, ND, QW, NW><<<(unsigned)(d.nb * d.S), F::THREADS, F::LDS, st>>>(d);
    return check_launch("mlp_fused");
}

// instantiated shapes: (gate, rank of z_u and z_g, r_d, rows per workgroup, waves)
struct FusedVariant {
    bool gate;
    int rank, rd, bm, nw;
    fsvd_status_t (*launch)(const FusedArgsDev&, hipStream_t);
};
const FusedVariant kVariants[] = {
    {false, 128, 128, 128, 8, launch_fused_t<false, 4, 8, 1, 8>},
    {false, 256, 256, 128, 8, launch_fused_t<false, 8, 16, 1, 8>},
    {false, 384, 384, 128, 8, launch_fused_t<false, 12, 24, 1, 8>},
    {true, 128, 128, 128, 8, launch_fused_t<true, 4, 8, 1, 8>},
    {true, 256, 256, 128, 8, launch_fused_t<true, 8, 16, 1, 8>},
};

#ifndef FSVD_FUSED_MLP
#define FSVD_FUSED_MLP 1     // 0: always the two-product path (for comparisons)
#endif

const FusedVariant* find_variant(bool gate, int rank, int rd, int nw) {
    for (const FusedVariant& v : kVariants)
        if (v.gate == gate && v.rank == rank && v.rd == rd && (nw == 0 || v.nw == nw)) return &v;
    return nullptr;
}

}  // namespace

bool mlp_fused_plan(int64_t M, int64_t rg, int64_t ru, int64_t d_ff, int64_t rd, MlpFusedPlan* p) {
    const bool gate = rg != 0;
    if (!FSVD_FUSED_MLP || M <= 0 || d_ff % 8 != 0 || (gate && rg != ru) || rd * d_ff >= (int64_t(1) << 31)) return false;
    const FusedVariant* v = find_variant(gate, (int)ru, (int)rd, 0);
    if (!v) return false;
    const int64_t nch = (d_ff + kChunk - 1) / kChunk;
    const int64_t nb = (M + v->bm - 1) / v->bm;
    // about one workgroup per CU (one fits per CU): split d_ff while the row blocks alone leave
    // CUs idle
    int64_t S = std::max<int64_t>(1, std::min<int64_t>(nch, 256 / std::max<int64_t>(nb, 1)));
    const int64_t cps = (nch + S - 1) / S;
    S = (nch + cps - 1) / cps;
    if (nb * S > INT32_MAX) return false;
    p->bm = v->bm;
    p->nw = v->nw;
    p->nb = (int)nb;
    p->S = (int)S;
    p->cps = (int)cps;
    p->part_bytes = S > 1 ? (size_t)S * M * rd * 2 : 0;
    return true;
}

fsvd_status_t launch_mlp_fused(const MlpFusedArgs& a, const MlpFusedPlan& p, hipStream_t st) {
    const bool gate = a.rg != 0;
    const FusedVariant* v = find_variant(gate, a.ru, a.rd, p.nw);
    if (!v) return fail(FSVD_ERR_UNSUPPORTED, "fused MLP: no kernel for rank %d, r_d %d", a.ru, a.rd);
    if (!aligned16(a.z) || !aligned16(a.Vu) || !aligned16(a.Ud) || (gate && !aligned16(a.Vg)) || !aligned16(a.z_d) ||
        (p.S > 1 && !aligned16(a.part)) || a.ldz % 8 || a.ldu % 8)
        return fail(FSVD_ERR_INVALID_ARG, "fused MLP: operands must be 16-byte aligned");
    FusedArgsDev d{};
    d.z = a.z; d.ldz = a.ldz; d.zu_off = a.rg;
    d.Vg = a.Vg; d.Vu = a.Vu; d.Ud = a.Ud; d.ldu = a.ldu;
    d.M = a.M; d.d_ff = a.d_ff; d.nb = p.nb; d.S = p.S; d.cps = p.cps;
    d.part = p.S > 1 ? a.part : a.z_d;
    if (const fsvd_status_t s = v->launch(d, st)) return s;
    if (p.S == 1) return FSVD_OK;
    const int64_t n8 = (int64_t)a.M * a.rd / 8;
    const int grid = (int)std::min<int64_t>((n8 + 255) / 256, 256 * 8);
    part_sum_kernel<<<grid, 256, 0, st>>>(a.part, p.S, n8, a.z_d);
    return check_launch("mlp_fused_sum");
}

}  // namespace fsvd
