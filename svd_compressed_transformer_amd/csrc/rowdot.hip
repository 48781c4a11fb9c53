// Decode-size (M <= 32 activation rows) low-rank projection kernels for gfx950.
//
// At decode the fused projection y = (x . U) . V is bound by streaming the factor bytes once
// from HBM (about M flop per factor byte, far below the MFMA ridge), so each phase is a
// "row-dot": every output n is the dot product of one K-contiguous factor row with the M
// activation rows.  A wave owns R rows; each lane loads 16 contiguous bytes of every row per
// step (one wave instruction = a 1 KiB coalesced segment of each row), multiplies them with the
// matching activation bytes using v_dot2_f32_bf16 (fp32 accumulation), and the 64 lanes are
// reduced with DPP row operations plus a small LDS combine.  Measured on MI355X, these streams are
// bound by how many bytes are in flight and by the activation re-reads, not by arithmetic: a wave
// owns 4 rows (each activation load feeds 4 rows), issues its loads in passes of 1-4 steps, and
// long reductions are split over the 4-8 waves of a workgroup, giving thousands of short waves.
//
// Phase 1 (z = a . Ut^T, EPI_Z) fuses the RMSNorm prologue: the sum of squares of each
// activation row is accumulated in the same pass and z is scaled by rstd at the end.  Phase 2
// epilogues: linear (+bias, +residual), Q/K/V (rotate-half RoPE and the dense KV-cache append,
// a bit copy of the bf16 value), SwiGLU (gate and up rows of one output column are owned by the
// same wave) and GELU.
//
// Sources: fused low-rank projection ("FlashSVD: Memory-Efficient Inference with Streaming for
// Low-Rank Models", abstract); current-token Q/K/V reconstruction into a dense cache and the
// packed gate|up projection ("FlashSVD v1.5" explainer, Methodology 2 and 3).
#include <type_traits>

#include "kernels.h"

namespace fsvd {

namespace {

#ifndef FSVD_ROWS
#define FSVD_ROWS 4
#endif
constexpr int kR = FSVD_ROWS;  // factor rows per wave (even)
constexpr int kH = kR / 2;     // paired units per wave
constexpr int kMaxWaves = 8; // waves per workgroup (4 or 8, chosen per launch)
#ifndef FSVD_RD_KPW
#define FSVD_RD_KPW 1024    // longest reduction slice per wave before the reduction is split
#endif
#ifndef FSVD_RD_WAVES
#define FSVD_RD_WAVES 2048  // the split is doubled while the launch has fewer waves than this
#endif
constexpr size_t kRdPartBytes = (size_t)1280 * 1024;  // split-reduction partial tiles per launch

template <typename T>
struct Vec;
template <>
struct Vec<bf16_t> {
    static constexpr int E = 8;
};
template <>
struct Vec<float> {
    static constexpr int E = 4;
};

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// factor bytes are read exactly once: stream them past the caches so the activation rows, which
// every wave re-reads, stay resident
#ifndef FSVD_WEIGHT_NT
#define FSVD_WEIGHT_NT 1
#endif
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
#if FSVD_WEIGHT_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
    return *reinterpret_cast<const u32x4*>(p);
#endif
}

__device__ __forceinline__ float vdot(u32x4 w, u32x4 a, float c, bf16_t) {
    c = dot2bf(w.x, a.x, c);
    c = dot2bf(w.y, a.y, c);
    c = dot2bf(w.z, a.z, c);
    c = dot2bf(w.w, a.w, c);
    return c;
}
__device__ __forceinline__ float vdot(u32x4 w, u32x4 a, float c, float) {
    c = fmaf(__uint_as_float(w.x), __uint_as_float(a.x), c);
    c = fmaf(__uint_as_float(w.y), __uint_as_float(a.y), c);
    c = fmaf(__uint_as_float(w.z), __uint_as_float(a.z), c);
    c = fmaf(__uint_as_float(w.w), __uint_as_float(a.w), c);
    return c;
}

// sum of squares of a 16-byte activation vector (RMSNorm statistics): x . x with v_dot2, added to s
__device__ __forceinline__ float vsq(u32x4 a, float s, bf16_t) { return vdot(a, a, s, bf16_t()); }
__device__ __forceinline__ float vsq(u32x4 a, float s, float) { return vdot(a, a, s, float()); }
// a * w rounded to bf16 (the norm weight applied before the product)
__device__ __forceinline__ u32x4 vmulw(u32x4 a, u32x4 w) {
    u32x4 r;
    r.x = pack_bf2(bf_lo(a.x) * bf_lo(w.x), bf_hi(a.x) * bf_hi(w.x));
    r.y = pack_bf2(bf_lo(a.y) * bf_lo(w.y), bf_hi(a.y) * bf_hi(w.y));
    r.z = pack_bf2(bf_lo(a.z) * bf_lo(w.z), bf_hi(a.z) * bf_hi(w.z));
    r.w = pack_bf2(bf_lo(a.w) * bf_lo(w.w), bf_hi(a.w) * bf_hi(w.w));
    return r;
}

template <typename T>
__device__ __forceinline__ void store_t(void* base, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_t<bf16_t>(void* base, int64_t idx, float v) {
    reinterpret_cast<bf16_t*>(base)[idx] = f2bf(v);
}
template <>
__device__ __forceinline__ void store_t<float>(void* base, int64_t idx, float v) {
    reinterpret_cast<float*>(base)[idx] = v;
}
template <typename T>
__device__ __forceinline__ float load_t(const void* base, int64_t idx);
template <>
__device__ __forceinline__ float load_t<bf16_t>(const void* base, int64_t idx) {
    return bf2f(reinterpret_cast<const bf16_t*>(base)[idx]);
}
template <>
__device__ __forceinline__ float load_t<float>(const void* base, int64_t idx) {
    return reinterpret_cast<const float*>(base)[idx];
}

// Q and K rows are owned in RoPE pairs (both rows of a pair in one wave, one output unit)
__host__ __device__ __forceinline__ bool seg_paired(int epi, int kind) {
    return epi == EPI_QKV && (kind == SEG_Q || kind == SEG_K);
}
// SwiGLU: the gate rows and the up rows of the same kR output columns are owned by two sibling
// wave sets (each wave reads one activation vector, z_gate or z_up), joined in the LDS combine
__host__ __device__ __forceinline__ int wave_sets(int epi) { return epi == EPI_SWIGLU ? 2 : 1; }

// Epilogue shared by the row-dot kernels: output unit j of unit group g for activation row m, from
// the fully reduced values val(g, h, r, m) (h: wave set, r: factor row within the group) and, in
// phase 1 with the RMSNorm prologue, the activation row's sum of squares ssq(g, m).  A RoPE pair's
// second row sits pair_off rows after its first.  Threads tid, tid + nthreads, ... share the
// (g, j, m) triples of the workgroup.
template <typename T, int EPI, class Val, class Ssq>
__device__ __forceinline__ void rowdot_epilogue(const RowdotArgs& a, const RowdotSeg& sg, int unit_base, int ngroups,
                                                int upw, int pair_off, int n_units, int tid, int nthreads, Val val,
                                                Ssq ssq) {
    const int M = a.M;
    const int halfD = a.D >> 1;
    const int total = ngroups * upw * M;
    for (int idx = tid; idx < total; idx += nthreads) {
        const int g = idx / (upw * M);
        const int rem = idx - g * upw * M;
        const int j = rem / M;           // unit within the wave
        const int m = rem - j * M;       // activation row
        const int u = unit_base + g * upw + j;
        if (u >= n_units) continue;
        if constexpr (EPI == EPI_Z) {
            float v = val(g, 0, j, m);
            if (a.norm) {
                const float sq = ssq(g, m);
                v *= 1.0f / sqrtf(sq / (float)a.norm_K + a.norm_eps);
            }
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, v);
        } else if constexpr (EPI == EPI_LINEAR) {
            float v = val(g, 0, j, m);
            if (a.bias) v += load_t<T>(a.bias, u);
            if (a.residual) v += load_t<T>(a.residual, (int64_t)m * a.ldr + u);
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, v);
        } else if constexpr (EPI == EPI_GELU) {
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, gelu_f(val(g, 0, j, m)));
        } else if constexpr (EPI == EPI_SWIGLU) {
            const float gv = val(g, 0, j, m), uv = val(g, 1, j, m);
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, silu_f(gv) * uv);
        } else if constexpr (EPI == EPI_QKV) {
            const int b = m / a.S, s = m - b * a.S;
            const int64_t p = (int64_t)a.seqlens[b] + s;
            const bool in_cache = p >= 0 && p < a.L_max;
            if (sg.kind == SEG_V) {
                const bf16_t bits = f2bf(val(g, 0, j, m));
                const int hd = a.Hkv * a.D;
                if (in_cache) a.v_cache[((int64_t)b * a.L_max + p) * hd + u] = bits;
                else set_dev_error(a.err, FSVD_DEVERR_KV_OVERFLOW);
                if (a.v_out) a.v_out[(int64_t)m * hd + u] = bits;
            } else {
                const float x1 = val(g, 0, j, m), x2 = val(g, 0, j + pair_off, m);
                const int h = u / halfD, i = u - h * halfD;
                const int n1 = h * a.D + i, n2 = n1 + halfD;
                float y1 = x1, y2 = x2;
                if (a.rope_theta > 0.f) {
                    float c, sn;
                    rope_cs(p, i, a.rope_base, &c, &sn);
                    y1 = x1 * c - x2 * sn;
                    y2 = x2 * c + x1 * sn;
                }
                const bf16_t b1 = f2bf(y1), b2 = f2bf(y2);
                if (sg.kind == SEG_Q) {
                    bf16_t* q = reinterpret_cast<bf16_t*>(sg.out);
                    q[(int64_t)m * sg.ldo + n1] = b1;
                    q[(int64_t)m * sg.ldo + n2] = b2;
                } else {
                    const int hd = a.Hkv * a.D;
                    if (in_cache) {
                        bf16_t* kc = a.k_cache + ((int64_t)b * a.L_max + p) * hd;
                        kc[n1] = b1;
                        kc[n2] = b2;
                    } else {
                        set_dev_error(a.err, FSVD_DEVERR_KV_OVERFLOW);
                    }
                    if (a.k_out) {
                        a.k_out[(int64_t)m * hd + n1] = b1;
                        a.k_out[(int64_t)m * hd + n2] = b2;
                    }
                }
            }
        }
    }
}


// NW: phase 1 with an RMSNorm weight to apply to the activation (its loads and registers are left
// out when the weight is folded into the factor or there is no norm: at 3-4 activation rows that
// keeps the kernel at 96 registers, 5 waves per SIMD instead of 4)
template <typename T, int BMAX, int EPI, bool NW = true>
__global__ __launch_bounds__(BMAX >= 32 ? 256 : 512) void rowdot_kernel(const RowdotArgs a) {
    constexpr int E = Vec<T>::E;
    // the wave index is uniform across the wave; saying so keeps every per-wave quantity (row
    // pointers, reduction bounds, step counts) in scalar registers and its branches scalar
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bid = blockIdx.x;

    // only the Q/K/V launch has several segments; the others read segment 0 directly (one round
    // of argument loads instead of two dependent ones)
    const int si = EPI != EPI_QKV ? 0
                   : ((a.nseg > 2 && bid >= a.seg[2].blk_begin) ? 2 : ((a.nseg > 1 && bid >= a.seg[1].blk_begin) ? 1 : 0));
    const RowdotSeg sg = EPI != EPI_QKV ? a.seg[0] : (si == 0 ? a.seg[0] : (si == 1 ? a.seg[1] : a.seg[2]));

    const bool paired = seg_paired(EPI, sg.kind);
    const int upw = paired ? kH : kR;                             // output units per wave
    const int n_units = (EPI == EPI_QKV && paired) ? sg.N / 2 : sg.N;
    const int ksplit = a.ksplit;
    constexpr int NS = EPI == EPI_SWIGLU ? 2 : 1;                 // wave sets per unit group
    const int grp = wave / (NS * ksplit);
    const int half = (wave / ksplit) % NS;                        // SwiGLU: 0 = gate, 1 = up
    const int ks = wave % ksplit;
    const int unit0 = (bid - sg.blk_begin) * sg.units_per_blk + grp * upw;
    const int halfD = a.D >> 1;

    // rows owned by this wave: paired units (RoPE pair, or gate/up of one column) use both rows
    // for one output unit; plain segments give each row its own unit
    const char* wrow[kR];
    int klen[kR];
    int aoff[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        int u, n;
        const int mat = EPI == EPI_SWIGLU ? half : 0;
        if (paired) {
            u = unit0 + r % kH;
            const int h = u / halfD, i = u - h * halfD;
            n = h * a.D + i + (r / kH) * halfD;
        } else {
            u = unit0 + r;
            n = u;
        }
        const bool valid = u < n_units;
        const void* W = mat ? sg.W2 : sg.W;
        const int64_t ld = mat ? sg.ldw2 : sg.ldw;
        wrow[r] = reinterpret_cast<const char*>(W) + (valid ? (int64_t)n * ld * (int64_t)sizeof(T) : 0);
        klen[r] = valid ? (mat ? sg.K2 : sg.K) : 0;
        aoff[r] = mat ? sg.act_off2 : sg.act_off;
    }
    // This wave's slice of the reduction: whole steps of 64 lanes x E elements (one 1 KiB segment
    // of a row per wave instruction), only the group's last slice can end inside a step.
    constexpr int SE = 64 * E;
    const int kmax = (EPI == EPI_SWIGLU) ? max(sg.K, sg.K2) : sg.K;
    const int st_per = ((kmax + SE - 1) / SE + ksplit - 1) / ksplit;  // steps per wave
    const int k_lo = ks * st_per * SE;
    const int k_hi = min(kmax, k_lo + st_per * SE);
    const int kw = EPI == EPI_SWIGLU ? (half ? sg.K2 : sg.K) : sg.K;  // length of this wave's rows
    const int k_end = min(k_hi, kw);                                  // products for k < k_end
    const int kc_max = kw - E;                                        // clamp for loads past it

    float acc[kR][BMAX];
    float ss[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        ss[b] = 0.f;
#pragma unroll
        for (int r = 0; r < kR; ++r) acc[r][b] = 0.f;
    }
    const int M = a.M;
    const int64_t lda_b = a.lda * (int64_t)sizeof(T);
    const bool norm = (EPI == EPI_Z) && a.norm;
    const bool norm_w = NW && norm && a.norm_w != nullptr;
    // activation rows past M re-read row M - 1 (their results are never stored); without a norm
    // weight its loads read the activation instead (valid memory, value unused)
    const char* arow[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b)
        arow[b] = reinterpret_cast<const char*>(a.act) + min(b, M - 1) * lda_b + (int64_t)aoff[0] * sizeof(T);
    const char* nwp = norm_w ? reinterpret_cast<const char*>(a.norm_w) : arow[0];

    // Passes of up to U steps.  Every load is unconditional (addresses clamped to valid elements),
    // so all of a pass's loads are in flight before its first product and no lane test or zero
    // fill runs in the common case; lanes past k_end get a zero activation (a wave's last pass).
    constexpr int U = BMAX <= 2 ? 4 : (BMAX <= 8 ? 2 : 1);
    const int nsteps = k_hi > k_lo ? (k_hi - k_lo + SE - 1) / SE : 0;
    auto pass = [&](auto nu_c, int s0) {
        constexpr int NU = decltype(nu_c)::value;  // steps in this pass
        u32x4 wv[NU][kR];
        u32x4 av[NU][BMAX];
        u32x4 nw[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int k = k_lo + ((s0 + u) * 64 + lane) * E;
            const int64_t kc = (int64_t)min(k, kc_max) * sizeof(T);
#pragma unroll
            for (int r = 0; r < kR; ++r) wv[u][r] = ldg16_stream(wrow[r] + kc);
            if constexpr (EPI == EPI_Z && NW) nw[u] = ldg16(nwp + kc);
#pragma unroll
            for (int b = 0; b < BMAX; ++b) av[u][b] = ldg16(arow[b] + kc);
        }
        if (k_lo + (s0 + NU) * SE > k_end) {  // wave-uniform: the pass reaches past k_end
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const bool ok = k_lo + ((s0 + u) * 64 + lane) * E < k_end;
#pragma unroll
                for (int b = 0; b < BMAX; ++b) av[u][b] = ok ? av[u][b] : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < NU; ++u) {
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                u32x4 x = av[u][b];
                if constexpr (EPI == EPI_Z) {
                    if (norm) {
                        ss[b] = vsq(x, ss[b], T());
                        if constexpr (NW) {
                            if (norm_w) x = vmulw(x, nw[u]);
                        }
                    }
                }
#pragma unroll
                for (int r = 0; r < kR; ++r) acc[r][b] = vdot(wv[u][r], x, acc[r][b], T());
            }
        }
    };
    // passes of U steps, then the rest of the slice in one pass, so all of its loads are in flight
    // together (no step past the slice is loaded).  With 1-2 activation rows (U = 4) a wave's slice
    // is usually 2 steps: one pass of 2, not two passes of 1 whose second waits for the first.
    int s0 = 0;
    for (; s0 + U <= nsteps; s0 += U) pass(std::integral_constant<int, U>(), s0);
    const int rest = nsteps - s0;  // 0 .. U - 1, wave-uniform
    if constexpr (U >= 4) {
        if (rest == 3) pass(std::integral_constant<int, 3>(), s0);
        else if (rest == 2) pass(std::integral_constant<int, 2>(), s0);
        else if (rest == 1) pass(std::integral_constant<int, 1>(), s0);
    } else {
        for (; s0 < nsteps; ++s0) pass(std::integral_constant<int, 1>(), s0);
    }

    // Cross-lane reduction: a reduce-scatter over each 16-lane row leaves every lane with the row
    // sums of its own block of the wave's values (the kR x BMAX products and, in phase 1, the BMAX
    // sums of squares); the 4 rows of a wave and the ksplit waves of a unit are summed from LDS.
    constexpr int NV = (EPI == EPI_Z ? kR + 1 : kR) * BMAX;
    constexpr int VP = pow2_ceil(NV);
    float vals[VP];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
#pragma unroll
        for (int r = 0; r < kR; ++r) vals[r * BMAX + b] = acc[r][b];
        if constexpr (EPI == EPI_Z) vals[kR * BMAX + b] = ss[b];
    }
#pragma unroll
    for (int i = NV; i < VP; ++i) vals[i] = 0.f;
    row16_reduce_scatter<VP>(vals, lane);
    __shared__ float red[kMaxWaves][4][VP];
    {
        float* dst = &red[wave][lane >> 4][rs16_first<VP>(lane)];
#pragma unroll
        for (int i = 0; i < rs16_count<VP>(); ++i) dst[i] = vals[i];
    }
    __syncthreads();

    if constexpr (EPI == EPI_LINEAR) {
        if (a.adv_seqlens != nullptr && bid == 0 && tid < a.adv_B) a.adv_seqlens[tid] += a.adv_n;
    }

    // value r (row or statistic) of unit group g, wave set h, activation row b: the sum over the
    // ksplit waves of that set and their 4 DPP rows
    auto val = [&](int g, int h, int r, int b) -> float {
        const int w0 = (g * NS + h) * ksplit;
        const int vi = r * BMAX + b;
        float s = 0.f;
        // all reads issued together: waves past the group's ksplit read a valid slot, weighted 0
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) {
            const float* e = &red[min(w0 + w, kMaxWaves - 1)][0][vi];
            const float t = (e[0] + e[VP]) + (e[2 * VP] + e[3 * VP]);
            s += w < ksplit ? t : 0.f;
        }
        return s;
    };

    rowdot_epilogue<T, EPI>(a, sg, (bid - sg.blk_begin) * sg.units_per_blk, a.waves / (NS * ksplit), upw, kH, n_units,
                            tid, 64 * a.waves, val, [&](int g, int m) { return val(g, 0, kR, m); });
}

// Skinny-MFMA variant for 5..32 activation rows (bf16).  Past about 4 rows the row-dot's dot
// products, which grow with the number of activation rows while the factor bytes do not, make
// the kernel vector-ALU bound (measured on MI355X: the instruction count and the time grow with
// the batch).  Here a wave owns a tile of 16 factor rows and its products run on the matrix
// cores as v_mfma_f32_16x16x32_bf16: the B operand is 16 factor rows x 32 k (lane l holds 8
// consecutive k of row l % 16 at k group l / 16), read from a wave-private LDS stage that the
// pass fills with row-contiguous direct loads; the A operand is 16 activation rows x 32 k with
// the same k groups (MB = 2 tiles for 17..32 rows); C[m][row] accumulates in fp32.  The k split
// over waves, the RMSNorm statistics and the epilogues are those of the row-dot; the partial
// tiles of the waves that split k are summed from LDS.
typedef __bf16 bf16x8_m __attribute__((ext_vector_type(8)));
typedef float f32x4_m __attribute__((ext_vector_type(4)));
constexpr int kMfmaRows = 16;  // factor rows per wave tile
constexpr int kAuxNonTemporal = 2;  // cache-policy operand of the direct-to-LDS load: nt
constexpr int kMfmaSteps = 8;  // 32-wide k steps whose loads one pass keeps in flight (16 activation rows)
// Factor rows of a pass staged through a wave-private LDS buffer with row-contiguous loads (an
// instruction reads 512 or 256 contiguous bytes of each of 2 or 4 rows) instead of loading the
// MFMA operand layout directly (64 bytes of each of 16 rows per instruction).  Measured on MI355X
// with a plain stream of the same bytes and waves: 4.8-5.4 TB/s against 3.0-4.4 TB/s.
typedef __attribute__((address_space(3))) void lds_void_rd;
template <int MB>
constexpr int mfma_pass_steps() { return MB == 1 ? kMfmaSteps : kMfmaSteps / 2; }
// 16-byte slots of one wave's stage: 16 rows x (steps x 32 elements x 2 bytes / 16)
template <int MB>
constexpr int mfma_stage_slots() { return kMfmaRows * mfma_pass_steps<MB>() * 4; }

// Segment of workgroup tile blk (Q/K/V launches hold up to three)
template <int EPI>
__device__ __forceinline__ RowdotSeg seg_of(const RowdotArgs& a, int blk) {
    const int si = EPI != EPI_QKV ? 0
                   : ((a.nseg > 2 && blk >= a.seg[2].blk_begin) ? 2 : ((a.nseg > 1 && blk >= a.seg[1].blk_begin) ? 1 : 0));
    return EPI != EPI_QKV ? a.seg[0] : (si == 0 ? a.seg[0] : (si == 1 ? a.seg[1] : a.seg[2]));
}

// Values one tile of workgroups leaves when its reduction is split over kpart workgroups: the
// k-split-reduced C values (g, h, r, m) and the RMSNorm sums of squares (g, m).
__host__ __device__ inline int part_vals(int ngroups, int ns) { return ngroups * ns * kMfmaRows * 32 + ngroups * 32; }
__host__ __device__ inline int part_val_idx(int g, int h, int r, int m, int ns) { return ((g * ns + h) * kMfmaRows + r) * 32 + m; }
__host__ __device__ inline int part_ss_idx(int g, int m, int ngroups, int ns) { return ngroups * ns * kMfmaRows * 32 + g * 32 + m; }

// Finishes tile blk of a split reduction: sums its kpart partial tiles in part order and runs the
// epilogue of the unsplit kernel on them (same threads, same unit mapping).  The partials were
// written in the same kernel by workgroups on any XCD, so they are read with agent-scope loads.
template <int EPI>
__device__ __forceinline__ void finish_split_tile(const RowdotArgs& a, int blk, int tid) {
    using T = bf16_t;
    const RowdotSeg sg = seg_of<EPI>(a, blk);
    constexpr int NS = EPI == EPI_SWIGLU ? 2 : 1;
    const bool paired = seg_paired(EPI, sg.kind);
    const int upw = paired ? kMfmaRows / 2 : kMfmaRows;
    const int n_units = (EPI == EPI_QKV && paired) ? sg.N / 2 : sg.N;
    const int ngroups = a.waves / (NS * a.ksplit);
    const int nv = part_vals(ngroups, NS);
    const float* src = a.part + (int64_t)blk * nv;
    const int64_t pstride = (int64_t)a.nblk * nv;
    auto sum_parts = [&](int idx) -> float {
        float s = 0.f;
        for (int p = 0; p < a.kpart; ++p) {
            s += __hip_atomic_load(src + p * pstride + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return s;
    };
    auto val = [&](int g, int h, int r, int m) -> float { return sum_parts(part_val_idx(g, h, r, m, NS)); };
    auto ssq = [&](int g, int m) -> float { return sum_parts(part_ss_idx(g, m, ngroups, NS)); };
    if constexpr (EPI == EPI_LINEAR) {
        if (a.adv_seqlens != nullptr && blk == 0 && tid < a.adv_B) a.adv_seqlens[tid] += a.adv_n;
    }
    rowdot_epilogue<T, EPI>(a, sg, (blk - sg.blk_begin) * sg.units_per_blk, ngroups, upw, kMfmaRows / 2, n_units, tid,
                            64 * a.waves, val, ssq);
}

template <int MB, int EPI, bool DB>
__global__ __launch_bounds__(512) void rowdot_mfma_kernel(const RowdotArgs a) {
    using T = bf16_t;
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroup = (tile blk, reduction part kp): with kpart > 1 the reduction of a tile is split
    // over kpart workgroups whose partial tiles a second kernel sums
    const int bid = (a.kpart > 1) ? (int)(blockIdx.x % a.nblk) : (int)blockIdx.x;
    const int kp = (a.kpart > 1) ? (int)(blockIdx.x / a.nblk) : 0;
    const int si = EPI != EPI_QKV ? 0
                   : ((a.nseg > 2 && bid >= a.seg[2].blk_begin) ? 2 : ((a.nseg > 1 && bid >= a.seg[1].blk_begin) ? 1 : 0));
    const RowdotSeg sg = EPI != EPI_QKV ? a.seg[0] : (si == 0 ? a.seg[0] : (si == 1 ? a.seg[1] : a.seg[2]));

    const bool paired = seg_paired(EPI, sg.kind);
    const int upw = paired ? kMfmaRows / 2 : kMfmaRows;           // output units per wave tile
    const int n_units = (EPI == EPI_QKV && paired) ? sg.N / 2 : sg.N;
    const int ksplit = a.ksplit;
    constexpr int NS = EPI == EPI_SWIGLU ? 2 : 1;
    const int grp = wave / (NS * ksplit);
    const int half = (wave / ksplit) % NS;
    const int ks = wave % ksplit;
    const int unit0 = (bid - sg.blk_begin) * sg.units_per_blk + grp * upw;
    const int halfD = a.D >> 1;

    // this lane's factor row (column rj of the B operand) and k group kq
    const int rj = lane & 15, kq = lane >> 4;
    const int mat = EPI == EPI_SWIGLU ? half : 0;
    int u, n;
    if (paired) {  // rows 0..7: first halves of 8 RoPE pairs, rows 8..15: their partners
        u = unit0 + (rj & 7);
        const int h = u / halfD, i = u - h * halfD;
        n = h * a.D + i + (rj >> 3) * halfD;
    } else {
        u = unit0 + rj;
        n = u;
    }
    const bool valid = u < n_units;
    const char* W = reinterpret_cast<const char*>(mat ? sg.W2 : sg.W);
    const int64_t ldw = mat ? sg.ldw2 : sg.ldw;
    // factor row of tile row j (the staged loads give a lane rows other than its own column rj)
    auto row_ptr = [&](int j) -> const char* {
        int uj, nj;
        if (paired) {
            uj = unit0 + (j & 7);
            const int h = uj / halfD, i = uj - h * halfD;
            nj = h * a.D + i + (j >> 3) * halfD;
        } else {
            uj = unit0 + j;
            nj = uj;
        }
        return W + (uj < n_units ? (int64_t)nj * ldw * (int64_t)sizeof(T) : 0);
    };
    extern __shared__ u32x4 rd_stage[];
    u32x4* stg = rd_stage + wave * mfma_stage_slots<MB>() * (DB ? 2 : 1);  // this wave's stage(s)

    constexpr int SE = 32;  // k per MFMA step
    const int kmax = (EPI == EPI_SWIGLU) ? max(sg.K, sg.K2) : sg.K;
    const int nparts = ksplit * a.kpart;  // slices of the reduction: ksplit waves x kpart workgroups
    const int st_per = ((kmax + SE - 1) / SE + nparts - 1) / nparts;
    const int k_lo = (kp * ksplit + ks) * st_per * SE;
    const int k_hi = min(kmax, k_lo + st_per * SE);
    const int kw = EPI == EPI_SWIGLU ? (half ? sg.K2 : sg.K) : sg.K;
    const int k_end = min(k_hi, kw);
    const int kc_max = kw - 8;

    const int M = a.M;
    const int64_t lda_b = a.lda * (int64_t)sizeof(T);
    const int aoff = mat ? sg.act_off2 : sg.act_off;
    const bool norm = (EPI == EPI_Z) && a.norm;
    const bool norm_w = norm && a.norm_w != nullptr;
    const char* arow[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
        arow[mb] = reinterpret_cast<const char*>(a.act) + min(mb * 16 + rj, M - 1) * lda_b + (int64_t)aoff * sizeof(T);
    const char* nwp = norm_w ? reinterpret_cast<const char*>(a.norm_w) : arow[0];

    f32x4_m acc[MB];
    float ss[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        acc[mb] = f32x4_m{0.f, 0.f, 0.f, 0.f};
        ss[mb] = 0.f;
    }
    const int nsteps = k_hi > k_lo ? (k_hi - k_lo + SE - 1) / SE : 0;
    // Whole passes of U steps (a shorter last pass would cost one round trip per step); steps past
    // the slice load clamped addresses (cache hits) and are zeroed by the activation mask.  The
    // factor rows of a pass go to the wave's stage: slot s holds row j = s / CPR, chunk
    // c = (s % CPR) ^ j of the pass (CPR = 4 U chunks of 16 bytes per row, a power of two >= 16 > j).
    constexpr int U = mfma_pass_steps<MB>();
    constexpr int CPR = U * 4, NI = kMfmaRows * CPR / 64, SLOTS = mfma_stage_slots<MB>();
    const int npass = (nsteps + U - 1) / U;
    auto stage = [&](int p, u32x4* dst) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int sl = i * 64 + lane, j = sl / CPR, c = (sl % CPR) ^ j;
            const int k = min(k_lo + p * U * SE + c * 8, kc_max);
            // factor rows are read once: the non-temporal policy bit (measured on MI355X, batch 8
            // layer-step 147.9 -> 144.6 us, batch 16 203.5 -> 201.3 us)
            __builtin_amdgcn_global_load_lds((const void*)(row_ptr(j) + (int64_t)k * sizeof(T)),
                                             (lds_void_rd*)(dst + i * 64), 16, 0, kAuxNonTemporal);
        }
    };
    if (npass > 0) stage(0, stg);
    for (int p = 0; p < npass; ++p) {
        const int s0 = p * U;
        u32x4 nw[U], av[U][MB];
#pragma unroll
        for (int q = 0; q < U; ++q) {
            const int k = k_lo + (s0 + q) * SE + kq * 8;
            const int64_t kc = (int64_t)min(k, kc_max) * sizeof(T);
            if (norm_w) nw[q] = ldg16(nwp + kc);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) av[q][mb] = ldg16(arow[mb] + kc);
        }
        if (k_lo + (s0 + U) * SE > k_end) {  // wave-uniform: the pass reaches past k_end
#pragma unroll
            for (int q = 0; q < U; ++q) {
                const bool ok = k_lo + (s0 + q) * SE + kq * 8 < k_end;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb) av[q][mb] = ok ? av[q][mb] : u32x4{0u, 0u, 0u, 0u};
            }
        }
        wait_vm(0);  // this pass's staged rows and activations have landed (private stage: no barrier)
        const u32x4* cur = stg + (DB ? (p & 1) * SLOTS : 0);
        u32x4 wv[U];
        if constexpr (DB) {
            // double-buffered: every fragment of this pass is read before the next pass's loads are
            // issued into the other buffer, so no read of the stage overlaps loads in flight
#pragma unroll
            for (int q = 0; q < U; ++q) wv[q] = cur[rj * CPR + ((q * 4 + kq) ^ rj)];
            if (p + 1 < npass) stage(p + 1, stg + ((p + 1) & 1) * SLOTS);
        }
#pragma unroll
        for (int q = 0; q < U; ++q) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                u32x4 x = av[q][mb];
                if constexpr (EPI == EPI_Z) {
                    if (norm) {
                        ss[mb] = vsq(x, ss[mb], T());
                        if (norm_w) x = vmulw(x, nw[q]);
                    }
                }
                if constexpr (!DB) {
                    if (mb == 0) wv[q] = cur[rj * CPR + ((q * 4 + kq) ^ rj)];  // B fragment of step q
                }
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_m, x),
                                                                   __builtin_bit_cast(bf16x8_m, wv[q]), acc[mb], 0, 0, 0);
            }
        }
        // single buffer: refill once this pass's reads have been consumed by the products
        if constexpr (!DB) {
            if (p + 1 < npass) stage(p + 1, stg);
        }
    }

    // C tile of this wave: lane holds C[m = 16 mb + 4 kq + e][row rj]; the k-split waves of a unit
    // group are summed from LDS.  Sums of squares: over the 4 k groups of an activation row.  The
    // combine arrays reuse the stage buffers once every wave is past its last pass.
    __syncthreads();
    float (*red)[32][kMfmaRows] = reinterpret_cast<float (*)[32][kMfmaRows]>(rd_stage);
    float (*red_ss)[32] = reinterpret_cast<float (*)[32]>(reinterpret_cast<float*>(rd_stage) + kMaxWaves * 32 * kMfmaRows);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][mb * 16 + kq * 4 + e][rj] = acc[mb][e];
    if (norm) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            float v = ss[mb];
            v += __shfl_xor(v, 16);
            v += __shfl_xor(v, 32);
            if (kq == 0) red_ss[wave][mb * 16 + rj] = v;
        }
    }
    __syncthreads();

    auto sum_waves = [&](int w0, auto get) -> float {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kMaxWaves; ++w) {
            const float t = get(min(w0 + w, kMaxWaves - 1));
            s += w < ksplit ? t : 0.f;
        }
        return s;
    };
    auto val = [&](int g, int h, int r, int m) -> float {
        return sum_waves((g * NS + h) * ksplit, [&](int w) { return red[w][m][r]; });
    };
    auto ssq = [&](int g, int m) -> float {
        return sum_waves(g * NS * ksplit, [&](int w) { return red_ss[w][m]; });
    };
    const int ngroups = a.waves / (NS * ksplit);
    if (a.kpart > 1) {  // partial tile of this reduction part
        const int nv = part_vals(ngroups, NS);
        float* dst = a.part + ((int64_t)kp * a.nblk + bid) * nv;
        for (int idx = tid; idx < nv; idx += 64 * a.waves) {
            const int nval = ngroups * NS * kMfmaRows * 32;
            float v;
            if (idx < nval) {
                const int m = idx % 32, r = (idx / 32) % kMfmaRows, gh = idx / (32 * kMfmaRows);
                v = (m < a.M) ? val(gh / NS, gh % NS, r, m) : 0.f;
            } else {
                const int m = (idx - nval) % 32, g = (idx - nval) / 32;
                v = (norm && m < a.M) ? ssq(g, m) : 0.f;
            }
            // agent-scope store: written through to the level every XCD reads coherently
            __hip_atomic_store(dst + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        // The last of the tile's kpart workgroups to finish sums the partials.  Every thread waits
        // until its partial stores have completed before the barrier, and only then is the part
        // counted, so the workgroup that takes the last count reads every part back with agent-scope
        // loads.  Nothing waits on another workgroup.  The counter is reset for the next launch.
        __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
        __syncthreads();
        __shared__ int is_last;
        if (tid == 0) {
            const unsigned old = __hip_atomic_fetch_add(a.split_cnt + bid, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const bool last = old + 1 == (unsigned)a.kpart;
            if (last) __hip_atomic_store(a.split_cnt + bid, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            is_last = last;
        }
        __syncthreads();
        if (is_last) finish_split_tile<EPI>(a, bid, tid);
        return;
    }
    if constexpr (EPI == EPI_LINEAR) {
        if (a.adv_seqlens != nullptr && bid == 0 && tid < a.adv_B) a.adv_seqlens[tid] += a.adv_n;
    }
    rowdot_epilogue<T, EPI>(a, sg, (bid - sg.blk_begin) * sg.units_per_blk, ngroups, upw, kMfmaRows / 2, n_units, tid,
                            64 * a.waves, val, ssq);
}

template <typename T, int EPI, bool NW>
void launch_bm(const RowdotArgs& a, int grid, hipStream_t st) {
    const int M = a.M;
    if (M <= 1) rowdot_kernel<T, 1, EPI, NW><<<grid, 64 * a.waves, 0, st>>>(a);
    else if (M <= 2) rowdot_kernel<T, 2, EPI, NW><<<grid, 64 * a.waves, 0, st>>>(a);
    else if (M <= 4) rowdot_kernel<T, 4, EPI, NW><<<grid, 64 * a.waves, 0, st>>>(a);
    else if (M <= 8) rowdot_kernel<T, 8, EPI, NW><<<grid, 64 * a.waves, 0, st>>>(a);
    else if (M <= 16) rowdot_kernel<T, 16, EPI, NW><<<grid, 64 * a.waves, 0, st>>>(a);
    else rowdot_kernel<T, 32, EPI, NW><<<grid, 64 * a.waves, 0, st>>>(a);
}

template <typename T, int EPI>
fsvd_status_t launch_b(const RowdotArgs& a, int grid, hipStream_t st) {
    if constexpr (EPI == EPI_Z) {
        if (a.norm && a.norm_w != nullptr) launch_bm<T, EPI, true>(a, grid, st);
        else launch_bm<T, EPI, false>(a, grid, st);
    } else {
        launch_bm<T, EPI, false>(a, grid, st);
    }
    return check_launch("rowdot");
}

}  // namespace

namespace {

// bf16 launches of 5..32 activation rows go to the matrix cores.  Measured on MI355X (Llama-7B
// layer-step over 2048 positions, factor rows staged through LDS): batch 8 159.9 us on the matrix
// cores against 172.2 us on v_dot2 (which runs 5..8 rows as 8), batch 4 134.3 against 121.7 us.
#ifndef FSVD_RD_MFMA_MIN_M
#define FSVD_RD_MFMA_MIN_M 5
#endif
bool use_mfma(const RowdotArgs& a, int epi, fsvd_dtype_t dtype) {
    (void)epi;
    return dtype == FSVD_BF16 && a.M >= FSVD_RD_MFMA_MIN_M;
}

// rows: factor rows per wave (kR for the v_dot2 kernel, 16 for the MFMA kernel)
int plan_rows(RowdotArgs& a, int epi, int rows, bool mfma) {
    // Reduction split: about 1024 elements per wave for long reductions (one or two load passes),
    // then doubled while the launch has fewer than ~2048 waves.  4 waves per workgroup, 8 when the
    // split needs them.
    const int rh = rows / 2;
    int kmax = 0, units = 0;
    for (int i = 0; i < a.nseg; ++i) {
        const RowdotSeg& s = a.seg[i];
        const bool paired = seg_paired(epi, s.kind);
        kmax = std::max(kmax, std::max(s.K, epi == EPI_SWIGLU ? s.K2 : 0));
        const int u = (epi == EPI_QKV && paired) ? s.N / 2 : s.N;
        units += wave_sets(epi) * (paired ? (u + rh - 1) / rh : (u + rows - 1) / rows);  // waves without split
    }
    // (measured on MI355X for the matrix-core variant too: a deeper split with 16-wave workgroups
    // and one pass per wave was slower than this)
    int ksplit = 1;
    while (ksplit < 8 && (kmax + ksplit - 1) / ksplit > FSVD_RD_KPW && kmax / (ksplit * 2) >= 256) ksplit *= 2;
    while (ksplit < 8 && (int64_t)units * ksplit < FSVD_RD_WAVES && kmax / (ksplit * 2) >= 256) ksplit *= 2;
    if (!mfma && a.M > 16) ksplit = std::min(ksplit, 4);  // the 32-row variant runs 4-wave workgroups
    if (epi == EPI_SWIGLU) ksplit = std::min(ksplit, (!mfma && a.M > 16) ? 2 : 4);  // two wave sets per group
    a.ksplit = ksplit;
    a.waves = wave_sets(epi) * ksplit > 4 ? 8 : 4;
    int blk = 0;
    for (int i = 0; i < a.nseg; ++i) {
        RowdotSeg& s = a.seg[i];
        const bool paired = seg_paired(epi, s.kind);
        const int upw = paired ? rh : rows;
        const int n_units = (epi == EPI_QKV && paired) ? s.N / 2 : s.N;
        s.units_per_blk = (a.waves / (wave_sets(epi) * ksplit)) * upw;
        s.blk_begin = blk;
        blk += (n_units + s.units_per_blk - 1) / s.units_per_blk;
    }
    // Very few tiles (at most 512 waves, a quarter of the CUs' worth of 8-wave workgroups, even at
    // the deepest in-workgroup split): split the reduction over kpart workgroups too, up to
    // FSVD_RD_WAVES waves, while each wave keeps at least 128 elements and the partial tiles fit
    // the workspace slice.  (Measured on MI355X: splitting launches of 100-300 workgroups costs
    // more in the second kernel than it saves; at 32-64 workgroups it pays.)
    a.nblk = blk;
    a.kpart = 1;
    if (mfma && a.part != nullptr && (int64_t)blk * a.waves <= 512) {
        const int ngroups = a.waves / (wave_sets(epi) * ksplit);
        const int64_t tile_bytes = (int64_t)part_vals(ngroups, wave_sets(epi)) * (int64_t)sizeof(float);
        while ((int64_t)blk * a.kpart * a.waves < FSVD_RD_WAVES && kmax / (ksplit * a.kpart * 2) >= 128 &&
               (int64_t)blk * a.kpart * 2 * tile_bytes <= (int64_t)kRdPartBytes)
            a.kpart *= 2;
    }
    return blk * a.kpart;
}

template <int MB, int EPI, bool DB>
fsvd_status_t launch_mfma_t(const RowdotArgs& a, int grid, hipStream_t st) {
    // the stages, or the combine arrays that reuse them, whichever is larger
    constexpr size_t kRed = (size_t)kMaxWaves * 32 * (kMfmaRows + 1) * sizeof(float);
    constexpr size_t kStage = (size_t)mfma_stage_slots<MB>() * 16 * (DB ? 2 : 1);
    const size_t lds = std::max((size_t)a.waves * kStage, kRed);
    // one limit per kernel (its largest workgroup), so the attribute is set once per device
    if (const fsvd_status_t s = allow_dynamic_lds((const void*)rowdot_mfma_kernel<MB, EPI, DB>,
                                                  std::max(kMaxWaves * kStage, kRed), "rowdot_mfma"))
        return s;
    rowdot_mfma_kernel<MB, EPI, DB><<<grid, 64 * a.waves, lds, st>>>(a);
    return check_launch("rowdot_mfma");
}

// Waves with 3 or more passes over their slice of the reduction (long K over few factor-row
// tiles, e.g. the down projection's phase 1) double-buffer their stage, so each pass's factor
// rows are loaded while the previous pass computes; the doubled stage leaves one 8-wave
// workgroup per CU, which the launches with 1-2 passes per wave keep for occupancy instead.
template <int EPI>
fsvd_status_t launch_mfma(const RowdotArgs& a, int grid, hipStream_t st) {
    int kmax = 0;
    for (int i = 0; i < a.nseg; ++i) kmax = std::max(kmax, std::max(a.seg[i].K, EPI == EPI_SWIGLU ? a.seg[i].K2 : 0));
    const int steps = ((kmax + 31) / 32 + a.ksplit * a.kpart - 1) / (a.ksplit * a.kpart);  // 32-wide k steps per wave
    fsvd_status_t s;
    if (a.M <= 16) {
        const bool db = (steps + mfma_pass_steps<1>() - 1) / mfma_pass_steps<1>() >= 3;
        s = db ? launch_mfma_t<1, EPI, true>(a, grid, st) : launch_mfma_t<1, EPI, false>(a, grid, st);
    } else {
        const bool db = (steps + mfma_pass_steps<2>() - 1) / mfma_pass_steps<2>() >= 3;
        s = db ? launch_mfma_t<2, EPI, true>(a, grid, st) : launch_mfma_t<2, EPI, false>(a, grid, st);
    }
    return s;
}

}  // namespace

size_t rowdot_part_bytes(int64_t M, fsvd_dtype_t dtype) {
    return (dtype == FSVD_BF16 && M >= FSVD_RD_MFMA_MIN_M && M <= 32) ? kRdPartBytes : 0;
}

int rowdot_plan(RowdotArgs& a, int epi, fsvd_dtype_t dtype) {
    const bool mfma = use_mfma(a, epi, dtype);
    return plan_rows(a, epi, mfma ? kMfmaRows : kR, mfma);
}

fsvd_status_t launch_rowdot(const RowdotArgs& a, int epi, fsvd_dtype_t dtype, hipStream_t st) {
    RowdotArgs c = a;
    if (c.M < 1 || c.M > 32) return fail(FSVD_ERR_UNSUPPORTED, "row-dot path supports 1..32 activation rows, got %d", c.M);
    // A split reduction counts its finished parts in the workspace header (err is its first word);
    // without a header the reduction is not split.
    if (c.err == nullptr) c.part = nullptr;
    int grid = rowdot_plan(c, epi, dtype);
    if (c.kpart > 1 && c.nblk > kWsSplitCounters) {  // cannot happen (a split launch has <= 128 tiles)
        c.part = nullptr;
        grid = rowdot_plan(c, epi, dtype);
    }
    if (grid <= 0) return FSVD_OK;
    c.split_cnt = c.kpart > 1 ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(c.err) + kWsSplitCounterOff)
                              : nullptr;
    if (dtype == FSVD_F32) {
        switch (epi) {
            case EPI_Z: return launch_b<float, EPI_Z>(c, grid, st);
            case EPI_LINEAR: return launch_b<float, EPI_LINEAR>(c, grid, st);
            default: return fail(FSVD_ERR_UNSUPPORTED, "fp32 row-dot supports the plain linear epilogues only");
        }
    }
    if (use_mfma(c, epi, dtype)) {
        switch (epi) {
            case EPI_Z: return launch_mfma<EPI_Z>(c, grid, st);
            case EPI_LINEAR: return launch_mfma<EPI_LINEAR>(c, grid, st);
            case EPI_QKV: return launch_mfma<EPI_QKV>(c, grid, st);
            case EPI_SWIGLU: return launch_mfma<EPI_SWIGLU>(c, grid, st);
            case EPI_GELU: return launch_mfma<EPI_GELU>(c, grid, st);
        }
        return fail(FSVD_ERR_UNSUPPORTED, "unknown row-dot epilogue %d", epi);
    }
    switch (epi) {
        case EPI_Z: return launch_b<bf16_t, EPI_Z>(c, grid, st);
        case EPI_LINEAR: return launch_b<bf16_t, EPI_LINEAR>(c, grid, st);
        case EPI_QKV: return launch_b<bf16_t, EPI_QKV>(c, grid, st);
        case EPI_SWIGLU: return launch_b<bf16_t, EPI_SWIGLU>(c, grid, st);
        case EPI_GELU: return launch_b<bf16_t, EPI_GELU>(c, grid, st);
    }
    return fail(FSVD_ERR_UNSUPPORTED, "unknown row-dot epilogue %d", epi);
}

}  // namespace fsvd
