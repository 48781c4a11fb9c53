// Decode-size (M <= 32 activation rows) low-rank projection kernels for gfx950.
//
// At decode the fused projection y = (x . U) . V is bound by streaming the factor bytes once
// from HBM (about M flop per factor byte, far below the MFMA ridge), so each phase is a
// "row-dot": every output n is the dot product of one K-contiguous factor row with the M
// activation rows.  A wave owns R rows; each lane loads 16 contiguous bytes of every row per
// step (one wave instruction = a 1 KiB coalesced segment of each row), multiplies them with the
// matching activation bytes using v_dot2_f32_bf16 (fp32 accumulation), and the 64 lanes are
// reduced with DPP row operations plus a small LDS combine.  Long reductions are split over
// the waves of a workgroup so the grid has enough waves in flight to cover HBM latency.
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
#include "kernels.h"

namespace fsvd {

namespace {

constexpr int kR = 4;       // factor rows per wave
constexpr int kWaves = 4;   // waves per workgroup
constexpr int kUnroll = 2;  // 16-byte steps issued before use

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

// sum of squares of a 16-byte activation vector (RMSNorm statistics)
__device__ __forceinline__ float vsq(u32x4 a, bf16_t) {
    float s = 0.f;
    uint32_t v[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float lo = bf_lo(v[i]), hi = bf_hi(v[i]);
        s = fmaf(lo, lo, s);
        s = fmaf(hi, hi, s);
    }
    return s;
}
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

__host__ __device__ __forceinline__ bool seg_paired(int epi, int kind) {
    return (epi == EPI_QKV && (kind == SEG_Q || kind == SEG_K)) || epi == EPI_SWIGLU;
}

template <typename T, int BMAX, int EPI>
__global__ __launch_bounds__(256) void rowdot_kernel(const RowdotArgs a) {
    constexpr int E = Vec<T>::E;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bid = blockIdx.x;

    const int si = (a.nseg > 2 && bid >= a.seg[2].blk_begin) ? 2 : ((a.nseg > 1 && bid >= a.seg[1].blk_begin) ? 1 : 0);
    const RowdotSeg sg = si == 0 ? a.seg[0] : (si == 1 ? a.seg[1] : a.seg[2]);

    const bool paired = seg_paired(EPI, sg.kind);
    const int upw = paired ? kR / 2 : kR;                        // output units per wave
    const int n_units = (EPI == EPI_QKV && paired) ? sg.N / 2 : sg.N;
    const int ksplit = a.ksplit;
    const int grp = wave / ksplit, ks = wave - grp * ksplit;
    const int unit0 = (bid - sg.blk_begin) * sg.units_per_blk + grp * upw;
    const int halfD = a.D >> 1;

    // rows owned by this wave
    const char* wrow[kR];
    int klen[kR];
    int aoff[kR];
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        int u, n, mat = 0;
        if (paired) {
            u = unit0 + (r & 1);
            if (EPI == EPI_SWIGLU) {
                mat = r >> 1;
                n = u;
            } else {
                const int h = u / halfD, i = u - h * halfD;
                n = h * a.D + i + (r >> 1) * halfD;
            }
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
    const int kmax = (EPI == EPI_SWIGLU) ? max(sg.K, sg.K2) : sg.K;
    const int nvec = kmax / E;
    const int per = (nvec + ksplit - 1) / ksplit;
    const int k_lo = ks * per * E;
    const int k_hi = min(kmax, (ks + 1) * per * E);

    float acc[kR][BMAX];
    float ss[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        ss[b] = 0.f;
#pragma unroll
        for (int r = 0; r < kR; ++r) acc[r][b] = 0.f;
    }
    const int M = a.M;
    const char* act = reinterpret_cast<const char*>(a.act);
    const int64_t lda_b = a.lda * (int64_t)sizeof(T);
    const bool norm = (EPI == EPI_Z) && a.norm;
    const bool norm_w = norm && a.norm_w != nullptr;

    for (int kb = k_lo; kb < k_hi; kb += 64 * E * kUnroll) {
        u32x4 wv[kUnroll][kR];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int k = kb + (u * 64 + lane) * E;
#pragma unroll
            for (int r = 0; r < kR; ++r) {
                if (k < k_hi && k < klen[r])
                    wv[u][r] = ldg16(wrow[r] + (int64_t)k * sizeof(T));
                else
                    wv[u][r] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int k = kb + (u * 64 + lane) * E;
            if (k >= k_hi) continue;
            u32x4 nw = u32x4{0u, 0u, 0u, 0u};
            if (norm_w) nw = ldg16(a.norm_w + k);
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                if (b >= M) continue;
                if (EPI == EPI_SWIGLU) {
                    if (k < sg.K) {
                        const u32x4 av = ldg16(act + b * lda_b + (int64_t)(aoff[0] + k) * sizeof(T));
                        acc[0][b] = vdot(wv[u][0], av, acc[0][b], T());
                        acc[1][b] = vdot(wv[u][1], av, acc[1][b], T());
                    }
                    if (k < sg.K2) {
                        const u32x4 av = ldg16(act + b * lda_b + (int64_t)(aoff[2] + k) * sizeof(T));
                        acc[2][b] = vdot(wv[u][2], av, acc[2][b], T());
                        acc[3][b] = vdot(wv[u][3], av, acc[3][b], T());
                    }
                } else {
                    u32x4 av = ldg16(act + b * lda_b + (int64_t)(aoff[0] + k) * sizeof(T));
                    if constexpr (EPI == EPI_Z) {
                        if (norm) {
                            ss[b] += vsq(av, T());
                            if (norm_w) av = vmulw(av, nw);
                        }
                    }
#pragma unroll
                    for (int r = 0; r < kR; ++r) acc[r][b] = vdot(wv[u][r], av, acc[r][b], T());
                }
            }
        }
    }

    // lanes -> 4 row partials per value (DPP), then waves/rows combined through LDS
    constexpr int NV = (kR + 1) * BMAX;
    __shared__ float red[kWaves][4][NV];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        if (b >= M) continue;
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const float v = row16_sum(acc[r][b]);
            if ((lane & 15) == 0) red[wave][lane >> 4][r * BMAX + b] = v;
        }
        if (norm) {
            const float v = row16_sum(ss[b]);
            if ((lane & 15) == 0) red[wave][lane >> 4][kR * BMAX + b] = v;
        }
    }
    __syncthreads();

    if constexpr (EPI == EPI_LINEAR) {
        if (a.adv_seqlens != nullptr && bid == 0 && tid < a.adv_B) a.adv_seqlens[tid] += a.adv_n;
    }

    auto val = [&](int g, int r, int b) -> float {
        float s = 0.f;
        for (int w = g * ksplit; w < (g + 1) * ksplit; ++w)
            s += red[w][0][r * BMAX + b] + red[w][1][r * BMAX + b] + red[w][2][r * BMAX + b] + red[w][3][r * BMAX + b];
        return s;
    };

    const int ngroups = kWaves / ksplit;
    const int total = ngroups * upw * M;
    for (int idx = tid; idx < total; idx += 256) {
        const int g = idx / (upw * M);
        const int rem = idx - g * upw * M;
        const int j = rem / M;           // unit within the wave
        const int m = rem - j * M;       // activation row
        const int u = (bid - sg.blk_begin) * sg.units_per_blk + g * upw + j;
        if (u >= n_units) continue;
        if constexpr (EPI == EPI_Z) {
            float v = val(g, j, m);
            if (a.norm) {
                const float sq = val(g, kR, m);
                v *= 1.0f / sqrtf(sq / (float)a.norm_K + a.norm_eps);
            }
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, v);
        } else if constexpr (EPI == EPI_LINEAR) {
            float v = val(g, j, m);
            if (a.bias) v += load_t<T>(a.bias, u);
            if (a.residual) v += load_t<T>(a.residual, (int64_t)m * a.ldr + u);
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, v);
        } else if constexpr (EPI == EPI_GELU) {
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, gelu_f(val(g, j, m)));
        } else if constexpr (EPI == EPI_SWIGLU) {
            const float gv = val(g, j, m), uv = val(g, j + 2, m);
            store_t<T>(sg.out, (int64_t)m * sg.ldo + u, silu_f(gv) * uv);
        } else if constexpr (EPI == EPI_QKV) {
            const int b = m / a.S, s = m - b * a.S;
            const int64_t p = (int64_t)a.seqlens[b] + s;
            const bool in_cache = p >= 0 && p < a.L_max;
            if (sg.kind == SEG_V) {
                const bf16_t bits = f2bf(val(g, j, m));
                const int hd = a.Hkv * a.D;
                if (in_cache) a.v_cache[((int64_t)b * a.L_max + p) * hd + u] = bits;
                else set_dev_error(a.err, FSVD_DEVERR_KV_OVERFLOW);
                if (a.v_out) a.v_out[(int64_t)m * hd + u] = bits;
            } else {
                const float x1 = val(g, j, m), x2 = val(g, j + 2, m);
                const int h = u / halfD, i = u - h * halfD;
                const int n1 = h * a.D + i, n2 = n1 + halfD;
                float y1 = x1, y2 = x2;
                if (a.rope_theta > 0.f) {
                    float c, sn;
                    rope_cs(p, i, a.D, a.rope_theta, &c, &sn);
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

template <typename T, int EPI>
fsvd_status_t launch_b(const RowdotArgs& a, int grid, hipStream_t st) {
    const int M = a.M;
    if (M <= 1) rowdot_kernel<T, 1, EPI><<<grid, 256, 0, st>>>(a);
    else if (M <= 2) rowdot_kernel<T, 2, EPI><<<grid, 256, 0, st>>>(a);
    else if (M <= 4) rowdot_kernel<T, 4, EPI><<<grid, 256, 0, st>>>(a);
    else if (M <= 8) rowdot_kernel<T, 8, EPI><<<grid, 256, 0, st>>>(a);
    else if (M <= 16) rowdot_kernel<T, 16, EPI><<<grid, 256, 0, st>>>(a);
    else rowdot_kernel<T, 32, EPI><<<grid, 256, 0, st>>>(a);
    return check_launch("rowdot");
}

}  // namespace

int rowdot_plan(RowdotArgs& a, int epi) {
    // pick the reduction split so the grid has enough waves, then lay segments out
    int ksplit = 1;
    for (;;) {
        int blocks = 0, kmax = 0;
        for (int i = 0; i < a.nseg; ++i) {
            const RowdotSeg& s = a.seg[i];
            const bool paired = seg_paired(epi, s.kind);
            const int upw = paired ? kR / 2 : kR;
            const int units = (epi == EPI_QKV && paired) ? s.N / 2 : s.N;
            const int upb = (kWaves / ksplit) * upw;
            blocks += (units + upb - 1) / upb;
            kmax = std::max(kmax, std::max(s.K, epi == EPI_SWIGLU ? s.K2 : 0));
        }
        if (blocks >= 600 || ksplit == 4 || kmax / (ksplit * 2) < 512) break;
        ksplit *= 2;
    }
    a.ksplit = ksplit;
    int blk = 0;
    for (int i = 0; i < a.nseg; ++i) {
        RowdotSeg& s = a.seg[i];
        const bool paired = seg_paired(epi, s.kind);
        const int upw = paired ? kR / 2 : kR;
        const int units = (epi == EPI_QKV && paired) ? s.N / 2 : s.N;
        s.units_per_blk = (kWaves / ksplit) * upw;
        s.blk_begin = blk;
        blk += (units + s.units_per_blk - 1) / s.units_per_blk;
    }
    return blk;
}

fsvd_status_t launch_rowdot(const RowdotArgs& a, int epi, fsvd_dtype_t dtype, hipStream_t st) {
    RowdotArgs c = a;
    const int grid = rowdot_plan(c, epi);
    if (grid <= 0) return FSVD_OK;
    if (c.M < 1 || c.M > 32) return fail(FSVD_ERR_UNSUPPORTED, "row-dot path supports 1..32 activation rows, got %d", c.M);
    if (dtype == FSVD_F32) {
        switch (epi) {
            case EPI_Z: return launch_b<float, EPI_Z>(c, grid, st);
            case EPI_LINEAR: return launch_b<float, EPI_LINEAR>(c, grid, st);
            default: return fail(FSVD_ERR_UNSUPPORTED, "fp32 row-dot supports the plain linear epilogues only");
        }
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
