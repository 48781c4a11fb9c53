// Attention of the new tokens over the contiguous dense KV cache, gfx950.
//
// "Reconstruct the present, read the past contiguously" ("FlashSVD v1.5" explainer,
// Methodology 2): the history lives in a standard dense cache [B, L_max, Hkv, D] and every
// decode step reads it in one attention pass.
//
// Decode (Sq == 1) is HBM-bound (each cached K/V byte is used by Hq/Hkv query heads only), so
// it streams the cache with 16-byte loads: a workgroup owns one (sequence, kv head, length
// partition); its 16 lane groups of 16 lanes each take one position at a time (16 lanes x 8
// bf16 = one 128-wide head vector), reduce q.k across the lane group with DPP, and keep an
// online softmax per query head of the GQA group, so a K/V line is read once for all heads
// that share it.  Partitions are merged by log-sum-exp in a second small kernel.  The length
// is read on the device from cache_seqlens, so a captured graph stays valid as the cache grows.
//
// Sq > 1 (prefill and encoder layers) runs on the matrix cores (attention_prefill.hip).
#include "kernels.h"

namespace fsvd {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;

// EPL: head elements per lane (D / 16): 8 for D = 128, 4 for D = 64.  G: query heads per kv head.
template <int EPL>
struct KV {
    uint32_t w[EPL / 2];
};

template <int EPL>
__device__ __forceinline__ KV<EPL> ld_kv(const bf16_t* p) {
    KV<EPL> r;
    if constexpr (EPL == 8) {
        const u32x4 v = *reinterpret_cast<const u32x4*>(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}

// One workgroup = (b, kv head, length partition); 256 threads = 16 lane groups.
template <int EPL, int G>
__global__ __launch_bounds__(256) void attn_decode_split(const AttnArgs a) {
    const int D = EPL * 16;
    const int tid = threadIdx.x, lg = tid >> 4, li = tid & 15;
    const int split = blockIdx.x % a.nsplit;
    const int bg = blockIdx.x / a.nsplit;
    const int kvh = bg % a.Hkv, b = bg / a.Hkv;

    int64_t n = (int64_t)a.seqlens[b] + 1;
    if (n > a.L_max) {
        if (tid == 0 && split == 0) set_dev_error(a.err, FSVD_DEVERR_SEQ_OVERFLOW);
        n = a.L_max;
    }
    const int64_t chunk = ((n + a.nsplit - 1) / a.nsplit + 15) / 16 * 16;
    const int64_t j0 = (int64_t)split * chunk;
    const int64_t j1 = min(n, j0 + chunk);

    // q fragments: lane li of each group holds elements [li*EPL, li*EPL+EPL) of every head
    uint32_t qf[G][EPL / 2];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int h = kvh * G + g;
        const KV<EPL> v = ld_kv<EPL>(a.q + ((int64_t)b * a.Hq + h) * D + li * EPL);
#pragma unroll
        for (int i = 0; i < EPL / 2; ++i) qf[g][i] = v.w[i];
    }
    const float sc = a.scale * kLog2e;

    float m[G], l[G], o[G][EPL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegBig;
        l[g] = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) o[g][i] = 0.f;
    }
    const int64_t rowstride = (int64_t)a.Hkv * D;
    const bf16_t* kbase = a.kc + ((int64_t)b * a.L_max * a.Hkv + kvh) * D + li * EPL;
    const bf16_t* vbase = a.vc + ((int64_t)b * a.L_max * a.Hkv + kvh) * D + li * EPL;

    constexpr int NP = 2;  // positions per lane group per iteration
    for (int64_t jb = j0 + lg; jb < j1; jb += 16 * NP) {
        KV<EPL> kv[NP], vv[NP];
        bool ok[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int64_t j = jb + 16 * p;
            ok[p] = j < j1;
            const int64_t jj = ok[p] ? j : jb;
            kv[p] = ld_kv<EPL>(kbase + jj * rowstride);
            vv[p] = ld_kv<EPL>(vbase + jj * rowstride);
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            if (!ok[p]) continue;  // uniform over the lane group (one DPP row)
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = 0.f;
#pragma unroll
                for (int i = 0; i < EPL / 2; ++i) d = dot2bf(qf[g][i], kv[p].w[i], d);
                d = row16_sum(d) * sc;
                const float mn = fmaxf(m[g], d);
                const float alpha = exp2f(m[g] - mn);
                const float pr = exp2f(d - mn);
                m[g] = mn;
                l[g] = l[g] * alpha + pr;
#pragma unroll
                for (int i = 0; i < EPL / 2; ++i) {
                    o[g][2 * i] = o[g][2 * i] * alpha + pr * bf_lo(vv[p].w[i]);
                    o[g][2 * i + 1] = o[g][2 * i + 1] * alpha + pr * bf_hi(vv[p].w[i]);
                }
            }
        }
    }

    // merge the 16 lane groups: LDS [16][G][D + 2]
    __shared__ float sm[16 * G * (16 * EPL + 2)];
    const int stride = D + 2;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float* row = sm + (lg * G + g) * stride;
#pragma unroll
        for (int i = 0; i < EPL; ++i) row[li * EPL + i] = o[g][i];
        if (li == 0) {
            row[D] = m[g];
            row[D + 1] = l[g];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, dd = idx - g * D;
        float M = kNegBig;
        for (int q = 0; q < 16; ++q) M = fmaxf(M, sm[(q * G + g) * stride + D]);
        float L = 0.f, O = 0.f;
        for (int q = 0; q < 16; ++q) {
            const float* row = sm + (q * G + g) * stride;
            const float w = exp2f(row[D] - M);
            L += w * row[D + 1];
            O += w * row[dd];
        }
        const int h = kvh * G + g;
        float* part = a.part + (((int64_t)b * a.Hq + h) * a.nsplit + split) * (D + 2);
        part[dd] = O;
        if (dd == 0) {
            part[D] = M;
            part[D + 1] = L;
        }
    }
}

// merge partitions: one workgroup per (b, h).  The first wave reads every partition's
// (max, sum) at once and forms the log-sum-exp weights; then each thread owns one head element
// and sums the weighted partial outputs (all loads independent, so one L2 round trip).
__global__ __launch_bounds__(128) void attn_decode_combine(const AttnArgs a) {
    const int D = a.D, ns = a.nsplit;
    const int bh = blockIdx.x;
    const int t = threadIdx.x;
    const float* part = a.part + (int64_t)bh * ns * (D + 2);
    __shared__ float w[64];
    __shared__ float inv_l;
    if (t < 64) {
        const bool ok = t < ns;
        const float ms = ok ? part[t * (D + 2) + D] : kNegBig;
        const float ls = ok ? part[t * (D + 2) + D + 1] : 0.f;
        float M = row16_max(ms);
        M = fmaxf(fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, M), 0)),
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, M), 16))),
                  fmaxf(__builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, M), 32)),
                        __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, M), 48))));
        const float ws = ok ? exp2f(ms - M) : 0.f;
        w[t] = ws;
        const float L = wave_sum(ws * ls);
        if (t == 0) inv_l = 1.0f / L;
    }
    __syncthreads();
    if (t >= D) return;
    float O = 0.f;
#pragma unroll 8
    for (int s = 0; s < ns; ++s) O += w[s] * part[s * (D + 2) + t];
    a.out[(int64_t)bh * D + t] = f2bf(O * inv_l);
}

template <int EPL>
fsvd_status_t launch_decode_d(const AttnArgs& a, hipStream_t st) {
    const int G = a.Hq / a.Hkv;
    const int grid = a.B * a.Hkv * a.nsplit;
    switch (G) {
        case 1: attn_decode_split<EPL, 1><<<grid, 256, 0, st>>>(a); break;
        case 2: attn_decode_split<EPL, 2><<<grid, 256, 0, st>>>(a); break;
        case 4: attn_decode_split<EPL, 4><<<grid, 256, 0, st>>>(a); break;
        case 8: attn_decode_split<EPL, 8><<<grid, 256, 0, st>>>(a); break;
        default: return fail(FSVD_ERR_UNSUPPORTED, "GQA group size %d not in {1,2,4,8}", G);
    }
    fsvd_status_t s = check_launch("attn_decode_split");
    if (s != FSVD_OK) return s;
    attn_decode_combine<<<a.B * a.Hq, 128, 0, st>>>(a);
    return check_launch("attn_decode_combine");
}

}  // namespace

size_t attn_decode_ws_bytes(int B, int Hq, int D, int nsplit) {
    return (size_t)B * Hq * nsplit * (D + 2) * sizeof(float);
}

int attn_default_splits(int B, int Hkv, int64_t L_max) {
    // aim for ~2048 workgroups with at least 64 positions per partition
    int64_t want = (2048 + (int64_t)B * Hkv - 1) / ((int64_t)B * Hkv);
    int64_t cap = (L_max + 63) / 64;
    int64_t s = std::max<int64_t>(1, std::min<int64_t>(want, cap));
    return (int)std::min<int64_t>(s, 64);
}

fsvd_status_t launch_attn_decode(const AttnArgs& a, hipStream_t st) {
    if (a.D == 128) return launch_decode_d<8>(a, st);
    if (a.D == 64) return launch_decode_d<4>(a, st);
    return fail(FSVD_ERR_UNSUPPORTED, "head dim %d not in {64,128}", a.D);
}

}  // namespace fsvd
