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
// that share it.  Partitions are merged by log-sum-exp: the last partition of each (sequence, kv
// head) to finish merges them (a counter per pair in the workspace header), or, without counters,
// a second small kernel does.  The length is read on the device from cache_seqlens, so a captured
// graph stays valid as the cache grows.
//
// Sq > 1 (prefill and encoder layers) runs on the matrix cores (attention_prefill.hip).
#include "kernels.h"

namespace fsvd {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kAuxNonTemporal = 2;  // cache-policy operand of a buffer load: nt
constexpr float kNegBig = -1.0e30f;
#ifndef FSVD_ATTN_WGS
// decode: target workgroups (sequence x kv head x length partition).  Few long partitions beat
// many short ones: each workgroup ends with its partial stores' round trip and the count, so
// workgroups that fit the CUs in one round stream best (measured on MI355X, batch 4, 32 heads
// of 128, 2112 positions, last-partition merge: 512 -> 27.8 us, 1024 -> 30.4 us, 2048 -> 32.4 us,
// 4096 -> 37.6 us; with the merge in a second kernel, 1024 -> 33.1 us and 4096 -> 34.4 us).
#define FSVD_ATTN_WGS 512
#endif
#ifndef FSVD_ATTN_NP
#define FSVD_ATTN_NP 2      // decode: positions per lane group per iteration (16 * NP per workgroup)
#endif
#ifndef FSVD_ATTN_NP_GQA
#define FSVD_ATTN_NP_GQA 4  // the same with 4 or more query heads per kv head (measured on MI355X,
                            // GQA batch 32 x 8 kv heads, 8192 positions: 172.0 against 179.7 us per
                            // call; with one head per kv head 4 is slower: batch 16 90.6 against 85.4)
#endif
#ifndef FSVD_ATTN_ROUND
#define FSVD_ATTN_ROUND 16  // decode: partition lengths are multiples of this
#endif
#ifndef FSVD_ATTN_MERGE_C
#define FSVD_ATTN_MERGE_C 32  // partition merge: partitions loaded per round trip
#endif
#ifndef FSVD_ATTN_LAST_MERGE_C
#define FSVD_ATTN_LAST_MERGE_C 16 // the same inside the split kernel, whose registers it shares
#endif
#ifndef FSVD_ATTN_FUSED_MERGE
#define FSVD_ATTN_FUSED_MERGE 1  // 0: always merge in the second kernel (for comparisons)
#endif

// EPL: head elements per lane (D / 16): 8 for D = 128, 4 for D = 64.  G: query heads per kv head.
template <int EPL>
struct KV {
    uint32_t w[EPL / 2];
};

// STREAM: the K/V history, read once per call: non-temporal loads, so the stream does not take
// the caches from the rest (measured on MI355X, batch 4, 32 heads of 128, 2112 positions: 25.1 us
// per call against 28.0 us with plain loads; batch 16: 85.4 against 98.2 us)
template <int EPL, bool STREAM = false>
__device__ __forceinline__ KV<EPL> ld_kv(const bf16_t* p) {
    KV<EPL> r;
    if constexpr (EPL == 8) {
        const u32x4 v = STREAM ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p))
                               : *reinterpret_cast<const u32x4*>(p);
        r.w[0] = v.x; r.w[1] = v.y; r.w[2] = v.z; r.w[3] = v.w;
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 v = STREAM ? __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p))
                               : *reinterpret_cast<const u32x2*>(p);
        r.w[0] = v.x; r.w[1] = v.y;
    }
    return r;
}

// Log-sum-exp merge of the ns partitions of one (b, h) at head element dd.  part points at the
// rows of (b, h): [ns][D + 2], the partition's D outputs, then its running max and sum.  Every
// thread loads its element of C partitions together with their statistics, so the merge costs
// one round trip to the cache per C partitions.  COHERENT: the rows were written in the same
// kernel by workgroups on any XCD, so they are read with agent-scope loads (which fetch from the
// coherent level, not from a line this XCD's L2 may hold).
template <bool COHERENT, int C>
__device__ __forceinline__ float merge_partitions(const float* part, int ns, int D, int dd) {
    auto ld = [](const float* p) {
        if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else return *p;
    };
    float M = kNegBig, L = 0.f, O = 0.f;
    for (int s0 = 0; s0 < ns; s0 += C) {
        float ms[C], ls[C], os[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const bool ok = s0 + c < ns;
            const float* row = part + (int64_t)(ok ? s0 + c : s0) * (D + 2);
            const float mv = ld(row + D);
            ms[c] = ok ? mv : kNegBig;
            ls[c] = ld(row + D + 1);
            os[c] = ld(row + dd);
        }
        float mc = M;
#pragma unroll
        for (int c = 0; c < C; ++c) mc = fmaxf(mc, ms[c]);
        const float r = exp2f(M - mc);
        L *= r;
        O *= r;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const float w = exp2f(ms[c] - mc);  // 0 for the padding entries (max = -1e30)
            L += w * ls[c];
            O += w * os[c];
        }
        M = mc;
    }
    return O / L;  // L > 0: the partition holding position n - 1 is never empty
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
    const int64_t chunk = ((n + a.nsplit - 1) / a.nsplit + FSVD_ATTN_ROUND - 1) / FSVD_ATTN_ROUND * FSVD_ATTN_ROUND;
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
    // Grouped heads (G > 1, 128-wide heads) read K/V through buffer loads: a 32-bit offset per lane
    // instead of a 64-bit address saves vector instructions in a loop that does G heads' work per
    // load (Llama-3-8B GQA, batch 32, 8192 positions: 179 against 189 us per call on MI355X; with
    // G = 1 the plain global loads are as fast or faster).  A sequence's cache slice,
    // L_max x Hkv x D bf16, is checked at launch to fit the 31-bit offsets.
    constexpr bool BUF = G > 1 && EPL == 8;
    const int64_t seq0 = ((int64_t)b * a.L_max * a.Hkv + kvh) * D;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.kc + seq0), 0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(a.vc + seq0), 0, 0x7fffffff, 0x00020000);

    // NP positions per lane group per iteration, the same number of iterations for every lane
    // group (uniform control flow).  The K/V vectors of the next iteration are loaded before the
    // current ones are used (two iterations in flight per wave); loads are unconditional, rows past
    // the partition re-read its first row, and such positions get zero weight.  The running max
    // is updated once per iteration for all NP positions, so the rescale of l and o is paid once.
    constexpr int NP = G >= 4 ? FSVD_ATTN_NP_GQA : FSVD_ATTN_NP;
    KV<EPL> kv[NP], vv[NP];
    auto load = [&](int64_t jb, KV<EPL> (&kk)[NP], KV<EPL> (&vk)[NP]) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int64_t j = jb + 16 * p;
            const int64_t jj = j < j1 ? j : j0;
            if constexpr (BUF) {
                const int off = (int)((li * EPL + jj * rowstride) * (int64_t)sizeof(bf16_t));
                const u32x4 k4 = __builtin_amdgcn_raw_buffer_load_b128(krs, off, 0, kAuxNonTemporal);
                const u32x4 v4 = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kAuxNonTemporal);
                kk[p].w[0] = k4.x; kk[p].w[1] = k4.y; kk[p].w[2] = k4.z; kk[p].w[3] = k4.w;
                vk[p].w[0] = v4.x; vk[p].w[1] = v4.y; vk[p].w[2] = v4.z; vk[p].w[3] = v4.w;
            } else {
                kk[p] = ld_kv<EPL, true>(kbase + jj * rowstride);
                vk[p] = ld_kv<EPL, true>(vbase + jj * rowstride);
            }
        }
    };
    const int niter = j1 > j0 ? (int)((j1 - j0 + 16 * NP - 1) / (16 * NP)) : 0;  // uniform
    if (niter > 0) load(j0 + lg, kv, vv);
    for (int it = 0; it < niter; ++it) {
        const int64_t jb = j0 + lg + (int64_t)it * 16 * NP;
        KV<EPL> kn[NP], vn[NP];
        load(jb + 16 * NP, kn, vn);  // past the partition: first row again (cheap, in cache)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d[NP];
            bool ok[NP];
            float mn = m[g];
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                float t = 0.f;
#pragma unroll
                for (int i = 0; i < EPL / 2; ++i) t = dot2bf(qf[g][i], kv[p].w[i], t);
                ok[p] = jb + 16 * p < j1;
                d[p] = row16_sum(t) * sc;
                if (ok[p]) mn = fmaxf(mn, d[p]);
            }
            const float alpha = exp2f(m[g] - mn);
            float pr[NP];
            float lsum = 0.f;
#pragma unroll
            for (int p = 0; p < NP; ++p) {
                pr[p] = ok[p] ? exp2f(d[p] - mn) : 0.f;
                lsum += pr[p];
            }
            m[g] = mn;
            l[g] = l[g] * alpha + lsum;
#pragma unroll
            for (int i = 0; i < EPL / 2; ++i) {
                float lo = o[g][2 * i] * alpha, hi = o[g][2 * i + 1] * alpha;
#pragma unroll
                for (int p = 0; p < NP; ++p) {
                    lo = fmaf(pr[p], bf_lo(vv[p].w[i]), lo);
                    hi = fmaf(pr[p], bf_hi(vv[p].w[i]), hi);
                }
                o[g][2 * i] = lo;
                o[g][2 * i + 1] = hi;
            }
        }
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            kv[p] = kn[p];
            vv[p] = vn[p];
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
        // agent-scope stores: written through to the level every XCD reads coherently
        __hip_atomic_store(part + dd, O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (dd == 0) {
            __hip_atomic_store(part + D, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(part + D + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (a.cnt == nullptr) return;  // attn_decode_combine merges

    // The last partition of (b, kv head) to finish merges all of them.  Every thread waits until
    // its partial stores have completed before the barrier, and only then is the partition
    // counted, so the workgroup that takes the last count reads every partition's rows back with
    // agent-scope loads.  Nothing waits on another workgroup: the others simply exit.  The
    // counter is reset for the next call.
    __builtin_amdgcn_s_waitcnt(0);  // vmcnt(0) expcnt(0) lgkmcnt(0)
    __syncthreads();
    __shared__ int is_last;
    if (tid == 0) {
        const unsigned old = __hip_atomic_fetch_add(a.cnt + bg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = old + 1 == (unsigned)a.nsplit;
        if (last) __hip_atomic_store(a.cnt + bg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        is_last = last;
    }
    __syncthreads();
    if (!is_last) return;
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, dd = idx - g * D;
        const int64_t bh = (int64_t)b * a.Hq + kvh * G + g;
        a.out[bh * D + dd] = f2bf(merge_partitions<true, FSVD_ATTN_LAST_MERGE_C>(a.part + bh * a.nsplit * (D + 2), a.nsplit, D, dd));
    }
}

// merge partitions in a second kernel: one workgroup per (b, h), one thread per head element
__global__ __launch_bounds__(128) void attn_decode_combine(const AttnArgs a) {
    const int D = a.D, ns = a.nsplit;
    const int bh = blockIdx.x;
    const int t = threadIdx.x;
    if (t >= D) return;
    a.out[(int64_t)bh * D + t] = f2bf(merge_partitions<false, FSVD_ATTN_MERGE_C>(a.part + (int64_t)bh * ns * (D + 2), ns, D, t));
}

template <int EPL>
fsvd_status_t launch_decode_d(const AttnArgs& args, hipStream_t st) {
    AttnArgs a = args;
    if (!FSVD_ATTN_FUSED_MERGE) a.cnt = nullptr;
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
    if (s != FSVD_OK || a.cnt) return s;
    attn_decode_combine<<<a.B * a.Hq, 128, 0, st>>>(a);
    return check_launch("attn_decode_combine");
}

}  // namespace

size_t attn_decode_ws_bytes(int B, int Hq, int D, int nsplit) {
    return (size_t)B * Hq * nsplit * (D + 2) * sizeof(float);
}

int attn_default_splits(int B, int Hkv, int64_t L_max) {
    // aim for ~FSVD_ATTN_WGS workgroups with at least 64 positions per partition
    int64_t want = (FSVD_ATTN_WGS + (int64_t)B * Hkv - 1) / ((int64_t)B * Hkv);
    int64_t cap = (L_max + 63) / 64;
    int64_t s = std::max<int64_t>(1, std::min<int64_t>(want, cap));
    return (int)std::min<int64_t>(s, 64);
}

fsvd_status_t launch_attn_decode(const AttnArgs& a, hipStream_t st) {
    // grouped 128-wide heads address a sequence's cache slice with 31-bit buffer offsets
    if (a.D == 128 && a.Hq > a.Hkv && a.L_max * a.Hkv * a.D * (int64_t)sizeof(bf16_t) > 0x7fffffffLL)
        return fail(FSVD_ERR_UNSUPPORTED, "decode attention: one sequence's cache (%lld bytes) exceeds 2 GiB",
                    (long long)(a.L_max * a.Hkv * a.D * (int64_t)sizeof(bf16_t)));
    if (a.D == 128) return launch_decode_d<8>(a, st);
    if (a.D == 64) return launch_decode_d<4>(a, st);
    return fail(FSVD_ERR_UNSUPPORTED, "head dim %d not in {64,128}", a.D);
}

}  // namespace fsvd
