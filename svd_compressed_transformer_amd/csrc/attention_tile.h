// Shared MFMA flash-attention tile step (gfx950, v_mfma_f32_16x16x32_bf16): used by the prefill
// attention over the dense cache and by the factorised attention that rebuilds its tiles on chip.
#pragma once

#include "kernels.h"

namespace fsvd {
namespace {

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNeg = -1.0e30f;
constexpr int BQ = 64, BKV = 64;  // queries per workgroup (16 per wave), keys per tile

// 8-byte slot of the V^T tile (D head dimensions x 64 keys, bf16) holding the 4 keys of key
// group kc (0 .. 15) at head dimension d.  For each 32-key half c the tile step reads groups
// 8c + j and 8c + 4 + j (j = 0 .. 3) of a dimension as one 16-byte operand, so those two sit side by
// side: pair 4c + j, halves 0 and 1.  The 8 pairs of a dimension (128 bytes) are XOR-swizzled by
// (d >> 1) & 7, so the 16 dimensions a quarter-wave reads fall in 16 distinct 16-byte bank groups.
__device__ __forceinline__ int vts_slot(int d, int kc) {
    const int c = kc >> 3, h = (kc >> 2) & 1, j = kc & 3;
    return 2 * (d * 8 + ((4 * c + j) ^ ((d >> 1) & 7))) + h;
}

// One key tile of the MFMA flash attention: the 64 keys j0 .. j0 + 63 staged in LDS (Ks: K rows
// with XOR-swizzled 16-byte chunks; Vt: V transposed, slots as vts_slot gives them)
// against QW sets of 16 queries of this wave (qf[q]: the B operand, lane (li, lg) holding
// q[query li of set q][t*32 + lg*8 .. +7]).  Every K or V fragment read from LDS feeds the
// matrix-core products of all QW sets, so LDS traffic per product falls as 1 / QW.  With MASK,
// keys at or past n_lane[q] are masked (without it every key of the tile is below every n_lane of
// the wave).  Updates the running max m, sum l and the O^T accumulators o (lane (li, lg): dims
// db*16 + 4*lg + 0..3 of query li).  exp2 is the hardware v_exp_f32.
template <int D, int QW, bool MASK>
__device__ __forceinline__ void attn_tile_m(const u32x4* Ks, const u32x4* Vt, const bf16x8_v (&qf)[QW][D / 32],
                                            int j0, const int (&n_lane)[QW], float sc, float (&m)[QW],
                                            float (&l)[QW], f32x4 (&o)[QW][D / 16], int li, int lg) {
    constexpr int NT = D / 32, ND = D / 16, KCH = D / 8, KSW = KCH - 1;
    // S^T blocks: lane holds keys j0 + kb*16 + 4*lg + i for its query of set q
    f32x4 s[QW][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int q = 0; q < QW; ++q) s[q][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int key = kb * 16 + li;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const bf16x8_v kf = __builtin_bit_cast(bf16x8_v, Ks[key * KCH + ((t * 4 + lg) ^ (key & KSW))]);
#pragma unroll
            for (int q = 0; q < QW; ++q) s[q][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[q][t], s[q][kb], 0, 0, 0);
        }
    }
    // Online softmax in the log2 domain.  Maxima are taken over the raw scores (sc > 0, so they
    // are the maxima of the scaled ones) and the scale enters the exponent's fma.  The running max
    // m of a query (the same in its 4 lanes) is raised, and l and o rescaled, only when some lane
    // of the wave holds a score more than kStaleLog2 above it; only then are the query's 4 lanes
    // combined (two cross-lane exchanges).  Until then p = 2^(s*sc - m) <= 2^kStaleLog2 with the
    // stale m, which changes no result (m cancels in o / l) and skips the rescale and the
    // exchanges on most tiles.
    constexpr float kStaleLog2 = 8.0f;
    bf16x8_v pf[QW][2];
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        float tmax = kNeg;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = s[q][kb][i];
                if constexpr (MASK) {
                    v = j0 + kb * 16 + 4 * lg + i < n_lane[q] ? v : kNeg;
                    s[q][kb][i] = v;
                }
                tmax = fmaxf(tmax, v);
            }
        if (__builtin_amdgcn_ballot_w64(tmax * sc > m[q] + kStaleLog2) != 0) {  // wave-uniform
            tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
            const float mn = fmaxf(m[q], tmax * sc);
            const float alpha = __builtin_amdgcn_exp2f(m[q] - mn);
            l[q] *= alpha;
#pragma unroll
            for (int i = 0; i < ND; ++i) o[q][i] *= alpha;
            m[q] = mn;
        }
        const float mq = m[q];
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float p = __builtin_amdgcn_exp2f(fmaf(s[q][kb][i], sc, -mq));
                if constexpr (MASK) p = s[q][kb][i] > 0.5f * kNeg ? p : 0.f;
                s[q][kb][i] = p;
                psum += p;
            }
        l[q] += psum;
        // P^T of the two 32-key halves as B operands
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            u32x4 pw;
            pw.x = pack_bf2(s[q][2 * c][0], s[q][2 * c][1]);
            pw.y = pack_bf2(s[q][2 * c][2], s[q][2 * c][3]);
            pw.z = pack_bf2(s[q][2 * c + 1][0], s[q][2 * c + 1][1]);
            pw.w = pack_bf2(s[q][2 * c + 1][2], s[q][2 * c + 1][3]);
            pf[q][c] = __builtin_bit_cast(bf16x8_v, pw);
        }
    }

    // O^T += V^T . P^T over the two 32-key halves
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int pr = 4 * c + lg;  // key groups 8c + lg and 8c + 4 + lg: this lane's 8 keys of half c
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            const int d = db * 16 + li;
            const bf16x8_v vf = __builtin_bit_cast(bf16x8_v, Vt[d * 8 + (pr ^ ((d >> 1) & 7))]);
#pragma unroll
            for (int q = 0; q < QW; ++q) o[q][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[q][c], o[q][db], 0, 0, 0);
        }
    }
}

// The tile step for a wave whose queries all see at least n_min keys: the mask is applied only to
// tiles that reach n_min.
template <int D, int QW>
__device__ __forceinline__ void attn_tile(const u32x4* Ks, const u32x4* Vt, const bf16x8_v (&qf)[QW][D / 32], int j0,
                                          const int (&n_lane)[QW], int n_min, float sc, float (&m)[QW], float (&l)[QW],
                                          f32x4 (&o)[QW][D / 16], int li, int lg) {
    if (j0 + BKV <= n_min) attn_tile_m<D, QW, false>(Ks, Vt, qf, j0, n_lane, sc, m, l, o, li, lg);
    else attn_tile_m<D, QW, true>(Ks, Vt, qf, j0, n_lane, sc, m, l, o, li, lg);
}

}  // namespace
}  // namespace fsvd
