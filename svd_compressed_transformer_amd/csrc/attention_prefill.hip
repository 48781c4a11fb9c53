// Attention of several new tokens per sequence (prefill, encoder layers) over the contiguous
// dense KV cache, on the matrix cores (gfx950, v_mfma_f32_16x16x32_bf16).
//
// A workgroup owns 64 x QW consecutive queries of one (sequence, query head); each of its 4 waves
// owns QW sets of 16 (set q of wave w: queries q*64 + w*16 .. +15 of the block, so causal work is
// balanced over the waves) and every K/V fragment it reads from LDS feeds the products of all its
// sets.  Key/value tiles of 64 positions are staged in LDS (K row-major, V transposed so
// keys are contiguous) with XOR-swizzled chunk positions, prefetched into registers one tile
// ahead.  Each wave computes S^T = K . Q^T (keys x queries) so that a lane ends up holding the
// scores of ONE query for 16 keys; after the online-softmax update those probabilities are
// exactly the B operand of O^T = V^T . P^T for the same lane, so P never leaves registers.
// Causal masking skips key tiles past the workgroup's last query and the heaviest query tiles are
// dispatched first.  Softmax in fp32 with exp2, accumulation in fp32, bf16 output.
//
// Source: dense-KV attention over a contiguous cache ("FlashSVD v1.5" explainer, Methodology 2);
// prefill attention on the full sequence (same page, Methodology 2, prefill paragraph).
#include "attention_tile.h"

namespace fsvd {

namespace {

template <int D, int QW>
__global__ __launch_bounds__(256, 2) void attn_prefill_mfma(const AttnArgs a) {
    constexpr int BQW = BQ * QW;      // queries per workgroup
    constexpr int NT = D / 32;        // 32-wide k steps of q . k
    constexpr int ND = D / 16;        // 16-wide d blocks of the output
    constexpr int KCH = D / 8;        // 16-byte chunks per K row
    constexpr int KSW = KCH - 1;      // K swizzle mask (KCH is 8 or 16)
    constexpr int KLD = BKV * KCH / 256;   // K chunks staged per thread
    constexpr int VG = 16 * (D / 8);       // V staging groups of 4 keys x 8 dims
    constexpr int VLD = (VG + 255) / 256;  // groups per thread
    __shared__ u32x4 Ks[BKV * KCH];
    __shared__ u32x4 Vt[D * 8];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n_qt = (a.Sq + BQW - 1) / BQW;
    const int bh_count = a.B * a.Hq;
    const int qt = n_qt - 1 - (int)(blockIdx.x / bh_count);
    const int bh = blockIdx.x % bh_count;
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int g = (h * a.Hkv) / a.Hq;
    const int64_t base = (int64_t)a.seqlens[b] + a.pos_off;

    int64_t kend = a.causal ? base + min(a.Sq, qt * BQW + BQW) : base + a.Sq;
    if (kend > a.L_max) {
        if (tid == 0 && qt == n_qt - 1) set_dev_error(a.err, FSVD_DEVERR_SEQ_OVERFLOW);
        kend = a.L_max;
    }
    // per query set: this lane's query, the keys it sees, and the fewest keys any query of the
    // wave sees (tiles below that need no mask); cache lengths fit int (checked at launch)
    int s_lane[QW], n_lane[QW];
    int64_t n_min = a.L_max;
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        const int first = qt * BQW + q * BQ + wave * 16;
        s_lane[q] = first + li;
        int64_t nl = a.causal ? base + s_lane[q] + 1 : base + a.Sq;
        if (nl > a.L_max) nl = a.L_max;
        if (s_lane[q] >= a.Sq) nl = 0;
        n_lane[q] = (int)nl;
        int64_t nm = a.causal ? base + first + 1 : base + a.Sq;
        if (nm > a.L_max) nm = a.L_max;
        if (first + 15 >= a.Sq) nm = 0;
        n_min = min(n_min, nm);
    }

    // Q as the B operand: lane (li, lg) holds q[s_lane[q]][t*32 + lg*8 .. +7]
    bf16x8_v qf[QW][NT];
#pragma unroll
    for (int q = 0; q < QW; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (s_lane[q] < a.Sq)
                v = *reinterpret_cast<const u32x4*>(a.q + (((int64_t)b * a.Sq + s_lane[q]) * a.Hq + h) * D + t * 32 + lg * 8);
            qf[q][t] = __builtin_bit_cast(bf16x8_v, v);
        }

    const int64_t rowstride = (int64_t)a.Hkv * D;
    const bf16_t* kb0 = a.kc + ((int64_t)b * a.L_max * a.Hkv + g) * D;
    const bf16_t* vb0 = a.vc + ((int64_t)b * a.L_max * a.Hkv + g) * D;

    // Rows past kend (the last tile's tail) re-read row kend - 1, a written cache row: their keys
    // are masked (a select, so any finite K will do) and their values get probability 0 (finite V
    // keeps 0 * v at 0).  Unconditional loads keep the prefetch free of branches.
    u32x4 kreg[KLD];
    u32x4 vreg[VLD][4];
    auto prefetch = [&](int64_t j0) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int q = tid + 256 * i;
            const int key = q / KCH, ch = q % KCH;
            const int64_t j = min(j0 + key, kend - 1);
            kreg[i] = *reinterpret_cast<const u32x4*>(kb0 + j * rowstride + ch * 8);
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int gi = tid + 256 * i;
            if (gi >= VG) continue;  // wave-uniform (D = 64: the upper half of the workgroup)
            const int kc = gi & 15, dg = gi >> 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t j = min(j0 + kc * 4 + r, kend - 1);
                vreg[i][r] = *reinterpret_cast<const u32x4*>(vb0 + j * rowstride + dg * 8);
            }
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int q = tid + 256 * i;
            const int key = q / KCH, ch = q % KCH;
            Ks[key * KCH + (ch ^ (key & KSW))] = kreg[i];
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int gi = tid + 256 * i;
            if (gi >= VG) continue;
            const int kc = gi & 15, dg = gi >> 4;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1, sh = (e & 1) * 16;
                const uint32_t v0 = (vreg[i][0][w] >> sh) & 0xffffu, v1 = (vreg[i][1][w] >> sh) & 0xffffu;
                const uint32_t v2 = (vreg[i][2][w] >> sh) & 0xffffu, v3 = (vreg[i][3][w] >> sh) & 0xffffu;
                const int d = dg * 8 + e;
                reinterpret_cast<uint2*>(Vt)[vts_slot(d, kc)] = uint2{v0 | (v1 << 16), v2 | (v3 << 16)};
            }
        }
    };

    float m[QW], l[QW];
    f32x4 o[QW][ND];
#pragma unroll
    for (int q = 0; q < QW; ++q) {
        m[q] = kNeg;
        l[q] = 0.f;
#pragma unroll
        for (int i = 0; i < ND; ++i) o[q][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float sc = a.scale * kLog2e;

    if (kend > 0) prefetch(0);
    for (int64_t j0 = 0; j0 < kend; j0 += BKV) {
        __syncthreads();
        stage();
        __syncthreads();
        if (j0 + BKV < kend) prefetch(j0 + BKV);

        attn_tile<D, QW>(Ks, Vt, qf, (int)j0, n_lane, (int)n_min, sc, m, l, o, li, lg);
    }

#pragma unroll
    for (int q = 0; q < QW; ++q) {
        float lt = l[q];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (s_lane[q] < a.Sq) {
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;
            bf16_t* orow = a.out + (((int64_t)b * a.Sq + s_lane[q]) * a.Hq + h) * D;
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const uint2 w = uint2{pack_bf2(o[q][db][0] * inv, o[q][db][1] * inv),
                                      pack_bf2(o[q][db][2] * inv, o[q][db][3] * inv)};
                *reinterpret_cast<uint2*>(orow + db * 16 + 4 * lg) = w;
            }
        }
    }
}

template <int D, int QW>
fsvd_status_t launch_prefill_t(const AttnArgs& a, hipStream_t st) {
    const int64_t grid = (int64_t)((a.Sq + BQ * QW - 1) / (BQ * QW)) * a.B * a.Hq;
    if (grid > 0x7fffffff) return fail(FSVD_ERR_UNSUPPORTED, "attention grid too large");
    attn_prefill_mfma<D, QW><<<(unsigned)grid, 256, 0, st>>>(a);
    return check_launch("attn_prefill_mfma");
}

#ifndef FSVD_PREFILL_QW
#define FSVD_PREFILL_QW 0  // query sets per wave: 0 = chosen per launch
#endif

}  // namespace

// Two query sets per wave halve the LDS reads per product but also the workgroup count, so they
// are used when at least 1024 workgroups of 128 queries remain to fill the 256 CUs.
fsvd_status_t launch_attn_prefill(const AttnArgs& a, hipStream_t st) {
    if (a.Sq <= 0 || a.B <= 0 || a.Hq <= 0) return FSVD_OK;
    if (a.L_max > 0x7fffffff - 64) return fail(FSVD_ERR_UNSUPPORTED, "cache length %lld too large", (long long)a.L_max);
    const int64_t wg2 = (int64_t)((a.Sq + 2 * BQ - 1) / (2 * BQ)) * a.B * a.Hq;
    const int qw = FSVD_PREFILL_QW ? FSVD_PREFILL_QW : (wg2 >= 1024 ? 2 : 1);
    if (a.D == 128) return qw == 2 ? launch_prefill_t<128, 2>(a, st) : launch_prefill_t<128, 1>(a, st);
    if (a.D == 64) return qw == 2 ? launch_prefill_t<64, 2>(a, st) : launch_prefill_t<64, 1>(a, st);
    return fail(FSVD_ERR_UNSUPPORTED, "head dim %d not in {64,128}", a.D);
}

}  // namespace fsvd
