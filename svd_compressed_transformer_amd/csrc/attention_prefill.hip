// Attention of several new tokens per sequence (prefill, encoder layers) over the contiguous
// dense KV cache, on the matrix cores (gfx950, v_mfma_f32_16x16x32_bf16).
//
// A workgroup owns 64 consecutive queries of one (sequence, query head); each of its 4 waves owns
// 16 of them.  Key/value tiles of 64 positions are staged in LDS (K row-major, V transposed so
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

template <int D>
__global__ __launch_bounds__(256) void attn_prefill_mfma(const AttnArgs a) {
    constexpr int NT = D / 32;        // 32-wide k steps of q . k
    constexpr int ND = D / 16;        // 16-wide d blocks of the output
    constexpr int KCH = D / 8;        // 16-byte chunks per K row
    constexpr int KSW = KCH - 1;      // K swizzle mask (KCH is 8 or 16)
    constexpr int KLD = BKV * KCH / 256;   // K chunks staged per thread
    constexpr int VG = 16 * (D / 8);       // V staging groups of 4 keys x 8 dims
    constexpr int VLD = (VG + 255) / 256;  // groups per thread
    __shared__ u32x4 Ks[BKV * KCH];
    __shared__ uint2 Vts[D * 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n_qt = (a.Sq + BQ - 1) / BQ;
    const int bh_count = a.B * a.Hq;
    const int qt = n_qt - 1 - (int)(blockIdx.x / bh_count);
    const int bh = blockIdx.x % bh_count;
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int g = (h * a.Hkv) / a.Hq;
    const int64_t base = a.seqlens[b];

    int64_t kend = a.causal ? base + min(a.Sq, qt * BQ + BQ) : base + a.Sq;
    if (kend > a.L_max) {
        if (tid == 0 && qt == n_qt - 1) set_dev_error(a.err, FSVD_DEVERR_SEQ_OVERFLOW);
        kend = a.L_max;
    }
    const int s_lane = qt * BQ + wave * 16 + li;           // this lane's query
    int64_t n_lane = a.causal ? base + s_lane + 1 : base + a.Sq;
    if (n_lane > a.L_max) n_lane = a.L_max;
    if (s_lane >= a.Sq) n_lane = 0;
    // fewest keys any query of this wave sees (tiles below it need no mask)
    const int first = qt * BQ + wave * 16;
    int64_t n_min = a.causal ? base + first + 1 : base + a.Sq;
    if (n_min > a.L_max) n_min = a.L_max;
    if (first + 15 >= a.Sq) n_min = 0;

    // Q as the B operand: lane (li, lg) holds q[s_lane][t*32 + lg*8 .. +7]
    bf16x8_v qf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        u32x4 v = u32x4{0u, 0u, 0u, 0u};
        if (s_lane < a.Sq) v = *reinterpret_cast<const u32x4*>(a.q + (((int64_t)b * a.Sq + s_lane) * a.Hq + h) * D + t * 32 + lg * 8);
        qf[t] = __builtin_bit_cast(bf16x8_v, v);
    }

    const int64_t rowstride = (int64_t)a.Hkv * D;
    const bf16_t* kb0 = a.kc + ((int64_t)b * a.L_max * a.Hkv + g) * D;
    const bf16_t* vb0 = a.vc + ((int64_t)b * a.L_max * a.Hkv + g) * D;

    u32x4 kreg[KLD];
    u32x4 vreg[VLD][4];
    auto prefetch = [&](int64_t j0) {
#pragma unroll
        for (int i = 0; i < KLD; ++i) {
            const int q = tid + 256 * i;
            const int key = q / KCH, ch = q % KCH;
            const int64_t j = j0 + key;
            kreg[i] = j < kend ? *reinterpret_cast<const u32x4*>(kb0 + j * rowstride + ch * 8) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const int gi = tid + 256 * i;
            const int kc = gi & 15, dg = gi >> 4;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t j = j0 + kc * 4 + r;
                vreg[i][r] = (gi < VG && j < kend) ? *reinterpret_cast<const u32x4*>(vb0 + j * rowstride + dg * 8)
                                                   : u32x4{0u, 0u, 0u, 0u};
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
                Vts[d * 16 + (kc ^ (d & 15))] = uint2{v0 | (v1 << 16), v2 | (v3 << 16)};
            }
        }
    };

    float m = kNeg, l = 0.f;
    f32x4 o[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float sc = a.scale * kLog2e;

    if (kend > 0) prefetch(0);
    for (int64_t j0 = 0; j0 < kend; j0 += BKV) {
        __syncthreads();
        stage();
        __syncthreads();
        if (j0 + BKV < kend) prefetch(j0 + BKV);

        attn_tile<D>(Ks, Vts, qf, (int)j0, (int)n_lane, (int)n_min, sc, m, l, o, li, lg);
    }

    float lt = l;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (s_lane < a.Sq) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        bf16_t* orow = a.out + (((int64_t)b * a.Sq + s_lane) * a.Hq + h) * D;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            const uint2 w = uint2{pack_bf2(o[db][0] * inv, o[db][1] * inv), pack_bf2(o[db][2] * inv, o[db][3] * inv)};
            *reinterpret_cast<uint2*>(orow + db * 16 + 4 * lg) = w;
        }
    }
}

}  // namespace

fsvd_status_t launch_attn_prefill(const AttnArgs& a, hipStream_t st) {
    const int n_qt = (a.Sq + BQ - 1) / BQ;
    const int64_t grid = (int64_t)n_qt * a.B * a.Hq;
    if (grid <= 0) return FSVD_OK;
    if (grid > 0x7fffffff) return fail(FSVD_ERR_UNSUPPORTED, "attention grid too large");
    if (a.L_max > 0x7fffffff - 64) return fail(FSVD_ERR_UNSUPPORTED, "cache length %lld too large", (long long)a.L_max);
    if (a.D == 128) attn_prefill_mfma<128><<<(unsigned)grid, 256, 0, st>>>(a);
    else if (a.D == 64) attn_prefill_mfma<64><<<(unsigned)grid, 256, 0, st>>>(a);
    else return fail(FSVD_ERR_UNSUPPORTED, "head dim %d not in {64,128}", a.D);
    return check_launch("attn_prefill_mfma");
}

}  // namespace fsvd
