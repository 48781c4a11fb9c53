// Factorised attention: the attention of S tokens per sequence among themselves with the Q, K and
// V tiles rebuilt on chip from the rank-r activations z (q = z_q . Vt_q^T, k = z_k . Vt_k^T,
// v = z_v . Vt_v^T), so the full-sequence q, k and v are never written to memory - the streaming
// form of the fused low-rank attention ("FlashSVD: Memory-Efficient Inference with Streaming for
// Low-Rank Models", abstract).  Each key tile is rebuilt once per query tile that reads it: the
// price of not materialising K and V is that recomputation.
//
// A workgroup owns 64 queries of one (sequence, query head), a wave 16 of them.  Rebuild of a
// 16-row tile on the matrix cores (v_mfma_f32_16x16x32_bf16): the A operand is 16 rows of z x 32
// rank components, the B operand 16 rows of Vt (16 head dimensions) x the same 32 components, so
// C holds 16 rows x 16 dimensions in fp32; RoPE rotates the pair (d, d + D/2) in registers (both
// halves sit in the same lane).  The rebuilt tiles are written as bf16 into the LDS layouts of the
// MFMA flash-attention tile step (attention_tile.h), which then runs unchanged.
#include "attention_tile.h"

namespace fsvd {

namespace {

// acc[db] = C[row 4*(lane/16) + e][dimension db*16 + lane%16] of rows row0 .. row0 + 15 of z
// (clamped to row_last) times rows vrow0 .. vrow0 + D - 1 of Vt (row stride r).
template <int D>
__device__ __forceinline__ void rebuild_rows(const bf16_t* z, int64_t ldz, int64_t row0, int64_t row_last,
                                             const bf16_t* Vt, int64_t vrow0, int r, f32x4 (&acc)[D / 16], int lane) {
    constexpr int ND = D / 16;
    const int rj = lane & 15, kq = lane >> 4;
    const bf16_t* zp = z + min(row0 + rj, row_last) * ldz;
    const bf16_t* vp = Vt + (vrow0 + rj) * (int64_t)r;
#pragma unroll
    for (int db = 0; db < ND; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nst = (r + 31) / 32;
    for (int st = 0; st < nst; ++st) {
        const int k = st * 32 + kq * 8;
        const int kc = min(k, r - 8);  // r is a multiple of 8: a lane's 8 components are all in or all out
        u32x4 av = *reinterpret_cast<const u32x4*>(zp + kc);
        if (k >= r) av = u32x4{0u, 0u, 0u, 0u};
        const bf16x8_v af = __builtin_bit_cast(bf16x8_v, av);
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            const u32x4 bv = *reinterpret_cast<const u32x4*>(vp + (int64_t)db * 16 * r + kc);
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, __builtin_bit_cast(bf16x8_v, bv), acc[db], 0, 0, 0);
        }
    }
}

// rotate-half RoPE on a rebuilt tile: row 4*kq + e sits at position pos0 + 4*kq + e
template <int D>
__device__ __forceinline__ void rope_rows(f32x4 (&acc)[D / 16], int64_t pos0, double base, int lane) {
    constexpr int ND = D / 16;
    const int rj = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int db = 0; db < ND / 2; ++db) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float c, s;
            rope_cs(pos0 + 4 * kq + e, db * 16 + rj, base, &c, &s);
            const float x1 = acc[db][e], x2 = acc[db + ND / 2][e];
            acc[db][e] = x1 * c - x2 * s;
            acc[db + ND / 2][e] = x2 * c + x1 * s;
        }
    }
}

template <int D>
__global__ __launch_bounds__(256) void attn_factorized_mfma(const FactAttnArgs a) {
    constexpr int NT = D / 32, ND = D / 16, KCH = D / 8, KSW = KCH - 1;
    __shared__ u32x4 Ks[BKV * KCH];  // K rows (first: the Q tile, row-major, unswizzled)
    __shared__ uint2 Vts[D * 16];
    bf16_t* Ks16 = reinterpret_cast<bf16_t*>(Ks);
    bf16_t* Vt16 = reinterpret_cast<bf16_t*>(Vts);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int li = lane & 15, lg = lane >> 4;
    const int n_qt = (a.S + BQ - 1) / BQ;
    const int bh_count = a.B * a.Hq;
    const int qt = n_qt - 1 - (int)(blockIdx.x / bh_count);  // heaviest (causal) tiles first
    const int bh = blockIdx.x % bh_count;
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int g = (h * a.Hkv) / a.Hq;
    const int64_t zrow0 = (int64_t)b * a.S;           // z row of this sequence's token 0
    const int64_t zlast = zrow0 + a.S - 1;
    const bool rope = a.rope_theta > 0.f;

    const int64_t kend = a.causal ? min(a.S, qt * BQ + BQ) : a.S;
    const int s_lane = qt * BQ + wave * 16 + li;
    int64_t n_lane = a.causal ? s_lane + 1 : a.S;
    if (s_lane >= a.S) n_lane = 0;

    // Q tile: rebuilt, rotated, staged row-major in Ks, read back as the B operand
    f32x4 acc[ND];
    {
        const int64_t q0 = qt * BQ + wave * 16;
        rebuild_rows<D>(a.zq, a.ldz, zrow0 + q0, zlast, a.Vq, (int64_t)h * D, a.rq, acc, lane);
        if (rope) rope_rows<D>(acc, q0, a.rope_base, lane);
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e) Ks16[(wave * 16 + 4 * lg + e) * D + db * 16 + li] = f2bf(acc[db][e]);
    }
    __syncthreads();
    bf16x8_v qf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        qf[t] = __builtin_bit_cast(bf16x8_v, *reinterpret_cast<const u32x4*>(Ks16 + (wave * 16 + li) * D + t * 32 + lg * 8));

    float m = kNeg, l = 0.f;
    f32x4 o[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    const float sc = a.scale * kLog2e;

    for (int64_t j0 = 0; j0 < kend; j0 += BKV) {
        __syncthreads();  // the previous tile (or the Q staging) has been read by every wave
        const int64_t k0 = j0 + wave * 16;
        rebuild_rows<D>(a.zk, a.ldz, zrow0 + k0, zlast, a.Vk, (int64_t)g * D, a.rk, acc, lane);
        if (rope) rope_rows<D>(acc, k0, a.rope_base, lane);
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = wave * 16 + 4 * lg + e, d = db * 16 + li;
                Ks16[(key * KCH + ((d >> 3) ^ (key & KSW))) * 8 + (d & 7)] = f2bf(acc[db][e]);
            }
        rebuild_rows<D>(a.zv, a.ldz, zrow0 + k0, zlast, a.Vv, (int64_t)g * D, a.rv, acc, lane);
#pragma unroll
        for (int db = 0; db < ND; ++db)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int key = wave * 16 + 4 * lg + e, d = db * 16 + li;
                Vt16[(d * 16 + ((key >> 2) ^ (d & 15))) * 4 + (key & 3)] = f2bf(acc[db][e]);
            }
        __syncthreads();
        attn_tile<D>(Ks, Vts, qf, j0, n_lane, sc, m, l, o, li, lg);
    }

    float lt = l;
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (s_lane < a.S) {
        const float inv = lt > 0.f ? 1.0f / lt : 0.f;
        bf16_t* orow = a.out + (((int64_t)b * a.S + s_lane) * a.Hq + h) * D;
#pragma unroll
        for (int db = 0; db < ND; ++db) {
            const uint2 w = uint2{pack_bf2(o[db][0] * inv, o[db][1] * inv), pack_bf2(o[db][2] * inv, o[db][3] * inv)};
            *reinterpret_cast<uint2*>(orow + db * 16 + 4 * lg) = w;
        }
    }
}

}  // namespace

fsvd_status_t launch_attn_factorized(const FactAttnArgs& a, hipStream_t st) {
    const int n_qt = (a.S + BQ - 1) / BQ;
    const int64_t grid = (int64_t)n_qt * a.B * a.Hq;
    if (grid <= 0) return FSVD_OK;
    if (grid > 0x7fffffff) return fail(FSVD_ERR_UNSUPPORTED, "attention grid too large");
    if (a.D == 128) attn_factorized_mfma<128><<<(unsigned)grid, 256, 0, st>>>(a);
    else if (a.D == 64) attn_factorized_mfma<64><<<(unsigned)grid, 256, 0, st>>>(a);
    else return fail(FSVD_ERR_UNSUPPORTED, "head dim %d not in {64,128}", a.D);
    return check_launch("attn_factorized_mfma");
}

}  // namespace fsvd
