// Factorised attention: the attention of S tokens per sequence among themselves with the Q, K and
// V tiles rebuilt on chip from the rank-r activations z (q = z_q . Vt_q^T, k = z_k . Vt_k^T,
// v = z_v . Vt_v^T), so the full-sequence q, k and v are never written to memory - the streaming
// form of the fused low-rank attention ("FlashSVD: Memory-Efficient Inference with Streaming for
// Low-Rank Models", abstract).  Each key tile is rebuilt once per query tile that reads it: the
// price of not materialising K and V is that recomputation, so the query tile is large (128 or
// 256 queries, 8 waves) to rebuild each key tile as few times as possible.
//
// Per workgroup (one sequence, one query head, QROWS queries):
//   - the rank dimension is streamed in chunks of 64 components: the chunk of every operand row
//     (z rows of the queries or of the 64 keys, the head's D rows of Vt) goes global -> LDS with
//     direct loads (one 128-byte line per row, XOR-swizzled 16-byte slots) into 2 or 3 buffers, so
//     the next chunks are in flight while the current one feeds the matrix cores;
//   - the rebuild runs on v_mfma_f32_16x16x32_bf16: waves 0-3 rebuild the key tile, waves 4-7
//     the value tile, each wave a pair of 16-dimension blocks (d, d + D/2: a RoPE rotation pair)
//     times a group of 16-key blocks, so every fragment read from LDS feeds several products;
//   - Q and K are computed transposed (head dimension as the row of the product), which leaves a
//     lane holding 4 consecutive dimensions of one query or key: Q goes straight into the B
//     operand registers of the score product and K into the LDS key tile with 8-byte stores.
//     Both use the same order of the head dimension inside a 32-wide k step (dims 4q..4q+3 and
//     16+4q..16+4q+3 for lane group q), which leaves every q . k unchanged;
//   - rotate-half RoPE is applied to the rebuilt fp32 tiles in registers, the tiles are rounded to
//     bf16 (the precision of a materialised q, k, v) and the key tile is consumed by the MFMA
//     flash-attention tile step (attention_tile.h) for every query of the workgroup.
#include "attention_tile.h"

namespace fsvd {

namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kFThreads = 512;  // 8 waves
constexpr int kChunk = 64;      // rank components per staged chunk

// LDS slot of 16-byte chunk c (0..7) of staged row r: the 16 rows a quarter-wave reads for one
// MFMA fragment land in 16 distinct 16-byte bank groups
__device__ __forceinline__ int cslot(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int D, int QW>
struct FCfg {
    static constexpr int ND = D / 16, NT = D / 32, KCH = D / 8, KSW = KCH - 1;
    static constexpr int NDP = ND / 2;                  // RoPE pairs of 16-dimension blocks
    static constexpr int KB = NDP;                      // 16-key blocks per rebuild wave
    static constexpr int QROWS = 8 * 16 * QW;           // queries per workgroup (QW sets of 16 per wave)
    static constexpr int KV_ROWS = 2 * BKV + 2 * D;     // staged rows of a key-tile chunk: zk, zv, Vk, Vv
    static constexpr int Q_ROWS = QROWS + D;            // staged rows of a query chunk: zq, Vq
    static constexpr int ROWS = KV_ROWS > Q_ROWS ? KV_ROWS : Q_ROWS;
    static constexpr int SLOTS = ROWS * 8;              // 16-byte slots of one chunk buffer
    static constexpr int NB = D == 64 ? 3 : 2;          // chunk buffers (jobs in flight + 1)
    static constexpr int Q_LOADS = Q_ROWS / 64, KV_LOADS = KV_ROWS / 64;  // load instructions per wave and job
    static constexpr size_t LDS = (size_t)NB * SLOTS * 16;  // dynamic: the chunk buffers
    static_assert(4 % NDP == 0, "dimension pairs must divide the 4 rebuild waves");
    static_assert(KV_ROWS % 64 == 0 && Q_ROWS % 64 == 0, "whole load instructions per wave");
};

// Per-lane constants of the direct loads.  A wave instruction fills 64 consecutive 16-byte slots,
// i.e. 8 staged rows of 8 chunks: lane l takes row l / 8 of the block and the global chunk whose
// swizzled home is its slot, cc = (l % 8) ^ ((row / 2) % 8); blocks start at multiples of 8 rows
// and a wave's blocks all have the parity of the wave index, so cc is the same for all of them.
struct LoadLane {
    int rl, cc8;  // row within the 8-row block, element offset of the lane's chunk
};

// rows row0 .. row0 + 7 (positions in the sequence; past S the last row is re-read) of the z
// matrix 'src' (leading dimension ld, rank r), rank chunk c0: the base address is wave-uniform,
// the lane offset 32-bit.  CLAMP = false: the rows are all below S and the chunk is within r.
template <bool CLAMP>
__device__ __forceinline__ void load_z_rows(const bf16_t* src, int64_t ld, int64_t zrow0, int row0, int S, int r,
                                            int c0, const LoadLane& ll, u32x4* dst) {
    if constexpr (CLAMP) {
        const int rs = min(row0, S - 1);
        const int lim = S - 1 - rs;
        const uint32_t off = (uint32_t)(min(ll.rl, lim) * (int)ld + min(c0 * kChunk + ll.cc8, r - 8));
        __builtin_amdgcn_global_load_lds((const void*)(src + (zrow0 + rs) * ld + off), (lds_void_t*)dst, 16, 0, 0);
    } else {
        const uint32_t off = (uint32_t)(ll.rl * (int)ld + ll.cc8);
        const bf16_t* base = src + (zrow0 + row0) * ld + c0 * kChunk;
        __builtin_amdgcn_global_load_lds((const void*)(base + off), (lds_void_t*)dst, 16, 0, 0);
    }
}
// rows row0 .. row0 + 7 of a factor Vt [*, r] (row-major, leading dimension r), rank chunk c0
template <bool CLAMP>
__device__ __forceinline__ void load_v_rows(const bf16_t* src, int64_t row0, int r, int c0, const LoadLane& ll,
                                            u32x4* dst) {
    const uint32_t off = CLAMP ? (uint32_t)(ll.rl * r + min(c0 * kChunk + ll.cc8, r - 8)) : (uint32_t)(ll.rl * r + ll.cc8);
    const bf16_t* base = src + row0 * r + (CLAMP ? 0 : c0 * kChunk);
    __builtin_amdgcn_global_load_lds((const void*)(base + off), (lds_void_t*)dst, 16, 0, 0);
}

// Direct global -> LDS loads of one chunk job into the buffer 'dst'; returns the number of load
// instructions this wave issued.  t < 0: rank chunk c0 of the query rows (q0 ..) and of Vt_q's
// head rows; t >= 0: rank chunk c0 of key tile t's z_k and z_v rows and of Vt_k's and Vt_v's
// kv-head rows.  Rank columns past r re-read the row's last 8 (masked in the products).
template <int D, int QW, bool CLAMP>
__device__ __forceinline__ int issue_job_t(const FactAttnArgs& a, int t, int c0, int64_t zrow0, int q0, int h, int g,
                                           int wave, const LoadLane& ll, u32x4* dst) {
    using C = FCfg<D, QW>;
    if (t < 0) {
#pragma unroll
        for (int i = 0; i < C::Q_LOADS; ++i) {
            const int blk = i * 8 + wave, rb = blk * 8;
            u32x4* d = dst + blk * 64;
            if (rb < C::QROWS) load_z_rows<CLAMP>(a.zq, a.ldz, zrow0, q0 + rb, a.S, a.rq, c0, ll, d);
            else load_v_rows<CLAMP>(a.Vq, (int64_t)h * D + (rb - C::QROWS), a.rq, c0, ll, d);
        }
        return C::Q_LOADS;
    }
    const int k0 = t * BKV;
#pragma unroll
    for (int i = 0; i < C::KV_LOADS; ++i) {
        const int blk = i * 8 + wave, rb = blk * 8;
        u32x4* d = dst + blk * 64;
        if (rb < BKV) load_z_rows<CLAMP>(a.zk, a.ldz, zrow0, k0 + rb, a.S, a.rk, c0, ll, d);
        else if (rb < 2 * BKV) load_z_rows<CLAMP>(a.zv, a.ldz, zrow0, k0 + (rb - BKV), a.S, a.rv, c0, ll, d);
        else if (rb < 2 * BKV + D) load_v_rows<CLAMP>(a.Vk, (int64_t)g * D + (rb - 2 * BKV), a.rk, c0, ll, d);
        else load_v_rows<CLAMP>(a.Vv, (int64_t)g * D + (rb - 2 * BKV - D), a.rv, c0, ll, d);
    }
    return C::KV_LOADS;
}
// the clamps only matter for the last rank chunk or rows reaching the end of the sequence
template <int D, int QW>
__device__ __forceinline__ int issue_job(const FactAttnArgs& a, int t, int c0, int64_t zrow0, int q0, int h, int g,
                                         int wave, const LoadLane& ll, u32x4* dst) {
    using C = FCfg<D, QW>;
    const int rmin = t < 0 ? a.rq : min(a.rk, a.rv);
    const int rows_end = t < 0 ? q0 + C::QROWS : (t + 1) * BKV;
    if ((c0 + 1) * kChunk <= rmin && rows_end <= a.S)
        return issue_job_t<D, QW, false>(a, t, c0, zrow0, q0, h, g, wave, ll, dst);
    return issue_job_t<D, QW, true>(a, t, c0, zrow0, q0, h, g, wave, ll, dst);
}

__device__ __forceinline__ bf16x8_v frag(const u32x4* buf, int row, int c) {
    return __builtin_bit_cast(bf16x8_v, buf[cslot(row, c)]);
}
__device__ __forceinline__ bf16x8_v frag_masked(const u32x4* buf, int row, int c, bool zero) {
    u32x4 v = buf[cslot(row, c)];
    if (zero) v = u32x4{0u, 0u, 0u, 0u};
    return __builtin_bit_cast(bf16x8_v, v);
}

// wait until at most n (0..15) of this wave's vector-memory operations are outstanding
__device__ __forceinline__ void wait_vm_upto(int n) {
    switch (n) {
#define FSVD_WV(k) case k: __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(k)); break;
        FSVD_WV(1) FSVD_WV(2) FSVD_WV(3) FSVD_WV(4) FSVD_WV(5) FSVD_WV(6) FSVD_WV(7) FSVD_WV(8)
        FSVD_WV(9) FSVD_WV(10) FSVD_WV(11) FSVD_WV(12) FSVD_WV(13) FSVD_WV(14) FSVD_WV(15)
#undef FSVD_WV
        default: __builtin_amdgcn_s_waitcnt(FSVD_VMCNT(0)); break;
    }
}

// rotate-half RoPE on a transposed tile: lane (li, lg) holds dims db*16 + 4*lg + e of the row at
// position pos; the partner of block db < NDP is block db + NDP in the same lane
template <int NPAIR>
__device__ __forceinline__ void rope_t(f32x4* lo, f32x4* hi, int db0, int64_t pos, double base, int lg) {
#pragma unroll
    for (int p = 0; p < NPAIR; ++p)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float c, s;
            rope_cs(pos, (db0 + p) * 16 + 4 * lg + e, base, &c, &s);
            const float x1 = lo[p][e], x2 = hi[p][e];
            lo[p][e] = x1 * c - x2 * s;
            hi[p][e] = x2 * c + x1 * s;
        }
}

__device__ __forceinline__ uint2 pack4(const f32x4& v) {
    return uint2{pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3])};
}

template <int D, int QW>
__global__ __launch_bounds__(kFThreads) void attn_factorized_mfma(const FactAttnArgs a) {
    using C = FCfg<D, QW>;
    constexpr int ND = C::ND, NT = C::NT, NDP = C::NDP, KB = C::KB, KCH = C::KCH, KSW = C::KSW, NB = C::NB;
    // The rebuilt tiles are arrays of their own, apart from the chunk buffers that the direct
    // loads fill, so the compiler can tell that writing and reading them does not touch LDS
    // still being filled and keeps the chunk prefetch in flight across the attention step.
    extern __shared__ u32x4 CH[];                      // NB chunk buffers
    __shared__ u32x4 Ks[BKV * KCH];                    // key tile, permuted head order, swizzled
    __shared__ u32x4 Vt[D * 8];                        // value tile, transposed (vts_slot)
    bf16_t* Ks16 = reinterpret_cast<bf16_t*>(Ks);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int li = lane & 15, lg = lane >> 4;
    const int n_qt = (a.S + C::QROWS - 1) / C::QROWS;
    const int bh_count = a.B * a.Hq;
    // Heaviest (causal) query tiles first.  Workgroup i runs on XCD i mod 8: when the (sequence,
    // head) pairs split evenly over the 8 XCDs, XCD x takes a contiguous block of them, so its L2
    // holds the z rows of few sequences and the Vt rows of few heads.
    int qt, bh;
    if (bh_count % 8 == 0) {
        const int per = bh_count / 8, slot = (int)(blockIdx.x >> 3);
        qt = n_qt - 1 - slot / per;
        bh = (int)(blockIdx.x & 7) * per + slot % per;
    } else {
        qt = n_qt - 1 - (int)(blockIdx.x / bh_count);
        bh = blockIdx.x % bh_count;
    }
    const int h = bh % a.Hq, b = bh / a.Hq;
    const int g = (h * a.Hkv) / a.Hq;
    const int64_t zrow0 = (int64_t)b * a.S;  // z row of this sequence's token 0
    const int q0 = qt * C::QROWS;
    const bool rope = a.rope_theta > 0.f;

    const int kend = a.causal ? min(a.S, q0 + C::QROWS) : a.S;
    const int nq = (a.rq + kChunk - 1) / kChunk;
    const int nkv = (max(a.rk, a.rv) + kChunk - 1) / kChunk;
    const int ntile = (kend + BKV - 1) / BKV;

    int n_lane[QW], s_lane[QW];  // keys seen by this lane's query of each set
    int n_min_w = a.S;           // fewest keys any query of the wave sees
#pragma unroll
    for (int qs = 0; qs < QW; ++qs) {
        const int first = q0 + wave * 16 * QW + qs * 16;
        s_lane[qs] = first + li;
        n_lane[qs] = a.causal ? s_lane[qs] + 1 : a.S;
        if (s_lane[qs] >= a.S) n_lane[qs] = 0;
        n_min_w = min(n_min_w, first + 15 >= a.S ? 0 : (a.causal ? first + 1 : a.S));
    }

    // rebuild role: waves 0-3 the key tile (transposed), 4-7 the value tile; dimension blocks
    // dp and dp + NDP, key blocks kg * KB .. kg * KB + KB - 1
    const bool kwave = wave < 4;
    const int wr = wave & 3, dp = wr % NDP, kg = wr / NDP;
    const int r_mat = kwave ? a.rk : a.rv;

    // ---------------------------------------------------------------- chunk pipeline
    // Jobs in order: the nq rank chunks of the query tile (t = -1), then for each key tile t the
    // nkv rank chunks.  The issue cursor (it, ic) runs NB - 1 jobs ahead of the consumer.
    LoadLane ll;
    ll.rl = lane >> 3;
    ll.cc8 = ((lane & 7) ^ (((wave & 1) * 4 + (ll.rl >> 1)) & 7)) * 8;
    int it = -1, ic = 0, islot = 0;
    int nl[NB > 2 ? NB - 2 : 1] = {};  // load instructions of the issued jobs not yet consumed (after the next)
    // Key-tile chunks away from the sequence end and the rank tail take their addresses from a
    // plan made once per tile: a wave-uniform row base per load instruction and the lane's offset
    // (row within the block, swizzled chunk), to which each chunk adds 64 rank columns.
    const int rkv_min = min(a.rk, a.rv);
    const bf16_t* pbase[C::KV_LOADS];
    uint32_t poff[C::KV_LOADS];
    int plan_t = -1;
    auto make_plan = [&](int t) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::KV_LOADS; ++i) {
            const int rb = (i * 8 + wave) * 8;
            const bf16_t* src;
            int64_t row, ld;
            if (rb < BKV) { src = a.zk; row = zrow0 + t * BKV + rb; ld = a.ldz; }
            else if (rb < 2 * BKV) { src = a.zv; row = zrow0 + t * BKV + (rb - BKV); ld = a.ldz; }
            else if (rb < 2 * BKV + D) { src = a.Vk; row = (int64_t)g * D + (rb - 2 * BKV); ld = a.rk; }
            else { src = a.Vv; row = (int64_t)g * D + (rb - 2 * BKV - D); ld = a.rv; }
            pbase[i] = src + row * ld;
            poff[i] = (uint32_t)(ll.rl * (int)ld + ll.cc8);
        }
        plan_t = t;
    };
    auto issue_next = [&]() __attribute__((always_inline)) -> int {
        if (it >= ntile) return 0;
        int n;
        u32x4* dst = CH + islot * C::SLOTS;
        if (it >= 0 && (it + 1) * BKV <= a.S && (ic + 1) * kChunk <= rkv_min) {
            if (plan_t != it) make_plan(it);
#pragma unroll
            for (int i = 0; i < C::KV_LOADS; ++i)
                __builtin_amdgcn_global_load_lds((const void*)(pbase[i] + ic * kChunk + poff[i]),
                                                 (lds_void_t*)(dst + (i * 8 + wave) * 64), 16, 0, 0);
            n = C::KV_LOADS;
        } else {
            n = issue_job<D, QW>(a, it, ic, zrow0, q0, h, g, wave, ll, dst);
        }
        islot = islot + 1 == NB ? 0 : islot + 1;
        if (++ic == (it < 0 ? nq : nkv)) { ic = 0; ++it; }
        return n;
    };
#pragma unroll
    for (int j = 0; j < NB - 1; ++j) {
        const int n = issue_next();
        if (NB > 2 && j >= 1) nl[j - 1] = n;
    }
    int cslot_buf = 0;
    // wait for the consumed job's chunk (the NB - 2 jobs after it stay in flight), barrier (every
    // wave's part landed; every wave is done with the buffer about to be refilled), refill
    auto step = [&]() __attribute__((always_inline)) -> const u32x4* {
        int pending = 0;
#pragma unroll
        for (int d = 0; d < NB - 2; ++d) pending += nl[d];
        wait_vm_upto(pending);
        lds_barrier();
        const int n = issue_next();
        if constexpr (NB > 2) {
#pragma unroll
            for (int d = 0; d + 1 < NB - 2; ++d) nl[d] = nl[d + 1];
            nl[NB - 3] = n;
        }
        const u32x4* buf = CH + cslot_buf * C::SLOTS;
        cslot_buf = cslot_buf + 1 == NB ? 0 : cslot_buf + 1;
        return buf;
    };

    bf16x8_v qf[QW][NT];
    float m[QW], l[QW];
    f32x4 o[QW][ND];
    const float sc = a.scale * kLog2e;

    // ---------------------------------------------------------------- Q^T = Vt_q . z_q^T
    {
        f32x4 accq[QW][ND];
#pragma unroll
        for (int qs = 0; qs < QW; ++qs)
#pragma unroll
            for (int db = 0; db < ND; ++db) accq[qs][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nq; ++c0) {
            const u32x4* buf = step();
            const bool last = (c0 + 1) * kChunk > a.rq;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int c = s * 4 + lg;
                const bool zero = last && c0 * kChunk + c * 8 >= a.rq;
                bf16x8_v av[ND];
#pragma unroll
                for (int db = 0; db < ND; ++db) av[db] = frag(buf, C::QROWS + db * 16 + li, c);
#pragma unroll
                for (int qs = 0; qs < QW; ++qs) {
                    const bf16x8_v bz = frag_masked(buf, wave * 16 * QW + qs * 16 + li, c, zero);
#pragma unroll
                    for (int db = 0; db < ND; ++db)
                        accq[qs][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[db], bz, accq[qs][db], 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int qs = 0; qs < QW; ++qs) {
            if (rope) rope_t<NDP>(&accq[qs][0], &accq[qs][NDP], 0, s_lane[qs], a.rope_base, lg);
            // B operand of the score product: elements 0-3 from block 2t, 4-7 from block 2t + 1
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const uint2 lo = pack4(accq[qs][2 * t]), hi = pack4(accq[qs][2 * t + 1]);
                qf[qs][t] = __builtin_bit_cast(bf16x8_v, u32x4{lo.x, lo.y, hi.x, hi.y});
            }
            m[qs] = kNeg;
            l[qs] = 0.f;
#pragma unroll
            for (int db = 0; db < ND; ++db) o[qs][db] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }

    // ---------------------------------------------------------------- key tiles
    for (int t = 0; t < ntile; ++t) {
        f32x4 acc[KB][2];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[kb][0] = acc[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int c0 = 0; c0 < nkv; ++c0) {
            const u32x4* buf = step();  // chunk landed everywhere; previous chunk and tile fully read
            if (c0 * kChunk >= r_mat) continue;  // this wave's rank is shorter than the other one
            const bool last = (c0 + 1) * kChunk > r_mat;  // the chunk reaches past r: mask its tail
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int c = s * 4 + lg;
                const bool zero = last && c0 * kChunk + c * 8 >= r_mat;
                if (kwave) {  // K^T[d][key] = Vt_k[d] . z_k[key]
                    bf16x8_v vk[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) vk[hh] = frag(buf, 2 * BKV + (dp + hh * NDP) * 16 + li, c);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const bf16x8_v zf = frag_masked(buf, (kg * KB + kb) * 16 + li, c, zero);
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            acc[kb][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vk[hh], zf, acc[kb][hh], 0, 0, 0);
                    }
                } else {  // V[key][d] = z_v[key] . Vt_v[d]
                    bf16x8_v vv[2];
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) vv[hh] = frag(buf, 2 * BKV + D + (dp + hh * NDP) * 16 + li, c);
#pragma unroll
                    for (int kb = 0; kb < KB; ++kb) {
                        const bf16x8_v zf = frag_masked(buf, BKV + (kg * KB + kb) * 16 + li, c, zero);
#pragma unroll
                        for (int hh = 0; hh < 2; ++hh)
                            acc[kb][hh] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zf, vv[hh], acc[kb][hh], 0, 0, 0);
                    }
                }
            }
        }

        // tile t rebuilt: RoPE on K, round to bf16 into the LDS tiles, attend
        const int j0 = t * BKV;
        if (kwave) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int key = (kg * KB + kb) * 16 + li;
                if (rope) rope_t<1>(&acc[kb][0], &acc[kb][1], dp, j0 + key, a.rope_base, lg);
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int db = dp + hh * NDP, tt = db >> 1, half = db & 1;
                    *reinterpret_cast<uint2*>(Ks16 + (key * KCH + ((tt * 4 + lg) ^ (key & KSW))) * 8 + half * 4) =
                        pack4(acc[kb][hh]);
                }
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const int d = (dp + hh * NDP) * 16 + li, kc = (kg * KB + kb) * 4 + lg;
                    reinterpret_cast<uint2*>(Vt)[vts_slot(d, kc)] = pack4(acc[kb][hh]);
                }
        }
        lds_barrier();
        attn_tile<D, QW>(Ks, Vt, qf, j0, n_lane, n_min_w, sc, m, l, o, li, lg);
    }

#pragma unroll
    for (int qs = 0; qs < QW; ++qs) {
        float lt = l[qs];
        lt += __shfl_xor(lt, 16);
        lt += __shfl_xor(lt, 32);
        if (s_lane[qs] < a.S) {
            const float inv = lt > 0.f ? 1.0f / lt : 0.f;
            bf16_t* orow = a.out + (((int64_t)b * a.S + s_lane[qs]) * a.Hq + h) * D;
#pragma unroll
            for (int db = 0; db < ND; ++db) {
                const f32x4 v = o[qs][db] * inv;
                *reinterpret_cast<uint2*>(orow + db * 16 + 4 * lg) = pack4(v);
            }
        }
    }
}

template <int D, int QW>
fsvd_status_t launch_fact(const FactAttnArgs& a, hipStream_t st) {
    using C = FCfg<D, QW>;
    const int64_t n_qt = (a.S + C::QROWS - 1) / C::QROWS;
    const int64_t grid = n_qt * a.B * a.Hq;
    if (grid <= 0) return FSVD_OK;
    if (grid > 0x7fffffff) return fail(FSVD_ERR_UNSUPPORTED, "attention grid too large");
    if (const fsvd_status_t s = allow_dynamic_lds((const void*)attn_factorized_mfma<D, QW>, C::LDS,
                                                  "attn_factorized_mfma"))
        return s;
    attn_factorized_mfma<D, QW><<<(unsigned)grid, kFThreads, C::LDS, st>>>(a);
    return check_launch("attn_factorized_mfma");
}

#ifndef FSVD_FACT_QW
#define FSVD_FACT_QW 0  // queries per wave / 16: 0 = chosen per launch
#endif

}  // namespace

fsvd_status_t launch_attn_factorized(const FactAttnArgs& a, hipStream_t st) {
    if (a.D != 64 && a.D != 128) return fail(FSVD_ERR_UNSUPPORTED, "head dim %d not in {64,128}", a.D);
    // D = 64: 256 queries per workgroup (every key tile rebuilt half as often) while that still
    // gives at least 128 workgroups (measured faster than twice as many 128-query workgroups at
    // the BERT-Base shape), else 128.  D = 128: 128 (256 would not fit the registers).
    if (a.D == 128) return launch_fact<128, 1>(a, st);
    int qw = FSVD_FACT_QW;
    if (qw == 0) {
        const int64_t wg256 = (int64_t)((a.S + 255) / 256) * a.B * a.Hq;
        qw = wg256 >= 128 ? 2 : 1;
    }
    return qw == 2 ? launch_fact<64, 2>(a, st) : launch_fact<64, 1>(a, st);
}

}  // namespace fsvd
