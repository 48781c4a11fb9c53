// C-ABI front of the fused low-rank layer library: argument validation, workspace carving,
// dispatch between the decode row-dot kernels (M <= 32 activation rows) and the bf16 MFMA
// kernels (larger M), the whole decoder layer, and its per-layer hipGraph.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <tuple>

#include "kernels.h"

namespace fsvd {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

fsvd_status_t fail(fsvd_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

fsvd_status_t check_launch(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FSVD_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return FSVD_OK;
}

fsvd_status_t allow_dynamic_lds(const void* fn, size_t bytes, const char* what) {
    static std::mutex mu;
    static std::set<std::tuple<const void*, int, size_t>> done;  // (kernel, device, bytes) set
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FSVD_ERR_HIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_tuple(fn, dev, bytes);
    if (done.count(key)) return FSVD_OK;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess)
        return fail(FSVD_ERR_HIP, "%s: raising dynamic LDS to %zu bytes: %s", what, bytes, hipGetErrorString(e));
    done.insert(key);
    return FSVD_OK;
}

namespace {

constexpr int kRowdotMaxM = 32;

// ------------------------------------------------------------------ validation helpers

fsvd_status_t need_ptr(const void* p, const char* name) {
    if (p == nullptr) return fail(FSVD_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p)) return fail(FSVD_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return FSVD_OK;
}
fsvd_status_t opt_ptr(const void* p, const char* name) {
    if (p != nullptr && !aligned16(p)) return fail(FSVD_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return FSVD_OK;
}
fsvd_status_t need_dim(int64_t v, const char* name) {
    if (v <= 0) return fail(FSVD_ERR_INVALID_ARG, "%s must be positive (got %lld)", name, (long long)v);
    if (v > (int64_t)1 << 30) return fail(FSVD_ERR_INVALID_ARG, "%s too large (%lld)", name, (long long)v);
    return FSVD_OK;
}
fsvd_status_t need_vec(int64_t v, fsvd_dtype_t t, const char* name) {
    const int64_t e = 16 / (int64_t)esize(t);
    if (v % e) return fail(FSVD_ERR_INVALID_ARG, "%s = %lld must be a multiple of %lld for 16-byte rows", name, (long long)v, (long long)e);
    return FSVD_OK;
}
fsvd_status_t need_ld(int64_t ld, int64_t extent, fsvd_dtype_t t, const char* name) {
    if (ld < extent) return fail(FSVD_ERR_INVALID_ARG, "%s = %lld smaller than the row extent %lld", name, (long long)ld, (long long)extent);
    if ((ld * (int64_t)esize(t)) % 16) return fail(FSVD_ERR_INVALID_ARG, "%s * element size must be a multiple of 16 bytes", name);
    return FSVD_OK;
}
// a rank above min(K, N) is never the truncation of a K x N map (and a padded rank stays within
// the bound, K and N being multiples of the padding)
fsvd_status_t need_rank(int64_t r, int64_t K, int64_t N, const char* name) {
    if (r > K || r > N)
        return fail(FSVD_ERR_INVALID_ARG, "%s = %lld exceeds min(K, N) = min(%lld, %lld)", name, (long long)r,
                    (long long)K, (long long)N);
    return FSVD_OK;
}
fsvd_status_t need_dtype(fsvd_dtype_t t, bool allow_f32) {
    if (t == FSVD_BF16) return FSVD_OK;
    if (t == FSVD_F32 && allow_f32) return FSVD_OK;
    if (t == FSVD_F32) return fail(FSVD_ERR_UNSUPPORTED, "this call supports bf16 only");
    return fail(FSVD_ERR_INVALID_ARG, "unknown dtype %d", (int)t);
}

#define TRY(expr)                                   \
    do {                                            \
        const fsvd_status_t _s = (expr);            \
        if (_s != FSVD_OK) return _s;               \
    } while (0)

// bump allocator over a workspace (256-byte aligned slices after the header)
struct Carve {
    char* base;
    size_t off;
    explicit Carve(void* ws) : base((char*)ws), off(kWsHeader) {}
    void* take(size_t bytes) {
        void* p = base ? base + off : nullptr;
        off += align256(bytes);
        return p;
    }
};

// ------------------------------------------------------------------ enqueue (no validation)

struct LinearBufs {
    void* z;        // [M, r] (dtype)
    int* err;
    float* part;    // row-dot split-reduction partials (rowdot_part_bytes), or NULL
};

fsvd_status_t enqueue_linear(const void* x, int M, int K, int64_t ldx, const void* Ut, int r, int64_t ldu,
                             const void* Vt, int N, int64_t ldv, const void* bias, const void* residual, int64_t ldr,
                             void* y, int64_t ldy, fsvd_dtype_t dt, const LinearBufs& wb, int32_t* adv, int advB,
                             int advn, hipStream_t st) {
    if (M <= kRowdotMaxM) {
        RowdotArgs a{};
        a.nseg = 1;
        a.act = x; a.lda = ldx; a.M = M; a.err = wb.err;
        a.seg[0].W = Ut; a.seg[0].ldw = ldu; a.seg[0].N = r; a.seg[0].K = K; a.seg[0].out = wb.z; a.seg[0].ldo = r;
        a.part = wb.part;
        TRY(launch_rowdot(a, EPI_Z, dt, st));
        RowdotArgs b{};
        b.nseg = 1;
        b.act = wb.z; b.lda = r; b.M = M; b.err = wb.err; b.part = wb.part;
        b.seg[0].W = Vt; b.seg[0].ldw = ldv; b.seg[0].N = N; b.seg[0].K = r; b.seg[0].out = y; b.seg[0].ldo = ldy;
        b.bias = bias; b.residual = residual; b.ldr = ldr;
        b.adv_seqlens = adv; b.adv_B = advB; b.adv_n = advn;
        return launch_rowdot(b, EPI_LINEAR, dt, st);
    }
    if (dt != FSVD_BF16) return fail(FSVD_ERR_UNSUPPORTED, "the MFMA path (M > %d) is bf16 only", kRowdotMaxM);
    GemmArgs g{};
    g.A = (const bf16_t*)x; g.lda = ldx; g.Bm = (const bf16_t*)Ut; g.ldb = ldu;
    g.M = M; g.N = r; g.K = K; g.C = (bf16_t*)wb.z; g.ldc = r; g.err = wb.err;
    TRY(launch_gemm(g, GEPI_STORE, st));
    GemmArgs h{};
    h.A = (const bf16_t*)wb.z; h.lda = r; h.Bm = (const bf16_t*)Vt; h.ldb = ldv;
    h.M = M; h.N = N; h.K = r; h.C = (bf16_t*)y; h.ldc = ldy;
    h.bias = (const bf16_t*)bias; h.residual = (const bf16_t*)residual; h.ldr = ldr; h.err = wb.err;
    TRY(launch_gemm(h, GEPI_LINEAR, st));
    if (adv) return launch_seqlens_advance(adv, advB, advn, st);
    return FSVD_OK;
}

struct QkvDims {
    int B, S, d, rq, rk, rv, Hq, Hkv, D;
    int64_t L_max;
    float eps, theta;
    int rows;     // token rows of this launch (0: all B * S)
    int row_off;  // first token row of this launch within the call's [B, S] tokens
};
struct QkvBufs {
    void* z;       // [M, rq+rk+rv] bf16
    void* xn;      // MFMA path: [M, d] bf16
    float* rstd;   // MFMA path: [M]
    int* err;
    float* part;   // row-dot split-reduction partials, or NULL
};

size_t qkv_scratch(int64_t M, int64_t d, int64_t rtot) {
    size_t s = align256((size_t)M * rtot * 2) + align256(rowdot_part_bytes(M, FSVD_BF16));
    if (M > kRowdotMaxM) s += align256((size_t)M * d * 2) + align256((size_t)M * 4);
    return s;
}

// norm: apply RMSNorm to x first; norm_w: its weight, or NULL when the weight is folded into A
fsvd_status_t enqueue_qkv(const QkvDims& q, const void* x, bool norm, const void* norm_w, const void* A, const void* Vq,
                          const void* Vk, const void* Vv, void* q_out, void* kc, void* vc, const int32_t* seqlens,
                          void* k_out, void* v_out, const QkvBufs& wb, hipStream_t st) {
    const int M = q.rows > 0 ? q.rows : q.B * q.S;
    const int rtot = q.rq + q.rk + q.rv;
    if (M <= kRowdotMaxM) {
        if (q.row_off != 0) return fail(FSVD_ERR_UNSUPPORTED, "row-dot Q/K/V launch with a row offset");
        RowdotArgs a{};
        a.nseg = 1;
        a.act = x; a.lda = q.d; a.M = M; a.err = wb.err;
        a.norm = norm; a.norm_w = (const bf16_t*)norm_w; a.norm_eps = q.eps; a.norm_K = q.d;
        a.seg[0].W = A; a.seg[0].ldw = q.d; a.seg[0].N = rtot; a.seg[0].K = q.d; a.seg[0].out = wb.z; a.seg[0].ldo = rtot;
        a.part = wb.part;
        TRY(launch_rowdot(a, EPI_Z, FSVD_BF16, st));
        RowdotArgs b{};
        b.nseg = 3;
        b.act = wb.z; b.lda = rtot; b.M = M; b.err = wb.err; b.part = wb.part;
        b.S = q.S; b.Hq = q.Hq; b.Hkv = q.Hkv; b.D = q.D; b.rope_theta = q.theta; b.L_max = q.L_max;
        b.rope_base = q.theta > 0.f ? std::pow((double)q.theta, -2.0 / (double)q.D) : 0.0;
        b.seqlens = seqlens; b.k_cache = (bf16_t*)kc; b.v_cache = (bf16_t*)vc;
        b.k_out = (bf16_t*)k_out; b.v_out = (bf16_t*)v_out;
        RowdotSeg& s0 = b.seg[0];
        s0.W = Vq; s0.ldw = q.rq; s0.N = q.Hq * q.D; s0.K = q.rq; s0.act_off = 0; s0.kind = SEG_Q;
        s0.out = q_out; s0.ldo = (int64_t)q.Hq * q.D;
        RowdotSeg& s1 = b.seg[1];
        s1.W = Vk; s1.ldw = q.rk; s1.N = q.Hkv * q.D; s1.K = q.rk; s1.act_off = q.rq; s1.kind = SEG_K;
        RowdotSeg& s2 = b.seg[2];
        s2.W = Vv; s2.ldw = q.rv; s2.N = q.Hkv * q.D; s2.K = q.rv; s2.act_off = q.rq + q.rk; s2.kind = SEG_V;
        return launch_rowdot(b, EPI_QKV, FSVD_BF16, st);
    }
    const bf16_t* a_in = (const bf16_t*)x;
    const float* rstd = nullptr;
    if (norm) {  // rstd per row; the weighted copy x.w only when the weight is not folded into A
        TRY(launch_rms_prep((const bf16_t*)x, (const bf16_t*)norm_w, q.eps, M, q.d, norm_w ? (bf16_t*)wb.xn : nullptr,
                            wb.rstd, st));
        if (norm_w) a_in = (const bf16_t*)wb.xn;
        rstd = wb.rstd;
    }
    GemmArgs g{};
    g.A = a_in; g.lda = q.d; g.Bm = (const bf16_t*)A; g.ldb = q.d;
    g.M = M; g.N = rtot; g.K = q.d; g.C = (bf16_t*)wb.z; g.ldc = rtot; g.rstd = rstd; g.err = wb.err;
    TRY(launch_gemm(g, GEPI_STORE, st));
    // phase 2: the three branches (different ranks and output widths) as column segments of one
    // grouped launch, RoPE + cache append in the epilogue
    const void* Vs[3] = {Vq, Vk, Vv};
    const int rs[3] = {q.rq, q.rk, q.rv};
    const int offs[3] = {0, q.rq, q.rq + q.rk};
    const int Ns[3] = {q.Hq * q.D, q.Hkv * q.D, q.Hkv * q.D};
    GemmArgs h{};
    h.A = (const bf16_t*)wb.z; h.lda = rtot;
    h.nseg = 3;
    for (int i = 0; i < 3; ++i) h.segs[i] = GemmArgs::Seg{(const bf16_t*)Vs[i], (int64_t)rs[i], rs[i], offs[i], Ns[i]};
    h.Bm = (const bf16_t*)Vq; h.ldb = q.rq; h.K = std::max(q.rq, std::max(q.rk, q.rv));
    h.M = M; h.N = Ns[0] + Ns[1] + Ns[2];
    h.S = q.S; h.Hq = q.Hq; h.Hkv = q.Hkv; h.D = q.D; h.rope_theta = q.theta; h.L_max = q.L_max;
    h.seqlens = seqlens; h.row_off = q.row_off;
    h.q_out = (bf16_t*)q_out; h.k_cache = (bf16_t*)kc; h.v_cache = (bf16_t*)vc;
    h.k_out = (bf16_t*)k_out; h.v_out = (bf16_t*)v_out;
    h.err = wb.err;
    return launch_gemm(h, GEPI_QKV, st);
}

struct MlpDims {
    int M, d, rg, ru, d_ff, rd;
    float eps;
    fsvd_act_t act;
};
struct MlpBufs {
    void* z_gu;   // [M, rg+ru]
    void* t;      // [M, d_ff] (not used by the fused path)
    void* z_d;    // [M, rd]
    void* xn;     // MFMA path: [M, d]
    float* rstd;  // MFMA path: [M]
    int* err;
    float* part;  // row-dot split-reduction partials, or NULL
    const MlpFusedPlan* fused;  // MFMA path: t kept on chip (mlp_fused.hip), or NULL
    void* fpart;  // fused path: per-slice partial z_d (fused->part_bytes)
};

size_t mlp_scratch(int64_t M, int64_t d, int64_t rgu, int64_t d_ff, int64_t rd) {
    size_t s = align256((size_t)M * rgu * 2) + align256((size_t)M * d_ff * 2) + align256((size_t)M * rd * 2) +
               align256(rowdot_part_bytes(M, FSVD_BF16));
    if (M > kRowdotMaxM) s += align256((size_t)M * d * 2) + align256((size_t)M * 4);
    return s;
}

fsvd_status_t enqueue_mlp(const MlpDims& p, const void* x, bool norm, const void* norm_w, const void* A_gu, const void* Vg,
                          const void* Vu, const void* Ud, const void* Vd, const void* residual, void* y,
                          const MlpBufs& wb, int32_t* adv, int advB, int advn, hipStream_t st) {
    const int rgu = p.rg + p.ru;
    if (p.M <= kRowdotMaxM) {
        RowdotArgs a{};
        a.nseg = 1;
        a.act = x; a.lda = p.d; a.M = p.M; a.err = wb.err;
        a.norm = norm; a.norm_w = (const bf16_t*)norm_w; a.norm_eps = p.eps; a.norm_K = p.d;
        a.seg[0].W = A_gu; a.seg[0].ldw = p.d; a.seg[0].N = rgu; a.seg[0].K = p.d; a.seg[0].out = wb.z_gu; a.seg[0].ldo = rgu;
        a.part = wb.part;
        TRY(launch_rowdot(a, EPI_Z, FSVD_BF16, st));
        RowdotArgs b{};
        b.nseg = 1;
        b.act = wb.z_gu; b.lda = rgu; b.M = p.M; b.err = wb.err; b.part = wb.part;
        if (p.act == FSVD_ACT_SWIGLU) {
            b.seg[0].W = Vg; b.seg[0].ldw = p.rg; b.seg[0].K = p.rg; b.seg[0].act_off = 0;
            b.seg[0].W2 = Vu; b.seg[0].ldw2 = p.ru; b.seg[0].K2 = p.ru; b.seg[0].act_off2 = p.rg;
            b.seg[0].N = p.d_ff; b.seg[0].out = wb.t; b.seg[0].ldo = p.d_ff;
            TRY(launch_rowdot(b, EPI_SWIGLU, FSVD_BF16, st));
        } else {
            b.seg[0].W = Vu; b.seg[0].ldw = p.ru; b.seg[0].K = p.ru; b.seg[0].act_off = p.rg;
            b.seg[0].N = p.d_ff; b.seg[0].out = wb.t; b.seg[0].ldo = p.d_ff;
            TRY(launch_rowdot(b, EPI_GELU, FSVD_BF16, st));
        }
        LinearBufs lb{wb.z_d, wb.err, wb.part};
        return enqueue_linear(wb.t, p.M, p.d_ff, p.d_ff, Ud, p.rd, p.d_ff, Vd, p.d, p.rd, nullptr, residual, p.d, y,
                              p.d, FSVD_BF16, lb, adv, advB, advn, st);
    }
    const bf16_t* a_in = (const bf16_t*)x;
    const float* rstd = nullptr;
    if (norm) {
        TRY(launch_rms_prep((const bf16_t*)x, (const bf16_t*)norm_w, p.eps, p.M, p.d, norm_w ? (bf16_t*)wb.xn : nullptr,
                            wb.rstd, st));
        if (norm_w) a_in = (const bf16_t*)wb.xn;
        rstd = wb.rstd;
    }
    GemmArgs g{};
    g.A = a_in; g.lda = p.d; g.Bm = (const bf16_t*)A_gu; g.ldb = p.d;
    g.M = p.M; g.N = rgu; g.K = p.d; g.C = (bf16_t*)wb.z_gu; g.ldc = rgu; g.rstd = rstd; g.err = wb.err;
    TRY(launch_gemm(g, GEPI_STORE, st));
    if (wb.fused) {
        // up (gate) phase 2, activation and down phase 1 in one kernel: t stays on chip
        MlpFusedArgs f{};
        f.z = (const bf16_t*)wb.z_gu; f.ldz = rgu;
        f.rg = p.act == FSVD_ACT_SWIGLU ? p.rg : 0; f.ru = p.ru; f.rd = p.rd; f.M = p.M; f.d_ff = p.d_ff;
        f.Vg = (const bf16_t*)Vg; f.Vu = (const bf16_t*)Vu; f.Ud = (const bf16_t*)Ud; f.ldu = p.d_ff;
        f.part = (bf16_t*)wb.fpart; f.z_d = (bf16_t*)wb.z_d;
        TRY(launch_mlp_fused(f, *wb.fused, st));
        GemmArgs dn{};
        dn.A = (const bf16_t*)wb.z_d; dn.lda = p.rd; dn.Bm = (const bf16_t*)Vd; dn.ldb = p.rd;
        dn.M = p.M; dn.N = p.d; dn.K = p.rd; dn.C = (bf16_t*)y; dn.ldc = p.d;
        dn.residual = (const bf16_t*)residual; dn.ldr = p.d; dn.err = wb.err;
        TRY(launch_gemm(dn, GEPI_LINEAR, st));
        if (adv) return launch_seqlens_advance(adv, advB, advn, st);
        return FSVD_OK;
    }
    GemmArgs h{};
    h.A = (const bf16_t*)wb.z_gu; h.lda = rgu;
    h.M = p.M; h.N = p.d_ff; h.C = (bf16_t*)wb.t; h.ldc = p.d_ff; h.err = wb.err;
    if (p.act == FSVD_ACT_SWIGLU) {
        h.Bm = (const bf16_t*)Vg; h.ldb = p.rg; h.K = p.rg; h.a_col_off = 0;
        h.B2 = (const bf16_t*)Vu; h.ldb2 = p.ru; h.a_col_off2 = p.rg; h.K2 = p.ru;
        TRY(launch_gemm(h, GEPI_SWIGLU, st));
    } else {
        h.Bm = (const bf16_t*)Vu; h.ldb = p.ru; h.K = p.ru; h.a_col_off = p.rg;
        TRY(launch_gemm(h, GEPI_GELU, st));
    }
    LinearBufs lb{wb.z_d, wb.err, nullptr};
    return enqueue_linear(wb.t, p.M, p.d_ff, p.d_ff, Ud, p.rd, p.d_ff, Vd, p.d, p.rd, nullptr, residual, p.d, y, p.d,
                          FSVD_BF16, lb, adv, advB, advn, st);
}

// ws: the workspace (its header holds the device error word and the decode partition counters)
fsvd_status_t enqueue_attn(const void* q, const void* kc, const void* vc, int64_t L_max, const int32_t* seqlens, int B,
                           int Sq, int Hq, int Hkv, int D, float scale, int causal, void* out, float* part, int nsplit,
                           void* ws, hipStream_t st) {
    int* err = (int*)ws;
    unsigned* cnt = (ws && (int64_t)B * Hkv <= kWsCounters) ? (unsigned*)((char*)ws + kWsCounterOff) : nullptr;
    AttnArgs a{};
    a.q = (const bf16_t*)q; a.kc = (const bf16_t*)kc; a.vc = (const bf16_t*)vc; a.seqlens = seqlens;
    a.out = (bf16_t*)out; a.B = B; a.Sq = Sq; a.Hq = Hq; a.Hkv = Hkv; a.D = D; a.L_max = L_max;
    a.scale = scale > 0.f ? scale : 1.0f / sqrtf((float)D);
    a.causal = causal; a.nsplit = nsplit; a.part = part; a.cnt = cnt; a.err = err;
    if (Sq == 1) return launch_attn_decode(a, st);
    return launch_attn_prefill(a, st);
}

fsvd_status_t check_attn_shape(int64_t Hq, int64_t Hkv, int64_t D) {
    if (Hq % Hkv) return fail(FSVD_ERR_INVALID_ARG, "Hq (%lld) must be a multiple of Hkv (%lld)", (long long)Hq, (long long)Hkv);
    const int64_t G = Hq / Hkv;
    if (G != 1 && G != 2 && G != 4 && G != 8) return fail(FSVD_ERR_UNSUPPORTED, "GQA group size %lld not in {1,2,4,8}", (long long)G);
    if (D != 64 && D != 128) return fail(FSVD_ERR_UNSUPPORTED, "head dim %lld not in {64,128}", (long long)D);
    return FSVD_OK;
}

// ------------------------------------------------------------------ decoder layer

struct LayerPlan {
    size_t bytes;
    int64_t chunk;   // token rows per pass through the layer (prefill); M at decode sizes
    void *q, *o, *h;
    QkvBufs qb;
    float* attn_part;
    int nsplit;
    void* z_o;
    MlpBufs mb;
    float* part;
};

constexpr int64_t kPrefillChunk = 8192;   // default rows per prefill pass
constexpr int64_t kMinPrefillChunk = 256;

// Rows per prefill pass: the call's M = B * S tokens run in ceil(M / limit) passes of nearly equal
// size (each at least limit / 2 rows, so never a row-dot-sized pass).
int64_t prefill_chunk_rows(const fsvd_decoder_layer_desc* d) {
    const int64_t M = d->B * d->S;
    const int64_t lim = d->prefill_chunk > 0 ? d->prefill_chunk : kPrefillChunk;
    const int64_t n = (M + lim - 1) / lim;
    return (M + n - 1) / n;
}

LayerPlan plan_layer(const fsvd_decoder_layer_desc* d, void* ws) {
    LayerPlan p{};
    Carve c(ws);
    const int64_t M = d->B * d->S;
    const int64_t qd = d->Hq * d->D;
    if (M > kRowdotMaxM) {
        // Prefill: one pass per chunk of Mc token rows; the workspace holds one chunk, so it does
        // not grow with the sequence.  Buffers share two slots by liveness (each one is dead
        // before the next one in its slot is written):
        //   slot A: z_qkv (Q/K/V phase 1 -> 2), o (attention -> O phase 1), z_gu (gate|up
        //           phase 1 -> 2), z_d (down phase 1 -> 2)
        //   slot B: xn (RMSNorm -> Q/K/V phase 1), q (phase 2 -> attention), z_o (O phase 1 -> 2),
        //           xn (RMSNorm -> gate|up phase 1), t (gate|up phase 2 -> down phase 1)
        // plus h (O output, MLP input and residual; live to the end) and the per-row rstd.
        const int64_t Mc = prefill_chunk_rows(d);
        p.chunk = Mc;
        const int64_t rtot = d->r_q + d->r_k + d->r_v, rgu = d->r_g + d->r_u;
        const int64_t wa = std::max(std::max(rtot, qd), std::max(rgu, d->r_d));
        const int64_t wb = std::max(std::max(qd, d->r_o), std::max(d->d_ff, d->d));
        p.h = c.take((size_t)Mc * d->d * 2);
        void* sa = c.take((size_t)Mc * wa * 2);
        void* sb = c.take((size_t)Mc * wb * 2);
        float* rstd = (float*)c.take((size_t)Mc * 4);
        p.qb.z = sa; p.qb.xn = sb; p.qb.rstd = rstd;
        p.q = sb;
        p.o = sa;
        p.z_o = sb;
        p.mb.xn = sb; p.mb.rstd = rstd; p.mb.z_gu = sa; p.mb.t = sb; p.mb.z_d = sa;
        int* err = ws ? (int*)ws : nullptr;
        p.qb.err = err;
        p.mb.err = err;
        p.bytes = c.off;
        return p;
    }
    p.chunk = M;
    p.q = c.take((size_t)M * qd * 2);
    p.o = c.take((size_t)M * qd * 2);
    p.h = c.take((size_t)M * d->d * 2);
    const int64_t rtot = d->r_q + d->r_k + d->r_v;
    p.qb.z = c.take((size_t)M * rtot * 2);
    p.nsplit = attn_default_splits((int)d->B, (int)d->Hkv, d->L_max);
    p.attn_part = (float*)c.take(attn_decode_ws_bytes((int)d->B, (int)d->Hq, (int)d->D, p.nsplit));
    p.z_o = c.take((size_t)M * d->r_o * 2);
    p.mb.z_gu = c.take((size_t)M * (d->r_g + d->r_u) * 2);
    p.mb.t = c.take((size_t)M * d->d_ff * 2);
    p.mb.z_d = c.take((size_t)M * d->r_d * 2);
    if (rowdot_part_bytes(M, FSVD_BF16)) {  // one partials slice, used by one launch at a time
        p.part = (float*)c.take(rowdot_part_bytes(M, FSVD_BF16));
        p.qb.part = p.part;
        p.mb.part = p.part;
    }
    int* err = ws ? (int*)ws : nullptr;
    p.qb.err = err;
    p.mb.err = err;
    p.bytes = c.off;
    return p;
}

fsvd_status_t validate_layer(const fsvd_decoder_layer_desc* d) {
    if (!d) return fail(FSVD_ERR_INVALID_ARG, "descriptor is NULL");
    const fsvd_dtype_t t = FSVD_BF16;
    TRY(need_dim(d->B, "B")); TRY(need_dim(d->S, "S")); TRY(need_dim(d->d, "d"));
    TRY(need_dim(d->Hq, "Hq")); TRY(need_dim(d->Hkv, "Hkv")); TRY(need_dim(d->D, "D"));
    TRY(need_dim(d->d_ff, "d_ff")); TRY(need_dim(d->L_max, "L_max"));
    TRY(check_attn_shape(d->Hq, d->Hkv, d->D));
    const int64_t ranks[7] = {d->r_q, d->r_k, d->r_v, d->r_o, d->r_g, d->r_u, d->r_d};
    const char* rn[7] = {"r_q", "r_k", "r_v", "r_o", "r_g", "r_u", "r_d"};
    for (int i = 0; i < 7; ++i) {
        TRY(need_dim(ranks[i], rn[i]));
        TRY(need_vec(ranks[i], t, rn[i]));
    }
    TRY(need_vec(d->d, t, "d")); TRY(need_vec(d->d_ff, t, "d_ff"));
    const int64_t qd = d->Hq * d->D, kd = d->Hkv * d->D;
    TRY(need_rank(d->r_q, d->d, qd, "r_q")); TRY(need_rank(d->r_k, d->d, kd, "r_k"));
    TRY(need_rank(d->r_v, d->d, kd, "r_v")); TRY(need_rank(d->r_o, qd, d->d, "r_o"));
    TRY(need_rank(d->r_g, d->d, d->d_ff, "r_g")); TRY(need_rank(d->r_u, d->d, d->d_ff, "r_u"));
    TRY(need_rank(d->r_d, d->d_ff, d->d, "r_d"));
    const void* ptrs[] = {d->x, d->y, d->A_qkv, d->Vt_q, d->Vt_k, d->Vt_v, d->Ut_o, d->Vt_o, d->A_gu, d->Vt_g, d->Vt_u,
                          d->Ut_d, d->Vt_d, d->k_cache, d->v_cache, d->ws};
    const char* pn[] = {"x", "y", "A_qkv", "Vt_q", "Vt_k", "Vt_v", "Ut_o", "Vt_o", "A_gu", "Vt_g", "Vt_u",
                        "Ut_d", "Vt_d", "k_cache", "v_cache", "ws"};
    for (size_t i = 0; i < sizeof(ptrs) / sizeof(ptrs[0]); ++i) TRY(need_ptr(ptrs[i], pn[i]));
    TRY(opt_ptr(d->attn_norm_w, "attn_norm_w")); TRY(opt_ptr(d->mlp_norm_w, "mlp_norm_w"));
    if (d->flags & ~FSVD_LAYER_NORM_FOLDED) return fail(FSVD_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)d->flags);
    if (!d->cache_seqlens) return fail(FSVD_ERR_INVALID_ARG, "cache_seqlens is NULL");
    if (d->x == d->y) return fail(FSVD_ERR_INVALID_ARG, "y must not alias x");
    if (d->S > d->L_max) return fail(FSVD_ERR_INVALID_ARG, "S (%lld) exceeds L_max", (long long)d->S);
    if (d->prefill_chunk != 0 && (d->prefill_chunk < kMinPrefillChunk || d->prefill_chunk > ((int64_t)1 << 30)))
        return fail(FSVD_ERR_INVALID_ARG, "prefill_chunk = %lld: 0 (default) or %lld .. 2^30 rows",
                    (long long)d->prefill_chunk, (long long)kMinPrefillChunk);
    const LayerPlan p = plan_layer(d, nullptr);
    if (d->ws_bytes < p.bytes)
        return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", d->ws_bytes, p.bytes);
    return FSVD_OK;
}

// Attention of token rows [r0, r0 + rows) of a prefill call (queries at q, outputs at out, both
// [rows, Hq, D]) over the dense cache: one launch per run of whole sequences, one per partial
// sequence, each query at position cache_seqlens[b] + s.
fsvd_status_t enqueue_attn_rows(const fsvd_decoder_layer_desc* d, const bf16_t* q, bf16_t* out, int64_t r0,
                                int64_t rows, int* err, hipStream_t st) {
    const int64_t S = d->S, qd = d->Hq * d->D, kv_seq = d->L_max * d->Hkv * d->D;
    int64_t r = r0;
    const int64_t r1 = r0 + rows;
    while (r < r1) {
        const int64_t b = r / S, s0 = r - b * S;
        int64_t nseq = 1, len;
        if (s0 == 0 && r + S <= r1) {  // whole sequences b .. b + nseq - 1
            nseq = (r1 - r) / S;
            len = S;
        } else {
            len = std::min(S - s0, r1 - r);
        }
        AttnArgs a{};
        a.q = q + (r - r0) * qd; a.out = out + (r - r0) * qd;
        a.kc = (const bf16_t*)d->k_cache + b * kv_seq; a.vc = (const bf16_t*)d->v_cache + b * kv_seq;
        a.seqlens = d->cache_seqlens + b;
        a.B = (int)nseq; a.Sq = (int)len; a.Hq = (int)d->Hq; a.Hkv = (int)d->Hkv; a.D = (int)d->D;
        a.L_max = d->L_max; a.pos_off = (int)s0;
        a.scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / sqrtf((float)d->D);
        a.causal = 1; a.err = err;
        TRY(launch_attn_prefill(a, st));
        r += nseq * len;
    }
    return FSVD_OK;
}

fsvd_status_t enqueue_layer(const fsvd_decoder_layer_desc* d, hipStream_t st) {
    const LayerPlan p = plan_layer(d, d->ws);
    const int B = (int)d->B, S = (int)d->S, M = B * S;
    QkvDims qd{B, S, (int)d->d, (int)d->r_q, (int)d->r_k, (int)d->r_v, (int)d->Hq, (int)d->Hkv, (int)d->D,
               d->L_max, d->norm_eps, d->rope_theta, 0, 0};
    const bool folded = (d->flags & FSVD_LAYER_NORM_FOLDED) != 0;
    if (M > kRowdotMaxM) {
        // prefill: passes of p.chunk token rows; the lengths advance once, after the last pass
        const int qdim = (int)(d->Hq * d->D);
        const int64_t nchunk = (M + p.chunk - 1) / p.chunk;
        for (int64_t c = 0; c < nchunk; ++c) {
            const int64_t r0 = c * M / nchunk, r1 = (c + 1) * M / nchunk, mc = r1 - r0;
            const bf16_t* xc = (const bf16_t*)d->x + r0 * d->d;
            bf16_t* yc = (bf16_t*)d->y + r0 * d->d;
            QkvDims qc = qd;
            qc.rows = (int)mc;
            qc.row_off = (int)r0;
            TRY(enqueue_qkv(qc, xc, folded || d->attn_norm_w != nullptr, folded ? nullptr : d->attn_norm_w, d->A_qkv,
                            d->Vt_q, d->Vt_k, d->Vt_v, p.q, d->k_cache, d->v_cache, d->cache_seqlens, nullptr,
                            nullptr, p.qb, st));
            TRY(enqueue_attn_rows(d, (const bf16_t*)p.q, (bf16_t*)p.o, r0, mc, p.qb.err, st));
            LinearBufs lb{p.z_o, p.qb.err, nullptr};
            TRY(enqueue_linear(p.o, (int)mc, qdim, qdim, d->Ut_o, (int)d->r_o, qdim, d->Vt_o, (int)d->d, d->r_o,
                               nullptr, xc, d->d, p.h, d->d, FSVD_BF16, lb, nullptr, 0, 0, st));
            MlpDims md{(int)mc, (int)d->d, (int)d->r_g, (int)d->r_u, (int)d->d_ff, (int)d->r_d, d->norm_eps,
                       FSVD_ACT_SWIGLU};
            const bool last = c + 1 == nchunk;
            TRY(enqueue_mlp(md, p.h, folded || d->mlp_norm_w != nullptr, folded ? nullptr : d->mlp_norm_w, d->A_gu,
                            d->Vt_g, d->Vt_u, d->Ut_d, d->Vt_d, p.h, yc, p.mb,
                            (last && d->advance_seqlens) ? d->cache_seqlens : nullptr, B, S, st));
        }
        return FSVD_OK;
    }
    TRY(enqueue_qkv(qd, d->x, folded || d->attn_norm_w != nullptr, folded ? nullptr : d->attn_norm_w, d->A_qkv, d->Vt_q, d->Vt_k, d->Vt_v, p.q, d->k_cache, d->v_cache,
                    d->cache_seqlens, nullptr, nullptr, p.qb, st));
    TRY(enqueue_attn(p.q, d->k_cache, d->v_cache, d->L_max, d->cache_seqlens, B, S, (int)d->Hq, (int)d->Hkv,
                     (int)d->D, d->softmax_scale, 1, p.o, p.attn_part, p.nsplit, d->ws, st));
    const int qdim = (int)(d->Hq * d->D);
    LinearBufs lb{p.z_o, p.qb.err, p.part};
    TRY(enqueue_linear(p.o, M, qdim, qdim, d->Ut_o, (int)d->r_o, qdim, d->Vt_o, (int)d->d, d->r_o, nullptr, d->x, d->d,
                       p.h, d->d, FSVD_BF16, lb, nullptr, 0, 0, st));
    MlpDims md{M, (int)d->d, (int)d->r_g, (int)d->r_u, (int)d->d_ff, (int)d->r_d, d->norm_eps, FSVD_ACT_SWIGLU};
    return enqueue_mlp(md, p.h, folded || d->mlp_norm_w != nullptr, folded ? nullptr : d->mlp_norm_w, d->A_gu, d->Vt_g, d->Vt_u, d->Ut_d, d->Vt_d, p.h, d->y, p.mb,
                       d->advance_seqlens ? d->cache_seqlens : nullptr, B, S, st);
}

// ------------------------------------------------------------------ graphs

std::mutex g_graph_mu;
std::set<void*> g_live_graphs;
hipStream_t g_capture_stream[64] = {};

}  // namespace
}  // namespace fsvd

struct fsvd_graph {
    hipGraph_t graph;
    hipGraphExec_t exec;
    int device;
};

using namespace fsvd;

namespace {
fsvd_status_t prepack_impl(void* dst, int64_t ld_dst, int64_t cols_pad, const fsvd_pack_item* items, int n_items,
                           const void* col_scale, fsvd_dtype_t dtype, fsvd_stream_t stream);
}  // namespace

extern "C" {

int fsvd_abi_version(void) { return FSVD_ABI_VERSION; }

const char* fsvd_status_str(fsvd_status_t s) {
    switch (s) {
        case FSVD_OK: return "ok";
        case FSVD_ERR_INVALID_ARG: return "invalid argument";
        case FSVD_ERR_UNSUPPORTED: return "unsupported";
        case FSVD_ERR_WORKSPACE: return "workspace too small";
        case FSVD_ERR_HIP: return "HIP runtime error";
        case FSVD_ERR_CAPTURE: return "graph capture/replay error";
        case FSVD_ERR_DEVICE: return "device error word set";
    }
    return "unknown status";
}

const char* fsvd_last_error(void) { return g_err; }


fsvd_status_t fsvd_prepack(void* dst, int64_t ld_dst, int64_t cols_pad, const fsvd_pack_item* items, int n_items,
                           fsvd_dtype_t dtype, fsvd_stream_t stream) {
    return prepack_impl(dst, ld_dst, cols_pad, items, n_items, nullptr, dtype, stream);
}

fsvd_status_t fsvd_prepack_colscale(void* dst, int64_t ld_dst, int64_t cols_pad, const fsvd_pack_item* items,
                                    int n_items, const void* col_scale, fsvd_dtype_t dtype, fsvd_stream_t stream) {
    TRY(need_ptr(col_scale, "col_scale"));
    return prepack_impl(dst, ld_dst, cols_pad, items, n_items, col_scale, dtype, stream);
}

}  // extern "C"

namespace {
fsvd_status_t prepack_impl(void* dst, int64_t ld_dst, int64_t cols_pad, const fsvd_pack_item* items, int n_items,
                           const void* col_scale, fsvd_dtype_t dtype, fsvd_stream_t stream) {
    TRY(need_dtype(dtype, true));
    if (!dst) return fail(FSVD_ERR_INVALID_ARG, "dst is NULL");
    if (!items || n_items <= 0) return fail(FSVD_ERR_INVALID_ARG, "no items");
    TRY(need_dim(cols_pad, "cols_pad"));
    if (ld_dst < cols_pad) return fail(FSVD_ERR_INVALID_ARG, "ld_dst < cols_pad");
    for (int i = 0; i < n_items; ++i) {
        const fsvd_pack_item& it = items[i];
        if (!it.src) return fail(FSVD_ERR_INVALID_ARG, "item %d src is NULL", i);
        if (it.rows <= 0 || it.cols <= 0 || it.cols > cols_pad || it.rows_pad < it.rows || it.ld_src < it.cols)
            return fail(FSVD_ERR_INVALID_ARG, "item %d has inconsistent extents", i);
    }
    int64_t row = 0;
    for (int i = 0; i < n_items; ++i) {
        const fsvd_pack_item& it = items[i];
        TRY(launch_prepack(dst, ld_dst, cols_pad, row, it.src, it.rows, it.cols, it.ld_src, it.rows_pad, esize(dtype),
                           col_scale, (hipStream_t)stream));
        row += it.rows_pad;
    }
    return FSVD_OK;
}
}  // namespace

extern "C" {

size_t fsvd_lowrank_linear_ws(int64_t M, int64_t K, int64_t r, int64_t N, fsvd_dtype_t dtype) {
    (void)K; (void)N;
    return kWsHeader + align256((size_t)M * r * esize(dtype)) + align256(rowdot_part_bytes(M, dtype));
}

}  // extern "C"

namespace {

// every argument of a low-rank linear call but the workspace
fsvd_status_t validate_linear(const void* x, int64_t M, int64_t K, int64_t ldx, const void* Ut, int64_t r, int64_t ldu,
                              const void* Vt, int64_t N, int64_t ldv, const void* bias, const void* residual,
                              int64_t ldr, void* y, int64_t ldy, fsvd_dtype_t dtype) {
    TRY(need_dtype(dtype, true));
    TRY(need_dim(M, "M")); TRY(need_dim(K, "K")); TRY(need_dim(r, "r")); TRY(need_dim(N, "N"));
    TRY(need_vec(K, dtype, "K")); TRY(need_vec(r, dtype, "r")); TRY(need_vec(N, dtype, "N"));
    TRY(need_rank(r, K, N, "r"));
    TRY(need_ptr(x, "x")); TRY(need_ptr(Ut, "Ut")); TRY(need_ptr(Vt, "Vt")); TRY(need_ptr(y, "y"));
    TRY(opt_ptr(bias, "bias")); TRY(opt_ptr(residual, "residual"));
    TRY(need_ld(ldx, K, dtype, "ldx")); TRY(need_ld(ldu, K, dtype, "ldu")); TRY(need_ld(ldv, r, dtype, "ldv"));
    TRY(need_ld(ldy, N, dtype, "ldy"));
    if (residual) TRY(need_ld(ldr, N, dtype, "ldr"));
    return FSVD_OK;
}

// carves (z, partials) out of a validated workspace and enqueues both phases
fsvd_status_t run_linear(const void* x, int64_t M, int64_t K, int64_t ldx, const void* Ut, int64_t r, int64_t ldu,
                         const void* Vt, int64_t N, int64_t ldv, const void* bias, const void* residual, int64_t ldr,
                         void* y, int64_t ldy, fsvd_dtype_t dtype, void* ws, hipStream_t st) {
    Carve c(ws);
    void* z = c.take((size_t)M * r * esize(dtype));
    float* part = rowdot_part_bytes(M, dtype) ? (float*)c.take(rowdot_part_bytes(M, dtype)) : nullptr;
    LinearBufs lb{z, (int*)ws, part};
    return enqueue_linear(x, (int)M, (int)K, ldx, Ut, (int)r, ldu, Vt, (int)N, ldv, bias, residual, ldr, y, ldy, dtype,
                          lb, nullptr, 0, 0, st);
}

// Scratch of the allocation-free linear: one copy per GPU, resident until the process ends.  In
// host code `scratch` only names the symbol; its device address on each GPU comes from
// hipGetSymbolAddress (resolved once per device, with that device current) and is what the
// kernels receive.
static __device__ __align__(256) unsigned char scratch[FSVD_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

fsvd_status_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FSVD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(FSVD_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FSVD_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FSVD_OK;
}

}  // namespace

extern "C" {

fsvd_status_t fsvd_lowrank_linear(const void* x, int64_t M, int64_t K, int64_t ldx, const void* Ut, int64_t r,
                                  int64_t ldu, const void* Vt, int64_t N, int64_t ldv, const void* bias,
                                  const void* residual, int64_t ldr, void* y, int64_t ldy, fsvd_dtype_t dtype, void* ws,
                                  size_t ws_bytes, fsvd_stream_t stream) {
    TRY(validate_linear(x, M, K, ldx, Ut, r, ldu, Vt, N, ldv, bias, residual, ldr, y, ldy, dtype));
    TRY(need_ptr(ws, "ws"));
    const size_t need = fsvd_lowrank_linear_ws(M, K, r, N, dtype);
    if (ws_bytes < need) return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    return run_linear(x, M, K, ldx, Ut, r, ldu, Vt, N, ldv, bias, residual, ldr, y, ldy, dtype, ws, (hipStream_t)stream);
}

fsvd_status_t fsvd_dense_linear(const void* x, int64_t M, int64_t K, int64_t ldx, const void* W, int64_t N,
                                int64_t ldw, const void* bias, const void* residual, int64_t ldr, void* y,
                                int64_t ldy, fsvd_dtype_t dtype, fsvd_stream_t stream) {
    TRY(need_dtype(dtype, true));
    TRY(need_dim(M, "M")); TRY(need_dim(K, "K")); TRY(need_dim(N, "N"));
    TRY(need_vec(K, dtype, "K")); TRY(need_vec(N, dtype, "N"));
    TRY(need_ptr(x, "x")); TRY(need_ptr(W, "W")); TRY(need_ptr(y, "y"));
    TRY(opt_ptr(bias, "bias")); TRY(opt_ptr(residual, "residual"));
    TRY(need_ld(ldx, K, dtype, "ldx")); TRY(need_ld(ldw, K, dtype, "ldw")); TRY(need_ld(ldy, N, dtype, "ldy"));
    if (residual) TRY(need_ld(ldr, N, dtype, "ldr"));
    const hipStream_t st = (hipStream_t)stream;
    if (M <= kRowdotMaxM) {
        RowdotArgs b{};  // no error word: the reduction is not split
        b.nseg = 1;
        b.act = x; b.lda = ldx; b.M = (int)M;
        b.seg[0].W = W; b.seg[0].ldw = ldw; b.seg[0].N = (int)N; b.seg[0].K = (int)K; b.seg[0].out = y;
        b.seg[0].ldo = ldy;
        b.bias = bias; b.residual = residual; b.ldr = ldr;
        return launch_rowdot(b, EPI_LINEAR, dtype, st);
    }
    if (dtype != FSVD_BF16) return fail(FSVD_ERR_UNSUPPORTED, "the MFMA path (M > %d) is bf16 only", kRowdotMaxM);
    GemmArgs h{};
    h.A = (const bf16_t*)x; h.lda = ldx; h.Bm = (const bf16_t*)W; h.ldb = ldw;
    h.M = (int)M; h.N = (int)N; h.K = (int)K; h.C = (bf16_t*)y; h.ldc = ldy;
    h.bias = (const bf16_t*)bias; h.residual = (const bf16_t*)residual; h.ldr = ldr;
    return launch_gemm(h, GEPI_LINEAR, st);
}

fsvd_status_t fsvd_lowrank_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx, const void* Ut, int64_t r,
                                          int64_t ldu, const void* Vt, int64_t N, int64_t ldv, const void* bias,
                                          const void* residual, int64_t ldr, void* y, int64_t ldy, fsvd_dtype_t dtype,
                                          fsvd_stream_t stream) {
    TRY(validate_linear(x, M, K, ldx, Ut, r, ldu, Vt, N, ldv, bias, residual, ldr, y, ldy, dtype));
    const size_t need = fsvd_lowrank_linear_ws(M, K, r, N, dtype);
    if (need > (size_t)FSVD_NOALLOC_SCRATCH_BYTES)
        return fail(FSVD_ERR_WORKSPACE, "this call needs %zu bytes of scratch, above the %zu-byte static scratch", need,
                    (size_t)FSVD_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    TRY(scratch_on_current_device(&ws));
    return run_linear(x, M, K, ldx, Ut, r, ldu, Vt, N, ldv, bias, residual, ldr, y, ldy, dtype, ws, (hipStream_t)stream);
}

size_t fsvd_lowrank_qkv_ws(int64_t B, int64_t S, int64_t d, int64_t r_q, int64_t r_k, int64_t r_v, int64_t Hq,
                           int64_t Hkv, int64_t D) {
    (void)Hq; (void)Hkv; (void)D;
    return kWsHeader + qkv_scratch(B * S, d, r_q + r_k + r_v);
}

fsvd_status_t fsvd_lowrank_qkv(const void* x, int64_t B, int64_t S, int64_t d, const void* norm_w, float norm_eps,
                               const void* A_qkv, int64_t r_q, int64_t r_k, int64_t r_v, const void* Vt_q,
                               const void* Vt_k, const void* Vt_v, int64_t Hq, int64_t Hkv, int64_t D, float rope_theta,
                               void* q_out, void* k_cache, void* v_cache, int64_t L_max, const int32_t* cache_seqlens,
                               void* k_out, void* v_out, fsvd_dtype_t dtype, void* ws, size_t ws_bytes,
                               fsvd_stream_t stream) {
    TRY(need_dtype(dtype, false));
    TRY(need_dim(B, "B")); TRY(need_dim(S, "S")); TRY(need_dim(d, "d")); TRY(need_dim(Hq, "Hq"));
    TRY(need_dim(Hkv, "Hkv")); TRY(need_dim(D, "D")); TRY(need_dim(L_max, "L_max"));
    TRY(need_dim(r_q, "r_q")); TRY(need_dim(r_k, "r_k")); TRY(need_dim(r_v, "r_v"));
    TRY(need_vec(d, dtype, "d")); TRY(need_vec(r_q, dtype, "r_q")); TRY(need_vec(r_k, dtype, "r_k"));
    TRY(need_vec(r_v, dtype, "r_v"));
    if (D != 64 && D != 128) return fail(FSVD_ERR_UNSUPPORTED, "head dim %lld not in {64,128}", (long long)D);
    if (Hq % Hkv) return fail(FSVD_ERR_INVALID_ARG, "Hq must be a multiple of Hkv");
    TRY(need_rank(r_q, d, Hq * D, "r_q")); TRY(need_rank(r_k, d, Hkv * D, "r_k")); TRY(need_rank(r_v, d, Hkv * D, "r_v"));
    TRY(need_ptr(x, "x")); TRY(need_ptr(A_qkv, "A_qkv")); TRY(need_ptr(Vt_q, "Vt_q")); TRY(need_ptr(Vt_k, "Vt_k"));
    TRY(need_ptr(Vt_v, "Vt_v")); TRY(need_ptr(q_out, "q_out")); TRY(need_ptr(k_cache, "k_cache"));
    TRY(need_ptr(v_cache, "v_cache")); TRY(need_ptr(ws, "ws")); TRY(opt_ptr(norm_w, "norm_w"));
    if (!cache_seqlens) return fail(FSVD_ERR_INVALID_ARG, "cache_seqlens is NULL");
    const size_t need = fsvd_lowrank_qkv_ws(B, S, d, r_q, r_k, r_v, Hq, Hkv, D);
    if (ws_bytes < need) return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    Carve c(ws);
    const int64_t M = B * S;
    QkvBufs qb{};
    qb.z = c.take((size_t)M * (r_q + r_k + r_v) * 2);
    if (M > kRowdotMaxM) {
        qb.xn = c.take((size_t)M * d * 2);
        qb.rstd = (float*)c.take((size_t)M * 4);
    }
    if (rowdot_part_bytes(M, FSVD_BF16)) qb.part = (float*)c.take(rowdot_part_bytes(M, FSVD_BF16));
    qb.err = (int*)ws;
    QkvDims qd{(int)B, (int)S, (int)d, (int)r_q, (int)r_k, (int)r_v, (int)Hq, (int)Hkv, (int)D, L_max, norm_eps, rope_theta,
               0, 0};
    return enqueue_qkv(qd, x, norm_w != nullptr, norm_w, A_qkv, Vt_q, Vt_k, Vt_v, q_out, k_cache, v_cache, cache_seqlens, k_out, v_out, qb,
                       (hipStream_t)stream);
}

// The standalone MLP call at prefill sizes keeps t on chip whenever a fused kernel covers its
// ranks: its scratch is then z, the per-slice partial z_d and z_d instead of z, t and z_d.
bool mlp_call_fused(int64_t M, int64_t r_g, int64_t r_u, int64_t d_ff, int64_t r_d, MlpFusedPlan* plan) {
    return M > kRowdotMaxM && mlp_fused_plan(M, r_g, r_u, d_ff, r_d, plan);
}
size_t mlp_call_scratch(int64_t M, int64_t d, int64_t r_g, int64_t r_u, int64_t d_ff, int64_t r_d) {
    MlpFusedPlan plan{};
    if (!mlp_call_fused(M, r_g, r_u, d_ff, r_d, &plan)) return mlp_scratch(M, d, r_g + r_u, d_ff, r_d);
    return align256((size_t)M * (r_g + r_u) * 2) + align256(plan.part_bytes) + align256((size_t)M * r_d * 2) +
           align256((size_t)M * d * 2) + align256((size_t)M * 4);
}

size_t fsvd_lowrank_mlp_packed_ws(int64_t M, int64_t d, int64_t r_g, int64_t r_u, int64_t d_ff, int64_t r_d) {
    return kWsHeader + mlp_call_scratch(M, d, r_g, r_u, d_ff, r_d);
}

fsvd_status_t fsvd_lowrank_mlp_packed(const void* x, int64_t M, int64_t d, const void* norm_w, float norm_eps,
                                      fsvd_act_t act, const void* A_gu, int64_t r_g, int64_t r_u, const void* Vt_g,
                                      const void* Vt_u, int64_t d_ff, const void* Ut_d, const void* Vt_d, int64_t r_d,
                                      const void* residual, void* y, fsvd_dtype_t dtype, void* ws, size_t ws_bytes,
                                      fsvd_stream_t stream) {
    TRY(need_dtype(dtype, false));
    if (act != FSVD_ACT_SWIGLU && act != FSVD_ACT_GELU) return fail(FSVD_ERR_INVALID_ARG, "unknown activation %d", (int)act);
    TRY(need_dim(M, "M")); TRY(need_dim(d, "d")); TRY(need_dim(d_ff, "d_ff")); TRY(need_dim(r_u, "r_u"));
    TRY(need_dim(r_d, "r_d"));
    if (act == FSVD_ACT_SWIGLU) {
        TRY(need_dim(r_g, "r_g"));
        TRY(need_ptr(Vt_g, "Vt_g"));
    } else if (r_g != 0) {
        return fail(FSVD_ERR_INVALID_ARG, "GELU takes no gate: r_g must be 0");
    }
    TRY(need_vec(d, dtype, "d")); TRY(need_vec(d_ff, dtype, "d_ff")); TRY(need_vec(r_g, dtype, "r_g"));
    TRY(need_vec(r_u, dtype, "r_u")); TRY(need_vec(r_d, dtype, "r_d"));
    TRY(need_rank(r_g, d, d_ff, "r_g")); TRY(need_rank(r_u, d, d_ff, "r_u")); TRY(need_rank(r_d, d_ff, d, "r_d"));
    TRY(need_ptr(x, "x")); TRY(need_ptr(A_gu, "A_gu")); TRY(need_ptr(Vt_u, "Vt_u")); TRY(need_ptr(Ut_d, "Ut_d"));
    TRY(need_ptr(Vt_d, "Vt_d")); TRY(need_ptr(y, "y")); TRY(need_ptr(ws, "ws"));
    TRY(opt_ptr(norm_w, "norm_w")); TRY(opt_ptr(residual, "residual"));
    const size_t need = fsvd_lowrank_mlp_packed_ws(M, d, r_g, r_u, d_ff, r_d);
    if (ws_bytes < need) return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    Carve c(ws);
    MlpBufs mb{};
    MlpFusedPlan plan{};
    const bool fused = mlp_call_fused(M, r_g, r_u, d_ff, r_d, &plan);
    mb.z_gu = c.take((size_t)M * (r_g + r_u) * 2);
    if (fused) {
        mb.fused = &plan;
        if (plan.part_bytes) mb.fpart = c.take(plan.part_bytes);
    } else {
        mb.t = c.take((size_t)M * d_ff * 2);
    }
    mb.z_d = c.take((size_t)M * r_d * 2);
    if (M > kRowdotMaxM) {
        mb.xn = c.take((size_t)M * d * 2);
        mb.rstd = (float*)c.take((size_t)M * 4);
    }
    if (rowdot_part_bytes(M, FSVD_BF16)) mb.part = (float*)c.take(rowdot_part_bytes(M, FSVD_BF16));
    mb.err = (int*)ws;
    MlpDims md{(int)M, (int)d, (int)r_g, (int)r_u, (int)d_ff, (int)r_d, norm_eps, act};
    return enqueue_mlp(md, x, norm_w != nullptr, norm_w, A_gu, Vt_g, Vt_u, Ut_d, Vt_d, residual, y, mb, nullptr, 0, 0, (hipStream_t)stream);
}

size_t fsvd_decode_attn_dense_kv_ws(int64_t B, int64_t Sq, int64_t Hq, int64_t Hkv, int64_t D, int64_t L_max) {
    (void)Sq;
    if (Hkv <= 0) return kWsHeader;
    const int ns = attn_default_splits((int)B, (int)Hkv, L_max);
    return kWsHeader + align256(attn_decode_ws_bytes((int)B, (int)Hq, (int)D, ns));
}

fsvd_status_t fsvd_decode_attn_dense_kv(const void* q, const void* k_cache, const void* v_cache, int64_t L_max,
                                        const int32_t* cache_seqlens, int64_t B, int64_t Sq, int64_t Hq, int64_t Hkv,
                                        int64_t D, float softmax_scale, int causal, void* out, fsvd_dtype_t dtype,
                                        void* ws, size_t ws_bytes, fsvd_stream_t stream) {
    TRY(need_dtype(dtype, false));
    TRY(need_dim(B, "B")); TRY(need_dim(Sq, "Sq")); TRY(need_dim(Hq, "Hq")); TRY(need_dim(Hkv, "Hkv"));
    TRY(need_dim(D, "D")); TRY(need_dim(L_max, "L_max"));
    TRY(check_attn_shape(Hq, Hkv, D));
    TRY(need_ptr(q, "q")); TRY(need_ptr(k_cache, "k_cache")); TRY(need_ptr(v_cache, "v_cache"));
    TRY(need_ptr(out, "out")); TRY(need_ptr(ws, "ws"));
    if (!cache_seqlens) return fail(FSVD_ERR_INVALID_ARG, "cache_seqlens is NULL");
    if (softmax_scale < 0.f) return fail(FSVD_ERR_INVALID_ARG, "softmax_scale must be >= 0");
    const size_t need = fsvd_decode_attn_dense_kv_ws(B, Sq, Hq, Hkv, D, L_max);
    if (ws_bytes < need) return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    const int ns = attn_default_splits((int)B, (int)Hkv, L_max);
    Carve c(ws);
    float* part = (float*)c.take(attn_decode_ws_bytes((int)B, (int)Hq, (int)D, ns));
    return enqueue_attn(q, k_cache, v_cache, L_max, cache_seqlens, (int)B, (int)Sq, (int)Hq, (int)Hkv, (int)D,
                        softmax_scale, causal, out, part, ns, ws, (hipStream_t)stream);
}

size_t fsvd_decode_attn_lowrank_kv_ws(int64_t B, int64_t Sq, int64_t Hq, int64_t Hkv, int64_t D, int64_t L_max) {
    if (B <= 0 || Hkv <= 0 || D <= 0 || L_max <= 0) return kWsHeader;
    const size_t cache = align256((size_t)B * L_max * Hkv * D * 2);
    return fsvd_decode_attn_dense_kv_ws(B, Sq, Hq, Hkv, D, L_max) + 2 * cache;
}

fsvd_status_t fsvd_decode_attn_lowrank_kv(const void* q, const void* zk_cache, const void* zv_cache, int64_t ldz,
                                          const void* Vt_k, int64_t r_k, const void* Vt_v, int64_t r_v,
                                          int64_t L_max, const int32_t* cache_seqlens, int64_t B, int64_t Sq,
                                          int64_t Hq, int64_t Hkv, int64_t D, float rope_theta,
                                          float softmax_scale, int causal, void* out, fsvd_dtype_t dtype,
                                          void* ws, size_t ws_bytes, fsvd_stream_t stream) {
    TRY(need_dtype(dtype, false));
    TRY(need_dim(B, "B")); TRY(need_dim(Sq, "Sq")); TRY(need_dim(Hq, "Hq")); TRY(need_dim(Hkv, "Hkv"));
    TRY(need_dim(D, "D")); TRY(need_dim(L_max, "L_max")); TRY(need_dim(r_k, "r_k")); TRY(need_dim(r_v, "r_v"));
    TRY(check_attn_shape(Hq, Hkv, D));
    TRY(need_vec(r_k, dtype, "r_k")); TRY(need_vec(r_v, dtype, "r_v"));
    TRY(need_ld(ldz, r_k > r_v ? r_k : r_v, dtype, "ldz"));
    if (B * L_max > (int64_t)1 << 30) return fail(FSVD_ERR_UNSUPPORTED, "B * L_max too large");
    TRY(need_ptr(q, "q")); TRY(need_ptr(zk_cache, "zk_cache")); TRY(need_ptr(zv_cache, "zv_cache"));
    TRY(need_ptr(Vt_k, "Vt_k")); TRY(need_ptr(Vt_v, "Vt_v")); TRY(need_ptr(out, "out")); TRY(need_ptr(ws, "ws"));
    if (!cache_seqlens) return fail(FSVD_ERR_INVALID_ARG, "cache_seqlens is NULL");
    if (softmax_scale < 0.f) return fail(FSVD_ERR_INVALID_ARG, "softmax_scale must be >= 0");
    if (rope_theta < 0.f) return fail(FSVD_ERR_INVALID_ARG, "rope_theta must be >= 0");
    const size_t need = fsvd_decode_attn_lowrank_kv_ws(B, Sq, Hq, Hkv, D, L_max);
    if (ws_bytes < need) return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    const int ns = attn_default_splits((int)B, (int)Hkv, L_max);
    Carve c(ws);
    float* part = (float*)c.take(attn_decode_ws_bytes((int)B, (int)Hq, (int)D, ns));
    const size_t cache = (size_t)B * L_max * Hkv * D * 2;
    bf16_t* kc = (bf16_t*)c.take(cache);
    bf16_t* vc = (bf16_t*)c.take(cache);
    hipStream_t st = (hipStream_t)stream;
    // rebuild every cached position: rows (b, p) of the z caches are one M = B * L_max product
    // each; the Q/K/V epilogue (no offsets: position = p) rotates K and writes the dense rows
    const void* Zs[2] = {zk_cache, zv_cache};
    const void* Vs[2] = {Vt_k, Vt_v};
    const int64_t rs[2] = {r_k, r_v};
    for (int i = 0; i < 2; ++i) {
        GemmArgs h{};
        h.A = (const bf16_t*)Zs[i]; h.lda = ldz;
        h.Bm = (const bf16_t*)Vs[i]; h.ldb = rs[i];
        h.M = (int)(B * L_max); h.N = (int)(Hkv * D); h.K = (int)rs[i];
        h.S = (int)L_max; h.Hq = (int)Hq; h.Hkv = (int)Hkv; h.D = (int)D; h.rope_theta = rope_theta;
        h.L_max = L_max; h.seqlens = nullptr; h.k_cache = kc; h.v_cache = vc;
        h.seg = i + 1;
        h.err = (int*)ws;
        TRY(launch_gemm(h, GEPI_QKV, st));
    }
    return enqueue_attn(q, kc, vc, L_max, cache_seqlens, (int)B, (int)Sq, (int)Hq, (int)Hkv, (int)D, softmax_scale,
                        causal, out, part, ns, ws, st);
}

fsvd_status_t fsvd_attn_factorized(const void* zq, const void* zk, const void* zv, int64_t ldz, const void* Vt_q,
                                   int64_t r_q, const void* Vt_k, int64_t r_k, const void* Vt_v, int64_t r_v,
                                   int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, float rope_theta,
                                   float softmax_scale, int causal, void* out, fsvd_dtype_t dtype,
                                   fsvd_stream_t stream) {
    TRY(need_dtype(dtype, false));
    TRY(need_dim(B, "B")); TRY(need_dim(S, "S")); TRY(need_dim(Hq, "Hq")); TRY(need_dim(Hkv, "Hkv"));
    TRY(need_dim(D, "D")); TRY(need_dim(r_q, "r_q")); TRY(need_dim(r_k, "r_k")); TRY(need_dim(r_v, "r_v"));
    TRY(check_attn_shape(Hq, Hkv, D));
    TRY(need_vec(r_q, dtype, "r_q")); TRY(need_vec(r_k, dtype, "r_k")); TRY(need_vec(r_v, dtype, "r_v"));
    TRY(need_ld(ldz, std::max(r_q, std::max(r_k, r_v)), dtype, "ldz"));
    if (B * S > (int64_t)1 << 30) return fail(FSVD_ERR_UNSUPPORTED, "B * S too large");
    TRY(need_ptr(zq, "zq")); TRY(need_ptr(zk, "zk")); TRY(need_ptr(zv, "zv"));
    TRY(need_ptr(Vt_q, "Vt_q")); TRY(need_ptr(Vt_k, "Vt_k")); TRY(need_ptr(Vt_v, "Vt_v")); TRY(need_ptr(out, "out"));
    if (softmax_scale < 0.f) return fail(FSVD_ERR_INVALID_ARG, "softmax_scale must be >= 0");
    if (rope_theta < 0.f) return fail(FSVD_ERR_INVALID_ARG, "rope_theta must be >= 0");
    FactAttnArgs a{};
    a.zq = (const bf16_t*)zq; a.zk = (const bf16_t*)zk; a.zv = (const bf16_t*)zv; a.ldz = ldz;
    a.Vq = (const bf16_t*)Vt_q; a.Vk = (const bf16_t*)Vt_k; a.Vv = (const bf16_t*)Vt_v;
    a.rq = (int)r_q; a.rk = (int)r_k; a.rv = (int)r_v;
    a.B = (int)B; a.S = (int)S; a.Hq = (int)Hq; a.Hkv = (int)Hkv; a.D = (int)D;
    a.rope_theta = rope_theta;
    a.rope_base = rope_theta > 0.f ? std::pow((double)rope_theta, -2.0 / (double)D) : 0.0;
    a.scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)D);
    a.causal = causal;
    a.out = (bf16_t*)out;
    return launch_attn_factorized(a, (hipStream_t)stream);
}

size_t fsvd_swift_covariance_ws(int64_t T, int64_t d_in, int64_t d_out) {
    (void)d_in;
    if (T <= 0 || d_out <= 0) return kWsHeader;
    return kWsHeader + align256((size_t)d_out * T * 2);
}

fsvd_status_t fsvd_swift_covariance(const void* X, int64_t T, int64_t d_in, int64_t ldx, const void* Wt,
                                    int64_t d_out, float* C, int64_t ldc, void* ws, size_t ws_bytes,
                                    fsvd_stream_t stream) {
    TRY(need_dim(T, "T")); TRY(need_dim(d_in, "d_in")); TRY(need_dim(d_out, "d_out"));
    TRY(need_vec(T, FSVD_BF16, "T")); TRY(need_vec(d_in, FSVD_BF16, "d_in")); TRY(need_vec(d_out, FSVD_BF16, "d_out"));
    TRY(need_ld(ldx, d_in, FSVD_BF16, "ldx")); TRY(need_ld(ldc, d_out, FSVD_F32, "ldc"));
    TRY(need_ptr(X, "X")); TRY(need_ptr(Wt, "Wt")); TRY(need_ptr(C, "C")); TRY(need_ptr(ws, "ws"));
    const size_t need = fsvd_swift_covariance_ws(T, d_in, d_out);
    if (ws_bytes < need) return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    Carve c(ws);
    bf16_t* Yt = (bf16_t*)c.take((size_t)d_out * T * 2);
    hipStream_t st = (hipStream_t)stream;
    // Y^T = W^T . X^T: rows of Wt against rows of X (both K-contiguous over d_in)
    GemmArgs g{};
    g.A = (const bf16_t*)Wt; g.lda = d_in; g.Bm = (const bf16_t*)X; g.ldb = ldx;
    g.M = (int)d_out; g.N = (int)T; g.K = (int)d_in; g.C = Yt; g.ldc = T; g.err = (int*)ws;
    TRY(launch_gemm(g, GEPI_STORE, st));
    // C += Y^T . Y: rows of Y^T against themselves (K-contiguous over T), upper triangle
    GemmArgs h{};
    h.A = Yt; h.lda = T; h.Bm = Yt; h.ldb = T;
    h.M = (int)d_out; h.N = (int)d_out; h.K = (int)T; h.C32 = C; h.ldc = ldc; h.err = (int*)ws;
    return launch_gemm(h, GEPI_ACC32, st);
}

size_t fsvd_swift_factors_ws(int64_t d_in, int64_t d_out) {
    if (d_in <= 0 || d_out <= 0) return kWsHeader;
    return kWsHeader + align256((size_t)d_in * d_out * 2);
}

fsvd_status_t fsvd_swift_factors(const void* Wt, int64_t d_out, int64_t d_in, const void* VkT, int64_t k,
                                 void* Ut, void* Vt, void* ws, size_t ws_bytes, fsvd_stream_t stream) {
    TRY(need_dim(d_in, "d_in")); TRY(need_dim(d_out, "d_out")); TRY(need_dim(k, "k"));
    TRY(need_vec(d_in, FSVD_BF16, "d_in")); TRY(need_vec(d_out, FSVD_BF16, "d_out")); TRY(need_vec(k, FSVD_BF16, "k"));
    if (k > d_out || k > d_in) return fail(FSVD_ERR_INVALID_ARG, "k = %lld exceeds min(d_in, d_out)", (long long)k);
    TRY(need_ptr(Wt, "Wt")); TRY(need_ptr(VkT, "VkT")); TRY(need_ptr(Ut, "Ut")); TRY(need_ptr(Vt, "Vt"));
    TRY(need_ptr(ws, "ws"));
    const size_t need = fsvd_swift_factors_ws(d_in, d_out);
    if (ws_bytes < need) return fail(FSVD_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
    Carve c(ws);
    bf16_t* W = (bf16_t*)c.take((size_t)d_in * d_out * 2);
    hipStream_t st = (hipStream_t)stream;
    TRY(launch_transpose((const bf16_t*)Wt, d_out, d_in, d_in, W, d_out, st));
    // Ut = V_k^T . W^T: rows of VkT against rows of W (both K-contiguous over d_out)
    GemmArgs g{};
    g.A = (const bf16_t*)VkT; g.lda = d_out; g.Bm = W; g.ldb = d_out;
    g.M = (int)k; g.N = (int)d_in; g.K = (int)d_out; g.C = (bf16_t*)Ut; g.ldc = d_in; g.err = (int*)ws;
    TRY(launch_gemm(g, GEPI_STORE, st));
    return launch_transpose((const bf16_t*)VkT, k, d_out, d_out, (bf16_t*)Vt, k, st);
}

fsvd_status_t fsvd_layernorm(const void* x, const void* residual, const void* gamma, const void* beta, float eps,
                             int64_t M, int64_t d, void* y, fsvd_dtype_t dtype, fsvd_stream_t stream) {
    TRY(need_dtype(dtype, false));
    TRY(need_dim(M, "M")); TRY(need_dim(d, "d"));
    if (d > 16384) return fail(FSVD_ERR_UNSUPPORTED, "LayerNorm width %lld > 16384", (long long)d);
    TRY(need_ptr(x, "x")); TRY(need_ptr(gamma, "gamma")); TRY(need_ptr(beta, "beta")); TRY(need_ptr(y, "y"));
    TRY(opt_ptr(residual, "residual"));
    return launch_layernorm((const bf16_t*)x, (const bf16_t*)residual, (const bf16_t*)gamma, (const bf16_t*)beta, eps, M,
                            d, (bf16_t*)y, (hipStream_t)stream);
}

fsvd_status_t fsvd_read_stream_probe(const void* src, size_t bytes, void* out, fsvd_stream_t stream) {
    TRY(need_ptr(src, "src")); TRY(need_ptr(out, "out"));
    if (bytes < 16) return fail(FSVD_ERR_INVALID_ARG, "bytes must be at least 16");
    return launch_read_stream(src, bytes, (uint32_t*)out, (hipStream_t)stream);
}

fsvd_status_t fsvd_seqlens_advance(int32_t* cache_seqlens, int64_t B, int32_t n, fsvd_stream_t stream) {
    if (!cache_seqlens) return fail(FSVD_ERR_INVALID_ARG, "cache_seqlens is NULL");
    TRY(need_dim(B, "B"));
    return launch_seqlens_advance(cache_seqlens, B, n, (hipStream_t)stream);
}

size_t fsvd_decoder_layer_ws(const fsvd_decoder_layer_desc* desc) {
    if (!desc) return 0;
    return plan_layer(desc, nullptr).bytes;
}

fsvd_status_t fsvd_decoder_layer_run(const fsvd_decoder_layer_desc* desc, fsvd_stream_t stream) {
    TRY(validate_layer(desc));
    return enqueue_layer(desc, (hipStream_t)stream);
}

fsvd_status_t fsvd_decoder_layer_capture(const fsvd_decoder_layer_desc* desc, fsvd_graph** out) {
    return fsvd_decoder_stack_capture(desc, 1, out);
}

fsvd_status_t fsvd_decoder_stack_capture(const fsvd_decoder_layer_desc* descs, int n_layers, fsvd_graph** out) {
    if (!out) return fail(FSVD_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (!descs || n_layers <= 0) return fail(FSVD_ERR_INVALID_ARG, "no layers");
    for (int l = 0; l < n_layers; ++l) {
        TRY(validate_layer(&descs[l]));
        if (descs[l].S != 1) return fail(FSVD_ERR_UNSUPPORTED, "graph capture is for single-token decode steps (S == 1)");
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fail(FSVD_ERR_HIP, "hipGetDevice failed");
    hipStream_t cs;
    {
        std::lock_guard<std::mutex> lk(g_graph_mu);
        if (!g_capture_stream[dev]) {
            if (hipStreamCreateWithFlags(&g_capture_stream[dev], hipStreamNonBlocking) != hipSuccess)
                return fail(FSVD_ERR_HIP, "capture stream creation failed");
        }
        cs = g_capture_stream[dev];
    }
    hipGraph_t graph = nullptr;
    if (hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal) != hipSuccess)
        return fail(FSVD_ERR_CAPTURE, "hipStreamBeginCapture failed");
    fsvd_status_t s = FSVD_OK;
    for (int l = 0; l < n_layers && s == FSVD_OK; ++l) s = enqueue_layer(&descs[l], cs);
    const hipError_t e = hipStreamEndCapture(cs, &graph);
    if (s != FSVD_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        return s;
    }
    if (e != hipSuccess || !graph) return fail(FSVD_ERR_CAPTURE, "hipStreamEndCapture: %s", hipGetErrorString(e));
    hipGraphExec_t exec = nullptr;
    if (hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0) != hipSuccess) {
        (void)hipGraphDestroy(graph);
        return fail(FSVD_ERR_CAPTURE, "hipGraphInstantiate failed");
    }
    fsvd_graph* g = new (std::nothrow) fsvd_graph{graph, exec, dev};
    if (!g) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return fail(FSVD_ERR_CAPTURE, "out of host memory");
    }
    {
        std::lock_guard<std::mutex> lk(g_graph_mu);
        g_live_graphs.insert(g);
    }
    *out = g;
    return FSVD_OK;
}

fsvd_status_t fsvd_graph_replay(fsvd_graph* g, fsvd_stream_t stream) {
    {
        std::lock_guard<std::mutex> lk(g_graph_mu);
        if (!g || !g_live_graphs.count(g)) return fail(FSVD_ERR_CAPTURE, "graph handle is not live (destroyed or never captured)");
    }
    const hipError_t e = hipGraphLaunch(g->exec, (hipStream_t)stream);
    if (e != hipSuccess) return fail(FSVD_ERR_HIP, "hipGraphLaunch: %s", hipGetErrorString(e));
    return FSVD_OK;
}

fsvd_status_t fsvd_graph_destroy(fsvd_graph* g) {
    {
        std::lock_guard<std::mutex> lk(g_graph_mu);
        if (!g || !g_live_graphs.count(g)) return fail(FSVD_ERR_CAPTURE, "graph handle is not live");
        g_live_graphs.erase(g);
    }
    (void)hipGraphExecDestroy(g->exec);
    (void)hipGraphDestroy(g->graph);
    delete g;
    return FSVD_OK;
}

fsvd_status_t fsvd_poll_device_error(void* ws, fsvd_stream_t stream, int32_t* code) {
    if (!ws || !code) return fail(FSVD_ERR_INVALID_ARG, "ws and code must be non-NULL");
    int32_t v = 0;
    hipError_t e = hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return fail(FSVD_ERR_HIP, "poll: %s", hipGetErrorString(e));
    *code = v;
    if (v != 0) {
        const int32_t zero = 0;
        e = hipMemcpyAsync(ws, &zero, sizeof(zero), hipMemcpyHostToDevice, (hipStream_t)stream);
        if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
        if (e != hipSuccess) return fail(FSVD_ERR_HIP, "poll clear: %s", hipGetErrorString(e));
        return fail(FSVD_ERR_DEVICE, "device error word 0x%x", (unsigned)v);
    }
    return FSVD_OK;
}

}  // extern "C"
