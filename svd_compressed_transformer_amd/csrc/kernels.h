// Internal launcher interfaces between the C-ABI front (capi.hip) and the kernel files.
#pragma once
#include "common.h"

namespace fsvd {

// ---------------------------------------------------------------- decode row-dot (GEMV) kernels
//
// out[m, n] = sum_k act[m, k] * W[n, k] for the M (<= 32) activation rows, streaming each row of
// W once from HBM.  One launch covers up to 3 output segments (Q, K, V share one launch).

enum RowdotEpi : int {
    EPI_Z = 0,       // out[m, n] = acc (* rstd[m] when the RMSNorm prologue is on); store T
    EPI_LINEAR = 1,  // out[m, n] = acc + bias[n] + residual[m, n]
    EPI_QKV = 2,     // segment kinds below: q / k get RoPE; k, v are appended to the cache
    EPI_SWIGLU = 3,  // rows (gate n, up n): out[m, n] = SiLU(g) * u
    EPI_GELU = 4,    // out[m, n] = GELU(acc)
};
enum SegKind : int { SEG_PLAIN = 0, SEG_Q = 1, SEG_K = 2, SEG_V = 3 };

struct RowdotSeg {
    const void* W;   // [N, ldw]; for EPI_SWIGLU the gate matrix
    const void* W2;  // EPI_SWIGLU: the up matrix (same N), else null
    int64_t ldw, ldw2;
    int N;           // output rows of the segment
    int K, K2;       // reduction lengths of W / W2 (multiples of the vector width)
    int act_off, act_off2;  // activation column offsets used by W / W2
    int kind;        // SegKind
    int blk_begin;   // first workgroup of the segment
    int units_per_blk;
    void* out;       // EPI_Z / LINEAR / SWIGLU / GELU / SEG_Q output [M, ldo]
    int64_t ldo;
};

struct RowdotArgs {
    RowdotSeg seg[3];
    int nseg;
    int ksplit;      // waves sharing one row group (split of the reduction): 1, 2, 4 or 8
    int waves;       // waves per workgroup: 4 or 8
    // matrix-core launches with few tiles: the reduction is also split over kpart workgroups
    // (set by the planner when part and err are given); partial tiles go to part, and the last of a
    // tile's kpart workgroups to finish sums them and runs the epilogue, counted in the workspace
    // header behind err.  nblk: tiles (workgroups per reduction part).
    int kpart, nblk;
    float* part;     // fp32 partial tiles, rowdot_part_bytes(M, dtype) bytes (NULL: no split)
    unsigned* split_cnt;  // [nblk] counters in the workspace header (set by the launcher)
    const void* act; // [M, lda]
    int64_t lda;
    int M;
    // RMSNorm prologue (EPI_Z only): stats over act columns [0, norm_K)
    int norm;
    const bf16_t* norm_w;
    float norm_eps;
    int norm_K;
    // EPI_LINEAR
    const void* bias;
    const void* residual;
    int64_t ldr;
    // EPI_QKV
    int S, Hq, Hkv, D;
    float rope_theta;
    double rope_base;  // theta^(-2/D), set by the host when rope_theta > 0
    int64_t L_max;
    const int32_t* seqlens;
    bf16_t *k_cache, *v_cache, *k_out, *v_out;
    int* err;
    // advance cache_seqlens by adv_n after the launch (block 0 thread 0; EPI_LINEAR only)
    int32_t* adv_seqlens;
    int adv_B, adv_n;
};

// Launch one row-dot kernel.  dtype FSVD_BF16 (all epilogues) or FSVD_F32 (EPI_Z, EPI_LINEAR).
// bf16 launches with 5..32 activation rows run the products on the matrix cores.
fsvd_status_t launch_rowdot(const RowdotArgs& a, int epi, fsvd_dtype_t dtype, hipStream_t st);
// Helper filling seg.blk_begin / units_per_blk and returning the total grid size.
int rowdot_plan(RowdotArgs& a, int epi, fsvd_dtype_t dtype);
// Workspace bytes a row-dot launch of M activation rows may use for split-reduction partials.
size_t rowdot_part_bytes(int64_t M, fsvd_dtype_t dtype);

// ---------------------------------------------------------------- attention
struct AttnArgs {
    const bf16_t* q;   // [B, Sq, Hq, D]
    const bf16_t* kc;  // [B, L_max, Hkv, D]
    const bf16_t* vc;
    const int32_t* seqlens;
    bf16_t* out;       // [B, Sq, Hq, D]
    int B, Sq, Hq, Hkv, D;
    int64_t L_max;
    float scale;
    int causal;
    int nsplit;        // decode: partitions of the length
    float* part;       // decode partials [B, Hq, nsplit, D + 2]
    unsigned* cnt;     // decode: [B * Hkv] partition counters (zero on entry, zero on exit); the
                       // last partition of each (b, kv head) merges them.  Null: a second kernel merges
    int* err;
    int pos_off;       // Sq > 1: query s of sequence b sits at position seqlens[b] + pos_off + s (a
                       // prefill chunk that starts pos_off tokens into the call's new tokens)
};
// factorised attention: S tokens per sequence among themselves, Q/K/V rebuilt from z on chip
struct FactAttnArgs {
    const bf16_t *zq, *zk, *zv;  // [B * S, ldz] rank activations (may be column ranges of one buffer)
    int64_t ldz;
    const bf16_t *Vq, *Vk, *Vv;  // [Hq * D, rq], [Hkv * D, rk], [Hkv * D, rv]
    int rq, rk, rv;
    int B, S, Hq, Hkv, D;
    float rope_theta;            // 0: no RoPE
    double rope_base;            // theta^(-2/D)
    float scale;
    int causal;
    bf16_t* out;                 // [B, S, Hq, D]
};
fsvd_status_t launch_attn_factorized(const FactAttnArgs& a, hipStream_t st);
size_t attn_decode_ws_bytes(int B, int Hq, int D, int nsplit);
int attn_default_splits(int B, int Hkv, int64_t L_max);
fsvd_status_t launch_attn_decode(const AttnArgs& a, hipStream_t st);
fsvd_status_t launch_attn_prefill(const AttnArgs& a, hipStream_t st);

// ---------------------------------------------------------------- glue
fsvd_status_t launch_prepack(void* dst, int64_t ld_dst, int64_t cols_pad, int64_t row0, const void* src, int64_t rows,
                             int64_t cols, int64_t ld_src, int64_t rows_pad, size_t es, const void* col_scale,
                             hipStream_t st);
fsvd_status_t launch_layernorm(const bf16_t* x, const bf16_t* res, const bf16_t* g, const bf16_t* b, float eps,
                               int64_t M, int64_t d, bf16_t* y, hipStream_t st);
fsvd_status_t launch_seqlens_advance(int32_t* sl, int64_t B, int32_t n, hipStream_t st);
// reads `bytes` (rounded down to 16) once; folds an XOR of them into out[0..63]
fsvd_status_t launch_read_stream(const void* src, size_t bytes, uint32_t* out, hipStream_t st);

// ---------------------------------------------------------------- prefill (MFMA) GEMM
enum GemmEpi : int {
    GEPI_STORE = 0,    // C = acc (bf16) (* rstd[m] when rstd != null)
    GEPI_LINEAR = 1,   // C = acc + bias + residual
    GEPI_QKV = 2,      // column segments q | k | v with RoPE and cache append
    GEPI_SWIGLU = 3,   // dual B operand: C = SiLU(A.Bg^T) * (A.Bu^T)
    GEPI_GELU = 4,
    GEPI_ACC32 = 5,    // C32[m, n] += acc (fp32); square tiles, those wholly below the diagonal are
                       // skipped (symmetric products A . A^T: the upper triangle is computed)
};
struct GemmArgs {
    // C[M, N] = A[M, a_col_off : a_col_off + K] . B[N, K]^T ; bf16 operands, K-contiguous, fp32 accumulate
    const bf16_t* A; int64_t lda; int a_col_off;
    const bf16_t* Bm; int64_t ldb;
    const bf16_t* B2; int64_t ldb2; int a_col_off2; int K2;   // GEPI_SWIGLU: the up operand
    int M, N, K;
    bf16_t* C; int64_t ldc;
    const float* rstd;           // optional per-row scale [M] (RMSNorm folded after the product)
    const bf16_t* bias;
    const bf16_t* residual; int64_t ldr;
    int seg;                     // GEPI_QKV: 0 = q, 1 = k, 2 = v
    int S, Hq, Hkv, D;
    float rope_theta;
    int64_t L_max;
    const int32_t* seqlens;      // GEPI_QKV: position of row (b, s) = seqlens[b] + s (NULL: s)
    int row_off;                 // GEPI_QKV: row m of this launch is token row_off + m of the call
                                 // ([B, S] flattened: b = (row_off + m) / S); q_out keeps local rows
    // GEPI_QKV grouped launch: nseg (2 or 3) column segments side by side in one grid, segment s
    // with its own B operand, rank and A column range (seg s = q, k, v); nseg 0 or 1: the single
    // problem above (Bm, ldb, K, a_col_off, N, seg)
    int nseg;
    struct Seg {
        const bf16_t* Bm; int64_t ldb; int K; int a_col_off; int N;
    } segs[3];
    float* C32;                  // GEPI_ACC32: fp32 accumulator [M, ldc]
    bf16_t *q_out, *k_cache, *v_cache, *k_out, *v_out;
    int* err;
};
fsvd_status_t launch_gemm(const GemmArgs& g, int epi, hipStream_t st);
// ---------------------------------------------------------------- fused MLP middle (prefill)
// z_d = act(z_u . Vt_u^T [, z_g . Vt_g^T]) . Ut_d^T with t kept on chip (mlp_fused.hip)
struct MlpFusedArgs {
    const bf16_t* z; int64_t ldz;     // [M, ldz]: z_g = columns [0, rg), z_u = [rg, rg + ru)
    int rg, ru, rd, M, d_ff;          // rg = 0: GELU(u); else SiLU(g) * u
    const bf16_t *Vg, *Vu;            // [d_ff, rg], [d_ff, ru]
    const bf16_t* Ud; int64_t ldu;    // [rd, ldu]
    bf16_t* part;                     // [S, M, rd] per-slice partial sums (plan.part_bytes; S > 1 only)
    bf16_t* z_d;                      // [M, rd]
};
struct MlpFusedPlan {
    int bm, nw, nb, S, cps;           // rows and waves per workgroup, row blocks, d_ff slices, chunks per slice
    size_t part_bytes;
};
// false when no fused kernel covers these ranks (the two-product path is used instead)
bool mlp_fused_plan(int64_t M, int64_t rg, int64_t ru, int64_t d_ff, int64_t rd, MlpFusedPlan* p);
fsvd_status_t launch_mlp_fused(const MlpFusedArgs& a, const MlpFusedPlan& p, hipStream_t st);

// out[c, r] = in[r, c] for r < rows, c < cols (bf16, through 64 x 64 LDS tiles)
fsvd_status_t launch_transpose(const bf16_t* in, int64_t rows, int64_t cols, int64_t ld_in, bf16_t* out,
                               int64_t ld_out, hipStream_t st);
// per-row inverse RMS of x [M, d] (with norm weight folded by the caller) -> rstd [M], and
// xn = bf16(x * w) [M, d]
fsvd_status_t launch_rms_prep(const bf16_t* x, const bf16_t* w, float eps, int64_t M, int64_t d, bf16_t* xn,
                              float* rstd, hipStream_t st);

}  // namespace fsvd
