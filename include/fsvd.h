/*
 * fsvd.h - C ABI of the fused low-rank transformer-layer library for AMD Instinct MI355X (gfx950).
 *
 * The library implements the serving hot path of an SVD-compressed transformer layer: every
 * dense projection W is replaced by a factor pair and applied as y = (x . U) . V (two fused
 * kernels per projection: the rank-r intermediate z is accumulated in fp32 on chip and stored once
 * in bf16 for the second), on packed Q/K/V and O projections and on a packed
 * gate|up SwiGLU MLP (GELU for encoder layers), feeding attention over a contiguous dense KV
 * cache; each layer's decode step can be captured once as a hipGraph and replayed per token.
 *
 * Sources, cited by page title and section:
 *   [V1]    "FlashSVD: Memory-Efficient Inference with Streaming for Low-Rank Models", abstract:
 *           fused low-rank projections in attention and FFN; factor tiles streamed through
 *           on-chip memory so full-size activation buffers are never materialised.
 *   [V15-PS] "FlashSVD v1.5: Making Low-Rank Transformers Inference Actually Fast" (explainer),
 *           Problem Statement: rebuilding the attention history from the factors at every step
 *           means irregular access and recomputation.
 *   [V15-M1] same page, Methodology 1, Unified Runtime Abstraction: one common factorized
 *           representation.
 *   [V15-M2] same page, Methodology 2, Dense-KV Attention: rebuild dense Q/K/V for the current
 *           tokens only, keep history in a contiguous dense KV cache read in one attention step.
 *   [V15-M3] same page, Methodology 3, Packed MLP Execution: gate and up input-side factors
 *           packed offline into one tensor, one wide projection, then a split.
 *   [V15-M4] same page, Methodology 4, Per-Layer CUDA Graph Replay: the stable small-batch decode
 *           body of each layer captured once and replayed.
 *   [SWIFT-2A] "Swift-SVD: Theoretical Optimality Meets Practical Efficiency in Low-Rank LLM
 *           Compression" (explainer), section 2A: the output covariance aggregated batch by
 *           batch, one eigendecomposition, the rank-k optimum W V_k V_k^T in closed form.
 *
 * General conventions (apply to every call unless its comment says otherwise)
 *   - Pointers are DEVICE pointers unless marked (host).  Matrices are row-major; "ld" is the row
 *     stride in elements.  Activations are row vectors: y = x . U . V.
 *   - Factor storage ("common factorized representation"): a projection of input width K and
 *     output width N with rank r is stored as Ut = U^T [r, K] (row i = input-side factor of rank
 *     component i) and Vt = V^T [N, r], both K-contiguous like two linear-layer weights.
 *   - Ranks passed to the library are STORED ranks: they must be multiples of 8 (bf16) or 4
 *     (fp32) so rows are 16-byte vectors.  A caller whose logical rank is not a multiple pads
 *     Ut with zero rows and Vt with zero columns (fsvd_prepack does this); padding is exact.
 *   - Alignment: every pointer must be 16-byte aligned and every ld * element size a multiple
 *     of 16 bytes.  Hidden sizes K, N must be multiples of 8 (bf16) / 4 (fp32).
 *   - dtype: FSVD_BF16 means bf16 storage for every tensor of the call (weights, activations,
 *     outputs, KV cache), fp32 accumulation, fp32 softmax; FSVD_F32 means fp32 throughout.
 *     Documented bf16 rounding points: the normalised input of a projection, the rank
 *     activations z, and the MLP product t are rounded to bf16 before their next product.
 *   - Ownership: the caller owns every buffer, including the workspace ("ws").  The library
 *     never allocates device memory inside these calls and never synchronises, except where a
 *     call says so (capture, poll).
 *   - Workspace: each call that needs scratch takes (ws, ws_bytes); the matching *_ws() query
 *     returns the size.  The first 4096 bytes of every workspace are a header: its first int32
 *     is the DEVICE ERROR WORD, and from byte 64 on it holds counters of the decode kernels (the
 *     split reductions' tiles, then the attention's partitions), which every call leaves at zero.
 *     A workspace must be zero-filled once before its first use; after that the header stays
 *     valid whichever calls share the workspace.
 *   - Errors: every call returns fsvd_status_t.  Arguments are validated before any launch
 *     (null pointers, non-positive sizes, misalignment, too-small workspace, unsupported
 *     combinations); on failure nothing is launched and fsvd_last_error() explains.  Launch
 *     failures return FSVD_ERR_HIP.  Conditions only the device can see (a KV position at or
 *     beyond L_max) skip the offending write, never write out of bounds, and set the device
 *     error word, which fsvd_poll_device_error() reads.  C++ exceptions never cross the ABI.
 *   - Streams: every call is asynchronous on the caller's hipStream_t (0 = default stream).
 *   - Thread safety: calls are stateless apart from graph objects and the thread-local error
 *     string; concurrent calls on different streams must use different workspaces.
 */
#ifndef FSVD_H
#define FSVD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* fsvd_stream_t; /* a hipStream_t */

#define FSVD_ABI_VERSION 8

typedef enum {
    FSVD_OK = 0,
    FSVD_ERR_INVALID_ARG = 1, /* bad pointer, size, alignment or leading dimension */
    FSVD_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. dtype for this call) */
    FSVD_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the *_ws() query */
    FSVD_ERR_HIP = 4,         /* a HIP runtime call failed (launch, capture, copy) */
    FSVD_ERR_CAPTURE = 5,     /* graph capture / instantiate / replay failed or graph destroyed */
    FSVD_ERR_DEVICE = 6       /* poll found a non-zero device error word */
} fsvd_status_t;

typedef enum { FSVD_F32 = 0, FSVD_BF16 = 1 } fsvd_dtype_t;
typedef enum { FSVD_ACT_SWIGLU = 0, FSVD_ACT_GELU = 1 } fsvd_act_t;

/* Device error word bits (OR-ed). */
#define FSVD_DEVERR_KV_OVERFLOW 0x1 /* a token position >= L_max: its KV write was skipped */
#define FSVD_DEVERR_SEQ_OVERFLOW 0x2 /* attention length > L_max: clamped to L_max */

int fsvd_abi_version(void);
const char* fsvd_status_str(fsvd_status_t s); /* static string */
const char* fsvd_last_error(void);            /* thread-local detail of this thread's last failure */

/* ------------------------------------------------------------------------------------------
 * a1. Offline prepack  [V15-M3] (input-side factors that share an input are packed into one
 * tensor; this library also packs Q/K/V that way).  Not on the timed path.
 *
 * Writes the n_items source matrices one below the other into dst [sum(rows_pad), cols_pad]
 * (row stride ld_dst >= cols_pad): item i occupies rows_pad[i] rows; its first rows[i] rows
 * hold src[i] (columns [0, cols[i]), the rest of the row zero) and the remaining rows are
 * zero.  Used both to stack Ut blocks (A_qkv = [Ut_q; Ut_k; Ut_v], A_gu = [Ut_gate; Ut_up],
 * each rank padded to a multiple of 8, or better 32) and to zero-pad the rank columns of a Vt.
 * Ranks padded to a multiple of 32 make every factor row and every row of the rank
 * activations z start on a 64-byte boundary, which the prefill-size products read faster.
 * Bit-exact copy.  items is a HOST array; src pointers are device pointers.
 * ------------------------------------------------------------------------------------------ */
typedef struct {
    const void* src;
    int64_t rows, cols, ld_src; /* source extent and row stride (elements) */
    int64_t rows_pad;           /* rows this item occupies in dst (>= rows) */
} fsvd_pack_item;

fsvd_status_t fsvd_prepack(void* dst, int64_t ld_dst, int64_t cols_pad, const fsvd_pack_item* items /*host*/,
                           int n_items, fsvd_dtype_t dtype, fsvd_stream_t stream);

/* As fsvd_prepack, and every column c < cols[i] of every item is multiplied by col_scale[c]
 * (device, at least max cols[i] entries, same dtype; product in fp32, bf16 rounded to nearest
 * even).  Folds an RMSNorm weight w into the input-side factor that follows the norm:
 * RMSNorm(x) . A^T = rstd(x) * (x . (A diag(w))^T), so a layer built from A diag(w) runs the
 * norm without its per-element weight multiply (fsvd_decoder_layer_desc flag
 * FSVD_LAYER_NORM_FOLDED).  Rounding moves from bf16(x * w) to bf16(A * w).  Not timed. */
fsvd_status_t fsvd_prepack_colscale(void* dst, int64_t ld_dst, int64_t cols_pad,
                                    const fsvd_pack_item* items /*host*/, int n_items, const void* col_scale,
                                    fsvd_dtype_t dtype, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * a2+a3. Fused low-rank linear  [V1] [V15-M1]
 *   y[m, :] = residual[m, :] + bias + (x[m, :] . Ut^T) . Vt^T        (z = x . Ut^T is rank-r)
 * x [M, K] (ldx), Ut [r, K] (ldu), Vt [N, r] (ldv), bias [N] or NULL, residual [M, N] (ldr)
 * or NULL (may alias y for in-place accumulation), y [M, N] (ldy).  r <= min(K, N) (else
 * FSVD_ERR_INVALID_ARG).  dtype FSVD_F32 or FSVD_BF16.
 * Decode-sized M (<= 32) runs the HBM-streaming row-dot kernels (z passes through the
 * workspace as a B x r vector; bf16 launches of 5..32 rows also keep a 1.25 MiB slice there for
 * the partial tiles of reductions split across workgroups); larger M runs the bf16 MFMA path
 * (bf16 only).
 * ------------------------------------------------------------------------------------------ */
size_t fsvd_lowrank_linear_ws(int64_t M, int64_t K, int64_t r, int64_t N, fsvd_dtype_t dtype);
fsvd_status_t fsvd_lowrank_linear(const void* x, int64_t M, int64_t K, int64_t ldx,
                                  const void* Ut, int64_t r, int64_t ldu,
                                  const void* Vt, int64_t N, int64_t ldv,
                                  const void* bias, const void* residual, int64_t ldr,
                                  void* y, int64_t ldy, fsvd_dtype_t dtype,
                                  void* ws, size_t ws_bytes, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Allocation-free fused low-rank linear, for callers that cannot allocate device memory or
 * hand the library a workspace: code under hipGraph stream capture, tight serving loops, and
 * harnesses that forbid allocation.
 * Same arguments, kernels and result (bit for bit) as fsvd_lowrank_linear without (ws,
 * ws_bytes): the scratch (the rank-r intermediate z and the split-reduction partials) lives in a
 * static device array of FSVD_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held
 * from the first call on that GPU until the process ends.  A call whose
 * fsvd_lowrank_linear_ws(M, K, r, N, dtype) exceeds FSVD_NOALLOC_SCRATCH_BYTES returns
 * FSVD_ERR_WORKSPACE before anything is launched.  The call itself allocates nothing; its first
 * call on a GPU resolves that GPU's copy of the array once (hipGetSymbolAddress, with the
 * device current), so make that first call outside stream capture.  Every call on one GPU
 * shares that GPU's array and finds it as the previous call left it (nothing in it has to start
 * at zero): calls ordered on one stream are safe; calls that overlap on one GPU (concurrent
 * streams, unordered host threads) race on it and must not be issued.
 * ------------------------------------------------------------------------------------------ */
#define FSVD_NOALLOC_SCRATCH_BYTES (32u << 20) /* 32 MiB per GPU */
fsvd_status_t fsvd_lowrank_linear_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx,
                                          const void* Ut, int64_t r, int64_t ldu,
                                          const void* Vt, int64_t N, int64_t ldv,
                                          const void* bias, const void* residual, int64_t ldr,
                                          void* y, int64_t ldy, fsvd_dtype_t dtype, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * a2+a3+a5. Packed Q/K/V projection with KV append  [V15-M2] [V15-M3]
 *   a = RMSNorm(x) (if norm_w) = x / sqrt(mean(x^2) + eps) * norm_w, else x
 *   [z_q | z_k | z_v] = a . A_qkv^T   (one wide projection, split at r_q and r_q + r_k)
 *   q = z_q . Vt_q^T, k = z_k . Vt_k^T, v = z_v . Vt_v^T; RoPE (rotate-half, pair (i, i+D/2)
 *   turned by angle p * theta^(-2i/D)) on q and k when rope_theta > 0, at position
 *   p = cache_seqlens[b] + s for token s of sequence b;
 *   q -> q_out [B, S, Hq, D]; k, v -> k_cache, v_cache [B, L_max, Hkv, D] at position p
 *   (bit-exact copy of the bf16 k/v); optional k_out, v_out [B, S, Hkv, D] (NULL = skip)
 *   receive the same bits (for checking).
 * x [B, S, d] contiguous; A_qkv [r_q + r_k + r_v, d]; Vt_q [Hq*D, r_q], Vt_k [Hkv*D, r_k],
 * Vt_v [Hkv*D, r_v] contiguous; cache_seqlens [B] int32 = tokens already cached (read only).
 * Positions >= L_max: the KV write is skipped and FSVD_DEVERR_KV_OVERFLOW set.  bf16 only.
 * ------------------------------------------------------------------------------------------ */
size_t fsvd_lowrank_qkv_ws(int64_t B, int64_t S, int64_t d, int64_t r_q, int64_t r_k, int64_t r_v,
                           int64_t Hq, int64_t Hkv, int64_t D);
fsvd_status_t fsvd_lowrank_qkv(const void* x, int64_t B, int64_t S, int64_t d,
                               const void* norm_w, float norm_eps,
                               const void* A_qkv, int64_t r_q, int64_t r_k, int64_t r_v,
                               const void* Vt_q, const void* Vt_k, const void* Vt_v,
                               int64_t Hq, int64_t Hkv, int64_t D, float rope_theta,
                               void* q_out, void* k_cache, void* v_cache, int64_t L_max,
                               const int32_t* cache_seqlens, void* k_out, void* v_out,
                               fsvd_dtype_t dtype, void* ws, size_t ws_bytes, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * a2+a3+a4. Packed low-rank MLP  [V15-M3] [V1]
 *   b = RMSNorm(x) if norm_w else x
 *   z = b . A_gu^T, z_g = z[:, :r_g], z_u = z[:, r_g:r_g+r_u]   (A_gu = [Ut_gate; Ut_up])
 *   SWIGLU: t = SiLU(z_g . Vt_g^T) * (z_u . Vt_u^T);  GELU: t = GELU(z_u . Vt_u^T) (r_g = 0,
 *   Vt_g NULL; exact erf form);  y = residual + (t . Ut_d^T) . Vt_d^T
 * x [M, d]; A_gu [r_g + r_u, d]; Vt_g, Vt_u [d_ff, r_g|r_u]; Ut_d [r_d, d_ff]; Vt_d [d, r_d];
 * residual [M, d] or NULL (may alias y); y [M, d].  All contiguous.  bf16 only.
 * g and u never leave the registers of the kernel that forms them.  At prefill sizes (M > 32)
 * with equal gate/up and down ranks of 128, 256 or 384 (stored), t does not leave the chip either:
 * one kernel forms t for 32 columns of d_ff at a time and folds it into z_d = t . Ut_d^T, and
 * the workspace holds only rank-wide activations (z, per-slice partial sums of z_d, z_d).
 * Otherwise t [M, d_ff] passes through the workspace between two kernels: at decode sizes
 * (M <= 32) a few hundred KB that stay in L2; at prefill sizes it is written once and read once
 * (the decoder layer bounds that by running its tokens in passes of at most prefill_chunk rows).
 * ------------------------------------------------------------------------------------------ */
size_t fsvd_lowrank_mlp_packed_ws(int64_t M, int64_t d, int64_t r_g, int64_t r_u, int64_t d_ff, int64_t r_d);
fsvd_status_t fsvd_lowrank_mlp_packed(const void* x, int64_t M, int64_t d,
                                      const void* norm_w, float norm_eps, fsvd_act_t act,
                                      const void* A_gu, int64_t r_g, int64_t r_u,
                                      const void* Vt_g, const void* Vt_u, int64_t d_ff,
                                      const void* Ut_d, const void* Vt_d, int64_t r_d,
                                      const void* residual, void* y, fsvd_dtype_t dtype,
                                      void* ws, size_t ws_bytes, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * a6. Attention over the contiguous dense KV cache  [V15-M2]
 *   o[b, s, h] = sum_{j < n} softmax_j(scale * q[b, s, h] . k[b, j, g]) v[b, j, g],
 *   g = floor(h * Hkv / Hq), n = cache_seqlens[b] + s + 1 (causal) or cache_seqlens[b] + Sq.
 * q, out [B, Sq, Hq, D]; caches [B, L_max, Hkv, D]; cache_seqlens [B] int32 = valid length
 * BEFORE this call's Sq tokens were appended (they must already be in the cache).
 * softmax_scale 0 -> 1/sqrt(D).  Sq == 1 uses split-length partitions merged by log-sum-exp
 * (the partition count is fixed by the workspace; lengths are read on the device, so a
 * captured graph stays valid as the cache grows).  The last partition of each (sequence, kv
 * head) to finish does the merge, counted in the workspace header when B * Hkv <= 880; beyond
 * that a second kernel merges.  Sq > 1 (prefill and encoder layers) runs on the matrix cores.
 * D must be 64 or 128; Hq % Hkv == 0.  bf16 only.  Layout advice: L_max a multiple of 64 keeps each
 * sequence's cache on a 64-position boundary, which decode streams faster (MI355X, batch 4, 32 heads
 * of 128, 2048 positions: 27.3 us per call with L_max 2176 against 29.8 us with L_max 2049).
 * n > L_max is clamped to L_max and sets FSVD_DEVERR_SEQ_OVERFLOW.
 * ------------------------------------------------------------------------------------------ */
size_t fsvd_decode_attn_dense_kv_ws(int64_t B, int64_t Sq, int64_t Hq, int64_t Hkv, int64_t D, int64_t L_max);
fsvd_status_t fsvd_decode_attn_dense_kv(const void* q, const void* k_cache, const void* v_cache, int64_t L_max,
                                        const int32_t* cache_seqlens, int64_t B, int64_t Sq, int64_t Hq,
                                        int64_t Hkv, int64_t D, float softmax_scale, int causal, void* out,
                                        fsvd_dtype_t dtype, void* ws, size_t ws_bytes, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Comparator: attention over a low-rank history  [V15-PS] [V15-M2]
 * The layout the dense cache replaces: the history keeps only the rank-r projections of each
 * token, z_k = a . Ut_k^T and z_v = a . Ut_v^T, and every step rebuilds the whole K and V
 * from them before attending:
 *   K[b, p] = RoPE(z_k[b, p] . Vt_k^T, position p),  V[b, p] = z_v[b, p] . Vt_v^T
 * for every cached position p < L_max, then the attention of fsvd_decode_attn_dense_kv over
 * (K, V) with the same q, cache_seqlens, scale and causal arguments.  The result equals the
 * dense-KV path's whenever the dense cache holds RoPE(z_k . Vt_k^T) and z_v . Vt_v^T; the
 * cost is the rebuild, a (B * L_max) x r x (Hkv * D) contraction per cache every step.
 * zk_cache, zv_cache [B, L_max, ldz] bf16 (rows of r_k resp. r_v used; the caller appends
 * the new tokens' z rows before the call); Vt_k [Hkv*D, r_k], Vt_v [Hkv*D, r_v] (stored,
 * padded ranks, multiples of 8); q, out [B, Sq, Hq, D].  rope_theta 0 -> no RoPE.  The
 * rebuilt K and V live in the workspace (2 * B * L_max * Hkv * D bf16).  bf16 only.
 * ------------------------------------------------------------------------------------------ */
size_t fsvd_decode_attn_lowrank_kv_ws(int64_t B, int64_t Sq, int64_t Hq, int64_t Hkv, int64_t D, int64_t L_max);
fsvd_status_t fsvd_decode_attn_lowrank_kv(const void* q, const void* zk_cache, const void* zv_cache, int64_t ldz,
                                          const void* Vt_k, int64_t r_k, const void* Vt_v, int64_t r_v,
                                          int64_t L_max, const int32_t* cache_seqlens, int64_t B, int64_t Sq,
                                          int64_t Hq, int64_t Hkv, int64_t D, float rope_theta,
                                          float softmax_scale, int causal, void* out, fsvd_dtype_t dtype,
                                          void* ws, size_t ws_bytes, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Factorised attention  [V1] [V15-M2]
 * Attention of S tokens per sequence among themselves with the Q, K and V tiles rebuilt on chip
 * from the rank-r activations, so the full-sequence q, k and v are never written:
 *   q[b, s, h] = RoPE(z_q[b, s] . Vt_q[h*D .. h*D+D-1]^T, position s)   (k likewise, kv head g),
 *   v[b, s, g] = z_v[b, s] . Vt_v[g*D .. g*D+D-1]^T,
 *   o[b, s, h] = sum_{j < n} softmax_j(scale * q[b, s, h] . k[b, j, g]) v[b, j, g],
 * with g = floor(h * Hkv / Hq) and n = s + 1 (causal) or S.  Each key tile is rebuilt once per
 * query tile that reads it (the recomputation that replaces materialising K and V).
 * zq, zk, zv [B * S, ldz] bf16 (row b * S + s; they may be column ranges of one packed z buffer,
 * 16-byte aligned); Vt_q [Hq*D, r_q], Vt_k [Hkv*D, r_k], Vt_v [Hkv*D, r_v] (stored ranks, multiples
 * of 8); out [B, S, Hq, D].  rope_theta 0 -> no RoPE; softmax_scale 0 -> 1/sqrt(D).  D 64 or 128,
 * Hq / Hkv in {1, 2, 4, 8}.  No workspace.  bf16 only.
 * ------------------------------------------------------------------------------------------ */
fsvd_status_t fsvd_attn_factorized(const void* zq, const void* zk, const void* zv, int64_t ldz, const void* Vt_q,
                                   int64_t r_q, const void* Vt_k, int64_t r_k, const void* Vt_v, int64_t r_v,
                                   int64_t B, int64_t S, int64_t Hq, int64_t Hkv, int64_t D, float rope_theta,
                                   float softmax_scale, int causal, void* out, fsvd_dtype_t dtype,
                                   fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * Swift-SVD factor production  [SWIFT-2A]
 * Activation-aware rank-k compression of a linear layer y = x . W (W [d_in, d_out]) from a
 * stream of calibration inputs X_t [T, d_in], in the page's order:
 *   1. fsvd_swift_covariance, once per batch: C += Y_t^T . Y_t with Y_t = X_t . W.  C is
 *      [d_out, d_out] fp32, accumulated across calls (the caller zero-fills it first); it is
 *      symmetric and only its upper triangle (column >= row, in whole tiles) is written.  Y_t
 *      is rounded to bf16 before the product; the products accumulate in fp32.
 *   2. the caller's eigendecomposition of C, eigenvalues descending: the top-k eigenvectors
 *      V_k [d_out, k] are the right singular vectors of Y = X . W.
 *   3. fsvd_swift_factors: W_k* = W . V_k . V_k^T as a factor pair in this library's storage,
 *      Ut = (W . V_k)^T [k, d_in] and Vt = V_k [d_out, k], from VkT = V_k^T [k, d_out] (bf16).
 * Wt = W^T [d_out, d_in] is the layer's weight in linear-layer storage (K-contiguous, like
 * Ut and Vt).  X [T, ldx].  T, d_in, d_out and k must be multiples of 8; ldc a multiple of 4.
 * The workspace holds Y_t^T [d_out, T] (covariance) or W [d_in, d_out] (factors).  bf16 inputs.
 * ------------------------------------------------------------------------------------------ */
size_t fsvd_swift_covariance_ws(int64_t T, int64_t d_in, int64_t d_out);
fsvd_status_t fsvd_swift_covariance(const void* X, int64_t T, int64_t d_in, int64_t ldx, const void* Wt,
                                    int64_t d_out, float* C, int64_t ldc, void* ws, size_t ws_bytes,
                                    fsvd_stream_t stream);
size_t fsvd_swift_factors_ws(int64_t d_in, int64_t d_out);
fsvd_status_t fsvd_swift_factors(const void* Wt, int64_t d_out, int64_t d_in, const void* VkT, int64_t k,
                                 void* Ut, void* Vt, void* ws, size_t ws_bytes, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * a7. Layer glue: y = LayerNorm(x + residual) * gamma + beta over rows of width d (BERT
 * post-norm); residual may be NULL; y may alias x.  bf16 only.  Llama-style RMSNorm is fused
 * into fsvd_lowrank_qkv / fsvd_lowrank_mlp_packed, residual adds into their epilogues.
 * ------------------------------------------------------------------------------------------ */
fsvd_status_t fsvd_layernorm(const void* x, const void* residual, const void* gamma, const void* beta,
                             float eps, int64_t M, int64_t d, void* y, fsvd_dtype_t dtype, fsvd_stream_t stream);

/* Comparator, not part of the layer path: the dense projection the factors replace, through the
 * same kernels as the low-rank linear's second phase ("FlashSVD v1.5" explainer, Results: the
 * low-rank path is measured against the model's dense weights).
 *   y[m, :] = residual[m, :] + bias + x[m, :] . W^T
 * x [M, K] (ldx), W [N, K] (ldw), bias [N] or NULL, residual [M, N] (ldr) or NULL (may alias y),
 * y [M, N] (ldy).  M <= 32 runs the row-dot kernels (bf16 launches of 5..32 rows on the matrix
 * cores, the reduction not split across workgroups); larger M the bf16 MFMA GEMM (bf16 only).
 * No workspace; argument errors are returned before anything is launched. */
fsvd_status_t fsvd_dense_linear(const void* x, int64_t M, int64_t K, int64_t ldx, const void* W, int64_t N,
                                int64_t ldw, const void* bias, const void* residual, int64_t ldr, void* y,
                                int64_t ldy, fsvd_dtype_t dtype, fsvd_stream_t stream);

/* Measurement helper, not part of the layer path: reads the bytes of src (rounded down to a
 * multiple of 16) once from HBM with 16-byte non-temporal loads over the whole chip, each
 * workgroup streaming one contiguous slice, so a timed call gives the read-stream bandwidth this
 * part sustains, the practical ceiling of the HBM-bound decode kernels.  out [64] uint32 (device)
 * receives an XOR of the data read (keeps the loads live; its value is meaningless). */
fsvd_status_t fsvd_read_stream_probe(const void* src, size_t bytes, void* out, fsvd_stream_t stream);

/* cache_seqlens[b] += n for b < B (one tiny kernel; also the optional last node of a graph). */
fsvd_status_t fsvd_seqlens_advance(int32_t* cache_seqlens, int64_t B, int32_t n, fsvd_stream_t stream);

/* ------------------------------------------------------------------------------------------
 * a7+a8. Whole Llama-style pre-norm decoder layer and its per-layer graph  [V15-M4]
 *   a = RMSNorm(x); q,k,v (RoPE, append) ; o = attention ; h = x + O(o) ;
 *   y = h + MLP(RMSNorm(h))
 * over S new tokens per sequence (S == 1 is a decode step; S > 1 a causal prefill that
 * appends at cache_seqlens[b]).  Every pointer in the descriptor is a device pointer that the
 * caller keeps alive (and, for a captured graph, at a fixed address) until the last use.
 * ------------------------------------------------------------------------------------------ */
/* flags: both RMSNorm weights are folded into A_qkv and A_gu (fsvd_prepack_colscale); the layer
 * applies RMSNorm without a weight and ignores attn_norm_w / mlp_norm_w */
#define FSVD_LAYER_NORM_FOLDED 0x1

typedef struct fsvd_decoder_layer_desc {
    int64_t B, S, d, Hq, Hkv, D, d_ff, L_max;
    int64_t r_q, r_k, r_v, r_o, r_g, r_u, r_d; /* stored (padded) ranks */
    float norm_eps, rope_theta, softmax_scale;  /* rope_theta 0 -> no RoPE; scale 0 -> 1/sqrt(D) */
    int32_t advance_seqlens;                    /* 1: cache_seqlens += S after the layer */
    int32_t flags;                              /* FSVD_LAYER_* bits, 0 by default */
    const void* x; /* [B, S, d] layer input */
    void* y;       /* [B, S, d] layer output (must not alias x) */
    const void* attn_norm_w;                    /* [d]; NULL: no norm (ignored when folded) */
    const void* mlp_norm_w;                     /* [d]; NULL: no norm (ignored when folded) */
    const void* A_qkv;                          /* [r_q + r_k + r_v, d] */
    const void *Vt_q, *Vt_k, *Vt_v;             /* [Hq*D, r_q], [Hkv*D, r_k], [Hkv*D, r_v] */
    const void *Ut_o, *Vt_o;                    /* [r_o, Hq*D], [d, r_o] */
    const void* A_gu;                           /* [r_g + r_u, d] */
    const void *Vt_g, *Vt_u;                    /* [d_ff, r_g], [d_ff, r_u] */
    const void *Ut_d, *Vt_d;                    /* [r_d, d_ff], [d, r_d] */
    void *k_cache, *v_cache;                    /* [B, L_max, Hkv, D] */
    int32_t* cache_seqlens;                     /* [B] */
    void* ws;
    size_t ws_bytes;
    /* S > 1 (prefill): the B * S token rows pass through the layer in ceil(B * S / prefill_chunk)
     * passes of nearly equal size, so the workspace holds one pass and does not grow with the
     * sequence; 0 -> 8192 rows, else at least 256.  The result does not depend on it. */
    int64_t prefill_chunk;
} fsvd_decoder_layer_desc;

typedef struct fsvd_graph fsvd_graph; /* opaque */

size_t fsvd_decoder_layer_ws(const fsvd_decoder_layer_desc* desc /*host*/);
/* Eager: launches the layer's kernels on stream (same kernels the graph holds). bf16 only. */
fsvd_status_t fsvd_decoder_layer_run(const fsvd_decoder_layer_desc* desc /*host*/, fsvd_stream_t stream);
/* Captures the layer (S must be 1) into a hipGraph on a library-owned capture stream and
 * instantiates it; synchronises the device once.  *out receives the graph handle (host). */
fsvd_status_t fsvd_decoder_layer_capture(const fsvd_decoder_layer_desc* desc /*host*/, fsvd_graph** out);
/* As fsvd_decoder_layer_capture for n_layers descriptors (host array) enqueued in order into ONE
 * graph: a whole decode step of a layer stack replayed with one hipGraphLaunch (the caller chains
 * layer l's y to layer l+1's x).  The per-layer graph is the pages' design; this variant removes
 * the per-graph launch boundary between layers. */
fsvd_status_t fsvd_decoder_stack_capture(const fsvd_decoder_layer_desc* descs /*host*/, int n_layers,
                                         fsvd_graph** out);
/* One hipGraphLaunch of the captured layer (or stack) on stream. */
fsvd_status_t fsvd_graph_replay(fsvd_graph* g, fsvd_stream_t stream);
fsvd_status_t fsvd_graph_destroy(fsvd_graph* g);

/* Reads (synchronising stream) and clears the device error word of a workspace; *code (host)
 * receives its value; returns FSVD_ERR_DEVICE when it was non-zero. */
fsvd_status_t fsvd_poll_device_error(void* ws, fsvd_stream_t stream, int32_t* code /*host*/);

#ifdef __cplusplus
}
#endif
#endif /* FSVD_H */
