"""Plain fp64 CPU oracle for the fused low-rank transformer-layer hot path.

TEST INFRASTRUCTURE.  Only the test suite, the package entry point's smoke check and the
benchmark's CPU-baseline leg may import this module.  It shares no code with the HIP path:
it imports numpy/scipy only, never the library, its binding or torch.

Every function takes host arrays (the exact values the GPU receives, already rounded to
float32 or bfloat16), widens them to float64 and never rounds an intermediate.  Where the
method reaches a result with a plain definition (re-associated products, a packed
projection, dense-KV attention), the function is that definition written out; the
Swift-SVD compression follows the page's steps in order.

Sources (by page title and section):
  [V15]  "FlashSVD v1.5: Making Low-Rank Transformers Inference Actually Fast"
         (gist.science explainer) - Problem Statement; Methodology 1 Unified Runtime
         Abstraction, 2 Dense-KV Attention, 3 Packed MLP Execution, 4 Per-Layer CUDA Graph
         Replay; Significance and Claims.
  [V1]   "FlashSVD: Memory-Efficient Inference with Streaming for Low-Rank Models"
         (abstract).
  [SWIFT] "Swift-SVD: Theoretical Optimality Meets Practical Efficiency in Low-Rank LLM
         Compression" (gist.science explainer) - 2A closed-form spectral solution.

Conventions the pages leave open (each is a stated reading, not a page fact):
  * row vectors, y = x U V, factors stored as Ut = U^T [r, d_in], Vt = V^T [d_out, r];
  * Llama pre-norm layer with RMSNorm and rotate-half RoPE, BERT post-norm layer with
    LayerNorm; SwiGLU t = SiLU(g) * u, GELU in its exact erf form;
  * a decode token is appended to the dense cache first and then attends to itself;
  * GQA maps query head h to kv head floor(h * Hkv / Hq).
The norm, RoPE and GQA conventions are pinned by closed forms and invariants in the tests,
not by the pages (the pages do not define them).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf as _erf

f64 = np.float64


def _a(x):
    return None if x is None else np.asarray(x, dtype=f64)


# ----------------------------------------------------------------------------- low-rank linear


def lowrank_linear(x, Ut, Vt, bias=None, residual=None):
    """y = residual + (x . U) . V + bias, U = Ut^T, V = Vt^T.

    [V1] abstract: the truncated factors of an SVD-compressed weight are applied in place of
    the dense weight; the fused kernels reach the same product ("no accuracy loss").
    [V15] Methodology 1: every checkpoint family maps to one factorized representation.
    x: [..., K]; Ut: [r, K]; Vt: [N, r]; bias: [N]; residual: [..., N].
    """
    x, Ut, Vt = _a(x), _a(Ut), _a(Vt)
    z = x @ Ut.T            # rank-r intermediate
    y = z @ Vt.T
    if bias is not None:
        y = y + _a(bias)
    if residual is not None:
        y = y + _a(residual)
    return y


def pack_rows(blocks, pad_to: int = 1):
    """Offline prepack: stack input-side factor blocks that share an input into one tensor.

    [V15] Methodology 3: compatible input-side factors are packed offline into a single
    tensor.  Each block's row count (its rank) is zero-padded up to a multiple of
    ``pad_to`` (exact: zero rows add zero terms).  Returns (packed, stored_ranks).
    """
    out, ranks = [], []
    for b in blocks:
        b = _a(b)
        rp = -(-b.shape[0] // pad_to) * pad_to
        pad = np.zeros((rp - b.shape[0], b.shape[1]), dtype=f64)
        out.append(np.vstack([b, pad]))
        ranks.append(rp)
    return np.vstack(out), ranks


def pad_cols(m, cols_to: int):
    """Zero-pad the columns (rank dimension of an output-side factor Vt) to ``cols_to``."""
    m = _a(m)
    return np.hstack([m, np.zeros((m.shape[0], cols_to - m.shape[1]), dtype=f64)])


# ----------------------------------------------------------------------------- layer glue


def rmsnorm(x, w, eps):
    """x / sqrt(mean(x^2) + eps) * w over the last axis (Llama convention; pages silent)."""
    x = _a(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * _a(w)


def layernorm(x, gamma, beta, eps):
    """(x - mean) / sqrt(var + eps) * gamma + beta over the last axis (BERT convention)."""
    x = _a(x)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _a(gamma) + _a(beta)


def rope(x, pos, theta):
    """Rotate-half rotary embedding of head vectors x [..., D] at integer positions pos [...].

    Pair (i, i + D/2), i < D/2, rotates by angle pos * theta^(-2i/D).
    """
    x = _a(x)
    D = x.shape[-1]
    half = D // 2
    inv = theta ** (-2.0 * np.arange(half, dtype=f64) / D)
    ang = np.asarray(pos, dtype=f64)[..., None] * inv
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(g):
    g = _a(g)
    return g / (1.0 + np.exp(-g))


def gelu(u):
    u = _a(u)
    return 0.5 * u * (1.0 + _erf(u / np.sqrt(2.0)))


# ----------------------------------------------------------------------------- Q/K/V with KV append


def qkv(x, norm_w, norm_eps, Ut_q, Vt_q, Ut_k, Vt_k, Ut_v, Vt_v, Hq, Hkv, D, rope_theta,
        k_cache, v_cache, cache_seqlens):
    """Current-token Q/K/V reconstruction and append to the dense cache.

    [V15] Methodology 2: dense Q, K, V are rebuilt only for the present tokens; K and V go
    into a standard contiguous dense KV cache.
    x: [B, S, d]; caches [B, L_max, Hkv, D]; cache_seqlens[b] = tokens already cached; new
    token s of sequence b lands at position p = cache_seqlens[b] + s.
    Returns q [B, S, Hq, D], k, v [B, S, Hkv, D] and the updated caches (copies).
    """
    x = _a(x)
    B, S, _ = x.shape
    a = rmsnorm(x, norm_w, norm_eps) if norm_w is not None else x
    q = lowrank_linear(a, Ut_q, Vt_q).reshape(B, S, Hq, D)
    k = lowrank_linear(a, Ut_k, Vt_k).reshape(B, S, Hkv, D)
    v = lowrank_linear(a, Ut_v, Vt_v).reshape(B, S, Hkv, D)
    pos = np.asarray(cache_seqlens, dtype=np.int64)[:, None] + np.arange(S)[None, :]   # [B, S]
    if rope_theta:
        q = rope(q, pos[:, :, None], rope_theta)
        k = rope(k, pos[:, :, None], rope_theta)
    kc, vc = _a(k_cache).copy(), _a(v_cache).copy()
    for b in range(B):
        for s in range(S):
            kc[b, pos[b, s]] = k[b, s]
            vc[b, pos[b, s]] = v[b, s]
    return q, k, v, kc, vc


def qkv_packed(x, norm_w, norm_eps, A_qkv, r_q, r_k, r_v, Vt_q, Vt_k, Vt_v, Hq, Hkv, D,
               rope_theta, k_cache, v_cache, cache_seqlens):
    """Same result via one wide projection z = a . A_qkv^T and a split of z at r_q, r_q+r_k.

    The packing of the Q/K/V input-side factors extends [V15] Methodology 3's gate/up
    packing to the three attention projections that share the same input.
    """
    A = _a(A_qkv)
    return qkv(x, norm_w, norm_eps, A[:r_q], Vt_q, A[r_q:r_q + r_k], Vt_k, A[r_q + r_k:r_q + r_k + r_v],
               Vt_v, Hq, Hkv, D, rope_theta, k_cache, v_cache, cache_seqlens)


def lowrank_history_kv(zk, zv, Vt_k, Vt_v, Hkv, D, rope_theta):
    """K and V of every cached position rebuilt from a rank-r history.

    [V15] Problem Statement: the layout that dense-KV decoding replaces keeps only the rank-r
    projections of past tokens, z_k = a . U_k and z_v = a . U_v, and reconstructs K and V from
    the factors at every step.  zk [B, L, r_k], zv [B, L, r_v] (position p of a sequence at row
    p); K rows are rotated by RoPE at their position.  Returns K, V [B, L, Hkv, D].
    """
    zk, zv = _a(zk), _a(zv)
    B, L, _ = zk.shape
    k = (zk @ _a(Vt_k).T).reshape(B, L, Hkv, D)
    v = (zv @ _a(Vt_v).T).reshape(B, L, Hkv, D)
    if rope_theta:
        k = rope(k, np.arange(L)[None, :, None], rope_theta)
    return k, v


# ----------------------------------------------------------------------------- MLP


def mlp(x, norm_w, norm_eps, act, Ut_g, Vt_g, Ut_u, Vt_u, Ut_d, Vt_d, residual=None):
    """Low-rank gated MLP: t = SiLU(g) * u (act='swiglu') or GELU(u) (act='gelu', no gate),
    y = residual + (t . Ut_d^T) . Vt_d^T with g, u the low-rank gate/up projections of
    b = RMSNorm(x) (or x when norm_w is None).  [V1] abstract (fused FFN); [V15] Methodology 3.
    """
    b = rmsnorm(x, norm_w, norm_eps) if norm_w is not None else _a(x)
    u = lowrank_linear(b, Ut_u, Vt_u)
    if act == "swiglu":
        g = lowrank_linear(b, Ut_g, Vt_g)
        t = silu(g) * u
    elif act == "gelu":
        t = gelu(u)
    else:
        raise ValueError(act)
    return lowrank_linear(t, Ut_d, Vt_d, residual=residual)


def mlp_packed(x, norm_w, norm_eps, act, A_gu, r_g, r_u, Vt_g, Vt_u, Ut_d, Vt_d, residual=None):
    """[V15] Methodology 3 packed execution: one wide projection z = b . A_gu^T with
    A_gu = [Ut_gate ; Ut_up] (gate rows first), then a split of the rank activations
    z_g = z[:, :r_g], z_u = z[:, r_g:r_g+r_u]; the rest as in ``mlp``."""
    b = rmsnorm(x, norm_w, norm_eps) if norm_w is not None else _a(x)
    z = b @ _a(A_gu).T
    z_g, z_u = z[..., :r_g], z[..., r_g:r_g + r_u]
    u = z_u @ _a(Vt_u).T
    if act == "swiglu":
        t = silu(z_g @ _a(Vt_g).T) * u
    else:
        t = gelu(u)
    return lowrank_linear(t, Ut_d, Vt_d, residual=residual)


# ----------------------------------------------------------------------------- dense-KV attention


def attention(q, k_cache, v_cache, cache_seqlens, causal, scale=None):
    """Attention of the Sq new tokens over the contiguous dense cache.

    [V15] Methodology 2: history is read contiguously from the dense cache in one attention
    step.  For token s of sequence b and query head h (kv head g = floor(h*Hkv/Hq)):
      n = cache_seqlens[b] + s + 1 (causal) or cache_seqlens[b] + Sq (non-causal),
      o = sum_{j<n} softmax_j(scale * q . k_j) v_j,   scale = 1/sqrt(D) by default.
    cache_seqlens holds the length BEFORE the Sq new tokens were appended.
    q: [B, Sq, Hq, D]; caches [B, L_max, Hkv, D]; returns o [B, Sq, Hq, D].
    """
    q, kc, vc = _a(q), _a(k_cache), _a(v_cache)
    B, Sq, Hq, D = q.shape
    Hkv = kc.shape[2]
    if scale is None or scale == 0:
        scale = 1.0 / np.sqrt(D)
    o = np.zeros_like(q)
    for b in range(B):
        base = int(cache_seqlens[b])
        for s in range(Sq):
            n = base + s + 1 if causal else base + Sq
            for h in range(Hq):
                g = (h * Hkv) // Hq
                sc = scale * (kc[b, :n, g, :] @ q[b, s, h])
                w = np.exp(sc - sc.max())
                o[b, s, h] = (w / w.sum()) @ vc[b, :n, g, :]
    return o


def attention_matrix(Q, K, V, scale=None, mask=None):
    """Naive softmax(Q K^T * scale) V for one head: Q [Sq, D], K, V [n, D]; mask [Sq, n] bool
    (True = attend).  The textbook matrix form the dense-KV step must reproduce."""
    Q, K, V = _a(Q), _a(K), _a(V)
    if scale is None:
        scale = 1.0 / np.sqrt(Q.shape[-1])
    S = scale * (Q @ K.T)
    if mask is not None:
        S = np.where(mask, S, -np.inf)
    P = np.exp(S - S.max(axis=-1, keepdims=True))
    P = P / P.sum(axis=-1, keepdims=True)
    return P @ V


def attention_partitioned(qv, K, V, bounds, scale=None):
    """One query vector over K, V [n, D] split into position ranges [bounds[i], bounds[i+1]),
    each reduced to (max, sum of exp, unnormalised output) and merged by log-sum-exp.
    Used to show the split-length reformulation of the single softmax is exact."""
    qv, K, V = _a(qv), _a(K), _a(V)
    if scale is None:
        scale = 1.0 / np.sqrt(qv.shape[-1])
    parts = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        if hi <= lo:
            continue
        sc = scale * (K[lo:hi] @ qv)
        m = sc.max()
        e = np.exp(sc - m)
        parts.append((m, e.sum(), e @ V[lo:hi]))
    M = max(p[0] for p in parts)
    den = sum(np.exp(m - M) * l for m, l, _ in parts)
    num = sum(np.exp(m - M) * acc for m, _, acc in parts)
    return num / den


# ----------------------------------------------------------------------------- whole layers


def decoder_layer(x, p, cfg, k_cache, v_cache, cache_seqlens, causal=True):
    """Llama-style pre-norm layer over S new tokens per sequence:
        a = RMSNorm(x); q, k, v = low-rank projections (RoPE on q, k; k, v appended);
        h = x + O(attention);  y = h + MLP(RMSNorm(h)).
    x: [B, S, d]; p: dict of factors (Ut_*/Vt_* for q,k,v,o,gate,up,down) and norm weights.
    Returns (y, k_cache', v_cache') - the caches with the new tokens appended."""
    x = _a(x)
    B, S, d = x.shape
    q, _, _, kc, vc = qkv(x, p["attn_norm_w"], cfg.norm_eps, p["Ut_q"], p["Vt_q"], p["Ut_k"], p["Vt_k"],
                          p["Ut_v"], p["Vt_v"], cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta,
                          k_cache, v_cache, cache_seqlens)
    o = attention(q, kc, vc, cache_seqlens, causal=causal)
    h = lowrank_linear(o.reshape(B, S, cfg.Hq * cfg.D), p["Ut_o"], p["Vt_o"], residual=x)
    y = mlp(h, p["mlp_norm_w"], cfg.norm_eps, "swiglu", p["Ut_gate"], p["Vt_gate"], p["Ut_up"], p["Vt_up"],
            p["Ut_down"], p["Vt_down"], residual=h)
    return y, kc, vc


def decoder_steps(x_steps, p, cfg, k_cache, v_cache, cache_seqlens):
    """N successive single-token decode steps of one layer: step t feeds x_steps[t] [B, d],
    appends at cache_seqlens + t.  Returns (y [N, B, d], caches, final seqlens).
    [V15] Methodology 4: the replayed per-layer graph repeats exactly this step."""
    kc, vc = _a(k_cache), _a(v_cache)
    sl = np.asarray(cache_seqlens, dtype=np.int64).copy()
    ys = []
    for xt in np.asarray(x_steps):
        y, kc, vc = decoder_layer(np.asarray(xt)[:, None, :], p, cfg, kc, vc, sl, causal=True)
        ys.append(y[:, 0, :])
        sl = sl + 1
    return np.stack(ys), kc, vc, sl


def encoder_layer(x, p, cfg):
    """BERT-style post-norm layer (no RoPE, bidirectional attention over the S tokens):
        h = LN(x + O(attention(q, k, v)));  y = LN(h + down(GELU(up(h)))).
    K/V are written into a fresh dense buffer [B, S, H, D] (cache length 0)."""
    x = _a(x)
    B, S, d = x.shape
    H, D = cfg.H, cfg.D
    zero = np.zeros((B, S, H, D))
    sl0 = np.zeros(B, dtype=np.int64)
    q, _, _, kc, vc = qkv(x, None, 0.0, p["Ut_q"], p["Vt_q"], p["Ut_k"], p["Vt_k"], p["Ut_v"], p["Vt_v"],
                          H, H, D, 0.0, zero, zero, sl0)
    o = attention(q, kc, vc, sl0, causal=False)
    h = layernorm(lowrank_linear(o.reshape(B, S, H * D), p["Ut_o"], p["Vt_o"], residual=x),
                  p["ln1_g"], p["ln1_b"], cfg.ln_eps)
    f = mlp(h, None, 0.0, "gelu", None, None, p["Ut_up"], p["Vt_up"], p["Ut_down"], p["Vt_down"], residual=h)
    return layernorm(f, p["ln2_g"], p["ln2_b"], cfg.ln_eps)


# ----------------------------------------------------------------------------- Swift-SVD


def swift_svd(X_batches, W, k):
    """Activation-aware closed-form rank-k compression, in the page's order ([SWIFT] 2A):

      1. incremental aggregation: C <- C + y_t^T y_t with y_t = x_t W over the batches;
      2. one eigendecomposition of C gives the squared singular values and right singular
         vectors of Y = X W (sorted descending; rounding negatives clamped to 0);
      3. W_k* = W V_k V_k^T, stored as the factor pair U = W V_k, V = V_k^T.
    Minimises ||X W - X W_k||_F over rank-k W_k.
    """
    W = _a(W)
    C = np.zeros((W.shape[1], W.shape[1]), dtype=f64)
    for Xt in X_batches:
        Yt = _a(Xt) @ W
        C += Yt.T @ Yt
    lam, vecs = np.linalg.eigh(C)
    order = np.argsort(lam)[::-1]
    lam = np.clip(lam[order], 0.0, None)
    vecs = vecs[:, order]
    Vk = vecs[:, :k]
    return {"C": C, "lam": lam, "sigma": np.sqrt(lam), "Vk": Vk, "Wk": W @ Vk @ Vk.T,
            "U": W @ Vk, "V": Vk.T}
