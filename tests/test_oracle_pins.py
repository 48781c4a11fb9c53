"""CPU pins of the fp64 oracle against what the pages and the mathematics fix.

Each ``pin_*`` function checks one property and raises AssertionError when it fails.  The
tests run every pin on the real oracle (must pass) and a few pins on planted mistakes in the
oracle (a dropped term, a wrong sign or index, a transposed operand; must fail), so the pins
are shown to have teeth.  Tolerances: 1e-12 relative for re-associated products, 1e-10 for
decomposition-based checks.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import fsvd_oracle as O
from oracle import loops as L
from svd_compressed_transformer_amd import inputs as I

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    den = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (den if den > 0 else 1.0))


# ============================================================================ low-rank linear


def pin_lowrank_bruteforce(O):
    rng = np.random.default_rng(11)
    x, Ut, Vt = rng.standard_normal((3, 5)), rng.standard_normal((2, 5)), rng.standard_normal((4, 2))
    bias, res = rng.standard_normal(4), rng.standard_normal((3, 4))
    y = O.lowrank_linear(x, Ut, Vt, bias=bias, residual=res)
    assert rel(y, L.lowrank_linear(x, Ut, Vt, bias=bias, residual=res)) <= 1e-12
    # re-association: (x U) V == x (U V) with the dense W = U V written by loops
    W = L.matmul(L.transpose(Ut), L.transpose(Vt))
    assert rel(O.lowrank_linear(x, Ut, Vt), L.matmul(x, W)) <= 1e-12


def pin_lowrank_golden(O):
    g = _load("lowrank_tiny.json")
    assert rel(O.lowrank_linear(g["x"], g["Ut"], g["Vt"]), g["y_plain"]) == 0.0
    assert rel(O.lowrank_linear(g["x"], g["Ut"], g["Vt"], bias=g["bias"], residual=g["residual"]), g["y_full"]) == 0.0
    assert rel(np.asarray(g["x"]) @ np.asarray(g["W_dense"]), g["y_plain"]) == 0.0


def pin_lowrank_fullrank_svd(O):
    """A full-rank factorisation from an exact SVD reproduces the dense W."""
    rng = np.random.default_rng(12)
    for m, n in ((6, 5), (5, 7), (8, 8)):
        W = rng.standard_normal((m, n))
        A, s, Bt = np.linalg.svd(W, full_matrices=False)
        Ut = (A * s).T                  # U = A diag(s), r = min(m, n)
        Vt = Bt.T                       # V = B^T
        assert rel(O.lowrank_linear(np.eye(m), Ut, Vt), W) <= 1e-10


def pin_lowrank_eckart_young(O):
    """Truncating the SVD at r leaves ||W - U_r V_r||_F^2 = sum_{i>r} s_i^2."""
    rng = np.random.default_rng(13)
    W = rng.standard_normal((9, 7))
    A, s, Bt = np.linalg.svd(W, full_matrices=False)
    for r in range(1, 7):
        Wr = O.lowrank_linear(np.eye(9), (A[:, :r] * s[:r]).T, Bt[:r].T)
        e2 = np.sum((W - Wr) ** 2)
        assert abs(e2 - np.sum(s[r:] ** 2)) <= 1e-10 * np.sum(s ** 2)


def pin_zero_padding(O):
    rng = np.random.default_rng(14)
    x, Ut, Vt = rng.standard_normal((4, 10)), rng.standard_normal((5, 10)), rng.standard_normal((6, 5))
    P, ranks = O.pack_rows([Ut], pad_to=8)
    assert ranks == [8] and P.shape == (8, 10) and np.all(P[5:] == 0)
    Vp = O.pad_cols(Vt, 8)
    assert Vp.shape == (6, 8) and np.all(Vp[:, 5:] == 0)
    assert rel(O.lowrank_linear(x, P, Vp), O.lowrank_linear(x, Ut, Vt)) <= 1e-13


# ============================================================================ glue: norms, RoPE, activations


def pin_rmsnorm(O):
    rng = np.random.default_rng(21)
    x, w = rng.standard_normal((3, 16)), 1 + 0.1 * rng.standard_normal(16)
    y = O.rmsnorm(x, w, 1e-6)
    for i in range(3):
        assert rel(y[i], L.rmsnorm_row(x[i], w, 1e-6)) <= 1e-12
    y0 = O.rmsnorm(x, np.ones(16), 0.0)
    assert np.allclose(np.sqrt(np.mean(y0 ** 2, axis=-1)), 1.0, atol=1e-12)       # unit RMS
    assert rel(O.rmsnorm(7.5 * x, np.ones(16), 0.0), y0) <= 1e-12                # scale invariant
    assert rel(O.rmsnorm(np.full((1, 4), -3.0), np.ones(4), 0.0), -np.ones((1, 4))) <= 1e-15


def pin_layernorm(O):
    rng = np.random.default_rng(22)
    x = 3 + 2 * rng.standard_normal((4, 32))
    y = O.layernorm(x, np.ones(32), np.zeros(32), 0.0)
    assert np.allclose(y.mean(-1), 0, atol=1e-12) and np.allclose(y.var(-1), 1, atol=1e-12)
    g, b = rng.standard_normal(32), rng.standard_normal(32)
    assert rel(O.layernorm(x, g, b, 0.0), y * g + b) <= 1e-12
    assert rel(O.layernorm(x + 100.0, np.ones(32), np.zeros(32), 0.0), y) <= 1e-10  # shift invariant


def pin_rope(O):
    rng = np.random.default_rng(23)
    D = 8
    x = rng.standard_normal(D)
    assert rel(O.rope(x, 0, 1e4), x) == 0.0                                          # identity at p = 0
    for p in (1, 5, 1000):
        y = O.rope(x, p, 1e4)
        assert rel(y, L.rope_vec(x, p, 1e4)) <= 1e-12
        h = D // 2
        assert np.allclose(y[:h] ** 2 + y[h:] ** 2, x[:h] ** 2 + x[h:] ** 2, rtol=1e-12)  # per-pair norm
    # D = 2: plain rotation by angle p (theta irrelevant); quarter turn maps (a, b) -> (-b, a)
    assert rel(O.rope(np.array([2.0, 5.0]), math.pi / 2, 1e4), [-5.0, 2.0]) <= 1e-15
    # relative-position property: <rope(q, p1), rope(k, p2)> depends only on p1 - p2
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    d1 = O.rope(q, 17, 1e4) @ O.rope(k, 10, 1e4)
    d2 = O.rope(q, 107, 1e4) @ O.rope(k, 100, 1e4)
    assert abs(d1 - d2) <= 1e-10 * (abs(d1) + 1)


def pin_activations(O):
    assert O.silu(0.0) == 0.0 and O.gelu(0.0) == 0.0
    assert abs(O.silu(1.0) - 0.7310585786300049) <= 1e-15          # 1 / (1 + e^-1)
    assert abs(O.gelu(1.0) - 0.8413447460685429) <= 1e-15          # Phi(1), standard normal CDF
    assert abs(O.silu(40.0) - 40.0) <= 1e-12 and abs(O.gelu(40.0) - 40.0) <= 1e-12
    s = O.silu(-40.0)
    assert s < 0 and abs(s) <= 1e-15
    x = np.linspace(-3, 3, 13)
    assert rel(O.gelu(-x), -x + O.gelu(x)) <= 1e-14                # Phi(-x) = 1 - Phi(x)


# ============================================================================ attention


def pin_attention_matrix(O):
    """Dense-KV attention equals naive softmax(QK^T/sqrt(D))V with the causal mask."""
    rng = np.random.default_rng(31)
    B, Sq, Hq, Hkv, D, Lmax = 2, 3, 4, 2, 8, 12
    seqlens = np.array([4, 6])
    q = rng.standard_normal((B, Sq, Hq, D))
    kc, vc = rng.standard_normal((B, Lmax, Hkv, D)), rng.standard_normal((B, Lmax, Hkv, D))
    for causal in (True, False):
        o = O.attention(q, kc, vc, seqlens, causal=causal)
        for b in range(B):
            n = seqlens[b] + Sq
            for h in range(Hq):
                g = h * Hkv // Hq
                mask = None
                if causal:
                    mask = np.arange(n)[None, :] <= (seqlens[b] + np.arange(Sq))[:, None]
                ref = O.attention_matrix(q[b, :, h], kc[b, :n, g], vc[b, :n, g], mask=mask)
                assert rel(o[b, :, h], ref) <= 1e-12
                for s in range(Sq):
                    nn = seqlens[b] + s + 1 if causal else n
                    lp = L.softmax_attention_one(q[b, s, h], kc[b, :nn, g], vc[b, :nn, g], 1 / math.sqrt(D))
                    assert rel(o[b, s, h], lp) <= 1e-12


def pin_attention_special(O):
    rng = np.random.default_rng(32)
    D, Lmax = 8, 10
    q = rng.standard_normal((1, 1, 2, D))
    kc, vc = rng.standard_normal((1, Lmax, 1, D)), rng.standard_normal((1, Lmax, 1, D))
    # n = 1 (empty history, the token attends only to itself): o = v_0
    o = O.attention(q, kc, vc, [0], causal=True)
    assert rel(o[0, 0, 0], vc[0, 0, 0]) <= 1e-15
    # identical keys: uniform weights, o = mean(v)
    kc2 = np.repeat(kc[:, :1], Lmax, axis=1)
    o = O.attention(q, kc2, vc, [6], causal=True)
    assert rel(o[0, 0, 1], vc[0, :7, 0].mean(0)) <= 1e-12
    # very large scale: o -> v at the argmax score
    o = O.attention(q, kc, vc, [6], causal=True, scale=1e4)
    j = int(np.argmax(kc[0, :7, 0] @ q[0, 0, 0]))
    assert rel(o[0, 0, 0], vc[0, j, 0]) <= 1e-9
    # golden hand example
    g = _load("attention_tiny.json")
    k = np.array([[0.0, 0.0], [math.sqrt(2) * math.log(3), 0.0]])
    o = O.attention(np.array(g["q"])[None, None, None], k[None, :, None], np.array(g["v"])[None, :, None], [1], True)
    assert rel(o[0, 0, 0], g["o"]) <= 1e-14


def pin_attention_split_merge(O):
    """Any split of the positions merged by log-sum-exp equals the single softmax."""
    rng = np.random.default_rng(33)
    n, D = 37, 16
    qv, K, V = 3 * rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    ref = O.attention_matrix(qv[None], K, V)[0]
    for bounds in ([0, n], [0, 5, 37], [0, 10, 20, 30, 37], [0, 0, 3, 37, 37], list(range(0, 38))):
        assert rel(O.attention_partitioned(qv, K, V, bounds), ref) <= 1e-12


def pin_attention_gqa(O):
    rng = np.random.default_rng(34)
    B, Sq, Hq, D, Lmax = 1, 2, 8, 4, 9
    q = rng.standard_normal((B, Sq, Hq, D))
    for Hkv in (1, 2, 4):
        kc, vc = rng.standard_normal((B, Lmax, Hkv, D)), rng.standard_normal((B, Lmax, Hkv, D))
        rep = Hq // Hkv
        o_gqa = O.attention(q, kc, vc, [5], causal=True)
        o_mha = O.attention(q, np.repeat(kc, rep, axis=2), np.repeat(vc, rep, axis=2), [5], causal=True)
        assert rel(o_gqa, o_mha) == 0.0
    kc, vc = rng.standard_normal((B, Lmax, Hq, D)), rng.standard_normal((B, Lmax, Hq, D))
    o = O.attention(q, kc, vc, [5], causal=True)                 # Hkv = Hq: head h uses kv head h
    for h in range(Hq):
        assert rel(o[0, 1, h], O.attention_matrix(q[0, 1:, h], kc[0, :7, h], vc[0, :7, h])[0]) <= 1e-12


# ============================================================================ Q/K/V, MLP, packing


def _small_decoder():
    return I.scaled_decoder(I.CFG2, d=32, Hq=4, Hkv=2, D=8, d_ff=48,
                            ranks={"q": 12, "k": 6, "v": 5, "o": 10, "gate": 9, "up": 11, "down": 7})


def pin_qkv_append_and_packing(O):
    cfg = _small_decoder()
    p = I.make_decoder_layer(cfg, B=2, S=3, seed=5, dtype="bf16", random_norm_weights=True)
    Lmax = 10
    kc0 = np.full((2, Lmax, cfg.Hkv, cfg.D), 7.25)
    vc0 = np.full((2, Lmax, cfg.Hkv, cfg.D), -1.5)
    sl = np.array([2, 5])
    q, k, v, kc, vc = O.qkv(p["x"], p["attn_norm_w"], cfg.norm_eps, p["Ut_q"], p["Vt_q"], p["Ut_k"], p["Vt_k"],
                            p["Ut_v"], p["Vt_v"], cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta, kc0, vc0, sl)
    for b in range(2):
        for pos in range(Lmax):
            s = pos - sl[b]
            if 0 <= s < 3:
                assert np.array_equal(kc[b, pos], k[b, s]) and np.array_equal(vc[b, pos], v[b, s])
            else:
                assert np.all(kc[b, pos] == 7.25) and np.all(vc[b, pos] == -1.5)
    # q equals RoPE of the plain low-rank product of the normalised input at position sl+s
    a = O.rmsnorm(p["x"], p["attn_norm_w"], cfg.norm_eps)
    qp = O.lowrank_linear(a, p["Ut_q"], p["Vt_q"]).reshape(2, 3, cfg.Hq, cfg.D)
    for b in range(2):
        for s in range(3):
            for h in range(cfg.Hq):
                assert rel(q[b, s, h], L.rope_vec(qp[b, s, h], sl[b] + s, cfg.rope_theta)) <= 1e-12
    # v carries no RoPE
    assert rel(v, O.lowrank_linear(a, p["Ut_v"], p["Vt_v"]).reshape(2, 3, cfg.Hkv, cfg.D)) <= 1e-13
    # packed (and zero-padded) input factors give the same result
    A, (rq, rk, rv) = O.pack_rows([p["Ut_q"], p["Ut_k"], p["Ut_v"]], pad_to=8)
    res = O.qkv_packed(p["x"], p["attn_norm_w"], cfg.norm_eps, A, rq, rk, rv,
                       O.pad_cols(p["Vt_q"], rq), O.pad_cols(p["Vt_k"], rk), O.pad_cols(p["Vt_v"], rv),
                       cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta, kc0, vc0, sl)
    for a_, b_ in zip(res, (q, k, v, kc, vc)):
        assert rel(a_, b_) <= 1e-13


def pin_lowrank_history_rebuild(O):
    """K/V rebuilt from the cached rank-r rows z_k, z_v equal what the current-token path appended
    to the dense cache for the same tokens (the two layouts hold the same history)."""
    cfg = _small_decoder()
    B, S = 2, 6
    p = I.make_decoder_layer(cfg, B=B, S=S, seed=9, dtype="bf16", random_norm_weights=True)
    z0 = np.zeros((B, S, cfg.Hkv, cfg.D))
    _, _, _, kc, vc = O.qkv(p["x"], p["attn_norm_w"], cfg.norm_eps, p["Ut_q"], p["Vt_q"], p["Ut_k"], p["Vt_k"],
                            p["Ut_v"], p["Vt_v"], cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta, z0, z0, np.zeros(B))
    a = O.rmsnorm(p["x"], p["attn_norm_w"], cfg.norm_eps)
    zk = a @ np.asarray(p["Ut_k"], dtype=float).T
    zv = a @ np.asarray(p["Ut_v"], dtype=float).T
    K, V = O.lowrank_history_kv(zk, zv, p["Vt_k"], p["Vt_v"], cfg.Hkv, cfg.D, cfg.rope_theta)
    assert rel(K, kc) <= 1e-12 and rel(V, vc) <= 1e-12
    # without RoPE, K is the plain product
    K0, _ = O.lowrank_history_kv(zk, zv, p["Vt_k"], p["Vt_v"], cfg.Hkv, cfg.D, 0.0)
    assert rel(K0, (zk @ np.asarray(p["Vt_k"], dtype=float).T).reshape(B, S, cfg.Hkv, cfg.D)) <= 1e-14
    # position p of the history is rotated at p: the first position is unrotated
    assert rel(K[:, 0], K0[:, 0]) <= 1e-14


def pin_mlp_packed(O):
    cfg = _small_decoder()
    p = I.make_decoder_layer(cfg, B=2, S=2, seed=6, dtype="bf16", random_norm_weights=True)
    x = p["x"].reshape(4, cfg.d)
    y = O.mlp(x, p["mlp_norm_w"], cfg.norm_eps, "swiglu", p["Ut_gate"], p["Vt_gate"], p["Ut_up"], p["Vt_up"],
              p["Ut_down"], p["Vt_down"], residual=x)
    A, (rg, ru) = O.pack_rows([p["Ut_gate"], p["Ut_up"]], pad_to=8)
    yp = O.mlp_packed(x, p["mlp_norm_w"], cfg.norm_eps, "swiglu", A, rg, ru, O.pad_cols(p["Vt_gate"], rg),
                      O.pad_cols(p["Vt_up"], ru), p["Ut_down"], p["Vt_down"], residual=x)
    assert rel(yp, y) <= 1e-13
    # written out term by term
    b = O.rmsnorm(x, p["mlp_norm_w"], cfg.norm_eps)
    g = L.lowrank_linear(b, p["Ut_gate"], p["Vt_gate"])
    u = L.lowrank_linear(b, p["Ut_up"], p["Vt_up"])
    t = [[gi / (1 + math.exp(-gi)) * ui for gi, ui in zip(gr, ur)] for gr, ur in zip(g, u)]
    ref = L.lowrank_linear(t, p["Ut_down"], p["Vt_down"], residual=x)
    assert rel(y, ref) <= 1e-12
    # GELU variant (no gate)
    yg = O.mlp(x, None, 0, "gelu", None, None, p["Ut_up"], p["Vt_up"], p["Ut_down"], p["Vt_down"])
    u2 = np.asarray(L.lowrank_linear(x, p["Ut_up"], p["Vt_up"]))
    t2 = [[0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in row] for row in u2]
    assert rel(yg, L.lowrank_linear(t2, p["Ut_down"], p["Vt_down"])) <= 1e-12


# ============================================================================ whole layers


def pin_prefill_then_decode(O):
    """Prefill of S tokens then N single-token decode steps equals one causal prefill of S+N
    tokens on the new tokens' outputs (dense-KV decode reads the same history)."""
    cfg = _small_decoder()
    B, S, N, Lmax = 2, 5, 3, 12
    p = I.make_decoder_layer(cfg, B=B, S=S + N, seed=7, dtype="bf16", random_norm_weights=True)
    kc0 = np.zeros((B, Lmax, cfg.Hkv, cfg.D))
    vc0 = np.zeros_like(kc0)
    y_all, kc_all, vc_all = O.decoder_layer(p["x"], p, cfg, kc0, vc0, np.zeros(B, dtype=np.int64))
    y_pre, kc, vc = O.decoder_layer(p["x"][:, :S], p, cfg, kc0, vc0, np.zeros(B, dtype=np.int64))
    assert rel(y_pre, y_all[:, :S]) <= 1e-10
    ys, kc, vc, sl = O.decoder_steps(np.transpose(p["x"][:, S:], (1, 0, 2)), p, cfg, kc, vc, [S, S])
    assert list(sl) == [S + N, S + N]
    assert rel(np.transpose(ys, (1, 0, 2)), y_all[:, S:]) <= 1e-10
    assert rel(kc, kc_all) <= 1e-10 and rel(vc, vc_all) <= 1e-10


def _decoder_token_loops(x_row, p, cfg, pos, K_hist, V_hist):
    """One token of the pre-norm decoder layer written out with the pure-Python loops: RMSNorm,
    the three low-rank projections, RoPE at ``pos`` on q and k, the new k/v appended to the
    per-kv-head history lists K_hist[g], V_hist[g] (mutated), softmax attention over the whole
    history, then h = x + O(o) and y = h + down(SiLU(gate(n)) * up(n)) with n = RMSNorm(h).
    FlashSVD v1.5 explainer, Methodology 2 (current-token Q/K/V, dense history) and 3 (MLP)."""
    D, Hq, Hkv = cfg.D, cfg.Hq, cfg.Hkv
    a = L.rmsnorm_row(x_row, p["attn_norm_w"], cfg.norm_eps)
    q = L.lowrank_linear([a], p["Ut_q"], p["Vt_q"])[0]
    k = L.lowrank_linear([a], p["Ut_k"], p["Vt_k"])[0]
    v = L.lowrank_linear([a], p["Ut_v"], p["Vt_v"])[0]
    for g in range(Hkv):
        K_hist[g].append(L.rope_vec(k[g * D:(g + 1) * D], pos, cfg.rope_theta))
        V_hist[g].append(list(v[g * D:(g + 1) * D]))
    o = []
    for h in range(Hq):
        g = h * Hkv // Hq
        qh = L.rope_vec(q[h * D:(h + 1) * D], pos, cfg.rope_theta)
        o += L.softmax_attention_one(qh, K_hist[g], V_hist[g], 1.0 / math.sqrt(D))
    hrow = L.lowrank_linear([o], p["Ut_o"], p["Vt_o"], residual=[list(map(float, x_row))])[0]
    n = L.rmsnorm_row(hrow, p["mlp_norm_w"], cfg.norm_eps)
    gt = L.lowrank_linear([n], p["Ut_gate"], p["Vt_gate"])[0]
    up = L.lowrank_linear([n], p["Ut_up"], p["Vt_up"])[0]
    t = [gi / (1.0 + math.exp(-gi)) * ui for gi, ui in zip(gt, up)]
    return L.lowrank_linear([t], p["Ut_down"], p["Vt_down"], residual=[hrow])[0]


def pin_decoder_layer(O):
    """The decoder-layer composition written out token by token with the loops: one decode step
    over a cached history, a small causal prefill that starts mid-cache, and two successive decode
    steps of ``decoder_steps``; outputs and the appended cache rows at 1e-10."""
    cfg = _small_decoder()
    rng = np.random.default_rng(31)
    B, Lmax = 2, 12
    p = I.make_decoder_layer(cfg, B=B, S=4, seed=17, dtype="bf16", random_norm_weights=True)
    kc0 = I.round_bf16(rng.standard_normal((B, Lmax, cfg.Hkv, cfg.D)))
    vc0 = I.round_bf16(rng.standard_normal((B, Lmax, cfg.Hkv, cfg.D)))

    def run_loops(x, sl):
        Bx, S, _ = np.asarray(x).shape
        y = np.zeros((Bx, S, cfg.d))
        kc, vc = np.array(kc0, dtype=float), np.array(vc0, dtype=float)
        for b in range(Bx):
            K = [[list(kc0[b, j, g]) for j in range(int(sl[b]))] for g in range(cfg.Hkv)]
            V = [[list(vc0[b, j, g]) for j in range(int(sl[b]))] for g in range(cfg.Hkv)]
            for s in range(S):
                pos = int(sl[b]) + s
                y[b, s] = _decoder_token_loops(x[b, s], p, cfg, pos, K, V)
                for g in range(cfg.Hkv):
                    kc[b, pos, g], vc[b, pos, g] = K[g][-1], V[g][-1]
        return y, kc, vc

    for S, sl in ((1, np.array([3, 7])), (4, np.array([0, 5]))):
        x = p["x"][:, :S]
        y, kc, vc = O.decoder_layer(x, p, cfg, kc0, vc0, sl)
        y_l, kc_l, vc_l = run_loops(x, sl)
        assert rel(y, y_l) <= 1e-10, S
        assert rel(kc, kc_l) <= 1e-10 and rel(vc, vc_l) <= 1e-10
    # two decode steps: the second reads the first one's appended row
    sl = np.array([2, 6])
    xs = np.transpose(p["x"][:, :2], (1, 0, 2))
    ys, kc, vc, sl2 = O.decoder_steps(xs, p, cfg, kc0, vc0, sl)
    y_l, kc_l, vc_l = run_loops(p["x"][:, :2], sl)
    assert list(sl2) == list(sl + 2)
    assert rel(np.transpose(ys, (1, 0, 2)), y_l) <= 1e-10
    assert rel(kc, kc_l) <= 1e-10 and rel(vc, vc_l) <= 1e-10


def pin_encoder_layer(O):
    cfg = I.EncoderLayerConfig(name="tiny-bert", d=16, H=2, D=8, d_ff=24,
                               ranks={"q": 8, "k": 8, "v": 8, "o": 8, "up": 8, "down": 8})
    p = I.make_encoder_layer(cfg, B=2, S=5, seed=8, dtype="bf16")
    y = O.encoder_layer(p["x"], p, cfg)
    # written out with the matrix attention form and loops for the projections
    x = p["x"]
    for b in range(2):
        q = np.asarray(L.lowrank_linear(x[b], p["Ut_q"], p["Vt_q"]))
        k = np.asarray(L.lowrank_linear(x[b], p["Ut_k"], p["Vt_k"]))
        v = np.asarray(L.lowrank_linear(x[b], p["Ut_v"], p["Vt_v"]))
        o = np.concatenate([O.attention_matrix(q[:, h * 8:(h + 1) * 8], k[:, h * 8:(h + 1) * 8],
                                               v[:, h * 8:(h + 1) * 8]) for h in range(2)], axis=1)
        h1 = O.layernorm(np.asarray(L.lowrank_linear(o, p["Ut_o"], p["Vt_o"], residual=x[b])),
                         p["ln1_g"], p["ln1_b"], cfg.ln_eps)
        u = np.asarray(L.lowrank_linear(h1, p["Ut_up"], p["Vt_up"]))
        t = 0.5 * u * (1 + np.vectorize(math.erf)(u / math.sqrt(2)))
        f = np.asarray(L.lowrank_linear(t, p["Ut_down"], p["Vt_down"], residual=h1))
        assert rel(y[b], O.layernorm(f, p["ln2_g"], p["ln2_b"], cfg.ln_eps)) <= 1e-10


# ============================================================================ Swift-SVD


def pin_swift_golden(O):
    for c in _load("swift_svd_2x2.json")["cases"]:
        res = O.swift_svd([np.array(c["X"], dtype=float)], np.array(c["W"], dtype=float), c["k"])
        assert rel(res["lam"], c["lam"]) <= 1e-12
        assert rel(res["Wk"], c["Wk"]) <= 1e-12
        X = np.array(c["X"], dtype=float)
        e2 = np.sum((X @ np.array(c["W"]) - X @ res["Wk"]) ** 2)
        assert abs(e2 - c["err2"]) <= 1e-10
    # the rank-deficient case: the data-independent truncation is strictly worse on X
    c = _load("swift_svd_2x2.json")["cases"][1]
    X, W = np.array(c["X"], dtype=float), np.array(c["W"], dtype=float)
    A, s, Bt = np.linalg.svd(W)
    W1 = s[0] * np.outer(A[:, 0], Bt[0])
    assert np.sum((X @ W - X @ W1) ** 2) > 1e-3


def pin_swift_closed_form(O):
    rng = np.random.default_rng(41)
    d_in, d_out, k = 12, 9, 4
    # activations with a decaying spectrum, in 5 batches
    mix = rng.standard_normal((d_in, d_in)) * (np.arange(1, d_in + 1) ** -1.0)
    Xs = [rng.standard_normal((7, d_in)) @ mix for _ in range(5)]
    W = rng.standard_normal((d_in, d_out))
    X = np.vstack(Xs)
    Y = X @ W
    res = O.swift_svd(Xs, W, k)
    assert rel(res["C"], Y.T @ Y) <= 1e-12                                   # incremental = batch
    lam = res["lam"]
    assert np.all(np.diff(lam) <= 0)
    err2 = np.sum((Y - X @ res["Wk"]) ** 2)
    assert abs(err2 - lam[k:].sum()) <= 1e-10 * lam.sum()                   # error = tail eigenvalues
    A, s, Bt = np.linalg.svd(Y, full_matrices=False)                         # Eckart-Young on Y
    Yk = (A[:, :k] * s[:k]) @ Bt[:k]
    assert rel(X @ res["Wk"], Yk) <= 1e-10
    assert rel(res["sigma"][:len(s)], s) <= 1e-10
    assert rel(res["U"] @ res["V"], res["Wk"]) <= 1e-12
    # no random rank-k W' does better; the data-independent SVD truncation of W does worse
    for _ in range(200):
        Wp = rng.standard_normal((d_in, k)) @ rng.standard_normal((k, d_out))
        assert np.sum((Y - X @ Wp) ** 2) >= err2 - 1e-9
    Aw, sw, Bw = np.linalg.svd(W, full_matrices=False)
    Wplain = (Aw[:, :k] * sw[:k]) @ Bw[:k]
    assert np.sum((Y - X @ Wplain) ** 2) >= err2 - 1e-9
    # nested subspaces: span(V_k) lies inside span(V_{k+1})
    for kk in range(1, d_out):
        a = O.swift_svd(Xs, W, kk)
        b = O.swift_svd(Xs, W, kk + 1)
        P = b["Vk"] @ b["Vk"].T
        assert rel(P @ a["Vk"], a["Vk"]) <= 1e-10


def pin_swift_reuse(O):
    rng = np.random.default_rng(42)
    Xs = [rng.standard_normal((10, 6))]
    W = rng.standard_normal((6, 6))
    full = O.swift_svd(Xs, W, 6)
    for k in range(1, 6):
        one = O.swift_svd(Xs, W, k)
        Vk = full["Vk"][:, :k]
        assert rel(one["Wk"], W @ Vk @ Vk.T) <= 1e-10


# ============================================================================ test drivers

PINS = [pin_lowrank_bruteforce, pin_lowrank_golden, pin_lowrank_fullrank_svd, pin_lowrank_eckart_young,
        pin_zero_padding, pin_rmsnorm, pin_layernorm, pin_rope, pin_activations, pin_attention_matrix,
        pin_attention_special, pin_attention_split_merge, pin_attention_gqa, pin_qkv_append_and_packing,
        pin_lowrank_history_rebuild, pin_mlp_packed, pin_prefill_then_decode, pin_decoder_layer, pin_encoder_layer,
        pin_swift_golden, pin_swift_closed_form, pin_swift_reuse]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(O)


# ---------------------------------------------------------------------------- planted mistakes


def _mut_lowrank_transposed(x, Ut, Vt, bias=None, residual=None):
    x, Ut, Vt = map(np.asarray, (x, Ut, Vt))
    y = (x @ Ut.T) @ Vt[:, ::-1].T                                 # rank index of V reversed
    if bias is not None:
        y = y + bias
    if residual is not None:
        y = y + residual
    return y


def _mut_lowrank_drop_bias(x, Ut, Vt, bias=None, residual=None):
    y = np.asarray(x, dtype=float) @ np.asarray(Ut, dtype=float).T @ np.asarray(Vt, dtype=float).T
    return y if residual is None else y + residual


def _mut_rope_sign(x, pos, theta):
    x = np.asarray(x, dtype=float)
    D = x.shape[-1]
    h = D // 2
    ang = np.asarray(pos, dtype=float)[..., None] * theta ** (-2.0 * np.arange(h) / D)
    c, s = np.cos(ang), np.sin(ang)
    return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., h:] * c + x[..., :h] * s], axis=-1)


def _mut_rmsnorm_meanabs(x, w, eps):
    x = np.asarray(x, dtype=float)
    return x / (np.mean(np.abs(x), axis=-1, keepdims=True) + eps) * w


def _mut_attention_offbyone(q, k_cache, v_cache, cache_seqlens, causal, scale=None):
    q, kc, vc = map(lambda a: np.asarray(a, dtype=float), (q, k_cache, v_cache))
    B, Sq, Hq, D = q.shape
    Hkv = kc.shape[2]
    scale = scale or 1 / np.sqrt(D)
    o = np.zeros_like(q)
    for b in range(B):
        for s in range(Sq):
            n = int(cache_seqlens[b]) + s + (2 if causal else Sq)       # reads one position too many
            for h in range(Hq):
                g = h * Hkv // Hq
                sc = scale * (kc[b, :n, g] @ q[b, s, h])
                w = np.exp(sc - sc.max())
                o[b, s, h] = w / w.sum() @ vc[b, :n, g]
    return o


def _mut_attention_gqa_modulo(q, k_cache, v_cache, cache_seqlens, causal, scale=None):
    q, kc, vc = map(lambda a: np.asarray(a, dtype=float), (q, k_cache, v_cache))
    B, Sq, Hq, D = q.shape
    Hkv = kc.shape[2]
    scale = scale or 1 / np.sqrt(D)
    o = np.zeros_like(q)
    for b in range(B):
        for s in range(Sq):
            n = int(cache_seqlens[b]) + s + 1 if causal else int(cache_seqlens[b]) + Sq
            for h in range(Hq):
                g = h % Hkv                                              # interleaved instead of grouped
                sc = scale * (kc[b, :n, g] @ q[b, s, h])
                w = np.exp(sc - sc.max())
                o[b, s, h] = w / w.sum() @ vc[b, :n, g]
    return o


def _mut_history_rope_offset(zk, zv, Vt_k, Vt_v, Hkv, D, rope_theta):
    zk, zv = np.asarray(zk, dtype=float), np.asarray(zv, dtype=float)
    B, L, _ = zk.shape
    k = (zk @ np.asarray(Vt_k, dtype=float).T).reshape(B, L, Hkv, D)
    v = (zv @ np.asarray(Vt_v, dtype=float).T).reshape(B, L, Hkv, D)
    if rope_theta:
        k = O.rope(k, np.arange(1, L + 1)[None, :, None], rope_theta)   # positions counted from 1
    return k, v


def _mut_silu_sign(g):
    g = np.asarray(g, dtype=float)
    return g / (1.0 + np.exp(g))


def _mut_swift_ascending(X_batches, W, k):
    W = np.asarray(W, dtype=float)
    C = sum((np.asarray(X) @ W).T @ (np.asarray(X) @ W) for X in X_batches)
    lam, vecs = np.linalg.eigh(C)                                       # left ascending
    Vk = vecs[:, :k]
    return {"C": C, "lam": np.clip(lam, 0, None), "sigma": np.sqrt(np.clip(lam, 0, None)), "Vk": Vk,
            "Wk": W @ Vk @ Vk.T, "U": W @ Vk, "V": Vk.T}


def _mut_layer(kind):
    """decoder_layer with one planted slip in its composition."""
    def layer(x, p, cfg, k_cache, v_cache, cache_seqlens, causal=True):
        x = np.asarray(x, dtype=float)
        B, S, d = x.shape
        q, _, _, kc, vc = O.qkv(x, p["attn_norm_w"], cfg.norm_eps, p["Ut_q"], p["Vt_q"], p["Ut_k"], p["Vt_k"],
                                p["Ut_v"], p["Vt_v"], cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta, k_cache, v_cache,
                                cache_seqlens)
        o = O.attention(q, kc, vc, cache_seqlens, causal=causal)
        h = O.lowrank_linear(o.reshape(B, S, cfg.Hq * cfg.D), p["Ut_o"], p["Vt_o"],
                             residual=None if kind == "drop_o_residual" else x)
        mlp_in = x if kind == "mlp_norm_x" else h
        res = x if kind == "mlp_residual_x" else h
        y = O.mlp(mlp_in, p["mlp_norm_w"], cfg.norm_eps, "swiglu", p["Ut_gate"], p["Vt_gate"], p["Ut_up"],
                  p["Vt_up"], p["Ut_down"], p["Vt_down"], residual=res)
        return y, kc, vc
    layer.__name__ = f"_mut_layer_{kind}"
    return layer


MUTANTS = [
    ("decoder_layer", _mut_layer("mlp_residual_x"), pin_decoder_layer),
    ("decoder_layer", _mut_layer("mlp_norm_x"), pin_decoder_layer),
    ("decoder_layer", _mut_layer("drop_o_residual"), pin_decoder_layer),
    ("lowrank_linear", _mut_lowrank_transposed, pin_lowrank_bruteforce),
    ("lowrank_linear", _mut_lowrank_drop_bias, pin_lowrank_golden),
    ("rope", _mut_rope_sign, pin_rope),
    ("rmsnorm", _mut_rmsnorm_meanabs, pin_rmsnorm),
    ("attention", _mut_attention_offbyone, pin_attention_special),
    ("attention", _mut_attention_offbyone, pin_prefill_then_decode),
    ("attention", _mut_attention_gqa_modulo, pin_attention_gqa),
    ("lowrank_history_kv", _mut_history_rope_offset, pin_lowrank_history_rebuild),
    ("silu", _mut_silu_sign, pin_activations),
    ("silu", _mut_silu_sign, pin_mlp_packed),
    ("swift_svd", _mut_swift_ascending, pin_swift_closed_form),
    ("swift_svd", _mut_swift_ascending, pin_swift_golden),
]


@pytest.mark.parametrize("name,mutant,pin", MUTANTS, ids=[f"{m[0]}-{m[1].__name__}-{m[2].__name__}" for m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pin):
    monkeypatch.setattr(O, name, mutant)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        pin(O)


# ---------------------------------------------------------------------------- input module


def test_bf16_rounding_rne():
    vals = np.array([1.0, 1.00390625, 1.005859375, 1.0078125, -2.5, 3.0e-39, 65504.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8],
                    dtype=np.float32)
    got = I.round_bf16(vals)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa wins (1.0); 1 + 3*2^-8 ties up to 1 + 2^-6
    assert got[7] == 1.0 and got[8] == np.float32(1.0 + 2 ** -6)
    assert got[0] == 1.0 and got[4] == -2.5
    assert np.all(I.round_bf16(got) == got)
    assert np.all(np.abs(got - vals) <= np.abs(vals) * 2 ** -8 + 1e-40)


def test_factor_recipe_shapes_and_ranks():
    assert I.CFG2.rank("q") == 1638 and I.CFG2.rank("down") == 1638
    assert all(v == 384 for v in I.CFG1.ranks.values())
    c = I.make_linear_case()
    assert c["x"].shape == (16, 256) and c["Ut"].shape == (64, 256) and c["Vt"].shape == (256, 64)
    # V rows scaled by i^-0.5: column norms of Vt decay
    n = np.linalg.norm(c["Vt"], axis=0)
    assert n[0] > n[15] > n[63]
