"""GPU parity of the prefill-size (M > 32) MFMA path against the fp64 oracle: every entry point,
ragged M/N/K tails, several tiles per dimension, RoPE + KV append bit checks, and whole prefill
decoder and encoder layers."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import fsvd_oracle as O  # noqa: E402
from svd_compressed_transformer_amd import fsvd, inputs as I  # noqa: E402
from svd_compressed_transformer_amd.device import DeviceLayer, bits, from_dev, pack_rows_dev, pad_cols_dev, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("M,K,r,N,extras", [(33, 256, 64, 256, False), (300, 1000, 40, 1032, True),
                                            (1000, 4096, 1640, 1672, False), (513, 768, 392, 3000, True),
                                            (4096, 768, 384, 768, True),
                                            # 128 x 192 tiles (short reductions): phase 1 with a ragged
                                            # last row tile, then phase 2 with bias and residual
                                            (4001, 1000, 960, 1000, False), (3001, 1000, 768, 1536, True)])
def test_linear_mfma(M, K, r, N, extras):
    say("mfma linear", M, K, r, N, extras)
    rng = np.random.default_rng(M)
    x = I.round_bf16(rng.standard_normal((M, K)))
    Ut, Vt = I.factor_pair(rng, K, N, r)
    Ut, Vt = I.round_bf16(Ut), I.round_bf16(Vt)
    b = I.round_bf16(rng.standard_normal(N)) if extras else None
    res = I.round_bf16(rng.standard_normal((M, N))) if extras else None
    xd, Ud, Vd = to_dev(x), to_dev(Ut), to_dev(Vt)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    nb = fsvd.fsvd_lowrank_linear_ws(M, K, r, N, fsvd.FSVD_BF16)
    ws = fsvd.workspace(nb)
    fsvd.fsvd_lowrank_linear(xd, M, K, K, Ud, r, K, Vd, N, r, to_dev(b) if extras else None,
                             to_dev(res) if extras else None, N, y, N, fsvd.FSVD_BF16, ws, nb)
    torch.cuda.synchronize()
    ref = O.lowrank_linear(x, Ut, Vt, bias=b, residual=res)
    assert rel(from_dev(y), ref) <= BF16_TOL


SMALL = I.scaled_decoder(I.CFG4, d=512, Hq=8, Hkv=2, D=128, d_ff=1024,
                         ranks={"q": 200, "k": 64, "v": 40, "o": 96, "gate": 136, "up": 200, "down": 72})
SMALL64 = I.scaled_decoder(I.CFG2, d=384, Hq=6, Hkv=6, D=64, d_ff=640,
                           ranks={"q": 96, "k": 96, "v": 96, "o": 96, "gate": 120, "up": 120, "down": 96})


@pytest.mark.parametrize("cfg,B,S,seqlens", [(SMALL, 2, 40, [0, 13]), (SMALL64, 3, 100, [5, 0, 60]),
                                             (SMALL, 1, 300, [0])])
def test_qkv_prefill(cfg, B, S, seqlens):
    L_max = 400
    say("qkv prefill", cfg.name, B, S, seqlens)
    p = I.make_decoder_layer(cfg, B=B, S=S, seed=S, random_norm_weights=True)
    sent = I.round_bf16(np.full((B, L_max, cfg.Hkv, cfg.D), -0.75))
    Ud = {k: to_dev(p[k]) for k in ("Ut_q", "Ut_k", "Ut_v", "Vt_q", "Vt_k", "Vt_v")}
    A, (rq, rk, rv) = pack_rows_dev([Ud["Ut_q"], Ud["Ut_k"], Ud["Ut_v"]])
    Vq, Vk, Vv = pad_cols_dev(Ud["Vt_q"], rq), pad_cols_dev(Ud["Vt_k"], rk), pad_cols_dev(Ud["Vt_v"], rv)
    kc, vc = to_dev(sent), to_dev(sent)
    q = torch.empty((B, S, cfg.Hq, cfg.D), dtype=torch.bfloat16, device="cuda")
    kout = torch.empty((B, S, cfg.Hkv, cfg.D), dtype=torch.bfloat16, device="cuda")
    vout = torch.empty_like(kout)
    sl = torch.from_numpy(np.asarray(seqlens, dtype=np.int32)).cuda()
    nb = fsvd.fsvd_lowrank_qkv_ws(B, S, cfg.d, rq, rk, rv, cfg.Hq, cfg.Hkv, cfg.D)
    ws = fsvd.workspace(nb)
    fsvd.fsvd_lowrank_qkv(to_dev(p["x"]), B, S, cfg.d, to_dev(p["attn_norm_w"]), cfg.norm_eps, A, rq, rk, rv, Vq, Vk,
                          Vv, cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta, q, kc, vc, L_max, sl, kout, vout,
                          fsvd.FSVD_BF16, ws, nb)
    torch.cuda.synchronize()
    qr, kr, vr, _, _ = O.qkv(p["x"], p["attn_norm_w"], cfg.norm_eps, p["Ut_q"], p["Vt_q"], p["Ut_k"], p["Vt_k"],
                             p["Ut_v"], p["Vt_v"], cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta, sent, sent, seqlens)
    assert rel(from_dev(q), qr) <= BF16_TOL
    assert rel(from_dev(kout), kr) <= BF16_TOL
    assert rel(from_dev(vout), vr) <= BF16_TOL
    kb, vb, kob, vob, sb = bits(kc), bits(vc), bits(kout), bits(vout), I.bf16_bits(sent)
    for b in range(B):
        lo, hi = seqlens[b], seqlens[b] + S
        assert np.array_equal(kb[b, lo:hi], kob[b]) and np.array_equal(vb[b, lo:hi], vob[b])
        assert np.array_equal(kb[b, :lo], sb[b, :lo]) and np.array_equal(kb[b, hi:], sb[b, hi:])
        assert np.array_equal(vb[b, hi:], sb[b, hi:])
    assert fsvd.fsvd_poll_device_error(ws) == 0


@pytest.mark.parametrize("M", [40, 777])
def test_mlp_prefill_swiglu(M):
    cfg = SMALL
    say("mlp prefill swiglu", M)
    p = I.make_decoder_layer(cfg, B=M, S=1, seed=M, random_norm_weights=True)
    x = p["x"].reshape(M, cfg.d)
    Ud = {k: to_dev(p[k]) for k in ("Ut_gate", "Ut_up", "Vt_gate", "Vt_up", "Ut_down", "Vt_down")}
    A, (rg, ru) = pack_rows_dev([Ud["Ut_gate"], Ud["Ut_up"]])
    Vg, Vu = pad_cols_dev(Ud["Vt_gate"], rg), pad_cols_dev(Ud["Vt_up"], ru)
    Udn, (rd,) = pack_rows_dev([Ud["Ut_down"]])
    Vdn = pad_cols_dev(Ud["Vt_down"], rd)
    xd = to_dev(x)
    y = torch.empty_like(xd)
    nb = fsvd.fsvd_lowrank_mlp_packed_ws(M, cfg.d, rg, ru, cfg.d_ff, rd)
    ws = fsvd.workspace(nb)
    fsvd.fsvd_lowrank_mlp_packed(xd, M, cfg.d, to_dev(p["mlp_norm_w"]), cfg.norm_eps, fsvd.FSVD_ACT_SWIGLU, A, rg, ru,
                                 Vg, Vu, cfg.d_ff, Udn, Vdn, rd, None, y, fsvd.FSVD_BF16, ws, nb)
    torch.cuda.synchronize()
    ref = O.mlp(x, p["mlp_norm_w"], cfg.norm_eps, "swiglu", p["Ut_gate"], p["Vt_gate"], p["Ut_up"], p["Vt_up"],
                p["Ut_down"], p["Vt_down"])
    assert rel(from_dev(y), ref) <= BF16_TOL


# The MLP middle with t kept on chip (one kernel from z_g, z_u to z_d) covers equal gate, up and
# down ranks of 128, 256, 384 or 512: ragged row blocks and d_ff chunks, many d_ff slices, one
# slice (z_d written directly), both row-set widths and both pipeline depths.
@pytest.mark.parametrize("act,r,d,d_ff,M", [
    ("gelu", 128, 256, 1000, 777),
    ("gelu", 256, 512, 640, 1500),
    ("gelu", 384, 768, 3072, 4096),
    ("gelu", 512, 640, 2048, 300),
    ("gelu", 128, 256, 264, 16600),
    ("swiglu", 128, 256, 520, 200),
    ("swiglu", 256, 512, 1024, 1500),
])
def test_mlp_fused_prefill(act, r, d, d_ff, M):
    say("mlp fused prefill", act, r, d, d_ff, M)
    rng = np.random.default_rng(r + M)
    rb = I.round_bf16
    x = rb(rng.standard_normal((M, d)))
    res = rb(rng.standard_normal((M, d)))
    Uu, Vu = map(rb, I.factor_pair(rng, d, d_ff, r))
    Udn, Vdn = map(rb, I.factor_pair(rng, d_ff, d, r))
    if act == "swiglu":
        Ug, Vg = map(rb, I.factor_pair(rng, d, d_ff, r))
        nw = rb(1.0 + 0.1 * rng.standard_normal(d))
        A, rg, fact = np.concatenate([Ug, Uu]), r, fsvd.FSVD_ACT_SWIGLU
    else:
        Ug = Vg = nw = None
        A, rg, fact = Uu, 0, fsvd.FSVD_ACT_GELU
    xd = to_dev(x)
    y = torch.empty_like(xd)
    nb = fsvd.fsvd_lowrank_mlp_packed_ws(M, d, rg, r, d_ff, r)
    ws = fsvd.workspace(nb)
    fsvd.fsvd_lowrank_mlp_packed(xd, M, d, to_dev(nw) if nw is not None else None, 1e-6, fact, to_dev(A), rg, r,
                                 to_dev(Vg) if Vg is not None else None, to_dev(Vu), d_ff, to_dev(Udn), to_dev(Vdn), r,
                                 to_dev(res), y, fsvd.FSVD_BF16, ws, nb)
    torch.cuda.synchronize()
    assert fsvd.fsvd_poll_device_error(ws) == 0
    ref = O.mlp(x, nw, 1e-6, act, Ug, Vg, Uu, Vu, Udn, Vdn, residual=res)
    err = rel(from_dev(y), ref)
    say("  err", err)
    assert err <= BF16_TOL


@pytest.mark.parametrize("fold", [False, True])
def test_decoder_prefill_layer(fold):
    cfg = SMALL
    B, S, L_max = 2, 150, 200
    say("decoder prefill layer", B, S, "folded" if fold else "")
    p = I.make_decoder_layer(cfg, B=B, S=S, seed=77, random_norm_weights=True)
    lay = DeviceLayer(cfg, p, B=B, S=S, L_max=L_max, kc=None, vc=None, seqlens=[0, 30], fold_norm=fold)
    lay.run()
    torch.cuda.synchronize()
    z = np.zeros((B, L_max, cfg.Hkv, cfg.D))
    y_ref, kc_ref, _ = O.decoder_layer(p["x"], p, cfg, z, z, [0, 30])
    assert rel(lay.y_host(), y_ref) <= BF16_TOL
    assert rel(from_dev(lay.k_cache), kc_ref) <= BF16_TOL


@pytest.mark.parametrize("chunk,fold", [(256, False), (512, True), (1024, False)])
def test_decoder_prefill_layer_chunked(chunk, fold):
    """The prefill passes through the layer in chunks of token rows (the workspace holds one
    chunk): with 900 rows over 3 sequences of 300, chunk 256 runs 4 passes of 225 rows and 512
    runs 2 of 450, so passes start and end inside sequences and span sequence boundaries; 1024 is
    one pass.  Output, the whole K/V cache and the length advance against the oracle."""
    cfg = SMALL
    B, S, L_max = 3, 300, 340
    sl0 = [0, 17, 40]
    say("decoder prefill layer, chunk", chunk, "folded" if fold else "")
    p = I.make_decoder_layer(cfg, B=B, S=S, seed=91, random_norm_weights=True)
    lay = DeviceLayer(cfg, p, B=B, S=S, L_max=L_max, kc=None, vc=None, seqlens=sl0, fold_norm=fold, advance=True)
    full_ws = lay.ws.numel()
    lay.desc.prefill_chunk = chunk
    nb = fsvd.fsvd_decoder_layer_ws(lay.desc)
    if chunk < B * S:
        assert nb < full_ws, (nb, full_ws)
    ws = fsvd.workspace(nb)
    lay.desc.ws, lay.desc.ws_bytes = ws.data_ptr(), ws.numel()
    lay.run()
    torch.cuda.synchronize()
    assert fsvd.fsvd_poll_device_error(ws) == 0
    assert list(from_dev(lay.seqlens).astype(int)) == [v + S for v in sl0]
    z = np.zeros((B, L_max, cfg.Hkv, cfg.D))
    y_ref, kc_ref, vc_ref = O.decoder_layer(p["x"], p, cfg, z, z, sl0)
    e_y, e_k, e_v = rel(lay.y_host(), y_ref), rel(from_dev(lay.k_cache), kc_ref), rel(from_dev(lay.v_cache), vc_ref)
    say(f"  workspace {nb} B (one pass of all rows: {full_ws} B); y {e_y:.2e} K {e_k:.2e} V {e_v:.2e}")
    assert e_y <= BF16_TOL and e_k <= BF16_TOL and e_v <= BF16_TOL


def encoder_forward(cfg, p, B, S):
    """BERT-style post-norm layer composed from the C-ABI calls (qkv without norm/RoPE into a
    fresh K/V buffer, non-causal attention, O with residual, LayerNorm, GELU MLP with residual,
    LayerNorm)."""
    d, H, D = cfg.d, cfg.H, cfg.D
    M = B * S
    up = {k: to_dev(v) for k, v in p.items() if k.startswith(("Ut_", "Vt_"))}
    A, (rq, rk, rv) = pack_rows_dev([up["Ut_q"], up["Ut_k"], up["Ut_v"]])
    Vq, Vk, Vv = pad_cols_dev(up["Vt_q"], rq), pad_cols_dev(up["Vt_k"], rk), pad_cols_dev(up["Vt_v"], rv)
    Uo, (ro,) = pack_rows_dev([up["Ut_o"]])
    Vo = pad_cols_dev(up["Vt_o"], ro)
    Uu, (ru,) = pack_rows_dev([up["Ut_up"]])
    Vu = pad_cols_dev(up["Vt_up"], ru)
    Udn, (rd,) = pack_rows_dev([up["Ut_down"]])
    Vdn = pad_cols_dev(up["Vt_down"], rd)
    x = to_dev(p["x"]).reshape(M, d)
    kc = torch.zeros((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    q = torch.empty((M, H * D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    h = torch.empty((M, d), dtype=torch.bfloat16, device="cuda")
    f = torch.empty_like(h)
    y = torch.empty_like(h)
    sl = torch.zeros(B, dtype=torch.int32, device="cuda")
    bf = fsvd.FSVD_BF16
    ws = fsvd.workspace(max(fsvd.fsvd_lowrank_qkv_ws(B, S, d, rq, rk, rv, H, H, D),
                            fsvd.fsvd_decode_attn_dense_kv_ws(B, S, H, H, D, S),
                            fsvd.fsvd_lowrank_linear_ws(M, H * D, ro, d, bf),
                            fsvd.fsvd_lowrank_mlp_packed_ws(M, d, 0, ru, cfg.d_ff, rd)))
    n = ws.numel()
    fsvd.fsvd_lowrank_qkv(x, B, S, d, None, 0.0, A, rq, rk, rv, Vq, Vk, Vv, H, H, D, 0.0, q, kc, vc, S, sl, None, None,
                          bf, ws, n)
    fsvd.fsvd_decode_attn_dense_kv(q, kc, vc, S, sl, B, S, H, H, D, 0.0, 0, o, bf, ws, n)
    fsvd.fsvd_lowrank_linear(o, M, H * D, H * D, Uo, ro, H * D, Vo, d, ro, None, x, d, h, d, bf, ws, n)
    fsvd.fsvd_layernorm(h, None, to_dev(p["ln1_g"]), to_dev(p["ln1_b"]), cfg.ln_eps, M, d, h, bf)
    fsvd.fsvd_lowrank_mlp_packed(h, M, d, None, 0.0, fsvd.FSVD_ACT_GELU, Uu, 0, ru, None, Vu, cfg.d_ff, Udn, Vdn, rd,
                                 h, f, bf, ws, n)
    fsvd.fsvd_layernorm(f, None, to_dev(p["ln2_g"]), to_dev(p["ln2_b"]), cfg.ln_eps, M, d, y, bf)
    torch.cuda.synchronize()
    assert fsvd.fsvd_poll_device_error(ws) == 0
    return from_dev(y).reshape(B, S, d)


def test_encoder_layer_small():
    cfg = I.EncoderLayerConfig(name="enc", d=256, H=4, D=64, d_ff=1024,
                               ranks={"q": 128, "k": 128, "v": 128, "o": 128, "up": 128, "down": 128})
    B, S = 3, 70
    say("encoder layer small", B, S)
    p = I.make_encoder_layer(cfg, B=B, S=S, seed=5)
    y = encoder_forward(cfg, p, B, S)
    assert rel(y, O.encoder_layer(p["x"], p, cfg)) <= BF16_TOL


# ----------------------------------------------------------------------------- factorised attention


def _factorized_case(B, S, Hq, Hkv, D, rq, rk, rv, theta, causal, packed, seed):
    rng = np.random.default_rng(seed)
    ldz = rq + rk + rv if packed else max(rq, rk, rv) + 8
    z = [I.round_bf16(rng.standard_normal((B * S, ldz))) for _ in range(1 if packed else 3)]
    Vq = I.round_bf16(rng.standard_normal((Hq * D, rq)) / np.sqrt(rq))
    Vk = I.round_bf16(rng.standard_normal((Hkv * D, rk)) / np.sqrt(rk))
    Vv = I.round_bf16(rng.standard_normal((Hkv * D, rv)) / np.sqrt(rv))
    if packed:
        zq, zk, zv = z[0][:, :rq], z[0][:, rq:rq + rk], z[0][:, rq + rk:]
    else:
        zq, zk, zv = z[0][:, :rq], z[1][:, :rk], z[2][:, :rv]
    dz = [to_dev(a) for a in z]
    if packed:
        base = dz[0]
        ptrs = (base, base[:, rq:], base[:, rq + rk:])
    else:
        ptrs = tuple(dz)
    out = torch.empty((B, S, Hq, D), dtype=torch.bfloat16, device="cuda")
    fsvd.fsvd_attn_factorized(ptrs[0], ptrs[1], ptrs[2], ldz, to_dev(Vq), rq, to_dev(Vk), rk, to_dev(Vv), rv, B, S, Hq,
                              Hkv, D, theta, 0.0, causal, out, fsvd.FSVD_BF16)
    torch.cuda.synchronize()
    # oracle: the same products written out, then attention over the rebuilt K/V
    q = (np.asarray(zq, dtype=np.float64) @ Vq.T).reshape(B, S, Hq, D)
    if theta:
        q = O.rope(q, np.arange(S)[None, :, None], theta)
    K, V = O.lowrank_history_kv(np.asarray(zk).reshape(B, S, rk), np.asarray(zv).reshape(B, S, rv), Vk, Vv, Hkv, D,
                                theta)
    ref = O.attention(q, K, V, np.zeros(B, dtype=np.int64), causal=causal)
    return from_dev(out), ref


@pytest.mark.parametrize("B,S,Hq,Hkv,D,rq,rk,rv,theta,causal,packed", [
    (2, 100, 4, 4, 64, 40, 40, 40, 0.0, False, False),      # encoder: two query tiles, ragged ranks
    (1, 130, 8, 2, 128, 48, 24, 16, 1e4, True, True),       # causal GQA with RoPE, packed z columns
    (3, 64, 4, 1, 64, 32, 8, 64, 5e5, True, False),         # one tile, GQA 4:1
    (1, 200, 4, 2, 128, 136, 72, 200, 1e4, True, False),    # several rank chunks, ragged last chunk, rk != rv
    (4, 260, 32, 8, 64, 136, 200, 72, 1e4, True, True),     # 256-query workgroups (D = 64, enough of them)
    (2, 300, 6, 6, 64, 264, 264, 264, 0.0, False, True),    # encoder, 128-query workgroups, ragged tiles
])
def test_attention_factorized(B, S, Hq, Hkv, D, rq, rk, rv, theta, causal, packed):
    """Q/K/V rebuilt on chip from z: against the oracle's products, RoPE and attention."""
    say("factorised attention", B, S, Hq, Hkv, D, rq, rk, rv, theta, causal, packed)
    o, ref = _factorized_case(B, S, Hq, Hkv, D, rq, rk, rv, theta, causal, packed, seed=B * S)
    err = rel(o, ref)
    say(f"  err {err:.2e}")
    assert np.all(np.isfinite(o)) and err <= BF16_TOL


@pytest.mark.slow
def test_attention_factorized_bert_base():
    """The BERT-Base encoder shape: batch 8 x 512, 12 heads x 64, rank 384, no mask."""
    say("factorised attention, BERT-Base shape")
    o, ref = _factorized_case(8, 512, 12, 12, 64, 384, 384, 384, 0.0, False, True, seed=5)
    err = rel(o, ref)
    say(f"  err {err:.2e}")
    assert err <= BF16_TOL
