"""Parity at the full configured shapes, in the launch configurations the benchmark uses.

- Llama-7B-shaped decode layer (hidden 4096, 32 x 128 heads, d_ff 11008, rank 1638 on every
  projection), batch 1 / 8 / 16 over a dense KV history of 2048 tokens: one eager step and one
  replay of the captured per-layer graph (bit-identical), the whole output against the oracle,
  the appended K/V slot against the oracle, every other cache slot unchanged bit for bit, and a
  NaN-poisoned cache tail that must not reach the output.
- Llama-3-8B-shaped GQA layer (32 Q / 8 KV heads, d_ff 14336, per-projection ranks), batch 32
  over a history of 8192 tokens.
- The benchmark's prefill + decode sequence: a 4 x 2048-token prefill of the 7B-shaped layer
  (MFMA path, eager), then decode steps replayed from the captured graph with the in-graph
  length advance, with the RMSNorm weights folded into A_qkv / A_gu as the benchmark packs
  them.  The oracle runs its own prefill (never the GPU's), with the weights kept separate: the
  whole K/V cache it writes is compared, the layer output on whole 128-query blocks (first,
  middle and last of every sequence), and the replayed decode output of every one of the 128
  steps.
- The 7B-shaped decode layer at batch 4 over a 16,384-token history (the longest horizon).
- BERT-Base-shaped encoder layer (768, 12 x 64, d_ff 3072, rank 384), batch 8 x 512: whole output.
"""
import ctypes
import functools

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import fsvd_oracle as O  # noqa: E402
from svd_compressed_transformer_amd import fsvd, inputs as I  # noqa: E402
from svd_compressed_transformer_amd.device import DeviceLayer, bits, from_dev, to_dev  # noqa: E402

from .test_gpu_3_prefill import encoder_forward  # noqa: E402

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
BF16_TOL = 2e-2


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def say(*a):
    print(*a, flush=True)


@functools.lru_cache(maxsize=1)
def _params(name, B, S, seed):
    cfg = {"cfg2": I.CFG2, "cfg4": I.CFG4}[name]
    return I.make_decoder_layer(cfg, B=B, S=S, seed=seed, random_norm_weights=True)


def _decode_case(cfg, name, B, L0, pad_tail, seed):
    """One decode step of a full-size layer: eager, then one graph replay; checks against the oracle."""
    p_all = _params(name, 16 if name == "cfg2" else B, 1, seed)
    p = dict(p_all)
    p["x"] = p_all["x"][:B]
    L_max = L0 + 1 + pad_tail
    kc, vc = I.make_kv_history(B, L_max, cfg.Hkv, cfg.D, L0, seed=seed + 7)
    kc[:, L0 + 1:] = np.nan  # poisoned tail: never read (n = L0 + 1)
    vc[:, L0 + 1:] = np.nan
    lay = DeviceLayer(cfg, p, B=B, S=1, L_max=L_max, kc=kc, vc=vc, seqlens=np.full(B, L0))
    k_before, v_before = bits(lay.k_cache), bits(lay.v_cache)
    lay.run()
    torch.cuda.synchronize()
    y_eager = bits(lay.y)
    g = lay.capture()
    fsvd.fsvd_graph_replay(g)
    torch.cuda.synchronize()
    fsvd.fsvd_graph_destroy(g)
    assert np.array_equal(bits(lay.y), y_eager), "graph replay differs from the eager step"
    assert fsvd.fsvd_poll_device_error(lay.ws) == 0
    k_after, v_after = bits(lay.k_cache), bits(lay.v_cache)
    # every slot but the appended one keeps its exact bits (NaN tail included)
    keep = np.ones(L_max, dtype=bool)
    keep[L0] = False
    assert np.array_equal(k_after[:, keep], k_before[:, keep])
    assert np.array_equal(v_after[:, keep], v_before[:, keep])
    y = lay.y_host()
    assert np.all(np.isfinite(y))
    kc[:, L0 + 1:] = 0.0  # the oracle reads positions < n only; zeros keep its copies finite
    vc[:, L0 + 1:] = 0.0
    y_ref, kc_ref, vc_ref = O.decoder_layer(p["x"], p, cfg, kc, vc, np.full(B, L0))
    e_y = rel(y, y_ref)
    e_k = rel(from_dev(lay.k_cache)[:, L0], kc_ref[:, L0])
    e_v = rel(from_dev(lay.v_cache)[:, L0], vc_ref[:, L0])
    say(f"  {name} B={B} L0={L0}: y {e_y:.2e}  k {e_k:.2e}  v {e_v:.2e}")
    assert e_y <= BF16_TOL and e_k <= BF16_TOL and e_v <= BF16_TOL


@pytest.mark.parametrize("B", [1, 8, 16])
def test_llama7b_decode_layer_full(B):
    say("llama-7b decode layer, full size, B", B)
    _decode_case(I.CFG2, "cfg2", B, L0=2048, pad_tail=15, seed=3)


def test_llama3_8b_gqa_decode_layer_full_b32():
    say("llama-3-8b GQA decode layer, full size, B 32, history 8192")
    _decode_case(I.CFG4, "cfg4", 32, L0=8192, pad_tail=0, seed=4)


def test_llama7b_decode_layer_history_16384():
    """The longest decode horizon the stack sweep times: batch 4 over 16,384 cached tokens."""
    say("llama-7b decode layer, full size, B 4, history 16384")
    _decode_case(I.CFG2, "cfg2", 4, L0=16384, pad_tail=0, seed=3)


def test_llama7b_prefill_then_replayed_decode_full():
    """4 x 2048 prefill (eager, MFMA path) then all 128 graph-replayed decode steps with in-graph
    advance, exactly as the benchmark drives one layer."""
    cfg, B, S, ND = I.CFG3, I.CFG3_BATCH, I.CFG3_PREFILL, I.CFG3_DECODE_STEPS
    L_max = S + I.CFG3_DECODE_STEPS
    say("llama-7b prefill", B, "x", S, "then", ND, "replayed decode steps")
    p = I.make_decoder_layer(cfg, B=B, S=S, seed=8, random_norm_weights=True)
    nan_cache = np.full((B, L_max, cfg.Hkv, cfg.D), np.nan, dtype=np.float32)
    pre = DeviceLayer(cfg, p, B=B, S=S, L_max=L_max, kc=nan_cache, vc=nan_cache, seqlens=np.zeros(B),
                      advance=True, fold_norm=True)
    del nan_cache
    pre.run()
    torch.cuda.synchronize()
    assert fsvd.fsvd_poll_device_error(pre.ws) == 0
    assert np.array_equal(from_dev(pre.seqlens), np.full(B, S)), "prefill must advance the lengths by S"
    y_pre = pre.y_host()
    kb, vb = bits(pre.k_cache), bits(pre.v_cache)
    nan_bits = bits(torch.full((1,), float("nan"), dtype=torch.bfloat16))[0]
    assert np.all(kb[:, S:] == nan_bits) and np.all(vb[:, S:] == nan_bits), "slots past the prefill were written"
    k_gpu, v_gpu = from_dev(pre.k_cache)[:, :S], from_dev(pre.v_cache)[:, :S]
    del kb, vb

    # decode descriptor: the prefill descriptor with S = 1, in-graph advance, its own x / y / workspace
    rng = np.random.default_rng(81)
    xs = I.round_bf16(rng.standard_normal((ND, B, cfg.d)))
    x_dec = torch.empty((B, 1, cfg.d), dtype=torch.bfloat16, device="cuda")
    y_dec = torch.empty_like(x_dec)
    d = type(pre.desc)()
    ctypes.memmove(ctypes.addressof(d), ctypes.addressof(pre.desc), ctypes.sizeof(d))
    d.S = 1
    d.x, d.y = x_dec.data_ptr(), y_dec.data_ptr()
    d.advance_seqlens = 1
    ws = fsvd.workspace(fsvd.fsvd_decoder_layer_ws(d))
    d.ws, d.ws_bytes = ws.data_ptr(), ws.numel()
    g = fsvd.fsvd_decoder_layer_capture(d)
    ys = []
    for t in range(ND):
        x_dec.copy_(to_dev(xs[t]).reshape(B, 1, cfg.d))
        fsvd.fsvd_graph_replay(g)
        torch.cuda.synchronize()
        ys.append(from_dev(y_dec)[:, 0])
    fsvd.fsvd_graph_destroy(g)
    assert fsvd.fsvd_poll_device_error(ws) == 0
    assert np.array_equal(from_dev(pre.seqlens), np.full(B, S + ND))

    # oracle prefill: Q/K/V of every token (its own caches), then sampled rows of the layer output
    say("  oracle prefill projections ...")
    zero = np.zeros((B, L_max, cfg.Hkv, cfg.D))
    q, _, _, kc_ref, vc_ref = O.qkv(p["x"], p["attn_norm_w"], cfg.norm_eps, p["Ut_q"], p["Vt_q"], p["Ut_k"],
                                    p["Vt_k"], p["Ut_v"], p["Vt_v"], cfg.Hq, cfg.Hkv, cfg.D, cfg.rope_theta,
                                    zero, zero, np.zeros(B))
    del zero
    e_k, e_v = rel(k_gpu, kc_ref[:, :S]), rel(v_gpu, vc_ref[:, :S])
    say(f"  prefill K cache {e_k:.2e}  V cache {e_v:.2e}")
    assert e_k <= BF16_TOL and e_v <= BF16_TOL
    # whole 128-query blocks (the attention kernel's query tile): the first, a middle and the last
    # block of every sequence, every row of each
    QB = 128
    y_ref_rows, y_gpu_rows = [], []
    for b in range(B):
        for s0 in (0, S // 2, S - QB):
            o = O.attention(q[b:b + 1, s0:s0 + QB], kc_ref[b:b + 1], vc_ref[b:b + 1], [s0], causal=True)
            h = O.lowrank_linear(o.reshape(QB, cfg.Hq * cfg.D), p["Ut_o"], p["Vt_o"], residual=p["x"][b, s0:s0 + QB])
            yr = O.mlp(h, p["mlp_norm_w"], cfg.norm_eps, "swiglu", p["Ut_gate"], p["Vt_gate"], p["Ut_up"],
                       p["Vt_up"], p["Ut_down"], p["Vt_down"], residual=h)
            y_ref_rows.append(yr)
            y_gpu_rows.append(y_pre[b, s0:s0 + QB])
    e_y = rel(np.concatenate(y_gpu_rows), np.concatenate(y_ref_rows))
    say(f"  prefill output on {len(y_ref_rows)} whole {QB}-query blocks {e_y:.2e}")
    assert e_y <= BF16_TOL

    # oracle decode steps over the oracle's own prefill caches
    say(f"  oracle decode steps ({ND}) ...")
    y_steps, _, _, _ = O.decoder_steps(xs, p, cfg, kc_ref, vc_ref, np.full(B, S))
    errs = [rel(ys[t], y_steps[t]) for t in range(ND)]
    say(f"  replayed decode outputs, every step: max {max(errs):.2e} (step {int(np.argmax(errs))})")
    assert max(errs) <= BF16_TOL


def test_bert_base_encoder_layer_full():
    cfg, B, S = I.CFG1, 8, 512
    say("bert-base encoder layer, full size", B, "x", S)
    p = I.make_encoder_layer(cfg, B=B, S=S, seed=0)
    y = encoder_forward(cfg, p, B, S)
    y_ref = O.encoder_layer(p["x"], p, cfg)
    e = rel(y, y_ref)
    say(f"  encoder output {e:.2e}")
    assert e <= BF16_TOL
