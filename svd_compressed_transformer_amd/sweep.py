"""Sweeps of the low-rank layer stack on one GPU: history length, rank ratio, batch and stack depth.

    python -m svd_compressed_transformer_amd.sweep [--quick]

Each point builds a stack of distinct Llama-7B-shaped layers (hidden 4096, 32 x 128 heads, SwiGLU
11008, every projection at rank floor(ratio * 4096) stored padded to a multiple of 32, RMSNorm
weights folded into the packed phase-1 factors) with a dense KV history of random values, then
times decode steps replayed from per-layer graphs (and from one graph per step) and, for the rank
sweep, an eager 4 x 2048-token prefill of one layer.  Factors are drawn on the device with the
same distributions as the seeded host recipe (U ~ N(0, 1/d_in), V ~ N(0, 1/r) diag(i^-0.5)): only
timing is measured here, parity is the test suite's.  One JSON line per point on stdout.
"""
from __future__ import annotations

import argparse
import json
import math
import sys

import torch

from svd_compressed_transformer_amd import fsvd, inputs as I
from svd_compressed_transformer_amd.device import pack_rows_dev, pad_cols_dev

D_MODEL, HEADS, HEAD_DIM, D_FF = 4096, 32, 128, 11008
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _factor(gen, d_in, d_out, r, dev):
    """Ut [r, d_in] and Vt [d_out, r] (bf16) of one projection at rank r."""
    U = torch.randn((d_in, r), generator=gen, device=dev) / math.sqrt(d_in)
    sig = torch.arange(1, r + 1, device=dev, dtype=torch.float32) ** -0.5
    V = torch.randn((r, d_out), generator=gen, device=dev) / math.sqrt(r) * sig[:, None]
    return U.t().contiguous().to(torch.bfloat16), V.t().contiguous().to(torch.bfloat16)


class StackLayer:
    """One decoder layer's packed factors and KV cache on the device, and its descriptor.

    cfg gives the layer shape (hidden, heads, head dim, d_ff, norm eps, RoPE theta); ranks maps
    each projection (q, k, v, o, gate, up, down) to its logical rank."""

    def __init__(self, cfg, ranks, B, S, L_max, seed, dev, x, y, seqlens, advance=1):
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        d, qd, kd = cfg.d, cfg.Hq * cfg.D, cfg.Hkv * cfg.D
        dims = {"q": (d, qd), "k": (d, kd), "v": (d, kd), "o": (qd, d), "gate": (d, cfg.d_ff), "up": (d, cfg.d_ff),
                "down": (cfg.d_ff, d)}
        f = {p: _factor(gen, *dims[p], ranks[p], dev) for p in dims}
        self.attn_w = (1.0 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(torch.bfloat16)
        self.mlp_w = (1.0 + 0.1 * torch.randn(d, generator=gen, device=dev)).to(torch.bfloat16)
        self.A_qkv, (rq, rk, rv) = pack_rows_dev([f["q"][0], f["k"][0], f["v"][0]], device=dev, col_scale=self.attn_w)
        self.Vq, self.Vk, self.Vv = (pad_cols_dev(f["q"][1], rq, dev), pad_cols_dev(f["k"][1], rk, dev),
                                     pad_cols_dev(f["v"][1], rv, dev))
        self.Uo, (ro,) = pack_rows_dev([f["o"][0]], device=dev)
        self.Vo = pad_cols_dev(f["o"][1], ro, dev)
        self.A_gu, (rg, ru) = pack_rows_dev([f["gate"][0], f["up"][0]], device=dev, col_scale=self.mlp_w)
        self.Vg, self.Vu = pad_cols_dev(f["gate"][1], rg, dev), pad_cols_dev(f["up"][1], ru, dev)
        self.Ud, (rd,) = pack_rows_dev([f["down"][0]], device=dev)
        self.Vd = pad_cols_dev(f["down"][1], rd, dev)
        del f
        self.logical = dict(ranks)
        shape = (B, L_max, cfg.Hkv, cfg.D)
        self.kc = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
        self.vc = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
        self.desc = fsvd.decoder_layer_desc(
            B=B, S=S, d=d, Hq=cfg.Hq, Hkv=cfg.Hkv, D=cfg.D, d_ff=cfg.d_ff, L_max=L_max, r_q=rq, r_k=rk, r_v=rv,
            r_o=ro, r_g=rg, r_u=ru, r_d=rd, norm_eps=cfg.norm_eps, rope_theta=cfg.rope_theta, softmax_scale=0.0,
            advance_seqlens=advance, flags=fsvd.FSVD_LAYER_NORM_FOLDED, x=x, y=y, attn_norm_w=None, mlp_norm_w=None,
            A_qkv=self.A_qkv, Vt_q=self.Vq, Vt_k=self.Vk, Vt_v=self.Vv, Ut_o=self.Uo, Vt_o=self.Vo, A_gu=self.A_gu,
            Vt_g=self.Vg, Vt_u=self.Vu, Ut_d=self.Ud, Vt_d=self.Vd, k_cache=self.kc, v_cache=self.vc,
            cache_seqlens=seqlens)


def uniform_ranks(ratio):
    """Llama-7B-shaped layer: every projection at rank floor(ratio * 4096)."""
    r = int(math.floor(ratio * D_MODEL + 1e-9))
    return dict(q=r, k=r, v=r, o=r, gate=r, up=r, down=r)


def decode_bytes(cfg, logical, B, L_read):
    """Algorithmic HBM bytes of one decode layer-step: every factor byte once (logical ranks), the
    KV cache read once over L_read positions, the new K/V written, the layer input and output."""
    d, qd, kd = cfg.d, cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    r = logical
    fac = 2 * (r["q"] * (d + qd) + r["k"] * (d + kd) + r["v"] * (d + kd) + r["o"] * (qd + d) +
               r["gate"] * (d + cfg.d_ff) + r["up"] * (d + cfg.d_ff) + r["down"] * (cfg.d_ff + d))
    return fac + 2 * 2 * B * L_read * kd + 2 * 2 * B * kd + 2 * 2 * B * d


def run_decode(B, history, ratio, layers, steps, dev, stream, one_graph=True):
    L_max = (history + steps + 1 + 63) // 64 * 64  # cache rows: a multiple of 64 (sequence starts aligned)
    sl = torch.full((layers, B), history, dtype=torch.int32, device=dev)
    ys = [torch.randn((B, 1, D_MODEL), device=dev).to(torch.bfloat16) for _ in range(layers)]
    stack = []
    for l in range(layers):
        stack.append(StackLayer(I.CFG2, uniform_ranks(ratio), B, 1, L_max, 1000 + l, dev, ys[(l - 1) % layers], ys[l],
                                sl[l]))
    ws = fsvd.workspace(fsvd.fsvd_decoder_layer_ws(stack[0].desc), device=dev)
    for lay in stack:
        lay.desc.ws, lay.desc.ws_bytes = ws.data_ptr(), ws.numel()
    graphs = [fsvd.fsvd_decoder_layer_capture(lay.desc) for lay in stack]
    sg = fsvd.fsvd_decoder_stack_capture([lay.desc for lay in stack]) if one_graph else None
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(replay):
        sl.fill_(history)
        replay()  # warm
        sl.fill_(history)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (steps * layers)

    us = timed(lambda: [fsvd.fsvd_graph_replay(g, stream) for g in graphs])
    us_one = timed(lambda: fsvd.fsvd_graph_replay(sg, stream)) if sg else None
    assert fsvd.fsvd_poll_device_error(ws, stream) == 0
    for g in graphs:
        fsvd.fsvd_graph_destroy(g)
    if sg:
        fsvd.fsvd_graph_destroy(sg)
    by = decode_bytes(I.CFG2, stack[0].logical, B, history + 1 + steps // 2)
    res = {"sweep": "decode", "batch": B, "history": history, "rank_ratio": ratio, "layers": layers,
           "rank": stack[0].logical["q"], "us_per_layer_step": round(us, 2),
           "tokens_per_s_per_layer": round(B / (us * 1e-6), 1), "algorithmic_bytes": int(by),
           "hbm_frac": round(by / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if us_one is not None:
        res["us_per_layer_step_one_graph"] = round(us_one, 2)
    del stack, graphs, ws
    torch.cuda.empty_cache()
    return res


def run_prefill(B, S, ratio, dev, stream, reps=3):
    L_max = S
    sl = torch.zeros((1, B), dtype=torch.int32, device=dev)
    x = torch.randn((B, S, D_MODEL), device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    lay = StackLayer(I.CFG2, uniform_ranks(ratio), B, S, L_max, 7, dev, x, y, sl[0], advance=0)
    ws = fsvd.workspace(fsvd.fsvd_decoder_layer_ws(lay.desc), device=dev)
    lay.desc.ws, lay.desc.ws_bytes = ws.data_ptr(), ws.numel()
    fsvd.fsvd_decoder_layer_run(lay.desc, stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fsvd.fsvd_decoder_layer_run(lay.desc, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    r = lay.logical
    d, qd, M = D_MODEL, HEADS * HEAD_DIM, B * S
    flops = 2 * M * (r["q"] * (d + qd) * 3 + r["o"] * (qd + d) + r["gate"] * (d + D_FF) * 2 + r["down"] * (D_FF + d))
    del lay, ws
    torch.cuda.empty_cache()
    return {"sweep": "prefill", "batch": B, "seq": S, "rank_ratio": ratio, "rank": r["q"], "ms_per_layer": round(ms, 3),
            "tokens_per_s_per_layer": round(M / (ms * 1e-3), 1),
            "proj_mfma_frac": round(flops / (ms * 1e-3) / 2.5e15, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--quick", action="store_true", help="a few points only")
    ap.add_argument("--steps", type=int, default=32)
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)
    points = []
    if args.quick:
        points += [("decode", dict(B=4, history=2048, ratio=0.4, layers=4))]
    else:
        for L in (1024, 2048, 4096, 8192, 16384):
            points.append(("decode", dict(B=4, history=L, ratio=0.4, layers=4)))
        for B in (1, 8, 16, 32):
            points.append(("decode", dict(B=B, history=2048, ratio=0.4, layers=4)))
        for ratio in (0.2, 0.3, 0.5, 0.6):
            points.append(("decode", dict(B=4, history=2048, ratio=ratio, layers=4)))
        points.append(("decode", dict(B=4, history=2048, ratio=0.4, layers=32)))
        for ratio in (0.2, 0.3, 0.4, 0.5, 0.6):
            points.append(("prefill", dict(B=4, S=2048, ratio=ratio)))
    for kind, kw in points:
        log(kind, kw)
        if kind == "decode":
            res = run_decode(kw["B"], kw["history"], kw["ratio"], kw["layers"], args.steps, dev, stream)
        else:
            res = run_prefill(kw["B"], kw["S"], kw["ratio"], dev, stream)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
