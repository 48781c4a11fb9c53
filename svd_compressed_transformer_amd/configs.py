"""Measurements of the low-rank layer path at each configured shape, on one GPU.

    python -m svd_compressed_transformer_amd.configs [--only NAME[,NAME...]]

One JSON line per measurement on stdout:

- linear_fp32: one fused low-rank linear in fp32, x 16 x 256, U 256 x 64, V 64 x 256 (the
  operands stay in L2; launch-latency bound, time only).
- bert_layer: BERT-Base-shaped post-norm encoder layer, batch 8 x 512, rank 384 on every
  projection, composed of the entry points (Q/K/V, attention without mask, O + residual,
  LayerNorm, GELU MLP + residual, LayerNorm), eager: layer time, the projections' TFLOP/s and
  fraction of the bf16 MFMA peak, attention time, peak activation bytes.
- prefill_llama7b_chunks: one Llama-7B-shaped layer, prefill of 4 x 2048 tokens, at pass sizes
  of 8192 (the default: one pass), 4096, 2048 and 1024 token rows: time per layer, projection
  TFLOP/s over the layer time, and the workspace each pass size needs.
- decode_llama7b_b{1,8,16}: 4 distinct Llama-7B-shaped layers (rank 1638 on every projection),
  history held at 2048 (no length advance): per-layer graph replay (the measured configuration),
  one graph per decode step, and eager launches; tokens/s per layer, achieved GB/s of the
  algorithmic bytes and their fraction of 8 TB/s.
- decode_llama3_8b_gqa_b32: the same for 4 Llama-3-8B-shaped GQA layers (32 Q / 8 KV heads,
  d_ff 14336, ranks q 1536, k 512, v 256, o 1024, gate 1024, up 1536, down 512), batch 32,
  history 8192.
- swift_covariance_4096: one Swift-SVD calibration batch at the Llama-7B projection width
  (d_in = d_out = 4096, 4096 tokens): Y^T = W^T X^T and C += Y^T Y (upper triangle) on the matrix
  cores; TFLOP/s of the algorithmic flops (the product and the symmetric half of the covariance).
- attn_factorized_bert / attn_factorized_llama7b_s2048: attention with Q/K/V rebuilt on chip from
  the rank-r activations (nothing of q, k, v written) against the dense attention over
  materialised q, K, V: BERT-Base encoder (8 x 512, 12 x 64, rank 384, no mask) and a causal
  Llama-7B prefill of one 2048-token sequence (32 x 128, rank 1638 stored as 1664, RoPE); the bytes of q, k, v the
  factorised form never writes.
- dense_vs_lowrank_llama7b_m{1,4,8192}: the seven projections of a Llama-7B-shaped layer (q, k, v,
  o: 4096 -> 4096; gate, up: 4096 -> 11008; down: 11008 -> 4096) as plain linears over 1, 4 or
  8192 token rows, each once with the dense weight W = U.V (fsvd_dense_linear: one kernel) and once
  with the rank-1638 factors (fsvd_lowrank_linear: two kernels), through the same kernels; no
  norm, activation, RoPE or cache work on either side; 4 weight copies rotated.
- gemm_vs_vendor_llama7b_shapes: the library's MFMA GEMM (y = x . W^T, 8192 rows) against the
  vendor GEMM (hipBLASLt through torch.matmul, same bf16 operands) at the prefill products' (K, N).
- dense_vs_lowrank_ratios_llama7b_m{1,4,8192}: the same at rank ratios 0.1-0.6 of min(dims) on every
  projection: the low-rank speedup over the dense weights against the compression ratio.
- attn_lowrank_history_llama7b_b{1,4}: the decode attention of a Llama-7B-shaped layer over a
  2048-token history, from the dense KV cache against the layout the dense cache replaces
  (rank-1638 rows z_k, z_v cached per token, K and V rebuilt from them every step, then the same
  attention); 4 distinct caches rotated.

Timing: warm-up passes, then windows of K passes with K chosen so a window lasts at least 20 ms;
the median of 5 windows.  Factors are drawn on the device with the seeded recipe's
distributions (U ~ N(0, 1/d_in), V ~ N(0, 1/r) diag(i^-0.5)); only timing is measured here,
parity is the test suite's.
"""
from __future__ import annotations

import argparse
import json
import math
import statistics
import sys

import torch

from svd_compressed_transformer_amd import fsvd, inputs as I
from svd_compressed_transformer_amd.device import pack_rows_dev, pad_cols_dev
from svd_compressed_transformer_amd.sweep import StackLayer, _factor, decode_bytes

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def timed_median(fn, stream, min_ms=20.0, windows=5, warm=3):
    """Median over `windows` windows of K calls of fn (K so that a window lasts >= min_ms), in
    ms per call, timed with HIP events on `stream`."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0.record(stream)
    fn()
    e1.record(stream)
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1), 1e-3)
    K = max(1, math.ceil(min_ms / est))
    res = []
    for _ in range(windows):
        e0.record(stream)
        for _ in range(K):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / K)
    return statistics.median(res)


# ----------------------------------------------------------------------------- single linear, fp32


def run_linear_fp32(dev, stream):
    c = I.CFG0
    x = torch.randn((c.M, c.K), device=dev)
    Ut = torch.randn((c.r, c.K), device=dev) / math.sqrt(c.K)
    Vt = torch.randn((c.N, c.r), device=dev) / math.sqrt(c.r)
    y = torch.empty((c.M, c.N), device=dev)
    ws = fsvd.workspace(fsvd.fsvd_lowrank_linear_ws(c.M, c.K, c.r, c.N, fsvd.FSVD_F32), device=dev)

    def call():
        fsvd.fsvd_lowrank_linear(x, c.M, c.K, c.K, Ut, c.r, c.K, Vt, c.N, c.r, None, None, c.N, y, c.N,
                                 fsvd.FSVD_F32, ws, ws.numel(), stream)

    ms = timed_median(call, stream, min_ms=5.0)
    by = 4 * (c.M * c.K + c.r * c.K + c.N * c.r + c.M * c.N)
    return {"config": "linear_fp32", "M": c.M, "K": c.K, "rank": c.r, "N": c.N, "us_per_call": round(ms * 1e3, 2),
            "algorithmic_bytes": by, "note": "operands resident in L2; launch-latency bound"}


# ----------------------------------------------------------------------------- BERT-Base encoder layer


def run_bert_layer(dev, stream):
    cfg, B, S = I.CFG1, I.CFG1_BATCH, I.CFG1_SEQ
    d, H, D, dff = cfg.d, cfg.H, cfg.D, cfg.d_ff
    M = B * S
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    r = cfg.ranks
    f = {p: _factor(gen, *dims, r[p], dev) for p, dims in (
        ("q", (d, H * D)), ("k", (d, H * D)), ("v", (d, H * D)), ("o", (H * D, d)), ("up", (d, dff)),
        ("down", (dff, d)))}
    A, (rq, rk, rv) = pack_rows_dev([f["q"][0], f["k"][0], f["v"][0]], device=dev)
    Vq, Vk, Vv = (pad_cols_dev(f["q"][1], rq, dev), pad_cols_dev(f["k"][1], rk, dev), pad_cols_dev(f["v"][1], rv, dev))
    Uo, (ro,) = pack_rows_dev([f["o"][0]], device=dev)
    Vo = pad_cols_dev(f["o"][1], ro, dev)
    Uu, (ru,) = pack_rows_dev([f["up"][0]], device=dev)
    Vu = pad_cols_dev(f["up"][1], ru, dev)
    Ud, (rd,) = pack_rows_dev([f["down"][0]], device=dev)
    Vd = pad_cols_dev(f["down"][1], rd, dev)
    del f
    g1 = torch.ones(d, dtype=torch.bfloat16, device=dev)
    b1 = torch.zeros(d, dtype=torch.bfloat16, device=dev)
    x = torch.randn((M, d), generator=gen, device=dev).to(torch.bfloat16)
    torch.cuda.synchronize()

    # everything the layer call allocates beyond its inputs and weights: activations + workspace
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    bf = fsvd.FSVD_BF16
    kc = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    q = torch.empty((M, H * D), dtype=torch.bfloat16, device=dev)
    o = torch.empty_like(q)
    h = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    fo = torch.empty_like(h)
    y = torch.empty_like(h)
    sl = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = fsvd.workspace(max(fsvd.fsvd_lowrank_qkv_ws(B, S, d, rq, rk, rv, H, H, D),
                            fsvd.fsvd_decode_attn_dense_kv_ws(B, S, H, H, D, S),
                            fsvd.fsvd_lowrank_linear_ws(M, H * D, ro, d, bf),
                            fsvd.fsvd_lowrank_mlp_packed_ws(M, d, 0, ru, dff, rd)), device=dev)
    n = ws.numel()

    def qkv():
        fsvd.fsvd_lowrank_qkv(x, B, S, d, None, 0.0, A, rq, rk, rv, Vq, Vk, Vv, H, H, D, 0.0, q, kc, vc, S, sl, None,
                              None, bf, ws, n, stream)

    def attn():
        fsvd.fsvd_decode_attn_dense_kv(q, kc, vc, S, sl, B, S, H, H, D, 0.0, 0, o, bf, ws, n, stream)

    def oproj():
        fsvd.fsvd_lowrank_linear(o, M, H * D, H * D, Uo, ro, H * D, Vo, d, ro, None, x, d, h, d, bf, ws, n, stream)

    def ln1():
        fsvd.fsvd_layernorm(h, None, g1, b1, cfg.ln_eps, M, d, h, bf, stream)

    def mlp():
        fsvd.fsvd_lowrank_mlp_packed(h, M, d, None, 0.0, fsvd.FSVD_ACT_GELU, Uu, 0, ru, None, Vu, dff, Ud, Vd, rd, h,
                                     fo, bf, ws, n, stream)

    def ln2():
        fsvd.fsvd_layernorm(fo, None, g1, b1, cfg.ln_eps, M, d, y, bf, stream)

    def layer():
        qkv(); attn(); oproj(); ln1(); mlp(); ln2()

    layer()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev) - base
    assert fsvd.fsvd_poll_device_error(ws, stream) == 0
    t_layer = timed_median(layer, stream)
    t_qkv, t_attn, t_o, t_mlp = (timed_median(fn, stream) for fn in (qkv, attn, oproj, mlp))
    t_proj = t_qkv + t_o + t_mlp
    proj_flops = 2 * M * (r["q"] * (d + H * D) + r["k"] * (d + H * D) + r["v"] * (d + H * D) + r["o"] * (H * D + d) +
                          r["up"] * (d + dff) + r["down"] * (dff + d))
    attn_flops = 4 * B * H * S * S * D
    io = M * d * 2
    unfused = 2 * io + 2 * M * dff * 2 + B * H * S * S * 4  # u and GELU(u) in bf16, fp32 scores
    return {"config": "bert_layer", "batch": B, "seq": S, "rank": r["q"], "ms_per_layer": round(t_layer, 4),
            "tokens_per_s_per_layer": round(M / (t_layer * 1e-3), 1),
            "projections": {"ms": round(t_proj, 4), "qkv_ms": round(t_qkv, 4), "o_ms": round(t_o, 4),
                            "mlp_ms": round(t_mlp, 4), "flops": int(proj_flops),
                            "tflops": round(proj_flops / (t_proj * 1e-3) / 1e12, 1),
                            "mfma_frac": round(proj_flops / (t_proj * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
            "attention": {"ms": round(t_attn, 4), "flops": int(attn_flops),
                          "tflops": round(attn_flops / (t_attn * 1e-3) / 1e12, 1)},
            "peak_activation_bytes": int(peak), "unfused_activation_bytes": int(unfused),
            "layer_io_bytes": int(io)}


# ----------------------------------------------------------------------------- Llama-7B prefill passes


def run_prefill_chunks(dev, stream, chunks=(0, 4096, 2048, 1024)):
    """One Llama-7B-shaped layer (rank 1638, RMSNorm weights folded), prefill of 4 x 2048 tokens,
    at several pass sizes (prefill_chunk rows; 0 = the default, the whole 8192 rows in one pass):
    time per layer, projection TFLOP/s (the layer's flops less the causal attention's, over the
    whole layer time) and the workspace the pass size needs."""
    cfg, B, S = I.CFG3, I.CFG3_BATCH, I.CFG3_PREFILL
    M = B * S
    sl = torch.zeros((1, B), dtype=torch.int32, device=dev)
    x = torch.randn((B, S, cfg.d), device=dev).to(torch.bfloat16)
    y = torch.empty_like(x)
    lay = StackLayer(cfg, dict(cfg.ranks), B, S, S, 11, dev, x, y, sl[0], advance=0)
    r = lay.logical
    d, qd, kd = cfg.d, cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    proj_flops = 2 * M * (r["q"] * (d + qd) + r["k"] * (d + kd) + r["v"] * (d + kd) + r["o"] * (qd + d) +
                          r["gate"] * (d + cfg.d_ff) + r["up"] * (d + cfg.d_ff) + r["down"] * (cfg.d_ff + d))
    out = {"config": "prefill_llama7b_chunks", "batch": B, "seq": S, "rank": r["q"], "passes": []}
    for chunk in chunks:
        lay.desc.prefill_chunk = chunk
        ws = fsvd.workspace(fsvd.fsvd_decoder_layer_ws(lay.desc), device=dev)
        lay.desc.ws, lay.desc.ws_bytes = ws.data_ptr(), ws.numel()

        def layer():
            fsvd.fsvd_decoder_layer_run(lay.desc, stream)

        ms = timed_median(layer, stream)
        assert fsvd.fsvd_poll_device_error(ws, stream) == 0
        out["passes"].append({"chunk_rows": chunk or 8192, "ms_per_layer": round(ms, 4),
                              "tokens_per_s_per_layer": round(M / (ms * 1e-3), 1),
                              "proj_tflops_incl_attention_time": round(proj_flops / (ms * 1e-3) / 1e12, 1),
                              "workspace_bytes": int(ws.numel())})
        del ws
        torch.cuda.empty_cache()
    del lay
    torch.cuda.empty_cache()
    return out


# ----------------------------------------------------------------------------- decode stacks


def cache_len(n):
    """Cache rows for n positions, rounded up to a multiple of 64: each sequence's cache then starts
    on a 64-position boundary, which the decode attention streams measurably faster (batch 4, 32 x 128
    heads, 2048 positions: 27.3 us per call with 2176 rows against 29.8 us with 2049)."""
    return (n + 63) // 64 * 64


def run_decode_stack(name, cfg, ranks, B, history, layers, dev, stream):
    L_max = cache_len(history + 1)
    sl = torch.full((layers, B), history, dtype=torch.int32, device=dev)
    ys = [torch.randn((B, 1, cfg.d), device=dev).to(torch.bfloat16) for _ in range(layers)]
    stack = [StackLayer(cfg, ranks, B, 1, L_max, 2000 + l, dev, ys[(l - 1) % layers], ys[l], sl[l], advance=0)
             for l in range(layers)]
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    ws = fsvd.workspace(fsvd.fsvd_decoder_layer_ws(stack[0].desc), device=dev)
    for lay in stack:
        lay.desc.ws, lay.desc.ws_bytes = ws.data_ptr(), ws.numel()
    fsvd.fsvd_decoder_layer_run(stack[0].desc, stream)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev) - base
    graphs = [fsvd.fsvd_decoder_layer_capture(lay.desc) for lay in stack]
    sg = fsvd.fsvd_decoder_stack_capture([lay.desc for lay in stack])

    def per_layer():
        for g in graphs:
            fsvd.fsvd_graph_replay(g, stream)

    def one_graph():
        fsvd.fsvd_graph_replay(sg, stream)

    def eager():
        for lay in stack:
            fsvd.fsvd_decoder_layer_run(lay.desc, stream)

    us = {k: timed_median(fn, stream) * 1e3 / layers for k, fn in
          (("per_layer_graphs", per_layer), ("one_graph_per_step", one_graph), ("eager", eager))}
    assert fsvd.fsvd_poll_device_error(ws, stream) == 0
    for g in graphs:
        fsvd.fsvd_graph_destroy(g)
    fsvd.fsvd_graph_destroy(sg)
    by = decode_bytes(cfg, ranks, B, history + 1)
    u = us["per_layer_graphs"]
    res = {"config": name, "batch": B, "history": history, "layers": layers, "ranks": ranks,
           "us_per_layer_step": round(u, 2), "tokens_per_s_per_layer": round(B / (u * 1e-6), 1),
           "algorithmic_bytes": int(by), "achieved_gbs": round(by / (u * 1e-6) / 1e9, 1),
           "hbm_frac": round(by / (u * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "comparators_us_per_layer_step": {k: round(v, 2) for k, v in us.items() if k != "per_layer_graphs"},
           "peak_activation_bytes": int(peak)}
    del stack, graphs, ws
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- dense weights vs factors


def run_dense_vs_lowrank(M, dev, stream, copies=4, ratio=None, dense_us=None):
    """The layer's seven projections as plain linears, dense W against the rank-r factors (the
    configured ranks, or every rank at `ratio` of min(dims)); `dense_us` reuses dense timings."""
    c = I.CFG2
    d, dff = c.d, c.d_ff
    shapes = {"q": (d, d), "k": (d, d), "v": (d, d), "o": (d, d), "gate": (d, dff), "up": (d, dff), "down": (dff, d)}
    ranks = dict(c.ranks) if ratio is None else {p: I.rank_of(ratio, *shapes[p]) for p in shapes}
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    bf = fsvd.FSVD_BF16
    res = {"config": f"dense_vs_lowrank_llama7b_m{M}", "rows": M, "projections": {}}
    if ratio is not None:
        res["rank_ratio"] = ratio
    tot_d = tot_l = by_d = by_l = fl_d = fl_l = 0.0
    for name, (K, N) in shapes.items():
        r = ranks[name]
        rs = (r + 31) // 32 * 32  # stored rank, as the layer stores it
        x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        fac, dense = [], []
        for _ in range(copies):
            Ut, Vt = _factor(gen, K, N, r, dev)
            Ut = torch.cat([Ut, torch.zeros((rs - r, K), dtype=Ut.dtype, device=dev)]) if rs > r else Ut
            Vt = pad_cols_dev(Vt, rs)
            fac.append((Ut, Vt))
            if dense_us is None:
                dense.append((Vt.float() @ Ut.float()).to(torch.bfloat16))  # W [N, K] = (U V)^T
        ws = fsvd.workspace(fsvd.fsvd_lowrank_linear_ws(M, K, rs, N, bf), device=dev)
        it = {"d": 0, "l": 0}

        def dense_call():
            W = dense[it["d"] % copies]
            it["d"] += 1
            fsvd.fsvd_dense_linear(x, M, K, K, W, N, K, None, None, N, y, N, bf, stream)

        def lowrank_call():
            Ut, Vt = fac[it["l"] % copies]
            it["l"] += 1
            fsvd.fsvd_lowrank_linear(x, M, K, K, Ut, rs, K, Vt, N, rs, None, None, N, y, N, bf, ws, ws.numel(),
                                     stream)

        t_d = timed_median(dense_call, stream, min_ms=10.0) if dense_us is None else dense_us[name] * 1e-3
        t_l = timed_median(lowrank_call, stream, min_ms=10.0)
        b_d = 2 * (N * K + M * K + M * N)
        b_l = 2 * (r * (K + N) + M * K + M * N)
        f_d, f_l = 2.0 * M * K * N, 2.0 * M * r * (K + N)
        res["projections"][name] = {"K": K, "N": N, "rank": r, "dense_us": round(t_d * 1e3, 2),
                                    "lowrank_us": round(t_l * 1e3, 2)}
        tot_d += t_d; tot_l += t_l; by_d += b_d; by_l += b_l; fl_d += f_d; fl_l += f_l
        del fac, dense, ws
        torch.cuda.empty_cache()
    res.update({"dense_us": round(tot_d * 1e3, 2), "lowrank_us": round(tot_l * 1e3, 2),
                "lowrank_speedup": round(tot_d / tot_l, 3), "dense_bytes": int(by_d), "lowrank_bytes": int(by_l),
                "dense_flops": int(fl_d), "lowrank_flops": int(fl_l)})
    if M <= 32:
        res["dense_frac_of_8tbs"] = round(by_d / (tot_d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        res["lowrank_frac_of_8tbs"] = round(by_l / (tot_l * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    else:
        res["dense_mfma_frac"] = round(fl_d / (tot_d * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
        res["lowrank_mfma_frac"] = round(fl_l / (tot_l * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)
    return res


def run_gemm_vs_vendor(dev, stream, M=8192):
    """The library's MFMA GEMM (fsvd_dense_linear: y = x . W^T) against the vendor GEMM (hipBLASLt,
    through torch.matmul on the same bf16 operands) at the prefill products' shapes."""
    bf = fsvd.FSVD_BF16
    out = {"config": "gemm_vs_vendor_llama7b_shapes", "rows": M, "shapes": []}
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    for K, N in ((4096, 4992), (1664, 4096), (4096, 1664), (4096, 3328), (11008, 1664), (1664, 12288),
                 (4096, 4096)):
        x = torch.randn((M, K), generator=gen, device=dev).to(torch.bfloat16)
        Ws = [torch.randn((N, K), generator=gen, device=dev).to(torch.bfloat16) for _ in range(2)]
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        it = [0]

        def ours():
            fsvd.fsvd_dense_linear(x, M, K, K, Ws[it[0] % 2], N, K, None, None, N, y, N, bf, stream)
            it[0] += 1

        def vendor():
            torch.matmul(x, Ws[it[0] % 2].t(), out=y)
            it[0] += 1

        t_o = timed_median(ours, stream)
        t_v = timed_median(vendor, stream)
        fl = 2.0 * M * K * N
        out["shapes"].append({"K": K, "N": N, "ours_us": round(t_o * 1e3, 1), "vendor_us": round(t_v * 1e3, 1),
                              "ours_mfma_frac": round(fl / (t_o * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                              "vendor_mfma_frac": round(fl / (t_v * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)})
        del x, Ws, y
    return out


def run_dense_vs_lowrank_ratios(M, dev, stream, ratios=(0.1, 0.2, 0.3, 0.4, 0.5, 0.6)):
    """Low-rank speedup over the dense weights against the rank ratio (every projection at `ratio`
    of min(dims)), the dense side timed once."""
    base = run_dense_vs_lowrank(M, dev, stream)
    dense_us = {p: v["dense_us"] for p, v in base["projections"].items()}
    out = {"config": f"dense_vs_lowrank_ratios_llama7b_m{M}", "rows": M, "dense_us": base["dense_us"], "ratios": []}
    for q in ratios:
        r = run_dense_vs_lowrank(M, dev, stream, ratio=q, dense_us=dense_us)
        out["ratios"].append({"rank_ratio": q, "lowrank_us": r["lowrank_us"], "lowrank_speedup": r["lowrank_speedup"],
                              "byte_ratio": round(r["lowrank_bytes"] / r["dense_bytes"], 4),
                              "flop_ratio": round(r["lowrank_flops"] / r["dense_flops"], 4)})
    return out


# ----------------------------------------------------------------------------- dense KV vs low-rank history


def run_attn_history(B, history, dev, stream, copies=4):
    cfg = I.CFG2
    Hq, Hkv, D = cfg.Hq, cfg.Hkv, cfg.D
    r = 1664  # rank 1638 stored padded to a multiple of 32
    n = history + 1          # positions attended (the new token's included)
    L_max = cache_len(n)     # dense cache rows
    L_z = n                  # the low-rank history is rebuilt over every row of its cache
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    bf = torch.bfloat16
    sets = []
    for _ in range(copies):
        sets.append(dict(
            kc=torch.randn((B, L_max, Hkv, D), generator=gen, device=dev).to(bf),
            vc=torch.randn((B, L_max, Hkv, D), generator=gen, device=dev).to(bf),
            zk=torch.randn((B, L_z, r), generator=gen, device=dev).to(bf),
            zv=torch.randn((B, L_z, r), generator=gen, device=dev).to(bf),
            Vk=(torch.randn((Hkv * D, r), generator=gen, device=dev) / math.sqrt(r)).to(bf),
            Vv=(torch.randn((Hkv * D, r), generator=gen, device=dev) / math.sqrt(r)).to(bf)))
    q = torch.randn((B, 1, Hq, D), generator=gen, device=dev).to(bf)
    out = torch.empty_like(q)
    sl = torch.full((B,), history, dtype=torch.int32, device=dev)
    ws_d = fsvd.workspace(fsvd.fsvd_decode_attn_dense_kv_ws(B, 1, Hq, Hkv, D, L_max), device=dev)
    ws_l = fsvd.workspace(fsvd.fsvd_decode_attn_lowrank_kv_ws(B, 1, Hq, Hkv, D, L_z), device=dev)
    it = {"d": 0, "l": 0}

    def dense():
        c = sets[it["d"] % copies]
        it["d"] += 1
        fsvd.fsvd_decode_attn_dense_kv(q, c["kc"], c["vc"], L_max, sl, B, 1, Hq, Hkv, D, 0.0, 1, out, fsvd.FSVD_BF16,
                                       ws_d, ws_d.numel(), stream)

    def lowrank():
        c = sets[it["l"] % copies]
        it["l"] += 1
        fsvd.fsvd_decode_attn_lowrank_kv(q, c["zk"], c["zv"], r, c["Vk"], r, c["Vv"], r, L_z, sl, B, 1, Hq, Hkv, D,
                                         cfg.rope_theta, 0.0, 1, out, fsvd.FSVD_BF16, ws_l, ws_l.numel(), stream)

    # One call over each cache copy, captured into a graph and replayed: launched one by one from
    # Python, a call of a few tens of microseconds would be timed at the host's pace.
    def captured(fn):
        for _ in range(copies):
            fn()  # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for _ in range(copies):
                fn()
        return g

    g_d, g_l = captured(dense), captured(lowrank)
    t_d = timed_median(g_d.replay, stream) * 1e3 / copies
    t_l = timed_median(g_l.replay, stream) * 1e3 / copies
    del g_d, g_l
    assert fsvd.fsvd_poll_device_error(ws_l, stream) == 0
    kv_bytes = 2 * 2 * B * n * Hkv * D
    z_bytes = 2 * 2 * B * n * 1638
    rebuild_flops = 2 * B * n * 2 * 1638 * Hkv * D
    res = {"config": f"attn_lowrank_history_llama7b_b{B}", "batch": B, "history": history, "rank": 1638,
           "dense_kv_us": round(t_d, 2), "lowrank_history_us": round(t_l, 2), "slowdown": round(t_l / t_d, 2),
           "dense_kv_bytes": int(kv_bytes), "lowrank_history_bytes": int(z_bytes),
           "rebuild_flops": int(rebuild_flops),
           "rebuild_tflops": round(rebuild_flops / ((t_l - t_d) * 1e-6) / 1e12, 1) if t_l > t_d else None,
           "lowrank_workspace_bytes": int(ws_l.numel())}
    del sets, ws_l, ws_d
    torch.cuda.empty_cache()
    return res


# ----------------------------------------------------------------------------- factorised attention


def run_attn_factorized(name, B, S, H, D, r, theta, causal, dev, stream):
    gen = torch.Generator(device=dev)
    gen.manual_seed(8)
    bf = torch.bfloat16
    M = B * S
    z = torch.randn((M, 3 * r), generator=gen, device=dev).to(bf)  # packed [z_q | z_k | z_v]
    Vq, Vk, Vv = ((torch.randn((H * D, r), generator=gen, device=dev) / math.sqrt(r)).to(bf) for _ in range(3))
    out = torch.empty((B, S, H, D), dtype=bf, device=dev)
    # the materialised operands of the dense path: q [B, S, H, D] and the K/V cache rows
    q = torch.randn((B, S, H, D), generator=gen, device=dev).to(bf)
    kc = torch.randn((B, S, H, D), generator=gen, device=dev).to(bf)
    vc = torch.randn((B, S, H, D), generator=gen, device=dev).to(bf)
    sl = torch.zeros(B, dtype=torch.int32, device=dev)
    ws = fsvd.workspace(fsvd.fsvd_decode_attn_dense_kv_ws(B, S, H, H, D, S), device=dev)

    def fact():
        fsvd.fsvd_attn_factorized(z, z[:, r:], z[:, 2 * r:], 3 * r, Vq, r, Vk, r, Vv, r, B, S, H, H, D, theta, 0.0,
                                  int(causal), out, fsvd.FSVD_BF16, stream)

    def dense():
        fsvd.fsvd_decode_attn_dense_kv(q, kc, vc, S, sl, B, S, H, H, D, 0.0, int(causal), out, fsvd.FSVD_BF16, ws,
                                       ws.numel(), stream)

    t_f = timed_median(fact, stream)
    t_d = timed_median(dense, stream)
    qkv_bytes = 3 * M * H * D * 2
    return {"config": name, "batch": B, "seq": S, "heads": H, "head_dim": D, "rank": r, "causal": causal,
            "factorized_ms": round(t_f, 4), "dense_attention_ms": round(t_d, 4),
            "qkv_bytes_not_written": int(qkv_bytes),
            "note": "factorized = Q/K/V rebuilt from z inside the attention; dense = attention over materialised "
                    "q, K, V (their phase-2 products are not in dense_attention_ms)"}


# ----------------------------------------------------------------------------- Swift-SVD covariance


def run_swift_covariance(dev, stream, d=4096, T=4096):
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    Wt = (torch.randn((d, d), generator=gen, device=dev) / math.sqrt(d)).to(torch.bfloat16)
    Xs = [torch.randn((T, d), generator=gen, device=dev).to(torch.bfloat16) for _ in range(4)]
    C = torch.zeros((d, d), dtype=torch.float32, device=dev)
    ws = fsvd.workspace(fsvd.fsvd_swift_covariance_ws(T, d, d), device=dev)
    it = {"i": 0}

    def call():
        X = Xs[it["i"] % len(Xs)]
        it["i"] += 1
        fsvd.fsvd_swift_covariance(X, T, d, d, Wt, d, C, d, ws, ws.numel(), stream)

    ms = timed_median(call, stream)
    flops = 2 * T * d * d + d * (d + 1) * T  # Y^T = W^T X^T, then the upper half of Y^T Y
    return {"config": "swift_covariance_4096", "d_in": d, "d_out": d, "tokens": T, "ms_per_batch": round(ms, 4),
            "flops": int(flops), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", default="", help="comma-separated subset of the measurement names")
    args = ap.parse_args()
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)
    runs = [("linear_fp32", lambda: run_linear_fp32(dev, stream)),
            ("bert_layer", lambda: run_bert_layer(dev, stream)),
            ("prefill_llama7b_chunks", lambda: run_prefill_chunks(dev, stream))]
    for B in I.CFG2_BATCHES:
        runs.append((f"decode_llama7b_b{B}",
                     lambda B=B: run_decode_stack(f"decode_llama7b_b{B}", I.CFG2, dict(I.CFG2.ranks), B,
                                                  I.CFG2_KV_LEN, 4, dev, stream)))
    runs.append(("decode_llama3_8b_gqa_b32",
                 lambda: run_decode_stack("decode_llama3_8b_gqa_b32", I.CFG4, dict(I.CFG4.ranks), I.CFG4_BATCH,
                                          I.CFG4_KV_LEN, 4, dev, stream)))
    runs.append(("swift_covariance_4096", lambda: run_swift_covariance(dev, stream)))
    runs.append(("attn_factorized_bert", lambda: run_attn_factorized("attn_factorized_bert", 8, 512, 12, 64, 384, 0.0,
                                                                     False, dev, stream)))
    runs.append(("attn_factorized_llama7b_s2048",
                 lambda: run_attn_factorized("attn_factorized_llama7b_s2048", 1, 2048, 32, 128, 1664, 1e4, True, dev,
                                             stream)))
    for M in (1, 4, 8192):
        runs.append((f"dense_vs_lowrank_llama7b_m{M}", lambda M=M: run_dense_vs_lowrank(M, dev, stream)))
    runs.append(("gemm_vs_vendor_llama7b_shapes", lambda: run_gemm_vs_vendor(dev, stream)))
    for M in (1, 4, 8192):
        runs.append((f"dense_vs_lowrank_ratios_llama7b_m{M}", lambda M=M: run_dense_vs_lowrank_ratios(M, dev, stream)))
    for B in (1, 4):
        runs.append((f"attn_lowrank_history_llama7b_b{B}", lambda B=B: run_attn_history(B, 2048, dev, stream)))
    only = set(filter(None, args.only.split(",")))
    for name, fn in runs:
        if only and name not in only:
            continue
        log(name, "...")
        print(json.dumps(fn()), flush=True)


if __name__ == "__main__":
    main()
