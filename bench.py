"""Benchmark of the fused low-rank layer hot path on one MI355X.

Workload (one "step"): a stack of distinct Llama-7B-shaped low-rank decoder layers (hidden 4096,
32 heads x 128, SwiGLU 11008 with packed gate|up factors, every rank 40% -> 1638, stored padded
to 1664), batch 4: prefill of 2048 tokens per sequence through every layer (bf16 MFMA path,
dense KV written), then 128 decode steps, each one hipGraph replay per layer.  The stack holds
several layer copies (weights and KV caches) so the working set far exceeds the 256 MB
Infinity Cache.  Inputs are seeded synthetic draws (see svd_compressed_transformer_amd.inputs).

Prints ONE JSON line.  value = layer-tokens per second over the whole step (prefill and decode
tokens, each counted once per layer it passes through).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode & prefill tokens/s per low-rank layer; % HBM BW / % MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# HBM bytes per decode-attention call, from counter runs of this script (FETCH_SIZE and
# WRITE_SIZE, calibrated on a plain copy of known size); valid only for the kernel source whose
# hash the summary records
TRAFFIC_NOTE = os.path.join(ROOT, "profiles", "attn_decode_dense_kv_llama7b_b4_hbm_traffic.md")
ATTN_SRC = os.path.join(ROOT, "svd_compressed_transformer_amd", "csrc", "attention.hip")
CAL_COPY_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=4, help="distinct layer copies in the stack")
    ap.add_argument("--decode-steps", type=int, default=128)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    return ap.parse_args()


# ----------------------------------------------------------------------------- algorithmic work


def layer_bytes_decode(cfg, B, L_read, logical_ranks):
    """Algorithmic HBM bytes of one decode layer-step: every factor byte once (logical ranks),
    the KV cache read once (L_read positions), the new K/V written, layer input/output, norms."""
    d, qd, kd = cfg.d, cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    r = logical_ranks
    fac = 2 * (r["q"] * (d + qd) + r["k"] * (d + kd) + r["v"] * (d + kd) + r["o"] * (qd + d) +
               r["gate"] * (d + cfg.d_ff) + r["up"] * (d + cfg.d_ff) + r["down"] * (cfg.d_ff + d))
    kv = 2 * 2 * B * L_read * kd + 2 * 2 * B * kd
    io = 2 * 2 * B * d + 2 * 2 * d
    return fac + kv + io


def attn_decode_bytes(cfg, B, L_read):
    """Algorithmic bytes of the decode attention kernel: K and V read once over L_read positions,
    q read, output written."""
    kd = cfg.Hkv * cfg.D
    return 2 * 2 * B * L_read * kd + 2 * 2 * B * cfg.Hq * cfg.D


def layer_flops_prefill(cfg, M, r):
    d, qd, kd = cfg.d, cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    proj = 2 * M * (r["q"] * (d + qd) + r["k"] * (d + kd) + r["v"] * (d + kd) + r["o"] * (qd + d) +
                    r["gate"] * (d + cfg.d_ff) + r["up"] * (d + cfg.d_ff) + r["down"] * (cfg.d_ff + d))
    return proj


def attn_flops_prefill(cfg, B, S):
    """Causal attention of S tokens per sequence: q.k and p.v over the keys each query sees."""
    return 4 * B * cfg.Hq * cfg.D * (S * (S + 1) // 2)


def unfused_prefill_bytes(cfg, B, S, r):
    """Activation bytes an unfused low-rank prefill layer would hold (bf16, scores fp32): layer I/O,
    the normalised inputs, z of every projection, q, o, h, g, u, t and the naive attention scores."""
    M = B * S
    qd = cfg.Hq * cfg.D
    z = M * (r["q"] + r["k"] + r["v"] + r["o"] + r["gate"] + r["up"] + r["down"])
    return 2 * (2 * M * cfg.d + 2 * M * cfg.d + z + 2 * M * qd + M * cfg.d + 3 * M * cfg.d_ff) + \
        4 * B * cfg.Hq * S * S


def recorded_traffic():
    """Measured HBM bytes per decode-attention call, or None when no summary exists or the kernel
    source changed since the counters were taken."""
    try:
        with open(TRAFFIC_NOTE) as f:
            txt = f.read()
        with open(ATTN_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    m_sha = re.search(r"attention\.hip sha256: ([0-9a-f]{64})", txt)
    m_val = re.search(r"traffic_bytes_per_call: (\d+)", txt)
    if not (m_sha and m_val) or m_sha.group(1) != sha:
        return None
    return int(m_val.group(1))


# ----------------------------------------------------------------------------- CPU oracle baseline


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1]), \
            ",".join(sorted({i.get("internal_api", "?") for i in threadpool_info()}))
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0)), "?"


def _median_rate(fn, runs=3):
    """Median over runs of (work units, seconds) -> units/s."""
    rates = []
    for _ in range(runs):
        units, sec = fn()
        rates.append(units / sec)
    return float(np.median(rates))


def cpu_baseline(cfg, prefill_tokens_per_layer, decode_tokens_per_layer):
    """The fp64 oracle, as it stands, on bounded samples of the benchmark's own units, on this
    host's cores: the prefill of one 512-token sequence through one full-size layer (tokens/s per
    layer) and 10 batch-4 decode layer-steps over a 2048-token history (tokens/s per layer), each the
    median of 3 runs; plus single-thread figures for the fp32 linear (x 16 x 256, rank 64) and one
    batch-1 decode layer-step.  ``value`` is the step's mix of prefill and decode tokens (the GPU
    line's unit) at those two rates."""
    from oracle import fsvd_oracle as O
    from svd_compressed_transformer_amd import inputs as I
    threads, blas = _blas_threads()
    t_all = time.perf_counter()
    S_pre = 512
    p = I.make_decoder_layer(cfg, B=1, S=S_pre, seed=100)
    z = np.zeros((1, S_pre, cfg.Hkv, cfg.D))

    def prefill():
        t0 = time.perf_counter()
        O.decoder_layer(p["x"], p, cfg, z, z, np.zeros(1, dtype=np.int64))
        return S_pre, time.perf_counter() - t0

    r_pre = _median_rate(prefill)
    B, L = 4, 2048
    n_dec = 10  # decode steps per run: with the prefill, about 10-15 s of CPU work in all
    kc, vc = I.make_kv_history(B, L + n_dec, cfg.Hkv, cfg.D, L, seed=101)
    rng = np.random.default_rng(102)
    xs = [I.round_bf16(rng.standard_normal((B, 1, cfg.d))) for _ in range(n_dec)]

    def decode():
        sl = np.full(B, L)
        k, v = kc, vc
        t0 = time.perf_counter()
        for x in xs:
            _, k, v = O.decoder_layer(x, p, cfg, k, v, sl)
            sl = sl + 1
        return B * len(xs), time.perf_counter() - t0

    r_dec = _median_rate(decode)
    # single thread: the fp32 linear and one batch-1 decode layer-step
    single = {}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            c = I.make_linear_case(I.CFG0)

            def lin():
                t0 = time.perf_counter()
                for _ in range(200):
                    O.lowrank_linear(c["x"], c["Ut"], c["Vt"])
                return 200, time.perf_counter() - t0

            single["linear_fp32_calls_per_s"] = round(_median_rate(lin), 1)

            def dec1():
                t0 = time.perf_counter()
                O.decoder_layer(xs[0][:1], p, cfg, kc[:1], vc[:1], np.full(1, L))
                return 1, time.perf_counter() - t0

            single["decode_b1_tokens_per_s_per_layer"] = round(_median_rate(dec1), 3)
    except Exception as e:  # pragma: no cover
        single["error"] = str(e)
    t_step = prefill_tokens_per_layer / r_pre + decode_tokens_per_layer / r_dec
    value = (prefill_tokens_per_layer + decode_tokens_per_layer) / t_step
    return {"value": round(value, 3), "unit": "tokens/s per layer", "cores": int(threads), "kind": "oracle",
            "blas": blas,
            "prefill_tokens_per_s_per_layer": round(r_pre, 2), "decode_tokens_per_s_per_layer": round(r_dec, 3),
            "single_thread": single,
            "sample": f"numpy fp64 oracle, one full-size layer: prefill of 1 x {S_pre} tokens and {n_dec} decode "
                      f"steps at batch 4 over history {L}, median of 3 runs each; value = the benchmark step's "
                      f"mix ({prefill_tokens_per_layer} prefill + {decode_tokens_per_layer} decode tokens per layer) "
                      f"at those rates; {time.perf_counter() - t_all:.1f} s of CPU work"}


# ----------------------------------------------------------------------------- GPU run


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the multi-GPU split is a design "
              "note, not a run", file=sys.stderr)
        sys.exit(2)
    import torch
    from svd_compressed_transformer_amd import fsvd, inputs as I
    from svd_compressed_transformer_amd.device import DeviceLayer, to_dev

    cfg = I.CFG3
    B, S, ND, NL = I.CFG3_BATCH, I.CFG3_PREFILL, args.decode_steps, args.layers
    L_max = S + ND
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.set_stream(stream)

    log(f"building {NL} layers ...")
    layers_pre, layers_dec = [], []
    sl_all = torch.zeros((NL, B), dtype=torch.int32, device=dev)
    xs_pre = [torch.empty((B, S, cfg.d), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    ys_dec = [torch.empty((B, 1, cfg.d), dtype=torch.bfloat16, device=dev) for _ in range(NL)]
    logical = dict(cfg.ranks)
    x0 = None
    for l in range(NL):
        p = I.make_decoder_layer(cfg, B=B, S=S, seed=l)
        if x0 is None:
            x0 = p["x"]
        pre = DeviceLayer(cfg, p, B=B, S=S, L_max=L_max, kc=None, vc=None, seqlens=np.zeros(B), device=dev,
                          advance=True, x=np.zeros((B, S, cfg.d), np.float32), fold_norm=True)
        del p
        # prefill reads/writes the ping-pong activation buffers and this layer's cache / seqlens
        pre.desc.x = xs_pre[l % 2].data_ptr()
        pre.desc.y = xs_pre[(l + 1) % 2].data_ptr()
        pre.desc.cache_seqlens = sl_all[l].data_ptr()
        layers_pre.append(pre)
        torch.cuda.synchronize()
        log(f"  layer {l} ready")
    xs_pre[0].copy_(to_dev(x0, device=dev).reshape(B, S, cfg.d))
    del x0
    # decode descriptors share each layer's factors and cache; one decode workspace for all
    import ctypes
    dec_ws = None
    for l, pre in enumerate(layers_pre):
        d = type(pre.desc)()
        ctypes.memmove(ctypes.addressof(d), ctypes.addressof(pre.desc), ctypes.sizeof(d))
        d.S = 1
        d.x = ys_dec[(l - 1) % NL].data_ptr()
        d.y = ys_dec[l].data_ptr()
        d.advance_seqlens = 1
        if dec_ws is None:
            dec_ws = fsvd.workspace(fsvd.fsvd_decoder_layer_ws(d), device=dev)
        d.ws = dec_ws.data_ptr()
        d.ws_bytes = dec_ws.numel()
        layers_dec.append(d)
    # the prefill workspaces are the same size: keep one and point every prefill layer at it
    pre_ws = layers_pre[0].ws
    for pre in layers_pre[1:]:
        pre.ws = None
        pre.desc.ws = pre_ws.data_ptr()
        pre.desc.ws_bytes = pre_ws.numel()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    graphs = [fsvd.fsvd_decoder_layer_capture(d) for d in layers_dec]

    def step(mid=None):
        sl_all.zero_()
        for pre in layers_pre:
            fsvd.fsvd_decoder_layer_run(pre.desc, stream)
        if mid is not None:
            mid.record(stream)  # end of the prefill half
        ys_dec[NL - 1].copy_(xs_pre[NL % 2][:, S - 1:S, :])
        for _ in range(ND):
            for g in graphs:
                fsvd.fsvd_graph_replay(g, stream)

    # warmup (the first pass pays first-touch and first-launch costs), with the two halves logged
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    for w in range(max(1, args.warmup)):
        sl_all.zero_()
        e[0].record(stream)
        for pre in layers_pre:
            fsvd.fsvd_decoder_layer_run(pre.desc, stream)
        e[1].record(stream)
        ys_dec[NL - 1].copy_(xs_pre[NL % 2][:, S - 1:S, :])
        for _ in range(ND):
            for g in graphs:
                fsvd.fsvd_graph_replay(g, stream)
        e[2].record(stream)
        torch.cuda.synchronize()
        log(f"warmup {w}: prefill {e[0].elapsed_time(e[1]):.2f} ms, decode {e[1].elapsed_time(e[2]):.2f} ms")

    # a plain device copy of known size (256 MiB read, 256 MiB written): the calibration point of
    # the HBM byte counters in a counter-collection run of this script
    cal_src = torch.zeros(CAL_COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    cal_dst = torch.empty_like(cal_src)
    cal_dst.copy_(cal_src)
    torch.cuda.synchronize()
    del cal_src, cal_dst
    torch.cuda.empty_cache()
    assert fsvd.fsvd_poll_device_error(dec_ws, stream) == 0
    assert fsvd.fsvd_poll_device_error(pre_ws, stream) == 0

    torch.cuda.synchronize()
    # timed steps; an event at the end of each step's prefill half splits the step into its prefill
    # and decode halves (reported below as the means over the timed steps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2 * args.steps + 1)]
    ev[0].record(stream)
    for k in range(args.steps):
        step(mid=ev[2 * k + 1])
        ev[2 * k + 2].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[-1]) / args.steps
    t_pre_ms = sum(ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(args.steps)) / args.steps
    t_dec_ms = sum(ev[2 * k + 1].elapsed_time(ev[2 * k + 2]) for k in range(args.steps)) / args.steps
    log(f"timed: {args.steps} steps, {ms:.2f} ms/step (prefill {t_pre_ms:.2f} ms, decode {t_dec_ms:.2f} ms)")

    # ------------------------------------------------ dominant kernel: decode attention, timed live
    # The decode-attention kernel (the largest single consumer of bytes in the step) timed with
    # HIP events on the benchmark stream, on a layer's own cache at the mean decode length.
    lay = layers_dec[0]
    q = torch.empty((B, 1, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=dev).normal_()
    out = torch.empty_like(q)
    L_mid = S + ND // 2
    sl_mid = torch.full((B,), L_mid - 1, dtype=torch.int32, device=dev)
    a_ws = fsvd.workspace(fsvd.fsvd_decode_attn_dense_kv_ws(B, 1, cfg.Hq, cfg.Hkv, cfg.D, L_max), device=dev)
    kcs = [pre.k_cache for pre in layers_pre]
    vcs = [pre.v_cache for pre in layers_pre]
    for _ in range(3):
        fsvd.fsvd_decode_attn_dense_kv(q, kcs[0], vcs[0], L_max, sl_mid, B, 1, cfg.Hq, cfg.Hkv, cfg.D, 0.0, 1, out,
                                       fsvd.FSVD_BF16, a_ws, a_ws.numel(), stream)
    n_rep = 64
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for i in range(n_rep):
        l = i % NL
        fsvd.fsvd_decode_attn_dense_kv(q, kcs[l], vcs[l], L_max, sl_mid, B, 1, cfg.Hq, cfg.Hkv, cfg.D, 0.0, 1, out,
                                       fsvd.FSVD_BF16, a_ws, a_ws.numel(), stream)
    eb.record(stream)
    torch.cuda.synchronize()
    attn_us = ea.elapsed_time(eb) * 1e3 / n_rep
    attn_bytes = attn_decode_bytes(cfg, B, L_mid)
    attn_gbs = attn_bytes / (attn_us * 1e-6) / 1e9

    # ------------------------------------------------ comparator: one graph per decode step
    # The measured configuration replays one graph per layer (the pages' design).  For comparison,
    # the same decode steps with all layers captured into one graph, from the same state.
    stack_g = fsvd.fsvd_decoder_stack_capture(layers_dec)
    for run in range(2):  # the first pass warms the graph up
        sl_all.fill_(S)
        ys_dec[NL - 1].copy_(xs_pre[NL % 2][:, S - 1:S, :])
        torch.cuda.synchronize()
        ea.record(stream)
        for _ in range(ND):
            fsvd.fsvd_graph_replay(stack_g, stream)
        eb.record(stream)
        torch.cuda.synchronize()
    t_dec_stack_ms = ea.elapsed_time(eb)
    fsvd.fsvd_graph_destroy(stack_g)

    # ------------------------------------------------ prefill attention, timed live
    # The causal attention of the prefill (the MFMA attention kernel over each layer's cache), so the
    # projections' share of the prefill time and the whole prefill's flops can be reported apart.
    qp = torch.empty((B, S, cfg.Hq, cfg.D), dtype=torch.bfloat16, device=dev).normal_()
    op = torch.empty_like(qp)
    sl0 = torch.zeros((B,), dtype=torch.int32, device=dev)
    pa_ws = fsvd.workspace(fsvd.fsvd_decode_attn_dense_kv_ws(B, S, cfg.Hq, cfg.Hkv, cfg.D, L_max), device=dev)

    def prefill_attn(l):
        fsvd.fsvd_decode_attn_dense_kv(qp, kcs[l], vcs[l], L_max, sl0, B, S, cfg.Hq, cfg.Hkv, cfg.D, 0.0, 1, op,
                                       fsvd.FSVD_BF16, pa_ws, pa_ws.numel(), stream)

    for l in range(NL):
        prefill_attn(l)
    ea.record(stream)
    for rep in range(3):
        for l in range(NL):
            prefill_attn(l)
    eb.record(stream)
    torch.cuda.synchronize()
    t_pattn_ms = ea.elapsed_time(eb) / 3  # per stack pass (NL layers)
    del qp, op

    # ------------------------------------------------ peak activation bytes (torch's allocator)
    # Everything one prefill layer call holds beyond its inputs, weights and KV cache: the
    # workspace the call needs and its output, from the allocator's peak across the call; at the
    # default pass size (the whole 4 x 2048 prefill in one pass) and at 2048-row passes, with the
    # 2048-row passes also timed over the stack.
    def one_layer_peak(chunk):
        d = type(layers_pre[0].desc)()
        ctypes.memmove(ctypes.addressof(d), ctypes.addressof(layers_pre[0].desc), ctypes.sizeof(d))
        d.prefill_chunk = chunk
        d.advance_seqlens = 0
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        ws = fsvd.workspace(fsvd.fsvd_decoder_layer_ws(d), device=dev)
        y = torch.empty((B, S, cfg.d), dtype=torch.bfloat16, device=dev)
        d.ws, d.ws_bytes, d.y = ws.data_ptr(), ws.numel(), y.data_ptr()
        sl_all[0].zero_()
        fsvd.fsvd_decoder_layer_run(d, stream)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated(dev) - base
        return {"chunk_rows": chunk or 8192, "allocator_peak": int(peak), "workspace": int(ws.numel())}

    act = {"cfg3_prefill_layer": one_layer_peak(0), "cfg3_prefill_layer_chunk2048": one_layer_peak(2048)}
    act["unfused_count_cfg3"] = int(unfused_prefill_bytes(cfg, B, S, logical))
    # the 2048-row passes over the whole stack: time against the default
    ws2 = fsvd.workspace(act["cfg3_prefill_layer_chunk2048"]["workspace"], device=dev)
    saved = [(pre.desc.prefill_chunk, pre.desc.ws, pre.desc.ws_bytes) for pre in layers_pre]
    for pre in layers_pre:
        pre.desc.prefill_chunk = 2048
        pre.desc.ws, pre.desc.ws_bytes = ws2.data_ptr(), ws2.numel()
    t_chunk = []
    for rep in range(3):
        sl_all.zero_()
        ea.record(stream)
        for pre in layers_pre:
            fsvd.fsvd_decoder_layer_run(pre.desc, stream)
        eb.record(stream)
        torch.cuda.synchronize()
        t_chunk.append(ea.elapsed_time(eb))
    for pre, (c, w, wb) in zip(layers_pre, saved):
        pre.desc.prefill_chunk, pre.desc.ws, pre.desc.ws_bytes = c, w, wb
    act["cfg3_prefill_layer_chunk2048"]["prefill_ms_per_stack"] = round(float(np.median(t_chunk[1:])), 3)
    act["decode_workspace_bytes"] = int(dec_ws.numel())
    assert fsvd.fsvd_poll_device_error(ws2, stream) == 0
    del ws2

    # ------------------------------------------------ measured stream bandwidth of this part
    # The library's read-stream probe (every byte of 4 GiB read once with 16-byte non-temporal
    # loads) and a torch device copy (1 GiB read + 1 GiB written), beside the 8 TB/s specification.
    big = torch.empty((2 << 30,), dtype=torch.bfloat16, device=dev).normal_()
    sink = torch.zeros((64,), dtype=torch.int32, device=dev)
    nbytes = big.numel() * 2
    for _ in range(2):
        fsvd.fsvd_read_stream_probe(big, nbytes, sink, stream)
    ea.record(stream)
    for _ in range(5):
        fsvd.fsvd_read_stream_probe(big, nbytes, sink, stream)
    eb.record(stream)
    torch.cuda.synchronize()
    read_gbs = 5 * nbytes / (ea.elapsed_time(eb) * 1e-3) / 1e9
    half = big[: big.numel() // 4]
    dst = torch.empty_like(half)
    dst.copy_(half)
    ea.record(stream)
    for _ in range(5):
        dst.copy_(half)
    eb.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * half.numel() * 2 / (ea.elapsed_time(eb) * 1e-3) / 1e9
    del big, half, dst, sink
    torch.cuda.empty_cache()

    # ------------------------------------------------ the BERT-Base encoder layer (8 x 512, rank 384)
    from svd_compressed_transformer_amd import configs as CF
    bert = CF.run_bert_layer(dev, stream)
    act["cfg1_bert_layer"] = {"allocator_peak": bert["peak_activation_bytes"],
                              "unfused_count": bert["unfused_activation_bytes"]}

    # ------------------------------------------------ report
    M = B * S
    tok_layers = (M + B * ND) * NL
    value = tok_layers / (ms * 1e-3)
    dec_bytes = sum(layer_bytes_decode(cfg, B, S + t + 1, logical) for t in range(ND)) * NL
    dec_gbs = dec_bytes / (t_dec_ms * 1e-3) / 1e9
    proj_flops = layer_flops_prefill(cfg, M, logical) * NL
    attn_flops = attn_flops_prefill(cfg, B, S) * NL
    t_proj_ms = t_pre_ms - t_pattn_ms
    proj_tflops = proj_flops / (t_proj_ms * 1e-3) / 1e12
    whole_tflops = (proj_flops + attn_flops) / (t_pre_ms * 1e-3) / 1e12

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, random low-rank factors of the stated shapes)",
        "config": {"workload": "llama-7b-shaped low-rank layer stack: prefill 4x2048 then 128 graph-replayed "
                               "decode steps (batch 4)",
                   "layers": NL, "batch": B, "prefill_len": S, "decode_steps": ND, "hidden": cfg.d,
                   "heads": cfg.Hq, "head_dim": cfg.D, "d_ff": cfg.d_ff, "rank": logical["q"], "stored_rank": int(layers_pre[0].ranks["r_q"])},
        "prefill": {"ms": round(t_pre_ms, 3), "tokens_per_s_per_layer": round(M * NL / (t_pre_ms * 1e-3), 1),
                    "attention_ms": round(t_pattn_ms, 3),
                    "proj_tflops": round(proj_tflops, 1), "proj_mfma_frac": round(proj_tflops / BF16_PEAK_TFLOPS, 4),
                    "whole_tflops": round(whole_tflops, 1),
                    "whole_mfma_frac": round(whole_tflops / BF16_PEAK_TFLOPS, 4),
                    "note": "proj: projection flops over the prefill time less the live-timed attention (RMSNorm "
                            "statistics kernels stay in); whole: projection + causal attention flops over the "
                            "whole prefill time"},
        "decode": {"ms": round(t_dec_ms, 3), "tokens_per_s_per_layer": round(B * ND * NL / (t_dec_ms * 1e-3), 1),
                   "us_per_layer_step": round(t_dec_ms * 1e3 / (ND * NL), 2),
                   "algorithmic_gbs": round(dec_gbs, 1), "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
                   "hbm_frac_of_measured_read": round(dec_gbs / read_gbs, 4),
                   "one_graph_per_step": {"ms": round(t_dec_stack_ms, 3),
                                          "us_per_layer_step": round(t_dec_stack_ms * 1e3 / (ND * NL), 2)}},
        "roofline": {"bound": "hbm", "kernel": "attn_decode_split", "achieved": round(attn_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(), "avg_us": round(attn_us, 2),
                     "algorithmic_bytes": int(attn_bytes), "kv_positions": int(L_mid),
                     "frac_of_measured_read": round(attn_gbs / read_gbs, 4)},
        "measured_stream_gbs": {"read": round(read_gbs, 1), "copy": round(copy_gbs, 1),
                                "note": "fsvd_read_stream_probe over 4 GiB (read) and a 1 GiB torch device copy (read + write)"},
        "peak_activation_bytes": act,
        "bert_layer": {"ms": bert["ms_per_layer"], "tokens_per_s_per_layer": bert["tokens_per_s_per_layer"],
                       "proj_tflops": bert["projections"]["tflops"],
                       "proj_mfma_frac": bert["projections"]["mfma_frac"]},
    }
    if not args.no_cpu:
        log("cpu oracle baseline ...")
        res["cpu_baseline"] = cpu_baseline(cfg, M, B * ND)
    for g in graphs:
        fsvd.fsvd_graph_destroy(g)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
