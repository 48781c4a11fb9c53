"""GPU parity of the whole decoder layer (eager and per-layer hipGraph replay) against the oracle.

Graph replay changes launch overhead, not arithmetic: N replays must equal N eager steps bit
for bit (the kernels are deterministic), and both must match the oracle's N-step composition.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import fsvd_oracle as O  # noqa: E402
from svd_compressed_transformer_amd import fsvd, inputs as I  # noqa: E402
from svd_compressed_transformer_amd.device import DeviceLayer, bits, from_dev, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def say(*a):
    print(*a, flush=True)


SMALL = I.scaled_decoder(I.CFG2, d=512, Hq=8, Hkv=8, D=64, d_ff=768,
                         ranks={"q": 200, "k": 200, "v": 200, "o": 200, "gate": 300, "up": 300, "down": 300})
SMALL_GQA = I.scaled_decoder(I.CFG4, d=512, Hq=8, Hkv=2, D=128, d_ff=1024,
                             ranks={"q": 256, "k": 128, "v": 64, "o": 192, "gate": 128, "up": 256, "down": 96})


@pytest.mark.parametrize("cfg,B,L0,fold", [(SMALL, 1, 0, False), (SMALL, 3, 45, False), (SMALL_GQA, 4, 130, False),
                                            (SMALL_GQA, 32, 17, False), (SMALL, 3, 45, True), (SMALL_GQA, 32, 17, True)])
def test_decode_layer_eager(cfg, B, L0, fold):
    """fold: RMSNorm weights folded into A_qkv / A_gu (FSVD_LAYER_NORM_FOLDED); the oracle keeps
    them separate."""
    L_max = 160
    say("decode layer eager", cfg.name, B, L0, "folded" if fold else "")
    p = I.make_decoder_layer(cfg, B=B, S=1, seed=B, random_norm_weights=True)
    kc, vc = I.make_kv_history(B, L_max, cfg.Hkv, cfg.D, L0, seed=11)
    lay = DeviceLayer(cfg, p, B=B, S=1, L_max=L_max, kc=kc, vc=vc, seqlens=np.full(B, L0), fold_norm=fold)
    lay.run()
    torch.cuda.synchronize()
    y_ref, kc_ref, vc_ref = O.decoder_layer(p["x"], p, cfg, kc, vc, np.full(B, L0))
    assert rel(lay.y_host(), y_ref) <= BF16_TOL
    assert rel(from_dev(lay.k_cache)[:, L0], kc_ref[:, L0]) <= BF16_TOL
    assert fsvd.fsvd_poll_device_error(lay.ws) == 0


@pytest.mark.parametrize("fold", [False, True])
def test_prefill_layer_small_rowdot_path(fold):
    """S > 1 with M = B*S <= 32 exercises the row-dot kernels with several tokens per sequence."""
    cfg = SMALL_GQA
    B, S, L_max = 2, 5, 64
    say("prefill layer (row-dot sizes)", "folded" if fold else "")
    p = I.make_decoder_layer(cfg, B=B, S=S, seed=21, random_norm_weights=True)
    lay = DeviceLayer(cfg, p, B=B, S=S, L_max=L_max, kc=None, vc=None, seqlens=[0, 9], fold_norm=fold)
    lay.run()
    torch.cuda.synchronize()
    z = np.zeros((B, L_max, cfg.Hkv, cfg.D))
    y_ref, _, _ = O.decoder_layer(p["x"], p, cfg, z, z, [0, 9])
    assert rel(lay.y_host(), y_ref) <= BF16_TOL


# batch 8 and 12 run the projections on the matrix cores, and phase 1 of the small GQA layer splits
# its reduction over workgroups (a reduce kernel in the graph)
@pytest.mark.parametrize("cfg,B,fold", [(SMALL, 2, False), (SMALL_GQA, 4, False), (SMALL_GQA, 4, True),
                                        (SMALL_GQA, 8, False), (SMALL, 12, True)])
def test_graph_replay_equals_eager_and_oracle(cfg, B, fold):
    L_max, L0, N = 96, 20, 6
    say("graph replay", cfg.name, B, "folded" if fold else "")
    p = I.make_decoder_layer(cfg, B=B, S=1, seed=5, random_norm_weights=True)
    kc, vc = I.make_kv_history(B, L_max, cfg.Hkv, cfg.D, L0, seed=12)
    rng = np.random.default_rng(99)
    xs = I.round_bf16(rng.standard_normal((N, B, cfg.d)))

    eager = DeviceLayer(cfg, p, B=B, S=1, L_max=L_max, kc=kc, vc=vc, seqlens=np.full(B, L0), advance=True,
                        fold_norm=fold)
    graph_l = DeviceLayer(cfg, p, B=B, S=1, L_max=L_max, kc=kc, vc=vc, seqlens=np.full(B, L0), advance=True,
                          fold_norm=fold)
    g = graph_l.capture()
    try:
        ys_e, ys_g = [], []
        for t in range(N):
            xt = to_dev(xs[t]).reshape(B, 1, cfg.d)
            eager.x.copy_(xt)
            graph_l.x.copy_(xt)
            eager.run()
            fsvd.fsvd_graph_replay(g)
            torch.cuda.synchronize()
            ys_e.append(bits(eager.y))
            ys_g.append(bits(graph_l.y))
        for t in range(N):
            assert np.array_equal(ys_e[t], ys_g[t]), f"replay {t} differs from eager"
        assert np.array_equal(bits(eager.k_cache), bits(graph_l.k_cache))
        assert list(graph_l.seqlens.cpu().numpy()) == [L0 + N] * B
        y_ref, _, _, sl = O.decoder_steps(xs, p, cfg, kc, vc, np.full(B, L0))
        got = np.stack([from_dev(torch.from_numpy(y.view(np.int16)).view(torch.bfloat16)).reshape(B, cfg.d)
                        for y in ys_g])
        assert rel(got, y_ref) <= BF16_TOL
    finally:
        fsvd.fsvd_graph_destroy(g)
    with pytest.raises(fsvd.FsvdError):
        fsvd.fsvd_graph_replay(g)


def test_stack_graph_equals_per_layer_graphs_and_oracle_chain():
    """Three layers chained (y of layer l is x of layer l+1): one whole-stack graph replay per step
    gives the same bits as three per-layer graph replays, step after step, and both follow the
    oracle applied layer after layer (the oracle's own chain: layer l+1 takes the oracle's output of
    layer l, never the GPU's) over every step, with every layer's cache compared at the end."""
    cfg, B, L_max, L0, N, NL = SMALL_GQA, 3, 64, 10, 4, 3
    say("stack graph vs per-layer graphs vs oracle chain", NL, "layers")
    rng = np.random.default_rng(7)
    xs = I.round_bf16(rng.standard_normal((N, B, cfg.d)))
    params = [I.make_decoder_layer(cfg, B=B, S=1, seed=40 + l, random_norm_weights=True) for l in range(NL)]
    hist = [I.make_kv_history(B, L_max, cfg.Hkv, cfg.D, L0, seed=50 + l) for l in range(NL)]

    def build():
        lays = []
        for l in range(NL):
            kc, vc = hist[l]
            lays.append(DeviceLayer(cfg, params[l], B=B, S=1, L_max=L_max, kc=kc, vc=vc, seqlens=np.full(B, L0),
                                    advance=True, fold_norm=True))
        for l in range(1, NL):  # chain: layer l reads layer l-1's output
            lays[l].desc.x = lays[l - 1].y.data_ptr()
        return lays

    per, stack = build(), build()
    graphs = [lay.capture() for lay in per]
    sg = fsvd.fsvd_decoder_stack_capture([lay.desc for lay in stack])
    ys = []
    try:
        for t in range(N):
            xt = to_dev(xs[t]).reshape(B, 1, cfg.d)
            per[0].x.copy_(xt)
            stack[0].x.copy_(xt)
            for g in graphs:
                fsvd.fsvd_graph_replay(g)
            fsvd.fsvd_graph_replay(sg)
            torch.cuda.synchronize()
            assert np.array_equal(bits(per[-1].y), bits(stack[-1].y)), f"step {t}"
            ys.append(stack[-1].y_host()[:, 0])
        for a, b in zip(per, stack):
            assert np.array_equal(bits(a.k_cache), bits(b.k_cache))
            assert list(b.seqlens.cpu().numpy()) == [L0 + N] * B
    finally:
        for g in graphs:
            fsvd.fsvd_graph_destroy(g)
        fsvd.fsvd_graph_destroy(sg)
    # the oracle, layer after layer: N decode steps of layer l over the N outputs of layer l-1
    x_l = xs
    for l in range(NL):
        kc, vc = hist[l]
        x_l, kc_ref, vc_ref, sl = O.decoder_steps(x_l, params[l], cfg, kc, vc, np.full(B, L0))
        e_k = rel(from_dev(stack[l].k_cache)[:, L0:L0 + N], kc_ref[:, L0:L0 + N])
        e_v = rel(from_dev(stack[l].v_cache)[:, L0:L0 + N], vc_ref[:, L0:L0 + N])
        say(f"  layer {l}: appended K {e_k:.2e}  V {e_v:.2e}")
        assert e_k <= BF16_TOL and e_v <= BF16_TOL
        assert np.array_equal(bits(stack[l].k_cache)[:, :L0], bits(to_dev(kc))[:, :L0])
    e_y = rel(np.stack(ys), x_l)
    say(f"  last layer outputs over {N} steps {e_y:.2e}")
    assert e_y <= BF16_TOL
