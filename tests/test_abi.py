"""CPU checks of the C-ABI library: it loads, exports every function include/fsvd.h declares,
answers host-only queries, and rejects bad arguments before launching anything (no GPU needed:
every call below fails validation on the host)."""
import ctypes as C
import os
import re

import pytest

from svd_compressed_transformer_amd import fsvd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = 4096  # workspace header: the device error word, then the decode attention's partition counters


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fsvd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(fsvd_\w+)\s*\(", src, flags=re.M))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fsvd.LIB_PATH):
        pytest.fail("libfsvd.so is not built (run __graft_entry__.build())")
    return fsvd.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 20, names
    raw = C.CDLL(fsvd.LIB_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing
    # the binding mirrors the same names
    assert all(hasattr(fsvd, n) for n in names), [n for n in names if not hasattr(fsvd, n)]


def test_version_and_status_strings(L):
    import re
    hdr = open(os.path.join(ROOT, "include", "fsvd.h")).read()
    assert fsvd.fsvd_abi_version() == int(re.search(r"#define FSVD_ABI_VERSION (\d+)", hdr).group(1))
    assert fsvd.fsvd_status_str(0) == "ok"
    assert "workspace" in fsvd.fsvd_status_str(fsvd.FSVD_ERR_WORKSPACE)


def test_workspace_queries(L):
    # header + 256-aligned z: M * r * 2 bytes
    assert fsvd.fsvd_lowrank_linear_ws(4, 4096, 1640, 4096, fsvd.FSVD_BF16) == HDR + ((4 * 1640 * 2 + 255) // 256) * 256
    assert fsvd.fsvd_lowrank_linear_ws(16, 256, 64, 256, fsvd.FSVD_F32) == HDR + 16 * 64 * 4
    assert fsvd.fsvd_decode_attn_dense_kv_ws(4, 1, 32, 32, 128, 2176) > HDR
    assert fsvd.fsvd_lowrank_qkv_ws(1, 1, 4096, 1640, 1640, 1640, 32, 32, 128) >= HDR + 4920 * 2
    d = fsvd.decoder_layer_desc(B=4, S=1, d=4096, Hq=32, Hkv=32, D=128, d_ff=11008, L_max=2176, r_q=1640, r_k=1640,
                                r_v=1640, r_o=1640, r_g=1640, r_u=1640, r_d=1640)
    assert fsvd.fsvd_decoder_layer_ws(d) > HDR


def test_mlp_workspace_keeps_t_on_chip(L):
    """At prefill sizes the packed MLP keeps t [M, d_ff] on chip when a fused kernel covers its
    ranks (equal up and down ranks of 128, 256 or 384): the workspace holds z, the per-slice
    partial z_d (BERT-Base, 4096 rows: 32 blocks of 128 rows x 8 slices of d_ff) and z_d; with
    ranks no fused kernel covers it holds t instead, and so does every decode-size call."""
    al = lambda n: (n + 255) // 256 * 256
    M, d, dff = 4096, 768, 3072
    common = al(M * d * 2) + al(M * 4)  # normalised input and its per-row rstd (MFMA path)
    r = 384
    assert fsvd.fsvd_lowrank_mlp_packed_ws(M, d, 0, r, dff, r) == HDR + al(M * r * 2) + al(8 * M * r * 2) + al(M * r * 2) + common
    r = 392
    assert fsvd.fsvd_lowrank_mlp_packed_ws(M, d, 0, r, dff, r) == HDR + al(M * r * 2) + al(M * dff * 2) + al(M * r * 2) + common
    # one slice when the row blocks alone fill the chip: z_d written directly, no partials
    M = 16600
    common = al(M * 256 * 2) + al(M * 4)
    assert fsvd.fsvd_lowrank_mlp_packed_ws(M, 256, 0, 128, 264, 128) == HDR + 2 * al(M * 128 * 2) + common
    # decode sizes keep the two-kernel path (t of a few rows stays in L2)
    assert fsvd.fsvd_lowrank_mlp_packed_ws(16, d, 0, 384, dff, 384) >= HDR + al(16 * dff * 2)


def _status(f):
    try:
        f()
    except fsvd.FsvdError as e:
        return e.status, str(e)
    return 0, ""


def test_validation_errors_return_before_launch(L, monkeypatch):
    monkeypatch.setattr(fsvd, "_s", lambda stream: 0)   # default stream; nothing reaches the GPU
    bf = fsvd.FSVD_BF16
    # null pointers
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear(None, 1, 8, 8, None, 8, 8, None, 8, 8, None, None, 8, None, 8,
                                                      bf, None, 0))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "NULL" in msg
    # non-positive size (checked before pointers)
    s, _ = _status(lambda: fsvd.fsvd_lowrank_linear(None, 0, 8, 8, None, 8, 8, None, 8, 8, None, None, 8, None, 8,
                                                    bf, None, 0))
    assert s == fsvd.FSVD_ERR_INVALID_ARG
    # rank not a multiple of 8 for bf16 rows
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear(None, 1, 8, 8, None, 12, 8, None, 8, 12, None, None, 8, None, 8,
                                                      bf, None, 0))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "multiple" in msg
    # misaligned pointer (never dereferenced: validation stops first)
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear(0x1002, 1, 8, 8, 0x2000, 8, 8, 0x3000, 8, 8, None, None, 8,
                                                      0x4000, 8, bf, 0x5000, 4096))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "aligned" in msg
    # workspace too small
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear(0x1000, 1, 8, 8, 0x2000, 8, 8, 0x3000, 8, 8, None, None, 8,
                                                      0x4000, 8, bf, 0x5000, 16))
    assert s == fsvd.FSVD_ERR_WORKSPACE
    # fp32 where only bf16 is supported
    s, _ = _status(lambda: fsvd.fsvd_lowrank_mlp_packed(0x1000, 1, 8, None, 0.0, 0, 0x1000, 8, 8, 0x1000, 0x1000, 8,
                                                        0x1000, 0x1000, 8, None, 0x1000, fsvd.FSVD_F32, 0x1000, 1 << 20))
    assert s == fsvd.FSVD_ERR_UNSUPPORTED
    # GELU with a gate rank
    s, msg = _status(lambda: fsvd.fsvd_lowrank_mlp_packed(0x1000, 1, 8, None, 0.0, fsvd.FSVD_ACT_GELU, 0x1000, 8, 8,
                                                          None, 0x1000, 8, 0x1000, 0x1000, 8, None, 0x1000, bf, 0x1000,
                                                          1 << 20))
    assert s == fsvd.FSVD_ERR_INVALID_ARG
    # attention: unsupported head dim and GQA ratio
    s, _ = _status(lambda: fsvd.fsvd_decode_attn_dense_kv(0x1000, 0x1000, 0x1000, 8, 0x1000, 1, 1, 4, 4, 96, 0.0, 1,
                                                          0x1000, bf, 0x1000, 1 << 20))
    assert s == fsvd.FSVD_ERR_UNSUPPORTED
    s, _ = _status(lambda: fsvd.fsvd_decode_attn_dense_kv(0x1000, 0x1000, 0x1000, 8, 0x1000, 1, 1, 6, 4, 64, 0.0, 1,
                                                          0x1000, bf, 0x1000, 1 << 20))
    assert s == fsvd.FSVD_ERR_INVALID_ARG
    # layer: y aliasing x, and a graph capture of a multi-token layer
    d = fsvd.decoder_layer_desc(B=1, S=1, d=64, Hq=1, Hkv=1, D=64, d_ff=64, L_max=8, r_q=8, r_k=8, r_v=8, r_o=8,
                                r_g=8, r_u=8, r_d=8, **{k: 0x1000 for k in (
                                    "x", "y", "A_qkv", "Vt_q", "Vt_k", "Vt_v", "Ut_o", "Vt_o", "A_gu", "Vt_g",
                                    "Vt_u", "Ut_d", "Vt_d", "k_cache", "v_cache", "cache_seqlens", "ws")})
    d.ws_bytes = 1 << 30
    s, msg = _status(lambda: fsvd.fsvd_decoder_layer_run(d))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "alias" in msg
    # destroyed / bogus graph handles
    s, _ = _status(lambda: fsvd.fsvd_graph_replay(0x1234))
    assert s == fsvd.FSVD_ERR_CAPTURE
    s, _ = _status(lambda: fsvd.fsvd_graph_destroy(0x1234))
    assert s == fsvd.FSVD_ERR_CAPTURE
    # dense-weight comparator: NULL weight, short leading dimension, fp32 beyond the row-dot sizes
    s, msg = _status(lambda: fsvd.fsvd_dense_linear(0x1000, 1, 8, 8, None, 8, 8, None, None, 8, 0x2000, 8, bf))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "NULL" in msg
    s, msg = _status(lambda: fsvd.fsvd_dense_linear(0x1000, 1, 16, 16, 0x2000, 8, 8, None, None, 8, 0x3000, 8, bf))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "ldw" in msg
    s, _ = _status(lambda: fsvd.fsvd_dense_linear(0x1000, 64, 8, 8, 0x2000, 8, 8, None, None, 8, 0x3000, 8,
                                                  fsvd.FSVD_F32))
    assert s == fsvd.FSVD_ERR_UNSUPPORTED
    # prepack with inconsistent extents
    s, _ = _status(lambda: fsvd.fsvd_prepack(0x1000, 8, 8, [(0x1000, 4, 16, 16, 4)], bf))
    assert s == fsvd.FSVD_ERR_INVALID_ARG


def test_rank_and_head_dim_bounds(L, monkeypatch):
    """A rank above min(K, N) and a Q/K/V head dim outside {64, 128} are refused on the host,
    before anything is enqueued (every pointer below is a fake, never dereferenced)."""
    monkeypatch.setattr(fsvd, "_s", lambda stream: 0)
    bf = fsvd.FSVD_BF16
    P = 0x1000
    # linear: r = 24 > N = 16, and r = 24 > K = 16
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear(P, 1, 64, 64, P, 24, 64, P, 16, 24, None, None, 16, P, 16,
                                                      bf, P, 1 << 20))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "min(K, N)" in msg
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear(P, 1, 16, 16, P, 24, 16, P, 64, 24, None, None, 64, P, 64,
                                                      bf, P, 1 << 20))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "min(K, N)" in msg
    # r == min(K, N) is allowed: fails later only on the workspace size
    s, _ = _status(lambda: fsvd.fsvd_lowrank_linear(P, 1, 16, 16, P, 16, 16, P, 64, 16, None, None, 64, P, 64,
                                                    bf, P, 16))
    assert s == fsvd.FSVD_ERR_WORKSPACE
    # qkv: head dim 256 (RoPE pairs are handled for D in {64, 128} only), and r_k > Hkv * D
    s, msg = _status(lambda: fsvd.fsvd_lowrank_qkv(P, 1, 1, 512, None, 0.0, P, 8, 8, 8, P, P, P, 2, 2, 256, 1e4,
                                                   P, P, P, 8, P, None, None, bf, P, 1 << 20))
    assert s == fsvd.FSVD_ERR_UNSUPPORTED and "head dim" in msg
    s, msg = _status(lambda: fsvd.fsvd_lowrank_qkv(P, 1, 1, 512, None, 0.0, P, 64, 136, 8, P, P, P, 2, 2, 64, 1e4,
                                                   P, P, P, 8, P, None, None, bf, P, 1 << 20))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "r_k" in msg
    # mlp: r_d > min(d_ff, d)
    s, msg = _status(lambda: fsvd.fsvd_lowrank_mlp_packed(P, 1, 64, None, 0.0, fsvd.FSVD_ACT_SWIGLU, P, 8, 8, P, P,
                                                          128, P, P, 72, None, P, bf, P, 1 << 20))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "r_d" in msg
    # decoder layer: r_o > d
    d = fsvd.decoder_layer_desc(B=1, S=1, d=64, Hq=2, Hkv=2, D=64, d_ff=64, L_max=8, r_q=8, r_k=8, r_v=8, r_o=72,
                                r_g=8, r_u=8, r_d=8, **{k: P * (i + 1) for i, k in enumerate((
                                    "x", "y", "A_qkv", "Vt_q", "Vt_k", "Vt_v", "Ut_o", "Vt_o", "A_gu", "Vt_g",
                                    "Vt_u", "Ut_d", "Vt_d", "k_cache", "v_cache", "cache_seqlens", "ws"))})
    d.ws_bytes = 1 << 30
    s, msg = _status(lambda: fsvd.fsvd_decoder_layer_run(d))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "r_o" in msg


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    monkeypatch.setattr(fsvd, "_lib", None)
    monkeypatch.setattr(fsvd, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(RuntimeError, match="not built"):
        fsvd.lib()
