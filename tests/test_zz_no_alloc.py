"""The allocation-free linear (static per-GPU scratch) against the workspace entry point.

Same kernels, same launch configuration: the outputs must be identical bit for bit.  Two calls
in a row on one stream, the second with a smaller input, so the second finds the scratch as the
first left it; both the decode-sized (row-dot / skinny matrix-core) path and the prefill-sized
(MFMA GEMM) path, bf16 and fp32.
"""
import numpy as np
import pytest

from svd_compressed_transformer_amd import fsvd, inputs as I


def _status(f):
    try:
        f()
    except fsvd.FsvdError as e:
        return e.status, str(e)
    return 0, ""


def test_noalloc_rejects_oversize_before_launch(monkeypatch):
    """Scratch beyond the static array is refused on the host (fake pointers, never touched)."""
    if not fsvd.os.path.exists(fsvd.LIB_PATH):
        pytest.fail("libfsvd.so is not built")
    monkeypatch.setattr(fsvd, "_s", lambda stream: 0)
    P = 0x1000
    M, K, r, N = 8192, 4096, 4096, 4096          # z alone is 64 MiB
    assert fsvd.fsvd_lowrank_linear_ws(M, K, r, N, fsvd.FSVD_BF16) > fsvd.FSVD_NOALLOC_SCRATCH_BYTES
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear_noalloc(P, M, K, K, P, r, K, P, N, r, None, None, N, P, N,
                                                              fsvd.FSVD_BF16))
    assert s == fsvd.FSVD_ERR_WORKSPACE and "static scratch" in msg
    # argument checks come first, as in the workspace entry point
    s, msg = _status(lambda: fsvd.fsvd_lowrank_linear_noalloc(None, 4, 64, 64, P, 8, 64, P, 64, 8, None, None, 64, P,
                                                              64, fsvd.FSVD_BF16))
    assert s == fsvd.FSVD_ERR_INVALID_ARG and "NULL" in msg


@pytest.mark.gpu
@pytest.mark.parametrize("dtype,first,second", [
    ("bf16", (24, 4096, 1640, 4096), (3, 4096, 1024, 1032)),     # matrix-core split reduction, then row-dot
    ("bf16", (4096, 1024, 520, 2048), (300, 768, 392, 768)),     # MFMA GEMM path, twice
    ("f32", (16, 256, 64, 256), (5, 200, 40, 96)),                # fp32 row-dot
])
def test_noalloc_equals_workspace_entry(dtype, first, second):
    import torch
    from svd_compressed_transformer_amd.device import to_dev
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    fdt = fsvd.FSVD_BF16 if dtype == "bf16" else fsvd.FSVD_F32
    rng = np.random.default_rng(5)
    for i, (M, K, r, N) in enumerate((first, second)):
        print("noalloc linear", dtype, "call", i, (M, K, r, N), flush=True)
        x = to_dev(I.round_to(rng.standard_normal((M, K)), dtype), tdt)
        Ut = to_dev(I.round_to(rng.standard_normal((r, K)) / np.sqrt(K), dtype), tdt)
        Vt = to_dev(I.round_to(rng.standard_normal((N, r)) / np.sqrt(r), dtype), tdt)
        bias = to_dev(I.round_to(rng.standard_normal(N), dtype), tdt)
        res = to_dev(I.round_to(rng.standard_normal((M, N)), dtype), tdt)
        y_ws = torch.empty((M, N), dtype=tdt, device="cuda")
        y_na = torch.full((M, N), float("nan"), dtype=tdt, device="cuda")
        nb = fsvd.fsvd_lowrank_linear_ws(M, K, r, N, fdt)
        assert nb <= fsvd.FSVD_NOALLOC_SCRATCH_BYTES
        ws = fsvd.workspace(nb)
        fsvd.fsvd_lowrank_linear(x, M, K, K, Ut, r, K, Vt, N, r, bias, res, N, y_ws, N, fdt, ws, nb)
        fsvd.fsvd_lowrank_linear_noalloc(x, M, K, K, Ut, r, K, Vt, N, r, bias, res, N, y_na, N, fdt)
        torch.cuda.synchronize()
        a = y_ws.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
        b = y_na.view(torch.int16 if dtype == "bf16" else torch.int32).cpu().numpy()
        assert np.array_equal(a, b), f"call {i}: allocation-free output differs from the workspace entry point"
