"""GPU parity of the Swift-SVD factor production ("Swift-SVD: Theoretical Optimality Meets
Practical Efficiency in Low-Rank LLM Compression", section 2A) against the oracle.

- the covariance accumulated over several calibration batches (upper triangle; tiles wholly
  below the diagonal are never written);
- the factor pair from given eigenvectors (Ut = (W V_k)^T, Vt = V_k bit for bit);
- the whole compression on inputs whose output spectrum has a clear gap after k, so the top-k
  subspace is well defined: the rank-k reconstruction W V_k V_k^T and the reconstruction error
  against the oracle's optimum;
- the covariance at the Llama-7B projection width (4096 x 4096).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import fsvd_oracle as O  # noqa: E402
from svd_compressed_transformer_amd import fsvd, inputs as I, swift  # noqa: E402
from svd_compressed_transformer_amd.device import from_dev, to_dev  # noqa: E402

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2


def rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))


def say(*a):
    print(*a, flush=True)


def upper_tiles_mask(n, tile):
    """Entries the symmetric accumulation writes: every tile that reaches the diagonal or above."""
    r = np.arange(n)[:, None] // tile
    c = np.arange(n)[None, :] // tile
    return r <= c


@pytest.mark.parametrize("T,d_in,d_out,nb", [(296, 200, 136, 2), (64, 64, 512, 3)])
def test_covariance_accumulates(T, d_in, d_out, nb):
    say("swift covariance", T, d_in, d_out, nb)
    rng = np.random.default_rng(1)
    W = I.round_bf16(rng.standard_normal((d_in, d_out)) / np.sqrt(d_in))
    Xs = [I.round_bf16(rng.standard_normal((T, d_in))) for _ in range(nb)]
    Wt = to_dev(np.ascontiguousarray(W.T))
    C = swift.covariance(Wt, [to_dev(X) for X in Xs])
    torch.cuda.synchronize()
    Cg = from_dev(C)
    ref = O.swift_svd(Xs, W, 8)["C"]
    tile = 256 if ((d_out + 255) // 256) ** 2 >= 1024 else 128
    m = upper_tiles_mask(d_out, tile)
    up = np.triu(np.ones((d_out, d_out), dtype=bool))
    err = rel(Cg[up], ref[up])
    say(f"  upper triangle err {err:.2e}")
    assert err <= BF16_TOL
    assert np.all(Cg[~m] == 0.0), "tiles below the diagonal were written"


def test_factors_from_eigenvectors():
    d_in, d_out, k = 200, 136, 24
    say("swift factors", d_in, d_out, k)
    rng = np.random.default_rng(2)
    W = I.round_bf16(rng.standard_normal((d_in, d_out)) / np.sqrt(d_in))
    Q, _ = np.linalg.qr(rng.standard_normal((d_out, k)))
    Vk = I.round_bf16(Q)
    Ut, Vt = swift.factors(to_dev(np.ascontiguousarray(W.T)), Vk)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(Vt), Vk), "Vt must be V_k bit for bit"
    err = rel(from_dev(Ut), (W @ Vk).T)
    say(f"  Ut err {err:.2e}")
    assert err <= BF16_TOL


def test_swift_compress_end_to_end():
    d_in, d_out, T, nb, k = 256, 192, 512, 3, 32
    say("swift compress", d_in, d_out, T, nb, k)
    rng = np.random.default_rng(3)
    # calibration inputs concentrated on a k-dimensional subspace (plus small noise), so the
    # output spectrum has a clear gap after k
    basis, _ = np.linalg.qr(rng.standard_normal((d_in, d_in)))
    scale = np.where(np.arange(d_in) < k, 1.0, 0.01)
    Xs = [I.round_bf16((rng.standard_normal((T, d_in)) * scale) @ basis.T) for _ in range(nb)]
    W = I.round_bf16(rng.standard_normal((d_in, d_out)) / np.sqrt(d_in))
    Ut, Vt, lam = swift.swift_compress(to_dev(np.ascontiguousarray(W.T)), [to_dev(X) for X in Xs], k)
    torch.cuda.synchronize()
    ref = O.swift_svd(Xs, W, k)
    assert lam[k - 1] > 50 * lam[k], "the test spectrum needs a gap after k"
    Wk = from_dev(Ut).T @ from_dev(Vt).T                      # U . V = (W V_k) V_k^T
    err = rel(Wk, ref["Wk"])
    say(f"  W_k err {err:.2e}, eigenvalue err {rel(lam[:k], ref['lam'][:k]):.2e}")
    assert err <= BF16_TOL
    assert rel(lam[:k], ref["lam"][:k]) <= BF16_TOL
    # the reconstruction error ||X W - X W_k|| is the oracle's optimum up to the bf16 rounding of
    # the factors (a few 1e-3 of ||X W||)
    X = np.concatenate(Xs)
    e_gpu = np.linalg.norm(X @ W - X @ Wk)
    e_opt = np.linalg.norm(X @ W - X @ ref["Wk"])
    say(f"  ||XW - XW_k||: gpu {e_gpu:.4e}, optimum {e_opt:.4e}, ||XW|| {np.linalg.norm(X @ W):.4e}")
    assert e_gpu <= e_opt + 1e-2 * np.linalg.norm(X @ W)


@pytest.mark.slow
def test_covariance_llama7b_width():
    d, T = 4096, 512
    say("swift covariance at width", d, "T", T)
    rng = np.random.default_rng(4)
    W = I.round_bf16(rng.standard_normal((d, d)) / np.sqrt(d))
    X = I.round_bf16(rng.standard_normal((T, d)))
    C = swift.covariance(to_dev(np.ascontiguousarray(W.T)), [to_dev(X)])
    torch.cuda.synchronize()
    Cg = from_dev(C)
    ref = O.swift_svd([X], W, 1)["C"]     # the oracle's aggregated covariance
    up = np.triu(np.ones((d, d), dtype=bool))
    err = rel(Cg[up], ref[up])
    say(f"  upper triangle err {err:.2e}")
    assert err <= BF16_TOL
