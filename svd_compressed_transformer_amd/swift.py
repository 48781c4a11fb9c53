"""Swift-SVD factor production on the GPU ("Swift-SVD: Theoretical Optimality Meets Practical
Efficiency in Low-Rank LLM Compression", explainer, section 2A).

    Ut, Vt, lam = swift_compress(Wt, X_batches, k)

Activation-aware rank-k compression of a linear layer y = x . W in the page's order:

1. the output covariance C = sum_t Y_t^T Y_t, Y_t = X_t W, aggregated batch by batch on the
   matrix cores (``fsvd_swift_covariance``: fp32 accumulation, upper triangle);
2. one eigendecomposition of C, on the host (numpy, from the upper triangle), eigenvalues sorted
   descending and rounding negatives clamped to 0: the top-k eigenvectors V_k are the right
   singular vectors of Y = X W, and the eigenvalues its squared singular values;
3. the closed-form optimum W_k* = W V_k V_k^T as this library's factor pair (``fsvd_swift_factors``):
   Ut = (W V_k)^T [k, d_in] and Vt = V_k [d_out, k], bf16.

Wt = W^T [d_out, d_in] is the layer weight in linear-layer storage (bf16, on the device); each
batch X_t is a device tensor [T, d_in] bf16.  d_in, d_out, T and k must be multiples of 8.
"""
from __future__ import annotations

import numpy as np
import torch

from svd_compressed_transformer_amd import fsvd


def covariance(Wt, X_batches, stream=None):
    """C = sum_t (X_t W)^T (X_t W) as an fp32 device tensor [d_out, d_out]; only the upper
    triangle (in whole tiles) is defined."""
    d_out, d_in = Wt.shape
    C = torch.zeros((d_out, d_out), dtype=torch.float32, device=Wt.device)
    ws = None
    for X in X_batches:
        T = X.shape[0]
        need = fsvd.fsvd_swift_covariance_ws(T, d_in, d_out)
        if ws is None or ws.numel() < need:
            ws = fsvd.workspace(need, device=Wt.device)
        fsvd.fsvd_swift_covariance(X, T, d_in, X.stride(0), Wt, d_out, C, d_out, ws, ws.numel(), stream)
    return C


def top_eigvecs(C, k):
    """Eigen-decomposition of the symmetric C from its upper triangle: eigenvalues descending
    (negatives clamped to 0) and the top-k eigenvectors as columns [d_out, k] (float64, host)."""
    Ch = C.detach().to("cpu", torch.float64).numpy()
    lam, vecs = np.linalg.eigh(Ch, UPLO="U")
    order = np.argsort(lam)[::-1]
    return np.clip(lam[order], 0.0, None), vecs[:, order[:k]]


def factors(Wt, Vk, stream=None):
    """Ut = (W V_k)^T [k, d_in] and Vt = V_k [d_out, k] (bf16 device tensors) from V_k [d_out, k]."""
    d_out, d_in = Wt.shape
    k = Vk.shape[1]
    VkT = torch.from_numpy(np.ascontiguousarray(Vk.T)).to(device=Wt.device, dtype=torch.bfloat16)
    Ut = torch.empty((k, d_in), dtype=torch.bfloat16, device=Wt.device)
    Vt = torch.empty((d_out, k), dtype=torch.bfloat16, device=Wt.device)
    ws = fsvd.workspace(fsvd.fsvd_swift_factors_ws(d_in, d_out), device=Wt.device)
    fsvd.fsvd_swift_factors(Wt, d_out, d_in, VkT, k, Ut, Vt, ws, ws.numel(), stream)
    return Ut, Vt


def swift_compress(Wt, X_batches, k, stream=None):
    """Rank-k factor pair (Ut, Vt) of W minimising ||X W - X W_k||_F over the calibration
    batches, and the eigenvalues of C (descending)."""
    C = covariance(Wt, X_batches, stream)
    lam, Vk = top_eigvecs(C, k)
    Ut, Vt = factors(Wt, Vk, stream)
    return Ut, Vt, lam
