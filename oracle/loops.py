"""Pure-Python brute force for tiny shapes (no numpy arithmetic): an independent second
computation of the oracle's definitions, used only to pin ``fsvd_oracle`` in the CPU tests.

TEST INFRASTRUCTURE (same import rule as ``fsvd_oracle``).  Inputs are nested lists or
numpy arrays; everything is converted to Python floats and looped over explicitly.
"""
from __future__ import annotations

import math


def _l(a):
    return a.tolist() if hasattr(a, "tolist") else a


def matmul(A, B):
    """C[i][j] = sum_k A[i][k] * B[k][j]."""
    A, B = _l(A), _l(B)
    n, m, p = len(A), len(B), len(B[0])
    return [[sum(float(A[i][k]) * float(B[k][j]) for k in range(m)) for j in range(p)] for i in range(n)]


def transpose(A):
    A = _l(A)
    return [list(r) for r in zip(*A)]


def lowrank_linear(x, Ut, Vt, bias=None, residual=None):
    """y[m][n] = residual[m][n] + bias[n] + sum_j (sum_k x[m][k] Ut[j][k]) Vt[n][j]."""
    x, Ut, Vt = _l(x), _l(Ut), _l(Vt)
    M, r, N = len(x), len(Ut), len(Vt)
    y = []
    for m in range(M):
        z = [sum(float(x[m][k]) * float(Ut[j][k]) for k in range(len(x[m]))) for j in range(r)]
        row = []
        for n in range(N):
            v = sum(z[j] * float(Vt[n][j]) for j in range(r))
            if bias is not None:
                v += float(_l(bias)[n])
            if residual is not None:
                v += float(_l(residual)[m][n])
            row.append(v)
        y.append(row)
    return y


def softmax_attention_one(qv, K, V, scale):
    """One query vector over key/value lists: sum_j softmax_j(scale q.k_j) v_j."""
    qv, K, V = _l(qv), _l(K), _l(V)
    s = [scale * sum(float(a) * float(b) for a, b in zip(qv, kj)) for kj in K]
    mx = max(s)
    e = [math.exp(t - mx) for t in s]
    tot = sum(e)
    D = len(V[0])
    return [sum(e[j] * float(V[j][i]) for j in range(len(V))) / tot for i in range(D)]


def rmsnorm_row(x, w, eps):
    x, w = _l(x), _l(w)
    ms = sum(float(t) * float(t) for t in x) / len(x)
    r = 1.0 / math.sqrt(ms + eps)
    return [float(t) * r * float(wi) for t, wi in zip(x, w)]


def rope_vec(x, pos, theta):
    x = _l(x)
    D = len(x)
    h = D // 2
    out = [0.0] * D
    for i in range(h):
        a = pos * theta ** (-2.0 * i / D)
        c, s = math.cos(a), math.sin(a)
        out[i] = float(x[i]) * c - float(x[i + h]) * s
        out[i + h] = float(x[i + h]) * c + float(x[i]) * s
    return out
