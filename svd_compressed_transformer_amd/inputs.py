"""Seeded synthetic inputs for the fused low-rank layer, shared by the GPU path's tests and the oracle.

This module draws numbers and rounds them to the storage dtype; it holds none of the
method's arithmetic (no projection, norm, activation or attention).  Everything is numpy.

Recipe (one generator per case, ``numpy.random.default_rng(seed)``, seed 0 unless a test
says otherwise), in this draw order: the layer input x, then one factor pair per projection
in the order q, k, v, o, gate, up, down, then the dense KV history.

* x ~ N(0, 1).
* A projection W (d_in x d_out, row-vector convention y = x W) is replaced by a factor pair
  U (d_in x r) ~ N(0, 1/d_in) and V (r x d_out) ~ N(0, 1/r) with rank row i (1-based)
  scaled by sigma_i = i^-0.5, i.e. the singular-value profile is folded into V.  This is
  the FlashSVD pages' "truncated factors" representation (FlashSVD v1 abstract; FlashSVD
  v1.5 Methodology 1, "common native factorized representation").
* Factors are stored K-contiguous like two linear-layer weights: Ut = U^T (r x d_in) and
  Vt = V^T (d_out x r).
* KV history ~ N(0, 1), drawn in float32 (to bound host memory at long contexts).
* Values are drawn in float64 and rounded once to the storage dtype: float32 by a cast,
  bfloat16 by round-to-nearest-even on the float32 bit pattern.
"""
from __future__ import annotations

from dataclasses import dataclass, field
import numpy as np

# ----------------------------------------------------------------------------- dtype helpers


def bf16_bits(a) -> np.ndarray:
    """Round to bfloat16 (round-to-nearest-even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 values."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_bf16(a) -> np.ndarray:
    """float32 array holding the bfloat16-rounded values of ``a``."""
    return bf16_to_f32(bf16_bits(a))


def round_to(a, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def rank_of(ratio: float, d_in: int, d_out: int) -> int:
    """Retained rank = floor(ratio * min(d_in, d_out))."""
    return int(np.floor(ratio * min(d_in, d_out) + 1e-9))


# ----------------------------------------------------------------------------- factor draws


def factor_pair(rng: np.random.Generator, d_in: int, d_out: int, r: int):
    """Draw (Ut [r, d_in], Vt [d_out, r]) in float64 following the module recipe."""
    U = rng.standard_normal((d_in, r)) / np.sqrt(d_in)
    sigma = np.arange(1, r + 1, dtype=np.float64) ** -0.5
    V = rng.standard_normal((r, d_out)) / np.sqrt(r) * sigma[:, None]
    return np.ascontiguousarray(U.T), np.ascontiguousarray(V.T)


# ----------------------------------------------------------------------------- configurations


@dataclass(frozen=True)
class LinearCase:
    M: int = 16
    K: int = 256
    r: int = 64
    N: int = 256
    dtype: str = "f32"


@dataclass(frozen=True)
class DecoderLayerConfig:
    """Llama-style pre-norm decoder layer with per-projection ranks."""
    name: str
    d: int
    Hq: int
    Hkv: int
    D: int
    d_ff: int
    ranks: dict = field(hash=False, compare=False, default_factory=dict)
    norm_eps: float = 1e-6
    rope_theta: float = 1e4

    def rank(self, proj: str) -> int:
        return self.ranks[proj]


@dataclass(frozen=True)
class EncoderLayerConfig:
    """BERT-style post-norm encoder layer (GELU FFN)."""
    name: str
    d: int
    H: int
    D: int
    d_ff: int
    ranks: dict = field(hash=False, compare=False, default_factory=dict)
    ln_eps: float = 1e-12


def _uniform_ranks(ratio, d, qkv_out, o_in, d_ff):
    return {
        "q": rank_of(ratio, d, qkv_out[0]),
        "k": rank_of(ratio, d, qkv_out[1]),
        "v": rank_of(ratio, d, qkv_out[2]),
        "o": rank_of(ratio, o_in, d),
        "gate": rank_of(ratio, d, d_ff),
        "up": rank_of(ratio, d, d_ff),
        "down": rank_of(ratio, d_ff, d),
    }


# single fused low-rank linear, float32: 16x256 . (256x64) . (64x256)
CFG0 = LinearCase()

# BERT-Base-shaped encoder layer, rank 50% of min(dims), batch 8 x seq 512
CFG1 = EncoderLayerConfig(
    name="bert-base", d=768, H=12, D=64, d_ff=3072,
    ranks={"q": 384, "k": 384, "v": 384, "o": 384, "up": 384, "down": 384}, ln_eps=1e-12)
CFG1_BATCH, CFG1_SEQ = 8, 512

# Llama-7B-shaped decoder layer, rank 40% of min(dims) = 1638 on every projection
CFG2 = DecoderLayerConfig(
    name="llama-7b", d=4096, Hq=32, Hkv=32, D=128, d_ff=11008,
    ranks=_uniform_ranks(0.4, 4096, (4096, 4096, 4096), 4096, 11008), norm_eps=1e-6, rope_theta=1e4)
CFG2_BATCHES, CFG2_KV_LEN = (1, 8, 16), 2048

# same layer: prefill 4 x 2048 then 128 graph-replayed decode steps
CFG3 = CFG2
CFG3_BATCH, CFG3_PREFILL, CFG3_DECODE_STEPS = 4, 2048, 128

# Llama-3-8B-shaped GQA layer with non-uniform ranks (fixed table)
CFG4 = DecoderLayerConfig(
    name="llama3-8b-gqa", d=4096, Hq=32, Hkv=8, D=128, d_ff=14336,
    ranks={"q": 1536, "k": 512, "v": 256, "o": 1024, "gate": 1024, "up": 1536, "down": 512},
    norm_eps=1e-5, rope_theta=5e5)
CFG4_BATCH, CFG4_KV_LEN = 32, 8192

# allowed rank values per projection of the GQA layer (each <= min(d_in, d_out))
CFG4_RANK_CHOICES = (256, 512, 1024, 1536)


def scaled_decoder(cfg: DecoderLayerConfig, d: int, Hq: int, Hkv: int, D: int, d_ff: int,
                   ranks: dict, name: str = "small") -> DecoderLayerConfig:
    """A smaller decoder layer with the same conventions (for oracle-speed parity tests)."""
    return DecoderLayerConfig(name=name, d=d, Hq=Hq, Hkv=Hkv, D=D, d_ff=d_ff, ranks=dict(ranks),
                              norm_eps=cfg.norm_eps, rope_theta=cfg.rope_theta)


# ----------------------------------------------------------------------------- whole-case draws


def make_linear_case(case: LinearCase = CFG0, seed: int = 0):
    """x [M, K], Ut [r, K], Vt [N, r] rounded to the case dtype (float32 arrays)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((case.M, case.K))
    Ut, Vt = factor_pair(rng, case.K, case.N, case.r)
    return {k: round_to(v, case.dtype) for k, v in (("x", x), ("Ut", Ut), ("Vt", Vt))}


def make_decoder_layer(cfg: DecoderLayerConfig, B: int, S: int, seed: int = 0, dtype: str = "bf16",
                       random_norm_weights: bool = False):
    """Input x [B, S, d] plus every factor of one decoder layer, rounded to ``dtype``.

    Returns a dict of float32 arrays holding exactly representable ``dtype`` values:
    x, Ut_q/Vt_q, Ut_k/Vt_k, Ut_v/Vt_v, Ut_o/Vt_o, Ut_gate/Vt_gate, Ut_up/Vt_up,
    Ut_down/Vt_down, attn_norm_w, mlp_norm_w.  Norm weights are ones unless
    ``random_norm_weights`` (then drawn after the factors, 1 + 0.1 N(0,1)).
    """
    rng = np.random.default_rng(seed)
    out = {"x": rng.standard_normal((B, S, cfg.d))}
    qd, kd = cfg.Hq * cfg.D, cfg.Hkv * cfg.D
    dims = {"q": (cfg.d, qd), "k": (cfg.d, kd), "v": (cfg.d, kd), "o": (qd, cfg.d),
            "gate": (cfg.d, cfg.d_ff), "up": (cfg.d, cfg.d_ff), "down": (cfg.d_ff, cfg.d)}
    for p in ("q", "k", "v", "o", "gate", "up", "down"):
        d_in, d_out = dims[p]
        out["Ut_" + p], out["Vt_" + p] = factor_pair(rng, d_in, d_out, cfg.rank(p))
    if random_norm_weights:
        out["attn_norm_w"] = 1.0 + 0.1 * rng.standard_normal(cfg.d)
        out["mlp_norm_w"] = 1.0 + 0.1 * rng.standard_normal(cfg.d)
    else:
        out["attn_norm_w"] = np.ones(cfg.d)
        out["mlp_norm_w"] = np.ones(cfg.d)
    return {k: round_to(v, dtype) for k, v in out.items()}


def make_encoder_layer(cfg: EncoderLayerConfig, B: int, S: int, seed: int = 0, dtype: str = "bf16"):
    """Input x [B, S, d] plus factors q, k, v, o, up, down and LayerNorm gamma/beta."""
    rng = np.random.default_rng(seed)
    out = {"x": rng.standard_normal((B, S, cfg.d))}
    hd = cfg.H * cfg.D
    dims = {"q": (cfg.d, hd), "k": (cfg.d, hd), "v": (cfg.d, hd), "o": (hd, cfg.d),
            "up": (cfg.d, cfg.d_ff), "down": (cfg.d_ff, cfg.d)}
    for p in ("q", "k", "v", "o", "up", "down"):
        d_in, d_out = dims[p]
        out["Ut_" + p], out["Vt_" + p] = factor_pair(rng, d_in, d_out, cfg.ranks[p])
    out["ln1_g"], out["ln1_b"] = np.ones(cfg.d), np.zeros(cfg.d)
    out["ln2_g"], out["ln2_b"] = np.ones(cfg.d), np.zeros(cfg.d)
    return {k: round_to(v, dtype) for k, v in out.items()}


def make_kv_history(B: int, L_max: int, Hkv: int, D: int, n_hist, seed: int = 1, dtype: str = "bf16"):
    """Dense KV caches [B, L_max, Hkv, D]; positions < n_hist[b] hold N(0,1) history,
    the rest hold zeros.  Returns (k_cache, v_cache) as float32 arrays of ``dtype`` values."""
    rng = np.random.default_rng(seed)
    n_hist = np.broadcast_to(np.asarray(n_hist, dtype=np.int64), (B,))
    kc = np.zeros((B, L_max, Hkv, D), dtype=np.float32)
    vc = np.zeros((B, L_max, Hkv, D), dtype=np.float32)
    for b in range(B):
        n = int(n_hist[b])
        kc[b, :n] = rng.standard_normal((n, Hkv, D), dtype=np.float32)
        vc[b, :n] = rng.standard_normal((n, Hkv, D), dtype=np.float32)
    return round_to(kc, dtype), round_to(vc, dtype)


def make_attention_case(B: int, Sq: int, Hq: int, Hkv: int, D: int, L_max: int, seqlens,
                        seed: int = 2, q_scale: float = 1.0, dtype: str = "bf16"):
    """q [B, Sq, Hq, D] ~ q_scale * N(0,1) and dense caches whose first seqlens[b] + Sq
    positions are filled (history plus the Sq new tokens)."""
    rng = np.random.default_rng(seed)
    seqlens = np.broadcast_to(np.asarray(seqlens, dtype=np.int64), (B,)).copy()
    q = q_scale * rng.standard_normal((B, Sq, Hq, D))
    kc, vc = make_kv_history(B, L_max, Hkv, D, np.minimum(seqlens + Sq, L_max), seed=seed + 1000, dtype=dtype)
    return round_to(q, dtype), kc, vc, seqlens.astype(np.int32)
