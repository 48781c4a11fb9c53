"""Thin Python binding of the fsvd C ABI (``include/fsvd.h``): the same function names and
argument order, marshalling only.  Tensor arguments are device tensors (their data pointers are
passed); ``stream=None`` means torch's current stream.  Every computation happens in the HIP
library; if ``libfsvd.so`` is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libfsvd.so")

FSVD_OK, FSVD_ERR_INVALID_ARG, FSVD_ERR_UNSUPPORTED, FSVD_ERR_WORKSPACE = 0, 1, 2, 3
FSVD_ERR_HIP, FSVD_ERR_CAPTURE, FSVD_ERR_DEVICE = 4, 5, 6
FSVD_F32, FSVD_BF16 = 0, 1
FSVD_ACT_SWIGLU, FSVD_ACT_GELU = 0, 1
FSVD_DEVERR_KV_OVERFLOW, FSVD_DEVERR_SEQ_OVERFLOW = 0x1, 0x2
FSVD_LAYER_NORM_FOLDED = 0x1

_i64, _sz, _vp, _f32, _i32 = C.c_int64, C.c_size_t, C.c_void_p, C.c_float, C.c_int32


class FsvdError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str):
        super().__init__(f"fsvd status {status} ({what}): {detail}")
        self.status = status


class PackItem(C.Structure):
    _fields_ = [("src", _vp), ("rows", _i64), ("cols", _i64), ("ld_src", _i64), ("rows_pad", _i64)]


class DecoderLayerDesc(C.Structure):
    _fields_ = [(n, _i64) for n in ("B", "S", "d", "Hq", "Hkv", "D", "d_ff", "L_max",
                                     "r_q", "r_k", "r_v", "r_o", "r_g", "r_u", "r_d")] + [
        ("norm_eps", _f32), ("rope_theta", _f32), ("softmax_scale", _f32),
        ("advance_seqlens", _i32), ("flags", _i32)] + [
        (n, _vp) for n in ("x", "y", "attn_norm_w", "mlp_norm_w", "A_qkv", "Vt_q", "Vt_k", "Vt_v", "Ut_o", "Vt_o",
                           "A_gu", "Vt_g", "Vt_u", "Ut_d", "Vt_d", "k_cache", "v_cache", "cache_seqlens", "ws")] + [
        ("ws_bytes", _sz), ("prefill_chunk", _i64)]


_SIGS = {
    "fsvd_abi_version": (C.c_int, []),
    "fsvd_status_str": (C.c_char_p, [C.c_int]),
    "fsvd_last_error": (C.c_char_p, []),
    "fsvd_prepack": (C.c_int, [_vp, _i64, _i64, C.POINTER(PackItem), C.c_int, C.c_int, _vp]),
    "fsvd_prepack_colscale": (C.c_int, [_vp, _i64, _i64, C.POINTER(PackItem), C.c_int, _vp, C.c_int, _vp]),
    "fsvd_lowrank_linear_ws": (_sz, [_i64, _i64, _i64, _i64, C.c_int]),
    "fsvd_lowrank_linear": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64,
                                      _vp, _i64, C.c_int, _vp, _sz, _vp]),
    "fsvd_lowrank_linear_noalloc": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _vp,
                                              _i64, _vp, _i64, C.c_int, _vp]),
    "fsvd_lowrank_qkv_ws": (_sz, [_i64] * 9),
    "fsvd_lowrank_qkv": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _f32, _vp, _i64, _i64, _i64, _vp, _vp, _vp,
                                   _i64, _i64, _i64, _f32, _vp, _vp, _vp, _i64, _vp, _vp, _vp, C.c_int, _vp, _sz,
                                   _vp]),
    "fsvd_lowrank_mlp_packed_ws": (_sz, [_i64] * 6),
    "fsvd_lowrank_mlp_packed": (C.c_int, [_vp, _i64, _i64, _vp, _f32, C.c_int, _vp, _i64, _i64, _vp, _vp, _i64,
                                          _vp, _vp, _i64, _vp, _vp, C.c_int, _vp, _sz, _vp]),
    "fsvd_decode_attn_dense_kv_ws": (_sz, [_i64] * 6),
    "fsvd_decode_attn_dense_kv": (C.c_int, [_vp, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _f32, C.c_int,
                                            _vp, C.c_int, _vp, _sz, _vp]),
    "fsvd_decode_attn_lowrank_kv_ws": (_sz, [_i64, _i64, _i64, _i64, _i64, _i64]),
    "fsvd_decode_attn_lowrank_kv": (C.c_int, [_vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _i64,
                                              _i64, _i64, _f32, _f32, C.c_int, _vp, C.c_int, _vp, _sz, _vp]),
    "fsvd_attn_factorized": (C.c_int, [_vp, _vp, _vp, _i64, _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i64, _i64, _i64,
                                       _i64, _f32, _f32, C.c_int, _vp, C.c_int, _vp]),
    "fsvd_swift_covariance_ws": (_sz, [_i64, _i64, _i64]),
    "fsvd_swift_covariance": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _vp, _sz, _vp]),
    "fsvd_swift_factors_ws": (_sz, [_i64, _i64]),
    "fsvd_swift_factors": (C.c_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
    "fsvd_layernorm": (C.c_int, [_vp, _vp, _vp, _vp, _f32, _i64, _i64, _vp, C.c_int, _vp]),
    "fsvd_seqlens_advance": (C.c_int, [_vp, _i64, _i32, _vp]),
    "fsvd_dense_linear": (C.c_int, [_vp, _i64, _i64, _i64, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _i64, C.c_int,
                                    _vp]),
    "fsvd_read_stream_probe": (C.c_int, [_vp, _sz, _vp, _vp]),
    "fsvd_decoder_layer_ws": (_sz, [C.POINTER(DecoderLayerDesc)]),
    "fsvd_decoder_layer_run": (C.c_int, [C.POINTER(DecoderLayerDesc), _vp]),
    "fsvd_decoder_layer_capture": (C.c_int, [C.POINTER(DecoderLayerDesc), C.POINTER(_vp)]),
    "fsvd_decoder_stack_capture": (C.c_int, [C.POINTER(DecoderLayerDesc), C.c_int, C.POINTER(_vp)]),
    "fsvd_graph_replay": (C.c_int, [_vp, _vp]),
    "fsvd_graph_destroy": (C.c_int, [_vp]),
    "fsvd_poll_device_error": (C.c_int, [_vp, _vp, C.POINTER(_i32)]),
}

_lib = None


def lib():
    """Load libfsvd.so (built in-tree by ``__graft_entry__.build()``); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"fsvd HIP library not built: {LIB_PATH} is missing (run __graft_entry__.build())")
        # torch ships its own HIP runtime under the same soname (libamdhip64.so.7) but links it by
        # file name; loaded first, torch's copy satisfies this library's dependency and the process
        # has one runtime, so tensors, streams and device state are shared.  Loaded after this
        # library, torch would bring a second runtime that holds the device on its own.
        import torch  # noqa: F401
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _p(t):
    """Device pointer of a tensor (or None / an int passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != FSVD_OK:
        L = lib()
        raise FsvdError(status, L.fsvd_status_str(status).decode(), L.fsvd_last_error().decode())


def dtype_of(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FSVD_BF16
    if t.dtype == torch.float32:
        return FSVD_F32
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def workspace(nbytes: int, device="cuda"):
    """A zero-filled byte workspace (its header, the device error word and the decode attention's
    partition counters, must start at zero)."""
    import torch
    return torch.zeros(max(int(nbytes), 4096), dtype=torch.uint8, device=device)


# ----------------------------------------------------------------------------- the ABI calls


def fsvd_abi_version() -> int:
    return lib().fsvd_abi_version()


def fsvd_status_str(s: int) -> str:
    return lib().fsvd_status_str(s).decode()


def fsvd_last_error() -> str:
    return lib().fsvd_last_error().decode()


def fsvd_prepack(dst, ld_dst, cols_pad, items, dtype, stream=None):
    """items: sequence of (src_tensor, rows, cols, ld_src, rows_pad)."""
    arr = (PackItem * len(items))(*[PackItem(_p(s), r, c, ld, rp) for (s, r, c, ld, rp) in items])
    _check(lib().fsvd_prepack(_p(dst), ld_dst, cols_pad, arr, len(items), dtype, _s(stream)))


def fsvd_prepack_colscale(dst, ld_dst, cols_pad, items, col_scale, dtype, stream=None):
    """As fsvd_prepack, every column c scaled by col_scale[c] (folds an RMSNorm weight into A)."""
    arr = (PackItem * len(items))(*[PackItem(_p(s), r, c, ld, rp) for (s, r, c, ld, rp) in items])
    _check(lib().fsvd_prepack_colscale(_p(dst), ld_dst, cols_pad, arr, len(items), _p(col_scale), dtype, _s(stream)))


def fsvd_lowrank_linear_ws(M, K, r, N, dtype) -> int:
    return lib().fsvd_lowrank_linear_ws(M, K, r, N, dtype)


def fsvd_lowrank_linear(x, M, K, ldx, Ut, r, ldu, Vt, N, ldv, bias, residual, ldr, y, ldy, dtype, ws, ws_bytes,
                        stream=None):
    _check(lib().fsvd_lowrank_linear(_p(x), M, K, ldx, _p(Ut), r, ldu, _p(Vt), N, ldv, _p(bias), _p(residual), ldr,
                                     _p(y), ldy, dtype, _p(ws), ws_bytes, _s(stream)))


def fsvd_lowrank_linear_noalloc(x, M, K, ldx, Ut, r, ldu, Vt, N, ldv, bias, residual, ldr, y, ldy, dtype,
                                stream=None):
    """fsvd_lowrank_linear with the library's static per-GPU scratch instead of a workspace."""
    _check(lib().fsvd_lowrank_linear_noalloc(_p(x), M, K, ldx, _p(Ut), r, ldu, _p(Vt), N, ldv, _p(bias),
                                             _p(residual), ldr, _p(y), ldy, dtype, _s(stream)))


FSVD_NOALLOC_SCRATCH_BYTES = 32 << 20


def fsvd_lowrank_qkv_ws(B, S, d, r_q, r_k, r_v, Hq, Hkv, D) -> int:
    return lib().fsvd_lowrank_qkv_ws(B, S, d, r_q, r_k, r_v, Hq, Hkv, D)


def fsvd_lowrank_qkv(x, B, S, d, norm_w, norm_eps, A_qkv, r_q, r_k, r_v, Vt_q, Vt_k, Vt_v, Hq, Hkv, D, rope_theta,
                     q_out, k_cache, v_cache, L_max, cache_seqlens, k_out, v_out, dtype, ws, ws_bytes, stream=None):
    _check(lib().fsvd_lowrank_qkv(_p(x), B, S, d, _p(norm_w), norm_eps, _p(A_qkv), r_q, r_k, r_v, _p(Vt_q),
                                  _p(Vt_k), _p(Vt_v), Hq, Hkv, D, rope_theta, _p(q_out), _p(k_cache), _p(v_cache),
                                  L_max, _p(cache_seqlens), _p(k_out), _p(v_out), dtype, _p(ws), ws_bytes,
                                  _s(stream)))


def fsvd_lowrank_mlp_packed_ws(M, d, r_g, r_u, d_ff, r_d) -> int:
    return lib().fsvd_lowrank_mlp_packed_ws(M, d, r_g, r_u, d_ff, r_d)


def fsvd_lowrank_mlp_packed(x, M, d, norm_w, norm_eps, act, A_gu, r_g, r_u, Vt_g, Vt_u, d_ff, Ut_d, Vt_d, r_d,
                            residual, y, dtype, ws, ws_bytes, stream=None):
    _check(lib().fsvd_lowrank_mlp_packed(_p(x), M, d, _p(norm_w), norm_eps, act, _p(A_gu), r_g, r_u, _p(Vt_g),
                                         _p(Vt_u), d_ff, _p(Ut_d), _p(Vt_d), r_d, _p(residual), _p(y), dtype, _p(ws),
                                         ws_bytes, _s(stream)))


def fsvd_decode_attn_dense_kv_ws(B, Sq, Hq, Hkv, D, L_max) -> int:
    return lib().fsvd_decode_attn_dense_kv_ws(B, Sq, Hq, Hkv, D, L_max)


def fsvd_decode_attn_dense_kv(q, k_cache, v_cache, L_max, cache_seqlens, B, Sq, Hq, Hkv, D, softmax_scale, causal,
                              out, dtype, ws, ws_bytes, stream=None):
    _check(lib().fsvd_decode_attn_dense_kv(_p(q), _p(k_cache), _p(v_cache), L_max, _p(cache_seqlens), B, Sq, Hq, Hkv,
                                           D, softmax_scale, int(causal), _p(out), dtype, _p(ws), ws_bytes,
                                           _s(stream)))


def fsvd_decode_attn_lowrank_kv_ws(B, Sq, Hq, Hkv, D, L_max) -> int:
    return lib().fsvd_decode_attn_lowrank_kv_ws(B, Sq, Hq, Hkv, D, L_max)


def fsvd_decode_attn_lowrank_kv(q, zk_cache, zv_cache, ldz, Vt_k, r_k, Vt_v, r_v, L_max, cache_seqlens, B, Sq, Hq,
                                Hkv, D, rope_theta, softmax_scale, causal, out, dtype, ws, ws_bytes, stream=None):
    _check(lib().fsvd_decode_attn_lowrank_kv(_p(q), _p(zk_cache), _p(zv_cache), ldz, _p(Vt_k), r_k, _p(Vt_v), r_v,
                                             L_max, _p(cache_seqlens), B, Sq, Hq, Hkv, D, rope_theta, softmax_scale,
                                             int(causal), _p(out), dtype, _p(ws), ws_bytes, _s(stream)))


def fsvd_attn_factorized(zq, zk, zv, ldz, Vt_q, r_q, Vt_k, r_k, Vt_v, r_v, B, S, Hq, Hkv, D, rope_theta, softmax_scale,
                         causal, out, dtype, stream=None):
    _check(lib().fsvd_attn_factorized(_p(zq), _p(zk), _p(zv), ldz, _p(Vt_q), r_q, _p(Vt_k), r_k, _p(Vt_v), r_v, B, S,
                                      Hq, Hkv, D, rope_theta, softmax_scale, int(causal), _p(out), dtype, _s(stream)))


def fsvd_swift_covariance_ws(T, d_in, d_out) -> int:
    return lib().fsvd_swift_covariance_ws(T, d_in, d_out)


def fsvd_swift_covariance(X, T, d_in, ldx, Wt, d_out, C, ldc, ws, ws_bytes, stream=None):
    _check(lib().fsvd_swift_covariance(_p(X), T, d_in, ldx, _p(Wt), d_out, _p(C), ldc, _p(ws), ws_bytes, _s(stream)))


def fsvd_swift_factors_ws(d_in, d_out) -> int:
    return lib().fsvd_swift_factors_ws(d_in, d_out)


def fsvd_swift_factors(Wt, d_out, d_in, VkT, k, Ut, Vt, ws, ws_bytes, stream=None):
    _check(lib().fsvd_swift_factors(_p(Wt), d_out, d_in, _p(VkT), k, _p(Ut), _p(Vt), _p(ws), ws_bytes, _s(stream)))


def fsvd_layernorm(x, residual, gamma, beta, eps, M, d, y, dtype, stream=None):
    _check(lib().fsvd_layernorm(_p(x), _p(residual), _p(gamma), _p(beta), eps, M, d, _p(y), dtype, _s(stream)))


def fsvd_dense_linear(x, M, K, ldx, W, N, ldw, bias, residual, ldr, y, ldy, dtype, stream=None):
    """Comparator: y = residual + bias + x . W^T through the low-rank linear's second-phase kernels."""
    _check(lib().fsvd_dense_linear(_p(x), M, K, ldx, _p(W), N, ldw, _p(bias), _p(residual), ldr, _p(y), ldy, dtype,
                                   _s(stream)))


def fsvd_read_stream_probe(src, nbytes, out, stream=None):
    _check(lib().fsvd_read_stream_probe(_p(src), nbytes, _p(out), _s(stream)))


def fsvd_seqlens_advance(cache_seqlens, B, n, stream=None):
    _check(lib().fsvd_seqlens_advance(_p(cache_seqlens), B, n, _s(stream)))


def fsvd_decoder_layer_ws(desc: DecoderLayerDesc) -> int:
    return lib().fsvd_decoder_layer_ws(C.byref(desc))


def fsvd_decoder_layer_run(desc: DecoderLayerDesc, stream=None):
    _check(lib().fsvd_decoder_layer_run(C.byref(desc), _s(stream)))


def fsvd_decoder_layer_capture(desc: DecoderLayerDesc) -> int:
    out = _vp()
    _check(lib().fsvd_decoder_layer_capture(C.byref(desc), C.byref(out)))
    return out.value


def fsvd_decoder_stack_capture(descs) -> int:
    """One graph holding the decode steps of every layer descriptor in order."""
    arr = (DecoderLayerDesc * len(descs))(*descs)
    out = _vp()
    _check(lib().fsvd_decoder_stack_capture(arr, len(descs), C.byref(out)))
    return out.value


def fsvd_graph_replay(graph: int, stream=None):
    _check(lib().fsvd_graph_replay(graph, _s(stream)))


def fsvd_graph_destroy(graph: int):
    _check(lib().fsvd_graph_destroy(graph))


def fsvd_poll_device_error(ws, stream=None) -> int:
    """Returns the device error word (0 when clean); clears it."""
    code = _i32(0)
    st = lib().fsvd_poll_device_error(_p(ws), _s(stream), C.byref(code))
    if st not in (FSVD_OK, FSVD_ERR_DEVICE):
        _check(st)
    return code.value


def decoder_layer_desc(**kw) -> DecoderLayerDesc:
    """Fill a DecoderLayerDesc; tensor values become their data pointers."""
    d = DecoderLayerDesc()
    for k, v in kw.items():
        if not hasattr(d, k):
            raise KeyError(k)
        if hasattr(v, "data_ptr"):
            v = v.data_ptr()
        setattr(d, k, v)
    return d
