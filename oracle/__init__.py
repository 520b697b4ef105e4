"""CPU oracle for the low-precision MoE expert forward: ctypes wrapper.

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU-baseline leg import this package.  The product library never loads it.

The arithmetic lives in moe_oracle.c (plain C, fp64 accumulation, OpenMP);
this module only builds that file with gcc and marshals numpy arrays.
Parity pins are in tests/test_oracle_*.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

FMT_INT4, FMT_FP8, FMT_MXFP4, FMT_FP8_POW2, FMT_NVFP4 = 1, 2, 3, 4, 5


def build(force: bool = False) -> str:
    """Compile moe_oracle.c -> liboracle.so with gcc (IEEE semantics, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Layer(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("fmt", ctypes.c_int32),
                ("oft_block", ctypes.c_int32), ("adapter_expert_stride", ctypes.c_int64),
                ("materialized", ctypes.c_int32), ("g13", ctypes.c_void_p), ("g2", ctypes.c_void_p)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            _lib = ctypes.CDLL(build())
            _lib.oracle_route.restype = ctypes.c_int
            _lib.oracle_permute.restype = ctypes.c_int
            _lib.oracle_forward.restype = ctypes.c_int
            _lib.oracle_combine.restype = ctypes.c_int
            _lib.oracle_lm_head_logprob.restype = ctypes.c_int
            _lib.oracle_num_threads.restype = ctypes.c_int
            _lib.oracle_backward.restype = ctypes.c_int
        return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    return lib().oracle_num_threads()


def route(logits: np.ndarray, k: int):
    """-> (topk_ids[T][k] int32, topk_w[T][k] float32)."""
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    if lib().oracle_route(T, E, k, _p(logits), _p(ids), _p(w)) != 0:
        raise ValueError("oracle_route: invalid arguments")
    return ids, w


def permute(ids: np.ndarray, E: int):
    """-> dict(counts, offsets, sorted_rows, row_of, active) (int32 arrays)."""
    ids = _c(ids, np.int32)
    T, k = ids.shape
    R = T * k
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    sorted_rows = np.empty(R, np.int32)
    row_of = np.empty(R, np.int32)
    active = np.empty(E, np.int32)
    na = ctypes.c_int32(0)
    if lib().oracle_permute(T, E, k, _p(ids), _p(counts), _p(offsets), _p(sorted_rows), _p(row_of),
                            _p(active), ctypes.byref(na)) != 0:
        raise ValueError("oracle_permute: invalid ids")
    return dict(counts=counts, offsets=offsets, sorted_rows=sorted_rows, row_of=row_of,
                active=active[:na.value].copy())


def decode(kind: str, codes: np.ndarray) -> np.ndarray:
    """kind in bf16 | int4 | e4m3 | e2m1 | e8m0 -> float64 values."""
    fmt = {"bf16": 0, "int4": 1, "e4m3": 2, "e2m1": 3, "e8m0": 4}[kind]
    codes = _c(codes, np.uint16 if fmt == 0 else np.uint8)
    out = np.empty(codes.shape, np.float64)
    lib().oracle_decode(fmt, ctypes.c_int64(codes.size), _p(codes), _p(out))
    return out


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_encode_e4m3(ctypes.c_int64(v.size), _p(v), _p(out))
    return out


def quant_fp8(v: np.ndarray):
    """[R][K] fp32 -> (codes [R][K] uint8, scales [R][K/128] fp32)."""
    v = _c(v, np.float32)
    R, K = v.shape
    q = np.empty((R, K), np.uint8)
    s = np.empty((R, K // 128), np.float32)
    lib().oracle_quant_fp8(R, K, _p(v), _p(q), _p(s))
    return q, s


def quant_fp8_pow2(v: np.ndarray):
    """[R][K] fp32 -> (codes [R][K] uint8, power-of-two scales [R][K/128] fp32)."""
    v = _c(v, np.float32)
    R, K = v.shape
    q = np.empty((R, K), np.uint8)
    s = np.empty((R, K // 128), np.float32)
    lib().oracle_quant_fp8_pow2(R, K, _p(v), _p(q), _p(s))
    return q, s


def quant_mxfp8(v: np.ndarray):
    """[R][K] fp32 -> (codes [R][K] uint8, E8M0 scale bytes [R][K/32])."""
    v = _c(v, np.float32)
    R, K = v.shape
    q = np.empty((R, K), np.uint8)
    e = np.empty((R, K // 32), np.uint8)
    lib().oracle_quant_mxfp8(R, K, _p(v), _p(q), _p(e))
    return q, e


def dequant(fmt: int, N: int, K: int, q: np.ndarray, s: np.ndarray, g: float = 1.0) -> np.ndarray:
    """One expert's packed [N][K] weights -> fp32 [N][K] (g: NVFP4 second-level scale)."""
    out = np.empty((N, K), np.float32)
    lib().oracle_dequant(fmt, N, K, _p(_c(q, np.uint8)), _p(np.ascontiguousarray(s)), ctypes.c_double(g), _p(out))
    return out


def round_bf16(v: np.ndarray) -> np.ndarray:
    """float64 values -> nearest bf16 value (ties to even), as float64."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.float64)
    lib().oracle_round_bf16(ctypes.c_int64(v.size), _p(v), _p(out))
    return out


def dequant_bf16(fmt: int, N: int, K: int, q: np.ndarray, s: np.ndarray, g: float = 1.0) -> np.ndarray:
    """One expert's packed [N][K] weights -> the BF16 temporary copy's values (fp32)."""
    out = np.empty((N, K), np.float32)
    lib().oracle_dequant_bf16(fmt, N, K, _p(_c(q, np.uint8)), _p(np.ascontiguousarray(s)), ctypes.c_double(g),
                              _p(out))
    return out


def _layer(T, H, I, E, k, fmt, oft, stride, materialized, g13, g2):
    """oracle_layer plus the arrays its pointers reference (kept alive by the caller)."""
    g13 = None if g13 is None else _c(g13, np.float32)
    g2 = None if g2 is None else _c(g2, np.float32)
    layer = _Layer(T, H, I, E, k, fmt, 32 if oft is not None else 0, stride, 1 if materialized else 0,
                   _p(g13), _p(g2))
    return layer, (g13, g2)


def forward(T, H, I, E, k, fmt, x, logits, w13, w2, s13, s2, oft=None, chunk_experts=1,
            tokens=None, adapter_expert_stride=None, return_y=False, return_routing=False,
            materialized=False, g13=None, g2=None):
    """Oracle MoE expert forward.  x: [T][H] bf16 bits (uint16); logits [T][E] fp32;
    weights/scales in the packed storage layouts; oft [E][H/32][32][32] bf16 bits
    (or [H/32][32][32] with adapter_expert_stride=0) or None.
    tokens: optional int array of token indices to compute (default: all).
    materialized: BF16 temporary weights and bf16 GEMM inputs instead of the
    format's activation quantizers (the chunk dequantized to a BF16 copy).
    g13, g2: NVFP4 per-expert second-level scales of W13 and W2 (fp32 [E]).
    Returns out [n][H] fp32 (+ y [n][k][H], + (ids, w) when requested)."""
    layer, keep = _layer(T, H, I, E, k, fmt, oft,
                         (32 * 32 * (H // 32)) if adapter_expert_stride is None else adapter_expert_stride,
                         materialized, g13, g2)
    x = _c(x, np.uint16)
    logits = _c(logits, np.float32)
    w13 = _c(w13, np.uint8)
    w2 = _c(w2, np.uint8)
    s13 = np.ascontiguousarray(s13)
    s2 = np.ascontiguousarray(s2)
    oft_a = None if oft is None else _c(oft, np.uint16)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tok is None else len(tok)
    out = np.empty((n, H), np.float32)
    y = np.empty((n, k, H), np.float32) if return_y else None
    ids = np.empty((T, k), np.int32) if return_routing else None
    w = np.empty((T, k), np.float32) if return_routing else None
    rc = lib().oracle_forward(ctypes.byref(layer), _p(x), _p(logits), _p(w13), _p(w2), _p(s13), _p(s2),
                              _p(oft_a), int(chunk_experts), _p(tok), int(n), _p(out), _p(y), _p(ids), _p(w))
    if rc != 0:
        raise ValueError("oracle_forward: invalid arguments")
    res = [out]
    if return_y:
        res.append(y)
    if return_routing:
        res.append((ids, w))
    return res[0] if len(res) == 1 else tuple(res)


def forward_inputs(li, chunk_experts=None, tokens=None, **kw):
    """oracle forward on a synth.LayerInputs bundle."""
    c = li.cfg
    return forward(c.T, c.H, c.I, c.E, c.k, c.fmt, li.x, li.logits, li.w13, li.w2, li.s13, li.s2,
                   oft=li.oft, chunk_experts=c.chunk if chunk_experts is None else chunk_experts,
                   tokens=tokens, g13=getattr(li, "g13", None), g2=getattr(li, "g2", None), **kw)


def backward(T, H, I, E, k, fmt, x, logits, w13, w2, s13, s2, dout, oft=None, chunk_experts=1, tokens=None,
             adapter_expert_stride=None, return_g=False, g13=None, g2=None):
    """Frozen-base backward of the oracle forward.  dout: [n][H] fp32 gradient of
    the requested tokens' outputs (all tokens if tokens is None).
    Returns (dx [n][H] fp32, dlogits [n][E] fp32, doft or None), doft float64
    shaped like the adapter, summed over the requested tokens' rows; with
    return_g also g [n][k] float64 (g_tj = <dout_t, y_tj>)."""
    stride = (32 * 32 * (H // 32)) if adapter_expert_stride is None else adapter_expert_stride
    layer, keep = _layer(T, H, I, E, k, fmt, oft, stride, False, g13, g2)
    tok = None if tokens is None else _c(tokens, np.int32)
    n = T if tok is None else len(tok)
    dout = _c(dout, np.float32).reshape(n, H)
    dx = np.empty((n, H), np.float32)
    dl = np.empty((n, E), np.float32)
    doft = None
    if oft is not None:
        doft = np.zeros((E * stride if stride else H * 32,), np.float64)
    g = np.empty((n, k), np.float64) if return_g else None
    rc = lib().oracle_backward(ctypes.byref(layer), _p(_c(x, np.uint16)), _p(_c(logits, np.float32)),
                               _p(_c(w13, np.uint8)), _p(_c(w2, np.uint8)), _p(np.ascontiguousarray(s13)),
                               _p(np.ascontiguousarray(s2)), _p(None if oft is None else _c(oft, np.uint16)),
                               _p(dout), int(chunk_experts), _p(tok), int(n), _p(dx), _p(dl), _p(doft), _p(g))
    if rc != 0:
        raise ValueError("oracle_backward: invalid arguments")
    if doft is not None:
        doft = doft.reshape((E, H // 32, 32, 32) if stride else (H // 32, 32, 32))
    return (dx, dl, doft, g) if return_g else (dx, dl, doft)


def backward_inputs(li, dout, chunk_experts=None, tokens=None, return_g=False):
    """oracle backward on a synth.LayerInputs bundle."""
    c = li.cfg
    return backward(c.T, c.H, c.I, c.E, c.k, c.fmt, li.x, li.logits, li.w13, li.w2, li.s13, li.s2, dout,
                    oft=li.oft, chunk_experts=c.chunk if chunk_experts is None else chunk_experts, tokens=tokens,
                    return_g=return_g, g13=getattr(li, "g13", None), g2=getattr(li, "g2", None))


def combine(y_perm_bf16: np.ndarray, w: np.ndarray, row_of: np.ndarray) -> np.ndarray:
    y = _c(y_perm_bf16, np.uint16)
    w = _c(w, np.float32)
    row_of = _c(row_of, np.int32)
    T, k = w.shape
    H = y.shape[1]
    out = np.empty((T, H), np.float32)
    lib().oracle_combine(T, k, H, _p(y), _p(w), _p(row_of), _p(out))
    return out


def lm_head_logprob(h: np.ndarray, w_lm_bf16: np.ndarray, targets: np.ndarray) -> np.ndarray:
    h = _c(h, np.float32)
    w = _c(w_lm_bf16, np.uint16)
    tg = _c(targets, np.int32)
    T, H = h.shape
    V = w.shape[0]
    lp = np.empty(T, np.float32)
    if lib().oracle_lm_head_logprob(T, H, V, _p(h), _p(w), _p(tg), _p(lp)) != 0:
        raise ValueError("oracle_lm_head_logprob: target out of range")
    return lp
