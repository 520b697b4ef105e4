"""ctypes binding of libmoe_lp.so (include/moe_lp.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the MoE expert forward runs in the library's kernels.
If the library is missing the first call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_lp.so")
_lib = None

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_DEVICE = range(5)
FMT_INT4, FMT_FP8, FMT_MXFP4, FMT_FP8_POW2, FMT_NVFP4 = 1, 2, 3, 4, 5
WL_ROWS, WL_KBLOCKED = 0, 1

EXPORTED = ("moe_abi_version", "moe_status_str", "moe_workspace_bytes", "moe_route_workspace_bytes", "moe_tile_rows",
            "moe_route_permute", "moe_expert_forward", "moe_expert_forward_timed", "moe_combine",
            "moe_lm_head_workspace_bytes", "moe_lm_head_logprob", "moe_materialized_workspace_bytes",
            "moe_expert_forward_materialized", "moe_backward_weights_bytes", "moe_prepare_backward_weights",
            "moe_backward_workspace_bytes", "moe_expert_backward", "moe_pack_weights_kblocked",
            "moe_quantize_activations", "moe_expert_forward_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES
STAGES = ("route", "permute", "act", "gemm1", "gemm2", "combine", "dequant")


class MoeLayer(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("wformat", ctypes.c_int32),
                ("oft_block", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
                ("adapter_expert_stride", ctypes.c_int64), ("weight_layout", ctypes.c_int32)]


class MoeQWeights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p)]


class MoeScales(ctypes.Structure):
    _fields_ = [("s13", ctypes.c_void_p), ("s2", ctypes.c_void_p), ("g13", ctypes.c_void_p), ("g2", ctypes.c_void_p)]


class MoeRouteOut(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p), ("expert_offsets", ctypes.c_void_p),
                ("sorted_rows", ctypes.c_void_p), ("row_of", ctypes.c_void_p), ("active_experts", ctypes.c_void_p),
                ("num_active", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_str(status)} (status {status})")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(_LIB_PATH)
        L.moe_abi_version.restype = ctypes.c_int32
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_workspace_bytes.restype = ctypes.c_size_t
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_int32]
        L.moe_tile_rows.restype = ctypes.c_int32
        L.moe_tile_rows.argtypes = [ctypes.POINTER(MoeLayer)]
        L.moe_route_workspace_bytes.restype = ctypes.c_size_t
        L.moe_route_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayer)]
        L.moe_lm_head_workspace_bytes.restype = ctypes.c_size_t
        L.moe_lm_head_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.moe_route_permute.restype = ctypes.c_int
        L.moe_route_permute.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_void_p, ctypes.POINTER(MoeRouteOut),
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.moe_expert_forward.restype = ctypes.c_int
        L.moe_expert_forward.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.POINTER(MoeQWeights), ctypes.POINTER(MoeScales), ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
        L.moe_expert_forward_noalloc.restype = ctypes.c_int
        L.moe_expert_forward_noalloc.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.POINTER(MoeQWeights), ctypes.POINTER(MoeScales),
                                                 ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
        L.moe_expert_forward_timed.restype = ctypes.c_int
        L.moe_expert_forward_timed.argtypes = L.moe_expert_forward.argtypes + [ctypes.POINTER(ctypes.c_float),
                                                                                ctypes.POINTER(ctypes.c_int32)]
        L.moe_materialized_workspace_bytes.restype = ctypes.c_size_t
        L.moe_materialized_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_int32]
        L.moe_expert_forward_materialized.restype = ctypes.c_int
        L.moe_expert_forward_materialized.argtypes = L.moe_expert_forward_timed.argtypes
        L.moe_backward_weights_bytes.restype = ctypes.c_size_t
        L.moe_backward_weights_bytes.argtypes = [ctypes.POINTER(MoeLayer)]
        L.moe_pack_weights_kblocked.restype = ctypes.c_int
        L.moe_pack_weights_kblocked.argtypes = [ctypes.POINTER(MoeLayer), ctypes.POINTER(MoeQWeights),
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.moe_prepare_backward_weights.restype = ctypes.c_int
        L.moe_prepare_backward_weights.argtypes = [ctypes.POINTER(MoeLayer), ctypes.POINTER(MoeQWeights),
                                                   ctypes.POINTER(MoeScales), ctypes.c_void_p, ctypes.c_size_t,
                                                   ctypes.c_void_p]
        L.moe_backward_workspace_bytes.restype = ctypes.c_size_t
        L.moe_backward_workspace_bytes.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_int32]
        L.moe_expert_backward.restype = ctypes.c_int
        L.moe_expert_backward.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.POINTER(MoeQWeights), ctypes.POINTER(MoeScales), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_void_p, ctypes.POINTER(ctypes.c_float),
                                          ctypes.POINTER(ctypes.c_int32)]
        L.moe_quantize_activations.restype = ctypes.c_int
        L.moe_quantize_activations.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_void_p, ctypes.c_void_p,
                                               ctypes.c_void_p, ctypes.c_void_p]
        L.moe_combine.restype = ctypes.c_int
        L.moe_combine.argtypes = [ctypes.POINTER(MoeLayer), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p]
        L.moe_lm_head_logprob.restype = ctypes.c_int
        L.moe_lm_head_logprob.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    return t.data_ptr()


def _need(t, name: str, nbytes: int, elem: int | None = None):
    """A device tensor, contiguous, of at least nbytes (and elem-byte elements
    when given): the library reads and writes exactly the sizes the layer
    implies, so a smaller or strided tensor would be accessed out of bounds."""
    if t is None:
        raise ValueError(f"{name}: tensor required")
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name}: contiguous device tensor expected")
    if elem is not None and t.element_size() != elem:
        raise ValueError(f"{name}: {elem}-byte elements expected, got {t.dtype}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, the layer needs {nbytes}")


def _weight_bytes(fmt: int, N: int, K: int, E: int):
    """(packed code bytes, scale bytes) of E expert matrices [N][K]."""
    codes = E * N * K if fmt in (FMT_FP8, FMT_FP8_POW2) else E * N * K // 2
    if fmt == FMT_INT4:
        sc = E * (K // 32) * N * 2
    elif fmt in (FMT_FP8, FMT_FP8_POW2):
        sc = E * (N // 128) * (K // 128) * 4
    elif fmt == FMT_NVFP4:
        sc = E * (K // 16) * N
    else:
        sc = E * (K // 32) * N
    return codes, sc


def _check_forward_args(layer: MoeLayer, x, logits, w13, w2, s13, s2, adapter, out, g13, g2):
    T, H, I, E = layer.num_tokens, layer.hidden, layer.inter, layer.num_experts
    if T == 0:
        return
    fmt = layer.wformat
    _need(x, "x", T * H * 2, 2)
    _need(logits, "logits", T * E * 4, 4)
    _need(out, "out", T * H * 2, 2)
    c13, sc13 = _weight_bytes(fmt, 2 * I, H, E)
    c2, sc2 = _weight_bytes(fmt, H, I, E)
    _need(w13, "w13", c13)
    _need(w2, "w2", c2)
    _need(s13, "s13", sc13)
    _need(s2, "s2", sc2)
    if fmt == FMT_NVFP4:
        _need(g13, "g13", E * 4, 4)
        _need(g2, "g2", E * 4, 4)
    if layer.oft_block:
        stride = layer.adapter_expert_stride
        _need(adapter, "adapter", ((E - 1) * stride + H * 32) * 2 if stride else H * 32 * 2, 2)


def _stream():
    return torch.cuda.current_stream().cuda_stream


def make_layer(T, H, I, E, k, fmt, oft=False, adapter_expert_stride=None, tile_rows=0,
               weight_layout=0) -> MoeLayer:
    stride = (H // 32) * 1024 if adapter_expert_stride is None else adapter_expert_stride
    return MoeLayer(T, H, I, E, k, fmt, 32 if oft else 0, tile_rows, stride if oft else 0, weight_layout)


def workspace_bytes(layer: MoeLayer, chunk_experts: int = 1) -> int:
    return lib().moe_workspace_bytes(ctypes.byref(layer), int(chunk_experts))


def tile_rows(layer: MoeLayer) -> int:
    return lib().moe_tile_rows(ctypes.byref(layer))


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def route_permute(logits: torch.Tensor, layer: MoeLayer, ws: torch.Tensor | None = None) -> dict:
    """Router top-k + permutation; returns a dict of device tensors."""
    T, E, k = layer.num_tokens, layer.num_experts, layer.top_k
    dev = logits.device
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(topk_ids=torch.empty((T, k), **i32), topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
               expert_offsets=torch.empty(E + 1, **i32), sorted_rows=torch.empty(T * k, **i32),
               row_of=torch.empty(T * k, **i32), active_experts=torch.empty(E, **i32),
               num_active=torch.zeros(4, **i32))
    ro = MoeRouteOut(*[_ptr(out[n]) for n in ("topk_ids", "topk_w", "expert_offsets", "sorted_rows", "row_of",
                                              "active_experts", "num_active")])
    if ws is None:
        ws = alloc_workspace(lib().moe_route_workspace_bytes(ctypes.byref(layer)), dev)
    _check(lib().moe_route_permute(ctypes.byref(layer), _ptr(logits), ctypes.byref(ro), _ptr(ws), ws.numel(),
                                   _stream()), "moe_route_permute")
    return out


def expert_forward(layer: MoeLayer, x: torch.Tensor, logits: torch.Tensor, w13, w2, s13, s2, adapter=None,
                   chunk_experts: int = 1, out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                   g13=None, g2=None):
    """moe_expert_forward: x [T][H] bf16, logits [T][E] fp32 -> out [T][H] bf16."""
    if out is None:
        out = torch.empty((layer.num_tokens, layer.hidden), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = alloc_workspace(workspace_bytes(layer, chunk_experts), x.device)
    _check_forward_args(layer, x, logits, w13, w2, s13, s2, adapter, out, g13, g2)
    qw = MoeQWeights(_ptr(w13), _ptr(w2))
    sc = MoeScales(_ptr(s13), _ptr(s2), _ptr(g13), _ptr(g2))
    _check(lib().moe_expert_forward(ctypes.byref(layer), _ptr(x), _ptr(logits), ctypes.byref(qw), ctypes.byref(sc),
                                    _ptr(adapter), int(chunk_experts), _ptr(out), _ptr(ws), ws.numel(), _stream()),
           "moe_expert_forward")
    return out


def expert_forward_noalloc(layer: MoeLayer, x, logits, w13, w2, s13, s2, adapter=None, chunk_experts: int = 1,
                           out: torch.Tensor | None = None, g13=None, g2=None):
    """moe_expert_forward_noalloc: as expert_forward, with the library's static
    per-GPU scratch in place of a workspace (layers whose workspace fits it)."""
    if out is None:
        out = torch.empty((layer.num_tokens, layer.hidden), dtype=torch.bfloat16, device=x.device)
    if workspace_bytes(layer, chunk_experts) <= NOALLOC_SCRATCH_BYTES:  # else the library refuses first
        _check_forward_args(layer, x, logits, w13, w2, s13, s2, adapter, out, g13, g2)
    qw = MoeQWeights(_ptr(w13), _ptr(w2))
    sc = MoeScales(_ptr(s13), _ptr(s2), _ptr(g13), _ptr(g2))
    _check(lib().moe_expert_forward_noalloc(ctypes.byref(layer), _ptr(x), _ptr(logits), ctypes.byref(qw),
                                            ctypes.byref(sc), _ptr(adapter), int(chunk_experts), _ptr(out),
                                            _stream()), "moe_expert_forward_noalloc")
    return out


def expert_forward_timed(layer: MoeLayer, x, logits, w13, w2, s13, s2, adapter=None, chunk_experts: int = 1,
                         out=None, ws=None, g13=None, g2=None):
    """moe_expert_forward_timed: same result, plus per-stage event times.
    Returns (out, {stage: (ms, launches)})."""
    if out is None:
        out = torch.empty((layer.num_tokens, layer.hidden), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = alloc_workspace(workspace_bytes(layer, chunk_experts), x.device)
    _check_forward_args(layer, x, logits, w13, w2, s13, s2, adapter, out, g13, g2)
    qw = MoeQWeights(_ptr(w13), _ptr(w2))
    sc = MoeScales(_ptr(s13), _ptr(s2), _ptr(g13), _ptr(g2))
    ms = (ctypes.c_float * len(STAGES))()
    n = (ctypes.c_int32 * len(STAGES))()
    _check(lib().moe_expert_forward_timed(ctypes.byref(layer), _ptr(x), _ptr(logits), ctypes.byref(qw),
                                          ctypes.byref(sc), _ptr(adapter), int(chunk_experts), _ptr(out), _ptr(ws),
                                          ws.numel(), _stream(), ms, n), "moe_expert_forward_timed")
    return out, {name: (float(ms[i]), int(n[i])) for i, name in enumerate(STAGES)}


def materialized_workspace_bytes(layer: MoeLayer, chunk_experts: int) -> int:
    return lib().moe_materialized_workspace_bytes(ctypes.byref(layer), int(chunk_experts))


def expert_forward_materialized(layer: MoeLayer, x, logits, w13, w2, s13, s2, adapter=None, chunk_experts: int = 1,
                                out=None, ws=None, timed: bool = False, g13=None, g2=None):
    """moe_expert_forward_materialized: per chunk, the experts' BF16 copy in ws,
    then BF16 GEMMs.  Returns out, or (out, {stage: (ms, launches)}) if timed."""
    if out is None:
        out = torch.empty((layer.num_tokens, layer.hidden), dtype=torch.bfloat16, device=x.device)
    if ws is None:
        ws = alloc_workspace(materialized_workspace_bytes(layer, chunk_experts), x.device)
    _check_forward_args(layer, x, logits, w13, w2, s13, s2, adapter, out, g13, g2)
    qw = MoeQWeights(_ptr(w13), _ptr(w2))
    sc = MoeScales(_ptr(s13), _ptr(s2), _ptr(g13), _ptr(g2))
    ms = (ctypes.c_float * len(STAGES))() if timed else None
    n = (ctypes.c_int32 * len(STAGES))() if timed else None
    _check(lib().moe_expert_forward_materialized(ctypes.byref(layer), _ptr(x), _ptr(logits), ctypes.byref(qw),
                                                 ctypes.byref(sc), _ptr(adapter), int(chunk_experts), _ptr(out),
                                                 _ptr(ws), ws.numel(), _stream(), ms, n),
           "moe_expert_forward_materialized")
    if timed:
        return out, {name: (float(ms[i]), int(n[i])) for i, name in enumerate(STAGES)}
    return out


def backward_weights_bytes(layer: MoeLayer) -> int:
    return lib().moe_backward_weights_bytes(ctypes.byref(layer))


def prepare_backward_weights(layer: MoeLayer, w13, w2, s13, s2, out: torch.Tensor | None = None) -> torch.Tensor:
    """moe_prepare_backward_weights: the transposed copy of the frozen weights."""
    n = backward_weights_bytes(layer)
    if n == 0:
        raise MoeError(MOE_ERR_UNSUPPORTED, "moe_backward_weights_bytes")
    if out is None:
        out = torch.empty(n, dtype=torch.uint8, device=w13.device)
    qw = MoeQWeights(_ptr(w13), _ptr(w2))
    sc = MoeScales(_ptr(s13), _ptr(s2), None, None)
    _check(lib().moe_prepare_backward_weights(ctypes.byref(layer), ctypes.byref(qw), ctypes.byref(sc), _ptr(out),
                                              out.numel(), _stream()), "moe_prepare_backward_weights")
    return out


def pack_weights_kblocked(layer: MoeLayer, w13, w2):
    """moe_pack_weights_kblocked -> (w13, w2) in 16-row x 128-K tiles (same sizes)."""
    o13, o2 = torch.empty_like(w13), torch.empty_like(w2)
    qw = MoeQWeights(_ptr(w13), _ptr(w2))
    _check(lib().moe_pack_weights_kblocked(ctypes.byref(layer), ctypes.byref(qw), _ptr(o13), _ptr(o2), _stream()),
           "moe_pack_weights_kblocked")
    return o13, o2


def backward_workspace_bytes(layer: MoeLayer, chunk_experts: int = 1) -> int:
    return lib().moe_backward_workspace_bytes(ctypes.byref(layer), int(chunk_experts))


def expert_backward(layer: MoeLayer, x, logits, w13, w2, s13, s2, bwd_weights, d_out, adapter=None,
                    chunk_experts: int = 1, ws=None, d_x=None, d_logits=None, d_adapter=None, timed: bool = False,
                    g13=None, g2=None):
    """moe_expert_backward -> (d_x [T][H] bf16, d_logits [T][E] fp32, d_adapter fp32 or None)
    (+ {stage: (ms, launches)} if timed)."""
    T, H, E = layer.num_tokens, layer.hidden, layer.num_experts
    dev = x.device
    if d_x is None:
        d_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if d_logits is None:
        d_logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    if adapter is not None and d_adapter is None:
        d_adapter = torch.empty(adapter.shape, dtype=torch.float32, device=dev)
    if ws is None:
        ws = alloc_workspace(backward_workspace_bytes(layer, chunk_experts), dev)
    qw = MoeQWeights(_ptr(w13), _ptr(w2))
    sc = MoeScales(_ptr(s13), _ptr(s2), _ptr(g13), _ptr(g2))
    ms = (ctypes.c_float * len(STAGES))() if timed else None
    n = (ctypes.c_int32 * len(STAGES))() if timed else None
    _check(lib().moe_expert_backward(ctypes.byref(layer), _ptr(x), _ptr(logits), ctypes.byref(qw), ctypes.byref(sc),
                                     _ptr(bwd_weights), _ptr(adapter), _ptr(d_out), int(chunk_experts), _ptr(d_x),
                                     _ptr(d_logits), _ptr(d_adapter), _ptr(ws), ws.numel(), _stream(), ms, n),
           "moe_expert_backward")
    if timed:
        return d_x, d_logits, d_adapter, {name: (float(ms[i]), int(n[i])) for i, name in enumerate(STAGES)}
    return d_x, d_logits, d_adapter


def quantize_activations(layer: MoeLayer, x: torch.Tensor):
    """moe_quantize_activations -> (codes [T][H] uint8, scales): fp32 [T][H/128]
    for FP8 layers, E8M0 bytes [T][H/32] for MXFP4 layers."""
    T, H = layer.num_tokens, layer.hidden
    codes = torch.empty((T, H), dtype=torch.uint8, device=x.device)
    if layer.wformat in (FMT_FP8, FMT_FP8_POW2):
        scales = torch.empty((T, H // 128), dtype=torch.float32, device=x.device)
    else:
        scales = torch.empty((T, H // 32), dtype=torch.uint8, device=x.device)
    _check(lib().moe_quantize_activations(ctypes.byref(layer), _ptr(x), _ptr(codes), _ptr(scales), _stream()),
           "moe_quantize_activations")
    return codes, scales


def combine(layer: MoeLayer, y_perm: torch.Tensor, topk_w: torch.Tensor, row_of: torch.Tensor,
            out: torch.Tensor | None = None):
    if out is None:
        out = torch.empty((layer.num_tokens, layer.hidden), dtype=torch.bfloat16, device=y_perm.device)
    _check(lib().moe_combine(ctypes.byref(layer), _ptr(y_perm), _ptr(topk_w), _ptr(row_of), _ptr(out), _stream()),
           "moe_combine")
    return out


def lm_head_logprob(h: torch.Tensor, w_lm: torch.Tensor, targets: torch.Tensor, ws: torch.Tensor | None = None):
    T, H = h.shape
    V = w_lm.shape[0]
    lp = torch.empty(T, dtype=torch.float32, device=h.device)
    if ws is None:
        ws = alloc_workspace(lib().moe_lm_head_workspace_bytes(T, V), h.device)
    _check(lib().moe_lm_head_logprob(T, H, V, _ptr(h), _ptr(w_lm), _ptr(targets), _ptr(lp), _ptr(ws), ws.numel(),
                                     _stream()), "moe_lm_head_logprob")
    return lp
