"""MI355X (gfx950) Mixture-of-Experts layer forward and backward: Python binding.

A thin ctypes layer over libmoe.so (include/moe.h).  Every function here has
the name of the C entry point it calls and only marshals arguments: it checks
tensor devices, dtypes and shapes, allocates outputs and the workspace with
torch (device memory only), passes raw pointers and the current HIP stream,
and raises on a non-OK status.  All computation happens in the HIP kernels.

MoEFunction and MoELayer wrap moe_forward_train and moe_backward as a torch
autograd operation and module (again only calls into the library).

Importing this package fails if libmoe.so has not been built
(python mixture_experts_layer_21_amd/build.py).  MOE_LIBRARY, if set, names
another build of the same library to load instead (the tests use it for the
host-AddressSanitizer build).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LIBRARY") or os.path.join(_PKG, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with "
                      "'python mixture_experts_layer_21_amd/build.py' (needs ROCm hipcc)")

_lib = ctypes.CDLL(LIB_PATH)

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_LAUNCH = 0, 1, 2, 3
MOE_F32, MOE_BF16 = 0, 1
MOE_STAGE_ROUTE, MOE_STAGE_PERMUTE, MOE_STAGE_EXPERT_FFN, MOE_STAGE_COMBINE, MOE_STAGE_FORWARD = \
    0, 1, 2, 3, 4
MOE_STAGE_EXPERT_FFN_BACKWARD = 5
MOE_STAGE_EXPERT_FFN_GATHER = 6
MOE_GATE_TOPK_SOFTMAX, MOE_GATE_SOFTMAX_TOPK = 0, 1
EXPORTS = ("moe_status_string", "moe_workspace_bytes", "moe_stage_workspace_bytes", "moe_route",
           "moe_route_ex", "moe_expert_capacity", "moe_permute", "moe_permute_ex",
           "moe_expert_ffn", "moe_expert_ffn_gather", "moe_combine", "moe_forward",
           "moe_forward_ex", "moe_forward_noalloc", "moe_saved_bytes",
           "moe_backward_workspace_bytes", "moe_forward_train", "moe_backward",
           "moe_expert_ffn_backward")

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_lib.moe_status_string.restype = ctypes.c_char_p
_lib.moe_status_string.argtypes = [_i32]
_lib.moe_workspace_bytes.restype = _i32
_lib.moe_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64, _i32, ctypes.POINTER(_sz)]
_lib.moe_stage_workspace_bytes.restype = _i32
_lib.moe_stage_workspace_bytes.argtypes = [_i32, _i64, _i64, _i64, _i32, _i64, _i32,
                                           ctypes.POINTER(_sz)]
_lib.moe_route.restype = _i32
_lib.moe_route.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
_lib.moe_route_ex.restype = _i32
_lib.moe_route_ex.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _i32, _vp, _vp,
                              _vp, _sz, _vp]
_lib.moe_expert_capacity.restype = _i32
_lib.moe_expert_capacity.argtypes = [_i64, _i32, _i64, _i64, _i64, ctypes.POINTER(_i32)]
_lib.moe_permute.restype = _i32
_lib.moe_permute.argtypes = [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                             _sz, _vp]
_lib.moe_permute_ex.restype = _i32
_lib.moe_permute_ex.argtypes = [_vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                _vp, _sz, _vp]
_lib.moe_expert_ffn.restype = _i32
_lib.moe_expert_ffn.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32, _vp, _vp,
                                _sz, _vp]
_lib.moe_expert_ffn_gather.restype = _i32
_lib.moe_expert_ffn_gather.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i32,
                                       _vp, _vp, _sz, _vp]
_lib.moe_combine.restype = _i32
_lib.moe_combine.argtypes = [_vp, _vp, _vp, _i64, _i64, _i32, _i32, _vp, _vp]
_lib.moe_forward.restype = _i32
_lib.moe_forward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _i32, _vp,
                             _vp, _vp, _vp, _sz, _vp]
_lib.moe_forward_ex.restype = _i32
_lib.moe_forward_ex.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _i32, _i32,
                                _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_forward_noalloc.restype = _i32
_lib.moe_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _i32,
                                     _vp, _vp, _vp, _vp]
_lib.moe_expert_ffn_backward.restype = _i32
_lib.moe_expert_ffn_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                         _i32, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_saved_bytes.restype = _i32
_lib.moe_saved_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64, _i32, ctypes.POINTER(_sz)]
_lib.moe_backward_workspace_bytes.restype = _i32
_lib.moe_backward_workspace_bytes.argtypes = [_i64, _i64, _i64, _i32, _i64, _i32,
                                              ctypes.POINTER(_sz)]
_lib.moe_forward_train.restype = _i32
_lib.moe_forward_train.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _i32,
                                   _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp, _sz, _vp]
_lib.moe_backward.restype = _i32
_lib.moe_backward.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i32, _i64, _i32, _i32,
                              _i32, _vp, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                              _vp]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {_lib.moe_status_string(status).decode()}")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library (for callers that pass raw pointers)."""
    return _lib


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return MOE_F32
    if t == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {t}: use torch.float32 or torch.bfloat16")


def _check(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ok(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def moe_workspace_bytes(T: int, H: int, E: int, top_k: int, F: int, dtype: torch.dtype) -> int:
    n = _sz(0)
    _ok(_lib.moe_workspace_bytes(T, H, E, top_k, F, _dtype_code(dtype), ctypes.byref(n)),
        "moe_workspace_bytes")
    return n.value


def moe_stage_workspace_bytes(stage: int, T: int, H: int, E: int, top_k: int, F: int,
                              dtype: torch.dtype) -> int:
    n = _sz(0)
    _ok(_lib.moe_stage_workspace_bytes(stage, T, H, E, top_k, F, _dtype_code(dtype),
                                       ctypes.byref(n)), "moe_stage_workspace_bytes")
    return n.value


def _workspace(ws, nbytes: int, dev):
    if ws is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(ws, "ws", torch.uint8)
    if ws.numel() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes} bytes")
    return ws


def moe_route(x, w_r, router_bias, top_k: int, topk_ids=None, topk_w=None, ws=None):
    """Routing + gating.  Returns (topk_ids[T,k] int32, topk_w[T,k] fp32)."""
    _check(x, "x")
    T, H = x.shape
    E = w_r.shape[1]
    _check(w_r, "w_r", x.dtype, (H, E))
    if router_bias is not None:
        _check(router_bias, "router_bias", torch.float32, (E,))
    dev = x.device
    topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if topk_ids is None else \
        _check(topk_ids, "topk_ids", torch.int32, (T, top_k))
    topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if topk_w is None else \
        _check(topk_w, "topk_w", torch.float32, (T, top_k))
    ws = _workspace(ws, moe_stage_workspace_bytes(MOE_STAGE_ROUTE, T, H, E, top_k, 8, x.dtype),
                    dev)
    _ok(_lib.moe_route(_ptr(x), _ptr(w_r), _ptr(router_bias), T, H, E, top_k,
                       _dtype_code(x.dtype), _ptr(topk_ids), _ptr(topk_w), _ptr(ws),
                       ws.numel(), _stream(dev)), "moe_route")
    return topk_ids, topk_w


def moe_route_ex(x, w_r, router_bias, top_k: int, gating: int = MOE_GATE_TOPK_SOFTMAX,
                 topk_ids=None, topk_w=None, ws=None):
    """Routing + gating with the variants: w_r may be fp32 for bf16 x (an fp32
    router), gating is MOE_GATE_TOPK_SOFTMAX or MOE_GATE_SOFTMAX_TOPK.
    Returns (topk_ids[T,k] int32, topk_w[T,k] fp32)."""
    _check(x, "x")
    T, H = x.shape
    E = w_r.shape[1]
    _check(w_r, "w_r", None, (H, E))
    if router_bias is not None:
        _check(router_bias, "router_bias", torch.float32, (E,))
    dev = x.device
    topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if topk_ids is None else \
        _check(topk_ids, "topk_ids", torch.int32, (T, top_k))
    topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if topk_w is None else \
        _check(topk_w, "topk_w", torch.float32, (T, top_k))
    ws = _workspace(ws, moe_stage_workspace_bytes(MOE_STAGE_ROUTE, T, H, E, top_k, 8, x.dtype),
                    dev)
    _ok(_lib.moe_route_ex(_ptr(x), _ptr(w_r), _ptr(router_bias), T, H, E, top_k,
                          _dtype_code(x.dtype), _dtype_code(w_r.dtype), gating, _ptr(topk_ids),
                          _ptr(topk_w), _ptr(ws), ws.numel(), _stream(dev)), "moe_route_ex")
    return topk_ids, topk_w


def moe_expert_capacity(T: int, top_k: int, E: int, factor_num: int, factor_den: int) -> int:
    """Rows each expert keeps: ceil(factor_num * T * top_k / (factor_den * E));
    0 (no limit) for factor_num <= 0."""
    c = _i32(0)
    _ok(_lib.moe_expert_capacity(T, top_k, E, factor_num, factor_den, ctypes.byref(c)),
        "moe_expert_capacity")
    return c.value


def moe_permute(x, topk_ids, E: int, expert_offsets=None, sorted_token=None, inv_pos=None,
                xp=None, ws=None, with_rows: bool = True):
    """Dispatch.  Returns (expert_offsets[E+1], sorted_token[R], inv_pos[R], xp[R,H]);
    with_rows=False builds the indices only (xp is None)."""
    _check(x, "x")
    T, H = x.shape
    top_k = topk_ids.shape[1]
    _check(topk_ids, "topk_ids", torch.int32, (T, top_k))
    R, dev = T * top_k, x.device
    expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if expert_offsets is None \
        else _check(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    sorted_token = torch.empty(R, dtype=torch.int32, device=dev) if sorted_token is None else \
        _check(sorted_token, "sorted_token", torch.int32, (R,))
    inv_pos = torch.empty(R, dtype=torch.int32, device=dev) if inv_pos is None else \
        _check(inv_pos, "inv_pos", torch.int32, (R,))
    if not with_rows:
        xp = None
    else:
        xp = torch.empty((R, H), dtype=x.dtype, device=dev) if xp is None else \
            _check(xp, "xp", x.dtype, (R, H))
    ws = _workspace(ws, moe_stage_workspace_bytes(MOE_STAGE_PERMUTE, T, H, E, top_k, 8, x.dtype),
                    dev)
    _ok(_lib.moe_permute(_ptr(x), _ptr(topk_ids), T, H, E, top_k, _dtype_code(x.dtype),
                         _ptr(expert_offsets), _ptr(sorted_token), _ptr(inv_pos), _ptr(xp),
                         _ptr(ws), ws.numel(), _stream(dev)), "moe_permute")
    return expert_offsets, sorted_token, inv_pos, xp


def moe_permute_ex(x, topk_ids, E: int, capacity: int, expert_offsets=None, sorted_token=None,
                   inv_pos=None, xp=None, ws=None, with_rows: bool = True):
    """Capacity-limited dispatch (capacity <= 0: dropless).  Returns
    (expert_offsets[E+1], sorted_token[R], inv_pos[R], xp[R,H]); dropped pairs
    have inv_pos -1 and only the first expert_offsets[E] rows are written;
    with_rows=False builds the indices only (xp is None)."""
    _check(x, "x")
    T, H = x.shape
    top_k = topk_ids.shape[1]
    _check(topk_ids, "topk_ids", torch.int32, (T, top_k))
    R, dev = T * top_k, x.device
    expert_offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if expert_offsets is None \
        else _check(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    sorted_token = torch.empty(R, dtype=torch.int32, device=dev) if sorted_token is None else \
        _check(sorted_token, "sorted_token", torch.int32, (R,))
    inv_pos = torch.empty(R, dtype=torch.int32, device=dev) if inv_pos is None else \
        _check(inv_pos, "inv_pos", torch.int32, (R,))
    if not with_rows:
        xp = None
    else:
        xp = torch.empty((R, H), dtype=x.dtype, device=dev) if xp is None else \
            _check(xp, "xp", x.dtype, (R, H))
    ws = _workspace(ws, moe_stage_workspace_bytes(MOE_STAGE_PERMUTE, T, H, E, top_k, 8, x.dtype),
                    dev)
    _ok(_lib.moe_permute_ex(_ptr(x), _ptr(topk_ids), T, H, E, top_k, _dtype_code(x.dtype),
                            capacity, _ptr(expert_offsets), _ptr(sorted_token), _ptr(inv_pos),
                            _ptr(xp), _ptr(ws), ws.numel(), _stream(dev)), "moe_permute_ex")
    return expert_offsets, sorted_token, inv_pos, xp


def moe_expert_ffn(xp, expert_offsets, w1, w2, yp=None, ws=None):
    """Experts.  Returns yp[R,H] with yp[rows_e] = GELU(xp[rows_e] W1[e]) W2[e]."""
    _check(xp, "xp")
    R, H = xp.shape
    E, _, F = w1.shape
    _check(w1, "w1", xp.dtype, (E, H, F))
    _check(w2, "w2", xp.dtype, (E, F, H))
    _check(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    dev = xp.device
    yp = torch.empty((R, H), dtype=xp.dtype, device=dev) if yp is None else \
        _check(yp, "yp", xp.dtype, (R, H))
    ws = _workspace(ws, moe_stage_workspace_bytes(MOE_STAGE_EXPERT_FFN, R, H, E, 1, F, xp.dtype),
                    dev)
    _ok(_lib.moe_expert_ffn(_ptr(xp), _ptr(expert_offsets), _ptr(w1), _ptr(w2), R, H, E, F,
                            _dtype_code(xp.dtype), _ptr(yp), _ptr(ws), ws.numel(),
                            _stream(dev)), "moe_expert_ffn")
    return yp


def moe_expert_ffn_gather(x, sorted_token, expert_offsets, w1, w2, yp=None, ws=None):
    """Experts over rows gathered from x: yp[p] = FFN_e(x[sorted_token[p]]) for
    the rows p of expert e (the expert stage as moe_forward runs it)."""
    _check(x, "x")
    T, H = x.shape
    E, _, F = w1.shape
    _check(sorted_token, "sorted_token", torch.int32)
    R = sorted_token.numel()
    _check(w1, "w1", x.dtype, (E, H, F))
    _check(w2, "w2", x.dtype, (E, F, H))
    _check(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    dev = x.device
    yp = torch.empty((R, H), dtype=x.dtype, device=dev) if yp is None else \
        _check(yp, "yp", x.dtype, (R, H))
    ws = _workspace(ws, moe_stage_workspace_bytes(MOE_STAGE_EXPERT_FFN_GATHER, R, H, E, 1, F,
                                                  x.dtype), dev)
    _ok(_lib.moe_expert_ffn_gather(_ptr(x), T, _ptr(sorted_token), _ptr(expert_offsets), _ptr(w1),
                                   _ptr(w2), R, H, E, F, _dtype_code(x.dtype), _ptr(yp),
                                   _ptr(ws), ws.numel(), _stream(dev)), "moe_expert_ffn_gather")
    return yp


def moe_combine(yp, inv_pos, topk_w, y=None):
    """Combine.  Returns y[T,H] = sum_j topk_w[t,j] * yp[inv_pos[t*k+j]]."""
    _check(yp, "yp")
    _check(topk_w, "topk_w", torch.float32)
    T, top_k = topk_w.shape
    H = yp.shape[1]
    _check(inv_pos, "inv_pos", torch.int32)
    if inv_pos.numel() != T * top_k or yp.shape[0] != T * top_k:
        raise ValueError("inv_pos / yp do not match topk_w's [T, k]")
    y = torch.empty((T, H), dtype=yp.dtype, device=yp.device) if y is None else \
        _check(y, "y", yp.dtype, (T, H))
    _ok(_lib.moe_combine(_ptr(yp), _ptr(inv_pos), _ptr(topk_w), T, H, top_k,
                         _dtype_code(yp.dtype), _ptr(y), _stream(yp.device)), "moe_combine")
    return y


def moe_forward(x, w_r, router_bias, w1, w2, top_k: int, y=None, topk_ids_out=None,
                topk_w_out=None, ws=None):
    """The whole layer forward.  Returns y[T,H]."""
    _check(x, "x")
    T, H = x.shape
    E = w_r.shape[1]
    F = w1.shape[2]
    _check(w_r, "w_r", x.dtype, (H, E))
    if router_bias is not None:
        _check(router_bias, "router_bias", torch.float32, (E,))
    _check(w1, "w1", x.dtype, (E, H, F))
    _check(w2, "w2", x.dtype, (E, F, H))
    dev = x.device
    y = torch.empty((T, H), dtype=x.dtype, device=dev) if y is None else \
        _check(y, "y", x.dtype, (T, H))
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", torch.int32, (T, top_k))
    if topk_w_out is not None:
        _check(topk_w_out, "topk_w_out", torch.float32, (T, top_k))
    ws = _workspace(ws, moe_workspace_bytes(T, H, E, top_k, F, x.dtype), dev)
    _ok(_lib.moe_forward(_ptr(x), _ptr(w_r), _ptr(router_bias), _ptr(w1), _ptr(w2), T, H, E,
                         top_k, F, _dtype_code(x.dtype), _ptr(y), _ptr(topk_ids_out),
                         _ptr(topk_w_out), _ptr(ws), ws.numel(), _stream(dev)), "moe_forward")
    return y


def moe_forward_ex(x, w_r, router_bias, w1, w2, top_k: int, gating: int = MOE_GATE_TOPK_SOFTMAX,
                   capacity: int = 0, y=None, topk_ids_out=None, topk_w_out=None, ws=None):
    """The layer forward with the variants: w_r may be fp32 for bf16 x, gating
    as in moe_route_ex, capacity as in moe_permute_ex.  Returns y[T,H]."""
    _check(x, "x")
    T, H = x.shape
    E = w_r.shape[1]
    F = w1.shape[2]
    _check(w_r, "w_r", None, (H, E))
    if router_bias is not None:
        _check(router_bias, "router_bias", torch.float32, (E,))
    _check(w1, "w1", x.dtype, (E, H, F))
    _check(w2, "w2", x.dtype, (E, F, H))
    dev = x.device
    y = torch.empty((T, H), dtype=x.dtype, device=dev) if y is None else \
        _check(y, "y", x.dtype, (T, H))
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", torch.int32, (T, top_k))
    if topk_w_out is not None:
        _check(topk_w_out, "topk_w_out", torch.float32, (T, top_k))
    ws = _workspace(ws, moe_workspace_bytes(T, H, E, top_k, F, x.dtype), dev)
    _ok(_lib.moe_forward_ex(_ptr(x), _ptr(w_r), _ptr(router_bias), _ptr(w1), _ptr(w2), T, H, E,
                            top_k, F, _dtype_code(x.dtype), _dtype_code(w_r.dtype), gating,
                            capacity, _ptr(y), _ptr(topk_ids_out), _ptr(topk_w_out), _ptr(ws),
                            ws.numel(), _stream(dev)), "moe_forward_ex")
    return y


def moe_forward_noalloc(x, w_r, router_bias, w1, w2, top_k: int, y, topk_ids_out=None,
                        topk_w_out=None):
    """The layer forward with the library's own fixed scratch as workspace (for
    callers that cannot allocate): y (preallocated, [T,H]) is filled and
    returned.  Layers whose workspace exceeds the scratch raise MoEError
    (MOE_ERR_UNSUPPORTED)."""
    _check(x, "x")
    T, H = x.shape
    E = w_r.shape[1]
    F = w1.shape[2]
    _check(w_r, "w_r", x.dtype, (H, E))
    if router_bias is not None:
        _check(router_bias, "router_bias", torch.float32, (E,))
    _check(w1, "w1", x.dtype, (E, H, F))
    _check(w2, "w2", x.dtype, (E, F, H))
    _check(y, "y", x.dtype, (T, H))
    if topk_ids_out is not None:
        _check(topk_ids_out, "topk_ids_out", torch.int32, (T, top_k))
    if topk_w_out is not None:
        _check(topk_w_out, "topk_w_out", torch.float32, (T, top_k))
    _ok(_lib.moe_forward_noalloc(_ptr(x), _ptr(w_r), _ptr(router_bias), _ptr(w1), _ptr(w2), T, H,
                                 E, top_k, F, _dtype_code(x.dtype), _ptr(y), _ptr(topk_ids_out),
                                 _ptr(topk_w_out), _stream(x.device)), "moe_forward_noalloc")
    return y


def moe_saved_bytes(T: int, H: int, E: int, top_k: int, F: int, dtype: torch.dtype) -> int:
    n = _sz(0)
    _ok(_lib.moe_saved_bytes(T, H, E, top_k, F, _dtype_code(dtype), ctypes.byref(n)),
        "moe_saved_bytes")
    return n.value


def moe_backward_workspace_bytes(T: int, H: int, E: int, top_k: int, F: int,
                                 dtype: torch.dtype) -> int:
    n = _sz(0)
    _ok(_lib.moe_backward_workspace_bytes(T, H, E, top_k, F, _dtype_code(dtype),
                                          ctypes.byref(n)), "moe_backward_workspace_bytes")
    return n.value


def moe_forward_train(x, w_r, router_bias, w1, w2, top_k: int,
                      gating: int = MOE_GATE_TOPK_SOFTMAX, capacity: int = 0, y=None,
                      topk_ids=None, topk_w=None, saved=None, ws=None):
    """moe_forward_ex that also keeps the state moe_backward needs.
    Returns (y, topk_ids, topk_w, saved)."""
    _check(x, "x")
    T, H = x.shape
    E = w_r.shape[1]
    F = w1.shape[2]
    _check(w_r, "w_r", None, (H, E))
    if router_bias is not None:
        _check(router_bias, "router_bias", torch.float32, (E,))
    _check(w1, "w1", x.dtype, (E, H, F))
    _check(w2, "w2", x.dtype, (E, F, H))
    dev = x.device
    y = torch.empty((T, H), dtype=x.dtype, device=dev) if y is None else \
        _check(y, "y", x.dtype, (T, H))
    topk_ids = torch.empty((T, top_k), dtype=torch.int32, device=dev) if topk_ids is None else \
        _check(topk_ids, "topk_ids", torch.int32, (T, top_k))
    topk_w = torch.empty((T, top_k), dtype=torch.float32, device=dev) if topk_w is None else \
        _check(topk_w, "topk_w", torch.float32, (T, top_k))
    saved = _workspace(saved, moe_saved_bytes(T, H, E, top_k, F, x.dtype), dev)
    ws = _workspace(ws, moe_workspace_bytes(T, H, E, top_k, F, x.dtype), dev)
    _ok(_lib.moe_forward_train(_ptr(x), _ptr(w_r), _ptr(router_bias), _ptr(w1), _ptr(w2), T, H,
                               E, top_k, F, _dtype_code(x.dtype), _dtype_code(w_r.dtype), gating,
                               capacity, _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(saved),
                               saved.numel(), _ptr(ws), ws.numel(), _stream(dev)),
        "moe_forward_train")
    return y, topk_ids, topk_w, saved


def moe_backward(dy, x, w_r, w1, w2, top_k: int, topk_ids, topk_w, saved,
                 gating: int = MOE_GATE_TOPK_SOFTMAX, with_bias_grad: bool = False, out=None,
                 ws=None):
    """Backward of the layer after moe_forward_train (same inputs and gating).
    Returns dict(dx, dw_r, db_r (None unless with_bias_grad), dw1, dw2, dw): dw is
    the gradient with respect to the gate weights.  `out` may hold preallocated
    tensors under those names."""
    _check(x, "x")
    T, H = x.shape
    E = w_r.shape[1]
    F = w1.shape[2]
    _check(dy, "dy", x.dtype, (T, H))
    _check(w_r, "w_r", None, (H, E))
    _check(w1, "w1", x.dtype, (E, H, F))
    _check(w2, "w2", x.dtype, (E, F, H))
    _check(topk_ids, "topk_ids", torch.int32, (T, top_k))
    _check(topk_w, "topk_w", torch.float32, (T, top_k))
    _check(saved, "saved", torch.uint8)
    dev = x.device
    out = dict(out or {})
    shapes = {"dx": ((T, H), x.dtype), "dw_r": ((H, E), w_r.dtype), "dw1": ((E, H, F), x.dtype),
              "dw2": ((E, F, H), x.dtype), "dw": ((T, top_k), torch.float32)}
    if with_bias_grad:
        shapes["db_r"] = ((E,), torch.float32)
    for name, (shape, dt) in shapes.items():
        if out.get(name) is None:
            out[name] = torch.empty(shape, dtype=dt, device=dev)
        else:
            _check(out[name], name, dt, shape)
    out.setdefault("db_r", None)
    ws = _workspace(ws, moe_backward_workspace_bytes(T, H, E, top_k, F, x.dtype), dev)
    _ok(_lib.moe_backward(_ptr(dy), _ptr(x), _ptr(w_r), _ptr(w1), _ptr(w2), T, H, E, top_k, F,
                          _dtype_code(x.dtype), _dtype_code(w_r.dtype), gating, _ptr(topk_ids),
                          _ptr(topk_w), _ptr(saved), saved.numel(), _ptr(out["dx"]),
                          _ptr(out["dw_r"]), _ptr(out["db_r"]), _ptr(out["dw1"]),
                          _ptr(out["dw2"]), _ptr(out["dw"]), _ptr(ws), ws.numel(),
                          _stream(dev)), "moe_backward")
    return out


def moe_expert_ffn_backward(dyp, xp, expert_offsets, z, h, w1, w2, dxp=None, dw1=None, dw2=None,
                            ws=None):
    """Backward of moe_expert_ffn over the dispatched rows.  Returns
    (dxp[R,H], dw1[E,H,F], dw2[E,F,H]); dxp may be dyp itself."""
    _check(xp, "xp")
    R, H = xp.shape
    E, _, F = w1.shape
    dt = xp.dtype
    _check(dyp, "dyp", dt, (R, H))
    _check(expert_offsets, "expert_offsets", torch.int32, (E + 1,))
    _check(z, "z", dt, (R, F))
    _check(h, "h", dt, (R, F))
    _check(w1, "w1", dt, (E, H, F))
    _check(w2, "w2", dt, (E, F, H))
    dev = xp.device
    dxp = torch.empty((R, H), dtype=dt, device=dev) if dxp is None else \
        _check(dxp, "dxp", dt, (R, H))
    dw1 = torch.empty((E, H, F), dtype=dt, device=dev) if dw1 is None else \
        _check(dw1, "dw1", dt, (E, H, F))
    dw2 = torch.empty((E, F, H), dtype=dt, device=dev) if dw2 is None else \
        _check(dw2, "dw2", dt, (E, F, H))
    ws = _workspace(ws, moe_stage_workspace_bytes(MOE_STAGE_EXPERT_FFN_BACKWARD, R, H, E, 1, F,
                                                  dt), dev)
    _ok(_lib.moe_expert_ffn_backward(_ptr(dyp), _ptr(xp), _ptr(expert_offsets), _ptr(z), _ptr(h),
                                     _ptr(w1), _ptr(w2), R, H, E, F, _dtype_code(dt), _ptr(dxp),
                                     _ptr(dw1), _ptr(dw2), _ptr(ws), ws.numel(), _stream(dev)),
        "moe_expert_ffn_backward")
    return dxp, dw1, dw2


class MoEFunction(torch.autograd.Function):
    """The layer as a differentiable torch operation: forward runs
    moe_forward_train (keeping its state for the backward) and backward runs
    moe_backward.  apply(x, w_r, router_bias, w1, w2, top_k, gating, capacity)
    returns y; gradients reach x, w_r, router_bias (when given), w1 and w2.
    The expert choice itself carries no gradient (the gate weights do)."""

    @staticmethod
    def forward(ctx, x, w_r, router_bias, w1, w2, top_k: int,
                gating: int = MOE_GATE_TOPK_SOFTMAX, capacity: int = 0):
        y, ids, w, saved = moe_forward_train(x, w_r, router_bias, w1, w2, top_k, gating,
                                             capacity)
        ctx.save_for_backward(x, w_r, w1, w2, ids, w, saved)
        ctx.top_k, ctx.gating, ctx.has_bias = top_k, gating, router_bias is not None
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_r, w1, w2, ids, w, saved = ctx.saved_tensors
        g = moe_backward(dy.contiguous(), x, w_r, w1, w2, ctx.top_k, ids, w, saved,
                         gating=ctx.gating, with_bias_grad=ctx.has_bias)
        return g["dx"], g["dw_r"], g["db_r"], g["dw1"], g["dw2"], None, None, None


class MoELayer(torch.nn.Module):
    """A Mixture-of-Experts layer with this library's kernels, forward and
    backward: y = sum over the top_k experts e of x of gate_e * GELU(x W1[e]) W2[e],
    routed by x W_r (+ bias).  Parameters: w_r [H,E], w1 [E,H,F], w2 [E,F,H]
    (dtype: torch.bfloat16 or torch.float32), bias [E] fp32 when bias=True;
    initialised N(0, 1/fan_in).  forward(x) takes [..., H] on the GPU."""

    def __init__(self, hidden: int, experts: int, ffn: int, top_k: int,
                 dtype: torch.dtype = torch.bfloat16, bias: bool = False,
                 gating: int = MOE_GATE_TOPK_SOFTMAX, capacity: int = 0, device="cuda"):
        super().__init__()
        self.top_k, self.gating, self.capacity = top_k, gating, capacity

        def init(shape, fan_in):
            return torch.nn.Parameter(
                (torch.randn(shape, device=device) / fan_in ** 0.5).to(dtype))

        self.w_r = init((hidden, experts), hidden)
        self.w1 = init((experts, hidden, ffn), hidden)
        self.w2 = init((experts, ffn, hidden), ffn)
        self.bias = torch.nn.Parameter(torch.zeros(experts, device=device)) if bias else None

    def forward(self, x):
        shape = x.shape
        y = MoEFunction.apply(x.reshape(-1, shape[-1]).contiguous(), self.w_r, self.bias,
                              self.w1, self.w2, self.top_k, self.gating, self.capacity)
        return y.reshape(shape)
