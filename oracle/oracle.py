"""ctypes wrapper of the C oracle (``oracle.c``) -- test infrastructure only.

Every function takes and returns CPU tensors / numpy arrays.  The C library computes the
local MoE forward pass of the ruDNN user guide (sections 3-6: route, dispatch, SwiGLU
experts, combine) in double precision with one rounding per stored tensor.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import build as _build

_DT_CODE = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}
_CODE_DT = {v: k for k, v in _DT_CODE.items()}

_lib = None


def lib() -> ctypes.CDLL:
    """The oracle library; ``ORACLE_LIB`` may name another build of ``oracle.c`` (the
    mutation tests load deliberately broken copies that way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("ORACLE_LIB")
        if not path:
            path = _build.LIB
            if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_build.SRC):
                _build.build()
        L = ctypes.CDLL(path)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_route.argtypes = [P, I32, I64, I64, I64, I32, P, P, P]
        L.oracle_dispatch.argtypes = [P, I64, I64, I64, P, I32, I64, P, P, P, P]
        L.oracle_expert_rows.argtypes = [P, I64, I32, P, P, P, I64, I64, I64, P, P, P]
        L.oracle_experts_forward.argtypes = [P, P, I64, I32, P, P, P, I64, I64, P, P]
        L.oracle_combine.argtypes = [P, I32, P, P, I32, I64, I64, I64, P]
        L.oracle_forward.argtypes = [P, I32, P, I32, I64, I64, I64, I32, P, P, P, I64, I64, P]
        L.oracle_project.argtypes = [P, I32, P, I64, I64, I64, P]
        L.oracle_route_projected.argtypes = [P, I32, P, I64, I64, I64, I64, I32, P, P, P]
        L.oracle_forward_projected.argtypes = [P, I32, P, I64, I64, I64, I32, P, P, P, I64, I64, P]
        D = ctypes.c_double
        L.oracle_route_sigmoid_grouped.argtypes = [P, I32, I64, I64, P, I64, I64, I64, I32, I32, D, P, P, P]
        L.oracle_forward_sigmoid_grouped.argtypes = [P, I32, P, I32, I64, I64, P, I64, I64, I64, I32, I32, D,
                                                     P, P, P, I64, I64, P]
        L.oracle_selected_router_weights.argtypes = [P, I32, I64, I64, P, I64, I32, I32, D, P, P]
        L.oracle_selected_router_backward.argtypes = [P, I32, I64, I64, P, I64, I32, I32, D, P, P]
        L.oracle_combine_backward.argtypes = [P, I32, P, P, I32, P, I64, I64, I64, I64, P, P]
        L.oracle_dispatch_backward.argtypes = [P, I32, P, I64, I64, I64, I64, P]
        L.oracle_experts_backward.argtypes = [P, P, I64, I32, P, P, P, I64, I64, P, P, P, P, P]
        L.oracle_decode.argtypes = [P, I32, I64, P]
        L.oracle_encode.argtypes = [P, I32, I64, P]
        L.oracle_set_num_threads.argtypes = [I32]
        for f in ("oracle_route", "oracle_dispatch", "oracle_expert_rows", "oracle_experts_forward",
                  "oracle_combine", "oracle_forward", "oracle_num_threads", "oracle_route_sigmoid_grouped",
                  "oracle_forward_sigmoid_grouped", "oracle_project", "oracle_route_projected",
                  "oracle_forward_projected", "oracle_selected_router_weights", "oracle_selected_router_backward",
                  "oracle_combine_backward", "oracle_dispatch_backward", "oracle_experts_backward"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _cpu(t: torch.Tensor) -> torch.Tensor:
    if t.device.type != "cpu":
        t = t.cpu()
    return t.contiguous()


def _p(x) -> int:
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return x.ctypes.data


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(n)


def decode(t: torch.Tensor) -> np.ndarray:
    """Exact widening of an f32/f16/bf16 tensor to float64 by the oracle's own codec."""
    t = _cpu(t)
    out = np.empty(t.numel(), np.float64)
    lib().oracle_decode(_p(t), _DT_CODE[t.dtype], t.numel(), _p(out))
    return out.reshape(tuple(t.shape))


def encode(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """One round-to-nearest-even of float64 values to ``dtype`` by the oracle's own codec."""
    a = np.ascontiguousarray(a, dtype=np.float64)
    out = torch.empty(a.shape, dtype=dtype)
    lib().oracle_encode(_p(a), _DT_CODE[dtype], a.size, _p(out))
    return out


def route(logits: torch.Tensor, top_k: int, renormalize: bool):
    """Returns ``(indices uint32 [T,k], weights [T,k] in the logits dtype, exact float64 weights)``."""
    logits = _cpu(logits)
    T, E = logits.shape
    idx = np.empty((T, top_k), np.uint32)
    w = torch.empty(T, top_k, dtype=logits.dtype)
    wx = np.empty((T, top_k), np.float64)
    rc = lib().oracle_route(_p(logits), _DT_CODE[logits.dtype], T, E, top_k, int(bool(renormalize)),
                            _p(idx), _p(w), _p(wx))
    if rc:
        raise ValueError("oracle_route: bad arguments")
    return idx, w, wx


def dispatch(indices: np.ndarray, x: torch.Tensor, E: int, copy_rows: bool = True):
    """Returns ``(dispatched [T*k,H] or None, offsets int32 [E+1], token_map int32 [T,k], counts int32 [E])``."""
    indices = np.ascontiguousarray(indices, dtype=np.uint32)
    x = _cpu(x)
    T, k = indices.shape
    H = x.shape[1]
    disp = torch.empty(T * k, H, dtype=x.dtype) if copy_rows else None
    offs = np.empty(E + 1, np.int32)
    tmap = np.empty((T, k), np.int32)
    counts = np.empty(E, np.int32)
    rc = lib().oracle_dispatch(_p(indices), T, k, E, _p(x), _DT_CODE[x.dtype], H, _p(disp), _p(offs),
                               _p(tmap), _p(counts))
    if rc:
        raise ValueError("oracle_dispatch: bad arguments")
    return disp, offs, tmap, counts


def expert_rows(x: torch.Tensor, experts_of_rows, gate, up, down, want_hidden: bool = False):
    """Row r of ``x`` through expert ``experts_of_rows[r]``; returns ``y`` (and ``h``)."""
    x = _cpu(x)
    gate, up, down = _cpu(gate), _cpu(up), _cpu(down)
    E, I, H = gate.shape
    eor = np.ascontiguousarray(experts_of_rows, dtype=np.int32)
    n = x.shape[0]
    y = torch.empty(n, H, dtype=x.dtype)
    h = torch.empty(n, I, dtype=x.dtype) if want_hidden else None
    rc = lib().oracle_expert_rows(_p(x), n, _DT_CODE[x.dtype], _p(gate), _p(up), _p(down), E, H, I,
                                  _p(eor), _p(y), _p(h))
    if rc:
        raise ValueError("oracle_expert_rows: bad arguments")
    return (y, h) if want_hidden else y


def experts_forward(dispatched: torch.Tensor, offsets: np.ndarray, gate, up, down, want_hidden=False):
    dispatched = _cpu(dispatched)
    gate, up, down = _cpu(gate), _cpu(up), _cpu(down)
    E, I, H = gate.shape
    offsets = np.ascontiguousarray(offsets, dtype=np.int32)
    y = torch.zeros_like(dispatched)
    h = torch.zeros(dispatched.shape[0], I, dtype=dispatched.dtype) if want_hidden else None
    rc = lib().oracle_experts_forward(_p(dispatched), _p(offsets), E, _DT_CODE[dispatched.dtype], _p(gate),
                                      _p(up), _p(down), H, I, _p(y), _p(h))
    if rc:
        raise ValueError("oracle_experts_forward: bad arguments")
    return (y, h) if want_hidden else y


def combine(expert_output: torch.Tensor, token_map: np.ndarray, weights: torch.Tensor):
    expert_output = _cpu(expert_output)
    weights = _cpu(weights)
    token_map = np.ascontiguousarray(token_map, dtype=np.int32)
    T, k = token_map.shape
    H = expert_output.shape[1]
    out = torch.empty(T, H, dtype=expert_output.dtype)
    rc = lib().oracle_combine(_p(expert_output), _DT_CODE[expert_output.dtype], _p(token_map), _p(weights),
                              _DT_CODE[weights.dtype], T, k, H, _p(out))
    if rc:
        raise ValueError("oracle_combine: bad arguments")
    return out


def forward(x: torch.Tensor, logits: torch.Tensor, top_k: int, renormalize: bool,
            gate=None, up=None, down=None):
    """The full local forward; ``gate=None`` means identity experts."""
    x, logits = _cpu(x), _cpu(logits)
    T, H = x.shape
    E = logits.shape[1]
    I = 0
    if gate is not None:
        gate, up, down = _cpu(gate), _cpu(up), _cpu(down)
        I = gate.shape[1]
    out = torch.empty(T, H, dtype=x.dtype)
    rc = lib().oracle_forward(_p(x), _DT_CODE[x.dtype], _p(logits), _DT_CODE[logits.dtype], T, E, top_k,
                              int(bool(renormalize)), _p(gate), _p(up), _p(down), H, I, _p(out))
    if rc:
        raise ValueError("oracle_forward: bad arguments")
    return out


def _bias(bias):
    if bias is None:
        return None
    b = _cpu(bias)
    if b.dtype != torch.float32:
        raise TypeError("the correction bias is FP32")
    return b


def route_sigmoid_grouped(logits: torch.Tensor, bias, top_k: int, groups: int, selected_groups: int,
                          top_two: bool, renormalize: bool, scale: float):
    """Group-limited sigmoid routing (user guide section 10).  Returns ``(indices uint32 [T,k],
    weights [T,k] in the logits dtype, exact float64 weights)``."""
    logits = _cpu(logits)
    b = _bias(bias)
    T, E = logits.shape
    idx = np.empty((T, top_k), np.uint32)
    w = torch.empty(T, top_k, dtype=logits.dtype)
    wx = np.empty((T, top_k), np.float64)
    rc = lib().oracle_route_sigmoid_grouped(_p(logits), _DT_CODE[logits.dtype], T, E, _p(b), top_k, groups,
                                            selected_groups, int(bool(top_two)), int(bool(renormalize)),
                                            float(scale), _p(idx), _p(w), _p(wx))
    if rc:
        raise ValueError("oracle_route_sigmoid_grouped: bad arguments")
    return idx, w, wx


def forward_sigmoid_grouped(x: torch.Tensor, logits: torch.Tensor, bias, top_k: int, groups: int,
                            selected_groups: int, top_two: bool, renormalize: bool, scale: float,
                            gate=None, up=None, down=None):
    """The full local forward with group-limited sigmoid routing; ``gate=None`` means identity experts."""
    x, logits = _cpu(x), _cpu(logits)
    b = _bias(bias)
    T, H = x.shape
    E = logits.shape[1]
    I = 0
    if gate is not None:
        gate, up, down = _cpu(gate), _cpu(up), _cpu(down)
        I = gate.shape[1]
    out = torch.empty(T, H, dtype=x.dtype)
    rc = lib().oracle_forward_sigmoid_grouped(_p(x), _DT_CODE[x.dtype], _p(logits), _DT_CODE[logits.dtype], T, E,
                                              _p(b), top_k, groups, selected_groups, int(bool(top_two)),
                                              int(bool(renormalize)), float(scale), _p(gate), _p(up), _p(down),
                                              H, I, _p(out))
    if rc:
        raise ValueError("oracle_forward_sigmoid_grouped: bad arguments")
    return out


def project(x: torch.Tensor, router: torch.Tensor) -> torch.Tensor:
    """logits [T, E] = x [T, H] . router [E, H]^T, summed in double, rounded once to x's dtype."""
    x, router = _cpu(x), _cpu(router)
    T, H = x.shape
    E = router.shape[0]
    if router.dtype != x.dtype or router.shape[1] != H:
        raise ValueError("router must be [E, H] in the token dtype")
    out = torch.empty(T, E, dtype=x.dtype)
    if lib().oracle_project(_p(x), _DT_CODE[x.dtype], _p(router), T, H, E, _p(out)):
        raise ValueError("oracle_project: bad arguments")
    return out


def route_projected(x: torch.Tensor, router: torch.Tensor, top_k: int, renormalize: bool):
    """Router projection then section 4 routing.  Returns ``(indices uint32 [T,k], weights [T,k],
    logits [T,E])`` (weights and logits in the token dtype)."""
    x, router = _cpu(x), _cpu(router)
    T, H = x.shape
    E = router.shape[0]
    idx = np.empty((T, top_k), np.uint32)
    w = torch.empty(T, top_k, dtype=x.dtype)
    lg = torch.empty(T, E, dtype=x.dtype)
    if lib().oracle_route_projected(_p(x), _DT_CODE[x.dtype], _p(router), T, H, E, top_k, int(bool(renormalize)),
                                    _p(idx), _p(w), _p(lg)):
        raise ValueError("oracle_route_projected: bad arguments")
    return idx, w, lg


def forward_projected(x: torch.Tensor, router: torch.Tensor, top_k: int, renormalize: bool, gate=None, up=None,
                      down=None):
    """The full local forward from hidden states: projection, route, dispatch, experts, combine."""
    x, router = _cpu(x), _cpu(router)
    T, H = x.shape
    E = router.shape[0]
    I = 0
    if gate is not None:
        gate, up, down = _cpu(gate), _cpu(up), _cpu(down)
        I = gate.shape[1]
    out = torch.empty(T, H, dtype=x.dtype)
    if lib().oracle_forward_projected(_p(x), _DT_CODE[x.dtype], _p(router), T, E, top_k, int(bool(renormalize)),
                                      _p(gate), _p(up), _p(down), H, I, _p(out)):
        raise ValueError("oracle_forward_projected: bad arguments")
    return out


# ---------------------------------------------------------------------------------------------
# First-order training (user guide section 12)
# ---------------------------------------------------------------------------------------------

SCORING = {"softmax": 0, "sigmoid": 1}


def _idx64(indices) -> np.ndarray:
    a = indices.cpu().numpy() if isinstance(indices, torch.Tensor) else np.asarray(indices)
    return np.ascontiguousarray(a.astype(np.int64))


def selected_router_weights(logits: torch.Tensor, indices, scoring: str, renormalize: bool, scale: float):
    """FP32 weights [T,k] of the fixed selection ``indices`` (any integer type; outside [0, E) =
    invalid row) and their double values."""
    logits = _cpu(logits)
    T, E = logits.shape
    ix = _idx64(indices)
    k = ix.shape[1]
    w = np.empty((T, k), np.float32)
    wx = np.empty((T, k), np.float64)
    if lib().oracle_selected_router_weights(_p(logits), _DT_CODE[logits.dtype], T, E, _p(ix), k, SCORING[scoring],
                                            int(bool(renormalize)), float(scale), _p(w), _p(wx)):
        raise ValueError("oracle_selected_router_weights: bad arguments")
    return torch.from_numpy(w), wx


def selected_router_backward(logits: torch.Tensor, indices, grad_weights, scoring: str, renormalize: bool,
                             scale: float) -> torch.Tensor:
    """Logits gradient [T,E] in the logits dtype."""
    logits = _cpu(logits)
    T, E = logits.shape
    ix = _idx64(indices)
    k = ix.shape[1]
    g = np.ascontiguousarray(np.asarray(grad_weights.cpu() if isinstance(grad_weights, torch.Tensor) else grad_weights,
                                        dtype=np.float32))
    out = torch.empty(T, E, dtype=logits.dtype)
    if lib().oracle_selected_router_backward(_p(logits), _DT_CODE[logits.dtype], T, E, _p(ix), k, SCORING[scoring],
                                             int(bool(renormalize)), float(scale), _p(g), _p(out)):
        raise ValueError("oracle_selected_router_backward: bad arguments")
    return out


def combine_backward(expert_output: torch.Tensor, token_map, weights: torch.Tensor, grad_output: torch.Tensor,
                     grad_expert: torch.Tensor | None = None):
    """Returns ``(dexpert [rows,H] (rows not named by a valid map entry keep grad_expert's
    values, zeros by default), dweights [T,k] FP32)``."""
    y, w, go = _cpu(expert_output), _cpu(weights), _cpu(grad_output)
    tm = np.ascontiguousarray(np.asarray(token_map.cpu() if isinstance(token_map, torch.Tensor) else token_map,
                                         dtype=np.int32))
    T, k = tm.shape
    rows, H = y.shape
    dexp = torch.zeros(rows, H, dtype=y.dtype) if grad_expert is None else grad_expert.cpu().clone()
    dw = np.empty((T, k), np.float32)
    if lib().oracle_combine_backward(_p(y), _DT_CODE[y.dtype], _p(tm), _p(w), _DT_CODE[w.dtype], _p(go), T, k, H,
                                     rows, _p(dexp), _p(dw)):
        raise ValueError("oracle_combine_backward: bad arguments")
    return dexp, torch.from_numpy(dw)


def dispatch_backward(grad_dispatched: torch.Tensor, token_map) -> torch.Tensor:
    d = _cpu(grad_dispatched)
    tm = np.ascontiguousarray(np.asarray(token_map.cpu() if isinstance(token_map, torch.Tensor) else token_map,
                                         dtype=np.int32))
    T, k = tm.shape
    rows, H = d.shape
    out = torch.empty(T, H, dtype=d.dtype)
    if lib().oracle_dispatch_backward(_p(d), _DT_CODE[d.dtype], _p(tm), T, k, H, rows, _p(out)):
        raise ValueError("oracle_dispatch_backward: bad arguments")
    return out


def experts_backward(dispatched: torch.Tensor, offsets, gate, up, down, grad_expert_output: torch.Tensor):
    """Returns ``(grad_dispatched [rows,H] dtype, dgate [E,I,H], dup [E,I,H], ddown [E,H,I] FP32)``;
    rows outside [offsets[0], offsets[E]) of grad_dispatched are zero."""
    x, dy = _cpu(dispatched), _cpu(grad_expert_output)
    gate, up, down = _cpu(gate), _cpu(up), _cpu(down)
    E, I, H = gate.shape
    offs = np.ascontiguousarray(np.asarray(offsets.cpu() if isinstance(offsets, torch.Tensor) else offsets,
                                           dtype=np.int32))
    dx = torch.zeros(x.shape[0], H, dtype=x.dtype)
    dg = torch.empty(E, I, H, dtype=torch.float32)
    du = torch.empty(E, I, H, dtype=torch.float32)
    dd = torch.empty(E, H, I, dtype=torch.float32)
    if lib().oracle_experts_backward(_p(x), _p(offs), E, _DT_CODE[x.dtype], _p(gate), _p(up), _p(down), H, I, _p(dy),
                                     _p(dx), _p(dg), _p(du), _p(dd)):
        raise ValueError("oracle_experts_backward: bad arguments")
    return dx, dg, du, dd
