"""Thin ctypes binding of ``librudnn_moe.so`` (C ABI: include/rudnn_moe.h).

Argument marshalling only: every step of the MoE path runs in the library's HIP kernels, on
torch's current stream of the tensors' device.  Output and workspace buffers are allocated
with torch (PyTorch is plumbing here: device memory and streams).  There is no fallback: if
the library is missing, or a call returns an error status, this module raises.

The functions follow the ruDNN user guide's MoE API (sections 3-6): ``route``,
``dispatch``, ``experts_forward`` (``SwiGluExperts.forward_dispatched``), ``combine`` and
``forward`` (``SwiGluExperts.forward``); group-limited sigmoid routing of section 10
(``route_sigmoid_grouped``, ``forward_sigmoid_grouped``); and the gate projection that the
guide leaves to the caller, fused with the routing (``route_projected``, ``forward_projected``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librudnn_moe.so")

_DT = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

STATUS = {0: "ok", 1: "shape", 2: "dtype", 3: "argument", 4: "device", 5: "unsupported", 6: "workspace",
          7: "runtime"}

KERNELS = ("route", "dispatch_count", "dispatch_scan", "dispatch_rank", "dispatch_copy", "experts_plan",
           "experts_gate_up", "experts_down", "combine", "experts_gate_up_reduce", "experts_down_reduce",
           "route_sigmoid_grouped", "route_projected", "route_projected_reduce", "selected_router", "combine_backward",
           "dispatch_backward", "experts_backward_plan", "experts_backward_gu", "experts_backward_dh",
           "experts_backward_dx", "experts_backward_dw")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _lib.rudnn_moe_status_string(status).decode() if _lib is not None else STATUS.get(status, "?")
        super().__init__(f"{fn}: {msg} (status {status})")


class RoutingOptions(ctypes.Structure):
    _fields_ = [("top_k", ctypes.c_int64), ("renormalize", ctypes.c_int32)]


class GroupRoutingOptions(ctypes.Structure):
    """GroupRoutingOptions of user guide section 10 (group-limited sigmoid routing)."""
    _fields_ = [("top_k", ctypes.c_int64), ("groups", ctypes.c_int64), ("selected_groups", ctypes.c_int64),
                ("group_top_two", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("scale", ctypes.c_double)]


class RouterWeightOptions(ctypes.Structure):
    """RouterWeightOptions of user guide section 12: scoring 0 = softmax, 1 = sigmoid."""
    _fields_ = [("scoring", ctypes.c_int32), ("renormalize", ctypes.c_int32), ("scale", ctypes.c_double)]




class ExpertsView(ctypes.Structure):
    _fields_ = [("gate", ctypes.c_void_p), ("up", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("num_experts", ctypes.c_int64), ("hidden", ctypes.c_int64), ("intermediate", ctypes.c_int64),
                ("dtype", ctypes.c_int)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        # torch was imported first, so the library binds to torch's HIP runtime (same soname);
        # a second runtime in the process would not know torch's streams and allocations.
        runtimes = _loaded_hip_runtimes()
        if len(runtimes) > 1:
            raise RuntimeError(f"more than one HIP runtime loaded: {runtimes}")
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        EXP = ctypes.POINTER(ExpertsView)
        L.rudnn_moe_route.argtypes = [P, I32, I64, I64, RoutingOptions, P, P, P]
        L.rudnn_moe_dispatch_workspace_size.argtypes = [I64, I64, I64]
        L.rudnn_moe_dispatch_workspace_size.restype = SZ
        L.rudnn_moe_dispatch.argtypes = [P, I64, I64, I64, P, I32, I64, P, P, P, P, SZ, P]
        L.rudnn_moe_dispatch_no_alloc.argtypes = [P, I64, I64, I64, P, I32, I64, P, P, P, P]
        L.rudnn_moe_route_dispatch.argtypes = [P, I32, I64, I64, RoutingOptions, P, I32, I64, P, P, P, P, P, P, SZ, P]
        L.rudnn_moe_experts_workspace_size.argtypes = [EXP, I64]
        L.rudnn_moe_experts_workspace_size.restype = SZ
        L.rudnn_moe_experts_forward.argtypes = [EXP, P, P, I64, P, P, SZ, P]
        L.rudnn_moe_experts_forward_training.argtypes = [EXP, P, P, I64, P, P, P, SZ, P]
        L.rudnn_moe_combine.argtypes = [P, I32, P, P, I32, I64, I64, I64, P, P]
        L.rudnn_moe_forward_workspace_size.argtypes = [EXP, I64, I64, I32]
        L.rudnn_moe_forward_workspace_size.restype = SZ
        L.rudnn_moe_forward.argtypes = [EXP, P, P, I32, I64, RoutingOptions, P, P, SZ, P]
        L.rudnn_moe_route_sigmoid_grouped.argtypes = [P, I32, I64, I64, P, GroupRoutingOptions, P, P, P]
        L.rudnn_moe_forward_sigmoid_grouped.argtypes = [EXP, P, P, I32, I64, P, GroupRoutingOptions, P, P, SZ, P]
        L.rudnn_moe_route_projected_workspace_size.argtypes = [I64, I64, I64, I32]
        L.rudnn_moe_route_projected_workspace_size.restype = SZ
        L.rudnn_moe_route_projected.argtypes = [P, I32, P, I64, I64, I64, RoutingOptions, P, P, P, P, SZ, P]
        L.rudnn_moe_forward_projected_workspace_size.argtypes = [EXP, I64, I64]
        L.rudnn_moe_forward_projected_workspace_size.restype = SZ
        L.rudnn_moe_forward_projected.argtypes = [EXP, P, P, I64, RoutingOptions, P, P, SZ, P]
        L.rudnn_moe_selected_router_weights.argtypes = [P, I32, I64, I64, P, I32, I64, RouterWeightOptions, P, P]
        L.rudnn_moe_selected_router_backward.argtypes = [P, I32, I64, I64, P, I32, I64, RouterWeightOptions, P, P, P]
        L.rudnn_moe_combine_backward.argtypes = [P, I32, P, P, I32, P, I64, I64, I64, P, P, P]
        L.rudnn_moe_dispatch_backward.argtypes = [P, I32, P, I64, I64, I64, P, P]
        L.rudnn_moe_experts_backward_workspace_size.argtypes = [EXP, I64, I32]
        L.rudnn_moe_experts_backward_workspace_size.restype = SZ
        L.rudnn_moe_experts_backward.argtypes = [EXP, P, P, I64, P, P, P, P, P, P, P, SZ, P]
        L.rudnn_moe_status_string.argtypes = [I32]
        L.rudnn_moe_status_string.restype = ctypes.c_char_p
        L.rudnn_moe_time_next_launch.argtypes = [I32, P, P]
        for f in ("rudnn_moe_route", "rudnn_moe_dispatch", "rudnn_moe_experts_forward", "rudnn_moe_combine",
                  "rudnn_moe_forward", "rudnn_moe_time_next_launch", "rudnn_moe_route_sigmoid_grouped",
                  "rudnn_moe_forward_sigmoid_grouped", "rudnn_moe_route_projected", "rudnn_moe_forward_projected",
                  "rudnn_moe_selected_router_weights", "rudnn_moe_selected_router_backward",
                  "rudnn_moe_combine_backward", "rudnn_moe_dispatch_backward", "rudnn_moe_experts_backward",
                  "rudnn_moe_experts_forward_training"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _loaded_hip_runtimes():
    import re
    try:
        maps = open("/proc/self/maps").read()
    except OSError:
        return []
    return sorted({os.path.realpath(p) for p in re.findall(r"(/\S*libamdhip64\.so\S*)", maps)})


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise MoeError(fn, status)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor):
    if t.device.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    return torch.cuda.current_stream(t.device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _contig(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def time_next_launch(kernel: str, before: int, after: int) -> None:
    """Record the raw ``hipEvent_t`` handles ``before``/``after`` on the launch stream around the
    next launch of ``kernel`` by this host thread (measurement only)."""
    _check("rudnn_moe_time_next_launch", lib().rudnn_moe_time_next_launch(KERNELS.index(kernel), before, after))


class SwiGluExperts:
    """Bias-free SwiGLU expert weights: gate/up [E, I, H], down [E, H, I], one dtype and device
    (user guide section 5).  Reusable across batches (section 6)."""

    def __init__(self, gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor):
        if gate.dim() != 3 or up.shape != gate.shape or down.dim() != 3:
            raise ValueError("gate and up must be [E, I, H] and down [E, H, I]")
        E, I, H = gate.shape
        if tuple(down.shape) != (E, H, I):
            raise ValueError("down must be [E, H, I]")
        if not (gate.dtype == up.dtype == down.dtype) or not (gate.device == up.device == down.device):
            raise ValueError("gate, up and down must share dtype and device")
        self.gate, self.up, self.down = (_contig(t, n) for t, n in ((gate, "gate"), (up, "up"), (down, "down")))
        self.E, self.I, self.H = E, I, H
        self.view = ExpertsView(gate.data_ptr(), up.data_ptr(), down.data_ptr(), E, H, I, _dt(gate))

    @property
    def dtype(self):
        return self.gate.dtype

    @property
    def device(self):
        return self.gate.device

    def forward(self, input: torch.Tensor, logits: torch.Tensor, top_k: int, renormalize: bool, out=None,
                workspace=None) -> torch.Tensor:
        return forward(self, input, logits, top_k, renormalize, out=out, workspace=workspace)

    def forward_sigmoid_grouped(self, input: torch.Tensor, logits: torch.Tensor, bias, options: GroupRoutingOptions,
                                out=None, workspace=None) -> torch.Tensor:
        return forward_sigmoid_grouped(self, input, logits, bias, options, out=out, workspace=workspace)

    def forward_projected(self, input: torch.Tensor, router: torch.Tensor, top_k: int, renormalize: bool, out=None,
                          workspace=None) -> torch.Tensor:
        return forward_projected(self, input, router, top_k, renormalize, out=out, workspace=workspace)

    def forward_dispatched(self, d: "Dispatched", out=None, workspace=None) -> torch.Tensor:
        return experts_forward(self, d.dispatched, d.expert_offsets, out=out, workspace=workspace)

    def backward_dispatched(self, d: "Dispatched", grad_expert_output: torch.Tensor, workspace=None):
        """Backward of forward_dispatched (user guide section 12, step 2): ``(grad_dispatched,
        dgate, dup, ddown)``, the weight gradients FP32; the gate and up products are recomputed."""
        return experts_backward(self, d.dispatched, d.expert_offsets, grad_expert_output, workspace=workspace)

    def forward_dispatched_training(self, d: "Dispatched", out=None, workspace=None):
        """User guide section 12: ``(output, cache)``; ``cache.backward(dexpert)`` gives
        ``(grad_dispatched, dgate, dup, ddown)``.  The dispatched rows must stay unchanged until then."""
        out, pre = experts_forward_training(self, d.dispatched, d.expert_offsets, out=out, workspace=workspace)
        return out, ExpertsCache(self, d.dispatched, d.expert_offsets, pre)


class ExpertsCache:
    """What the experts backward reads: the forward's dispatched rows and offsets and the FP32
    pre-activations [gate . x | up . x] [rows, 2I] it stored."""

    def __init__(self, experts: SwiGluExperts, dispatched: torch.Tensor, expert_offsets: torch.Tensor,
                 preactivations: torch.Tensor):
        self.experts, self.dispatched, self.expert_offsets = experts, dispatched, expert_offsets
        self.preactivations = preactivations

    def backward(self, grad_expert_output: torch.Tensor, workspace=None):
        return experts_backward(self.experts, self.dispatched, self.expert_offsets, grad_expert_output,
                                cache=self.preactivations, workspace=workspace)


def route(logits: torch.Tensor, top_k: int, renormalize: bool):
    """Returns ``(expert_indices [T, k] int32 holding the uint32 ids, weights [T, k] logits dtype)``."""
    logits = _contig(logits, "logits")
    T, E = logits.shape
    idx = torch.empty(T, top_k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, top_k, dtype=logits.dtype, device=logits.device)
    _check("rudnn_moe_route", lib().rudnn_moe_route(_ptr(logits), _dt(logits), T, E, RoutingOptions(top_k, int(renormalize)),
                                                    _ptr(idx), _ptr(w), _stream(logits)))
    return idx, w


def _bias(bias, logits: torch.Tensor):
    if bias is None:
        return None
    bias = _contig(bias, "bias")
    if bias.dtype != torch.float32 or bias.shape != (logits.shape[1],) or bias.device != logits.device:
        raise ValueError("the correction bias is FP32 [E] on the logits' device")
    return bias


def route_sigmoid_grouped(logits: torch.Tensor, bias, options: GroupRoutingOptions):
    """Group-limited sigmoid routing (user guide section 10).  ``bias``: FP32 [E] or None.
    Returns ``(expert_indices [T, k] int32 holding the uint32 ids, weights [T, k] logits dtype)``."""
    logits = _contig(logits, "logits")
    bias = _bias(bias, logits)
    T, E = logits.shape
    k = options.top_k
    idx = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, k, dtype=logits.dtype, device=logits.device)
    _check("rudnn_moe_route_sigmoid_grouped", lib().rudnn_moe_route_sigmoid_grouped(
        _ptr(logits), _dt(logits), T, E, _ptr(bias), options, _ptr(idx), _ptr(w), _stream(logits)))
    return idx, w


def route_projected_workspace_size(T: int, H: int, E: int, dtype: torch.dtype) -> int:
    return lib().rudnn_moe_route_projected_workspace_size(T, H, E, _DT[dtype])


def route_projected(input: torch.Tensor, router: torch.Tensor, top_k: int, renormalize: bool,
                    logits_out: bool = False, workspace=None):
    """Gate projection ``input [T, H] x router [E, H]^T`` fused with softmax routing.  Returns
    ``(expert_indices [T, k] int32 holding the uint32 ids, weights [T, k], logits [T, E] or None)``,
    all in the input dtype; the logits are the rounded values that were routed."""
    input = _contig(input, "input")
    router = _contig(router, "router")
    T, H = input.shape
    if router.dim() != 2 or router.shape[1] != H or router.dtype != input.dtype or router.device != input.device:
        raise ValueError("router must be [E, H] in the input's dtype, on its device")
    E = router.shape[0]
    dev = input.device
    idx = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, top_k, dtype=input.dtype, device=dev)
    lo = torch.empty(T, E, dtype=input.dtype, device=dev) if logits_out else None
    need = route_projected_workspace_size(T, H, E, input.dtype)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _check("rudnn_moe_route_projected", lib().rudnn_moe_route_projected(
        _ptr(input), _dt(input), _ptr(router), T, H, E, RoutingOptions(top_k, int(renormalize)), _ptr(lo), _ptr(idx),
        _ptr(w), _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream(input)))
    return idx, w, lo


@dataclass
class Dispatched:
    dispatched: torch.Tensor      # [T*k, H]
    expert_offsets: torch.Tensor  # [E+1] int32
    token_map: torch.Tensor       # [T, k] int32


def dispatch(expert_indices: torch.Tensor, input: torch.Tensor, num_experts: int, out: Dispatched | None = None,
             workspace=None) -> Dispatched:
    expert_indices = _contig(expert_indices, "expert_indices")
    input = _contig(input, "input")
    T, k = expert_indices.shape
    H = input.shape[1]
    dev = input.device
    if out is None:
        out = Dispatched(torch.empty(T * k, H, dtype=input.dtype, device=dev),
                         torch.empty(num_experts + 1, dtype=torch.int32, device=dev),
                         torch.empty(T, k, dtype=torch.int32, device=dev))
    need = lib().rudnn_moe_dispatch_workspace_size(T, k, num_experts)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("rudnn_moe_dispatch", lib().rudnn_moe_dispatch(
        _ptr(expert_indices), T, k, num_experts, _ptr(input), _dt(input), H, _ptr(out.dispatched),
        _ptr(out.expert_offsets), _ptr(out.token_map), _ptr(workspace), workspace.numel(), _stream(input)))
    return out


def route_dispatch(logits: torch.Tensor, top_k: int, renormalize: bool, input: torch.Tensor, out: Dispatched | None = None,
                   workspace=None):
    """``route`` then ``dispatch`` of its plan in one call (``rudnn_moe_route_dispatch``).  Returns
    ``(expert_indices [T, k] int32 holding the uint32 ids, weights [T, k] logits dtype, Dispatched)``."""
    logits = _contig(logits, "logits")
    input = _contig(input, "input")
    T, E = logits.shape
    H = input.shape[1]
    dev = input.device
    idx = torch.empty(T, top_k, dtype=torch.int32, device=dev)
    w = torch.empty(T, top_k, dtype=logits.dtype, device=dev)
    if out is None:
        out = Dispatched(torch.empty(T * top_k, H, dtype=input.dtype, device=dev),
                         torch.empty(E + 1, dtype=torch.int32, device=dev),
                         torch.empty(T, top_k, dtype=torch.int32, device=dev))
    need = lib().rudnn_moe_dispatch_workspace_size(T, top_k, E)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check("rudnn_moe_route_dispatch", lib().rudnn_moe_route_dispatch(
        _ptr(logits), _dt(logits), T, E, RoutingOptions(top_k, int(renormalize)), _ptr(input), _dt(input), H, _ptr(idx),
        _ptr(w), _ptr(out.dispatched), _ptr(out.expert_offsets), _ptr(out.token_map), _ptr(workspace), workspace.numel(),
        _stream(input)))
    return idx, w, out


# Bytes of the library's own per-device dispatch buffer (RUDNN_MOE_DISPATCH_NO_ALLOC_MAX_BYTES).
DISPATCH_NO_ALLOC_MAX_BYTES = 16 << 20


def dispatch_no_alloc(expert_indices: torch.Tensor, input: torch.Tensor, num_experts: int,
                      out: Dispatched) -> Dispatched:
    """``dispatch`` through ``rudnn_moe_dispatch_no_alloc``: the caller passes every output buffer
    and the library allocates nothing (its per-chunk counts live in a device array of its own)."""
    expert_indices = _contig(expert_indices, "expert_indices")
    input = _contig(input, "input")
    T, k = expert_indices.shape
    H = input.shape[1]
    _check("rudnn_moe_dispatch_no_alloc", lib().rudnn_moe_dispatch_no_alloc(
        _ptr(expert_indices), T, k, num_experts, _ptr(input), _dt(input), H, _ptr(out.dispatched),
        _ptr(out.expert_offsets), _ptr(out.token_map), _stream(input)))
    return out


def experts_workspace_size(experts: SwiGluExperts, rows: int) -> int:
    return lib().rudnn_moe_experts_workspace_size(ctypes.byref(experts.view), rows)


def experts_forward(experts: SwiGluExperts, dispatched: torch.Tensor, expert_offsets: torch.Tensor, out=None,
                    workspace=None) -> torch.Tensor:
    dispatched = _contig(dispatched, "dispatched")
    rows = dispatched.shape[0]
    if out is None:
        out = torch.empty_like(dispatched)
    if workspace is None:
        workspace = torch.empty(max(experts_workspace_size(experts, rows), 1), dtype=torch.uint8,
                                device=dispatched.device)
    _check("rudnn_moe_experts_forward", lib().rudnn_moe_experts_forward(
        ctypes.byref(experts.view), _ptr(dispatched), _ptr(expert_offsets), rows, _ptr(out), _ptr(workspace),
        workspace.numel(), _stream(dispatched)))
    return out


def experts_forward_training(experts: SwiGluExperts, dispatched: torch.Tensor, expert_offsets: torch.Tensor,
                             out=None, cache=None, workspace=None):
    """``experts_forward`` that also returns the FP32 pre-activations [rows, 2I] (the backward's cache)."""
    dispatched = _contig(dispatched, "dispatched")
    rows = dispatched.shape[0]
    if out is None:
        out = torch.empty_like(dispatched)
    if cache is None:
        cache = torch.empty(rows, 2 * experts.I, dtype=torch.float32, device=dispatched.device)
    if workspace is None:
        workspace = torch.empty(max(experts_workspace_size(experts, rows), 1), dtype=torch.uint8,
                                device=dispatched.device)
    _check("rudnn_moe_experts_forward_training", lib().rudnn_moe_experts_forward_training(
        ctypes.byref(experts.view), _ptr(dispatched), _ptr(expert_offsets), rows, _ptr(out), _ptr(_contig(cache, "cache")),
        _ptr(workspace), workspace.numel(), _stream(dispatched)))
    return out, cache


def combine(expert_output: torch.Tensor, token_map: torch.Tensor, weights: torch.Tensor, out=None) -> torch.Tensor:
    expert_output = _contig(expert_output, "expert_output")
    T, k = token_map.shape
    H = expert_output.shape[1]
    if out is None:
        out = torch.empty(T, H, dtype=expert_output.dtype, device=expert_output.device)
    _check("rudnn_moe_combine", lib().rudnn_moe_combine(
        _ptr(expert_output), _dt(expert_output), _ptr(_contig(token_map, "token_map")), _ptr(_contig(weights, "weights")),
        _dt(weights), T, k, H, _ptr(out), _stream(expert_output)))
    return out


def forward_workspace_size(experts: SwiGluExperts, T: int, top_k: int, logits_dtype: torch.dtype) -> int:
    return lib().rudnn_moe_forward_workspace_size(ctypes.byref(experts.view), T, top_k, _DT[logits_dtype])


def forward(experts: SwiGluExperts, input: torch.Tensor, logits: torch.Tensor, top_k: int, renormalize: bool,
            out=None, workspace=None) -> torch.Tensor:
    """The whole local forward route -> dispatch -> experts -> combine (user guide section 6)."""
    input = _contig(input, "input")
    logits = _contig(logits, "logits")
    T = input.shape[0]
    if out is None:
        out = torch.empty_like(input)
    if workspace is None:
        workspace = torch.empty(max(forward_workspace_size(experts, T, top_k, logits.dtype), 1), dtype=torch.uint8,
                                device=input.device)
    _check("rudnn_moe_forward", lib().rudnn_moe_forward(
        ctypes.byref(experts.view), _ptr(input), _ptr(logits), _dt(logits), T, RoutingOptions(top_k, int(renormalize)),
        _ptr(out), _ptr(workspace), workspace.numel(), _stream(input)))
    return out


def forward_sigmoid_grouped(experts: SwiGluExperts, input: torch.Tensor, logits: torch.Tensor, bias,
                            options: GroupRoutingOptions, out=None, workspace=None) -> torch.Tensor:
    """The whole local forward with group-limited sigmoid routing (user guide section 10)."""
    input = _contig(input, "input")
    logits = _contig(logits, "logits")
    bias = _bias(bias, logits)
    T = input.shape[0]
    if out is None:
        out = torch.empty_like(input)
    if workspace is None:
        workspace = torch.empty(max(forward_workspace_size(experts, T, options.top_k, logits.dtype), 1),
                                dtype=torch.uint8, device=input.device)
    _check("rudnn_moe_forward_sigmoid_grouped", lib().rudnn_moe_forward_sigmoid_grouped(
        ctypes.byref(experts.view), _ptr(input), _ptr(logits), _dt(logits), T, _ptr(bias), options,
        _ptr(out), _ptr(workspace), workspace.numel(), _stream(input)))
    return out


def forward_projected_workspace_size(experts: SwiGluExperts, T: int, top_k: int) -> int:
    return lib().rudnn_moe_forward_projected_workspace_size(ctypes.byref(experts.view), T, top_k)


def forward_projected(experts: SwiGluExperts, input: torch.Tensor, router: torch.Tensor, top_k: int,
                      renormalize: bool, out=None, workspace=None) -> torch.Tensor:
    """The local forward from the hidden states: fused gate projection + routing -> dispatch ->
    experts -> combine; ``router`` [E, H] in the experts' dtype."""
    input = _contig(input, "input")
    router = _contig(router, "router")
    T = input.shape[0]
    if out is None:
        out = torch.empty_like(input)
    if workspace is None:
        workspace = torch.empty(max(forward_projected_workspace_size(experts, T, top_k), 1), dtype=torch.uint8,
                                device=input.device)
    _check("rudnn_moe_forward_projected", lib().rudnn_moe_forward_projected(
        ctypes.byref(experts.view), _ptr(input), _ptr(router), T, RoutingOptions(top_k, int(renormalize)),
        _ptr(out), _ptr(workspace), workspace.numel(), _stream(input)))
    return out



# ---------------------------------------------------------------------------------------------
# First-order training (user guide section 12)
# ---------------------------------------------------------------------------------------------

def _index_type(indices: torch.Tensor, unsigned: bool) -> int:
    """0 = U32 (an int32 tensor holding uint32 ids, as ``route`` returns), 1 = I32, 2 = I64."""
    if indices.dtype == torch.int64:
        return 2
    if indices.dtype != torch.int32:
        raise TypeError("indices must be int32 (holding uint32 or int32 ids) or int64")
    return 0 if unsigned else 1


def _router_opts(scoring: str, renormalize: bool, scale: float) -> RouterWeightOptions:
    return RouterWeightOptions({"softmax": 0, "sigmoid": 1}[scoring], int(bool(renormalize)), float(scale))


def selected_router_weights(logits: torch.Tensor, indices: torch.Tensor, scoring: str = "softmax",
                            renormalize: bool = False, scale: float = 1.0, unsigned: bool = True) -> torch.Tensor:
    """FP32 weights [T, k] of the fixed selection ``indices`` (user guide section 12)."""
    logits, indices = _contig(logits, "logits"), _contig(indices, "indices")
    T, E = logits.shape
    k = indices.shape[1]
    w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _check("rudnn_moe_selected_router_weights", lib().rudnn_moe_selected_router_weights(
        _ptr(logits), _dt(logits), T, E, _ptr(indices), _index_type(indices, unsigned), k,
        _router_opts(scoring, renormalize, scale), _ptr(w), _stream(logits)))
    return w


def selected_router_backward(logits: torch.Tensor, indices: torch.Tensor, grad_weights: torch.Tensor,
                             scoring: str = "softmax", renormalize: bool = False, scale: float = 1.0,
                             unsigned: bool = True) -> torch.Tensor:
    """Logits gradient [T, E] (logits dtype) of those weights for FP32 ``grad_weights`` [T, k]."""
    logits, indices = _contig(logits, "logits"), _contig(indices, "indices")
    grad_weights = _contig(grad_weights, "grad_weights")
    if grad_weights.dtype != torch.float32:
        raise TypeError("grad_weights is FP32")
    T, E = logits.shape
    k = indices.shape[1]
    g = torch.empty_like(logits)
    _check("rudnn_moe_selected_router_backward", lib().rudnn_moe_selected_router_backward(
        _ptr(logits), _dt(logits), T, E, _ptr(indices), _index_type(indices, unsigned), k,
        _router_opts(scoring, renormalize, scale), _ptr(grad_weights), _ptr(g), _stream(logits)))
    return g


class RouterTrainingPlan:
    """User guide section 12 (RoutingPlan::into_training): the selection ``indices`` is kept and
    its FP32 weights are recomputed from ``logits``; ``routing()`` gives (indices, weights) for
    dispatch and combine, ``backward(grad_weights)`` the logits gradient.  The logits and indices
    must stay unchanged until then."""

    def __init__(self, logits: torch.Tensor, indices: torch.Tensor, scoring: str = "softmax",
                 renormalize: bool = False, scale: float = 1.0, unsigned: bool = True):
        self.logits, self.indices = logits, indices
        self.scoring, self.renormalize, self.scale, self.unsigned = scoring, renormalize, scale, unsigned
        self.weights = selected_router_weights(logits, indices, scoring, renormalize, scale, unsigned)

    def routing(self):
        return self.indices, self.weights

    def backward(self, grad_weights: torch.Tensor) -> torch.Tensor:
        return selected_router_backward(self.logits, self.indices, grad_weights, self.scoring, self.renormalize,
                                        self.scale, self.unsigned)


def into_training(logits: torch.Tensor, indices: torch.Tensor, scoring: str = "softmax", renormalize: bool = False,
                  scale: float = 1.0) -> RouterTrainingPlan:
    """A routing result (``indices`` as ``route`` returns them) turned into a training plan."""
    return RouterTrainingPlan(logits, indices, scoring, renormalize, scale, unsigned=True)


def combine_backward(expert_output: torch.Tensor, token_map: torch.Tensor, weights: torch.Tensor,
                     grad_output: torch.Tensor, grad_expert_output: torch.Tensor | None = None):
    """Returns ``(grad_expert_output [T*k, H], grad_weights [T, k] FP32)`` (user guide section 12, step 1).
    Rows of grad_expert_output named by no valid map entry keep their previous contents."""
    expert_output = _contig(expert_output, "expert_output")
    grad_output = _contig(grad_output, "grad_output")
    T, k = token_map.shape
    H = expert_output.shape[1]
    if grad_expert_output is None:
        grad_expert_output = torch.zeros_like(expert_output)
    gw = torch.empty(T, k, dtype=torch.float32, device=expert_output.device)
    _check("rudnn_moe_combine_backward", lib().rudnn_moe_combine_backward(
        _ptr(expert_output), _dt(expert_output), _ptr(_contig(token_map, "token_map")), _ptr(_contig(weights, "weights")),
        _dt(weights), _ptr(grad_output), T, k, H, _ptr(grad_expert_output), _ptr(gw), _stream(expert_output)))
    return grad_expert_output, gw


def dispatch_backward(grad_dispatched: torch.Tensor, token_map: torch.Tensor, out=None) -> torch.Tensor:
    """grad_input [T, H]: the selected rows summed back to their token (user guide section 12, step 3)."""
    grad_dispatched = _contig(grad_dispatched, "grad_dispatched")
    T, k = token_map.shape
    H = grad_dispatched.shape[1]
    if out is None:
        out = torch.empty(T, H, dtype=grad_dispatched.dtype, device=grad_dispatched.device)
    _check("rudnn_moe_dispatch_backward", lib().rudnn_moe_dispatch_backward(
        _ptr(grad_dispatched), _dt(grad_dispatched), _ptr(_contig(token_map, "token_map")), T, k, H, _ptr(out),
        _stream(grad_dispatched)))
    return out


def experts_backward_workspace_size(experts: SwiGluExperts, rows: int, cached: bool = False) -> int:
    return lib().rudnn_moe_experts_backward_workspace_size(ctypes.byref(experts.view), rows, int(bool(cached)))


def experts_backward(experts: SwiGluExperts, dispatched: torch.Tensor, expert_offsets: torch.Tensor,
                     grad_expert_output: torch.Tensor, cache=None, workspace=None):
    """Returns ``(grad_dispatched [rows, H] (rows outside the experts' ranges zero), dgate, dup [E, I, H],
    ddown [E, H, I] FP32)``.  ``cache``: the pre-activations from ``experts_forward_training``, or None
    to recompute them."""
    dispatched = _contig(dispatched, "dispatched")
    grad_expert_output = _contig(grad_expert_output, "grad_expert_output")
    rows = dispatched.shape[0]
    dev = dispatched.device
    E, I, H = experts.E, experts.I, experts.H
    dx = torch.zeros_like(dispatched)
    dg = torch.empty(E, I, H, dtype=torch.float32, device=dev)
    du = torch.empty(E, I, H, dtype=torch.float32, device=dev)
    dd = torch.empty(E, H, I, dtype=torch.float32, device=dev)
    if cache is not None:
        cache = _contig(cache, "cache")
        if cache.dtype != torch.float32 or tuple(cache.shape) != (rows, 2 * I):
            raise ValueError("cache must be FP32 [rows, 2I]")
    if workspace is None:
        workspace = torch.empty(max(experts_backward_workspace_size(experts, rows, cache is not None), 1),
                                dtype=torch.uint8, device=dev)
    _check("rudnn_moe_experts_backward", lib().rudnn_moe_experts_backward(
        ctypes.byref(experts.view), _ptr(dispatched), _ptr(_contig(expert_offsets, "expert_offsets")), rows,
        _ptr(cache), _ptr(grad_expert_output), _ptr(dx), _ptr(dg), _ptr(du), _ptr(dd), _ptr(workspace), workspace.numel(),
        _stream(dispatched)))
    return dx, dg, du, dd
