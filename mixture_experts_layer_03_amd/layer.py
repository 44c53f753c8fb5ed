"""torch-facing wrappers of the C ABI: route, permute, experts, forward.

PyTorch supplies device memory and the current stream; every step of the layer
runs in the HIP library.  Shapes are taken from the real tensors and checked
against the config before anything is launched (mlxcel #838 "Defensive
requirements": bounds from real shapes, never from config fields alone).
"""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass

import torch

from . import _lib
from .config import MoEConfig

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass
class MoEWeights:
    """Device tensors of one layer (see include/moe.h for layouts)."""

    router: torch.Tensor
    gate: torch.Tensor = None
    up: torch.Tensor = None
    down: torch.Tensor = None
    router_bias: torch.Tensor = None
    expert_bias: torch.Tensor = None
    gate_scale: torch.Tensor = None
    gate_zero: torch.Tensor = None
    up_scale: torch.Tensor = None
    up_zero: torch.Tensor = None
    down_scale: torch.Tensor = None
    down_zero: torch.Tensor = None
    shared_gate: torch.Tensor = None
    shared_up: torch.Tensor = None
    shared_down: torch.Tensor = None

    def to_c(self) -> _lib.moe_weights:
        def p(t):
            return None if t is None else t.data_ptr()
        return _lib.moe_weights(**{name: p(getattr(self, name)) for name, _ in _lib.moe_weights._fields_})


def host_tensor_to_device(a, device):
    """numpy array -> device tensor; uint16 arrays are bf16 bit patterns."""
    import numpy as np
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def weights_from_host(L: dict, device) -> MoEWeights:
    """Upload a dict of host arrays (names as in MoEWeights; u8 codes may be called
    gate_q/up_q/down_q, packed u4 codes gate_q4/up_q4/down_q4) to the device."""
    kw = {}
    for k, v in L.items():
        if v is None:
            continue
        name = k[:-2] if k.endswith("_q") else (k[:-3] if k.endswith("_q4") else k)
        kw[name] = host_tensor_to_device(v, device)
    return MoEWeights(**kw)


def _need(t, name, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def check_weights(cfg: MoEConfig, w: MoEWeights, device, need_router=True, need_experts=True):
    H, E, I, Is = cfg.hidden, cfg.num_experts, cfg.moe_intermediate, cfg.shared_intermediate
    adt = _TORCH_DT[cfg.act_dtype]
    if need_router:
        _need(w.router, "router", (E, H), adt, device)
        if w.router_bias is not None:
            _need(w.router_bias, "router_bias", (E,), torch.float32, device)
        if cfg.use_expert_bias:
            _need(w.expert_bias, "expert_bias", (E,), torch.float32, device)
    if need_experts:
        if cfg.expert_dtype in ("u8", "u4"):
            G = cfg.quant_group
            d = 2 if cfg.expert_dtype == "u4" else 1  # u4: two codes per byte along the row
            for n, shp, ss in (("gate", (E, I, H // d), (E, I, H // G)), ("up", (E, I, H // d), (E, I, H // G)),
                               ("down", (E, H, I // d), (E, H, I // G))):
                _need(getattr(w, n), n, shp, torch.uint8, device)
                _need(getattr(w, n + "_scale"), n + "_scale", ss, torch.float16, device)
                _need(getattr(w, n + "_zero"), n + "_zero", ss, torch.float16, device)
        else:
            edt = _TORCH_DT[cfg.expert_dtype]
            _need(w.gate, "gate", (E, I, H), edt, device)
            _need(w.up, "up", (E, I, H), edt, device)
            _need(w.down, "down", (E, H, I), edt, device)
        if Is > 0:
            _need(w.shared_gate, "shared_gate", (Is, H), adt, device)
            _need(w.shared_up, "shared_up", (Is, H), adt, device)
            _need(w.shared_down, "shared_down", (H, Is), adt, device)


class Workspace:
    """Scratch buffers that grow on demand, one per (device, stream).

    Calls on different streams get different buffers, so they never race on one.
    A buffer is allocated while its stream is current, so the caching allocator ties
    it to that stream: when a larger buffer replaces it, the old memory is reused
    only by work ordered after everything already queued on the same stream."""

    def __init__(self):
        self._buf = {}

    def get(self, device, nbytes: int) -> torch.Tensor:
        stream = torch.cuda.current_stream(device)
        key = (str(device), stream.cuda_stream)
        b = self._buf.get(key)
        if b is None or b.numel() < nbytes:
            with torch.cuda.stream(stream):
                b = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._buf[key] = b
        return b


_WS = Workspace()


def _stream(device):
    return C.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _x_checks(cfg: MoEConfig, x: torch.Tensor):
    if x.dim() != 2 or x.shape[1] != cfg.hidden:
        raise ValueError(f"x must be [T, {cfg.hidden}], got {tuple(x.shape)}")
    if x.dtype != _TORCH_DT[cfg.act_dtype]:
        raise ValueError(f"x has dtype {x.dtype}, expected {_TORCH_DT[cfg.act_dtype]}")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous device tensor")


def workspace_for(cfg: MoEConfig, T: int, device, ws: torch.Tensor | None):
    need = cfg.workspace_size(T)
    if ws is None:
        ws = _WS.get(device, need)
    elif ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {need}")
    return ws, need


def route(x: torch.Tensor, router_w: torch.Tensor, cfg: MoEConfig, router_bias=None,
          expert_bias=None, ws=None):
    """Router: returns (topk_idx [T,k] int32, topk_w [T,k] fp32)."""
    _x_checks(cfg, x)
    T = x.shape[0]
    w = MoEWeights(router=router_w, router_bias=router_bias, expert_bias=expert_bias)
    check_weights(cfg, w, x.device, need_router=True, need_experts=False)
    idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=x.device)
    wt = torch.empty((T, cfg.top_k), dtype=torch.float32, device=x.device)
    if T == 0:
        return idx, wt
    ws, nb = workspace_for(cfg, T, x.device, ws)
    c = cfg.to_c()
    _lib.check(_lib.lib().moe_route(
        C.byref(c), T, x.data_ptr(), router_w.data_ptr(),
        None if router_bias is None else router_bias.data_ptr(),
        None if expert_bias is None else expert_bias.data_ptr(),
        idx.data_ptr(), wt.data_ptr(), ws.data_ptr(), ws.numel(), _stream(x.device)))
    return idx, wt


def permute(topk_idx: torch.Tensor, cfg: MoEConfig, ws=None):
    """Permutation: returns (counts [E], offsets [E+1], perm [T*k]) int32."""
    if topk_idx.dim() != 2 or topk_idx.shape[1] != cfg.top_k or topk_idx.dtype != torch.int32:
        raise ValueError("topk_idx must be int32 [T, top_k]")
    if not topk_idx.is_contiguous():
        raise ValueError("topk_idx must be contiguous")
    T = topk_idx.shape[0]
    dev = topk_idx.device
    counts = torch.empty(cfg.num_experts, dtype=torch.int32, device=dev)
    offsets = torch.empty(cfg.num_experts + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * cfg.top_k, dtype=torch.int32, device=dev)
    if T == 0:
        counts.zero_()
        offsets.zero_()
        return counts, offsets, perm
    ws, _ = workspace_for(cfg, T, dev, ws)
    c = cfg.to_c()
    _lib.check(_lib.lib().moe_permute(C.byref(c), T, topk_idx.data_ptr(), counts.data_ptr(),
                                      offsets.data_ptr(), perm.data_ptr(), ws.data_ptr(),
                                      ws.numel(), _stream(dev)))
    return counts, offsets, perm


def experts(x: torch.Tensor, weights: MoEWeights, topk_idx: torch.Tensor, topk_w: torch.Tensor,
            cfg: MoEConfig, ws=None, out=None):
    """Expert stage with given routing: returns y [T,H]."""
    _x_checks(cfg, x)
    T = x.shape[0]
    check_weights(cfg, weights, x.device, need_router=False, need_experts=True)
    _need(topk_idx, "topk_idx", (T, cfg.top_k), torch.int32, x.device)
    _need(topk_w, "topk_w", (T, cfg.top_k), torch.float32, x.device)
    y = out if out is not None else torch.empty_like(x)
    if T == 0:
        return y
    ws, _ = workspace_for(cfg, T, x.device, ws)
    c = cfg.to_c()
    wc = weights.to_c()
    _lib.check(_lib.lib().moe_experts(C.byref(c), T, x.data_ptr(), C.byref(wc), topk_idx.data_ptr(),
                                      topk_w.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(),
                                      _stream(x.device)))
    return y


def forward(x: torch.Tensor, weights: MoEWeights, cfg: MoEConfig, return_routing=False, ws=None,
            out=None):
    """The whole layer: y = MoE(x).  With return_routing, also (idx, w, counts)."""
    _x_checks(cfg, x)
    T = x.shape[0]
    check_weights(cfg, weights, x.device, need_router=True, need_experts=True)
    y = out if out is not None else torch.empty_like(x)
    if out is not None:
        _need(out, "out", tuple(x.shape), x.dtype, x.device)
    idx = wt = counts = None
    if return_routing:
        idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=x.device)
        wt = torch.empty((T, cfg.top_k), dtype=torch.float32, device=x.device)
        counts = torch.zeros(cfg.num_experts, dtype=torch.int32, device=x.device)
    if T > 0:
        ws, _ = workspace_for(cfg, T, x.device, ws)
        c = cfg.to_c()
        wc = weights.to_c()
        _lib.check(_lib.lib().moe_forward(
            C.byref(c), T, x.data_ptr(), C.byref(wc), y.data_ptr(),
            None if idx is None else idx.data_ptr(), None if wt is None else wt.data_ptr(),
            None if counts is None else counts.data_ptr(), ws.data_ptr(), ws.numel(),
            _stream(x.device)))
    if return_routing:
        return y, (idx, wt, counts)
    return y


def forward_noalloc(x: torch.Tensor, weights: MoEWeights, cfg: MoEConfig, return_routing=False, out=None):
    """The whole layer through moe_forward_noalloc: no workspace argument; the library's
    fixed device scratch (64 MiB per GPU) is used instead.  Calls that overlap in time on
    one GPU share that scratch and race; the caller serialises them."""
    _x_checks(cfg, x)
    T = x.shape[0]
    check_weights(cfg, weights, x.device, need_router=True, need_experts=True)
    y = out if out is not None else torch.empty_like(x)
    if out is not None:
        _need(out, "out", tuple(x.shape), x.dtype, x.device)
    idx = wt = counts = None
    if return_routing:
        idx = torch.empty((T, cfg.top_k), dtype=torch.int32, device=x.device)
        wt = torch.empty((T, cfg.top_k), dtype=torch.float32, device=x.device)
        counts = torch.zeros(cfg.num_experts, dtype=torch.int32, device=x.device)
    if T > 0:
        c = cfg.to_c()
        wc = weights.to_c()
        _lib.check(_lib.lib().moe_forward_noalloc(
            C.byref(c), T, x.data_ptr(), C.byref(wc), y.data_ptr(),
            None if idx is None else idx.data_ptr(), None if wt is None else wt.data_ptr(),
            None if counts is None else counts.data_ptr(), _stream(x.device)))
    if return_routing:
        return y, (idx, wt, counts)
    return y


def dense_workspace_size(cfg: MoEConfig, intermediate: int, T: int) -> int:
    n = C.c_size_t(0)
    c = cfg.to_c()
    _lib.check(_lib.lib().moe_dense_workspace_size(C.byref(c), intermediate, T, C.byref(n)))
    return n.value


def dense_mlp(x: torch.Tensor, gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor, cfg: MoEConfig,
              ws=None, out=None):
    """Dense MLP of the layers before the MoE layers: y = (silu(x Wg^T) * (x Wu^T)) Wd^T.
    Uses cfg.hidden, cfg.act_dtype and cfg.path; the width is gate.shape[0]."""
    _x_checks(cfg, x)
    T, H = x.shape
    I = gate.shape[0] if gate is not None and gate.dim() == 2 else -1
    adt = _TORCH_DT[cfg.act_dtype]
    _need(gate, "gate", (I, H), adt, x.device)
    _need(up, "up", (I, H), adt, x.device)
    _need(down, "down", (H, I), adt, x.device)
    y = out if out is not None else torch.empty_like(x)
    if out is not None:
        _need(out, "out", tuple(x.shape), x.dtype, x.device)
    if T == 0:
        return y
    need = dense_workspace_size(cfg, I, T)
    if ws is None:
        ws = _WS.get(x.device, need)
    elif ws.numel() * ws.element_size() < need:
        raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {need}")
    c = cfg.to_c()
    _lib.check(_lib.lib().moe_dense_mlp(C.byref(c), I, T, x.data_ptr(), gate.data_ptr(), up.data_ptr(),
                                        down.data_ptr(), y.data_ptr(), ws.data_ptr(), ws.numel(),
                                        _stream(x.device)))
    return y
