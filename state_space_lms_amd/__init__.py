"""MI355X-native Routing Mamba (RoM) routed projections.

Python binding over ``librom.so``, the gfx950 HIP library whose C ABI is ``include/rom.h``. This module
only marshals arguments: every step of the routed path (router, histogram, stable counting sort,
permute, the Conv/Gate in-projection grouped GEMM and the Out-projection grouped GEMM) runs in the
library's kernels. torch supplies device memory and the current stream. There is no CPU fallback:
without the built library, or with tensors that are not on a ROCm device, calls raise.

Method: "Routing Mamba: Scaling State Space Models with Mixture-of-Experts Projection", landing page on
chapterpal.com, Knowl 1 (shared router; indicator-selected Conv and Gate experts; router-probability
scaled Out experts).

    r = route(X, W_router)                  # one routing decision per block ...
    x, z = in_proj(X, r, W_conv, W_gate)    # ... shared by the in-projections ...
    out = out_proj(z, h, r, W_out)          # ... and the out-projection (h stands in for the SSM output)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = ["route", "route_noalloc", "in_proj", "in_proj_weighted", "out_proj", "conv1d", "out_proj_backward", "in_proj_backward",
           "backward_workspace_bytes", "Routing", "RomError", "lib", "LIB_PATH", "ABI_VERSION",
           "route_workspace_bytes", "out_proj_workspace_bytes"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "librom.so")
ABI_VERSION = 8

ROM_OK, ROM_ERR_INVALID_ARGUMENT, ROM_ERR_UNSUPPORTED, ROM_ERR_WORKSPACE_TOO_SMALL, ROM_ERR_HIP = range(5)
ROM_DTYPE_F32, ROM_DTYPE_BF16 = 0, 1
ROM_ACT_NONE, ROM_ACT_SILU = 0, 1
ABI_SYMBOLS = ("rom_abi_version", "rom_route_workspace_bytes", "rom_route", "rom_route_noalloc", "rom_in_proj", "rom_in_proj_weighted", "rom_conv1d",
               "rom_backward_workspace_bytes", "rom_out_proj_backward", "rom_in_proj_backward",
               "rom_out_proj_workspace_bytes", "rom_out_proj", "rom_status_string", "rom_last_error")


class RomError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({detail})")
        self.status = status


class RoutingStruct(ctypes.Structure):
    """Mirror of ``rom_routing`` in include/rom.h."""
    _fields_ = [("T", ctypes.c_int32), ("E", ctypes.c_int32), ("top_k", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("expert_id", ctypes.c_void_p), ("prob", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm", ctypes.c_void_p), ("inv_perm", ctypes.c_void_p)]


_LIB = None
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t


def lib(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librom.so (raises if it has not been built: python -m state_space_lms_amd.build)."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m state_space_lms_amd.build` (needs hipcc)")
    L = ctypes.CDLL(path)
    L.rom_abi_version.restype = ctypes.c_int
    L.rom_route_workspace_bytes.argtypes = [_i32, _i32]
    L.rom_route_workspace_bytes.restype = _sz
    L.rom_route.argtypes = [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _i32, _i32, ctypes.POINTER(RoutingStruct),
                            _vp, _vp, _sz, _vp]
    L.rom_route.restype = ctypes.c_int
    L.rom_route_noalloc.argtypes = [_vp, ctypes.c_int, _i32, _i32, _vp, _vp, _i32, _i32,
                                    ctypes.POINTER(RoutingStruct), _vp, _vp]
    L.rom_route_noalloc.restype = ctypes.c_int
    L.rom_in_proj.argtypes = [_vp, ctypes.POINTER(RoutingStruct), ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                              _vp]
    L.rom_in_proj.restype = ctypes.c_int
    L.rom_in_proj_weighted.argtypes = [_vp, ctypes.POINTER(RoutingStruct), ctypes.c_int, _i32, _i32, _i32, _vp, _vp,
                                       _vp]
    L.rom_in_proj_weighted.restype = ctypes.c_int
    L.rom_conv1d.argtypes = [_vp, ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _i32, _i32, _vp, _vp]
    L.rom_conv1d.restype = ctypes.c_int
    L.rom_backward_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32, _i32]
    L.rom_backward_workspace_bytes.restype = _sz
    L.rom_out_proj_backward.argtypes = [_vp, _vp, _vp, ctypes.POINTER(RoutingStruct), ctypes.c_int, _i32, _i32, _i32,
                                        _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.rom_out_proj_backward.restype = ctypes.c_int
    L.rom_in_proj_backward.argtypes = [_vp, _vp, _vp, ctypes.POINTER(RoutingStruct), ctypes.c_int, _i32, _i32, _i32,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.rom_in_proj_backward.restype = ctypes.c_int
    L.rom_out_proj_workspace_bytes.argtypes = [_i32, _i32, ctypes.c_int]
    L.rom_out_proj_workspace_bytes.restype = _sz
    L.rom_out_proj.argtypes = [_vp, _vp, ctypes.POINTER(RoutingStruct), ctypes.c_int, _i32, _i32, _i32, _vp, _vp, _vp,
                               _sz, _vp]
    L.rom_out_proj.restype = ctypes.c_int
    L.rom_status_string.argtypes = [ctypes.c_int]
    L.rom_status_string.restype = ctypes.c_char_p
    L.rom_last_error.restype = ctypes.c_char_p
    if L.rom_abi_version() != ABI_VERSION:
        raise RuntimeError(f"librom ABI version {L.rom_abi_version()} != {ABI_VERSION}")
    if path == LIB_PATH:
        _LIB = L
    return L


def _check(status: int, where: str):
    if status != ROM_OK:
        L = lib()
        raise RomError(status, where, f"{L.rom_status_string(status).decode()}: {L.rom_last_error().decode()}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ROM_DTYPE_BF16
    if t.dtype == torch.float32:
        return ROM_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32 only")


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a ROCm device tensor (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _want(t: torch.Tensor, shape, dtype, name: str) -> torch.Tensor:
    """Shape and dtype of a tensor the library reads or writes in full: the C ABI receives only a pointer, so a
    wrong-sized tensor would be read or written out of bounds. Checked before the device and layout checks."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t


def _matrix(t: torch.Tensor, name: str):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    return t.shape


def _same_device(routing: "Routing", t: torch.Tensor):
    if torch.device(routing.device) != t.device:
        raise ValueError(f"the routing buffers are on {routing.device}, the data on {t.device}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else (t.data_ptr() or None)


def _stream(device: torch.device, stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return s.cuda_stream


def route_workspace_bytes(T: int, E: int) -> int:
    return int(lib().rom_route_workspace_bytes(T, E))


class Routing:
    """The device buffers of one routing decision (``rom_routing``), reusable across calls of the same T, E
    and top_k. With top_k = K every array holds K stacked top-1 routings (choice k = row k): expert_id,
    prob, perm, inv_perm are [K][T], counts [K][E], offsets [K][E+1]."""

    def __init__(self, T: int, E: int, device, top_k: int = 1):
        device = torch.device(device)
        i32 = dict(dtype=torch.int32, device=device)
        self.T, self.E, self.top_k, self.device = T, E, top_k, device
        K = top_k
        self.expert_id = torch.empty((K, T), **i32)
        self.prob = torch.empty((K, T), dtype=torch.float32, device=device)
        self.counts = torch.empty((K, E), **i32)
        self.offsets = torch.empty((K, E + 1), **i32)
        self.perm = torch.empty((K, T), **i32)
        self.inv_perm = torch.empty((K, T), **i32)
        self.workspace = torch.empty(max(route_workspace_bytes(T, E), 256), dtype=torch.uint8, device=device)
        self.x_perm: Optional[torch.Tensor] = None
        self.out_workspace: Optional[torch.Tensor] = None  # gated rows for rom_out_proj, sized on first use
        self.bwd_workspace: Optional[torch.Tensor] = None  # the backward calls' workspace, sized on first use
        self.struct = RoutingStruct(0, E, top_k, 0, _ptr(self.expert_id), _ptr(self.prob), _ptr(self.counts),
                                    _ptr(self.offsets), _ptr(self.perm), _ptr(self.inv_perm))


def route(X: torch.Tensor, W_router: torch.Tensor, bias: Optional[torch.Tensor] = None, top_k: int = 1,
          permute: bool = False, routing: Optional[Routing] = None, stream=None) -> Routing:
    """rom_route: fp32 router, top-1 or top-2, probabilities, histogram, stable counting sort (and the permute)."""
    T, dm = _matrix(X, "X")
    _dtype_code(X)
    if W_router.dtype != torch.float32:
        raise TypeError("W_router must be fp32")
    if W_router.dim() != 2 or W_router.shape[0] != dm:
        raise ValueError(f"W_router must be [d_model = {dm}][E], got shape {tuple(W_router.shape)}")
    E = W_router.shape[1]
    if bias is not None:
        _want(bias, (E,), torch.float32, "bias")
        _dev(bias, "bias")
    _dev(X, "X")
    _dev(W_router, "W_router")
    r = routing if routing is not None else Routing(T, E, X.device, top_k)
    if (r.T, r.E, r.top_k) != (T, E, top_k):
        raise ValueError("routing buffers were sized for another T, E or top_k")
    _same_device(r, X)
    if permute:
        if r.x_perm is None or r.x_perm.dtype != X.dtype or r.x_perm.shape != X.shape:
            r.x_perm = torch.empty_like(X)
    status = lib().rom_route(_ptr(X), _dtype_code(X), T, dm, _ptr(W_router), _ptr(bias), E, top_k,
                             ctypes.byref(r.struct), _ptr(r.x_perm) if permute else None, _ptr(r.workspace),
                             r.workspace.numel(), _stream(X.device, stream))
    _check(status, "rom_route")
    return r


def route_noalloc(X: torch.Tensor, W_router: torch.Tensor, routing: Routing, bias: Optional[torch.Tensor] = None,
                  permute: bool = False, stream=None) -> Routing:
    """rom_route_noalloc: rom_route with the library's static scratch instead of a workspace (for callers
    that cannot allocate). The routing buffers (and X_perm, with permute) must already exist: this call
    allocates nothing."""
    T, dm = _matrix(X, "X")
    _dtype_code(X)
    if W_router.dtype != torch.float32 or W_router.dim() != 2 or W_router.shape[0] != dm:
        raise ValueError(f"W_router must be fp32 [d_model = {dm}][E], got {W_router.dtype} {tuple(W_router.shape)}")
    E = W_router.shape[1]
    if (routing.T, routing.E) != (T, E):
        raise ValueError("routing buffers were sized for another T or E")
    if bias is not None:
        _want(bias, (E,), torch.float32, "bias")
        _dev(bias, "bias")
    if permute:
        if routing.x_perm is None:
            raise ValueError("permute needs routing.x_perm allocated beforehand")
        _want(routing.x_perm, (T, dm), X.dtype, "routing.x_perm")
    _dev(X, "X")
    _dev(W_router, "W_router")
    _same_device(routing, X)
    status = lib().rom_route_noalloc(_ptr(X), _dtype_code(X), T, dm, _ptr(W_router), _ptr(bias), E, routing.top_k,
                                     ctypes.byref(routing.struct), _ptr(routing.x_perm) if permute else None,
                                     _stream(X.device, stream))
    _check(status, "rom_route_noalloc")
    return routing


def in_proj(X: torch.Tensor, routing: Routing, W_conv: torch.Tensor, W_gate: torch.Tensor,
            x_out: Optional[torch.Tensor] = None, z_out: Optional[torch.Tensor] = None,
            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """rom_in_proj: x = sum over the token's experts of W_conv[e] X, z likewise with W_gate (token order, no
    probability scale)."""
    T, dm = _matrix(X, "X")
    _dtype_code(X)
    if W_conv.dim() != 3:
        raise ValueError("W_conv must be [E][d_inner][d_model]")
    E, di, dm2 = W_conv.shape
    if dm2 != dm or W_gate.shape != W_conv.shape or W_conv.dtype != X.dtype or W_gate.dtype != X.dtype:
        raise ValueError("W_conv/W_gate must be [E][d_inner][d_model] in X's dtype")
    if E != routing.E:
        raise ValueError("expert count differs from the routing's")
    if x_out is not None:
        _want(x_out, (T, di), X.dtype, "x_out")
    if z_out is not None:
        _want(z_out, (T, di), X.dtype, "z_out")
    for t, n in ((X, "X"), (W_conv, "W_conv"), (W_gate, "W_gate")):
        _dev(t, n)
    _same_device(routing, X)
    x_out = torch.empty((T, di), dtype=X.dtype, device=X.device) if x_out is None else _dev(x_out, "x_out")
    z_out = torch.empty((T, di), dtype=X.dtype, device=X.device) if z_out is None else _dev(z_out, "z_out")
    status = lib().rom_in_proj(_ptr(X), ctypes.byref(routing.struct), _dtype_code(X), T, dm, di, _ptr(W_conv),
                               _ptr(W_gate), _ptr(x_out), _ptr(z_out), _stream(X.device, stream))
    _check(status, "rom_in_proj")
    return x_out, z_out


def in_proj_weighted(X: torch.Tensor, routing: Routing, W_in: torch.Tensor, y_out: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """rom_in_proj_weighted (Swimba): y = sum over the token's experts of p_t,e * W_in[e] X (token order)."""
    T, dm = _matrix(X, "X")
    _dtype_code(X)
    if W_in.dim() != 3:
        raise ValueError("W_in must be [E][d_out][d_model]")
    E, dout, dm2 = W_in.shape
    if dm2 != dm or W_in.dtype != X.dtype:
        raise ValueError("W_in must be [E][d_out][d_model] in X's dtype")
    if E != routing.E:
        raise ValueError("expert count differs from the routing's")
    if y_out is not None:
        _want(y_out, (T, dout), X.dtype, "y_out")
    _dev(X, "X")
    _dev(W_in, "W_in")
    _same_device(routing, X)
    y_out = torch.empty((T, dout), dtype=X.dtype, device=X.device) if y_out is None else _dev(y_out, "y_out")
    status = lib().rom_in_proj_weighted(_ptr(X), ctypes.byref(routing.struct), _dtype_code(X), T, dm, dout,
                                        _ptr(W_in), _ptr(y_out), _stream(X.device, stream))
    _check(status, "rom_in_proj_weighted")
    return y_out


def conv1d(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, n_seq: int = 1,
           activation: bool = True, y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rom_conv1d: the shared short causal depthwise convolution of each of n_seq sequences of x [T][C]
    (T = n_seq * seq_len, token order), weight [C][width], optional bias [C], optional SiLU."""
    T, C = _matrix(x, "x")
    _dtype_code(x)
    if n_seq <= 0 or T % n_seq != 0:
        raise ValueError("T must be a multiple of n_seq")
    if weight.dim() != 2 or weight.shape[0] != C or weight.dtype != x.dtype:
        raise ValueError("weight must be [C][width] in x's dtype")
    if bias is not None:
        _want(bias, (C,), x.dtype, "bias")
    if y is not None:
        _want(y, (T, C), x.dtype, "y")
    _dev(x, "x")
    _dev(weight, "weight")
    if bias is not None:
        _dev(bias, "bias")
    y = torch.empty_like(x) if y is None else _dev(y, "y")
    status = lib().rom_conv1d(_ptr(x), _dtype_code(x), n_seq, T // n_seq, C, _ptr(weight), _ptr(bias),
                              weight.shape[1], ROM_ACT_SILU if activation else ROM_ACT_NONE, _ptr(y),
                              _stream(x.device, stream))
    _check(status, "rom_conv1d")
    return y


def backward_workspace_bytes(T: int, d_model: int, d_inner: int, E: int, top_k: int = 1) -> int:
    return int(lib().rom_backward_workspace_bytes(T, d_model, d_inner, E, top_k))


def _bwd_workspace(routing: "Routing", T: int, dm: int, di: int, device) -> torch.Tensor:
    need = backward_workspace_bytes(T, dm, di, routing.E, routing.top_k)
    if routing.bwd_workspace is None or routing.bwd_workspace.numel() < need:
        routing.bwd_workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
    return routing.bwd_workspace


def out_proj_backward(d_out: torch.Tensor, z: torch.Tensor, h: torch.Tensor, routing: "Routing", W_out: torch.Tensor,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """rom_out_proj_backward: (dz, dh, dW_out) for the upstream gradient d_out, router probabilities held fixed.
    dW_out is fp32."""
    T, di = _matrix(z, "z")
    if W_out.dim() != 3:
        raise ValueError("W_out must be [E][d_model][d_inner]")
    E, dm, di2 = W_out.shape
    if di2 != di or h.shape != z.shape or d_out.shape != (T, dm) or E != routing.E:
        raise ValueError("shapes: d_out [T][d_model], z, h [T][d_inner], W_out [E][d_model][d_inner]")
    if not (d_out.dtype == z.dtype == h.dtype == W_out.dtype):
        raise ValueError("d_out, z, h and W_out must share one dtype")
    for t, n in ((d_out, "d_out"), (z, "z"), (h, "h"), (W_out, "W_out")):
        _dev(t, n)
    _same_device(routing, z)
    dz, dh = torch.empty_like(z), torch.empty_like(z)
    dW = torch.empty((E, dm, di), dtype=torch.float32, device=z.device)
    ws = _bwd_workspace(routing, T, dm, di, z.device)
    status = lib().rom_out_proj_backward(_ptr(d_out), _ptr(z), _ptr(h), ctypes.byref(routing.struct), _dtype_code(z),
                                         T, dm, di, _ptr(W_out), _ptr(dz), _ptr(dh), _ptr(dW), _ptr(ws), ws.numel(),
                                         _stream(z.device, stream))
    _check(status, "rom_out_proj_backward")
    return dz, dh, dW


def in_proj_backward(X: torch.Tensor, dx: torch.Tensor, dz: torch.Tensor, routing: "Routing", W_conv: torch.Tensor,
                     W_gate: torch.Tensor, stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """rom_in_proj_backward: (dX, dW_conv, dW_gate) for the upstream gradients dx, dz; weight gradients are fp32."""
    T, dm = _matrix(X, "X")
    if W_conv.dim() != 3:
        raise ValueError("W_conv must be [E][d_inner][d_model]")
    E, di, dm2 = W_conv.shape
    if dm2 != dm or W_gate.shape != W_conv.shape or dx.shape != (T, di) or dz.shape != (T, di) or E != routing.E:
        raise ValueError("shapes: X [T][d_model], dx, dz [T][d_inner], W_conv, W_gate [E][d_inner][d_model]")
    if not (X.dtype == dx.dtype == dz.dtype == W_conv.dtype == W_gate.dtype):
        raise ValueError("X, dx, dz, W_conv and W_gate must share one dtype")
    for t, n in ((X, "X"), (dx, "dx"), (dz, "dz"), (W_conv, "W_conv"), (W_gate, "W_gate")):
        _dev(t, n)
    _same_device(routing, X)
    dX = torch.empty_like(X)
    dWc = torch.empty((E, di, dm), dtype=torch.float32, device=X.device)
    dWg = torch.empty_like(dWc)
    ws = _bwd_workspace(routing, T, dm, di, X.device)
    status = lib().rom_in_proj_backward(_ptr(X), _ptr(dx), _ptr(dz), ctypes.byref(routing.struct), _dtype_code(X), T,
                                        dm, di, _ptr(W_conv), _ptr(W_gate), _ptr(dX), _ptr(dWc), _ptr(dWg), _ptr(ws),
                                        ws.numel(), _stream(X.device, stream))
    _check(status, "rom_in_proj_backward")
    return dX, dWc, dWg


def out_proj_workspace_bytes(T: int, d_inner: int, dtype: torch.dtype) -> int:
    code = ROM_DTYPE_BF16 if dtype == torch.bfloat16 else ROM_DTYPE_F32
    return int(lib().rom_out_proj_workspace_bytes(T, d_inner, code))


def out_proj(z: torch.Tensor, h: torch.Tensor, routing: Routing, W_out: torch.Tensor,
             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             stream=None) -> torch.Tensor:
    """rom_out_proj: out = sum over the token's experts of p_t,e * W_out[e] (SiLU(z) * h) (token order)."""
    T, di = _matrix(z, "z")
    _dtype_code(z)
    if W_out.dim() != 3:
        raise ValueError("W_out must be [E][d_model][d_inner]")
    E, dm, di2 = W_out.shape
    if di2 != di or h.shape != z.shape or h.dtype != z.dtype or W_out.dtype != z.dtype:
        raise ValueError("W_out must be [E][d_model][d_inner]; z, h [T][d_inner]; one dtype")
    if E != routing.E:
        raise ValueError("expert count differs from the routing's")
    if out is not None:
        _want(out, (T, dm), z.dtype, "out")
    for t, n in ((z, "z"), (h, "h"), (W_out, "W_out")):
        _dev(t, n)
    out = torch.empty((T, dm), dtype=z.dtype, device=z.device) if out is None else _dev(out, "out")
    _same_device(routing, z)
    if workspace is not None:
        _dev(workspace, "workspace")
    need = out_proj_workspace_bytes(T, di, z.dtype)
    if workspace is None and need > 0:
        if routing.out_workspace is None or routing.out_workspace.numel() < need:
            routing.out_workspace = torch.empty(need, dtype=torch.uint8, device=z.device)
        workspace = routing.out_workspace
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    status = lib().rom_out_proj(_ptr(z), _ptr(h), ctypes.byref(routing.struct), _dtype_code(z), T, dm, di,
                                _ptr(W_out), _ptr(out), _ptr(workspace), wsb, _stream(z.device, stream))
    _check(status, "rom_out_proj")
    return out
