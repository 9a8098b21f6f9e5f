"""The C ABI without a GPU: librom.so loads, exports what include/rom.h declares, and validates arguments
before any HIP call (so these run on a machine with no GPU at all)."""
import ctypes
import os
import re

import pytest

import state_space_lms_amd as rom

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rom.h")

A = 0x10000  # fake, 16-byte-aligned "device" addresses: never dereferenced on these error paths
OK, INVALID, UNSUPPORTED, WS_SMALL = rom.ROM_OK, rom.ROM_ERR_INVALID_ARGUMENT, rom.ROM_ERR_UNSUPPORTED, \
    rom.ROM_ERR_WORKSPACE_TOO_SMALL
BF16 = rom.ROM_DTYPE_BF16


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(rom.LIB_PATH):
        from state_space_lms_amd import build
        build.build()
    return rom.lib()


def declared_symbols():
    with open(HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"ROM_API\s+[\w\s\*]*?\b(rom_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_symbols()
    assert set(names) == set(rom.ABI_SYMBOLS), names
    for n in names:
        assert hasattr(L, n), f"{n} missing from librom.so"


def test_version_and_status_strings(L):
    assert L.rom_abi_version() == rom.ABI_VERSION
    for code, name in enumerate(["ROM_OK", "ROM_ERR_INVALID_ARGUMENT", "ROM_ERR_UNSUPPORTED",
                                 "ROM_ERR_WORKSPACE_TOO_SMALL", "ROM_ERR_HIP"]):
        assert L.rom_status_string(code).decode() == name


def test_workspace_bytes(L):
    assert L.rom_route_workspace_bytes(0, 8) == 0
    for T, E in [(1, 8), (257, 8), (16384, 8), (65536, 64)]:
        b = L.rom_route_workspace_bytes(T, E)
        # a [top_k][E][workgroups] histogram for up to two choices, 8 tokens per workgroup at the least
        assert b >= 2 * E * ((T + 7) // 8) * 4 and b % 256 == 0


def _routing(T=512, E=8, top_k=1, **over):
    f = dict(expert_id=A, prob=A, counts=A, offsets=A, perm=A, inv_perm=A)
    f.update(over)
    return rom.RoutingStruct(T, E, top_k, 0, f["expert_id"], f["prob"], f["counts"], f["offsets"], f["perm"],
                             f["inv_perm"])


def _route(L, X=A, dt=BF16, T=512, dm=128, Wr=A, bias=None, E=8, k=1, r="default", Xp=None, ws=A, wsb=1 << 20):
    rs = _routing(T, E) if r == "default" else r
    ref = ctypes.byref(rs) if rs is not None else None
    return L.rom_route(X, dt, T, dm, Wr, bias, E, k, ref, Xp, ws, wsb, None), rs


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(E=0), INVALID), (dict(E=65), UNSUPPORTED), (dict(k=3), UNSUPPORTED),
    (dict(k=2, E=1), INVALID), (dict(k=2, Xp=A + (1 << 24)), UNSUPPORTED),  # the permute is top-1 only
    (dict(k=0), INVALID), (dict(k=9), INVALID), (dict(dm=0), INVALID), (dict(dm=96), UNSUPPORTED),
    (dict(dm=65536 + 64), UNSUPPORTED),
    (dict(dt=7), INVALID), (dict(X=None), INVALID), (dict(X=A + 8), INVALID), (dict(Wr=None), INVALID),
    (dict(r=None), INVALID), (dict(bias=A + 2), INVALID), (dict(ws=None), WS_SMALL), (dict(wsb=16), WS_SMALL),
    (dict(Xp=A + 4096), INVALID),  # overlaps X
    (dict(T=(1 << 24) + 1), UNSUPPORTED),
])
def test_route_rejects(L, kw, code):
    st, _ = _route(L, **kw)
    assert st == code
    assert L.rom_last_error().decode() != ""


def test_route_rejects_null_routing_buffer(L):
    for field in ("expert_id", "prob", "counts", "offsets", "perm", "inv_perm"):
        st, _ = _route(L, r=_routing(512, 8, **{field: None}))
        assert st == INVALID and field in L.rom_last_error().decode()


def test_route_T0_is_noop_and_stamps(L):
    rs = rom.RoutingStruct(99, 0, 0, 0, None, None, None, None, None, None)
    st, _ = _route(L, X=None, Wr=None, T=0, r=rs, ws=None, wsb=0)
    assert st == OK and (rs.T, rs.E, rs.top_k) == (0, 8, 1)


def _in(L, X=A, T=512, dm=128, di=256, Wc=A, Wg=A, xo=A + (1 << 24), zo=A + (1 << 26), r=None, dt=BF16):
    rs = r if r is not None else _routing(T, 8)
    return L.rom_in_proj(X, ctypes.byref(rs), dt, T, dm, di, Wc, Wg, xo, zo, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(di=100), UNSUPPORTED), (dict(dm=0), INVALID), (dict(X=None), INVALID),
    (dict(Wc=A + 2), INVALID), (dict(zo=None), INVALID), (dict(zo=A + (1 << 24) + 64), INVALID),
    (dict(xo=A + 256), INVALID), (dict(r=_routing(256, 8)), INVALID), (dict(r=_routing(512, 0)), INVALID),
    (dict(r=_routing(512, 8, offsets=None)), INVALID), (dict(dt=3), INVALID),
    (dict(r=_routing(512, 8, top_k=3)), UNSUPPORTED), (dict(r=_routing(512, 2, top_k=3)), INVALID),
])
def test_in_proj_rejects(L, kw, code):
    assert _in(L, **kw) == code


def test_in_proj_T0_noop(L):
    assert _in(L, X=None, T=0, Wc=None, Wg=None, xo=None, zo=None, r=_routing(0, 8)) == OK


def _inw(L, X=A, T=512, dm=128, do=384, W=A, y=A + (1 << 24), r=None, dt=BF16):
    rs = r if r is not None else _routing(T, 4)
    return L.rom_in_proj_weighted(X, ctypes.byref(rs), dt, T, dm, do, W, y, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), INVALID), (dict(do=100), UNSUPPORTED), (dict(do=0), INVALID), (dict(dm=32), UNSUPPORTED),
    (dict(X=None), INVALID), (dict(W=A + 8), INVALID), (dict(y=None), INVALID), (dict(y=A + 512), INVALID),
    (dict(r=_routing(256, 4)), INVALID), (dict(r=_routing(512, 4, prob=None)), INVALID), (dict(dt=2), INVALID),
    (dict(r=_routing(512, 4, top_k=3)), UNSUPPORTED), (dict(r=_routing(512, 1, top_k=2)), INVALID),
])
def test_in_proj_weighted_rejects(L, kw, code):
    assert _inw(L, **kw) == code


def test_in_proj_weighted_T0_noop(L):
    assert _inw(L, X=None, T=0, W=None, y=None, r=_routing(0, 4)) == OK


def _conv(L, x=A, dt=BF16, ns=4, sl=100, C=256, w=A + (1 << 26), b=None, width=4, act=1, y=A + (1 << 24)):
    return L.rom_conv1d(x, dt, ns, sl, C, w, b, width, act, y, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ns=-1), INVALID), (dict(sl=-3), INVALID), (dict(C=0), INVALID), (dict(C=96), UNSUPPORTED),
    (dict(width=0), INVALID), (dict(width=9), UNSUPPORTED), (dict(act=2), INVALID), (dict(dt=5), INVALID),
    (dict(x=None), INVALID), (dict(w=None), INVALID), (dict(y=None), INVALID), (dict(w=A + 8), INVALID),
    (dict(b=A + 4), INVALID), (dict(y=A + 1024), INVALID), (dict(ns=4096, sl=4097), UNSUPPORTED),
])
def test_conv1d_rejects(L, kw, code):
    assert _conv(L, **kw) == code


def test_conv1d_empty_is_noop(L):
    assert _conv(L, x=None, w=None, y=None, ns=0) == OK
    assert _conv(L, x=None, w=None, y=None, sl=0) == OK


BWS = A + (1 << 32)  # 256-byte aligned fake workspace, far from the other fake buffers


def _obwd(L, g=A, z=A + (1 << 24), h=A + (2 << 24), T=512, dm=128, di=256, Wo=A + (3 << 24), dz=A + (4 << 24),
          dh=A + (5 << 24), dW=A + (6 << 24), r=None, dt=BF16, ws=BWS, wsb=1 << 30):
    rs = r if r is not None else _routing(T, 8)
    return L.rom_out_proj_backward(g, z, h, ctypes.byref(rs), dt, T, dm, di, Wo, dz, dh, dW, ws, wsb, None)


def _ibwd(L, X=A, dx=A + (1 << 24), dz=A + (2 << 24), T=512, dm=128, di=256, Wc=A + (3 << 24), Wg=A + (4 << 24),
          dX=A + (5 << 24), dWc=A + (6 << 24), dWg=A + (7 << 24), r=None, dt=BF16, ws=BWS, wsb=1 << 30):
    rs = r if r is not None else _routing(T, 8)
    return L.rom_in_proj_backward(X, dx, dz, ctypes.byref(rs), dt, T, dm, di, Wc, Wg, dX, dWc, dWg, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dt=rom.ROM_DTYPE_F32), UNSUPPORTED), (dict(dt=9), INVALID), (dict(T=-1), INVALID), (dict(di=96), UNSUPPORTED),
    (dict(g=None), INVALID), (dict(dW=A + 8), INVALID), (dict(ws=None), WS_SMALL), (dict(wsb=1024), WS_SMALL),
    (dict(ws=BWS + 16), INVALID), (dict(dz=A + (2 << 24)), INVALID), (dict(dh=A + (4 << 24)), INVALID),
    (dict(r=_routing(256, 8)), INVALID), (dict(r=_routing(512, 8, top_k=3)), UNSUPPORTED),
])
def test_out_proj_backward_rejects(L, kw, code):
    assert _obwd(L, **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dt=rom.ROM_DTYPE_F32), UNSUPPORTED), (dict(dm=0), INVALID), (dict(dx=None), INVALID),
    (dict(dWg=None), INVALID), (dict(dX=A + 64), INVALID), (dict(dWg=A + (6 << 24)), INVALID),
    (dict(wsb=0), WS_SMALL), (dict(r=_routing(512, 8, offsets=None)), INVALID),
])
def test_in_proj_backward_rejects(L, kw, code):
    assert _ibwd(L, **kw) == code


def test_backward_T0_noop_and_workspace_bytes(L):
    assert _obwd(L, g=None, z=None, h=None, Wo=None, dz=None, dh=None, dW=None, ws=None, wsb=0, T=0,
                 r=_routing(0, 8)) == OK
    assert _ibwd(L, X=None, dx=None, dz=None, Wc=None, Wg=None, dX=None, dWc=None, dWg=None, ws=None, wsb=0, T=0,
                 r=_routing(0, 8)) == OK
    assert L.rom_backward_workspace_bytes(0, 128, 256, 8, 1) == 0
    b1 = L.rom_backward_workspace_bytes(16384, 1024, 2048, 8, 1)
    b2 = L.rom_backward_workspace_bytes(16384, 1024, 2048, 8, 2)
    # at least the transposed in-projection stacks and token-contiguous copies of dx, dz and X
    assert b1 >= 8 * 1024 * 4096 * 2 + (2 * 2048 + 1024) * 16384 * 2 and b2 > b1


WS = A + (1 << 28)


def _out(L, z=A, h=A + (1 << 24), T=512, dm=128, di=256, Wo=A, o=A + (1 << 26), r=None, ws=WS, wsb=1 << 24):
    rs = r if r is not None else _routing(T, 8)
    return L.rom_out_proj(z, h, ctypes.byref(rs), BF16, T, dm, di, Wo, o, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(T=-5), INVALID), (dict(dm=32), UNSUPPORTED), (dict(h=None), INVALID), (dict(o=A + 512), INVALID),
    (dict(o=A + (1 << 24)), INVALID), (dict(r=_routing(512, 8, perm=None)), INVALID), (dict(Wo=A + 1), INVALID),
    (dict(ws=None), WS_SMALL), (dict(wsb=512 * 256 * 2 - 1), WS_SMALL), (dict(ws=WS + 8), INVALID),
    (dict(ws=A + (1 << 24)), INVALID),  # overlaps h
])
def test_out_proj_rejects(L, kw, code):
    assert _out(L, **kw) == code


def test_out_proj_workspace_bytes(L):
    assert L.rom_out_proj_workspace_bytes(0, 2048, BF16) == 0
    assert L.rom_out_proj_workspace_bytes(64, 2048, BF16) == 64 * 2048 * 2  # gated rows, decode too
    assert L.rom_out_proj_workspace_bytes(1000, 2048, rom.ROM_DTYPE_F32) == 0
    assert L.rom_out_proj_workspace_bytes(16384, 2048, BF16) == 16384 * 2048 * 2


def test_binding_has_no_cpu_path(L):
    import torch
    X = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        rom.route(X, torch.zeros(64, 8))


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        rom.lib(os.path.join(tmp_path, "librom.so"))


# ---- the Python binding checks shapes and dtypes of everything the library reads or writes in full before it
# checks devices (the C ABI receives only pointers): CPU tensors of the wrong shape raise a shape error here

def _cpu(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


@pytest.mark.parametrize("case", ["router_rows", "router_1d", "bias", "x_out", "z_out_dtype", "y_out", "out",
                                  "conv_y", "conv_bias", "out_dtype"])
def test_binding_rejects_wrong_shapes_before_any_device_call(L, case):
    import torch
    T, dm, di, E = 40, 128, 64, 4
    X = _cpu(T, dm)
    Wr = torch.zeros((dm, E), dtype=torch.float32)
    r = rom.Routing(T, E, "cpu")
    Wc = _cpu(E, di, dm)
    Wo = _cpu(E, dm, di)
    z = _cpu(T, di)
    with pytest.raises(ValueError) as ei:
        if case == "router_rows":
            rom.route(X, torch.zeros((dm + 64, E), dtype=torch.float32))
        elif case == "router_1d":
            rom.route(X, torch.zeros((dm * E,), dtype=torch.float32))
        elif case == "bias":
            rom.route(X, Wr, torch.zeros((E + 1,), dtype=torch.float32))
        elif case == "x_out":
            rom.in_proj(X, r, Wc, Wc, x_out=_cpu(T, di + 64))
        elif case == "z_out_dtype":
            rom.in_proj(X, r, Wc, Wc, z_out=_cpu(T, di, dtype=torch.float32))
        elif case == "y_out":
            rom.in_proj_weighted(X, r, Wc, y_out=_cpu(T - 1, di))
        elif case == "out":
            rom.out_proj(z, z, r, Wo, out=_cpu(T, dm - 64))
        elif case == "out_dtype":
            rom.out_proj(z, z, r, Wo, out=_cpu(T, dm, dtype=torch.float32))
        elif case == "conv_y":
            rom.conv1d(z, _cpu(di, 4), y=_cpu(T, di + 64))
        elif case == "conv_bias":
            rom.conv1d(z, _cpu(di, 4), _cpu(di + 1))
    msg = str(ei.value)
    assert "ROCm device" not in msg, msg  # the shape check came first
