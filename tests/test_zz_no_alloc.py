"""rom_route_noalloc (the entry point that allocates nothing) against rom_route, through the C ABI: identical
routing on two calls in a row, the second with fewer tokens, and the size limit of its static scratch."""
import ctypes

import numpy as np
import pytest

import parity
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rom():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no ROCm GPU visible")
    import state_space_lms_amd as rom_mod
    rom_mod.lib()
    return rom_mod


FIELDS = ("expert_id", "prob", "counts", "offsets", "perm", "inv_perm")


def _routing_pair(rom, w, top_k, permute):
    import torch
    inp = workloads.make_inputs(w, which={"X", "W_router"})
    X = parity.to_device(inp["X"], w.dtype)
    Wr = parity.to_device(inp["W_router"], "f32")
    ref = rom.route(X, Wr, top_k=top_k, permute=permute)
    got = rom.Routing(w.T, w.E, X.device, top_k=top_k)
    if permute:
        got.x_perm = torch.empty_like(X)
    rom.route_noalloc(X, Wr, got, permute=permute)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("top_k,permute", [(1, True), (2, False)])
def test_noalloc_matches_route_twice_second_smaller(rom, top_k, permute):
    # a large call (matrix-core router, many workgroups), then a smaller one on the same scratch
    for w in (workloads.custom_workload("noalloc_big", T=70000, d_model=1024, d_inner=64, E=8, seed=901),
              workloads.custom_workload("noalloc_small", T=3001, d_model=256, d_inner=64, E=5, seed=902)):
        print(f"[noalloc] {w.name} T={w.T} E={w.E} top_k={top_k} permute={permute}", flush=True)
        ref, got = _routing_pair(rom, w, top_k, permute)
        for f in FIELDS:
            np.testing.assert_array_equal(parity.to_host(getattr(got, f)), parity.to_host(getattr(ref, f)),
                                          err_msg=f"{w.name}: {f}")
        assert (got.struct.T, got.struct.E, got.struct.top_k) == (w.T, w.E, top_k)
        if permute:
            np.testing.assert_array_equal(parity.to_host(got.x_perm), parity.to_host(ref.x_perm))


def test_noalloc_rejects_beyond_its_scratch(rom):
    import torch
    L = rom.lib()
    T, E = 600000, 8
    assert L.rom_route_workspace_bytes(T, E) > (4 << 20)
    X = torch.zeros((T, 64), dtype=torch.bfloat16, device="cuda")
    Wr = torch.zeros((64, E), dtype=torch.float32, device="cuda")
    r = rom.Routing(T, E, "cuda")
    st = L.rom_route_noalloc(X.data_ptr(), rom.ROM_DTYPE_BF16, T, 64, Wr.data_ptr(), None, E, 1,
                             ctypes.byref(r.struct), None, None)
    assert st == rom.ROM_ERR_UNSUPPORTED
    assert b"static scratch" in L.rom_last_error()
