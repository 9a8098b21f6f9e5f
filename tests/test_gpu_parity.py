"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same seeded inputs.

Small shapes compare every token; the full workload shapes compare sampled tokens (the first and last
slots of every expert group, slots around M-tile boundaries, and a seeded random sample), with routing
and grouping compared for every token.
"""
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
    rom_mod.lib()  # raises if the HIP library is not built: there is no fallback
    return rom_mod


def _run_chain(rom, w, inp, permute=False, isolated=True, top_k=1):
    import torch
    d = lambda k: parity.to_device(inp[k], w.dtype) if k != "W_router" else parity.to_device(inp[k], "f32")
    X, Wr, Wc, Wg, Wo, h = d("X"), d("W_router"), d("W_conv"), d("W_gate"), d("W_out"), d("h")
    bias = parity.to_device(inp["bias"], "f32") if inp.get("bias") is not None else None
    r = rom.route(X, Wr, bias, top_k=top_k, permute=permute)
    x, z = rom.in_proj(X, r, Wc, Wg)
    out = rom.out_proj(z, h, r, Wo)
    out_iso = None
    if isolated and inp.get("z") is not None:
        out_iso = rom.out_proj(parity.to_device(inp["z"], w.dtype), h, r, Wo)
    torch.cuda.synchronize()
    return dict(r=r, X=X, x=x, z=z, out=out, out_iso=out_iso)


def _route_host(r, squeeze=True):
    """Routing buffers on the host; for top-1 (squeeze) the [1][...] arrays become flat."""
    out = {k: parity.to_host(getattr(r, k)) for k in ("expert_id", "prob", "counts", "offsets", "perm", "inv_perm")}
    if squeeze and r.top_k == 1:
        out = {k: v[0] for k, v in out.items()}
    return out


def _rows(t, rows):
    import torch
    idx = torch.as_tensor(rows, dtype=torch.long, device=t.device)
    return parity.to_host(t.index_select(0, idx))


def _prob_rtol(inp, o_route):
    """Per-token fp32 bound on the router probability's relative error (both sides compute in fp32)."""
    return parity.router_prob_rtol(inp["X"], inp["W_router"], inp.get("bias"), o_route["logits"])


def _fwd_tiles(w, top_k=1):
    """Row tiles of the in-projection (Conv + Gate stacks) and out-projection GEMMs the library launches."""
    return [parity.gemm_row_tiles(w.T, w.d_inner, 2, w.E, w.dtype), parity.gemm_row_tiles(w.T, w.d_model, 1, w.E, w.dtype)]


def _choice_sorts(orc, ids, E):
    """The oracle's grouping of every routing choice (column k of ids [T][K])."""
    return [orc.sort(np.ascontiguousarray(ids[:, k:k + 1]), E) for k in range(ids.shape[1])]


def check_workload(rom, orc, w, inp=None, rows=None, label=""):
    """Full comparison of one workload; rows=None compares every token."""
    inp = inp if inp is not None else workloads.make_inputs(w)
    tol = parity.TOL[w.dtype]
    print(f"[parity] {label or w.name}: T={w.T} d_model={w.d_model} d_inner={w.d_inner} E={w.E} {w.dtype}",
          flush=True)
    parity.begin(label or w.name)
    g = _run_chain(rom, w, inp)
    gr = _route_host(g["r"])
    o_route = orc.route(inp["X"], inp["W_router"], inp.get("bias"), want_logits=True)
    o_sort = orc.sort(o_route["ids"], w.E)
    rep = parity.check_route(gr, o_route, o_sort, w.T, w.E, _prob_rtol(inp, o_route))
    if rows is None:
        rows = np.arange(w.T)
    ids_o = o_route["ids"][:, 0]
    agree = gr["expert_id"][rows] == ids_o[rows]
    rows = rows[agree]
    x_o, z_o = orc.in_proj(inp["X"][rows], o_route["ids"][rows], inp["W_conv"], inp["W_gate"])
    ex = parity.norm_max_err(_rows(g["x"], rows), x_o, "x")
    ez = parity.norm_max_err(_rows(g["z"], rows), z_o, "z")
    out_o = orc.out_proj(z_o, inp["h"][rows], o_route["ids"][rows], o_route["prob"][rows], inp["W_out"])
    eo = parity.norm_max_err(_rows(g["out"], rows), out_o, "out")
    ei = 0.0
    if g["out_iso"] is not None:
        out_i = orc.out_proj(inp["z"][rows].astype(np.float64), inp["h"][rows], o_route["ids"][rows],
                             o_route["prob"][rows], inp["W_out"])
        ei = parity.norm_max_err(_rows(g["out_iso"], rows), out_i, "out_isolated")
    print(f"[parity]   excluded(gap<1e-4)={rep.n_excluded} id-mismatch={rep.n_id_mismatch_excluded} "
          f"prob={rep.prob_err:.2e} x={ex:.2e} z={ez:.2e} out={eo:.2e} out_isolated={ei:.2e} rows={len(rows)}",
          flush=True)
    for name, err in (("x", ex), ("z", ez), ("out", eo), ("out_isolated", ei)):
        assert err <= tol, f"{name}: normalised max error {err:.3g} > {tol}"
    return g, gr, o_route, o_sort


# ------------------------------------------------------------------------------------------------
# small shapes: every token

SMALL = [
    workloads.get_workload("tiny_f32"),
    workloads.custom_workload("bf16_tiles", T=1000, d_model=256, d_inner=384, E=8, seed=101),
    workloads.custom_workload("bf16_bn64_E3", T=777, d_model=192, d_inner=320, E=3, seed=102),
    workloads.custom_workload("bf16_E1_dense", T=300, d_model=128, d_inner=256, E=1, seed=103),
    workloads.custom_workload("bf16_T1", T=1, d_model=256, d_inner=256, E=8, seed=104),
    workloads.custom_workload("bf16_T127", T=127, d_model=128, d_inner=128, E=8, seed=105),
    workloads.custom_workload("bf16_T129", T=129, d_model=128, d_inner=128, E=8, seed=106),
    workloads.custom_workload("bf16_T256_small_route", T=256, d_model=256, d_inner=128, E=8, seed=107),
    workloads.custom_workload("bf16_T257_multi_wg_route", T=257, d_model=256, d_inner=128, E=8, seed=108),
    workloads.custom_workload("bf16_E64", T=3000, d_model=128, d_inner=128, E=64, seed=109),
    workloads.custom_workload("bf16_E16_T2000", T=2000, d_model=320, d_inner=192, E=16, seed=110),
    workloads.custom_workload("bf16_T5_fused_route", T=5, d_model=512, d_inner=128, E=8, seed=113),
    workloads.custom_workload("bf16_T9_split_route", T=9, d_model=512, d_inner=128, E=4, seed=114),
    workloads.custom_workload("bf16_wide_route_E64", T=16400, d_model=128, d_inner=128, E=64, seed=115),
    workloads.custom_workload("bf16_wide_route_E3", T=16421, d_model=192, d_inner=128, E=3, seed=116),
    # wide router on the matrix cores (bf16, 8 experts): a ragged last workgroup, d_model 512 (no ring
    # refills) and 1536 (ring refilled)
    workloads.custom_workload("bf16_wide_mfma_dm512", T=16400, d_model=512, d_inner=128, E=8, seed=118),
    workloads.custom_workload("bf16_wide_mfma_dm1536", T=16390, d_model=1536, d_inner=128, E=8, seed=119),
    # wide router with W_r in LDS and fp32 rows: 144 chunks per row, so every lane has a second chunk in
    # flight at the barrier and some refill a third time
    workloads.custom_workload("f32_wide_route_dm1152", T=16400, d_model=1152, d_inner=128, E=8, dtype="f32", seed=117),
    # 320-row tiles with 160-row epilogue passes (the tile of every full-size workload), every token: few experts
    # keep the padding of 320-row tiles within 5% of 256-row ones at T = 4096; a ragged last tile
    workloads.custom_workload("bf16_tiles320_T4096_E2", T=4096, d_model=256, d_inner=256, E=2, seed=130),
    workloads.custom_workload("bf16_tiles320_T4100_E3", T=4100, d_model=512, d_inner=256, E=3, seed=131),
    # many router workgroups: the scatter reads per-workgroup bases from the prefix-scan kernel (8-token router
    # workgroups with 64 experts; 32-token workgroups at 300K tokens) instead of summing the partial histograms
    workloads.custom_workload("bf16_E64_T12000_prescan", T=12000, d_model=128, d_inner=64, E=64, seed=132),
    workloads.custom_workload("bf16_T300000_prescan", T=300000, d_model=64, d_inner=64, E=8, seed=133),
    workloads.custom_workload("f32_E5", T=333, d_model=128, d_inner=192, E=5, dtype="f32", seed=111),
    workloads.custom_workload("f32_T1000_E8", T=1000, d_model=64, d_inner=128, E=8, dtype="f32", seed=112),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_small_shapes(rom, oracle, w):
    if "tiles320" in w.name:
        assert all(t[0] == 320 for t in _fwd_tiles(w)), "the case no longer selects 320-row tiles"
    check_workload(rom, oracle, w)


def test_all_tokens_on_one_expert(rom, oracle):
    w = workloads.custom_workload("one_expert", T=900, d_model=128, d_inner=256, E=8, seed=120)
    bias = np.zeros(8, np.float32)
    bias[5] = 1e3
    inp = workloads.make_inputs(w, router_bias=bias)
    _, gr, _, _ = check_workload(rom, oracle, w, inp, label="all tokens on expert 5")
    assert gr["counts"][5] == w.T


# The wide decode GEMV (17..64 tokens, 64- to 256-row workgroups of 16 waves, token rows staged through LDS in
# chunks of 512 to 2048 values): every token compared. Each case names the waves per 16-row block (K split 1, 2
# or 4 ways) that its in- and out-projection take (0: another kernel), checked against the launcher's rule: one
# and several chunks, one to four token blocks, top-1 and top-2 (the second choice adds to the first), the
# out-projection (on the gated rows) with K split 2 and 4 ways.
WIDE = [
    # name, T, d_model, d_inner, E, seed, top_k, (in kq, out kq)
    ("wide_T32_E8", 32, 1024, 4096, 8, 140, 1, (1, 0)),
    ("wide_T50_E8", 50, 1024, 4096, 8, 141, 1, (1, 0)),
    ("wide_T32_E8_top2", 32, 512, 4096, 8, 142, 2, (1, 0)),
    ("wide_kq4_T40", 40, 2048, 1024, 8, 143, 1, (4, 4)),
    ("wide_kq4_T40_top2", 40, 2048, 1024, 8, 144, 2, (4, 4)),
    ("wide_kq2_out_T20_one_chunk", 20, 4096, 512, 8, 145, 1, (0, 2)),
    ("wide_kq2_T24", 24, 1024, 2048, 8, 146, 1, (2, 0)),
]


@pytest.mark.parametrize("case", WIDE, ids=[c[0] for c in WIDE])
def test_decode_wide_gemv(rom, oracle, case):
    name, T, dm, di, E, seed, k, (kq_in, kq_out) = case
    assert parity.wide_kq(T, E, di, dm, 2) == kq_in and parity.wide_kq(T, E, dm, di, 1) == kq_out, \
        "the case no longer selects the intended wide-kernel variant"
    w = workloads.custom_workload(name, T=T, d_model=dm, d_inner=di, E=E, seed=seed)
    if k == 1:
        check_workload(rom, oracle, w)
    else:
        check_workload_top2(rom, oracle, w)


WIDE_HOT_BIAS = 1.5  # with seed 147: 42 of the 64 tokens on expert 6, every expert active (oracle router)


def test_decode_wide_gemv_full_expert(rom, oracle):
    """Wide kernel (K split 4 ways) with one expert holding 33..64 tokens (three token blocks) while all eight
    experts stay active."""
    w = workloads.custom_workload("wide_kq4_hot_T64", T=64, d_model=2048, d_inner=1024, E=8, seed=147)
    assert parity.wide_kq(64, 8, 1024, 2048, 2) == 4 and parity.wide_kq(64, 8, 2048, 1024, 1) == 4
    bias = np.zeros(8, np.float32)
    bias[6] = WIDE_HOT_BIAS
    inp = workloads.make_inputs(w, router_bias=bias)
    _, gr, _, _ = check_workload(rom, oracle, w, inp, label="wide kernel, expert 6 hot")
    assert gr["counts"][6] > 32 and np.all(gr["counts"] > 0)


@pytest.mark.parametrize("T,hot", [(40, 1), (64, 3), (64, None)])
def test_decode_token_blocks(rom, oracle, T, hot):
    """Decode kernels: an expert holding 33..64 tokens takes the 3- and 4-block variants."""
    w = workloads.custom_workload(f"decode_blocks_T{T}", T=T, d_model=256, d_inner=320, E=4, seed=124 + T)
    bias = np.zeros(4, np.float32)
    if hot is not None:
        bias[hot] = 1e3
    inp = workloads.make_inputs(w, router_bias=bias)
    _, gr, _, _ = check_workload(rom, oracle, w, inp, label=f"decode blocks T={T} hot={hot}")
    if hot is not None:
        assert gr["counts"][hot] == T


def test_empty_experts(rom, oracle):
    w = workloads.custom_workload("empty_experts", T=700, d_model=128, d_inner=128, E=8, seed=121)
    bias = np.zeros(8, np.float32)
    bias[[0, 2, 7]] = -1e3
    inp = workloads.make_inputs(w, router_bias=bias)
    _, gr, _, _ = check_workload(rom, oracle, w, inp, label="experts 0, 2, 7 empty")
    assert gr["counts"][0] == gr["counts"][2] == gr["counts"][7] == 0


TIES = [
    workloads.custom_workload("ties", T=500, d_model=128, d_inner=128, E=8, seed=122),
    workloads.custom_workload("ties_wide_mfma", T=16400, d_model=512, d_inner=128, E=8, seed=160),
]


@pytest.mark.parametrize("w", TIES, ids=[w.name for w in TIES])
def test_tied_logits_lowest_index_and_exact_prob(rom, oracle, w):
    """W_router = 0: every logit ties; both sides pick expert 0 and p = 1/E exactly."""
    inp = workloads.make_inputs(w)
    inp["W_router"] = np.zeros_like(inp["W_router"])
    g = _run_chain(rom, w, inp, isolated=False)
    gr = _route_host(g["r"])
    assert np.all(gr["expert_id"] == 0) and np.all(gr["prob"] == np.float32(0.125))
    np.testing.assert_array_equal(gr["perm"], np.arange(w.T))
    g2 = _run_chain(rom, w, inp, isolated=False, top_k=2)
    gr2 = _route_host(g2["r"])
    assert np.all(gr2["expert_id"][0] == 0) and np.all(gr2["expert_id"][1] == 1)
    assert np.all(gr2["prob"] == np.float32(0.125))


def test_deterministic_and_permute(rom, oracle):
    """Two runs are bit-identical; the materialised permute is X[perm] exactly."""
    w = workloads.custom_workload("determinism", T=3000, d_model=256, d_inner=256, E=8, seed=123)
    inp = workloads.make_inputs(w)
    a = _run_chain(rom, w, inp, permute=True, isolated=False)
    b = _run_chain(rom, w, inp, permute=True, isolated=False)
    for k in ("x", "z", "out"):
        np.testing.assert_array_equal(parity.to_host(a[k]), parity.to_host(b[k]))
    for k in ("expert_id", "prob", "perm", "inv_perm"):
        np.testing.assert_array_equal(parity.to_host(getattr(a["r"], k)), parity.to_host(getattr(b["r"], k)))
    a2 = _run_chain(rom, w, inp, isolated=False, top_k=2)
    b2 = _run_chain(rom, w, inp, isolated=False, top_k=2)
    for k in ("x", "z", "out"):
        np.testing.assert_array_equal(parity.to_host(a2[k]), parity.to_host(b2[k]))
    perm = parity.to_host(a["r"].perm)[0]
    np.testing.assert_array_equal(parity.to_host(a["r"].x_perm), inp["X"][perm])
    o_route = oracle.route(inp["X"], inp["W_router"])
    o_sort = oracle.sort(o_route["ids"], w.E)
    if np.array_equal(parity.to_host(a["r"].expert_id)[0], o_route["ids"][:, 0]):
        np.testing.assert_array_equal(parity.to_host(a["r"].x_perm), oracle.permute(inp["X"], o_sort["perm"]))


# The one- and two-token router (bf16, at most 8 experts: one workgroup, a butterfly over the lanes): top-1 and
# top-2, d_model below and above one chunk per thread (64, 8192), E not a multiple of 4 (scalar W_r loads), one
# expert, a router bias, the materialised permute, and exact ties.
TINY_ROUTE = [
    # name, T, d_model, d_inner, E, seed, top_k
    ("tiny_T2_E8", 2, 512, 256, 8, 180, 1),
    ("tiny_T2_E8_dm8192_top2", 2, 8192, 128, 8, 181, 2),
    ("tiny_T1_E6_top2", 1, 1024, 192, 6, 182, 2),
    ("tiny_T2_E3_dm64", 2, 64, 64, 3, 183, 1),
    ("tiny_T1_E1", 1, 256, 128, 1, 184, 1),
    # one token with K a multiple of 512 for the in- and the out-projection: the one-token dot-product GEMV,
    # top-1 and top-2 (the second choice added onto the first), K from 512 to its largest, 16384
    ("one_token_dm512_di1024", 1, 512, 1024, 4, 186, 1),
    ("one_token_dm1536_di512_top2", 1, 1536, 512, 8, 187, 2),
    ("one_token_dm16384_di512", 1, 16384, 512, 4, 188, 1),
    ("one_token_dm512_di16384_top2", 1, 512, 16384, 4, 189, 2),
    # the decode GEMVs' weight-load rings with a rotated start where a wave's K steps are not a multiple of the
    # ring: the gated out-projection's 3 steps per wave (ring of 2), the in-projection's 10 (ring of 8)
    ("one_token_odd_ring", 1, 512, 1536, 4, 190, 1),
    ("two_token_ring_partial", 2, 2560, 4096, 4, 191, 1),
]


@pytest.mark.parametrize("case", TINY_ROUTE, ids=[c[0] for c in TINY_ROUTE])
def test_tiny_router(rom, oracle, case):
    name, T, dm, di, E, seed, k = case
    w = workloads.custom_workload(name, T=T, d_model=dm, d_inner=di, E=E, seed=seed)
    if k == 1:
        _, gr, _, _ = check_workload(rom, oracle, w)
        if E == 1:
            assert np.all(gr["prob"] == 1.0)
    else:
        check_workload_top2(rom, oracle, w)


def test_tiny_router_bias_permute_and_ties(rom, oracle):
    """Two tokens: a bias that moves the choice, the permute (X[perm] exactly), and W_router = 0 (expert 0,
    p = 1/E exactly; top-2 picks experts 0 and 1)."""
    w = workloads.custom_workload("tiny_bias_T2", T=2, d_model=256, d_inner=128, E=8, seed=185)
    bias = np.zeros(8, np.float32)
    bias[5] = 50.0
    inp = workloads.make_inputs(w, router_bias=bias)
    _, gr, _, _ = check_workload(rom, oracle, w, inp, label="tiny router with bias")
    assert np.all(gr["expert_id"] == 5)
    g = _run_chain(rom, w, inp, permute=True, isolated=False)
    perm = parity.to_host(g["r"].perm)[0]
    np.testing.assert_array_equal(parity.to_host(g["r"].x_perm), inp["X"][perm])
    inp["W_router"] = np.zeros_like(inp["W_router"])
    inp["bias"] = None
    g = _run_chain(rom, w, inp, isolated=False)
    gr = _route_host(g["r"])
    assert np.all(gr["expert_id"] == 0) and np.all(gr["prob"] == np.float32(0.125))
    g2 = _run_chain(rom, w, inp, isolated=False, top_k=2)
    gr2 = _route_host(g2["r"])
    assert np.all(gr2["expert_id"][0] == 0) and np.all(gr2["expert_id"][1] == 1)


def test_zero_tokens(rom):
    import torch
    X = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    Wr = torch.zeros((128, 8), dtype=torch.float32, device="cuda")
    r = rom.route(X, Wr)
    W = torch.zeros((8, 128, 128), dtype=torch.bfloat16, device="cuda")
    x, z = rom.in_proj(X, r, W, W)
    out = rom.out_proj(z, z.clone(), r, W)
    torch.cuda.synchronize()
    assert x.shape == (0, 128) and out.shape == (0, 128)


# ------------------------------------------------------------------------------------------------
# full workload shapes: routing for every token, projections on sampled tokens

FULL = ["samba421m", "rom1p3b", "skewed", "decode_T1", "decode_T8", "decode_T64"]


@pytest.mark.parametrize("name", FULL)
def test_full_workload(rom, oracle, name):
    w = workloads.get_workload(name)
    inp = workloads.make_inputs(w, which={"X", "W_router", "W_conv", "W_gate", "W_out", "h", "z"}
                                if w.T <= 64 else {"X", "W_router", "W_conv", "W_gate", "W_out", "h"})
    o_route = oracle.route(inp["X"], inp["W_router"], inp.get("bias"))
    o_sort = oracle.sort(o_route["ids"], w.E)
    rows = parity.sample_rows(o_sort, w.T, tiles=_fwd_tiles(w)) if w.T > 64 else None
    _, gr, _, _ = check_workload(rom, oracle, w, inp, rows=rows)
    if w.skew is not None:
        frac = gr["counts"] / w.T
        assert np.max(np.abs(frac - np.array(w.skew))) <= 0.0025, f"skewed loads {frac}"


# ------------------------------------------------------------------------------------------------
# top-2 routing (the page's 8top2 setting): two stacked top-1 routings, choices added in order

def check_workload_top2(rom, orc, w, inp=None, rows=None, label=""):
    K = 2
    inp = inp if inp is not None else workloads.make_inputs(w)
    tol = parity.TOL[w.dtype]
    print(f"[parity top2] {label or w.name}: T={w.T} d_model={w.d_model} d_inner={w.d_inner} E={w.E} {w.dtype}",
          flush=True)
    parity.begin((label or w.name) + " top-2")
    g = _run_chain(rom, w, inp, top_k=K)
    gr = _route_host(g["r"], squeeze=False)
    o_route = orc.route(inp["X"], inp["W_router"], inp.get("bias"), top_k=K, want_logits=True)
    agree = parity.check_route_topk(gr, o_route, w.T, w.E, K, _prob_rtol(inp, o_route))
    rows = np.arange(w.T) if rows is None else rows
    rows = rows[agree[rows]]
    ids_o, prob_o = o_route["ids"][rows], o_route["prob"][rows]
    x_o, z_o = orc.in_proj(inp["X"][rows], ids_o, inp["W_conv"], inp["W_gate"])
    ex = parity.norm_max_err(_rows(g["x"], rows), x_o, "x")
    ez = parity.norm_max_err(_rows(g["z"], rows), z_o, "z")
    out_o = orc.out_proj(z_o, inp["h"][rows], ids_o, prob_o, inp["W_out"])
    eo = parity.norm_max_err(_rows(g["out"], rows), out_o, "out")
    ei = 0.0
    if g["out_iso"] is not None:
        out_i = orc.out_proj(inp["z"][rows].astype(np.float64), inp["h"][rows], ids_o, prob_o, inp["W_out"])
        ei = parity.norm_max_err(_rows(g["out_iso"], rows), out_i, "out_isolated")
    print(f"[parity top2]   set-mismatch={int((~agree).sum())} x={ex:.2e} z={ez:.2e} out={eo:.2e} "
          f"out_isolated={ei:.2e} rows={len(rows)}", flush=True)
    for name, err in (("x", ex), ("z", ez), ("out", eo), ("out_isolated", ei)):
        assert err <= tol, f"{name}: normalised max error {err:.3g} > {tol}"
    return g, gr, o_route


TOP2 = [
    workloads.custom_workload("top2_f32", T=300, d_model=64, d_inner=128, E=8, dtype="f32", seed=201),
    workloads.custom_workload("top2_bf16_tiles", T=1000, d_model=256, d_inner=384, E=8, seed=202),
    workloads.custom_workload("top2_bf16_E2", T=513, d_model=128, d_inner=256, E=2, seed=203),
    workloads.custom_workload("top2_bf16_E16", T=2000, d_model=320, d_inner=192, E=16, seed=204),
    workloads.custom_workload("top2_T5_fused_route", T=5, d_model=512, d_inner=128, E=8, seed=205),
    workloads.custom_workload("top2_T40_decode", T=40, d_model=256, d_inner=320, E=4, seed=206),
    workloads.custom_workload("top2_T64_decode", T=64, d_model=512, d_inner=256, E=8, seed=207),
    workloads.custom_workload("top2_wide_route", T=16400, d_model=128, d_inner=128, E=8, seed=208),
    workloads.custom_workload("top2_wide_mfma_dm1024", T=16400, d_model=1024, d_inner=128, E=8, seed=211),
    # 256-row early-barrier tiles (their padding rules out 320 rows here) with the fp32 accumulate epilogue
    workloads.custom_workload("top2_T4096_tiles256", T=4096, d_model=512, d_inner=512, E=8, seed=210),
    # 320-row tiles (two 160-row passes of the fp32 accumulate epilogue for the second choice), every token
    workloads.custom_workload("top2_tiles320_T4096_E2", T=4096, d_model=256, d_inner=256, E=2, seed=212),
    workloads.custom_workload("top2_tiles320_T4100_E3", T=4100, d_model=512, d_inner=256, E=3, seed=213),
]


@pytest.mark.parametrize("w", TOP2, ids=[w.name for w in TOP2])
def test_top2_small_shapes(rom, oracle, w):
    check_workload_top2(rom, oracle, w)


def _random_shapes(n, seed):
    """Seeded random shapes over the supported range: T, E (including odd and non-power-of-two counts), widths,
    top-1 or top-2, bf16 or fp32. Every token is compared."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        E = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 33, 64]))
        k = 2 if E >= 2 and rng.random() < 0.4 else 1
        T = int(rng.integers(1, 2500))
        dm, di = 64 * int(rng.integers(1, 9)), 64 * int(rng.integers(1, 9))
        dtype = "f32" if rng.random() < 0.2 else "bf16"
        name = f"rand{i}_T{T}_dm{dm}_di{di}_E{E}_top{k}_{dtype}"
        out.append((workloads.custom_workload(name, T=T, d_model=dm, d_inner=di, E=E, dtype=dtype, seed=700 + i), k))
    return out


RANDOM = _random_shapes(24, 2024)


@pytest.mark.parametrize("w,k", RANDOM, ids=[w.name for w, _ in RANDOM])
def test_random_shapes(rom, oracle, w, k):
    if k == 1:
        check_workload(rom, oracle, w)
    else:
        check_workload_top2(rom, oracle, w)


def test_top2_hot_expert(rom, oracle):
    """A dominant bias: every token's first choice is expert 3, the second spreads over the others."""
    w = workloads.custom_workload("top2_hot", T=700, d_model=128, d_inner=128, E=8, seed=209)
    bias = np.zeros(8, np.float32)
    bias[3] = 1e3
    _, gr, _ = check_workload_top2(rom, oracle, w, workloads.make_inputs(w, router_bias=bias), label="hot expert 3")
    assert np.all(gr["expert_id"][0] == 3) and np.all(gr["expert_id"][1] != 3)


def test_top2_full_samba_shape(rom, oracle):
    w = workloads.get_workload("samba421m")
    inp = workloads.make_inputs(w, which={"X", "W_router", "W_conv", "W_gate", "W_out", "h"})
    o_route = oracle.route(inp["X"], inp["W_router"], top_k=2)
    rows = parity.sample_rows(_choice_sorts(oracle, o_route["ids"], w.E), w.T, tiles=_fwd_tiles(w))
    check_workload_top2(rom, oracle, w, inp, rows=rows, label="samba421m top-2")


# ------------------------------------------------------------------------------------------------
# Swimba's routing-weighted in-projection: y = sum over the token's choices of p * W_in[e] X

def check_weighted(rom, orc, w, top_k=1, inp=None, rows=None, label=""):
    import torch
    inp = inp if inp is not None else workloads.make_inputs(w, which={"X", "W_router", "W_in"})
    tol = parity.TOL[w.dtype]
    print(f"[parity weighted] {label or w.name}: T={w.T} d_model={w.d_model} d_out={w.dout} E={w.E} "
          f"top_k={top_k} {w.dtype}", flush=True)
    X = parity.to_device(inp["X"], w.dtype)
    Wr = parity.to_device(inp["W_router"], "f32")
    W = parity.to_device(inp["W_in"], w.dtype)
    bias = parity.to_device(inp["bias"], "f32") if inp.get("bias") is not None else None
    parity.begin((label or w.name) + " weighted")
    r = rom.route(X, Wr, bias, top_k=top_k)
    y = rom.in_proj_weighted(X, r, W)
    torch.cuda.synchronize()
    gr = _route_host(r, squeeze=False)
    o_route = orc.route(inp["X"], inp["W_router"], inp.get("bias"), top_k=top_k, want_logits=True)
    agree = parity.check_route_topk(gr, o_route, w.T, w.E, top_k, _prob_rtol(inp, o_route))
    rows = np.arange(w.T) if rows is None else rows
    rows = rows[agree[rows]]
    y_o = orc.in_proj_weighted(inp["X"][rows], o_route["ids"][rows], o_route["prob"][rows], inp["W_in"])
    ey = parity.norm_max_err(_rows(y, rows), y_o, "y")
    print(f"[parity weighted]   set-mismatch={int((~agree).sum())} y={ey:.2e} rows={len(rows)}", flush=True)
    assert ey <= tol, f"y: normalised max error {ey:.3g} > {tol}"
    return gr


WEIGHTED = [
    (workloads.custom_workload("w_f32", T=300, d_model=64, d_inner=96, E=4, dtype="f32", seed=301), 1),
    (workloads.custom_workload("w_f32_top2", T=257, d_model=128, d_inner=64, E=4, dtype="f32", seed=302), 2),
    (workloads.custom_workload("w_bf16_bn256", T=1000, d_model=256, d_inner=128, E=4, seed=303), 1),
    (workloads.custom_workload("w_bf16_bn64_E3", T=777, d_model=192, d_inner=160, E=3, seed=304), 1),
    (workloads.custom_workload("w_bf16_T4096", T=4096, d_model=512, d_inner=512, E=4, seed=305), 1),
    (workloads.custom_workload("w_bf16_top2", T=513, d_model=128, d_inner=192, E=4, seed=306), 2),
    (workloads.custom_workload("w_T1", T=1, d_model=256, d_inner=160, E=4, seed=307), 1),
    (workloads.custom_workload("w_T5", T=5, d_model=512, d_inner=128, E=4, seed=308), 1),
    (workloads.custom_workload("w_T40", T=40, d_model=256, d_inner=160, E=4, seed=309), 1),
    (workloads.custom_workload("w_T64_top2", T=64, d_model=512, d_inner=256, E=4, seed=310), 2),
    (workloads.custom_workload("w_tiles320_T4096_E2", T=4096, d_model=256, d_inner=128, E=2, seed=311), 1),
    (workloads.custom_workload("w_tiles320_top2_T4100_E3", T=4100, d_model=256, d_inner=256, E=3, seed=313), 2),
    # the LDS-staged GEMV's ring of 4 with a rotated start over 5 K steps per wave
    (workloads.custom_workload("w_T3_ring_rotated", T=3, d_model=2560, d_inner=512, E=4, seed=314), 1),
]


@pytest.mark.parametrize("w,k", WEIGHTED, ids=[w.name for w, _ in WEIGHTED])
def test_weighted_in_proj_small_shapes(rom, oracle, w, k):
    check_weighted(rom, oracle, w, top_k=k)


def test_weighted_in_proj_one_expert_is_dense_scaled(rom, oracle):
    """E = 1: p = 1 exactly, so the output is the dense projection (the oracle's E=1 special case)."""
    w = workloads.custom_workload("w_E1", T=700, d_model=128, d_inner=128, E=1, seed=311)
    gr = check_weighted(rom, oracle, w)
    assert np.all(gr["prob"] == 1.0)


@pytest.mark.parametrize("name", ["swimba_decode_T1", "swimba_decode_T8", "swimba_decode_T64"])
def test_weighted_in_proj_swimba_decode(rom, oracle, name):
    check_weighted(rom, oracle, workloads.get_workload(name))


def test_weighted_in_proj_prefill_shape(rom, oracle):
    """A 16K-token prefill at d_model 1024, d_out 4096, 4 experts: sampled tokens."""
    w = workloads.custom_workload("w_prefill", T=16384, d_model=1024, d_inner=2048, E=4, seed=312)
    inp = workloads.make_inputs(w, which={"X", "W_router", "W_in"})
    o_route = oracle.route(inp["X"], inp["W_router"])
    rows = parity.sample_rows(oracle.sort(o_route["ids"], w.E), w.T,
                              tiles=[parity.gemm_row_tiles(w.T, w.dout, 1, w.E, w.dtype)])
    check_weighted(rom, oracle, w, inp=inp, rows=rows)


# ------------------------------------------------------------------------------------------------
# the shared short causal convolution after the in-projection

CONV = [
    # (n_seq, seq_len, channels, width, activation, bias, dtype)
    (2, 37, 64, 4, True, True, "f32"),
    (3, 100, 192, 4, True, True, "bf16"),
    (1, 1, 128, 4, True, True, "bf16"),
    (5, 15, 128, 4, False, False, "bf16"),
    (2, 16, 320, 3, True, False, "bf16"),
    (2, 17, 256, 2, False, True, "f32"),
    (4, 4096, 2048, 4, True, True, "bf16"),    # the Samba-421M-like block: 4 sequences of 4K, d_inner 2048
    (1, 16384, 4096, 4, True, True, "bf16"),   # the 1.3B-scale block: one 16K sequence, d_inner 4096
] + [(3, 50, 192, w, True, True, "bf16") for w in (1, 5, 6, 7, 8)]


@pytest.mark.parametrize("case", CONV, ids=[f"ns{c[0]}_L{c[1]}_C{c[2]}_w{c[3]}_{'silu' if c[4] else 'lin'}"
                                              f"{'_b' if c[5] else ''}_{c[6]}" for c in CONV])
def test_conv1d(rom, oracle, case):
    import torch
    ns, L, C, w, act, with_bias, dt = case
    print(f"[parity conv1d] n_seq={ns} seq_len={L} channels={C} width={w} act={act} bias={with_bias} {dt}",
          flush=True)
    inp = workloads.make_conv_inputs(ns, L, C, w, dt, seed=400 + w + L, with_bias=with_bias)
    x = parity.to_device(inp["x"].reshape(ns * L, C), dt)
    W = parity.to_device(inp["weight"], dt)
    b = parity.to_device(inp["bias"], dt) if with_bias else None
    y = rom.conv1d(x, W, b, n_seq=ns, activation=act)
    torch.cuda.synchronize()
    ref = oracle.conv1d(inp["x"], inp["weight"], inp["bias"], activation=act).reshape(ns * L, C)
    parity.begin(f"conv1d ns{ns} L{L} C{C} w{w} {dt}")
    err = parity.norm_max_err(parity.to_host(y), ref, "y")
    print(f"[parity conv1d]   y={err:.2e}", flush=True)
    assert err <= parity.TOL[dt], f"conv1d: normalised max error {err:.3g}"


# ------------------------------------------------------------------------------------------------
# backward of the routed projections (router probabilities held fixed)

def _entries(rng, E, R, C, n):
    return np.stack([rng.integers(0, E, n), rng.integers(0, R, n), rng.integers(0, C, n)], axis=1)


def check_backward(rom, orc, w, top_k=1, inp=None, rows=None, n_entries=None, label=""):
    """GPU out_proj_backward and in_proj_backward against the oracle. rows=None compares every token and the
    full weight gradients; otherwise the given tokens and n_entries sampled weight-gradient entries."""
    import torch
    inp = inp if inp is not None else workloads.make_inputs(w)
    gr_in = workloads.make_grad_inputs(w)
    tol = parity.TOL[w.dtype]
    print(f"[parity bwd] {label or w.name}: T={w.T} d_model={w.d_model} d_inner={w.d_inner} E={w.E} "
          f"top_k={top_k}", flush=True)
    d = lambda a: parity.to_device(a, w.dtype)
    X, z, h = d(inp["X"]), d(inp["z"]), d(inp["h"])
    Wc, Wg, Wo = d(inp["W_conv"]), d(inp["W_gate"]), d(inp["W_out"])
    g, dx, dzu = d(gr_in["d_out"]), d(gr_in["dx"]), d(gr_in["dz"])
    Wr = parity.to_device(inp["W_router"], "f32")
    bias = parity.to_device(inp["bias"], "f32") if inp.get("bias") is not None else None
    parity.begin((label or w.name) + f" backward top-{top_k}")
    r = rom.route(X, Wr, bias, top_k=top_k)
    dz, dh, dWo = rom.out_proj_backward(g, z, h, r, Wo)
    dX, dWc, dWg = rom.in_proj_backward(X, dx, dzu, r, Wc, Wg)
    torch.cuda.synchronize()
    gr = _route_host(r, squeeze=False)
    o_route = orc.route(inp["X"], inp["W_router"], inp.get("bias"), top_k=top_k, want_logits=True)
    agree = parity.check_route_topk(gr, o_route, w.T, w.E, top_k, _prob_rtol(inp, o_route))
    ids_o, prob_o = o_route["ids"], o_route["prob"]
    # weight gradients sum over all tokens: compare only experts untouched by a token whose expert set differs
    bad = set(np.unique(ids_o[~agree]).tolist()) | set(np.unique(gr["expert_id"][:, ~agree]).tolist())
    zf = inp["z"].astype(np.float64)
    full = rows is None
    rows = np.arange(w.T) if full else rows
    rows = rows[agree[rows]]
    dz_o, dh_o = orc.out_proj_dgrad(gr_in["d_out"][rows], zf[rows], inp["h"][rows], ids_o[rows], prob_o[rows],
                                    inp["W_out"])
    dX_o = orc.in_proj_dgrad(gr_in["dx"][rows], gr_in["dz"][rows], ids_o[rows], inp["W_conv"], inp["W_gate"])
    errs = {"dz": parity.norm_max_err(_rows(dz, rows), dz_o, "dz"),
            "dh": parity.norm_max_err(_rows(dh, rows), dh_o, "dh"),
            "dX": parity.norm_max_err(_rows(dX, rows), dX_o, "dX")}
    keep_e = np.array([e for e in range(w.E) if e not in bad], dtype=np.int64)
    if full:
        dWo_o = orc.out_proj_wgrad(gr_in["d_out"], zf, inp["h"], ids_o, prob_o, w.E)
        dWc_o, dWg_o = orc.in_proj_wgrad(inp["X"], gr_in["dx"], gr_in["dz"], ids_o, w.E)
        errs["dW_out"] = parity.norm_max_err(parity.to_host(dWo)[keep_e], dWo_o[keep_e], "dW_out")
        errs["dW_conv"] = parity.norm_max_err(parity.to_host(dWc)[keep_e], dWc_o[keep_e], "dW_conv")
        errs["dW_gate"] = parity.norm_max_err(parity.to_host(dWg)[keep_e], dWg_o[keep_e], "dW_gate")
        # an expert that received no token has an exactly zero gradient
        used = np.unique(ids_o)
        for e in range(w.E):
            if e not in used and e not in bad:
                assert not parity.to_host(dWo)[e].any() and not parity.to_host(dWc)[e].any()
    else:
        rng = np.random.default_rng(7)
        eo = _entries(rng, w.E, w.d_model, w.d_inner, n_entries)
        eo = eo[np.isin(eo[:, 0], keep_e)]
        ei = _entries(rng, w.E, w.d_inner, w.d_model, n_entries)
        ei = ei[np.isin(ei[:, 0], keep_e)]
        vo = orc.out_proj_wgrad_entries(gr_in["d_out"], zf, inp["h"], ids_o, prob_o, eo)
        vc, vg = orc.in_proj_wgrad_entries(inp["X"], gr_in["dx"], gr_in["dz"], ids_o, ei)
        # normalised by the largest magnitude of the whole GPU tensor (the oracle has only the samples)
        host = {k: parity.to_host(t) for k, t in (("o", dWo), ("c", dWc), ("g", dWg))}
        for name, key, ent, ref in (("dW_out", "o", eo, vo), ("dW_conv", "c", ei, vc), ("dW_gate", "g", ei, vg)):
            got = host[key][tuple(ent.T)]
            errs[name] = float(np.max(np.abs(got - ref)) / np.max(np.abs(host[key]))) if len(ent) else 0.0
    print("[parity bwd]   set-mismatch=%d rows=%d " % (int((~agree).sum()), len(rows))
          + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    for name, err in errs.items():
        assert err <= tol, f"{name}: normalised max error {err:.3g} > {tol}"
    return gr


BWD = [
    (workloads.custom_workload("bwd_T300", T=300, d_model=128, d_inner=256, E=4, seed=501), 1),
    (workloads.custom_workload("bwd_T1000_tiles128", T=1000, d_model=256, d_inner=384, E=8, seed=502), 1),
    (workloads.custom_workload("bwd_T777_tiles64", T=777, d_model=192, d_inner=320, E=3, seed=503), 1),
    (workloads.custom_workload("bwd_T5", T=5, d_model=256, d_inner=128, E=8, seed=504), 1),
    (workloads.custom_workload("bwd_top2_T513", T=513, d_model=128, d_inner=192, E=4, seed=505), 2),
    (workloads.custom_workload("bwd_top2_T64", T=64, d_model=256, d_inner=256, E=4, seed=506), 2),
    (workloads.custom_workload("bwd_top2_E16", T=2000, d_model=320, d_inner=192, E=16, seed=507), 2),
    (workloads.custom_workload("bwd_T4096_tiles256", T=4096, d_model=512, d_inner=512, E=8, seed=508), 1),
    (workloads.custom_workload("bwd_T4096_tiles320", T=4096, d_model=256, d_inner=256, E=2, seed=510), 1),
    (workloads.custom_workload("bwd_top2_T4100_tiles320", T=4100, d_model=512, d_inner=256, E=3, seed=511), 2),
]


@pytest.mark.parametrize("w,k", BWD, ids=[w.name for w, _ in BWD])
def test_backward_small_shapes(rom, oracle, w, k):
    check_backward(rom, oracle, w, top_k=k)


def test_backward_hot_expert(rom, oracle):
    """Every token on expert 2: the other experts' weight gradients are exactly zero."""
    w = workloads.custom_workload("bwd_hot", T=900, d_model=128, d_inner=256, E=8, seed=509)
    bias = np.zeros(8, np.float32)
    bias[2] = 1e3
    check_backward(rom, oracle, w, inp=workloads.make_inputs(w, router_bias=bias), label="all tokens on expert 2")


@pytest.mark.parametrize("top_k", [1, 2])
def test_backward_full_samba_shape(rom, oracle, top_k):
    w = workloads.get_workload("samba421m")
    inp = workloads.make_inputs(w)
    o_route = oracle.route(inp["X"], inp["W_router"], top_k=top_k)
    # data-gradient GEMMs: d(gated rows) over d_inner columns, dX over d_model columns
    tiles = [parity.gemm_row_tiles(w.T, w.d_inner, 1, w.E, w.dtype), parity.gemm_row_tiles(w.T, w.d_model, 1, w.E, w.dtype)]
    rows = parity.sample_rows(_choice_sorts(oracle, o_route["ids"], w.E), w.T, tiles=tiles, n_random=96)
    check_backward(rom, oracle, w, top_k=top_k, inp=inp, rows=rows, n_entries=600, label=f"samba421m top-{top_k}")


def test_backward_full_skewed_shape(rom, oracle):
    """The skewed block (T = 65536, d_model 2048, d_inner 4096, 60% of the tokens on expert 0) at its full size:
    sampled token rows at the tile boundaries of both data-gradient GEMMs, and sampled weight-gradient entries of
    every expert, expert 0's 613 K steps included."""
    w = workloads.get_workload("skewed")
    inp = workloads.make_inputs(w, which={"X", "W_router", "W_conv", "W_gate", "W_out", "h", "z"})
    o_route = oracle.route(inp["X"], inp["W_router"], inp.get("bias"))
    tiles = [parity.gemm_row_tiles(w.T, w.d_inner, 1, w.E, w.dtype), parity.gemm_row_tiles(w.T, w.d_model, 1, w.E, w.dtype)]
    rows = parity.sample_rows(_choice_sorts(oracle, o_route["ids"], w.E), w.T, tiles=tiles, n_random=64)
    check_backward(rom, oracle, w, inp=inp, rows=rows, n_entries=600, label="skewed top-1")
