"""Parity helpers: run the HIP path through the C ABI and compare it with the CPU oracle.

Comparison rules (from the stated tolerances of the workloads):
  * expert ids match bit for bit, except on tokens whose oracle top-1/top-2 logit margin is below 1e-4:
    those are reported and excluded from the id check, and their outputs are compared only when the two
    sides happen to agree on the id;
  * the grouping (counts, offsets, perm, inv_perm) is fully determined by the ids: when every id agrees
    it must equal the oracle's bit for bit; otherwise it must be the valid stable grouping of the GPU's
    own ids (checked with numpy's bincount and stable argsort);
  * router probabilities (fp32 on both sides): per token, |p_gpu - p_oracle| / p_oracle within the fp32
    bound of router_prob_rtol (Higham's dot-product bound on both sides' logits, carried through the
    softmax);
  * floating-point outputs: normalised max error max|g - r| / max|r| over the compared tokens, at most
    1e-5 for fp32 data and 2e-2 for bf16 data (bf16 inputs, fp32 accumulation). The 99.9th percentile of
    the elementwise relative error |g - r| / |r| (over the nonzero reference entries) is recorded beside it
    for every compared tensor and printed in the session summary; it does not gate.
No value produced by the HIP path is ever fed to the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

import workloads

GAP_EXCLUDE = 1e-4
TOL = {"f32": 1e-5, "bf16": 2e-2}
U32 = 2.0 ** -24  # unit roundoff of fp32

# (label, tensor, normalised max error, 99.9th-percentile elementwise relative error, elements) of every
# comparison in the session; conftest prints them at the end
REPORT = []
_LABEL = [""]


def begin(label: str):
    """Label the comparisons that follow in the session report."""
    _LABEL[0] = label


def write_report(path: str):
    import json
    with open(path, "w") as f:
        json.dump([dict(label=a, tensor=b, norm_max_err=c, rel_err_p999=d, n=e) for a, b, c, d, e in REPORT], f,
                  indent=1)


def torch_mod():
    import torch
    return torch


def to_device(a: Optional[np.ndarray], dtype: str, device="cuda"):
    """float32 numpy -> device tensor holding the same bits (bf16 arrays must be bf16-representable)."""
    torch = torch_mod()
    if a is None:
        return None
    if dtype == "bf16":
        bits = workloads.bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits.copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def norm_max_err(g: np.ndarray, r: np.ndarray, name: Optional[str] = None) -> float:
    """max|g - r| / max|r|; with a name, the comparison (and its 99.9th-percentile elementwise relative
    error) goes into the session report."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    den = np.max(np.abs(r))
    num = np.max(np.abs(g - r))
    err = float(num / den) if den > 0 else float(num)
    if name is not None:
        nz = r != 0
        rel = np.abs(g[nz] - r[nz]) / np.abs(r[nz])
        p999 = float(np.percentile(rel, 99.9)) if rel.size else 0.0
        REPORT.append((_LABEL[0], name, err, p999, int(r.size)))
    return err


def gamma(n: int) -> float:
    """Higham's gamma_n = n u / (1 - n u) for fp32."""
    return n * U32 / (1.0 - n * U32)


def router_prob_rtol(X, W_router, bias, logits) -> np.ndarray:
    """Per-token bound on |p_gpu - p_oracle| / p_oracle for router probabilities computed in fp32 by both
    sides from the same bits.

    Each side's fp32 logits lie within gamma_n * (sum_k |x_k w_kj| + |b_j|) of the exact ones (Higham's
    dot-product bound; n = d_model + 1 for the oracle's ascending sum and for the VALU kernels, 3 d_model + 1
    for the matrix-core kernel, which adds the exact products of three bf16 parts of every weight). A shift
    delta of the logits moves p_e = exp(l_e - l_max) / sum_j exp(l_j - l_max) by a relative amount of at most
    2 max|delta| to first order (2.05 covers the second order). The GPU's fp32 softmax adds the rounding of
    the differences l_j - l_max (relative u, i.e. u |l_j - l_max| in each exponent), of E exponentials
    (<= 2 ulp each), of their sum and of the division; the oracle's double-precision softmax adds less."""
    X64 = np.abs(np.asarray(X, np.float64))
    W64 = np.abs(np.asarray(W_router, np.float64))
    absum = X64 @ W64
    if bias is not None:
        absum = absum + np.abs(np.asarray(bias, np.float64))
    dm, E = W64.shape
    beta = (gamma(dm + 1) + gamma(3 * dm + 1)) * absum.max(axis=1)
    lg = np.asarray(logits, np.float64)
    spread = lg.max(axis=1) - lg.min(axis=1)
    return 2.05 * beta + (3 * E + 8) * U32 + 2 * U32 * spread


@dataclasses.dataclass
class RouteReport:
    n_excluded: int
    n_id_mismatch_excluded: int
    ids_agree_everywhere: bool
    prob_err: float


def check_route(gpu, orc_route, orc_sort, T, E, prob_rtol) -> RouteReport:
    """gpu: dict of numpy arrays expert_id, prob, counts, offsets, perm, inv_perm; prob_rtol: the per-token
    relative bound of router_prob_rtol."""
    ids_o = orc_route["ids"][:, 0]
    gap = orc_route["gap"]
    excl = gap < GAP_EXCLUDE
    ids_g = gpu["expert_id"]
    assert ids_g.shape == (T,)
    assert np.all((ids_g >= 0) & (ids_g < E)), "expert id out of range"
    bad = (ids_g != ids_o) & ~excl
    assert not np.any(bad), f"{int(bad.sum())} expert ids differ on decided tokens, first at {np.flatnonzero(bad)[:5]}"
    agree = ids_g == ids_o
    if np.all(agree):
        for k in ("counts", "offsets", "perm", "inv_perm"):
            np.testing.assert_array_equal(gpu[k], orc_sort[k], err_msg=f"grouping array {k}")
    else:
        cnt = np.bincount(ids_g, minlength=E)
        np.testing.assert_array_equal(gpu["counts"], cnt)
        np.testing.assert_array_equal(gpu["offsets"], np.concatenate([[0], np.cumsum(cnt)]))
        np.testing.assert_array_equal(gpu["perm"], np.argsort(ids_g, kind="stable"))
        np.testing.assert_array_equal(gpu["inv_perm"][gpu["perm"]], np.arange(T))
    perr = check_prob(gpu["prob"][agree], orc_route["prob"][agree, 0], np.asarray(prob_rtol)[agree])
    return RouteReport(int(excl.sum()), int((~agree).sum()), bool(np.all(agree)), perr)


def check_prob(pg, po, rtol) -> float:
    """Elementwise relative check of router probabilities (rtol broadcast over trailing axes); returns the
    largest relative error."""
    pg = np.asarray(pg, np.float64)
    po = np.asarray(po, np.float64)
    if po.size == 0:
        return 0.0
    rt = np.asarray(rtol, np.float64)
    if pg.ndim == 2:
        rt = rt[:, None]
    rel = np.abs(pg - po) / po
    norm_max_err(pg, po, name="prob")
    bad = rel > rt
    assert not np.any(bad), (f"router probability off the fp32 bound on {int(bad.sum())} entries: worst relative "
                             f"error {float(rel.max()):.3g} (bound there {float(np.broadcast_to(rt, rel.shape)[np.unravel_index(np.argmax(rel / rt), rel.shape)]):.3g})")
    return float(rel.max())


def check_route_topk(gpu, orc_route, T, E, K, prob_rtol):
    """Top-K routing (K stacked top-1 routings on the GPU side, arrays [K][T]) against the oracle's
    ids/prob [T][K]. Returns the boolean mask of tokens whose expert set agrees with the oracle's.

    Sets must agree on every token whose oracle margin between the K-th and (K+1)-th logit is at least
    GAP_EXCLUDE; the order of the choices must agree where the oracle's margin between consecutive
    chosen logits is at least GAP_EXCLUDE too (computed from the oracle's own logits). Probabilities are
    compared expert by expert. Each choice's grouping must be the valid stable grouping of the GPU's own
    choice-k ids (numpy bincount / stable argsort). prob_rtol: the per-token bound of router_prob_rtol."""
    ids_g, prob_g = gpu["expert_id"], gpu["prob"]
    assert ids_g.shape == (K, T) and prob_g.shape == (K, T)
    assert np.all((ids_g >= 0) & (ids_g < E)), "expert id out of range"
    ids_o, prob_o = orc_route["ids"], orc_route["prob"]
    if K > 1:
        assert np.all(ids_g[0] != ids_g[1]), "a token chose the same expert twice"
    decided = orc_route["gap"] >= GAP_EXCLUDE
    same_set = np.all(np.sort(ids_g.T, axis=1) == np.sort(ids_o, axis=1), axis=1)
    bad = ~same_set & decided
    assert not np.any(bad), f"{int(bad.sum())} expert sets differ on decided tokens, first at {np.flatnonzero(bad)[:5]}"
    lg = orc_route["logits"]
    if lg is not None:
        chosen = np.take_along_axis(lg, ids_o.astype(np.int64), axis=1)  # [T][K], descending
        ordered = np.all(np.diff(-chosen, axis=1) >= GAP_EXCLUDE, axis=1) if K > 1 else np.ones(T, bool)
        mis = same_set & ordered & np.any(ids_g.T != ids_o, axis=1)
        assert not np.any(mis), f"{int(mis.sum())} tokens have their choices in another order"
    # probabilities paired by expert on the agreeing tokens
    rows = np.flatnonzero(same_set)
    if rows.size:
        order_g = np.argsort(ids_g.T[rows], axis=1)
        order_o = np.argsort(ids_o[rows], axis=1)
        pg = np.take_along_axis(prob_g.T[rows], order_g, axis=1)
        po = np.take_along_axis(prob_o[rows], order_o, axis=1)
        check_prob(pg, po, np.asarray(prob_rtol)[rows])
    for k in range(K):
        cnt = np.bincount(ids_g[k], minlength=E)
        np.testing.assert_array_equal(gpu["counts"][k], cnt, err_msg=f"counts of choice {k}")
        np.testing.assert_array_equal(gpu["offsets"][k], np.concatenate([[0], np.cumsum(cnt)]))
        np.testing.assert_array_equal(gpu["perm"][k], np.argsort(ids_g[k], kind="stable"))
        np.testing.assert_array_equal(gpu["inv_perm"][k][gpu["perm"][k]], np.arange(T))
    return same_set


def gemm_row_tiles(T: int, N0: int, nB: int, E: int, dtype: str, cus: int = 256):
    """(rows per M-tile, rows per epilogue band) of the grouped GEMM that the library launches for T tokens,
    N0 output columns per weight stack, nB stacks and E experts, or None for the decode kernels (T <= 64).

    Mirrors the launcher's tile choice: bf16 with T >= 4096 and N0 a multiple of 256 takes 320-row tiles
    (written back in two 160-row passes) when their padded-row bound T + E*319 is at most 5% above the
    256-row one or they need fewer rounds over the compute units, else 256-row tiles (one pass, wave bands of
    128 rows); smaller problems take 128-row tiles (wave bands of 64); fp32 data takes 64-row tiles."""
    if dtype != "bf16":
        return (64, 32)
    if T <= 64:
        return None
    if T >= 4096 and N0 % 256 == 0:
        nt = nB * (N0 // 256)
        rows256, rows320 = T + E * 255, T + E * 319
        t256, t320 = rows256 // 256 * nt, rows320 // 320 * nt
        r256, r320 = -(-t256 // cus), -(-t320 // cus)
        if rows320 * 20 <= rows256 * 21 or r320 * 320 < r256 * 256:
            return (320, 160)
        return (256, 128)
    return (128, 64)


WIDE_KC = 512        # K values per staged chunk of the wide decode kernel
WIDE_MIN_T = 17      # fewest tokens for which the launcher considers the wide decode kernel


def wide_kq(T: int, E: int, N0: int, K: int, nB: int, cus: int = 256, min_t: int = WIDE_MIN_T) -> int:
    """Waves per 16-row block (1, 2 or 4; rows per workgroup 256 / kq) of the wide decode kernel that the
    library launches for T tokens, N0 output rows per weight stack, nB stacks, K inputs and E experts, or 0
    when it takes another kernel. Mirrors the launcher: T in [min_t, 64], K a multiple of the chunk, and the
    fewest waves per row block whose workgroups (one per 256 / kq rows of every active expert) cover the
    compute units."""
    if T < min_t or T > 64 or K % WIDE_KC:
        return 0
    active = min(T, E)
    for kq in (1, 2, 4):
        rows = 256 // kq
        if N0 % rows == 0 and nB * N0 // rows * active >= cus:
            return kq
    return 0


def sample_rows(orc_sorts, T, tiles=((64, 32), (128, 64), (256, 128)), n_random=192, seed=0) -> np.ndarray:
    """Tokens to check at full size: for every routing choice (one oracle grouping per choice), the first two
    and last two slots of every expert group and of every M-tile the GEMMs launch in it, the slots on both
    sides of every epilogue band boundary inside those tiles, and a seeded random sample.

    orc_sorts: one oracle sort (dict with perm, offsets) or a list of them, one per choice; tiles: the
    (rows per tile, rows per band) pairs of the launched GEMMs (gemm_row_tiles), None entries skipped."""
    rng = np.random.default_rng(seed)
    if isinstance(orc_sorts, dict):
        orc_sorts = [orc_sorts]
    rows = set()
    for srt in orc_sorts:
        perm, off = srt["perm"], srt["offsets"]
        slots = set()
        for e in range(len(off) - 1):
            a, b = int(off[e]), int(off[e + 1])
            if b <= a:
                continue
            cand = [a, a + 1, b - 2, b - 1]
            for tile in tiles:
                if tile is None:
                    continue
                bm, band = tile
                for s0 in range(a, b, bm):
                    cand += [s0, s0 + 1, s0 + bm - 2, s0 + bm - 1]
                    for q in range(band, bm, band):
                        cand += [s0 + q - 1, s0 + q]
            slots.update(s for s in cand if a <= s < b)
        rows |= {int(perm[s]) for s in slots}
    rows |= set(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
