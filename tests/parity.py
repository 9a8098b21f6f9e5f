"""Parity helpers: run the HIP path through the C ABI and compare it with the CPU oracle.

Comparison rules (from the stated tolerances of the workloads):
  * expert ids match bit for bit, except on tokens whose oracle top-1/top-2 logit margin is below 1e-4:
    those are reported and excluded from the id check, and their outputs are compared only when the two
    sides happen to agree on the id;
  * the grouping (counts, offsets, perm, inv_perm) is fully determined by the ids: when every id agrees
    it must equal the oracle's bit for bit; otherwise it must be the valid stable grouping of the GPU's
    own ids (checked with numpy's bincount and stable argsort);
  * floating-point outputs: normalised max error max|g - r| / max|r| over the compared tokens, at most
    1e-5 for fp32 data and 2e-2 for bf16 data (bf16 inputs, fp32 accumulation).
No value produced by the HIP path is ever fed to the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

import workloads

GAP_EXCLUDE = 1e-4
TOL = {"f32": 1e-5, "bf16": 2e-2}


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


def norm_max_err(g: np.ndarray, r: np.ndarray) -> float:
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    if r.size == 0:
        return 0.0
    den = np.max(np.abs(r))
    num = np.max(np.abs(g - r))
    return float(num / den) if den > 0 else float(num)


@dataclasses.dataclass
class RouteReport:
    n_excluded: int
    n_id_mismatch_excluded: int
    ids_agree_everywhere: bool
    prob_err: float


def check_route(gpu, orc_route, orc_sort, T, E, tol) -> RouteReport:
    """gpu: dict of numpy arrays expert_id, prob, counts, offsets, perm, inv_perm."""
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
    perr = norm_max_err(gpu["prob"][agree], orc_route["prob"][agree, 0])
    assert perr <= tol, f"router probability error {perr:.3g} > {tol}"
    return RouteReport(int(excl.sum()), int((~agree).sum()), bool(np.all(agree)), perr)


def check_route_topk(gpu, orc_route, T, E, K, tol):
    """Top-K routing (K stacked top-1 routings on the GPU side, arrays [K][T]) against the oracle's
    ids/prob [T][K]. Returns the boolean mask of tokens whose expert set agrees with the oracle's.

    Sets must agree on every token whose oracle margin between the K-th and (K+1)-th logit is at least
    GAP_EXCLUDE; the order of the choices must agree where the oracle's margin between consecutive
    chosen logits is at least GAP_EXCLUDE too (computed from the oracle's own logits). Probabilities are
    compared expert by expert. Each choice's grouping must be the valid stable grouping of the GPU's own
    choice-k ids (numpy bincount / stable argsort)."""
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
        perr = norm_max_err(pg, po)
        assert perr <= tol, f"router probability error {perr:.3g} > {tol}"
    for k in range(K):
        cnt = np.bincount(ids_g[k], minlength=E)
        np.testing.assert_array_equal(gpu["counts"][k], cnt, err_msg=f"counts of choice {k}")
        np.testing.assert_array_equal(gpu["offsets"][k], np.concatenate([[0], np.cumsum(cnt)]))
        np.testing.assert_array_equal(gpu["perm"][k], np.argsort(ids_g[k], kind="stable"))
        np.testing.assert_array_equal(gpu["inv_perm"][k][gpu["perm"][k]], np.arange(T))
    return same_set


def sample_rows(orc_sort, T, n_random=192, bm=(64, 128, 256), seed=0) -> np.ndarray:
    """Tokens to check at full size: the first and last slots of every expert group, slots around
    M-tile boundaries inside each group, and a seeded random sample."""
    rng = np.random.default_rng(seed)
    perm, off = orc_sort["perm"], orc_sort["offsets"]
    slots = set()
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b <= a:
            continue
        for s in (a, a + 1, b - 2, b - 1):
            if a <= s < b:
                slots.add(s)
        for m in bm:
            for k in range(1, 3):
                for s in (a + k * m - 1, a + k * m):
                    if a <= s < b:
                        slots.add(s)
    rows = {int(perm[s]) for s in slots}
    rows |= set(rng.choice(T, size=min(n_random, T), replace=False).tolist())
    return np.array(sorted(rows), dtype=np.int64)
