"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes a loaded oracle (the real one, or a mutant build with a planted
mistake) and raises AssertionError when the oracle disagrees with
  * a float64 per-token brute force (numpy matmul per token; no sorting, no grouping),
  * numpy library routines (bincount, stable argsort, a dense BLAS matmul) on the special cases
    that reduce to them (E=1 is a dense projection; identical experts make routing irrelevant),
  * closed forms (two-expert softmax is the logistic sigmoid of the logit margin; W_r = 0 gives
    p = 1/E; SiLU(v) - SiLU(-v) = v; h = 0 gives out = 0; the output is linear in p),
  * the hand-worked example in golden/handworked_tiny.json.
Method: Routing Mamba landing page (chapterpal.com), Knowl 1.
"""
from __future__ import annotations

import ast
import json
import math
import operator
import os

import numpy as np
from scipy.special import expit

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U32 = 2.0 ** -24  # unit roundoff of fp32


def _gamma(n: int) -> float:
    """Higham's gamma_n = n u / (1 - n u) for fp32."""
    return n * U32 / (1.0 - n * U32)


def _rand(rng, shape, std=1.0):
    return (rng.standard_normal(shape) * std).astype(np.float32)


def _topk_ref(l64: np.ndarray, K: int):
    """Reference top-K on float64 logits, lowest index on ties, plus the K-th/(K+1)-th margin."""
    T, E = l64.shape
    ids = np.zeros((T, K), np.int64)
    gap = np.full((T,), np.inf)
    for t in range(T):
        order = sorted(range(E), key=lambda j: (-l64[t, j], j))
        ids[t] = order[:K]
        if K < E:
            gap[t] = l64[t, order[K - 1]] - l64[t, order[K]]
    return ids, gap


# ------------------------------------------------------------------------------------------------
# router

def pin_router_bruteforce(orc):
    rng = np.random.default_rng(11)
    for (T, dm, E, K, with_bias) in [(64, 16, 8, 1, False), (64, 16, 8, 1, True), (40, 33, 3, 1, True),
                                     (50, 24, 8, 2, False), (30, 8, 2, 1, False), (20, 12, 5, 3, True)]:
        X = _rand(rng, (T, dm))
        Wr = _rand(rng, (dm, E), 1.0 / math.sqrt(dm))
        b = _rand(rng, (E,), 0.5) if with_bias else None
        r = orc.route(X, Wr, b, top_k=K, want_logits=True)
        X64, W64 = X.astype(np.float64), Wr.astype(np.float64)
        l64 = X64 @ W64 + (0.0 if b is None else b.astype(np.float64))
        # fp32 sum of dm products then one bias addition: Higham's bound gamma_{dm+1} sum |terms|
        absum = np.abs(X64) @ np.abs(W64) + (0.0 if b is None else np.abs(b.astype(np.float64)))
        bound = _gamma(dm + 1) * absum + 1e-30
        err = np.abs(r["logits"].astype(np.float64) - l64)
        assert np.all(err <= bound), f"router logits outside the fp32 dot-product bound ({err.max()})"
        beta = bound.max(axis=1)
        ids_ref, gap_ref = _topk_ref(l64, K)
        decided = gap_ref > 2 * beta
        assert np.array_equal(r["ids"][decided], ids_ref[decided]), "router top-K differs from brute force"
        # selected set must be a valid top-K under the fp32 logits for every token
        l32 = r["logits"]
        for t in range(T):
            sel = list(r["ids"][t])
            assert len(set(sel)) == K
            rest = [j for j in range(E) if j not in sel]
            if rest:
                assert min(l32[t, sel]) >= max(l32[t, rest])
        p64 = np.exp(l64 - l64.max(axis=1, keepdims=True))
        p64 /= p64.sum(axis=1, keepdims=True)
        for t in range(T):
            for s in range(K):
                ref = p64[t, r["ids"][t, s]]
                tol = ref * (2.05 * beta[t] + 4 * U32) + 1e-30
                assert abs(float(r["prob"][t, s]) - ref) <= tol, "router probability off the softmax"
        fin = np.isfinite(gap_ref)
        assert np.all(np.abs(r["gap"][fin] - gap_ref[fin]) <= 2 * beta[fin] + 4 * U32 * np.abs(gap_ref[fin]) + 1e-12)
        assert np.all(np.isinf(r["gap"][~fin]))


def pin_router_special(orc):
    rng = np.random.default_rng(12)
    X = _rand(rng, (37, 16))
    # E = 1: the only expert, probability exactly 1, no margin
    r = orc.route(X, _rand(rng, (16, 1)))
    assert np.all(r["ids"] == 0) and np.all(r["prob"] == 1.0) and np.all(np.isinf(r["gap"]))
    # W_r = 0: all logits tie -> lowest index (top-1 and top-2), p = 1/E exactly
    for E in (2, 4, 8):
        r = orc.route(X, np.zeros((16, E), np.float32))
        assert np.all(r["ids"] == 0) and np.all(r["prob"] == np.float32(1.0 / E)) and np.all(r["gap"] == 0)
    r = orc.route(X, np.zeros((16, 8), np.float32), top_k=2)
    assert np.all(r["ids"] == np.array([0, 1])) and np.all(r["prob"] == np.float32(0.125))
    # a dominant bias on expert j routes every token to j
    Wr = _rand(rng, (16, 8), 0.25)
    for j in (0, 3, 7):
        b = np.zeros(8, np.float32)
        b[j] = 1e3
        r = orc.route(X, Wr, b)
        assert np.all(r["ids"] == j)
    # top-1 probability lies in [1/E, 1]; top-K probabilities are non-increasing
    r = orc.route(X, Wr, top_k=3)
    assert np.all(r["prob"][:, 0] >= np.float32(1.0 / 8) * (1 - 1e-6)) and np.all(r["prob"] <= 1.0)
    assert np.all(np.diff(r["prob"], axis=1) <= 0)
    # two experts: the softmax of the winner is the logistic sigmoid of the margin
    r = orc.route(X, _rand(rng, (16, 2)), want_logits=True)
    margin = np.abs(r["logits"][:, 0].astype(np.float64) - r["logits"][:, 1].astype(np.float64))
    np.testing.assert_allclose(r["prob"][:, 0], expit(margin), rtol=3e-7, atol=0)
    np.testing.assert_array_equal(r["ids"][:, 0], np.where(r["logits"][:, 1] > r["logits"][:, 0], 1, 0))


# ------------------------------------------------------------------------------------------------
# histogram, stable counting sort, permute

def pin_sort(orc):
    rng = np.random.default_rng(13)
    cases = [
        (rng.integers(0, 8, size=1000), 8),
        (rng.choice(8, size=777, p=[.6, .1, .1, .05, .05, .05, .03, .02]), 8),
        (np.where(rng.random(300) < 0.5, 1, 5), 7),          # empty experts in between and at the ends
        (np.zeros(50, np.int64), 4),                          # all tokens on one expert
        (np.array([], np.int64), 3),                          # no tokens
        (rng.integers(0, 3, size=1), 3),                      # one token
    ]
    for ids, E in cases:
        ids = ids.astype(np.int32)
        s = orc.sort(ids, E)
        n = ids.shape[0]
        np.testing.assert_array_equal(s["counts"], np.bincount(ids, minlength=E))
        np.testing.assert_array_equal(s["offsets"], np.concatenate([[0], np.cumsum(np.bincount(ids, minlength=E))]))
        np.testing.assert_array_equal(s["perm"], np.argsort(ids, kind="stable"))
        np.testing.assert_array_equal(np.sort(s["perm"]), np.arange(n))          # bijection
        np.testing.assert_array_equal(s["inv_perm"][s["perm"]], np.arange(n))  # inverse
        np.testing.assert_array_equal(s["perm"][s["inv_perm"]], np.arange(n))
    # top-2 assignments: flattened [T][K], assignment a = t*K + s
    ids2 = rng.integers(0, 5, size=(60, 2)).astype(np.int32)
    s = orc.sort(ids2, 5)
    np.testing.assert_array_equal(s["perm"], np.argsort(ids2.reshape(-1), kind="stable"))
    X = _rand(rng, (60, 7))
    Xp = orc.permute(X, s["perm"], top_k=2)
    np.testing.assert_array_equal(Xp, np.repeat(X, 2, axis=0)[s["perm"]])


# ------------------------------------------------------------------------------------------------
# projections

def _proj_case(rng, T, dm, di, E, K):
    X = _rand(rng, (T, dm))
    Wc = _rand(rng, (E, di, dm), 0.3)
    Wg = _rand(rng, (E, di, dm), 0.3)
    Wo = _rand(rng, (E, dm, di), 0.3)
    h = _rand(rng, (T, di))
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    prob = rng.uniform(0.1, 1.0, size=(T, K)).astype(np.float32)
    return X, Wc, Wg, Wo, h, ids, prob


def pin_in_proj(orc):
    rng = np.random.default_rng(14)
    for (T, dm, di, E, K) in [(30, 24, 40, 3, 1), (20, 40, 24, 8, 1), (16, 8, 12, 5, 2)]:
        X, Wc, Wg, _, _, ids, _ = _proj_case(rng, T, dm, di, E, K)
        x, z = orc.in_proj(X, ids, Wc, Wg)
        # per-token float64 brute force: the selected experts' row-vector products, unscaled
        xb = np.zeros((T, di))
        zb = np.zeros((T, di))
        for t in range(T):
            for s in range(K):
                e = ids[t, s]
                xb[t] += Wc[e].astype(np.float64) @ X[t].astype(np.float64)
                zb[t] += Wg[e].astype(np.float64) @ X[t].astype(np.float64)
        np.testing.assert_allclose(x, xb, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(z, zb, rtol=1e-12, atol=1e-12)
    # E = 1: a dense projection, X @ W^T (BLAS)
    X, Wc, Wg, _, _, _, _ = _proj_case(rng, 33, 20, 28, 1, 1)
    x, z = orc.in_proj(X, np.zeros((33, 1), np.int32), Wc, Wg)
    np.testing.assert_allclose(x, X.astype(np.float64) @ Wc[0].astype(np.float64).T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z, X.astype(np.float64) @ Wg[0].astype(np.float64).T, rtol=1e-12, atol=1e-12)
    # identical experts: the routing decision cannot change the result (bit-identical sums)
    X, Wc, Wg, _, _, ids, _ = _proj_case(rng, 25, 16, 20, 4, 1)
    Wc[:] = Wc[0]
    Wg[:] = Wg[0]
    a = orc.in_proj(X, ids, Wc, Wg)
    b = orc.in_proj(X, np.zeros_like(ids), Wc, Wg)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])
    # top-2 is the unscaled sum of the two single-expert projections
    X, Wc, Wg, _, _, ids, _ = _proj_case(rng, 12, 16, 20, 6, 2)
    x2, z2 = orc.in_proj(X, ids, Wc, Wg)
    xa, za = orc.in_proj(X, ids[:, :1].copy(), Wc, Wg)
    xb_, zb_ = orc.in_proj(X, ids[:, 1:].copy(), Wc, Wg)
    np.testing.assert_allclose(x2, xa + xb_, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(z2, za + zb_, rtol=1e-12, atol=1e-12)


def _silu64(v):
    return v * expit(v)


def pin_out_proj(orc):
    rng = np.random.default_rng(15)
    for (T, dm, di, E, K) in [(30, 24, 40, 3, 1), (20, 40, 24, 8, 1), (16, 12, 8, 5, 2)]:
        _, _, _, Wo, h, ids, prob = _proj_case(rng, T, dm, di, E, K)
        z = rng.standard_normal((T, di)) * 3
        out = orc.out_proj(z, h, ids, prob, Wo)
        ob = np.zeros((T, dm))
        for t in range(T):
            a = _silu64(z[t]) * h[t].astype(np.float64)
            for s in range(K):
                ob[t] += float(prob[t, s]) * (Wo[ids[t, s]].astype(np.float64) @ a)
        np.testing.assert_allclose(out, ob, rtol=1e-12, atol=1e-12)
    # E = 1 with p = 1: dense (SiLU(z) * h) @ W_out^T
    _, _, _, Wo, h, _, _ = _proj_case(rng, 21, 18, 26, 1, 1)
    z = rng.standard_normal((21, 26)) * 2
    out = orc.out_proj(z, h, np.zeros((21, 1), np.int32), np.ones((21, 1), np.float32), Wo)
    np.testing.assert_allclose(out, (_silu64(z) * h) @ Wo[0].astype(np.float64).T, rtol=1e-12, atol=1e-12)
    # h = 0 gives exactly zero
    out = orc.out_proj(z, np.zeros_like(h), np.zeros((21, 1), np.int32), np.ones((21, 1), np.float32), Wo)
    assert np.all(out == 0.0)
    # linear in the router probability: halving p halves the output exactly
    _, _, _, Wo, h, ids, prob = _proj_case(rng, 15, 10, 14, 4, 1)
    z = rng.standard_normal((15, 14))
    o1 = orc.out_proj(z, h, ids, prob, Wo)
    o2 = orc.out_proj(z, h, ids, (prob * np.float32(0.5)).astype(np.float32), Wo)
    np.testing.assert_array_equal(o2, 0.5 * o1)
    o3 = orc.out_proj(z, h, ids, np.ones_like(prob), Wo)
    np.testing.assert_allclose(o1, o3 * prob.astype(np.float64), rtol=1e-13, atol=1e-15)
    # with W_out = I and h = 1 the output is SiLU(z): SiLU(v) - SiLU(-v) = v and SiLU(0) = 0
    d = 9
    eye = np.eye(d, dtype=np.float32)[None]
    z = rng.standard_normal((11, d)) * 4
    z[0, :] = 0.0
    one = np.ones((11, d), np.float32)
    ids0 = np.zeros((11, 1), np.int32)
    p1 = np.ones((11, 1), np.float32)
    s_pos = orc.out_proj(z, one, ids0, p1, eye)
    s_neg = orc.out_proj(-z, one, ids0, p1, eye)
    np.testing.assert_allclose(s_pos - s_neg, z, rtol=1e-14, atol=1e-14)
    assert np.all(s_pos[0] == 0.0)
    assert np.all(s_pos[z > 0] > 0) and np.all(s_pos[z < 0] < 0)


def pin_in_proj_weighted(orc):
    """Swimba's routing-weighted in-projection (Swimba project page, extended abstract)."""
    rng = np.random.default_rng(16)
    for (T, dm, do, E, K) in [(30, 24, 40, 4, 1), (20, 40, 24, 8, 1), (16, 8, 12, 5, 2)]:
        X, W, _, _, _, ids, prob = _proj_case(rng, T, dm, do, E, K)
        y = orc.in_proj_weighted(X, ids, prob, W)
        # per-token float64 brute force: the selected experts' streams, each times its weight
        yb = np.zeros((T, do))
        for t in range(T):
            for s in range(K):
                yb[t] += float(prob[t, s]) * (W[ids[t, s]].astype(np.float64) @ X[t].astype(np.float64))
        np.testing.assert_allclose(y, yb, rtol=1e-12, atol=1e-12)
    # E = 1 with p = 1: a dense projection X @ W^T (BLAS)
    X, W, _, _, _, _, _ = _proj_case(rng, 33, 20, 28, 1, 1)
    y = orc.in_proj_weighted(X, np.zeros((33, 1), np.int32), np.ones((33, 1), np.float32), W)
    np.testing.assert_allclose(y, X.astype(np.float64) @ W[0].astype(np.float64).T, rtol=1e-12, atol=1e-12)
    # linear in the weight: halving p halves the output exactly
    X, W, _, _, _, ids, prob = _proj_case(rng, 15, 10, 14, 4, 1)
    y1 = orc.in_proj_weighted(X, ids, prob, W)
    y2 = orc.in_proj_weighted(X, ids, (prob * np.float32(0.5)).astype(np.float32), W)
    np.testing.assert_array_equal(y2, 0.5 * y1)
    # the page's two-expert construction (Swimba Theorem 5): with the router choosing both of two experts
    # and expert 0 projecting to zero, the output is the logistic sigmoid of the logit margin times
    # expert 1's projection
    T, dm, do = 40, 12, 10
    X = _rand(rng, (T, dm))
    Wr = _rand(rng, (dm, 2), 0.5)
    W = _rand(rng, (2, do, dm), 0.4)
    W[0] = 0.0
    r = orc.route(X, Wr, top_k=2)
    y = orc.in_proj_weighted(X, r["ids"], r["prob"], W)
    l64 = X.astype(np.float64) @ Wr.astype(np.float64)
    ref = expit(l64[:, 1] - l64[:, 0])[:, None] * (X.astype(np.float64) @ W[1].astype(np.float64).T)
    np.testing.assert_allclose(y, ref, rtol=2e-6, atol=1e-9)
    # identical experts, both chosen: the weights sum to 1, so the output is the single projection
    W[0] = W[1]
    y = orc.in_proj_weighted(X, r["ids"], r["prob"], W)
    np.testing.assert_allclose(y, X.astype(np.float64) @ W[0].astype(np.float64).T, rtol=2e-6, atol=1e-9)


def pin_conv1d(orc):
    """The shared short causal convolution (RoM landing page, Knowl 1 and Knowl 9)."""
    rng = np.random.default_rng(17)
    # each channel of each sequence against numpy's full linear convolution, truncated to the causal part:
    # numpy.convolve(h, k)[t] = sum_j h[t - j] k[j], so the taps go in reversed (newest-first) order
    for (nseq, L, C, w) in [(2, 37, 5, 4), (3, 9, 3, 2), (1, 6, 4, 7)]:
        H = _rand(rng, (nseq, L, C))
        W = _rand(rng, (C, w), 0.5)
        b = _rand(rng, (C,), 0.3)
        u = orc.conv1d(H, W, b, activation=False)
        y = orc.conv1d(H, W, b, activation=True)
        ref = np.zeros((nseq, L, C))
        for s in range(nseq):
            for c in range(C):
                ref[s, :, c] = np.convolve(H[s, :, c].astype(np.float64), W[c, ::-1].astype(np.float64))[:L] + b[c]
        np.testing.assert_allclose(u, ref, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y, ref * expit(ref), rtol=1e-12, atol=1e-12)
    # width 1: a per-channel scale and shift, exactly
    H = _rand(rng, (2, 11, 6))
    W = _rand(rng, (6, 1))
    b = _rand(rng, (6,))
    np.testing.assert_array_equal(orc.conv1d(H, W, b, activation=False),
                                  H.astype(np.float64) * W[:, 0].astype(np.float64) + b.astype(np.float64))
    # impulse response: a unit impulse at time t0 of one sequence shows the taps in order W[c][w-1], ..., W[c][0]
    # at times t0, t0+1, ..., and nothing before t0 or in the other sequence
    nseq, L, C, w = 2, 12, 3, 4
    H = np.zeros((nseq, L, C), np.float32)
    H[1, 5, :] = 1.0
    W = _rand(rng, (C, w))
    y = orc.conv1d(H, W, None, activation=False)
    assert np.all(y[0] == 0.0) and np.all(y[1, :5] == 0.0) and np.all(y[1, 5 + w:] == 0.0)
    np.testing.assert_array_equal(y[1, 5:5 + w], W[:, ::-1].T.astype(np.float64))
    # sequences are independent: a sequence's output does not depend on the one before it (the
    # convolution starts from zeros at every sequence's first token)
    H = _rand(rng, (2, 10, 4))
    W = _rand(rng, (4, 4))
    a = orc.conv1d(H, W, None)
    H2 = H.copy()
    H2[0] = 7.0
    b2 = orc.conv1d(H2, W, None)
    np.testing.assert_array_equal(a[1], b2[1])
    # causality: changing token t changes no output before t
    H3 = H.copy()
    H3[1, 6] += 1.0
    c3 = orc.conv1d(H3, W, None)
    np.testing.assert_array_equal(a[1, :6], c3[1, :6])
    assert np.all(c3[1, 6] != a[1, 6])


def _dyadic(rng, shape, scale=8):
    """Small dyadic values k / scale, k in [-8, 8]: sums and differences of them are exact in float32."""
    return (rng.integers(-8, 9, size=shape) / scale).astype(np.float32)


def _dsilu64(v):
    s = expit(v)
    return s * (1.0 + v * (1.0 - s))


def pin_out_proj_backward(orc):
    """Gradients of the out-projection (Knowl 1, O_t) with the router probabilities held fixed."""
    rng = np.random.default_rng(18)
    for (T, dm, di, E, K) in [(20, 12, 16, 3, 1), (14, 8, 10, 5, 2)]:
        _, _, _, Wo, h, ids, prob = _proj_case(rng, T, dm, di, E, K)
        z = rng.standard_normal((T, di)) * 2
        g = _rand(rng, (T, dm))
        dz, dh = orc.out_proj_dgrad(g, z, h, ids, prob, Wo)
        dW = orc.out_proj_wgrad(g, z, h, ids, prob, E)
        # per-token float64 brute force
        zb, hb, dWb = np.zeros((T, di)), np.zeros((T, di)), np.zeros((E, dm, di))
        for t in range(T):
            a = _silu64(z[t]) * h[t].astype(np.float64)
            da = np.zeros(di)
            for s in range(K):
                e = ids[t, s]
                da += float(prob[t, s]) * (Wo[e].astype(np.float64).T @ g[t].astype(np.float64))
                dWb[e] += float(prob[t, s]) * np.outer(g[t].astype(np.float64), a)
            zb[t] = da * h[t] * _dsilu64(z[t])
            hb[t] = da * _silu64(z[t])
        np.testing.assert_allclose(dz, zb, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dh, hb, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dW, dWb, rtol=1e-11, atol=1e-12)
        ent = np.array([[e, m, c] for e in range(E) for m in (0, dm - 1) for c in (0, di // 2)])
        np.testing.assert_array_equal(orc.out_proj_wgrad_entries(g, z, h, ids, prob, ent), dW[tuple(ent.T)])
    # directional derivatives of L = <g, out> computed by the forward oracle: a central difference in z
    # (smooth, float64 input), and exact differences in h and W_out, in which L is linear (dyadic values
    # keep h +- U and W +- V exact in float32)
    T, dm, di, E, K = 9, 6, 8, 3, 2
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    prob = (rng.integers(1, 8, size=(T, K)) / 8).astype(np.float32)
    Wo, V = _dyadic(rng, (E, dm, di)), _dyadic(rng, (E, dm, di), 16)
    h, U = _dyadic(rng, (T, di)), _dyadic(rng, (T, di), 16)
    g = _dyadic(rng, (T, dm))
    z = rng.standard_normal((T, di))
    Vz = rng.standard_normal((T, di))
    L = lambda z_, h_, W_: float(np.sum(g.astype(np.float64) * orc.out_proj(z_, h_, ids, prob, W_)))
    dz, dh = orc.out_proj_dgrad(g, z, h, ids, prob, Wo)
    dW = orc.out_proj_wgrad(g, z, h, ids, prob, E)
    eps = 1e-5
    fd = (L(z + eps * Vz, h, Wo) - L(z - eps * Vz, h, Wo)) / (2 * eps)
    assert abs(fd - np.sum(dz * Vz)) <= 1e-7 * (1 + abs(fd)), (fd, np.sum(dz * Vz))
    fd = (L(z, h + U, Wo) - L(z, h - U, Wo)) / 2
    assert abs(fd - np.sum(dh * U)) <= 1e-10 * (1 + abs(fd)), (fd, np.sum(dh * U))
    fd = (L(z, h, Wo + V) - L(z, h, Wo - V)) / 2
    assert abs(fd - np.sum(dW * V)) <= 1e-10 * (1 + abs(fd)), (fd, np.sum(dW * V))
    # E = 1 with p = 1: a dense layer, dW = g^T a (BLAS) and da = g W
    _, _, _, Wo, h, _, _ = _proj_case(rng, 17, 10, 12, 1, 1)
    z = rng.standard_normal((17, 12))
    g = _rand(rng, (17, 10))
    one, zero = np.ones((17, 1), np.float32), np.zeros((17, 1), np.int32)
    a = _silu64(z) * h.astype(np.float64)
    np.testing.assert_allclose(orc.out_proj_wgrad(g, z, h, zero, one, 1)[0], g.astype(np.float64).T @ a,
                               rtol=1e-11, atol=1e-12)
    _, dh = orc.out_proj_dgrad(g, z, h, zero, one, Wo)
    np.testing.assert_allclose(dh, (g.astype(np.float64) @ Wo[0].astype(np.float64)) * _silu64(z), rtol=1e-11,
                               atol=1e-12)


def pin_in_proj_backward(orc):
    """Gradients of the in-projections (Knowl 1, H_t and the argument of SiLU in G_t)."""
    rng = np.random.default_rng(19)
    for (T, dm, di, E, K) in [(20, 12, 16, 3, 1), (14, 8, 10, 5, 2)]:
        X, Wc, Wg, _, _, ids, _ = _proj_case(rng, T, dm, di, E, K)
        dx, dz = _rand(rng, (T, di)), _rand(rng, (T, di))
        dX = orc.in_proj_dgrad(dx, dz, ids, Wc, Wg)
        dWc, dWg = orc.in_proj_wgrad(X, dx, dz, ids, E)
        Xb, Wcb, Wgb = np.zeros((T, dm)), np.zeros((E, di, dm)), np.zeros((E, di, dm))
        for t in range(T):
            for s in range(K):
                e = ids[t, s]
                Xb[t] += Wc[e].astype(np.float64).T @ dx[t] + Wg[e].astype(np.float64).T @ dz[t]
                Wcb[e] += np.outer(dx[t].astype(np.float64), X[t])
                Wgb[e] += np.outer(dz[t].astype(np.float64), X[t])
        np.testing.assert_allclose(dX, Xb, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dWc, Wcb, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dWg, Wgb, rtol=1e-11, atol=1e-12)
        ent = np.array([[e, c, k] for e in range(E) for c in (0, di - 1) for k in (1, dm // 2)])
        oc, og = orc.in_proj_wgrad_entries(X, dx, dz, ids, ent)
        np.testing.assert_array_equal(oc, dWc[tuple(ent.T)])
        np.testing.assert_array_equal(og, dWg[tuple(ent.T)])
    # L = <dx, x> + <dz, z> from the forward oracle is linear in X, W_conv and W_gate: exact differences
    T, dm, di, E, K = 11, 6, 8, 4, 2
    ids = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    X, U = _dyadic(rng, (T, dm)), _dyadic(rng, (T, dm), 16)
    Wc, Vc = _dyadic(rng, (E, di, dm)), _dyadic(rng, (E, di, dm), 16)
    Wg, Vg = _dyadic(rng, (E, di, dm)), _dyadic(rng, (E, di, dm), 16)
    dx, dz = _dyadic(rng, (T, di)), _dyadic(rng, (T, di))

    def L(X_, Wc_, Wg_):
        x, z = orc.in_proj(X_, ids, Wc_, Wg_)
        return float(np.sum(dx * x) + np.sum(dz * z))
    dX = orc.in_proj_dgrad(dx, dz, ids, Wc, Wg)
    dWc, dWg = orc.in_proj_wgrad(X, dx, dz, ids, E)
    for fd, an in (((L(X + U, Wc, Wg) - L(X - U, Wc, Wg)) / 2, np.sum(dX * U)),
                   ((L(X, Wc + Vc, Wg) - L(X, Wc - Vc, Wg)) / 2, np.sum(dWc * Vc)),
                   ((L(X, Wc, Wg + Vg) - L(X, Wc, Wg - Vg)) / 2, np.sum(dWg * Vg))):
        assert abs(fd - an) <= 1e-10 * (1 + abs(fd)), (fd, an)
    # E = 1: a dense layer, dX = dx W_conv + dz W_gate and dW_conv = dx^T X (BLAS)
    X, Wc, Wg, _, _, _, _ = _proj_case(rng, 15, 10, 12, 1, 1)
    dx, dz = _rand(rng, (15, 12)), _rand(rng, (15, 12))
    zero = np.zeros((15, 1), np.int32)
    np.testing.assert_allclose(orc.in_proj_dgrad(dx, dz, zero, Wc, Wg),
                               dx.astype(np.float64) @ Wc[0] + dz.astype(np.float64) @ Wg[0], rtol=1e-11, atol=1e-12)
    dWc, dWg = orc.in_proj_wgrad(X, dx, dz, zero, 1)
    np.testing.assert_allclose(dWc[0], dx.astype(np.float64).T @ X, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dWg[0], dz.astype(np.float64).T @ X, rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------------------------------------------
# hand-worked example

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul, ast.Div: operator.truediv,
        ast.USub: operator.neg, ast.UAdd: operator.pos}
_FUNCS = {"s": lambda v: 1.0 / (1.0 + math.exp(-v)), "e": math.exp}


def closed_form(expr: str) -> float:
    """Evaluate a fixture expression: numbers, s(), e(), + - * / and parentheses only."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.UnaryOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.operand))
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and node.func.id in _FUNCS
                and len(node.args) == 1 and not node.keywords):
            return _FUNCS[node.func.id](ev(node.args[0]))
        raise ValueError(f"unsupported expression: {expr}")
    return ev(ast.parse(expr, mode="eval"))


def load_handworked():
    with open(os.path.join(GOLDEN, "handworked_tiny.json")) as f:
        return json.load(f)


def pin_handworked(orc):
    g = load_handworked()
    X = np.array(g["X"], np.float32)
    Wr = np.array(g["W_router"], np.float32)
    Wc = np.array(g["W_conv"], np.float32)
    Wg = np.array(g["W_gate"], np.float32)
    Wo = np.array(g["W_out"], np.float32)
    h = np.array(g["h"], np.float32)
    ev = np.vectorize(closed_form, otypes=[np.float64])
    # top-1
    e1 = g["top1"]
    r = orc.route(X, Wr)
    np.testing.assert_array_equal(r["ids"][:, 0], e1["ids"])
    np.testing.assert_array_equal(r["gap"], np.array(e1["gap"], np.float32))
    np.testing.assert_allclose(r["prob"][:, 0], ev(np.array(e1["prob"])), rtol=1e-7, atol=0)
    s = orc.sort(r["ids"], g["E"])
    for k in ("counts", "offsets", "perm", "inv_perm"):
        np.testing.assert_array_equal(s[k], e1[k])
    x, z = orc.in_proj(X, r["ids"], Wc, Wg)
    np.testing.assert_array_equal(x, ev(np.array(e1["x"])))
    np.testing.assert_array_equal(z, ev(np.array(e1["z"])))
    out = orc.out_proj(z, h, r["ids"], r["prob"], Wo)
    np.testing.assert_allclose(out, ev(np.array(e1["out"])), rtol=1e-6, atol=1e-12)
    # top-2
    e2 = g["top2"]
    r = orc.route(X, Wr, top_k=2)
    np.testing.assert_array_equal(r["ids"], e2["ids"])
    np.testing.assert_array_equal(r["gap"], np.array(e2["gap"], np.float32))
    np.testing.assert_allclose(r["prob"], ev(np.array(e2["prob"])), rtol=1e-7, atol=0)
    x, z = orc.in_proj(X[:1], r["ids"][:1], Wc, Wg)
    np.testing.assert_array_equal(x[0], ev(np.array(e2["x_t0"])))
    np.testing.assert_array_equal(z[0], ev(np.array(e2["z_t0"])))
    out = orc.out_proj(z, h[:1], r["ids"][:1], r["prob"][:1], Wo)
    np.testing.assert_allclose(out[0], ev(np.array(e2["out_t0"])), rtol=1e-6, atol=1e-12)


ALL_PINS = [pin_router_bruteforce, pin_router_special, pin_sort, pin_in_proj, pin_out_proj, pin_in_proj_weighted,
            pin_conv1d, pin_out_proj_backward, pin_in_proj_backward, pin_handworked]
