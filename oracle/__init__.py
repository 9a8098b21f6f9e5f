"""CPU oracle for the Routing Mamba routed projections: ctypes wrapper over ``rom_oracle.c``.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's CPU-baseline leg
are its only users. The HIP product path never imports this package and shares no code with it.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py`` against things other
than itself (float64 brute force per token, numpy library routines for the sort and for the E=1
dense special case, closed forms, a hand-worked example under ``tests/golden/``); the tests under
``tests/test_oracle_mutants.py`` plant mistakes in a copy of the C source and check that a pin
catches each one. The conventions the page leaves open (tie-break, stable order within an
expert, the skewed workload's router bias) are pinned only by their own specification.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_DIR, "rom_oracle.c")
LIBRARY = os.path.join(_DIR, "liborom.so")
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-shared", "-fPIC"]


def build(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over independent tokens)."""
    cmd = ["gcc", *CFLAGS, *extra_flags, source, "-o", output + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(output + ".tmp", output)
    return output


_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class Oracle:
    """One loaded copy of the oracle library (the real one, or a test's mutant build)."""

    def __init__(self, path: str = LIBRARY):
        if path == LIBRARY and (not os.path.exists(LIBRARY)
                                or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE)):
            build()
        self.path = path
        lib = ctypes.CDLL(path)
        lib.orom_version.restype = ctypes.c_int
        lib.orom_threads.restype = ctypes.c_int
        lib.orom_route.argtypes = [_f32p, _i64, _i64, _f32p, ctypes.c_void_p, _i32, _i32,
                                   _i32p, _f32p, _f32p, ctypes.c_void_p]
        lib.orom_route.restype = None
        lib.orom_sort.argtypes = [_i32p, _i64, _i32, _i32p, _i32p, _i32p, _i32p]
        lib.orom_sort.restype = ctypes.c_int
        lib.orom_permute.argtypes = [_f32p, _i64, _i32, _i64, _i32p, _f32p]
        lib.orom_permute.restype = None
        lib.orom_in_proj.argtypes = [_f32p, _i64, _i64, _i64, _i32p, _i32, _f32p, _f32p, _i32, _f64p, _f64p]
        lib.orom_in_proj.restype = None
        lib.orom_out_proj.argtypes = [_f64p, _f32p, _i64, _i64, _i64, _i32p, _f32p, _i32, _f32p, _i32, _f64p]
        lib.orom_out_proj.restype = None
        lib.orom_in_proj_weighted.argtypes = [_f32p, _i64, _i64, _i64, _i32p, _f32p, _i32, _f32p, _i32, _f64p]
        lib.orom_in_proj_weighted.restype = None
        lib.orom_conv1d.argtypes = [_f32p, _i64, _i64, _i64, _f32p, ctypes.c_void_p, _i32, _i32, _f64p]
        lib.orom_conv1d.restype = None
        lib.orom_out_proj_dgrad.argtypes = [_f32p, _f64p, _f32p, _i64, _i64, _i64, _i32p, _f32p, _i32, _f32p, _i32,
                                            _f64p, _f64p]
        lib.orom_out_proj_wgrad.argtypes = [_f32p, _f64p, _f32p, _i64, _i64, _i64, _i32p, _f32p, _i32, _i32, _f64p]
        lib.orom_out_proj_wgrad_entries.argtypes = [_f32p, _f64p, _f32p, _i64, _i64, _i64, _i32p, _f32p, _i32, _i64p,
                                                    _i64, _f64p]
        lib.orom_in_proj_dgrad.argtypes = [_f32p, _f32p, _i64, _i64, _i64, _i32p, _i32, _f32p, _f32p, _i32, _f64p]
        lib.orom_in_proj_wgrad.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i32p, _i32, _i32, _f64p, _f64p]
        lib.orom_in_proj_wgrad_entries.argtypes = [_f32p, _f32p, _f32p, _i64, _i64, _i64, _i32p, _i32, _i64p, _i64,
                                                   _f64p, _f64p]
        for f in ("orom_out_proj_dgrad", "orom_out_proj_wgrad", "orom_out_proj_wgrad_entries", "orom_in_proj_dgrad",
                  "orom_in_proj_wgrad", "orom_in_proj_wgrad_entries"):
            getattr(lib, f).restype = None
        self.lib = lib

    def threads(self) -> int:
        """OpenMP threads the oracle's per-token loops run on."""
        return int(self.lib.orom_threads())

    # -- router -------------------------------------------------------------------------------
    def route(self, X, W_router, bias=None, top_k: int = 1, want_logits: bool = False):
        """Returns dict(ids [T][K] int32, prob [T][K] fp32, gap [T] fp32, logits [T][E] fp32 or None)."""
        X = np.ascontiguousarray(X, dtype=np.float32)
        Wr = np.ascontiguousarray(W_router, dtype=np.float32)
        T, dm = X.shape
        E = Wr.shape[1]
        assert Wr.shape[0] == dm and 1 <= top_k <= E
        ids = np.empty((T, top_k), np.int32)
        prob = np.empty((T, top_k), np.float32)
        gap = np.empty((T,), np.float32)
        logits = np.empty((T, E), np.float32) if want_logits else None
        b = None
        if bias is not None:
            b = np.ascontiguousarray(bias, dtype=np.float32)
            assert b.shape == (E,)
        self.lib.orom_route(X, T, dm, Wr, None if b is None else b.ctypes.data, E, top_k, ids, prob, gap,
                            None if logits is None else logits.ctypes.data)
        return dict(ids=ids, prob=prob, gap=gap, logits=logits)

    # -- grouping -------------------------------------------------------------------------------
    def sort(self, ids, E: int):
        """Histogram + stable counting sort of the flattened assignments ids[T][K]."""
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(-1)
        n = ids.shape[0]
        counts = np.empty((E,), np.int32)
        offsets = np.empty((E + 1,), np.int32)
        perm = np.empty((n,), np.int32)
        inv_perm = np.empty((n,), np.int32)
        rc = self.lib.orom_sort(ids, n, E, counts, offsets, perm, inv_perm)
        if rc != 0:
            raise ValueError("expert id out of range")
        return dict(counts=counts, offsets=offsets, perm=perm, inv_perm=inv_perm)

    def permute(self, X, perm, top_k: int = 1):
        X = np.ascontiguousarray(X, dtype=np.float32)
        perm = np.ascontiguousarray(perm, dtype=np.int32)
        out = np.empty((perm.shape[0], X.shape[1]), np.float32)
        self.lib.orom_permute(X, perm.shape[0], top_k, X.shape[1], perm, out)
        return out

    # -- projections ----------------------------------------------------------------------------
    def in_proj(self, X, ids, W_conv, W_gate):
        """x, z [n][d_inner] in float64 for the n rows of X routed to ids[n][K]."""
        X = np.ascontiguousarray(X, dtype=np.float32)
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(X.shape[0], -1)
        Wc = np.ascontiguousarray(W_conv, dtype=np.float32)
        Wg = np.ascontiguousarray(W_gate, dtype=np.float32)
        n, dm = X.shape
        E, di, dm2 = Wc.shape
        assert dm2 == dm and Wg.shape == Wc.shape
        assert ids.size == 0 or (ids.min() >= 0 and ids.max() < E)
        x = np.empty((n, di), np.float64)
        z = np.empty((n, di), np.float64)
        self.lib.orom_in_proj(X, n, dm, di, ids, ids.shape[1], Wc, Wg, E, x, z)
        return x, z

    def out_proj(self, z, h, ids, prob, W_out):
        """out [n][d_model] in float64 for n tokens: sum_s prob * (SiLU(z) * h) W_out[ids]^T."""
        z = np.ascontiguousarray(z, dtype=np.float64)
        h = np.ascontiguousarray(h, dtype=np.float32)
        n, di = z.shape
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(n, -1)
        prob = np.ascontiguousarray(prob, dtype=np.float32).reshape(n, -1)
        Wo = np.ascontiguousarray(W_out, dtype=np.float32)
        E, dm, di2 = Wo.shape
        assert di2 == di and h.shape == z.shape and prob.shape == ids.shape
        assert ids.size == 0 or (ids.min() >= 0 and ids.max() < E)
        out = np.empty((n, dm), np.float64)
        self.lib.orom_out_proj(z, h, n, di, dm, ids, prob, ids.shape[1], Wo, E, out)
        return out

    def in_proj_weighted(self, X, ids, prob, W_in):
        """Swimba's routing-weighted in-projection: y [n][d_out] in float64,
        y[t] = sum_s prob[t][s] * W_in[ids[t][s]] X[t]."""
        X = np.ascontiguousarray(X, dtype=np.float32)
        n, dm = X.shape
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(n, -1)
        prob = np.ascontiguousarray(prob, dtype=np.float32).reshape(n, -1)
        W = np.ascontiguousarray(W_in, dtype=np.float32)
        E, dout, dm2 = W.shape
        assert dm2 == dm and prob.shape == ids.shape
        assert ids.size == 0 or (ids.min() >= 0 and ids.max() < E)
        y = np.empty((n, dout), np.float64)
        self.lib.orom_in_proj_weighted(X, n, dm, dout, ids, prob, ids.shape[1], W, E, y)
        return y

    def conv1d(self, H, weight, bias=None, activation: bool = True):
        """Shared short causal depthwise convolution of each sequence of H [nseq][L][C]; weight [C][w];
        returns y [nseq][L][C] in float64."""
        H = np.ascontiguousarray(H, dtype=np.float32)
        nseq, L, C = H.shape
        W = np.ascontiguousarray(weight, dtype=np.float32)
        assert W.shape[0] == C and W.ndim == 2
        b = None
        if bias is not None:
            b = np.ascontiguousarray(bias, dtype=np.float32)
            assert b.shape == (C,)
        y = np.empty((nseq, L, C), np.float64)
        self.lib.orom_conv1d(H, nseq, L, C, W, None if b is None else b.ctypes.data, W.shape[1],
                             1 if activation else 0, y)
        return y

    # -- backward ---------------------------------------------------------------------------------
    # Gradients of the routed projections with the router probabilities held fixed.

    @staticmethod
    def _out_args(g, z, h, ids, prob):
        g = np.ascontiguousarray(g, dtype=np.float32)
        z = np.ascontiguousarray(z, dtype=np.float64)
        h = np.ascontiguousarray(h, dtype=np.float32)
        n, di = z.shape
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(n, -1)
        prob = np.ascontiguousarray(prob, dtype=np.float32).reshape(n, -1)
        assert h.shape == z.shape and g.shape[0] == n and prob.shape == ids.shape
        return g, z, h, ids, prob, n, di, g.shape[1]

    def out_proj_dgrad(self, g, z, h, ids, prob, W_out):
        """dz, dh [n][d_inner] (float64) of out = sum_s prob * W_out[ids] (SiLU(z) * h) for upstream g [n][d_model]."""
        g, z, h, ids, prob, n, di, dm = self._out_args(g, z, h, ids, prob)
        Wo = np.ascontiguousarray(W_out, dtype=np.float32)
        E = Wo.shape[0]
        assert Wo.shape == (E, dm, di) and (ids.size == 0 or (ids.min() >= 0 and ids.max() < E))
        dz = np.empty((n, di), np.float64)
        dh = np.empty((n, di), np.float64)
        self.lib.orom_out_proj_dgrad(g, z, h, n, di, dm, ids, prob, ids.shape[1], Wo, E, dz, dh)
        return dz, dh

    def out_proj_wgrad(self, g, z, h, ids, prob, E: int):
        """dW_out [E][d_model][d_inner] (float64), summed over the given tokens."""
        g, z, h, ids, prob, n, di, dm = self._out_args(g, z, h, ids, prob)
        dW = np.empty((E, dm, di), np.float64)
        self.lib.orom_out_proj_wgrad(g, z, h, n, di, dm, ids, prob, ids.shape[1], E, dW)
        return dW

    def out_proj_wgrad_entries(self, g, z, h, ids, prob, entries):
        """dW_out[e][m][c] for each (e, m, c) row of entries."""
        g, z, h, ids, prob, n, di, dm = self._out_args(g, z, h, ids, prob)
        ent = np.ascontiguousarray(entries, dtype=np.int64).reshape(-1, 3)
        out = np.empty((ent.shape[0],), np.float64)
        self.lib.orom_out_proj_wgrad_entries(g, z, h, n, di, dm, ids, prob, ids.shape[1], ent, ent.shape[0], out)
        return out

    @staticmethod
    def _in_args(X, dx, dz, ids):
        X = np.ascontiguousarray(X, dtype=np.float32)
        dx = np.ascontiguousarray(dx, dtype=np.float32)
        dz = np.ascontiguousarray(dz, dtype=np.float32)
        n, dm = X.shape
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(n, -1)
        assert dx.shape == dz.shape and dx.shape[0] == n
        return X, dx, dz, ids, n, dm, dx.shape[1]

    def in_proj_dgrad(self, dx, dz, ids, W_conv, W_gate):
        """dX [n][d_model] (float64) of x = sum_s W_conv[ids] X, z = sum_s W_gate[ids] X for upstream dx, dz."""
        dx = np.ascontiguousarray(dx, dtype=np.float32)
        dz = np.ascontiguousarray(dz, dtype=np.float32)
        n, di = dx.shape
        ids = np.ascontiguousarray(ids, dtype=np.int32).reshape(n, -1)
        Wc = np.ascontiguousarray(W_conv, dtype=np.float32)
        Wg = np.ascontiguousarray(W_gate, dtype=np.float32)
        E, di2, dm = Wc.shape
        assert di2 == di and Wg.shape == Wc.shape and dz.shape == dx.shape
        assert ids.size == 0 or (ids.min() >= 0 and ids.max() < E)
        dX = np.empty((n, dm), np.float64)
        self.lib.orom_in_proj_dgrad(dx, dz, n, dm, di, ids, ids.shape[1], Wc, Wg, E, dX)
        return dX

    def in_proj_wgrad(self, X, dx, dz, ids, E: int):
        """dW_conv, dW_gate [E][d_inner][d_model] (float64), summed over the given tokens."""
        X, dx, dz, ids, n, dm, di = self._in_args(X, dx, dz, ids)
        dWc = np.empty((E, di, dm), np.float64)
        dWg = np.empty((E, di, dm), np.float64)
        self.lib.orom_in_proj_wgrad(X, dx, dz, n, dm, di, ids, ids.shape[1], E, dWc, dWg)
        return dWc, dWg

    def in_proj_wgrad_entries(self, X, dx, dz, ids, entries):
        """(dW_conv[e][c][k], dW_gate[e][c][k]) for each (e, c, k) row of entries."""
        X, dx, dz, ids, n, dm, di = self._in_args(X, dx, dz, ids)
        ent = np.ascontiguousarray(entries, dtype=np.int64).reshape(-1, 3)
        oc = np.empty((ent.shape[0],), np.float64)
        og = np.empty((ent.shape[0],), np.float64)
        self.lib.orom_in_proj_wgrad_entries(X, dx, dz, n, dm, di, ids, ids.shape[1], ent, ent.shape[0], oc, og)
        return oc, og

    # -- the whole routed path for a subset of tokens --------------------------------------------
    def forward_rows(self, inp: dict, rows: Optional[np.ndarray] = None, top_k: int = 1, routed=None):
        """Route all tokens, then project the given rows (all rows if None). Returns a dict."""
        r = routed if routed is not None else self.route(inp["X"], inp["W_router"], inp.get("bias"), top_k)
        srt = self.sort(r["ids"], inp["W_router"].shape[1])
        rows = np.arange(inp["X"].shape[0]) if rows is None else np.asarray(rows)
        x, z = self.in_proj(inp["X"][rows], r["ids"][rows], inp["W_conv"], inp["W_gate"])
        out = self.out_proj(z, inp["h"][rows], r["ids"][rows], r["prob"][rows], inp["W_out"])
        return dict(route=r, sort=srt, rows=rows, x=x, z=z, out=out)


_DEFAULT: Optional[Oracle] = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
