"""Seeded synthetic inputs for the Routing Mamba (RoM) routed-projection workloads.

This module holds shapes and random draws only: no routing, projection or
activation arithmetic lives here. Both the HIP path's tests/benchmark and the
CPU oracle read the same tensors from it, bit for bit.

Shapes follow the RoM pages: the Samba-421M setting trains 4K-token sequences
at microbatch 4 per GPU (landing page, Knowl 7 and Knowl 12); the 1.3B-active
model is trained and evaluated at 16K tokens (abstract; Knowl 5); one of eight
experts is active per token (Knowl 1); the decode regime borrows Swimba's
4-expert top-1 layer and its vLLM batch sizes 1..64 (Swimba page, extended
abstract). No dataset is used anywhere: the projections are token-wise and
data-agnostic, so Gaussian tensors of these shapes stand in for SlimPajama
activations.

Recipe (all draws from ``numpy.random.Generator(PCG64)``, one child stream per
tensor from ``SeedSequence(seed).spawn``, ``standard_normal(dtype=float32)``
times the stated standard deviation). For bf16 workloads every tensor except
the fp32 router weight is rounded to the nearest bf16 (ties to even) by bit
manipulation, so the values handed to the oracle as float32 are exactly the
bits uploaded to the GPU.
"""
from __future__ import annotations

import dataclasses
import json
import os
from typing import Optional

import numpy as np

# Order of the per-tensor child streams; never reorder (it would change every input).
_STREAMS = ("X", "W_router", "W_conv", "W_gate", "W_out", "h", "z", "W_in")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    d_inner: int
    E: int
    dtype: str            # "f32" or "bf16": storage type of X, the expert stacks, z, h and outputs
    seed: int
    x_std: float          # standard deviation of X
    wr_std: Optional[float]  # std of W_router; None means 1/sqrt(d_model) (router logits ~ N(0,1))
    w_std: float          # std of W_conv, W_gate, W_out
    h_std: float          # std of h, the stand-in for the SSM-core output Y
    z_std: float          # std of z when the out-projection is tested on its own
    skew: Optional[tuple] = None  # target expert loads (fractions) reached with a router bias
    top_k: int = 1
    method: str = "rom"   # "rom": routed Conv/Gate/Out projections; "swimba": routing-weighted in-projection
    d_out: Optional[int] = None  # Swimba in-projection width; None means 2 * d_inner
    n_seq: int = 1        # sequences the T tokens form (the short convolution never crosses one)

    @property
    def dout(self) -> int:
        return self.d_out if self.d_out is not None else 2 * self.d_inner

    @property
    def router_std(self) -> float:
        return self.wr_std if self.wr_std is not None else 1.0 / np.sqrt(self.d_model)

    def gemm_flops(self) -> int:
        """Top-1 projection flops: in-proj 2*T*d_m*(2*d_i), out-proj 2*T*d_i*d_m."""
        return 6 * self.T * self.d_model * self.d_inner * self.top_k


def _tiny():
    return Workload("tiny_f32", T=256, d_model=64, d_inner=128, E=8, dtype="f32", seed=1,
                    x_std=0.02, wr_std=0.02, w_std=0.02, h_std=0.02, z_std=1.0)


WORKLOADS = {
    # tiny RoM block in fp32: everything N(0, 0.02^2)
    "tiny_f32": _tiny(),
    # Samba-421M-like block: per-GPU share of 4 x 4096 tokens, expand=2, 8 experts
    "samba421m": Workload("samba421m", T=16384, d_model=1024, d_inner=2048, E=8, dtype="bf16", seed=2,
                          x_std=1.0, wr_std=None, w_std=0.02, h_std=1.0, z_std=1.0, n_seq=4),
    # 1.3B-active-scale block on one 16K-token sequence
    "rom1p3b": Workload("rom1p3b", T=16384, d_model=2048, d_inner=4096, E=8, dtype="bf16", seed=3,
                        x_std=1.0, wr_std=0.02, w_std=0.02, h_std=1.0, z_std=1.0),
    # the same block with top-2 routing (the page's 8top2 setting); same seed, hence the same tensors
    "samba421m_top2": Workload("samba421m_top2", T=16384, d_model=1024, d_inner=2048, E=8, dtype="bf16", seed=2,
                               x_std=1.0, wr_std=None, w_std=0.02, h_std=1.0, z_std=1.0, top_k=2, n_seq=4),
    # skewed routing without a balance loss: a router bias gives loads 60/10/10/5/5/5/3/2 %
    "skewed": Workload("skewed", T=65536, d_model=2048, d_inner=4096, E=8, dtype="bf16", seed=4,
                       x_std=1.0, wr_std=0.02, w_std=0.02, h_std=1.0, z_std=1.0,
                       skew=(0.60, 0.10, 0.10, 0.05, 0.05, 0.05, 0.03, 0.02), n_seq=16),
}


def decode_workload(T: int) -> Workload:
    """Decode regime: T tokens in {1, 8, 64}, 4 experts, weight streaming."""
    return Workload(f"decode_T{T}", T=T, d_model=4096, d_inner=8192, E=4, dtype="bf16", seed=50 + T,
                    x_std=1.0, wr_std=None, w_std=0.02, h_std=1.0, z_std=1.0)


def swimba_decode_workload(T: int) -> Workload:
    """Swimba decode: T tokens in {1, 8, 64}, 4 experts, top-1, routing-weighted in-projection of
    width 2 * d_inner (the x and z streams; the page gives no widths)."""
    return Workload(f"swimba_decode_T{T}", T=T, d_model=4096, d_inner=8192, E=4, dtype="bf16", seed=60 + T,
                    x_std=1.0, wr_std=None, w_std=0.02, h_std=1.0, z_std=1.0, method="swimba")


def custom_workload(name, T, d_model, d_inner, E, dtype="bf16", seed=7, **kw) -> Workload:
    """A workload of arbitrary shape with the large-config value recipe (for edge-case tests)."""
    args = dict(x_std=1.0, wr_std=None, w_std=0.02, h_std=1.0, z_std=1.0)
    if dtype == "f32":
        args = dict(x_std=0.02, wr_std=0.02, w_std=0.02, h_std=0.02, z_std=1.0)
    args.update(kw)
    return Workload(name, T=T, d_model=d_model, d_inner=d_inner, E=E, dtype=dtype, seed=seed, **args)


def get_workload(name: str) -> Workload:
    if name.startswith("swimba_decode_T"):
        return swimba_decode_workload(int(name[len("swimba_decode_T"):]))
    if name.startswith("decode_T"):
        return decode_workload(int(name[len("decode_T"):]))
    return WORKLOADS[name]


# ---------------------------------------------------------------------------------------------
# bf16 storage helpers (bit manipulation only)

def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (round to nearest, ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """The uint16 bf16 bit patterns of a float32 array whose values are already bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    return (a.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------------------------

def _draw(rng: np.random.Generator, shape, std: float, storage: str) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return round_to_bf16(a) if storage == "bf16" else a


def make_inputs(w: Workload, router_bias: Optional[np.ndarray] = None, which=None) -> dict:
    """All inputs of one workload as float32 numpy arrays (bf16-representable where stored as bf16).

    Keys: X [T][d_model], W_router [d_model][E] (always fp32), W_conv and W_gate [E][d_inner][d_model],
    W_out [E][d_model][d_inner], h [T][d_inner], z [T][d_inner] (only for testing the out-projection on its
    own), W_in [E][d_out][d_model] (Swimba's in-projection experts), bias [E] or None. Expert matrices are
    stored [out][in], i.e. K-contiguous.
    ``which`` restricts generation to a subset of keys (the streams stay the same); by default every key
    but W_in is drawn, and W_in only when ``which`` names it.
    """
    children = np.random.SeedSequence(w.seed).spawn(len(_STREAMS))
    rngs = {k: np.random.Generator(np.random.PCG64(c)) for k, c in zip(_STREAMS, children)}
    shapes = {
        "X": ((w.T, w.d_model), w.x_std, w.dtype),
        "W_router": ((w.d_model, w.E), w.router_std, "f32"),
        "W_conv": ((w.E, w.d_inner, w.d_model), w.w_std, w.dtype),
        "W_gate": ((w.E, w.d_inner, w.d_model), w.w_std, w.dtype),
        "W_out": ((w.E, w.d_model, w.d_inner), w.w_std, w.dtype),
        "h": ((w.T, w.d_inner), w.h_std, w.dtype),
        "z": ((w.T, w.d_inner), w.z_std, w.dtype),
        "W_in": ((w.E, w.dout, w.d_model), w.w_std, w.dtype),
    }
    out = {}
    for k in _STREAMS:
        if (which is None and k == "W_in") or (which is not None and k not in which):
            continue
        shape, std, storage = shapes[k]
        out[k] = _draw(rngs[k], shape, std, storage)
    if router_bias is None and w.skew is not None:
        router_bias = load_skew_bias(w)
    out["bias"] = None if router_bias is None else np.ascontiguousarray(router_bias, dtype=np.float32)
    return out


def make_conv_inputs(n_seq: int, seq_len: int, channels: int, width: int, dtype: str = "bf16", seed: int = 0,
                     with_bias: bool = True) -> dict:
    """Inputs of the shared short causal convolution: x [n_seq][seq_len][channels] ~ N(0, 1) (the Conv
    projection's output), weight [channels][width] ~ N(0, 1/width), bias [channels] ~ N(0, 0.1^2) or None.
    Same stream recipe as make_inputs (one PCG64 child stream per tensor)."""
    children = np.random.SeedSequence(seed).spawn(3)
    rng = [np.random.Generator(np.random.PCG64(c)) for c in children]
    out = {
        "x": _draw(rng[0], (n_seq, seq_len, channels), 1.0, dtype),
        "weight": _draw(rng[1], (channels, width), float(1.0 / np.sqrt(width)), dtype),
        "bias": _draw(rng[2], (channels,), 0.1, dtype) if with_bias else None,
    }
    return out


def make_grad_inputs(w: Workload, seed: int = 1000) -> dict:
    """Upstream gradients for the backward: d_out [T][d_model] (dL/dout), dx and dz [T][d_inner] (dL/dx_out,
    dL/dz_out), each ~ N(0, 1) in the workload's storage type, one PCG64 child stream per tensor."""
    children = np.random.SeedSequence([w.seed, seed]).spawn(3)
    rng = [np.random.Generator(np.random.PCG64(c)) for c in children]
    return {
        "d_out": _draw(rng[0], (w.T, w.d_model), 1.0, w.dtype),
        "dx": _draw(rng[1], (w.T, w.d_inner), 1.0, w.dtype),
        "dz": _draw(rng[2], (w.T, w.d_inner), 1.0, w.dtype),
    }


_BIAS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tests", "golden", "skewed_router_bias.json")


def load_skew_bias(w: Workload) -> np.ndarray:
    """The fp32 router bias that realises the skewed workload's target loads.

    It is a stored input written by the calibration script beside the file, which routes with the
    CPU oracle only.
    """
    with open(_BIAS_FILE) as f:
        rec = json.load(f)
    if rec["workload"] != w.name or rec["seed"] != w.seed or rec["T"] != w.T:
        raise ValueError(f"stored router bias is for {rec['workload']}, not {w.name}")
    return np.array(rec["bias"], dtype=np.float32)
