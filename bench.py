#!/usr/bin/env python3
"""Benchmark of the Routing Mamba (RoM) routed-projection hot path on one MI355X.

One step = the whole routed path over one batch of synthetic tokens, through the C ABI:
    rom_route    fp32 router logits + softmax + top-1 + probability, histogram, scan, stable scatter
    rom_in_proj  Conv/Gate expert grouped GEMM (bf16 MFMA), rows gathered through perm, un-permuted
    rom_out_proj Out expert grouped GEMM on SiLU(z)*h, scaled by the router probability, un-permuted
(Routing Mamba landing page on chapterpal.com, Knowl 1.) Inputs are resident in HBM before timing.
For the Swimba workloads (swimba_decode_T*) one step is rom_route + rom_in_proj_weighted, the routed part of a
Switch Mamba layer (Swimba project page, extended abstract): expert in-projections whose outputs are weighted
by the router probability.

Default workload: the largest single-GPU block, skewed routing without a balance loss: T = 65536 tokens
(16 x 4096), d_model 2048, d_inner 4096, 8 experts whose loads are 60/10/10/5/5/5/3/2 % (a router bias
realises them), bf16 data. Prints ONE JSON line: whole-step tokens/s, the roofline of the dominant kernel
(the in-projection grouped GEMM, timed live with HIP events on the stream it runs on), per-call medians
with p10/p90, and the CPU oracle timed on a bounded sample of the same workload on the host cores.

Decode workloads (T <= 64) run with cold caches by default (a 1 GiB read evicts L2 and the MALL before
every step) and report the whole step (router + both projections) against HBM bandwidth as their roofline.

Before the W warm-up steps the GPU runs steps for --ramp-seconds of wall time, so that its clocks have left
their idle state whatever W is (the time is reported as clock_ramp_s).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--cold | --warm]
                    [--backward] [--with-conv1d] [--event-every N] [--ramp-seconds S]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed-projection tokens/sec + % bf16 MFMA peak (GEMM) / % HBM peak (decode)"
PEAK_MFMA_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0                                # MI355X HBM3E
KERNEL_SOURCES = ["state_space_lms_amd/csrc/rom_gemm.hip", "state_space_lms_amd/csrc/rom_gemm.h",
                  "state_space_lms_amd/csrc/rom_device.h"]
COUNTERS_FILE = "profiles/counters_in_proj_{workload}.txt"
COPY_PROBE_BYTES = 256 << 20
CONV_WIDTH = 4   # the pages give no width for the short convolution; 4 is the value this benchmark takes


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence: recording it skips the
    system-scope release (an L2 write-back and invalidate) that a default event performs, which otherwise
    puts about 5 us between the event and the next kernel. Same interface as torch.cuda.Event (record on a
    torch stream, elapsed_time in ms). It calls the HIP runtime that torch has already loaded."""
    _hip = None
    _DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def _runtime(cls):
        if cls._hip is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("bench.py: the HIP runtime is not loaded")
            hip = ctypes.CDLL(path)
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = hip
        return cls._hip

    def __init__(self):
        import ctypes
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        err = self._runtime().hipEventCreateWithFlags(ctypes.byref(self.ev), self._DISABLE_SYSTEM_FENCE)
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")

    def record(self, stream):
        err = self._hip.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream))
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed ({err})")

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = self._ct.c_float()
        err = self._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per in-projection launch from committed rocprofv3 counters, or None when the counters
    are missing or were taken on another version of the kernel source."""
    path = os.path.join(ROOT, COUNTERS_FILE.format(workload=workload))
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != kernel_source_hash():
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, w, target_seconds: float, conv: bool = False, bwd: bool = False):
    """The CPU oracle as it stands, timed on a bounded prefix of the workload's tokens."""
    import numpy as np
    import oracle
    import workloads
    orc = oracle.default()

    def run(n):
        t0 = time.perf_counter()
        r = orc.route(inp["X"][:n], inp["W_router"], inp.get("bias"), top_k=w.top_k)
        orc.sort(r["ids"], w.E)
        if w.method == "swimba":
            orc.in_proj_weighted(inp["X"][:n], r["ids"], r["prob"], inp["W_in"])
        else:
            x, z = orc.in_proj(inp["X"][:n], r["ids"], inp["W_conv"], inp["W_gate"])
            if conv:
                cin = workloads.make_conv_inputs(1, 1, w.d_inner, CONV_WIDTH, w.dtype, seed=w.seed)
                orc.conv1d(x.astype(np.float32)[None], cin["weight"], cin["bias"])
            orc.out_proj(z, inp["h"][:n], r["ids"], r["prob"], inp["W_out"])
            if bwd:
                gin = workloads.make_grad_inputs(w)
                g, hh = gin["d_out"][:n], inp["h"][:n]
                dz, _ = orc.out_proj_dgrad(g, z, hh, r["ids"], r["prob"], inp["W_out"])
                orc.out_proj_wgrad(g, z, hh, r["ids"], r["prob"], w.E)
                dz32 = dz.astype(np.float32)
                orc.in_proj_dgrad(gin["dx"][:n], dz32, r["ids"], inp["W_conv"], inp["W_gate"])
                orc.in_proj_wgrad(inp["X"][:n], gin["dx"][:n], dz32, r["ids"], w.E)
        return time.perf_counter() - t0

    probe = min(w.T, 32)
    tp = run(probe)
    n = int(max(probe, min(w.T, probe * target_seconds / max(tp, 1e-6))))
    dt = run(n) if n > probe else tp
    path = "in_proj_weighted" if w.method == "swimba" else ("in_proj + conv1d + out_proj" if conv else
                                                            "in_proj + out_proj")
    if bwd:
        path += " + both backwards"
    cpu = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    # the forward GEMM flops of the sample (as the GPU's in + out figure), for the oracle's GFLOP/s
    n_in = w.dout if w.method == "swimba" else 2 * w.d_inner
    fl = 2.0 * n * w.d_model * (n_in + (0 if w.method == "swimba" else w.d_inner)) * w.top_k
    return {"value": n / dt, "unit": "tokens/s", "cores": orc.threads(), "kind": "oracle",
            "cpu": cpu, "gemm_gflops": None if bwd else round(fl / dt / 1e9, 2),
            "sample": f"first {n} of {w.T} tokens: route + histogram/sort + {path} in plain C "
                      f"(fp32 router, fp64 projection sums, OpenMP over tokens), {dt:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps after the clock ramp")
    ap.add_argument("--ramp-seconds", type=float, default=1.0,
                    help="run untimed steps for this much wall time before the warm-up steps: the GPU needs some "
                         "tens of milliseconds of work to leave its idle clocks (the first ~50 Samba-size steps "
                         "run ~40%% slower), whatever --warmup is")
    ap.add_argument("--event-every", type=int, default=5,
                    help="bracket the in-projection with HIP events on every n-th timed step (events cost a few "
                         "microseconds of GPU time each, which matters at decode sizes)")
    ap.add_argument("--workload", default="skewed")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--with-conv1d", action="store_true",
                    help="add the shared short causal convolution (width 4, SiLU, bias) on the in-projection's x to "
                         "the step (prefill RoM workloads)")
    ap.add_argument("--backward", action="store_true",
                    help="add the backward of both projections (out_proj_backward, then in_proj_backward on its dz) to "
                         "the step: a forward + backward pass of the routed projections (prefill RoM workloads)")
    ap.add_argument("--fenced-events", action="store_true",
                    help="time with default HIP events (system-scope release on record, about 5 us each) instead "
                         "of timing-only events")
    ap.add_argument("--cold", action="store_true",
                    help="read a 1 GiB buffer before every step, so weights and inputs come from HBM; the step is "
                         "then timed with GPU events around it (the default for decode workloads, T <= 64)")
    ap.add_argument("--warm", action="store_true", help="decode workloads: keep caches warm between steps")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the benchmark runs on one GPU only (the routed projections of a token need no data "
              "from other GPUs, and no multi-GPU path is built); run it with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import state_space_lms_amd as rom
    import workloads

    w = workloads.get_workload(args.workload)
    swimba = w.method == "swimba"
    conv = args.with_conv1d
    bwd = args.backward
    if bwd and (swimba or w.dtype != "bf16"):
        print("bench.py: --backward needs a bf16 RoM workload", file=sys.stderr)
        return 2
    if conv and (swimba or w.T <= 64):
        print("bench.py: --with-conv1d needs a prefill RoM workload (the decode-time convolution state is not "
              "built)", file=sys.stderr)
        return 2
    inp = workloads.make_inputs(w, which={"X", "W_router", "W_in"} if swimba else
                                {"X", "W_router", "W_conv", "W_gate", "W_out", "h"})
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def up(a, dt):
        if dt == "bf16":
            return torch.from_numpy(workloads.bf16_bits(a).view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    X = up(inp["X"], w.dtype)
    Wr = up(inp["W_router"], "f32")
    bias = up(inp["bias"], "f32") if inp.get("bias") is not None else None
    routing = rom.Routing(w.T, w.E, dev, top_k=w.top_k)
    if swimba:
        W_in = up(inp["W_in"], w.dtype)
        y = torch.empty((w.T, w.dout), dtype=X.dtype, device=dev)
    else:
        h = up(inp["h"], w.dtype)
        Wc, Wg, Wo = up(inp["W_conv"], w.dtype), up(inp["W_gate"], w.dtype), up(inp["W_out"], w.dtype)
        x = torch.empty((w.T, w.d_inner), dtype=X.dtype, device=dev)
        z = torch.empty_like(x)
        out = torch.empty((w.T, w.d_model), dtype=X.dtype, device=dev)
    if bwd:
        gin = workloads.make_grad_inputs(w)
        g_out, dx_up = up(gin["d_out"], w.dtype), up(gin["dx"], w.dtype)
        bwd_res = {}
    if conv:
        cin = workloads.make_conv_inputs(1, 1, w.d_inner, CONV_WIDTH, w.dtype, seed=w.seed)
        Wcv, bcv = up(cin["weight"], w.dtype), up(cin["bias"], w.dtype)
        xc = torch.empty((w.T, w.d_inner), dtype=X.dtype, device=dev)
    decode = w.T <= 64
    cold = (args.cold or decode) and not args.warm
    # cold runs stream this buffer through the caches before each step; reading (not writing) it leaves no
    # dirty lines whose write-back would be charged to the step (fp32, so that the sum needs no widened copy)
    flush = torch.zeros((1 << 30) // 4, dtype=torch.float32, device=dev) if cold else None
    # the materialised permute (X_perm[pos] = X[perm[pos]], top-1) is timed as its own call after the step
    xperm = rom.Routing(w.T, w.E, dev, top_k=1) if w.top_k == 1 else None

    # plain copy of known size: the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters
    cp_src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    cp_dst = torch.empty_like(cp_src)
    torch.neg(cp_src, out=cp_dst)
    del cp_src, cp_dst

    stream = torch.cuda.current_stream(dev)
    phases = ["route", "in"] + (["conv"] if conv else []) + ([] if swimba else ["out"]) + (["obwd", "ibwd"] if bwd else [])

    def run_phase(ph):
        if ph == "route":
            rom.route(X, Wr, bias, top_k=w.top_k, routing=routing, stream=stream)
        elif ph == "in":
            if swimba:
                rom.in_proj_weighted(X, routing, W_in, y, stream=stream)
            else:
                rom.in_proj(X, routing, Wc, Wg, x, z, stream=stream)
        elif ph == "conv":
            rom.conv1d(x, Wcv, bcv, n_seq=w.n_seq, activation=True, y=xc, stream=stream)
        elif ph == "obwd":
            bwd_res["o"] = rom.out_proj_backward(g_out, z, h, routing, Wo, stream=stream)
        elif ph == "ibwd":
            bwd_res["i"] = rom.in_proj_backward(X, dx_up, bwd_res["o"][0], routing, Wc, Wg, stream=stream)
        else:
            rom.out_proj(z, h, routing, Wo, out, stream=stream)

    def step(ev=None, around_in=None):
        """ev: an event before every phase and one after the last; around_in: two events bracketing the
        in-projection only."""
        for i, ph in enumerate(phases):
            if ev is not None:
                ev[i].record(stream)
            if around_in is not None and ph == "in":
                around_in[0].record(stream)
            run_phase(ph)
            if around_in is not None and ph == "in":
                around_in[1].record(stream)
        if ev is not None:
            ev[-1].record(stream)

    # clock ramp: steps for a fixed wall time (synchronised every few steps), then the warm-up steps
    t_ramp0 = time.perf_counter()
    n_ramp = 0
    while time.perf_counter() - t_ramp0 < args.ramp_seconds:
        for _ in range(4):
            if flush is not None:
                flush.sum()
            step()
            n_ramp += 1
        torch.cuda.synchronize()
    ramp_s = time.perf_counter() - t_ramp0
    for _ in range(args.warmup):
        if flush is not None:
            flush.sum()
        step()
    torch.cuda.synchronize()

    if args.fenced_events:
        new_ev = lambda n: [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    else:
        new_ev = lambda n: [TimingEvent() for _ in range(n)]
    events = [new_ev(len(phases) + 1) for _ in range(args.steps)]
    perm_ev = [new_ev(2) for _ in range(args.steps)] if xperm is not None else None

    def breakdown_pass():
        """Per-phase events on every step (untimed), then the route call with the materialised permute."""
        for k in range(args.steps):
            if flush is not None:
                flush.sum()
            step(ev=events[k])
            if perm_ev is not None:
                perm_ev[k][0].record(stream)
                rom.route(X, Wr, bias, top_k=1, permute=True, routing=xperm, stream=stream)
                perm_ev[k][1].record(stream)
        torch.cuda.synchronize()

    if flush is None:
        # warm: wall clock over K back-to-back steps; inside them the in-projection is bracketed by events
        # (the roofline's launch time) on every n-th step, so the timed region carries few markers
        every = max(1, args.event_every)
        ins = {k: new_ev(2) for k in range(0, args.steps, every)}
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(args.steps):
            step(around_in=ins.get(k))
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        t_in_timed = np.array([e[0].elapsed_time(e[1]) for e in ins.values()]) * 1e-3
        # per-phase breakdown from a second, untimed pass of the same K steps
        breakdown_pass()
    else:
        # cold cache: the eviction runs between steps and stays outside the timed sum, which adds up the
        # GPU time of each step between two events (none inside the step); the per-phase breakdown comes
        # from a second pass with an event between phases
        bounds = [new_ev(2) for _ in range(args.steps)]
        for k in range(args.steps):
            flush.sum()
            bounds[k][0].record(stream)
            step()
            bounds[k][1].record(stream)
        torch.cuda.synchronize()
        t_step_timed = np.array([b[0].elapsed_time(b[1]) for b in bounds]) * 1e-3
        elapsed = float(t_step_timed.sum())
        t_in_timed = None
        breakdown_pass()

    t_ph = {ph: np.array([e[i].elapsed_time(e[i + 1]) for e in events]) * 1e-3 for i, ph in enumerate(phases)}
    t_step = t_step_timed if flush is not None else np.array([e[0].elapsed_time(e[-1]) for e in events]) * 1e-3
    t_route, t_in = t_ph["route"], (t_in_timed if t_in_timed is not None else t_ph["in"])
    t_out = t_ph.get("out", np.zeros(1))
    # the in-projection's output width: Conv + Gate (2 * d_inner) for RoM, d_out for Swimba
    n_in = w.dout if swimba else 2 * w.d_inner
    fl_in = 2.0 * w.T * w.d_model * n_in * w.top_k
    fl_out = 0.0 if swimba else 2.0 * w.T * w.d_model * w.d_inner * w.top_k
    peak = PEAK_MFMA_TFLOPS[w.dtype]
    counts = routing.counts.cpu().numpy()  # [top_k][E]
    es = 2 if w.dtype == "bf16" else 4
    used = int(np.count_nonzero(counts))  # expert stacks streamed, summed over the choices
    # algorithmic bytes: every operand and result moved once, only the experts that received tokens
    bytes_in = es * (w.T * w.d_model + used * n_in * w.d_model + w.T * n_in)
    bytes_out = 0 if swimba else es * (2 * w.T * w.d_inner + used * w.d_model * w.d_inner + w.T * w.d_model) + 4 * w.T * 2
    # router: X once, W_r once, ids and probabilities out, perm and inv_perm out (per choice)
    bytes_route = es * w.T * w.d_model + 4 * w.d_model * w.E + 4 * w.T * 4 * w.top_k
    bytes_permute = 2 * es * w.T * w.d_model  # X rows read once and written once in slot order
    bytes_conv = es * (2 * w.T * w.d_inner + (CONV_WIDTH + 1) * w.d_inner)
    ms_per_step = elapsed / args.steps * 1e3
    mean_in, mean_out, mean_route = float(t_in.mean()), float(t_out.mean()), float(t_route.mean())
    step_bytes = bytes_route + bytes_in + bytes_out

    if decode:
        # the whole step (router included) against HBM: the used experts' weights dominate its bytes
        mean_step = float(t_step.mean())
        achieved = step_bytes / mean_step / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = fl_in / mean_in / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4)}
    roof["traffic"] = None if decode else measured_traffic(w.name)
    entry = "rom_in_proj_weighted" if swimba else "rom_in_proj"
    if decode:
        roof["kernel"] = ("whole step: rom_route + " + entry + ("" if swimba else " + rom_out_proj") +
                          ", cold caches")
        roof["algorithmic"] = {"bytes_per_step": step_bytes}
        roof["step_us"] = round(float(t_step.mean()) * 1e6, 2)
    else:
        roof["kernel"] = ("k_grouped_gemm_f32" if w.dtype != "bf16" else "k_grouped_gemm_bf16") + f" ({entry})"
        roof["algorithmic"] = {"flops_per_launch": fl_in}
        roof["launch_us"] = round(mean_in * 1e6, 2)

    def pct(a):
        a = np.asarray(a) * 1e6
        return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
                "p90": round(float(np.percentile(a, 90)), 2), "mean": round(float(a.mean()), 2)}

    names = {"route": "rom_route", "in": entry, "conv": "rom_conv1d", "out": "rom_out_proj",
             "obwd": "rom_out_proj_backward", "ibwd": "rom_in_proj_backward"}
    per_call = {names[ph]: pct(t_ph[ph]) for ph in phases}
    per_call["step"] = pct(t_step)

    config = {"workload": w.name, "T": w.T, "d_model": w.d_model, "d_inner": w.d_inner, "E": w.E,
              "top_k": w.top_k, "router": "fp32", "cache": "cold" if cold else "warm",
              "events": "default" if args.fenced_events else "timing-only (hipEventDisableSystemFence)",
              "expert_loads": counts[0].tolist() if w.top_k == 1 else counts.tolist()}
    if swimba:
        config["d_out"] = w.dout
    if conv:
        config["conv1d"] = {"width": CONV_WIDTH, "activation": "silu", "bias": True, "n_seq": w.n_seq}
    result = {
        "metric": METRIC,
        "value": round(w.T * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_s": round(ramp_s, 2),
        "clock_ramp_steps": n_ramp,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic: seeded Gaussian tensors of the workload's shapes (no dataset)",
        "config": config,
        "roofline": roof,
        "breakdown": {
            "route_us": round(mean_route * 1e6, 2),
            "in_proj_us": round(mean_in * 1e6, 2),
            "out_proj_us": round(mean_out * 1e6, 2),
            "in_proj_tflops": round(fl_in / mean_in / 1e12, 1),
            "out_proj_tflops": round(fl_out / mean_out / 1e12, 1) if mean_out > 0 else 0.0,
            "gemm_mfma_frac": round((fl_in + fl_out) / (mean_in + mean_out) / 1e12 / peak, 4),
            "route_gbs": round(bytes_route / mean_route / 1e9, 1),
            "in_proj_gbs": round(bytes_in / mean_in / 1e9, 1),
            "out_proj_gbs": round(bytes_out / mean_out / 1e9, 1) if mean_out > 0 else 0.0,
            "step_hbm_frac": round(step_bytes / (mean_route + mean_in + mean_out) / 1e9 / PEAK_HBM_GBS, 4),
            "in_proj_hbm_frac": round(bytes_in / mean_in / 1e9 / PEAK_HBM_GBS, 4),
            "per_call_us": per_call,
        },
        "cpu_baseline": None,
    }
    if perm_ev is not None:
        t_rp = np.array([e[0].elapsed_time(e[1]) for e in perm_ev]) * 1e-3
        # the permute runs inside the router's scatter kernel: its cost is the router call's extra time
        t_perm = max(float(np.median(t_rp)) - float(np.median(t_route)), 1e-9)
        result["breakdown"]["permute"] = {
            "route_with_permute_us": pct(t_rp),
            "permute_us": round(t_perm * 1e6, 2),
            "permute_bytes": bytes_permute,
            "permute_gbs": round(bytes_permute / t_perm / 1e9, 1),
        }
    if bwd:
        for ph, key, mult in (("obwd", "out_proj_backward", 4), ("ibwd", "in_proj_backward", 8)):
            tm = float(t_ph[ph].mean())
            fl = mult * w.T * w.d_model * w.d_inner * w.top_k
            result["breakdown"][key + "_us"] = round(tm * 1e6, 2)
            result["breakdown"][key + "_tflops"] = round(fl / tm / 1e12, 1)
        fwd_fl = fl_in + fl_out
        all_fl = fwd_fl + 12.0 * w.T * w.d_model * w.d_inner * w.top_k
        result["breakdown"]["fwd_bwd_tflops"] = round(all_fl / (elapsed / args.steps) / 1e12, 1)
        config["backward"] = True
    if conv:
        mean_conv = float(t_ph["conv"].mean())
        result["breakdown"]["conv1d_us"] = round(mean_conv * 1e6, 2)
        result["breakdown"]["conv1d_gbs"] = round(bytes_conv / mean_conv / 1e9, 1)
        result["breakdown"]["conv1d_hbm_frac"] = round(bytes_conv / mean_conv / 1e9 / PEAK_HBM_GBS, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_seconds, conv, bwd)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
