#!/usr/bin/env python3
"""Sign-Muon optimizer-step benchmark on one MI355X.

Times the fused step (signmuon_step: momentum sweep, PolarNS by Newton-Schulz
on the matrix cores, sign + 1-bit pack into the local worker's buffer, vote
over the M resident packed buffers fused with the update of W) on a synthetic
parameter set with all inputs resident in HBM.  Prints one JSON line with
steps/s, a per-phase breakdown measured with HIP events recorded on the
launch stream inside instrumented steps (the same work with the phases in
sequence), the roofline of the dominant kernel (the Newton-Schulz GEMM) and
the CPU oracle timed on a bounded sample.  `value` times plain steps, in
which the momentum sweep, Newton-Schulz and vote of different matrix groups
overlap on the library's internal streams.  An extra figure, `all_workers`,
times steps in which all M workers' pipelines run on this GPU
(signmuon_worker_pipeline for workers 1..M-1, then the step for worker 0).

`other_workloads` gives the plain steps/s and phase times of further sets
(by default the ResNet-50-shaped one and the nanoGPT set with both polar
steps, before the sign and after the vote).

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload nanogpt]
                    [--also resnet50,nanogpt_prepost]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Sign-Muon steps/s on nanoGPT-124M params; NS MFMA util %; vote GB/s"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 matrix-core peak
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E


def ns_form(w) -> str:
    """The library's Newton-Schulz form for this workload: Gram space for
    bfloat16 cubic steps with the Frobenius scale (unless SIGNMUON_NS_FORM
    is 'iterate'), else the iterate form."""
    if os.environ.get("SIGNMUON_NS_FORM") == "iterate":
        return "iterate"
    if w.ns_precision == "bf16" and w.coeffs[2] == 0.0 and w.scale == "fro" and w.K > 0:
        return "gram_space"
    return "iterate"


def executed_ns_gflop(w) -> float:
    """MFMA flops the library executes for one step's Newton-Schulz work:
    operands padded to multiples of 128, symmetric outputs (Grams, the
    quintic square, the Gram-space products) on their upper-triangular
    128x128 tiles only, the update on every tile; split-bfloat16 runs three
    MFMAs per product.  Gram space: one Gram, 3K - 3 symmetric Rp x Rp
    products and one Rp x Rp by Rp x Np product."""
    r128 = lambda x: (x + 127) // 128 * 128  # noqa: E731
    gram_space = ns_form(w) == "gram_space"
    tot = 0.0
    for r, c in w.mats:
        Rp, Np = r128(min(r, c)), r128(max(r, c))
        T = Rp // 128
        sym = T * (T + 1) // 2 * 2.0 * 128 * 128
        if gram_space:
            tot += sym * Np + max(0, 3 * w.K - 3) * sym * Rp + 2.0 * Rp * Rp * Np
            continue
        per = sym * Np + 2.0 * Rp * Rp * Np
        if w.coeffs[2] != 0.0:
            per += sym * Rp
        tot += w.K * per
    return tot * (3 if w.ns_precision == "bf16x3" else 1) / 1e9


def gemm_traffic(workload):
    """HBM bytes of one step's Newton-Schulz GEMM launches from the committed
    counter summary, if it was taken on the current GEMM source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"k_gemm_{workload}_hbm_traffic.md")
    src = os.path.join(ROOT, "distributed_bit_matrix_amd", "csrc", "sm_gemm.hip")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if fields.get("gemm_source_sha256") != digest:
        return None
    try:
        return int(fields["gemm_traffic_bytes_per_step"])
    except (KeyError, ValueError):
        return None


def hip_runtime():
    L = ctypes.CDLL("libamdhip64.so")
    L.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    L.hipEventDestroy.argtypes = [ctypes.c_void_p]
    L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                      ctypes.c_void_p]
    return L


def describe(w):
    shapes = {}
    for s in w.mats:
        shapes[s] = shapes.get(s, 0) + 1
    parts = ", ".join(f"{n}x({r}x{c})" for (r, c), n in shapes.items())
    ns = {"f32": "f32", "bf16": "bf16 operands / f32 accumulate",
          "bf16x3": "split-bf16 (x3)"}[w.ns_precision]
    coeffs = "quintic" if w.coeffs[2] else "cubic"
    enc = "int8 ternary" if w.encoding == "ternary" else "packed"
    return (f"{w.name}: {parts}; W {w.w_dtype}, momentum f32; M={w.M} resident {enc} "
            f"sign buffers; K={w.K} {coeffs} Newton-Schulz ({ns}), {w.scale} scaling"
            + (f" P={w.P}" if w.scale == "spectral" else "")
            + {0: "", 1: "; post-vote polar", 2: "; pre-sign and post-vote polar"}[int(w.post_vote)])


def cpu_baseline(w, budget_s):
    """Oracle seconds per step on a bounded sample, scaled to the whole set."""
    import oracle as O
    from distributed_bit_matrix_amd import workloads as WL
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # threadpoolctl missing: report the visible CPUs
        cores = os.cpu_count()
    # sample: the first 1/L of the matrices (one transformer layer for the
    # nanoGPT set), worker 0's pipeline + vote over M + apply
    per_layer = 4 if w.name == "nanogpt" else 1
    n_layers = len(w.mats) // per_layer
    sub = WL.scaled(w, w.mats[:per_layer], name=w.name + "-sample")
    hp = dict(eta=w.eta, beta=w.beta, lam=w.lam, eps=w.eps, K=w.K, scale=w.scale,
              P=w.P, coeffs=w.coeffs)
    W = WL.init_weights(sub).astype(np.float64)
    Mom = np.zeros(sub.d)
    G = WL.gradient(sub, 0, 0).astype(np.float64)
    others = WL.random_bits(sub, w.M)
    u0s = WL.power_start(sub) if w.scale == "spectral" else None
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        Mn = O.momentum_update(Mom, G, W, hp["beta"], hp["lam"])
        bits = others.copy()
        for i, ((r, c), off, woff) in enumerate(zip(sub.mats, sub.elem_offsets,
                                                    sub.word_offsets)):
            U, _ = O.polar_ns(Mn[off:off + r * c].reshape(r, c), hp["K"], hp["eps"],
                              hp["scale"], hp["P"], hp["coeffs"],
                              None if u0s is None else u0s[i])
            bits[0, woff:woff + (r * c + 31) // 32] = O.pack_signs(U)
            sums = O.vote_sums_from_bits(bits[:, woff:woff + (r * c + 31) // 32], r * c)
            D = O.majority_from_sums(sums, w.tie_value)
            O.apply_update(W[off:off + r * c], D, hp["eta"], w.w_dtype)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s or len(times) >= 5:
            break
    t_sample = float(np.median(times))
    t_step = t_sample * n_layers
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{per_layer} of {len(w.mats)} matrices ({sub.d} of {w.d} parameters), "
                       f"worker-0 momentum + float64 Newton-Schulz + pack, vote over M={w.M} "
                       f"and apply; median of {len(times)} runs = {t_sample:.3f} s, "
                       f"x{n_layers} for the whole set"),
            "seconds_per_step": t_step}


class Run:
    """One workload on the GPU: its plan, resident inputs, and the timing of
    K plain steps followed by K instrumented steps (phases in sequence, an
    event after each phase)."""

    def __init__(self, w, dev):
        import torch
        from distributed_bit_matrix_amd import binding as B
        from distributed_bit_matrix_amd import workloads as WL
        self.w = w
        hp = B.HParams(eta=w.eta, beta=w.beta, lam=w.lam, eps=w.eps, K=w.K, scale=w.scale,
                       P=w.P, coeffs=w.coeffs, precision=w.ns_precision,
                       tie_value=w.tie_value, encoding=w.encoding)
        layout, self.d, self.words = B.default_layout(w.mats)
        self.plan = B.StepPlan(layout, hp, w.post_vote, device=dev)
        wdt = torch.bfloat16 if w.w_dtype == "bf16" else torch.float32
        self.W = torch.from_numpy(WL.init_weights(w)).to(dev).to(wdt)
        self.Mom = torch.zeros(self.d, dtype=torch.float32, device=dev)
        self.G = torch.from_numpy(WL.gradient(w, 0, 0)).to(dev)
        if w.encoding == "ternary":
            # int8 sign buffers: d bytes per worker, matrices at their offsets
            self.bits = torch.from_numpy(WL.random_ternary(w, w.M)).to(dev)
            self.words = self.d
        else:
            self.bits = torch.from_numpy(WL.random_bits(w, w.M).view(np.int32)).to(dev)
        self.u0 = (torch.from_numpy(np.concatenate(WL.power_start(w))).to(dev)
                   if w.scale == "spectral" else None)
        torch.cuda.synchronize()

    def step(self):
        self.plan(self.G, self.W, self.Mom, self.bits, self.words, self.w.M, 0, u0=self.u0)

    def measure(self, K, warmup):
        """Returns (seconds for K plain steps, mean per-phase microseconds)."""
        import torch
        from distributed_bit_matrix_amd import binding as B
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()

        # events for the instrumented steps
        hip = hip_runtime()
        cap = 64
        evs = (ctypes.c_void_p * (cap * K))()
        ev_list = []
        for i in range(cap * K):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            ev_list.append(e.value)
            evs[i] = e.value
        kinds = (ctypes.c_int32 * (cap * K))()
        profs = []
        for k in range(K):
            p = B.SmProfile()
            p.events = ctypes.cast(ctypes.byref(evs, k * cap * ctypes.sizeof(ctypes.c_void_p)),
                                   ctypes.POINTER(ctypes.c_void_p))
            p.kinds = ctypes.cast(ctypes.byref(kinds, k * cap * 4),
                                  ctypes.POINTER(ctypes.c_int32))
            p.capacity = cap
            p.count = 0
            profs.append(p)

        # timed region: K production steps (the whole step runs as concurrent
        # chains on the library's streams), bracketed by device synchronization
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(K):
            self.step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

        # K instrumented steps for the phase breakdown: the same work with the
        # phases in sequence and an event after each (Newton-Schulz chains
        # only inside the polar phase)
        torch.cuda.synchronize()
        w = self.w
        for k in range(K):
            self.plan.profiled(profs[k], self.G, self.W, self.Mom, self.bits, self.words,
                               w.M, 0, u0=self.u0)
        torch.cuda.synchronize()

        # per-phase durations from consecutive events of each step
        phase = {}
        ms = ctypes.c_float()
        for k in range(K):
            p = profs[k]
            base = k * cap
            for i in range(1, p.count):
                hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[base + i - 1]),
                                        ctypes.c_void_p(evs[base + i]))
                name = B.PHASES[kinds[base + i]]
                phase[name] = phase.get(name, 0.0) + ms.value * 1e3
        for e in ev_list:
            hip.hipEventDestroy(ctypes.c_void_p(e))
        return elapsed, {k: v / K for k, v in phase.items()}


def main():
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="nanogpt")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--rb-steps", type=int, default=5,
                    help="timed steps of the all-workers figure (every worker's pipeline "
                         "inside the step)")
    ap.add_argument("--also", default="resnet50,nanogpt_prepost,nanogpt_ternary",
                    help="comma-separated further workloads whose plain steps/s and phase "
                         "times are reported under other_workloads ('' = none)")
    ap.add_argument("--ternary", type=int, default=1,
                    help="also time the int8 ternary vote on the set's size (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one plain elementwise kernel that reads and writes "
                         "MIB MiB (reference for hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        sys.exit("bench.py measures one GPU: the method's M workers are resident sign "
                 "buffers on a single MI355X; --gpus above 1 is not supported")

    import torch
    from distributed_bit_matrix_amd import workloads as WL

    w = WL.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)          # reads and writes n * 4 bytes
        torch.cuda.synchronize()
        del src, dst

    run = Run(w, dev)
    K = args.steps
    elapsed, phase_us = run.measure(K, args.warmup)
    d, words, plan = run.d, run.words, run.plan
    G, W, bits, u0 = run.G, run.W, run.bits, run.u0
    step = run.step
    # The Newton-Schulz GEMM launches of a step run as concurrent chains on
    # the library's internal streams; the "gemm" phase is the span from the
    # fork to the join on the launching stream (pre-scale included).
    gemm_us = phase_us.get("gemm", float("nan"))
    quintic = w.coeffs[2] != 0.0
    # GEMM launches per chain and step: iterate form K Grams + K updates
    # (+ K squares for the quintic); Gram space one Gram, 3K - 3 symmetric
    # products and the final product
    gemm_per_step = 3 * w.K - 1 if ns_form(w) == "gram_space" else w.K * (3 if quintic else 2)

    ns_flop = w.ns_gflop() * 1e9
    ns_tflops = ns_flop / (gemm_us * 1e-6) / 1e12
    exec_tflops = executed_ns_gflop(w) * 1e9 / (gemm_us * 1e-6) / 1e12
    peak = PEAK_F32_TFLOPS if w.ns_precision == "f32" else PEAK_BF16_TFLOPS
    wbytes = 2 if w.w_dtype == "bf16" else 4
    vote_bytes = (w.M / 8.0 + 2 * wbytes) * d
    vote_gbps = vote_bytes / (phase_us.get("vote", float("nan")) * 1e-6) / 1e9
    mom_bytes = (4 + wbytes + 4 + 4 + 2) * d
    mom_gbps = mom_bytes / (phase_us.get("momentum", float("nan")) * 1e-6) / 1e9

    # An extra figure: every worker's pipeline inside the step.
    # Workers 1..M-1 run signmuon_worker_pipeline into their buffers with
    # momenta of their own (the gradient values do not change the time, so
    # they share G), then worker 0 runs the full step (its pipeline, the vote
    # over the M fresh buffers and the apply).
    # (At most 8 momentum buffers are kept and reused in turn: the work per
    # worker is the same, and 200 workers' momenta would not fit in HBM.)
    rb_steps = max(1, min(args.rb_steps, K))
    n_mom = min(w.M - 1, 8)
    Moms_b = [torch.zeros(d, dtype=torch.float32, device=dev) for _ in range(n_mom)]

    def step_all_workers():
        for m in range(1, w.M):
            plan.worker_pipeline(G, W, Moms_b[(m - 1) % n_mom], bits, words, w.M, m, u0=u0)
        step()

    step_all_workers()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(rb_steps):
        step_all_workers()
    torch.cuda.synchronize()
    rb_elapsed = time.perf_counter() - t0
    del Moms_b

    # Further workloads (by default the ResNet-50-shaped set and the nanoGPT
    # set with both polar steps): plain steps/s
    # and the instrumented phase times, same method as above.
    others = {}
    for name in [n for n in args.also.split(",") if n and n != w.name]:
        wo = WL.get(name)
        ro = Run(wo, dev)
        el, ph = ro.measure(K, args.warmup)
        others[name] = {"value": round(K / el, 3), "unit": "steps/s",
                        "ms_per_step": round(el / K * 1e3, 4), "config": describe(wo),
                        "params": ro.d,
                        "phases_us": {k: round(v, 2) for k, v in ph.items()}}
        del ro
        torch.cuda.synchronize()

    # The int8 ternary vote (separate entry point, not part of the step) on
    # the same set's size: M int8 buffers read, int8 D written.
    tern = None
    if args.ternary:
        from distributed_bit_matrix_amd import binding as B
        d_t, M_t = w.d, w.M
        S_t = torch.randint(-1, 2, (M_t * d_t,), dtype=torch.int8, device=dev)
        D_t = torch.empty(d_t, dtype=torch.int8, device=dev)
        for _ in range(2):
            B.majority_vote_ternary(S_t, M_t, d_t, 0, D=D_t)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 10
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            B.majority_vote_ternary(S_t, M_t, d_t, 0, D=D_t)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        by = (M_t + 1) * d_t
        tern = {"us": round(us, 2), "bytes": by, "gbps": round(by / (us * 1e-6) / 1e9, 1),
                "frac_hbm": round(by / (us * 1e-6) / 8e12, 4),
                "what": f"signmuon_majority_vote_ternary over M={M_t} int8 buffers of "
                        f"{d_t} entries (reads M d bytes, writes d)"}
        del S_t, D_t

    steps_per_s = K / elapsed
    out = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.ns_precision != "f32" else "f32",
        "data": "synthetic",
        "config": {"workload": describe(w), "params": d, "matrices": len(w.mats),
                   "workers": w.M, "reading": "local worker pipeline + vote over M "
                   "resident buffers + apply"},
        "roofline": {"bound": "mfma", "achieved": round(ns_tflops, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(ns_tflops / peak, 4),
                     "traffic": gemm_traffic(w.name), "traffic_unit": "bytes per step",
                     "kernel": "k_gemm: the step's Newton-Schulz GEMM launches, timed as one phase",
                     "work": "algorithmic: 4 m^2 n flops per Newton-Schulz step and matrix, the "
                             "pages' iteration; see ns_executed_tflops for the MFMA flops the "
                             "chosen form executes",
                     "ns_form": ns_form(w),
                     "gemm_phases_per_step": gemm_per_step,
                     "ns_phase_us": round(gemm_us, 2)},
        # MFMA utilisation: the MFMA flops actually executed (the chosen form,
        # symmetric outputs on their upper-triangular tiles, padded operands)
        # over the phase time, against the peak
        "ns_mfma_util_pct": round(100 * exec_tflops / peak, 2),
        "ns_executed_tflops": round(exec_tflops, 2),
        # the pages' iteration's flops over the same time (the roofline above)
        "ns_algorithmic_pct_of_peak": round(100 * ns_tflops / peak, 2),
        "vote_gbps": round(vote_bytes / (phase_us.get("vote", float("nan")) * 1e-6) / 1e9, 1),
        "vote_frac_hbm": round(vote_gbps / PEAK_HBM_GBPS, 4),
        "momentum_gbps": round(mom_gbps, 1),
        "phases_us": {k: round(v, 2) for k, v in phase_us.items()},
        "instrumented_us_per_step": round(sum(phase_us.values()), 2),
        "all_workers": {"value": round(rb_steps / rb_elapsed, 3), "unit": "steps/s",
                      "steps": rb_steps, "ms_per_step": round(rb_elapsed / rb_steps * 1e3, 3),
                      "what": f"all {w.M} workers' momentum + PolarNS + pack on this GPU, "
                              "then the vote over the M buffers and the apply",
                      "momentum_buffers": n_mom + 1},
        "other_workloads": others,
        "ternary_vote": tern,
    }
    if args.cpu_budget > 0:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
