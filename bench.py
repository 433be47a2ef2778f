#!/usr/bin/env python3
"""Sign-Muon optimizer-step benchmark on one MI355X.

Times the fused step (signmuon_step: momentum sweep, PolarNS by Newton-Schulz
on the matrix cores, sign + 1-bit pack into the local worker's buffer, vote
over the M resident packed buffers fused with the update of W) on a synthetic
parameter set with all inputs resident in HBM, and prints one JSON line:

* `value`: steps/s of plain steps (the PolarNS work of different matrix
  groups runs as concurrent chains on the plan's executor);
* `phases_us` and the `ns_*` / `vote_*` / `momentum_*` rates: instrumented
  steps with a HIP event after each phase, on the launch stream; the
  momentum pass and every vote launch are timed by their own kernel start
  and stop (the interval before each is `hbm_gap`), as are the matrix-core
  launches outside the concurrent chains (`gap`);
* `roofline`: the dominant matrix-core kernel, timed per launch between HIP
  events in sequential steps (no executor: each launch alone on the stream);
* `other_workloads`: the same figures for the other parameter sets (the
  ResNet-50-shaped set, the single 256x512 matrix, the LLM-MLP matrices with
  the cubic and the quintic, the post-vote set with M = 200, and the nanoGPT
  set with both polar steps, int8 ternary buffers and the normalized sign
  step); `k_curve`: the main set at other Newton-Schulz step counts;
* `all_workers`: steps in which all M workers' pipelines run on this GPU;
* `cpu_baseline`: the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload nanogpt]
                    [--also resnet50,...] [--k-curve 3,10]
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


def gemm_traffic(workload, kind):
    """HBM bytes (read + written) of one launch of the matrix-core kernel
    `kind` in the sequential steps, from the committed counter summary, if
    it was taken on the current GEMM source; else None."""
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
        return int(fields[f"traffic_bytes_per_launch_{kind}"])
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
            + {0: "", 1: "; post-vote polar", 2: "; pre-sign and post-vote polar",
               3: "; normalized sign step D/||D||_2"}[int(w.post_vote)])


def host_info():
    """CPU model, thread count and NumPy's BLAS on this host."""
    model = None
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    blas = None
    try:
        from threadpoolctl import threadpool_info
        infos = threadpool_info()
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}"
                                 for i in infos if i.get("user_api") == "blas"})) or None
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "numpy_blas": blas}


def cpu_baseline(w, budget_s):
    """Oracle seconds per step on a bounded sample, scaled to the whole set:
    worker 0's momentum, float64 Newton-Schulz and sign packing, the vote over
    M buffers and the apply for the first transformer layer's matrices, with
    all BLAS threads; then one pass of the same sample on one thread."""
    import oracle as O
    from distributed_bit_matrix_amd import workloads as WL
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:   # threadpoolctl missing: report the visible CPUs
        threadpool_limits = None
        cores = os.cpu_count()
    per_layer = 4 if w.name.startswith("nanogpt") else 1
    n_layers = len(w.mats) // per_layer
    sub = WL.scaled(w, w.mats[:per_layer], name=w.name + "-sample")
    hp = dict(eta=w.eta, beta=w.beta, lam=w.lam, eps=w.eps, K=w.K, scale=w.scale,
              P=w.P, coeffs=w.coeffs)
    W = WL.init_weights(sub).astype(np.float64)
    Mom = np.zeros(sub.d)
    G = WL.gradient(sub, 0, 0).astype(np.float64)
    others = WL.random_bits(sub, w.M)
    u0s = WL.power_start(sub) if w.scale == "spectral" else None

    def one_pass():
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
        return time.perf_counter() - t0

    times = []
    t_all = time.perf_counter()
    while True:
        times.append(one_pass())
        if time.perf_counter() - t_all > budget_s or len(times) >= 5:
            break
    t_sample = float(np.median(times))
    single = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            t1 = one_pass()
        single = {"value": 1.0 / (t1 * n_layers), "seconds_per_step": t1 * n_layers,
                  "cores": 1}
    t_step = t_sample * n_layers
    return {"value": 1.0 / t_step, "unit": "steps/s", "cores": int(cores), "kind": "oracle",
            "sample": (f"{per_layer} of {len(w.mats)} matrices ({sub.d} of {w.d} parameters), "
                       f"worker-0 momentum + float64 Newton-Schulz + pack, vote over M={w.M} "
                       f"and apply; median of {len(times)} runs = {t_sample:.3f} s, "
                       f"x{n_layers} for the whole set"),
            "seconds_per_step": t_step, "single_thread": single, "host": host_info()}


class Run:
    """One workload on the GPU: its plans, resident inputs, and the timing of
    K plain steps, K instrumented steps (phases in sequence, an event after
    each phase; the Newton-Schulz chains run concurrently inside their phase)
    and K sequential instrumented steps (no executor: every matrix-core launch
    alone on the stream, an event after each)."""

    def __init__(self, w, dev, seed=0):
        import torch
        from distributed_bit_matrix_amd import binding as B
        from distributed_bit_matrix_amd import workloads as WL
        self.w = w
        self.hp = B.HParams(eta=w.eta, beta=w.beta, lam=w.lam, eps=w.eps, K=w.K,
                            scale=w.scale, P=w.P, coeffs=w.coeffs, precision=w.ns_precision,
                            tie_value=w.tie_value, encoding=w.encoding)
        self.layout, self.d, self.words = B.default_layout(w.mats)
        self.plan = B.StepPlan(self.layout, self.hp, w.post_vote, device=dev)
        self.plan_seq = None
        wdt = torch.bfloat16 if w.w_dtype == "bf16" else torch.float32
        self.W = torch.from_numpy(WL.init_weights(w)).to(dev).to(wdt)
        self.Mom = torch.zeros(self.d, dtype=torch.float32, device=dev)
        self.G = torch.from_numpy(WL.gradient(w, 0, 0)).to(dev)
        # the other workers' buffers: seeded random signs generated on the
        # device (their values do not change the time)
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed + 1000 * seed)
        if w.encoding == "ternary":
            # int8 sign buffers: d bytes per worker, matrices at their offsets
            self.bits = torch.randint(-1, 2, (w.M, self.d), dtype=torch.int8, device=dev,
                                      generator=g)
            self.words = self.d
        else:
            self.bits = torch.randint(-2 ** 31, 2 ** 31 - 1, (w.M, self.words),
                                      dtype=torch.int32, device=dev, generator=g)
        self.u0 = (torch.from_numpy(np.concatenate(WL.power_start(w))).to(dev)
                   if w.scale == "spectral" else None)
        self.dev = dev
        torch.cuda.synchronize()

    def step(self):
        self.plan(self.G, self.W, self.Mom, self.bits, self.words, self.w.M, 0, u0=self.u0)

    def _profiled(self, plan, K):
        """K instrumented steps on `plan`: per-phase and per-kind durations
        (microseconds per step) and per-launch durations by kind."""
        import torch
        from distributed_bit_matrix_amd import binding as B
        hip = hip_runtime()
        cap = 128
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
        torch.cuda.synchronize()
        w = self.w
        for k in range(K):
            plan.profiled(profs[k], self.G, self.W, self.Mom, self.bits, self.words, w.M, 0,
                          u0=self.u0)
        torch.cuda.synchronize()
        phase, launches = {}, {}
        ms = ctypes.c_float()
        for k in range(K):
            p = profs[k]
            if p.count >= cap:
                raise RuntimeError("profile capacity too small")
            base = k * cap
            for i in range(1, p.count):
                hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[base + i - 1]),
                                        ctypes.c_void_p(evs[base + i]))
                name = B.PHASES[kinds[base + i]]
                # the gap before the sweep or the vote (which the profiled
                # step times by their own start and stop) is not part of
                # the Newton-Schulz phase
                if name == "gap" and i + 1 < p.count and \
                        B.PHASES[kinds[base + i + 1]] in ("momentum", "vote"):
                    name = "hbm_gap"
                phase[name] = phase.get(name, 0.0) + ms.value * 1e3
                launches.setdefault(name, []).append(ms.value * 1e3)
        for e in ev_list:
            hip.hipEventDestroy(ctypes.c_void_p(e))
        return {k: v / K for k, v in phase.items()}, launches

    def measure(self, K, warmup):
        """Returns (seconds for K plain steps, mean per-phase microseconds of
        the instrumented steps)."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        # timed region: K production steps (the PolarNS work runs as
        # concurrent chains on the plan's executor), bracketed by device
        # synchronization
        t0 = time.perf_counter()
        for k in range(K):
            self.step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        phase, _ = self._profiled(self.plan, K)
        return elapsed, phase

    def measure_launches(self, K):
        """K sequential instrumented steps: mean microseconds per launch of
        each matrix-core kernel kind (gram, square, update; the kernel's own
        start-to-stop time) and per step."""
        from distributed_bit_matrix_amd import binding as B
        if self.plan_seq is None:
            self.plan_seq = B.StepPlan(self.layout, self.hp, self.w.post_vote, device=self.dev,
                                       concurrent=False)
        self._profiled(self.plan_seq, 1)          # warm-up
        phase, launches = self._profiled(self.plan_seq, K)
        per_launch = {k: float(np.mean(v)) for k, v in launches.items()}
        counts = {k: len(v) // K for k, v in launches.items()}
        return phase, per_launch, counts


def launch_flops(w):
    """Executed MFMA flops of one launch of each matrix-core kernel kind over
    the whole set (operands padded to multiples of 128; symmetric outputs on
    their upper-triangular 128x128 tiles; three MFMAs per product in
    split-bfloat16), for the launches the sequential step makes."""
    r128 = lambda x: (x + 127) // 128 * 128  # noqa: E731
    mul = 3 if w.ns_precision == "bf16x3" else 1
    gram = square = update = 0.0
    for r, c in w.mats:
        Rp, Np = r128(min(r, c)), r128(max(r, c))
        T = Rp // 128
        sym = T * (T + 1) // 2 * 2.0 * 128 * 128
        gram += sym * Np
        square += sym * Rp
        update += 2.0 * Rp * Rp * Np
    return {"gram": gram * mul, "square": square * mul, "update": update * mul}


def workload_metrics(w, d, elapsed, K, phase_us):
    """Steps/s, the Newton-Schulz phase as algorithmic and executed TFLOP/s
    against the matrix-core peak, and vote / momentum GB/s against HBM."""
    peak = PEAK_F32_TFLOPS if w.ns_precision == "f32" else PEAK_BF16_TFLOPS
    # (the matrix-core launches and the gaps between them: launch latency and
    # split-k reductions)
    gemm_us = phase_us.get("gemm", 0.0) + phase_us.get("gram", 0.0) + \
        phase_us.get("square", 0.0) + phase_us.get("update", 0.0) + phase_us.get("gap", 0.0)
    wbytes = 2 if w.w_dtype == "bf16" else 4
    sign_bytes = 1.0 if w.encoding == "ternary" else 1 / 8.0
    out = {"value": round(K / elapsed, 3), "unit": "steps/s",
           "ms_per_step": round(elapsed / K * 1e3, 4), "config": describe(w), "params": d,
           "phases_us": {k: round(v, 2) for k, v in phase_us.items()}}
    if gemm_us > 0 and w.K > 0:
        alg = w.ns_gflop() * 1e9 / (gemm_us * 1e-6) / 1e12
        exe = executed_ns_gflop(w) * 1e9 / (gemm_us * 1e-6) / 1e12
        if w.post_vote == 2:      # two Newton-Schulz passes per step
            alg, exe = 2 * alg, 2 * exe
        out.update({"ns_phase_us": round(gemm_us, 2), "ns_form": ns_form(w),
                    "ns_algorithmic_tflops": round(alg, 1),
                    "ns_algorithmic_frac": round(alg / peak, 4),
                    "ns_executed_tflops": round(exe, 1),
                    "ns_mfma_util_pct": round(100 * exe / peak, 2)})
    if w.post_vote == 0 and phase_us.get("vote"):
        vb = (w.M * sign_bytes + 2 * wbytes) * d
        out["vote_apply_gbps"] = round(vb / (phase_us["vote"] * 1e-6) / 1e9, 1)
        out["vote_apply_frac_hbm"] = round(vb / (phase_us["vote"] * 1e-6) / 1e9 /
                                           PEAK_HBM_GBPS, 4)
    elif phase_us.get("vote"):
        # majority matrix written into the bfloat16 operand copy (the
        # normalized step then votes again, applying c D to W)
        vb = (w.M * sign_bytes + 2) * d
        if w.post_vote == 3:
            vb += (w.M * sign_bytes + 2 * wbytes) * d
        out["vote_gbps"] = round(vb / (phase_us["vote"] * 1e-6) / 1e9, 1)
        out["vote_frac_hbm"] = round(vb / (phase_us["vote"] * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)
    if phase_us.get("momentum"):
        mb = (4 + wbytes + 4 + 4 + (0 if w.post_vote == 1 else 2)) * d + \
            (sign_bytes * d if w.post_vote == 1 else 0)
        out["momentum_gbps"] = round(mb / (phase_us["momentum"] * 1e-6) / 1e9, 1)
        out["momentum_frac_hbm"] = round(mb / (phase_us["momentum"] * 1e-6) / 1e9 /
                                         PEAK_HBM_GBPS, 4)
    return out


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
                         "inside the step; 0 = skip)")
    ap.add_argument("--also", default=("resnet50,single,llm_mlp,llm_mlp_quintic,postvote,"
                                       "nanogpt_prepost,nanogpt_ternary,nanogpt_normalized"),
                    help="comma-separated further workloads whose steps/s, phase times and "
                         "rates are reported under other_workloads ('' = none)")
    ap.add_argument("--k-curve", default="3,10",
                    help="Newton-Schulz step counts K at which the main workload is also "
                         "timed ('' = none)")
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
    main_metrics = workload_metrics(w, run.d, elapsed, K, phase_us)
    # Roofline of the dominant kernel: the matrix-core launches of K
    # sequential instrumented steps (no executor), each timed alone between
    # HIP events on its stream.  In the Gram-space form the symmetric
    # Rp x Rp products take most of the Newton-Schulz time.
    seq_phase, per_launch, counts = run.measure_launches(K)
    lf = launch_flops(w)
    kinds = [k for k in ("gram", "square", "update") if k in per_launch]
    dom = max(kinds, key=lambda k: per_launch[k] * counts[k])
    peak = PEAK_F32_TFLOPS if w.ns_precision == "f32" else PEAK_BF16_TFLOPS
    achieved = lf[dom] / (per_launch[dom] * 1e-6) / 1e12
    names = {"gram": "k_gemm Gram S S^T (E_OP)",
             "square": "k_gemm symmetric Rp x Rp product (E_SQUARE)",
             "update": "k_gemm update / final product (E_UPDATE)"}
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": gemm_traffic(w.name, dom), "traffic_unit": "HBM bytes per launch",
                "kernel": names[dom] + f": one launch covers all {len(w.mats)} matrices",
                "work_per_launch_gflop": round(lf[dom] / 1e9, 3),
                "work": {"square": "2 Rp^3 flops per matrix (Rp = the short side padded "
                                   "to 128) on the upper-triangular 128x128 tiles of the "
                                   "symmetric output",
                         "gram": "2 Rp^2 Np flops per matrix on the upper-triangular tiles "
                                 "of the symmetric Gram",
                         "update": "2 Rp^2 Np flops per matrix"}[dom]
                        + (" (x3 MFMAs in split-bfloat16)" if w.ns_precision == "bf16x3" else ""),
                "avg_launch_us": round(per_launch[dom], 2), "launches_per_step": counts[dom],
                "timed_launches": counts[dom] * K,
                "per_kind": {k: {"avg_launch_us": round(per_launch[k], 2),
                                 "launches_per_step": counts[k],
                                 "tflops": round(lf[k] / (per_launch[k] * 1e-6) / 1e12, 1),
                                 "frac": round(lf[k] / (per_launch[k] * 1e-6) / 1e12 / peak, 4)}
                             for k in kinds},
                "sequential_step_phases_us": {k: round(v, 2) for k, v in seq_phase.items()}}
    d, words, plan = run.d, run.words, run.plan
    G, W, bits, u0 = run.G, run.W, run.bits, run.u0
    step = run.step

    # An extra figure: every worker's pipeline inside the step.
    # Workers 1..M-1 run signmuon_worker_pipeline into their buffers with
    # momenta of their own (the gradient values do not change the time, so
    # they share G), then worker 0 runs the full step (its pipeline, the vote
    # over the M fresh buffers and the apply).
    # (At most 8 momentum buffers are kept and reused in turn: the work per
    # worker is the same, and 200 workers' momenta would not fit in HBM.)
    all_workers = None
    if args.rb_steps > 0:
        rb_steps = min(args.rb_steps, K)
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
        all_workers = {"value": round(rb_steps / rb_elapsed, 3), "unit": "steps/s",
                       "steps": rb_steps, "ms_per_step": round(rb_elapsed / rb_steps * 1e3, 3),
                       "what": f"all {w.M} workers' momentum + PolarNS + pack on this GPU, "
                               "then the vote over the M buffers and the apply",
                       "momentum_buffers": n_mom + 1}

    # The int8 ternary vote (separate entry point) on the same set's size:
    # M int8 buffers read, int8 D written.
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
    del run, plan, G, W, bits, u0, step
    torch.cuda.empty_cache()

    # Further workloads: the same plain and instrumented timing
    others = {}
    for name in [n for n in args.also.split(",") if n and n != w.name]:
        wo = WL.get(name)
        ro = Run(wo, dev)
        el, ph = ro.measure(K, args.warmup)
        others[name] = workload_metrics(wo, ro.d, el, K, ph)
        del ro
        torch.cuda.empty_cache()

    # Newton-Schulz step count: the main workload at other K
    k_curve = {str(w.K): {"value": main_metrics["value"],
                          "ns_phase_us": main_metrics.get("ns_phase_us")}}
    for k in [int(x) for x in args.k_curve.split(",") if x]:
        wk = w.replace(K=k)
        rk = Run(wk, dev)
        el, ph = rk.measure(K, args.warmup)
        mk = workload_metrics(wk, rk.d, el, K, ph)
        k_curve[str(k)] = {"value": mk["value"], "ns_phase_us": mk.get("ns_phase_us")}
        del rk
        torch.cuda.empty_cache()

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
        "roofline": roofline,
        # the Newton-Schulz phase of the plain step's instrumented twin (the
        # chains run concurrently inside it): the pages' iteration's flops and
        # the MFMA flops the chosen form executes, over the phase time
        "ns_phase_us": main_metrics.get("ns_phase_us"),
        "ns_form": main_metrics.get("ns_form"),
        "ns_mfma_util_pct": main_metrics.get("ns_mfma_util_pct"),
        "ns_executed_tflops": main_metrics.get("ns_executed_tflops"),
        "ns_algorithmic_tflops": main_metrics.get("ns_algorithmic_tflops"),
        "ns_algorithmic_pct_of_peak": round(100 * main_metrics.get("ns_algorithmic_frac", 0), 2),
        "vote_gbps": main_metrics.get("vote_apply_gbps"),
        "vote_frac_hbm": main_metrics.get("vote_apply_frac_hbm"),
        "momentum_gbps": main_metrics.get("momentum_gbps"),
        "momentum_frac_hbm": main_metrics.get("momentum_frac_hbm"),
        "phases_us": {k: round(v, 2) for k, v in phase_us.items()},
        "instrumented_us_per_step": round(sum(phase_us.values()), 2),
        "all_workers": all_workers,
        "k_curve": k_curve,
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
