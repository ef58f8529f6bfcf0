"""Benchmark: CLiS attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload wan720p]

A step is one pass of the whole hot path on one batch of synthetic inputs
already resident in HBM: certification (Algorithm 1 of the CLiS pages) and
the routed attention forward, i.e. one clis_attn_fwd call in auto mode that
certifies internally.  The workload defaults to the Wan 2.2 720p x 81-frame
shape at one GPU's share of heads (B=1, H=20, N=75,600, d=128, bf16).

Printed: ONE JSON line with the step throughput (attention TFLOP/s), the
CLiS kernel alone, the online-softmax baseline and its lazy-rescale form
(FlashAttention-4's conditional rescaling), the speedups, the roofline
of the dominant kernel (the fixed-stabilizer attention kernel; per-launch
durations from HIP events on the stream the library launches on), the rates
of an MFMA-only probe on the same GPU (constant and random operands), the
fp64 CPU oracle timed on a
bounded sample of the same workload, and the step's output checked against
that oracle sample (and every head's certification flag against the
oracle's).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, published
METRIC = "attn fwd TFLOP/s & %MFMA peak, N=75600 H=20 d=128 bf16; CLiS vs online speedup"
CSRC = os.path.join(ROOT, "softmax_stabilization_video_amd", "csrc")


def dominant_kernel(w):
    """(name, source files) of the fixed-stabilizer kernel that runs this workload."""
    c = "true" if w.causal else "false"
    if w.dtype == "bf16":
        h = 2 if w.d == 128 else 1  # row halves per wave of the fixed kernel that returns O
        return (f"attn_fwd_bf16<{w.d}, true, {c}, 8, false, false, {h}>",
                (os.path.join(CSRC, "attn_bf16.hip"), os.path.join(CSRC, "tile_h2.inc")))
    # fp32: the kernel instance with every head on the fixed route (route 1)
    return f"attn_fwd_fp32<{w.d}, 1, {c}, false>", os.path.join(CSRC, "attn_fp32.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash(paths) -> str:
    """First 16 hex digits of the sha256 of the kernel's source files, in order."""
    h = hashlib.sha256()
    for path in ([paths] if isinstance(paths, str) else paths):
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def time_calls(fn, n: int, stream) -> list:
    """Per-call durations (ms) from HIP events recorded on `stream`."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def measured_traffic(kernel: str, source: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}/{workload}")
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_hash(source):
        return None
    return rec.get("bytes_per_launch")


def mfma_probe(device, random: bool, iters: int = 40000, blocks: int = 2048, reps: int = 5):
    """Rate (TFLOP/s) of an MFMA-only loop of the attention kernels' MFMA
    (libclis_probe.so), 18-25 ms per call.  With constant operands it runs at
    the chip's top clock, near the published peak; with random operands that
    differ from one MFMA to the next the power limit lowers the clock, and
    that rate is the ceiling a kernel whose operands keep changing can reach."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "softmax_stabilization_video_amd", "libclis_probe.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    L.clis_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.clis_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    L.clis_probe_mfma_flops.restype = ctypes.c_double
    out = torch.empty(blocks * 256, dtype=torch.float32, device=device)
    stream = torch.cuda.current_stream()

    def call():
        r = L.clis_probe_mfma(ctypes.c_void_p(out.data_ptr()), blocks, iters, int(random),
                              ctypes.c_void_p(stream.cuda_stream))
        if r != 0:
            raise RuntimeError(f"clis_probe_mfma failed: {r}")
    for _ in range(2):
        call()
    ms = statistics.median(time_calls(call, reps, stream))
    return L.clis_probe_mfma_flops(blocks, iters) / (ms * 1e-3) / 1e12


def cpu_baseline(w, Q, K, V, budget_s: float):
    """The fp64 oracle (as it stands) on a bounded sample of the workload:
    softmax attention for a seeded set of query rows of every head.  Returns
    the record and the sample ({(b, h): (rows, oracle rows)})."""
    import numpy as np
    import oracle
    threads = oracle.default_threads()
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def head_inputs(b, h):
        return tuple(oracle.decode(a[b, h], w.dtype) for a in (Q, K, V))

    rng = np.random.default_rng(12345)
    # calibrate on one batch of rows, then size the sample to the time budget
    q, k, v = head_inputs(*heads[0])
    rows = np.sort(rng.choice(w.Nq, size=min(w.Nq, 8 * threads), replace=False))
    oracle.attention_head(q, k, v, w.scale, w.causal, rows=rows[:threads], threads=threads)  # warm
    t0 = time.perf_counter()
    oracle.attention_head(q, k, v, w.scale, w.causal, rows=rows, threads=threads)
    dt = max(time.perf_counter() - t0, 1e-6)
    rate_rows = len(rows) / dt
    n_rows = int(max(len(heads), min(budget_s * rate_rows, w.B * w.H * w.Nq)))
    per_head = max(1, n_rows // len(heads))
    total_rows, flops, t_total = 0, 0.0, 0.0
    sample = {}
    for b, h in heads:
        q, k, v = head_inputs(b, h)
        rows = np.sort(rng.choice(w.Nq, size=min(w.Nq, per_head), replace=False))
        t0 = time.perf_counter()
        ref = oracle.attention_head(q, k, v, w.scale, w.causal, rows=rows, threads=threads)
        t_total += time.perf_counter() - t0
        sample[(b, h)] = (rows, ref)
        total_rows += len(rows)
        flops += float(np.sum([4.0 * w.d * ((r + 1) if w.causal else w.Nk) for r in rows]))
    # certification of every head (linear in N, so all of it fits the budget)
    t_cert = 0.0
    for b, h in heads:
        q, k, v = head_inputs(b, h)
        t0 = time.perf_counter()
        oracle.certify_head(q, k, v, w.scale, p_bf16=(w.dtype == "bf16"))
        t_cert += time.perf_counter() - t0
    full_s = t_total * (w.B * w.H * w.Nq) / total_rows + t_cert
    rec = {
        "value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"fp64 softmax attention of {total_rows} seeded query rows ({per_head} per head, all "
                  f"{len(heads)} heads) against all {w.Nk} keys; certification of all heads timed separately",
        "sample_seconds": round(t_total, 3), "certify_all_heads_s": round(t_cert, 3),
        "extrapolated_full_call_s": round(full_s, 1),
    }
    return rec, sample


def parity(w, Q, K, V, o_step, cert, sample):
    """The step's output on the oracle sample's rows against the oracle, and
    every head's certification flag against the oracle's (fp64 on both
    sides, so the flags must be identical)."""
    import numpy as np
    import torch
    import oracle
    err_max, err_sum, n, num, den = 0.0, 0.0, 0, 0.0, 0.0
    for (b, h), (rows, ref) in sample.items():
        idx = torch.as_tensor(rows, dtype=torch.long, device=o_step.device)
        got = o_step[b, h].index_select(0, idx).float().cpu().numpy().astype(np.float64)
        e = np.abs(got - ref)
        err_max = max(err_max, float(e.max()))
        err_sum += float(e.sum())
        n += e.size
        num += float(np.sum((got - ref) ** 2))
        den += float(np.sum(ref ** 2))
    cert_gpu = cert.cpu().numpy()
    agree = 0
    for b in range(w.B):
        for h in range(w.H):
            q, k, v = (oracle.decode(a[b, h], w.dtype) for a in (Q, K, V))
            c = oracle.certify_head(q, k, v, w.scale, p_bf16=(w.dtype == "bf16"))["cert"]
            agree += int(int(c) == int(cert_gpu[b, h]))
    return {"rows": sum(len(r) for r, _ in sample.values()), "max_abs": err_max, "mean_abs": err_sum / max(n, 1),
            "rel_l2": (num / den) ** 0.5 if den > 0 else 0.0,
            "flags_equal": f"{agree}/{w.B * w.H}", "vs": "fp64 oracle"}


# Fallback-rate and dispatch-cost sweep: synthetic inputs on the wan720p
# shape (B1 H20 d128) with one parameter varied at a time.  "heads" scaled by
# fail_qk_scale (and with outlier_frac of their key rows scaled by
# outlier_scale) are pushed toward or past the certificate's cap.
SWEEP = [
    ("failing_head_fraction", "fail_frac", (0.0, 0.1, 0.25, 0.5, 0.75, 1.0),
     dict(fail_qk_scale=40.0, outlier_frac=0.0, outlier_scale=1.0), 75600),
    ("qk_scale_all_heads", "fail_qk_scale", (1.0, 1.5, 1.9, 2.0, 2.02, 2.04, 2.1, 3.0),
     dict(fail_frac=1.0, outlier_frac=0.0, outlier_scale=1.0), 75600),
    ("outlier_key_scale_all_heads", "outlier_scale", (1.0, 2.0, 2.5, 2.8, 3.0, 3.5, 8.0),
     dict(fail_frac=1.0, fail_qk_scale=1.0, outlier_frac=0.001), 75600),
    ("tokens_at_qk_scale_2.04", "N", (17160, 32760, 65536, 75600),
     dict(fail_frac=1.0, fail_qk_scale=2.04, outlier_frac=0.0, outlier_scale=1.0), None),
]


def sweep(reps: int):
    """Certification rate and auto-mode throughput (certify inside) against
    the online kernel, for every point of SWEEP."""
    import torch
    import workloads
    import softmax_stabilization_video_amd as clis
    points = []
    for name, param, values, fixed, N in SWEEP:
        for val in values:
            kw = dict(fixed)
            n = int(val) if param == "N" else N
            if param != "N":
                kw[param] = val
            w = workloads.custom(f"sweep_{name}", 1, 20, n, 128, "bf16", False, key_bias_std=2.0, **kw)
            Q, K, V = workloads.make_inputs(w, 0)
            q, k, v = (workloads.to_torch(a, w.dtype) for a in (Q, K, V))
            o = torch.empty_like(q)
            ws = clis.new_workspace(w.B, w.H, w.Nq, w.Nk, w.d)
            stream = torch.cuda.current_stream()
            auto = lambda: clis.clis_attn_fwd(q, k, v, w.scale, mode="auto", out=o, workspace=ws)
            onl = lambda: clis.online_attn_fwd(q, k, v, w.scale, out=o, workspace=ws)
            for f in (auto, onl):
                f()
            _, cert = clis.clis_certify(q, k, v, w.scale, workspace=ws)
            t_auto = statistics.median(time_calls(auto, reps, stream))
            t_onl = statistics.median(time_calls(onl, reps, stream))
            n_cert = int(cert.sum().item())
            fl = w.flops()
            points.append({"sweep": name, param: val, "N": n, "certified": n_cert, "heads": w.B * w.H,
                           "auto_ms": round(t_auto, 3), "online_ms": round(t_onl, 3),
                           "auto_tflops": round(fl / t_auto / 1e9, 1), "online_tflops": round(fl / t_onl / 1e9, 1),
                           "speedup_vs_online": round(t_onl / t_auto, 4)})
            log(json.dumps(points[-1]))
            del q, k, v, o, ws, Q, K, V
            torch.cuda.empty_cache()
    return points


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="wan720p")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", choices=["all", "clis", "online", "certify"], default="all",
                   help="restrict the extra timings (for profiler runs)")
    p.add_argument("--reps", type=int, default=20, help="calls per extra timing")
    p.add_argument("--calibrate-copy-mb", type=float, default=0.0,
                   help="also run one plain device copy of this many MiB (scales HBM counters)")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the step benchmark: certification rate and auto-mode throughput vs input "
                        "scale, outlier keys, failing-head fraction and tokens (one JSON line)")
    args = p.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the CLiS path here is "
                                   "single-GPU (heads shard across GPUs with no communication)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import softmax_stabilization_video_amd as clis

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    if args.sweep:
        print(json.dumps({"sweep": sweep(max(3, min(args.reps, 7))), "unit": "ms / TFLOP/s",
                          "data": "synthetic (seeded Gaussians, wan720p shape B1 H20 d128 bf16)"}), flush=True)
        return
    w = workloads.WORKLOADS[args.workload]
    log(f"workload {w.name}: B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} d={w.d} {w.dtype} causal={w.causal}")
    t0 = time.perf_counter()
    Q, K, V = workloads.make_inputs(w, args.seed)
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")
    q, k, v = (workloads.to_torch(a, w.dtype) for a in (Q, K, V))
    o = torch.empty_like(q)
    ws = clis.new_workspace(w.B, w.H, w.Nq, w.Nk, w.d)
    stream = torch.cuda.current_stream()
    flops = w.flops()

    def step():
        clis.clis_attn_fwd(q, k, v, w.scale, w.causal, mode="auto", out=o, workspace=ws)

    # ---- whole-path steps: warmup, then exactly K timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3
    log(f"step (certify + attention): {ms_step:.3f} ms")
    step_events = time_calls(step, max(1, min(args.steps, args.reps)), stream)
    o_step = o.clone()  # the step's output, checked against the oracle below

    mu, cert = clis.clis_certify(q, k, v, w.scale, workspace=ws)
    torch.cuda.synchronize()
    n_cert = int(cert.sum().item())
    res = {}
    if args.only in ("all", "clis"):
        kern = time_calls(lambda: clis.clis_attn_fwd(q, k, v, w.scale, w.causal, mode="auto", mu=mu,
                                                     cert=cert, out=o, workspace=ws), args.reps, stream)
        res["clis_kernel_ms"] = statistics.median(kern)
        # the dominant kernel on its own: every head on the fixed-stabilizer kernel
        fixed = time_calls(lambda: clis.clis_attn_fwd(q, k, v, w.scale, w.causal, mode="fixed", mu=mu,
                                                      out=o, workspace=ws), args.reps, stream)
        res["fixed_kernel_ms_mean"] = statistics.mean(fixed)
        res["fixed_kernel_ms_median"] = statistics.median(fixed)
    if args.only in ("all", "online"):
        onl = time_calls(lambda: clis.online_attn_fwd(q, k, v, w.scale, w.causal, out=o, workspace=ws),
                         args.reps, stream)
        res["online_ms"] = statistics.median(onl)
        lazy = time_calls(lambda: clis.clis_attn_fwd(q, k, v, w.scale, w.causal, mode="online_lazy", out=o,
                                                     workspace=ws), args.reps, stream)
        res["online_lazy_ms"] = statistics.median(lazy)
    if args.only in ("all", "certify"):
        cer = time_calls(lambda: clis.clis_certify(q, k, v, w.scale, workspace=ws), args.reps, stream)
        res["certify_ms"] = statistics.median(cer)

    if args.calibrate_copy_mb > 0:
        nbytes = int(args.calibrate_copy_mb * 2 ** 20)
        src = torch.ones(nbytes, dtype=torch.uint8, device=q.device)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # one plain copy kernel: reads and writes nbytes
        torch.cuda.synchronize()
        log(f"calibration copy of {nbytes} bytes done")
        del src, dst

    value = flops / (ms_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussians shaped like the workload; no model weights)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                   "causal": w.causal, "seed": args.seed, "step": "clis_attn_fwd auto mode, certify inside",
                   "heads_certified": n_cert, "heads": w.B * w.H},
        "pct_mfma_peak": round(100 * value / MFMA_BF16_PEAK_TFLOPS, 2),
        "step_ms_median_events": round(statistics.median(step_events), 4),
        "step_ms_min_events": round(min(step_events), 4),
        "step_ms_mean_events": round(statistics.mean(step_events), 4),
    }
    props = torch.cuda.get_device_properties(q.device)
    out["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                     "compute_units": props.multi_processor_count,
                     "memory_gib": round(props.total_memory / 2 ** 30, 1)}
    if "clis_kernel_ms" in res:
        out["clis_kernel_tflops"] = round(flops / res["clis_kernel_ms"] / 1e9, 2)
        out["clis_kernel_ms"] = round(res["clis_kernel_ms"], 4)
    if "online_ms" in res:
        out["online_tflops"] = round(flops / res["online_ms"] / 1e9, 2)
        out["online_ms"] = round(res["online_ms"], 4)
        out["speedup_vs_online"] = round(res["online_ms"] / ms_step, 4)
        if "clis_kernel_ms" in res:
            out["kernel_speedup_vs_online"] = round(res["online_ms"] / res["clis_kernel_ms"], 4)
    if "online_lazy_ms" in res:
        out["online_lazy_tflops"] = round(flops / res["online_lazy_ms"] / 1e9, 2)
        out["online_lazy_ms"] = round(res["online_lazy_ms"], 4)
        if "clis_kernel_ms" in res:
            out["kernel_speedup_vs_online_lazy"] = round(res["online_lazy_ms"] / res["clis_kernel_ms"], 4)
    if "certify_ms" in res:
        out["certify_ms"] = round(res["certify_ms"], 4)
    if "fixed_kernel_ms_mean" in res:
        ms = res["fixed_kernel_ms_mean"]
        achieved = flops / (ms * 1e-3) / 1e12
        name, src = dominant_kernel(w)
        bf16 = w.dtype == "bf16"
        peak = MFMA_BF16_PEAK_TFLOPS if bf16 else FP32_MFMA_PEAK_TFLOPS
        out["roofline"] = {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
            "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
            "traffic": measured_traffic(name, src, w.name),
            "kernel": name + (" (fixed stabilizer; the timed call also runs the V transpose pre-pass and "
                              "the route kernel)" if bf16 else " (fixed stabilizer; the fp32 kernel takes each "
                              "head's route itself, so the timed call is this one launch)"),
            "algorithmic_flops_per_launch": flops, "launch_ms_mean": round(ms, 4),
        }
    if w.dtype == "bf16" and args.only == "all":
        probe = mfma_probe(q.device, random=False)
        if probe:
            out["mfma_probe_tflops"] = round(probe, 1)
            out["pct_measured_mfma_peak"] = round(100 * value / probe, 2)
            probe_rnd = mfma_probe(q.device, random=True)
            out["mfma_probe_random_tflops"] = round(probe_rnd, 1)
            out["pct_random_operand_mfma_ceiling"] = round(100 * value / probe_rnd, 2)
    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on a bounded sample")
        out["cpu_baseline"], sample = cpu_baseline(w, Q, K, V, args.cpu_budget)
        log("checking the step's output and flags against the oracle")
        out["parity"] = parity(w, Q, K, V, o_step, cert, sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
