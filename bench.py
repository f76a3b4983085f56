"""Benchmark of the Fast LapSum solver on one MI355X.

A step is one forward solve (threshold b and p) plus one VJP over one batch
of resident synthetic scores.  Default workload: n = 10^8 fp32 scores drawn
per element from U(0,1) w.p. 0.9 else N(2, sd 0.5), k = 10^5, t = 0.01, on
the bracketing path with certification (the largest configuration, 400 MB).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C4]

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded on
the library's stream in a second timed loop (options.profile); the roofline
entry uses the dominant kernel's algorithmic bytes per launch.  The smaller
workloads are timed warm (inputs left in the caches across steps) and cold
(1 GiB written before each step).  The CPU baseline times the fp64 oracle on
the same workload with all threads, and on one thread over a prefix.

The roofline's `traffic` is the dominant kernel's HBM bytes per launch from
hardware counters (FETCH_SIZE and WRITE_SIZE, calibrated against a plain
copy of known size), read from the summary committed under profiles/; it is
reported only while the sources it was measured on are unchanged (their
SHA-256 is recorded next to the figure), else null.
"""
import argparse
import hashlib
import json
import re
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "median ms and scores/s per forward+VJP solve at n=1e6/1e7/1e8; % peak HBM GB/s"
PEAK_HBM_GBPS = 8000.0

# algorithmic bytes per score moved by each kernel (reads + writes of n-sized arrays)
ALG_BYTES = {
    "filter": 4,        # read r
    "probs": 8,         # read r, write p
    "vjp_reduce": 8,    # read r, g
    "vjp_apply": 12,    # read r, g, write grad
    "radix_sort": 36,   # histogram read 4 + four digit passes (read 4 + write 4)
    "curve_solve": 4,   # read the sorted keys
    "cert": 4,          # read r (the certification as a pass of its own)
    "heavy_collect": 4,  # read r again (scores of overflowed buckets)
    "small_solve": 4,   # read r (one-workgroup sort and solve)
}


# sources whose kernels the counter-based traffic figure was taken on
TRAFFIC_SOURCES = ("differentiable_exact_budget_amd/csrc/lapsum_stream.hip",
                   "differentiable_exact_budget_amd/csrc/lapsum_streamio.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_C4.md")


def sources_sha256():
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary, or None."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"sources_sha256:\s*([0-9a-f]{64})", text)
    if not m or m.group(1) != sources_sha256():
        return None
    for line in text.splitlines():
        q = re.match(r"\|\s*" + re.escape(kernel) + r"\s*\|(.*)\|\s*$", line)
        if q:
            cells = [c.strip() for c in q.group(1).split("|")]
            try:
                return float(cells[-1])
            except ValueError:
                return None
    return None


def measure_ceilings(torch, L, dev, n=100_000_000, reps=10):
    """Achievable HBM rates of the library's plain streaming kernels on the
    same device: a copy (read + write n fp32) and a read of n fp32, launched
    like the solver's streaming passes."""
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    sink = torch.zeros(256, dtype=torch.float32, device=dev)
    lib = L.lib()
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for name, fn, nbytes in (("copy", lambda: lib.lapsum_test_copy(a.data_ptr(), b.data_ptr(), n, stream), 8 * n),
                             ("read", lambda: lib.lapsum_test_read(a.data_ptr(), n, sink.data_ptr(), stream), 4 * n)):
        assert fn() == 0
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for s0, s1 in ev:
            s0.record()
            fn()
            s1.record()
        torch.cuda.synchronize()
        ms = statistics.median(s0.elapsed_time(s1) for s0, s1 in ev)
        res[name + "_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del a, b, sink
    res["note"] = "k_copy and k_read over 10^8 fp32 (400 MB), median of 10"
    return res


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="C4")
    ap.add_argument("--force-fallback", action="store_true",
                    help="bracketing pass, then the full-sort fallback regardless (path 3)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=0,
                    help="oracle prefix size for the CPU baseline (0: the whole workload)")
    return ap.parse_args()


def describe(cfg):
    dist = {"normal": "N(0,1)", "student_t3": "Student-t(3)",
            "mixture": "0.9*U(0,1)+0.1*N(2,0.5)", "adversarial": "N(0,1) + 1% tied at the (1-k/n) quantile"}[cfg.dist]
    path = {"full": "full sort", "bracket": "bracketing+certification", "fallback": "forced full-sort fallback"}
    return f"{cfg.name}: n={cfg.n} fp32 {dist}, k={cfg.k:g}, t={cfg.t:g}, {path[cfg.path]}, forward+VJP"


def time_steps(L, torch, rd, gd, k, t, steps, warmup, options=None):
    """Time `steps` forward+VJP steps; returns (total_s, per-step ms list)."""
    p = torch.empty_like(rd)
    b = torch.empty(1, dtype=torch.float64, device=rd.device)
    grad = torch.empty_like(rd)
    for _ in range(warmup):
        L.forward(rd, k, t, options=options, p_out=p, b_out=b)
        L.vjp(rd, gd, t, b, grad_out=grad)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record()
        L.forward(rd, k, t, options=options, p_out=p, b_out=b)
        L.vjp(rd, gd, t, b, grad_out=grad)
        ends[i].record()
    torch.cuda.synchronize()
    total = time.perf_counter() - t0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return total, per


def time_steps_cold(L, torch, rd, gd, k, t, steps, options=None, flush_bytes=1 << 30):
    """Per-step ms with the caches cold: before each step (outside its events)
    a scratch buffer of `flush_bytes` is written, which evicts the inputs from
    the 256 MB memory-side cache and the L2s."""
    p = torch.empty_like(rd)
    b = torch.empty(1, dtype=torch.float64, device=rd.device)
    grad = torch.empty_like(rd)
    flush = torch.empty(flush_bytes // 4, dtype=torch.float32, device=rd.device)
    L.forward(rd, k, t, options=options, p_out=p, b_out=b)
    L.vjp(rd, gd, t, b, grad_out=grad)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        flush.fill_(float(i))
        starts[i].record()
        L.forward(rd, k, t, options=options, p_out=p, b_out=b)
        L.vjp(rd, gd, t, b, grad_out=grad)
        ends[i].record()
    torch.cuda.synchronize()
    del flush
    return [s.elapsed_time(e) for s, e in zip(starts, ends)]


def kernel_profile(L, torch, rd, gd, k, t, steps, path=0, cert_mode=0):
    """Per-kernel durations (ms) from HIP events recorded by the library."""
    opt = L.default_options(profile=1, path=path, cert_mode=cert_mode)
    acc = {}
    info = None
    p = torch.empty_like(rd)
    b = torch.empty(1, dtype=torch.float64, device=rd.device)
    grad = torch.empty_like(rd)
    for _ in range(steps):
        _, _, st = L.forward(rd, k, t, options=opt, stats=True, p_out=p, b_out=b)
        _, sv = L.vjp(rd, gd, t, b, grad_out=grad, options=opt, stats=True)
        info = st
        for name, ms in st["kernels"] + sv["kernels"]:
            acc.setdefault(name, []).append(ms)
    return {n: statistics.mean(v) for n, v in acc.items()}, info


def timed(torch, fn, reps=10, warm=2):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for s0, s1 in ev:
        s0.record()
        fn()
        s1.record()
    torch.cuda.synchronize()
    return statistics.median(s0.elapsed_time(s1) for s0, s1 in ev)


def extras(L, torch, rd, gd, cfg):
    """The operator's other entry points on the same resident input:
    the VJP with budget and temperature gradients, hard top-k (threshold and
    mask) and DFTopK (threshold and p).  Median ms over 10 calls; bytes are
    the n-sized arrays each call must move."""
    n, k, t = cfg.n, int(cfg.k), cfg.t
    _, b = L.forward(rd, cfg.k, t)
    grad = torch.empty_like(rd)
    res = {}
    for name, fn, bpe in (
            ("vjp", lambda: L.vjp(rd, gd, t, b, grad_out=grad), 20),
            ("vjp_kt", lambda: L.vjp_kt(rd, gd, t, b, grad_out=grad), 20),
            ("vjp_kt_scalars_only", lambda: L.vjp_kt(rd, gd, t, b, want_grad=False), 8),
            ("hard_topk", lambda: L.hard_topk(rd, k), 12),
            ("dftopk", lambda: L.dftopk(rd, k, t), 12)):
        ms = timed(torch, fn)
        res[name] = {"median_ms": round(ms, 5), "scores_per_s": n / (ms * 1e-3),
                     "alg_GBps": round(bpe * n / (ms * 1e-3) / 1e9, 1)}
    # DFTopK's mass at finite t (its threshold is the midpoint of the k-th and
    # (k+1)-th largest scores, so sum p is not held at k)
    _, _, sd = L.dftopk(rd, k, t, stats=True)
    res["dftopk"]["sum_p_over_k"] = sd["sum_p"] / k
    _, _, sl = L.forward(rd, cfg.k, t, stats=True)
    res["dftopk"]["lapsum_sum_p_over_k"] = sl["sum_p"] / cfg.k
    # many independent rows (seeded N(0,1) rows, k = n/32 per row, t = 0.05);
    # algorithmic bytes: forward reads r and writes p (8), VJP 12
    import numpy as np
    for rows, m in ((4096, 4096), (65536, 256), (1000, 65536)):
        rng = np.random.default_rng(rows + m)
        rr = torch.from_numpy(rng.standard_normal((rows, m)).astype(np.float32)).to(rd.device)
        gg = torch.from_numpy(rng.standard_normal((rows, m)).astype(np.float32)).to(rd.device)
        kk = m / 32.0
        _, bb = L.forward_rows(rr, kk, 0.05)
        fwd = timed(torch, lambda: L.forward_rows(rr, kk, 0.05))
        bwd = timed(torch, lambda: L.vjp_rows(rr, gg, 0.05, bb))
        gbps = 20 * rows * m / ((fwd + bwd) * 1e-3) / 1e9
        res[f"rows_{rows}x{m}"] = {"forward_ms": round(fwd, 5), "vjp_ms": round(bwd, 5),
                                   "scores_per_s": rows * m / ((fwd + bwd) * 1e-3),
                                   "alg_GBps": round(gbps, 1), "frac_peak": round(gbps / PEAK_HBM_GBPS, 4)}
        del rr, gg
    return res


def step_bytes_per_score(n, path_taken, cert_mode=0):
    """Algorithmic bytes per score of one forward + VJP step on the path it
    took: the n-sized arrays the method itself must read or write (O(s + m)
    terms left out).  VJP: reduce reads r, g (8); apply reads r, g, writes
    grad (12)."""
    vjp = 20
    if path_taken == 1:
        if n <= 16384:
            return 4 + 8 + vjp  # one workgroup reads r; p pass reads r, writes p
        return 4 + 4 * 8 + 4 + 8 + vjp  # histogram, four digit passes, curve, p
    if path_taken == 2:
        return 4 + 8 + vjp + (4 if cert_mode else 0)  # filter, [certification pass,] p
    return 4 + (4 + 4 * 8 + 4) + 8 + vjp  # filter, then the full sort and curve, p


def budget_error(L, torch, rd, k, t, options=None):
    """|sum p - k| / k of one forward (sum p: fp64 on the device over the
    written fp32 p) and the path it took."""
    _, _, st = L.forward(rd, k, t, options=options, stats=True)
    return abs(st["sum_p"] - k) / k, st


def config_entry(L, torch, a, b2, c2, options=None, cert_mode=0, steps=20, warmup=3, cold=10):
    """Warm and cold step medians of one workload, with its algorithmic
    bytes, rate and fraction of peak, and the budget error."""
    _, per = time_steps(L, torch, a, b2, c2.k, c2.t, steps, warmup, options)
    med = statistics.median(per)
    e = {"median_ms": round(med, 5), "scores_per_s": c2.n / (med * 1e-3)}
    if cold:
        e["cold_median_ms"] = round(statistics.median(time_steps_cold(L, torch, a, b2, c2.k, c2.t, cold, options)), 5)
    err, st = budget_error(L, torch, a, c2.k, c2.t, options)
    bps = step_bytes_per_score(c2.n, st["path_taken"], cert_mode)
    gbps = bps * c2.n / (med * 1e-3) / 1e9
    e.update({"path_taken": st["path_taken"], "alg_bytes_per_score": bps, "alg_GBps": round(gbps, 1),
              "frac_peak": round(gbps / PEAK_HBM_GBPS, 4), "budget_rel_err": err})
    return e


def cpu_baseline(cfg, r, g, n_sample):
    import numpy as np
    import oracle
    ns = min(n_sample, r.size) if n_sample > 0 else r.size
    rs = np.ascontiguousarray(r[:ns]).astype(np.float64)
    gs = np.ascontiguousarray(g[:ns]).astype(np.float64)
    ks = max(cfg.k * ns / r.size, 1.0)
    t = float(np.float32(cfg.t))
    oracle._load()

    def run(m):
        km = max(cfg.k * m / r.size, 1.0)
        t0 = time.perf_counter()
        b, _ = oracle.solve(rs[:m], km, t)
        oracle.probs(rs[:m], t, b)
        oracle.vjp(rs[:m], gs[:m], t, b)
        return time.perf_counter() - t0

    dt = run(ns)
    out = {"value": ns / dt, "unit": "scores/s", "cores": oracle.get_threads(), "kind": "oracle",
           "sample": (f"first {ns} scores of the {cfg.name} input (k scaled to {ks:g})" if ns < r.size else
                      f"the whole {cfg.name} input ({ns} scores, k={ks:g})") +
                     f": fp64 bisection solve + p + VJP, {dt:.2f} s wall"}
    # the same oracle on one thread, over a prefix sized to about 10 s
    threads = oracle.get_threads()
    n1 = int(min(ns, max(1 << 16, 10.0 * ns / dt / max(threads, 1))))
    oracle.set_threads(1)
    try:
        d1 = run(n1)
    finally:
        oracle.set_threads(threads)
    out["one_thread"] = {"value": n1 / d1, "unit": "scores/s", "cores": 1,
                         "sample": f"first {n1} scores (k scaled to {max(cfg.k * n1 / r.size, 1.0):g}), {d1:.2f} s wall"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import differentiable_exact_budget_amd as L
    import workloads

    cfg = workloads.CONFIGS[args.config]
    r, g, _ = workloads.config_inputs(cfg.name)
    dev = torch.device("cuda:0")
    rd = torch.from_numpy(r).to(dev)
    gd = torch.from_numpy(g).to(dev)
    forced = args.force_fallback or cfg.path == "fallback"
    opts = L.default_options(path=L.PATH_FORCE_FALLBACK) if forced else None

    total, per = time_steps(L, torch, rd, gd, cfg.k, cfg.t, args.steps, args.warmup, opts)
    ms_per_step = total * 1000.0 / args.steps
    med = statistics.median(per)
    kern, info = kernel_profile(L, torch, rd, gd, cfg.k, cfg.t, max(5, min(args.steps, 20)),
                                L.PATH_FORCE_FALLBACK if forced else 0)

    # roofline of the dominant kernel (largest average duration)
    dom = max(kern, key=kern.get)
    alg = ALG_BYTES.get(dom, 0) * cfg.n
    achieved = alg / (kern[dom] * 1e-3) / 1e9 if kern[dom] > 0 else 0.0
    roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": counter_traffic(dom) if cfg.name == "C4" else None,
            "alg_bytes_per_launch": alg, "avg_ms": round(kern[dom], 5)}
    ceil = measure_ceilings(torch, L, dev)
    roof["frac_of_copy_ceiling"] = round(achieved / ceil["copy_GBps"], 4)
    kernels = {}
    for name, ms in sorted(kern.items(), key=lambda kv: -kv[1]):
        e = {"avg_ms": round(ms, 5)}
        if name in ALG_BYTES and ms > 0:
            gbps = ALG_BYTES[name] * cfg.n / (ms * 1e-3) / 1e9
            e["alg_GBps"] = round(gbps, 1)
            e["frac_peak"] = round(gbps / PEAK_HBM_GBPS, 4)
        kernels[name] = e
    # whole-step byte roofline (bracketing path: 32 B per score)
    step_bytes = 32 * cfg.n if cfg.path == "bracket" and not forced else None

    out = {
        "metric": METRIC,
        "value": cfg.n * args.steps / total,
        "unit": "scores/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "median_ms": med,
        "p10_ms": float(np.percentile(per, 10)),
        "p90_ms": float(np.percentile(per, 90)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic (seeded numpy PCG64)",
        "config": {"workload": describe(cfg) + (" (forced full-sort fallback)" if forced and cfg.path != "fallback"
                                                else ""),
                   "n": cfg.n, "k": cfg.k, "t": cfg.t, "parallelism": "single GPU"},
        "roofline": roof,
        "ceilings": ceil,
        "kernels": kernels,
        "path": {"path_taken": info["path_taken"], "certified": info["certified"], "widenings": info["widenings"],
                 "band_size": info["band_size"], "buckets": info["buckets"], "sample_size": info["sample_size"]},
    }
    if step_bytes:
        out["step_roofline"] = {"alg_bytes": step_bytes, "ideal_ms_at_peak": step_bytes / PEAK_HBM_GBPS / 1e6,
                                "frac_of_median": round(step_bytes / PEAK_HBM_GBPS / 1e6 / med, 4)}

    err, _ = budget_error(L, torch, rd, cfg.k, cfg.t, opts)
    out["budget_rel_err"] = err
    out["alg_bytes_per_score"] = step_bytes_per_score(cfg.n, info["path_taken"])
    if not args.no_other_configs:
        others = {}
        for name in ("C1", "C2", "C3", "C5"):
            c2 = workloads.CONFIGS[name]
            r2, g2, _ = workloads.config_inputs(name)
            a = torch.from_numpy(r2).to(dev)
            b2 = torch.from_numpy(g2).to(dev)
            others[name] = config_entry(L, torch, a, b2, c2)
            if name == "C5":
                o5 = L.default_options(path=L.PATH_FORCE_FALLBACK)
                others["C5_forced_fallback"] = config_entry(L, torch, a, b2, c2, o5, steps=10, warmup=2)
            del a, b2
        if cfg.name == "C4" and not forced:
            # the same workload forced onto the full-sort fallback, and with the
            # certification as its own pass (cert_mode 1)
            o4 = L.default_options(path=L.PATH_FORCE_FALLBACK)
            e4 = config_entry(L, torch, rd, gd, cfg, o4, steps=5, warmup=2, cold=0)
            e4["forced_over_auto"] = round(e4["median_ms"] / med, 3)
            others["C4_forced_fallback"] = e4
            oc = L.default_options(cert_mode=1)
            ec = config_entry(L, torch, rd, gd, cfg, oc, cert_mode=1, steps=args.steps, warmup=3, cold=0)
            kc, _ = kernel_profile(L, torch, rd, gd, cfg.k, cfg.t, 5, 0, cert_mode=1)
            ec["cert_pass_ms"] = round(kc.get("cert", 0.0), 5)
            ec["cert_pass_GBps"] = round(4 * cfg.n / (kc["cert"] * 1e-3) / 1e9, 1) if kc.get("cert") else None
            ec["over_default"] = round(ec["median_ms"] / med, 4)
            others["C4_cert_pass"] = ec
        others["note"] = ("median_ms: inputs warm in the caches across steps; cold_median_ms: 1 GiB written "
                          "before each step, outside its timed events; alg_GBps: algorithmic bytes of the path "
                          "taken / warm median; budget_rel_err: |sum p - k| / k of one forward")
        out["other_configs"] = others

    if not args.no_other_configs and cfg.name == "C4":
        out["extras"] = extras(L, torch, rd, gd, cfg)

    out["pages_context_ms"] = {"forward_only_1e8": 5.23, "certified_median_1e8": 7.24,
                               "note": "the pages' forward solve times on unnamed hardware; not this metric"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, r, g, args.cpu_sample)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
