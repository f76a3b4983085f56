"""Seeded random sweeps against the oracle: forward + VJP, batched rows, and
the order statistics with hard top-k and DFTopK.

Each case draws, from its own seed: n log-uniform in [1, 3 * 10^6], a score
distribution (normal, Student-t(3), the C4 mixture, uniform, the C5 tie
cluster, integers with many ties, or scores offset by 10^4), the budget k
uniform in (0, n), the temperature t log-uniform in [1e-4, 10] (the range
the gist.science summary's experiments span) and the path (auto, full sort,
bracketing, or bracketing forced onto the full-sort fallback).  Every output
element is compared with the oracle, with the same tolerances as the other
parity tests; the point is breadth: shapes and combinations the targeted
tests do not name.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import P_TOL, SUM_TOL, check_forward, check_vjp, t32, to_dev

pytestmark = pytest.mark.gpu

L = pytest.importorskip("differentiable_exact_budget_amd")

DISTS = ["normal", "student_t3", "mixture", "uniform", "adversarial", "integers", "offset"]
PATHS = [L.PATH_AUTO, L.PATH_FULL, L.PATH_BRACKET, L.PATH_FORCE_FALLBACK]
CASES = list(range(160))


def draw(case):
    rng = np.random.default_rng(90_000 + case)
    n = int(np.exp(rng.uniform(0.0, np.log(3e6))))
    n = max(n, 1)
    dist = DISTS[case % len(DISTS)]
    path = PATHS[(case // len(DISTS)) % len(PATHS)]
    k = float(rng.uniform(0.0, n))
    k = min(max(k, 1e-3), n - 1e-3) if n > 1 else 0.5
    t = float(np.exp(rng.uniform(np.log(1e-4), np.log(10.0))))
    seed = 5000 + case
    if dist == "integers":
        r = np.random.default_rng(seed).integers(-50, 50, n).astype(np.float32)
    elif dist == "offset":
        r = (1e4 + np.random.default_rng(seed).standard_normal(n)).astype(np.float32)
    elif dist == "adversarial":
        r = workloads.scores("adversarial", n, seed, k=max(1.0, min(k, n - 1.0)))
    else:
        r = workloads.scores(dist, n, seed)
    g = workloads.upstream(n, seed + 1)
    return n, dist, path, k, t, r, g


@pytest.mark.parametrize("case", CASES)
def test_random_case(oracle_mod, case):
    n, dist, path, k, t, r, g = draw(case)
    label = f"case {case}: n={n} {dist} path={path} k={k:.6g} t={t:.3g}"
    print("\n" + label, flush=True)
    rd, gd = to_dev(r), to_dev(g)
    opts = L.default_options(path=path)
    p, b, st = L.forward(rd, k, t, options=opts, stats=True)
    grad = L.vjp(rd, gd, t, b)
    assert st["status"] == 0, label
    if path == L.PATH_FORCE_FALLBACK:
        assert st["path_taken"] == 3, label
    b_ref = check_forward(oracle_mod, r, k, t, p.cpu().numpy(), float(b.item()), label=label)
    check_vjp(oracle_mod, r, g, t, b_ref, grad.cpu().numpy(), label=label)


# ---------------------------------------------------------------------------
# batched rows: rows x n with n log-uniform in [1, 65536] (one workgroup per
# row up to 16384 scores, staging through HBM above), a budget per row or
# one for all
# ---------------------------------------------------------------------------
ROW_CASES = list(range(32))


@pytest.mark.parametrize("case", ROW_CASES)
def test_random_rows(oracle_mod, case):
    rng = np.random.default_rng(70_000 + case)
    n = max(1, int(np.exp(rng.uniform(0.0, np.log(65536.0)))))
    rows = int(rng.integers(1, max(2, min(64, 4_000_000 // n)) + 1))
    t = float(np.exp(rng.uniform(np.log(1e-4), np.log(10.0))))
    dist = DISTS[case % len(DISTS)]
    if dist in ("adversarial", "integers"):
        r = np.random.default_rng(case).integers(-20, 20, (rows, n)).astype(np.float32)
    elif dist == "offset":
        r = (1e4 + np.random.default_rng(case).standard_normal((rows, n))).astype(np.float32)
    else:
        r = workloads.scores(dist, rows * n, 7000 + case).reshape(rows, n)
    g = workloads.upstream(rows * n, 8000 + case).reshape(rows, n)
    if n == 1:
        ks = np.full(rows, 0.5)
    else:
        ks = np.clip(rng.uniform(0.0, n, rows), 1e-3, n - 1e-3)
    per_row = bool(case % 2)
    label = f"rows case {case}: {rows} x {n} {dist} t={t:.3g} per_row={per_row}"
    print("\n" + label, flush=True)
    rd, gd = to_dev(r), to_dev(g)
    k_arg = to_dev(ks.astype(np.float64)) if per_row else float(ks[0])
    p, b = L.forward_rows(rd, k_arg, t)
    grad = L.vjp_rows(rd, gd, t, b).cpu().numpy()
    ph, bh = p.cpu().numpy(), b.cpu().numpy()
    for i in range(rows):
        k = float(ks[i]) if per_row else float(ks[0])
        b_ref = check_forward(oracle_mod, r[i], k, t, ph[i], float(bh[i]), label=f"{label} row {i}")
        check_vjp(oracle_mod, r[i], g[i], t, b_ref, grad[i], label=f"{label} row {i}")


# ---------------------------------------------------------------------------
# order statistics, hard top-k and DFTopK on both paths
# ---------------------------------------------------------------------------
TOPK_CASES = list(range(32))


@pytest.mark.parametrize("case", TOPK_CASES)
def test_random_order_statistics(oracle_mod, case):
    rng = np.random.default_rng(60_000 + case)
    n = max(2, int(np.exp(rng.uniform(np.log(2.0), np.log(3e6)))))
    k = int(rng.integers(1, n))  # 1 <= k < n
    t = float(np.exp(rng.uniform(np.log(1e-4), np.log(10.0))))
    dist = DISTS[case % len(DISTS)]
    if dist in ("adversarial", "integers"):
        r = np.random.default_rng(case).integers(-100, 100, n).astype(np.float32)
    elif dist == "offset":
        r = (1e4 + np.random.default_rng(case).standard_normal(n)).astype(np.float32)
    else:
        r = workloads.scores(dist, n, 6000 + case)
    path = [L.PATH_AUTO, L.PATH_FULL, L.PATH_BRACKET][case % 3]
    label = f"top-k case {case}: n={n} {dist} k={k} t={t:.3g} path={path}"
    print("\n" + label, flush=True)
    rd = to_dev(r)
    o = L.default_options(path=path)
    tau, st = L.topk_threshold(rd, k, options=o, stats=True)
    assert st["status"] == 0, label
    r64 = r.astype(np.float64)
    tk, tk1 = oracle_mod.order_stats(r64, k)
    got = tau.cpu().numpy()
    assert got[0] == tk and got[1] == tk1, (label, got, tk, tk1)
    mask, _ = L.hard_topk(rd, k, options=o)
    mask_ref, _, _ = oracle_mod.hard_topk(r64, k)
    assert np.array_equal(mask.cpu().numpy().astype(np.float64), mask_ref), label
    p, b = L.dftopk(rd, k, t, options=o)
    p_ref, b_ref, s_ref = oracle_mod.dftopk(r64, k, t32(t))
    assert float(b.item()) == b_ref, label
    ph = p.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(ph - p_ref)) <= P_TOL, label
    assert abs(ph.sum() - s_ref) <= SUM_TOL * k, label
