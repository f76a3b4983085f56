"""A seeded random sweep of forward + VJP parity against the oracle.

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
from gpu_helpers import check_forward, check_vjp, to_dev

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
