"""GPU parity of the order-statistic entry points (hard top-k threshold and
mask, DFTopK) against the oracle, on every path: the one-workgroup sort, the
radix sort, the bracketing path and its forced fallback.  Order statistics
and masks are bit-exact; DFTopK's p is within the p gate and its mass (which
drifts from k by design) matches the oracle's."""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import P_TOL, SUM_TOL, t32, to_dev

pytestmark = pytest.mark.gpu

L = pytest.importorskip("differentiable_exact_budget_amd")


def inputs(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties":
        return rng.integers(-50, 50, size=n).astype(np.float32)
    if kind == "mixture":
        return workloads.scores("mixture", n, seed)
    if kind == "student":
        return workloads.scores("student_t3", n, seed)
    raise ValueError(kind)


CASES = [
    # (kind, n, ks, options, expected path)
    ("normal", 1, (1,), {}, 1),
    ("normal", 17, (1, 5, 16, 17), {}, 1),
    ("ties", 4096, (1, 64, 4000), {}, 1),
    ("normal", 16384, (1, 100, 16383), {}, 1),
    ("normal", 300_001, (1, 3000, 299_999), {}, 1),
    ("student", 2_000_001, (1, 2000, 150_000), {}, 2),
    ("mixture", 3_000_000, (3000, 1, 2_999_999), {}, None),
    ("ties", 2_000_000, (5000,), {}, None),
    ("normal", 2_000_000, (20_000,), {"path": 3}, 3),
]


@pytest.mark.parametrize("kind,n,ks,opts,path", CASES, ids=[f"{c[0]}-{c[1]}-{c[3].get('path', 0)}" for c in CASES])
def test_order_stats_and_mask(oracle_mod, kind, n, ks, opts, path):
    r = inputs(kind, n, 500 + n % 97)
    rd = to_dev(r)
    o = L.default_options(**opts) if opts else None
    for k in ks:
        tau, st = L.topk_threshold(rd, k, options=o, stats=True)
        assert st["status"] == 0
        if path is not None:
            assert st["path_taken"] == path, (k, st["path_taken"])
        tk, tk1 = oracle_mod.order_stats(r.astype(np.float64), k)
        got = tau.cpu().numpy()
        assert got[0] == tk and got[1] == tk1, (kind, n, k, got, tk, tk1)
        mask, tau2 = L.hard_topk(rd, k, options=o)
        ref_mask, _, ones = oracle_mod.hard_topk(r.astype(np.float64), k)
        assert np.array_equal(mask.cpu().numpy().astype(np.float64), ref_mask)
        assert torch.equal(tau, tau2)


@pytest.mark.parametrize("kind,n,k,t", [("normal", 4096, 64, 0.1), ("normal", 1_000_000, 200, 0.05),
                                        ("mixture", 3_000_000, 3000, 0.01), ("ties", 2_000_000, 5000, 0.5)])
def test_dftopk(oracle_mod, kind, n, k, t):
    r = inputs(kind, n, 900 + k)
    p, b = L.dftopk(to_dev(r), k, t)
    torch.cuda.synchronize()
    p_ref, b_ref, s_ref = oracle_mod.dftopk(r.astype(np.float64), k, t32(t))
    assert float(b.item()) == b_ref
    ph = p.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(ph - p_ref)) <= P_TOL
    assert abs(ph.sum() - s_ref) <= SUM_TOL * k


def test_nonfinite_scores_rejected_on_the_bracketing_path():
    r = np.random.default_rng(5).standard_normal(2_000_000).astype(np.float32)
    r[123457] = np.nan
    with pytest.raises(L.LapsumError):
        L.hard_topk(to_dev(r), 1000)
