"""lapsum_forward_noalloc, the forward entry point that allocates nothing,
against lapsum_forward on the same inputs, through the C ABI.

Calls in a row on one GPU share its scratch array: each call's result must
match lapsum_forward's to the parity bar (b within 1e-5 t plus the root's
conditioning, p within 2e-6, sum p within 1e-5 k) whatever ran before it,
including a larger call just before a smaller one.  The oracle checks the
first call as well.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import P_TOL, SUM_TOL, b_tolerance, check_forward, t32, to_dev

pytestmark = pytest.mark.gpu

L = pytest.importorskip("differentiable_exact_budget_amd")


def forward_both(r, k, t):
    rd = to_dev(r)
    lib = L.lib()
    stream = torch.cuda.current_stream().cuda_stream
    p0, b0 = torch.empty_like(rd), torch.empty(1, dtype=torch.float64, device=rd.device)
    p1, b1 = torch.empty_like(rd), torch.empty(1, dtype=torch.float64, device=rd.device)
    assert lib.lapsum_forward(rd.data_ptr(), r.size, k, t, p0.data_ptr(), b0.data_ptr(), stream) == 0
    assert lib.lapsum_forward_noalloc(rd.data_ptr(), r.size, k, t, p1.data_ptr(), b1.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    return p0.cpu().numpy(), float(b0.item()), p1.cpu().numpy(), float(b1.item())


def same_to_the_bar(r, k, t, p0, b0, p1, b1, label):
    tol = b_tolerance(r.astype(np.float64), t32(t), b0)
    assert abs(b1 - b0) <= tol, f"{label}: b {b1!r} vs lapsum_forward {b0!r}"
    assert float(np.max(np.abs(p1.astype(np.float64) - p0.astype(np.float64)))) <= P_TOL, label
    assert abs(float(p1.astype(np.float64).sum()) - k) <= SUM_TOL * k, label


def test_noalloc_matches_forward_on_calls_in_a_row(oracle_mod):
    cases = [("C2", 1_000_000, 200.0, 0.05), ("normal", 300_001, 3000.0, 0.01), ("C1", 4096, 64.0, 0.1),
             ("student_t3", 16385, 100.0, 0.02), ("normal", 1 << 20, 5000.0, 0.05), ("normal", 17, 4.0, 0.3)]
    for i, (dist, n, k, t) in enumerate(cases):
        print(f"\n  call {i}: {dist} n={n} k={k} t={t}", flush=True)
        if dist in workloads.CONFIGS:
            r, _, cfg = workloads.config_inputs(dist)
            k, t = cfg.k, cfg.t
        else:
            r = workloads.scores(dist, n, 500 + i)
        p0, b0, p1, b1 = forward_both(r, k, t)
        same_to_the_bar(r, k, t, p0, b0, p1, b1, f"call {i}")
        if i == 0:
            check_forward(oracle_mod, r, k, t, p1, b1, label="noalloc C2")


def test_noalloc_rejects_sizes_beyond_its_scratch():
    lib = L.lib()
    rd = torch.zeros(16, device="cuda")
    assert lib.lapsum_forward_noalloc(rd.data_ptr(), (1 << 20) + 1, 5.0, 0.1, rd.data_ptr(), rd.data_ptr(),
                                      None) == 1
    assert lib.lapsum_forward_noalloc(None, 16, 5.0, 0.1, rd.data_ptr(), rd.data_ptr(), None) == 1
    assert lib.lapsum_forward_noalloc(rd.data_ptr(), 16, 16.0, 0.1, rd.data_ptr(), rd.data_ptr(), None) == 1


def test_noalloc_nonfinite_scores_give_nan():
    r = workloads.scores("normal", 50_000, 9)
    r[77] = np.nan
    rd = to_dev(r)
    p, b = torch.empty_like(rd), torch.empty(1, dtype=torch.float64, device=rd.device)
    assert L.lib().lapsum_forward_noalloc(rd.data_ptr(), r.size, 10.0, 0.1, p.data_ptr(), b.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert np.isnan(b.item()) and np.isnan(p.cpu().numpy()).all()
