"""GPU parity of the row-wise (batched) operator against the oracle, row by
row: b, p, the mass of every row and the VJP, for each workgroup size, per-row
budgets, long rows that go through the single-vector solver, and rows that
must come out as NaN (a non-finite score, a budget outside (0, n))."""
import numpy as np
import pytest
import torch

from gpu_helpers import check_forward, check_vjp, t32, to_dev

pytestmark = pytest.mark.gpu

L = pytest.importorskip("differentiable_exact_budget_amd")


@pytest.mark.parametrize("rows,n,per_row_k,t", [
    (1000, 8, False, 0.3), (3000, 64, True, 0.05), (513, 257, False, 0.1), (200, 4096, True, 0.01),
    (20, 16384, False, 0.02), (3, 20000, True, 0.05),
])
def test_rows_match_oracle(oracle_mod, rows, n, per_row_k, t):
    rng = np.random.default_rng(rows * 7 + n)
    r = rng.standard_normal((rows, n)).astype(np.float32)
    g = rng.standard_normal((rows, n)).astype(np.float32)
    if per_row_k:
        k = rng.uniform(0.5, n - 0.5, size=rows)
        kd = torch.from_numpy(k).cuda()
    else:
        k = np.full(rows, max(1.0, n / 8))
        kd = float(k[0])
    rd = to_dev(r)
    p, b = L.forward_rows(rd, kd, t)
    grad = L.vjp_rows(rd, to_dev(g), t, b)
    torch.cuda.synchronize()
    ph, bh, gh = p.cpu().numpy(), b.cpu().numpy(), grad.cpu().numpy()
    check_rows = range(rows) if rows <= 200 else rng.choice(rows, 200, replace=False)
    for i in check_rows:
        b_ref = check_forward(oracle_mod, r[i], float(k[i]), t, ph[i], float(bh[i]), label=f"row {i}")
        check_vjp(oracle_mod, r[i], g[i], t, b_ref, gh[i], label=f"row {i}")


def test_rows_bad_rows_are_nan():
    rng = np.random.default_rng(3)
    r = rng.standard_normal((6, 100)).astype(np.float32)
    r[2, 17] = np.nan
    r[4, 3] = np.inf
    k = torch.tensor([5.0, 0.0, 5.0, 100.0, 5.0, 99.5], dtype=torch.float64, device="cuda")
    p, b = L.forward_rows(to_dev(r), k, 0.1)
    bh = b.cpu().numpy()
    ph = p.cpu().numpy()
    for i in range(6):
        bad = i in (1, 2, 3, 4)
        assert np.isnan(bh[i]) == bad
        assert np.all(np.isnan(ph[i])) == bad
        if not bad:
            assert abs(ph[i].astype(np.float64).sum() - float(k[i])) <= 1e-5 * float(k[i])


def test_rows_autograd_matches_vjp(oracle_mod):
    rng = np.random.default_rng(4)
    r = rng.standard_normal((64, 512)).astype(np.float32)
    w = rng.standard_normal((64, 512)).astype(np.float32)
    rd = to_dev(r).requires_grad_(True)
    p = L.soft_topk_rows(rd, 16.0, 0.05)
    (p * to_dev(w)).sum().backward()
    _, b = L.forward_rows(to_dev(r), 16.0, 0.05)
    ref = L.vjp_rows(to_dev(r), to_dev(w), 0.05, b)
    assert torch.equal(rd.grad, ref)
    b_ref, _ = oracle_mod.solve(r[5].astype(np.float64), 16.0, t32(0.05))
    assert abs(float(b[5].item()) - b_ref) <= 1e-5 * 0.05
