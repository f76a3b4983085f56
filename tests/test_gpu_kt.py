"""GPU parity of the budget and temperature gradients (lapsum_vjp_kt).

dL/dk and dL/dt are compared with the oracle's fp64 values with tolerances
scaled by the sums they are built from.  The score gradient of
lapsum_vjp_kt must equal lapsum_vjp's bit for bit, since both use the same
apply pass and the same c.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import t32, to_dev

pytestmark = pytest.mark.gpu

L = pytest.importorskip("differentiable_exact_budget_amd")

KT_TOL = 1e-5


def kt_scales(r64, g64, t, b):
    d = r64 - b
    f = 0.5 * np.exp(-np.abs(d) / t)
    sf = f.sum()
    mu = float((f * d).sum() / sf)
    scale_k = float((np.abs(g64) * f).sum() / sf)
    # dt = -(sum g f d - mu sum g f)/t^2 cancels terms of size sum |g| f |d| / t^2:
    # their fp64 rounding is a floor under the condition-aware scale
    scale_t = float((np.abs(g64) * f * np.abs(d - mu)).sum() / t ** 2)
    scale_t += 1e-8 * float((np.abs(g64) * f * np.abs(d)).sum() / t ** 2)
    return scale_k, scale_t


def check_kt(oracle_mod, r, g, t, b_gpu, dk, dt, label):
    t = t32(t)
    r64, g64 = r.astype(np.float64), g.astype(np.float64)
    dk_o, dt_o = oracle_mod.vjp_kt(r64, g64, t, b_gpu)
    sk, st_ = kt_scales(r64, g64, t, b_gpu)
    assert abs(dk - dk_o) <= KT_TOL * sk + 1e-300, f"{label}: dk {dk!r} vs {dk_o!r} (scale {sk:.3g})"
    assert abs(dt - dt_o) <= KT_TOL * st_ + 1e-300, f"{label}: dt {dt!r} vs {dt_o!r} (scale {st_:.3g})"


@pytest.mark.parametrize("name,n", [("C1", None), ("C2", None), ("C3", 2_000_000), ("C4", 3_000_000)])
def test_vjp_kt_matches_oracle(oracle_mod, name, n):
    cfg = workloads.CONFIGS[name]
    nn = n or cfg.n
    r = workloads.scores(cfg.dist, nn, 1000 + cfg.number, k=cfg.k * nn / cfg.n)
    g = workloads.upstream(nn, 2000 + cfg.number)
    k = cfg.k * nn / cfg.n
    rd, gd = to_dev(r), to_dev(g)
    p, b = L.forward(rd, k, cfg.t)
    grad_kt, dk, dt = L.vjp_kt(rd, gd, cfg.t, b)
    grad = L.vjp(rd, gd, cfg.t, b)
    torch.cuda.synchronize()
    assert torch.equal(grad_kt, grad), "score gradient must not depend on the entry point"
    check_kt(oracle_mod, r, g, cfg.t, float(b.item()), float(dk.item()), float(dt.item()), name)


def test_vjp_kt_scalars_only_and_edges(oracle_mod):
    rng = np.random.default_rng(41)
    for n, k, t in ((1, 0.4, 0.5), (7, 3.0, 0.2), (1001, 17.5, 0.05), (70001, 1234.0, 0.01)):
        r = rng.standard_normal(n).astype(np.float32)
        g = rng.standard_normal(n).astype(np.float32)
        rd, gd = to_dev(r), to_dev(g)
        _, b = L.forward(rd, k, t)
        none, dk, dt = L.vjp_kt(rd, gd, t, b, want_grad=False)
        assert none is None
        torch.cuda.synchronize()
        check_kt(oracle_mod, r, g, t, float(b.item()), float(dk.item()), float(dt.item()), f"n={n}")
    # g = 1: the loss is sum p = k exactly, so dk = 1 and dt = 0
    r = rng.standard_normal(5000).astype(np.float32)
    rd = to_dev(r)
    _, b = L.forward(rd, 50.0, 0.1)
    _, dk, dt = L.vjp_kt(rd, torch.ones_like(rd), 0.1, b, want_grad=False)
    assert abs(float(dk.item()) - 1.0) <= 1e-12
    _, st_ = kt_scales(r.astype(np.float64), np.ones(5000), t32(0.1), float(b.item()))
    assert abs(float(dt.item())) <= 1e-9 * st_


def test_autograd_budget_and_temperature(oracle_mod):
    rng = np.random.default_rng(42)
    n = 20000
    r = rng.standard_normal(n).astype(np.float32)
    w = rng.standard_normal(n).astype(np.float32)
    rd = to_dev(r).requires_grad_(True)
    k = torch.tensor(150.0, dtype=torch.float64, requires_grad=True)
    t = torch.tensor(0.05, dtype=torch.float32, device="cuda", requires_grad=True)
    p = L.soft_topk(rd, k, t)
    loss = (p * to_dev(w)).sum()
    loss.backward()
    assert k.grad is not None and t.grad is not None and rd.grad is not None
    assert k.grad.device.type == "cpu" and t.grad.device.type == "cuda"
    b_ref, _ = oracle_mod.solve(r.astype(np.float64), 150.0, t32(0.05))
    check_kt(oracle_mod, r, w, 0.05, b_ref, float(k.grad.item()), float(t.grad.item()), "autograd")
