"""Shared helpers for the GPU parity tests: run the HIP path through the
C ABI (via the thin binding) and compare with the CPU oracle.

Parity gates (from the solver's accuracy targets):
  |b - b_oracle| <= 1e-5 t (plus the root's conditioning, see b_tolerance)
  max |p - p_oracle| <= 2e-6
  |sum p - k| <= 1e-5 k           (sum of the GPU's fp32 p, in fp64)
  VJP: max_i |grad_i - o_i| / ((f_i/t)(|g_i| + |c|)) <= 1e-4  (condition-aware)
"""
import numpy as np
import torch

P_TOL = 2e-6
SUM_TOL = 1e-5
VJP_TOL = 1e-4


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def b_tolerance(r64: np.ndarray, t: float, b: float) -> float:
    """1e-5 t, widened where the root is ill-conditioned: fp64 G - k is
    resolved to ~1e-16 n, and dG/db = -sum f / t, so b is only determined to
    ~1e-16 n t / sum f when sum f is tiny (b in a wide gap between scores)."""
    f = 0.5 * np.exp(-np.abs(r64 - b) / t)
    sf = float(f.sum())
    cond = 1e-13 * r64.size * t / max(sf, 1e-300)
    return 1e-5 * t + cond


def vjp_error(grad: np.ndarray, o: np.ndarray, r64: np.ndarray, g64: np.ndarray, t: float, b: float, c: float):
    f = 0.5 * np.exp(-np.abs(r64 - b) / t)
    scale = (f / t) * (np.abs(g64) + abs(c))
    # An fp32 result below FLT_MIN is subnormal or flushed to zero and carries
    # no relative accuracy; floor the scale where a 1e-4 relative error is
    # FLT_MIN, so such entries only need |error| <= FLT_MIN.
    scale = np.maximum(scale, np.finfo(np.float32).tiny / VJP_TOL)
    return float(np.max(np.abs(grad.astype(np.float64) - o) / scale))


def t32(t: float) -> float:
    """The C ABI takes t as fp32: the oracle is given exactly that value."""
    return float(np.float32(t))


def check_forward(oracle_mod, r: np.ndarray, k: float, t: float, p_gpu: np.ndarray, b_gpu: float,
                  b_ref: float = None, label: str = ""):
    t = t32(t)
    r64 = r.astype(np.float64)
    if b_ref is None:
        b_ref, _ = oracle_mod.solve(r64, k, t)
    tol = b_tolerance(r64, t, b_ref)
    assert abs(b_gpu - b_ref) <= tol, f"{label}: b {b_gpu!r} vs oracle {b_ref!r} (tol {tol:.3g})"
    p_ref, _ = oracle_mod.probs(r64, t, b_ref)
    dp = float(np.max(np.abs(p_gpu.astype(np.float64) - p_ref)))
    assert dp <= P_TOL, f"{label}: max |p - p_oracle| = {dp:.3g}"
    s = float(np.sum(p_gpu.astype(np.float64)))
    assert abs(s - k) <= SUM_TOL * k, f"{label}: sum p = {s!r}, k = {k}"
    return b_ref


def check_vjp(oracle_mod, r: np.ndarray, g: np.ndarray, t: float, b_ref: float, grad_gpu: np.ndarray, label=""):
    t = t32(t)
    r64 = r.astype(np.float64)
    g64 = g.astype(np.float64)
    o, c, _ = oracle_mod.vjp(r64, g64, t, b_ref)
    err = vjp_error(grad_gpu, o, r64, g64, t, b_ref, c)
    assert err <= VJP_TOL, f"{label}: VJP condition-aware error {err:.3g}"
    return err
