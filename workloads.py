"""Seeded synthetic workloads for the LapSum solver (shared by tests and bench).

This module only draws inputs; it holds none of the solver's arithmetic.
All draws use numpy's PCG64 generator in fp64, then round to fp32.

The pages that describe the method (the Fast LapSum paper summaries) print no
workload: no distribution, k or t for any timing.  The five configurations
below are synthetic stand-ins with the stated sizes and shapes:

  C1  n = 4096,   N(0,1),                               k = 64,   t = 0.1
  C2  n = 10^6,   N(0,1),                               k = 200,  t = 0.05
  C3  n = 10^7,   Student-t with 3 degrees of freedom,   k = 10^4, t = 0.01
  C4  n = 10^8,   per element: U(0,1) w.p. 0.9, else N(2, sd 0.5),
                                                        k = 10^5, t = 0.01
  C5  n = 10^7,   N(0,1); then 10^5 positions (without replacement) are set
                  to q, nextafter(q, +inf) or nextafter(q, -inf) (prob 1/3
                  each), q = the ascending order statistic n - k of the base
                  draw (0-based index);                 k = 10^5, t = 1e-3

Scores use seed 1000 + config number, upstream gradients g ~ N(0,1) use
seed 2000 + config number.
"""
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Config:
    name: str
    n: int
    k: float
    t: float
    dist: str
    path: str  # the path the configuration exercises: "full", "bracket", "fallback"
    number: int


CONFIGS = {
    "C1": Config("C1", 4096, 64.0, 0.1, "normal", "full", 1),
    "C2": Config("C2", 1_000_000, 200.0, 0.05, "normal", "full", 2),
    "C3": Config("C3", 10_000_000, 1e4, 0.01, "student_t3", "bracket", 3),
    "C4": Config("C4", 100_000_000, 1e5, 0.01, "mixture", "bracket", 4),
    "C5": Config("C5", 10_000_000, 1e5, 1e-3, "adversarial", "bracket", 5),
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def scores(dist: str, n: int, seed: int, k: float = None) -> np.ndarray:
    """fp32 scores of length n drawn from `dist` with the given seed."""
    rng = _rng(seed)
    if dist == "normal":
        x = rng.standard_normal(n)
    elif dist == "student_t3":
        x = rng.standard_t(3.0, n)
    elif dist == "mixture":
        pick = rng.random(n) < 0.9
        u = rng.random(n)
        z = rng.normal(2.0, 0.5, n)
        x = np.where(pick, u, z)
        del u, z, pick
    elif dist == "adversarial":
        if k is None:
            raise ValueError("adversarial scores need k")
        base = rng.standard_normal(n).astype(np.float32)
        kk = int(k)
        q = np.partition(base, n - kk)[n - kk]
        pos = rng.choice(n, size=min(kk, n), replace=False)
        which = rng.integers(0, 3, size=pos.size)
        vals = np.empty(pos.size, dtype=np.float32)
        vals[which == 0] = q
        vals[which == 1] = np.nextafter(q, np.float32(np.inf))
        vals[which == 2] = np.nextafter(q, np.float32(-np.inf))
        base[pos] = vals
        return base
    elif dist == "uniform":
        x = rng.random(n)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float32)


def upstream(n: int, seed: int) -> np.ndarray:
    """Upstream gradient g ~ N(0,1), fp32."""
    return _rng(seed).standard_normal(n).astype(np.float32)


def config_inputs(name: str, n: int = None):
    """(r, g, cfg) for a named configuration.  `n` overrides the size (same
    distribution and seeds) for scaled-down parity runs."""
    cfg = CONFIGS[name]
    nn = cfg.n if n is None else int(n)
    r = scores(cfg.dist, nn, 1000 + cfg.number, k=cfg.k)
    g = upstream(nn, 2000 + cfg.number)
    return r, g, cfg
