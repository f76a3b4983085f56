"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests compares the oracle with itself: each uses an independent
derivation (50-digit interval enumeration, closed forms, limits, finite
differences, exact rational binomial sums, known-answer vectors, numpy masks).
Citations are to the Fast LapSum paper summaries: gist.science section 2.1
(the operator, its exact budget and analytic VJP), section 2.2 (bracketing),
section 2.3 (DFTopK as the zero-temperature limit).
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import workloads

mpmath.mp.dps = 50


# ---------------------------------------------------------------------------
# independent helpers (50-digit arithmetic, written from the definition)
# ---------------------------------------------------------------------------
def mp_G(r, t, b):
    """sum_i F((r_i - b)/t) at 50 digits."""
    t = mpmath.mpf(t)
    b = mpmath.mpf(b)
    s = mpmath.mpf(0)
    for v in r:
        x = (mpmath.mpf(float(v)) - b) / t
        s += mpmath.exp(x) / 2 if x < 0 else 1 - mpmath.exp(-x) / 2
    return s


def brute_force_roots(r, k, t):
    """Enumerate every interval between consecutive sorted scores.  On
    [v_j, v_{j+1}) the budget equation is, with w = e^{x/t},
        A/(2w) + (n - j - k) - B w / 2 = 0,
        A = sum_{i<=j} e^{v_i/t},  B = sum_{i>j} e^{-v_i/t},
    a quadratic with one positive root.  Returns every root that falls in
    its own interval."""
    t = mpmath.mpf(t)
    v = sorted(mpmath.mpf(float(x)) for x in r)
    n = len(v)
    roots = []
    for j in range(0, n + 1):  # j scores at or below the interval
        lo = v[j - 1] if j > 0 else -mpmath.inf
        hi = v[j] if j < n else mpmath.inf
        if j > 0 and j < n and lo == hi:
            continue
        A = mpmath.fsum(mpmath.exp(x / t) for x in v[:j])
        B = mpmath.fsum(mpmath.exp(-x / t) for x in v[j:])
        D = mpmath.mpf(n - j) - mpmath.mpf(k)
        sq = mpmath.sqrt(D * D + A * B)
        if D >= 0:
            if B == 0:
                continue
            w = (D + sq) / B
        else:
            w = A / (sq - D)  # same root, rationalised: no cancellation
        if w <= 0:
            continue
        x = t * mpmath.log(w)
        if lo <= x < hi:
            roots.append(x)
    return roots


def root_tolerance(r, t, root, b):
    """Forward-error bound for b: fp64 evaluation of G errs by a few ulps per
    term, and dG/db = -sum f / t, so |db| <= 8 n 2^-53 t / sum f (plus a
    1e-12 t floor).  Ill-conditioned roots (in a wide gap, sum f tiny) get a
    correspondingly wider bound."""
    tt = mpmath.mpf(t)
    sf = mpmath.fsum(mpmath.exp(-abs(mpmath.mpf(float(v)) - root) / tt) / 2 for v in r)
    return 1e-12 * t + 1e-15 * abs(b) + 8 * len(r) * 2.0 ** -53 * t / float(sf)


def laplace_quantile(y):
    """F^{-1}(y) for the scale-1 Laplace CDF."""
    return math.log(2 * y) if y < 0.5 else -math.log(2 * (1 - y))


# ---------------------------------------------------------------------------
# b and p
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,n,k,t", [
    (1, 1, 0.3, 0.5), (2, 2, 1.0, 0.1), (3, 3, 1.5, 1.0), (4, 5, 2.0, 0.05),
    (5, 8, 3.0, 0.2), (6, 12, 1.0, 0.01), (7, 16, 4.0, 0.3), (8, 16, 15.5, 2.0),
    (9, 16, 0.25, 0.1), (10, 11, 7.0, 0.001),
])
def test_bisection_matches_brute_force(oracle_mod, seed, n, k, t):
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(n).astype(np.float32)
    roots = brute_force_roots(r, k, t)
    assert len(roots) == 1, "the budget root must be unique (gist.science 2.1)"
    b, _ = oracle_mod.solve(r, k, t)
    assert abs(b - float(roots[0])) <= root_tolerance(r, t, roots[0], b)
    # and the 50-digit G at the oracle's b is k to fp64 accuracy
    assert abs(mp_G(r, t, b) - k) <= 1e-12 * max(1.0, k)


def test_brute_force_with_ties(oracle_mod):
    r = np.array([0.5, 0.5, 0.5, -1.0, 2.0, 2.0, 0.0, 0.0], dtype=np.float32)
    for k in (0.5, 1.0, 2.0, 3.0, 4.5, 7.9):
        for t in (0.01, 0.3, 3.0):
            roots = brute_force_roots(r, k, t)
            assert len(roots) == 1
            b, _ = oracle_mod.solve(r, k, t)
            assert abs(b - float(roots[0])) <= root_tolerance(r, t, roots[0], b)


def test_G_matches_50_digit_sum(oracle_mod):
    rng = np.random.default_rng(11)
    r = rng.standard_normal(300).astype(np.float32) * 3
    for b in (-2.0, 0.0, 0.7, 5.0):
        for t in (0.01, 1.0):
            assert abs(oracle_mod.budget_G(r, t, b) - float(mp_G(r, t, b))) <= 1e-13 * r.size


@pytest.mark.parametrize("c,n,k,t", [(0.0, 10, 3.0, 1.0), (1.25, 100, 50.0, 0.1),
                                     (-3.5, 1000, 999.0, 0.01), (2.0, 7, 0.001, 0.5)])
def test_all_equal_closed_form(oracle_mod, c, n, k, t):
    """r_i = c: n F((c-b)/t) = k  =>  b = c - t F^{-1}(k/n)."""
    r = np.full(n, c, dtype=np.float32)
    b, _ = oracle_mod.solve(r, k, t)
    expect = c - t * laplace_quantile(k / n)
    assert abs(b - expect) <= 1e-13 * max(1.0, abs(expect))


@pytest.mark.parametrize("k", [0.01, 0.3, 0.5, 0.99])
def test_single_score_closed_form(oracle_mod, k):
    b, _ = oracle_mod.solve(np.array([0.75], dtype=np.float32), k, 0.2)
    assert abs(b - (0.75 - 0.2 * laplace_quantile(k))) <= 1e-14


def test_zero_temperature_limit_is_hard_topk(oracle_mod):
    """gist.science 2.3: DFTopK (threshold at the midpoint of order statistics
    k and k+1) is LapSum's zero-temperature limit, so p -> the hard top-k
    indicator.  Tie-free integers with unit gaps, t = 0.01: every p is within
    e^{-gap/(2t)} / 2 = e^{-50}/2 of 0 or 1, below fp64 resolution next to 1."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "zero_temperature_topk.txt")
    row = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")][0]
    n, k, t, b_limit = int(row[0]), int(row[1]), float(row[2]), float(row[3])
    rng = np.random.default_rng(3)
    r = rng.permutation(np.arange(n, dtype=np.float32))
    b, _ = oracle_mod.solve(r, k, t)
    srt = np.sort(r)[::-1]
    mid = 0.5 * (srt[k - 1] + srt[k])
    assert mid == b_limit
    assert abs(b - mid) <= 1e-9
    p, s = oracle_mod.probs(r, t, b)
    hard = (r >= srt[k - 1]).astype(np.float64)
    assert np.max(np.abs(p - hard)) <= max(0.5 * math.exp(-50), 2.0 ** -53)
    assert abs(s - k) <= 1e-12 * k


def test_invariants_on_configs(oracle_mod):
    for name, n in (("C1", None), ("C2", 200_000), ("C3", 200_000), ("C4", 200_000), ("C5", 200_000)):
        r, _, cfg = workloads.config_inputs(name, n)
        k = min(cfg.k, 0.5 * r.size)
        b, _ = oracle_mod.solve(r, k, cfg.t)
        p, s = oracle_mod.probs(r, cfg.t, b)
        assert abs(s - k) <= 1e-11 * k  # exact budget, gist.science 2.1 / 4.1
        assert np.all(p >= 0) and np.all(p <= 1)
        order = np.argsort(r, kind="stable")
        assert np.all(np.diff(p[order]) >= 0), "p must be monotone in r"


def test_equivariance(oracle_mod):
    rng = np.random.default_rng(5)
    r = rng.standard_normal(2000).astype(np.float32)
    k, t = 37.0, 0.07
    b, _ = oracle_mod.solve(r, k, t)
    r64 = r.astype(np.float64)
    b_shift, _ = oracle_mod.solve(r64 + 0.5, k, t)  # exact shift in fp64
    assert abs(b_shift - (b + 0.5)) <= 1e-13
    b_scale, _ = oracle_mod.solve(r64 * 2.0, k, 2 * t)  # exact scaling
    assert abs(b_scale - 2.0 * b) <= 1e-13
    perm = rng.permutation(r.size)
    b_perm, _ = oracle_mod.solve(r[perm], k, t)
    assert abs(b_perm - b) <= 1e-14
    p, _ = oracle_mod.probs(r, t, b)
    p_perm, _ = oracle_mod.probs(r[perm], t, b_perm)
    assert np.max(np.abs(p_perm - p[perm])) <= 1e-15


def test_invalid_arguments(oracle_mod):
    r = np.zeros(4, dtype=np.float32)
    for k, t in ((0.0, 1.0), (4.0, 1.0), (-1.0, 1.0), (1.0, 0.0), (1.0, -1.0), (1.0, float("inf"))):
        with pytest.raises(ValueError):
            oracle_mod.solve(r, k, t)
    with pytest.raises(ValueError):
        oracle_mod.solve(np.array([0.0, np.nan], dtype=np.float32), 1.0, 1.0)


# ---------------------------------------------------------------------------
# VJP (gist.science 2.1: analytic vector-Jacobian product)
# ---------------------------------------------------------------------------
def _loss(oracle_mod, r64, g, k, t):
    b, _ = oracle_mod.solve(r64, k, t)
    p, _ = oracle_mod.probs(r64, t, b)
    return float(np.dot(g, p))


def test_vjp_central_differences(oracle_mod):
    rng = np.random.default_rng(8)
    n, k, t = 50, 7.0, 0.3
    r = rng.standard_normal(n)
    g = rng.standard_normal(n)
    b, _ = oracle_mod.solve(r, k, t)
    grad, _, _ = oracle_mod.vjp(r, g, t, b)
    h = 1e-6
    fd = np.empty(n)
    for j in range(n):
        rp = r.copy(); rp[j] += h
        rm = r.copy(); rm[j] -= h
        fd[j] = (_loss(oracle_mod, rp, g, k, t) - _loss(oracle_mod, rm, g, k, t)) / (2 * h)
    assert np.max(np.abs(fd - grad)) <= 1e-7 * max(1.0, np.max(np.abs(grad)))


def test_vjp_identities(oracle_mod):
    rng = np.random.default_rng(9)
    r = rng.standard_normal(500)
    k, t = 20.0, 0.2
    b, _ = oracle_mod.solve(r, k, t)
    g = rng.standard_normal(500)
    grad, c, sf = oracle_mod.vjp(r, g, t, b)
    # translation invariance of p: sum_j dp_i/dr_j = 0
    assert abs(grad.sum()) <= 1e-12 * np.abs(grad).sum()
    # sum p is constant (= k), so g = 1 gives a zero gradient
    g1, _, _ = oracle_mod.vjp(r, np.ones(500), t, b)
    assert np.max(np.abs(g1)) <= 1e-14
    # the Jacobian is symmetric: u.(J v) = v.(J u)
    u = rng.standard_normal(500)
    v = rng.standard_normal(500)
    ju, _, _ = oracle_mod.vjp(r, u, t, b)
    jv, _, _ = oracle_mod.vjp(r, v, t, b)
    assert abs(np.dot(u, jv) - np.dot(v, ju)) <= 1e-12 * (np.abs(u).sum() + np.abs(v).sum())
    # sum f is the negative t-scaled slope of G at b
    h = 1e-7
    slope = (oracle_mod.budget_G(r, t, b + h) - oracle_mod.budget_G(r, t, b - h)) / (2 * h)
    assert abs(slope + sf / t) <= 1e-6 * sf / t


# ---------------------------------------------------------------------------
# gradients with respect to the budget and the temperature
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed,n,k,t", [(11, 50, 7.3, 0.3), (12, 200, 0.7, 0.05), (13, 40, 33.0, 2.0)])
def test_vjp_kt_central_differences(oracle_mod, seed, n, k, t):
    """dL/dk and dL/dt against central differences of L = sum g p through
    the oracle's own solve."""
    rng = np.random.default_rng(seed)
    r = rng.standard_normal(n)
    g = rng.standard_normal(n)
    b, _ = oracle_mod.solve(r, k, t)
    dk, dt = oracle_mod.vjp_kt(r, g, t, b)
    hk = 1e-6 * k
    fdk = (_loss(oracle_mod, r, g, k + hk, t) - _loss(oracle_mod, r, g, k - hk, t)) / (2 * hk)
    ht = 1e-6 * t
    fdt = (_loss(oracle_mod, r, g, k, t + ht) - _loss(oracle_mod, r, g, k, t - ht)) / (2 * ht)
    scale_k = np.abs(g).max()
    scale_t = np.abs(g).sum() * (np.abs(r).max() + abs(b)) / t ** 2
    assert abs(fdk - dk) <= 1e-7 * abs(dk) + 1e-10 * scale_k, (fdk, dk)
    assert abs(fdt - dt) <= 1e-6 * abs(dt) + 1e-12 * scale_t, (fdt, dt)


def test_vjp_kt_closed_forms(oracle_mod):
    rng = np.random.default_rng(14)
    g = rng.standard_normal(64)
    # equal scores: p_i = k/n whatever t, so dL/dk = mean(g) and dL/dt = 0
    r = np.full(64, 0.75)
    b, _ = oracle_mod.solve(r, 10.0, 0.2)
    dk, dt = oracle_mod.vjp_kt(r, g, 0.2, b)
    assert abs(dk - g.mean()) <= 1e-14 * np.abs(g).sum()
    assert abs(dt) <= 1e-12 * np.abs(g).sum()
    # g = 1: L = sum p = k, so dL/dk = 1 and dL/dt = 0
    r = rng.standard_normal(300)
    b, _ = oracle_mod.solve(r, 12.5, 0.1)
    dk, dt = oracle_mod.vjp_kt(r, np.ones(300), 0.1, b)
    assert abs(dk - 1.0) <= 1e-14
    assert abs(dt) <= 1e-10


def test_vjp_kt_scale_identity(oracle_mod):
    """p is unchanged by (r, t) -> (a r, a t), so d/da L(a r, a t) = 0 at a = 1:
    t dL/dt = -sum_i r_i dL/dr_i, tying the temperature gradient to the
    score gradient."""
    rng = np.random.default_rng(15)
    r = rng.standard_normal(400) * 3.0 + 1.0
    g = rng.standard_normal(400)
    k, t = 31.0, 0.4
    b, _ = oracle_mod.solve(r, k, t)
    grad, _, _ = oracle_mod.vjp(r, g, t, b)
    _, dt = oracle_mod.vjp_kt(r, g, t, b)
    assert abs(t * dt + np.dot(r, grad)) <= 1e-12 * np.abs(r * grad).sum()


# ---------------------------------------------------------------------------
# order statistics, hard top-k and DFTopK (gist.science 2.3)
# ---------------------------------------------------------------------------
def _kth_largest_by_counts(r, k):
    """The k-th largest written as a count condition, no sorting: the score v
    with #(r > v) < k <= #(r >= v)."""
    cands = [v for v in set(r.tolist()) if np.sum(r > v) < k <= np.sum(r >= v)]
    assert len(cands) == 1
    return cands[0]


@pytest.mark.parametrize("seed", range(6))
def test_order_stats_count_definition(oracle_mod, seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 40))
    r = rng.integers(-3, 4, size=n).astype(np.float64)  # many ties
    for k in range(1, n + 1):
        tk, tk1 = oracle_mod.order_stats(r, k)
        assert tk == _kth_largest_by_counts(r, k)
        assert tk1 == (_kth_largest_by_counts(r, k + 1) if k < n else -np.inf)
        mask, tau, ones = oracle_mod.hard_topk(r, k)
        assert tau == tk and ones == int(np.sum(r >= tk)) and ones >= k
        assert np.array_equal(mask, (r >= tk).astype(np.float64))
    with pytest.raises(ValueError):
        oracle_mod.order_stats(r, 0)
    with pytest.raises(ValueError):
        oracle_mod.order_stats(r, n + 1)


def test_hard_topk_tie_free_selects_exactly_k(oracle_mod):
    rng = np.random.default_rng(7)
    r = rng.permutation(5000).astype(np.float64) * 0.37 - 100.0
    for k in (1, 2, 17, 2500, 4999, 5000):
        mask, tau, ones = oracle_mod.hard_topk(r, k)
        assert ones == k
        top = np.argpartition(-r, k - 1)[:k]
        expect = np.zeros(r.size)
        expect[top] = 1.0
        assert np.array_equal(mask, expect)


def test_dftopk_is_the_zero_temperature_limit(oracle_mod):
    """The DFTopK threshold is the value LapSum's b tends to as t -> 0 (the
    golden row: scores 0..19, k = 5, b -> 14.5)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "zero_temperature_topk.txt")
    row = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")][0]
    n, k, t, b_limit = int(row[0]), int(row[1]), float(row[2]), float(row[3])
    r = np.random.default_rng(3).permutation(np.arange(n, dtype=np.float64))
    p, b, s = oracle_mod.dftopk(r, k, t)
    assert b == b_limit
    b_lapsum, _ = oracle_mod.solve(r, k, t)
    assert abs(b - b_lapsum) <= 1e-9


def test_dftopk_mass_closed_forms(oracle_mod):
    """DFTopK keeps the midpoint whatever t, so its mass drifts from k.
    Scores {0, 1, 2}, k = 1: b = 1.5 and sum p = 1 + e^{-1.5/t}/2 exactly.
    Scores {0, 1}, k = 1: b = 0.5 and sum p = 1 by symmetry."""
    for t in (0.05, 0.5, 2.0):
        _, b, s = oracle_mod.dftopk(np.array([2.0, 0.0, 1.0]), 1, t)
        assert b == 1.5
        assert abs(s - (1.0 + 0.5 * math.exp(-1.5 / t))) <= 1e-15
        _, b, s = oracle_mod.dftopk(np.array([1.0, 0.0]), 1, t)
        assert b == 0.5 and abs(s - 1.0) <= 1e-15
    with pytest.raises(ValueError):
        oracle_mod.dftopk(np.array([1.0, 0.0]), 2, 0.1)


# ---------------------------------------------------------------------------
# bracket bookkeeping (gist.science 2.2, streaming and filtering)
# ---------------------------------------------------------------------------
def test_bracket_counts_band_and_tail_identity(oracle_mod):
    r, _, _ = workloads.config_inputs("C3", 100_000)
    t = 0.01
    for aL, aR in ((1.0, 2.5), (-np.inf, 0.0), (3.0, np.inf), (0.3, 0.3000001)):
        aL32, aR32 = np.float32(aL), np.float32(aR)
        res = oracle_mod.bracket(r, t, float(aL32), float(aR32))
        below = r < aL32
        above = r >= aR32
        band = ~below & ~above
        assert res["below"] == below.sum() and res["above"] == above.sum() and res["band"] == band.sum()
        assert np.array_equal(res["band_values"], np.sort(r[band]).astype(np.float64))
        # G(a_L) and G(a_R) rebuilt from the tail sums must equal the direct sums
        m, cR = res["band"], res["above"]
        if np.isfinite(aL32):
            cross = 0.0 if not np.isfinite(aR32) else math.exp((float(aL32) - float(aR32)) / t) * res["S_R"]
            G_aL = 0.5 * res["S_L"] + m - 0.5 * res["B_L"] + cR - 0.5 * cross
            assert abs(G_aL - res["G_aL"]) <= 1e-9 * max(1.0, res["G_aL"])
        if np.isfinite(aR32):
            cross = 0.0 if not np.isfinite(aL32) else math.exp((float(aL32) - float(aR32)) / t) * res["S_L"]
            G_aR = 0.5 * cross + 0.5 * res["B_R"] + cR - 0.5 * res["S_R"]
            assert abs(G_aR - res["G_aR"]) <= 1e-9 * max(1.0, res["G_aR"])


def test_sorted_keys_match_numpy(oracle_mod):
    r = np.array([0.0, -0.0, 1.0, -1.0, np.float32(1e-38), -np.float32(1e-45), 3.0, -0.0], dtype=np.float32)
    out = oracle_mod.sort_keys(r)
    ref = np.sort(np.where(r == 0, np.float32(0), r))
    assert np.array_equal(out.view(np.uint32), ref.view(np.uint32))
    r2, _, _ = workloads.config_inputs("C5", 50_000)
    assert np.array_equal(oracle_mod.sort_keys(r2), np.sort(r2))


# ---------------------------------------------------------------------------
# sampling: Philox and binomial order statistics (gist.science 2.2 step 1)
# ---------------------------------------------------------------------------
def _load_kat():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.txt")
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        w = [int(x, 16) for x in line.split()]
        rows.append((tuple(w[0:4]), tuple(w[4:6]), tuple(w[6:10])))
    return rows


# Known-answer vectors of the Random123 library (tests/golden, with citation)
PHILOX_KAT = _load_kat()


@pytest.mark.parametrize("ctr,key,expect", PHILOX_KAT)
def test_philox_known_answers(oracle_mod, ctr, key, expect):
    assert tuple(int(x) for x in oracle_mod.philox4x32_10(ctr, key)) == expect


def _exact_binomial_bounds(s, q, delta):
    """Exact rational CDF of Bin(s, q) (q as the rational value of the fp64)."""
    qf = Fraction(q)
    pmf = [Fraction(math.comb(s, i)) * qf ** i * (1 - qf) ** (s - i) for i in range(s + 1)]
    d = Fraction(delta)
    l, cdf = 0, Fraction(0)
    for y in range(s + 1):
        cdf += pmf[y]
        if cdf <= d:
            l = y + 1
        else:
            break
    h, tail = s + 1, Fraction(0)
    for i in range(s, -1, -1):
        tail += pmf[i]
        if tail <= d:
            h = i
        else:
            break
    miss = sum(pmf[:l], Fraction(0)) + sum(pmf[h:], Fraction(0))
    return l, h, float(miss)


@pytest.mark.parametrize("s,q,delta", [(50, 0.9, 0.01), (200, 0.99, 1e-3), (120, 0.5, 1e-5),
                                       (64, 0.999, 0.05), (30, 0.2, 0.1)])
def test_binomial_bounds_exact(oracle_mod, s, q, delta):
    l, h = oracle_mod.binomial_bounds(s, q, delta)
    el, eh, emiss = _exact_binomial_bounds(s, q, delta)
    assert (l, h) == (el, eh)
    assert abs(oracle_mod.binomial_miss(s, q, l, h) - emiss) <= 1e-12 + 1e-9 * emiss


def test_noised_sample_quantile_is_the_threshold(oracle_mod):
    """With x = r_I + Laplace(0, t) noise, P(x > b) = G(b)/n = k/n exactly, so
    the order statistics x_(l), x_(h) bracket b with the exact binomial miss
    probability.  Over many seeds the observed miss count must be consistent
    with it (two-sided binomial test)."""
    from scipy import stats
    rng = np.random.default_rng(21)
    r = rng.standard_t(3.0, 5000).astype(np.float32)
    k, t = 250.0, 0.3
    b, _ = oracle_mod.solve(r, k, t)
    s = 200
    q = 1.0 - k / r.size
    l, h = oracle_mod.binomial_bounds(s, q, 0.02)
    miss_p = oracle_mod.binomial_miss(s, q, l, h)
    trials, misses = 3000, 0
    for seed in range(trials):
        _, x = oracle_mod.sample(r, t, 0x5EED0000 + seed, s)
        xs = np.sort(x.astype(np.float64))
        aL = xs[l - 1] if l >= 1 else -np.inf
        aR = xs[h - 1] if h <= s else np.inf
        if not (aL <= b < aR):
            misses += 1
    pval = stats.binomtest(misses, trials, miss_p).pvalue
    assert pval > 1e-3, (misses, trials, miss_p)


def test_sample_indices_are_uniform(oracle_mod):
    r = np.arange(1000, dtype=np.float64)
    idx, _ = oracle_mod.sample(r, 1.0, 123, 200_000)
    assert idx.min() >= 0 and idx.max() < 1000
    counts = np.bincount(idx, minlength=1000)
    from scipy import stats
    assert stats.chisquare(counts).pvalue > 1e-4


def test_thread_count_does_not_change_results(oracle_mod):
    r, _, cfg = workloads.config_inputs("C3", 300_000)
    before = oracle_mod.get_threads()
    try:
        oracle_mod.set_threads(1)
        b1, _ = oracle_mod.solve(r, 300.0, cfg.t)
        oracle_mod.set_threads(4)
        b4, _ = oracle_mod.solve(r, 300.0, cfg.t)
    finally:
        oracle_mod.set_threads(before)
    assert b1 == b4
