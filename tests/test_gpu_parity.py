"""GPU parity: the HIP path (through the C ABI) against the CPU fp64 oracle
on the same seeded inputs.  Sizes here let the oracle finish in seconds while
spanning several tiles, buckets and a ragged tail; the full-size workloads are
in test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import check_forward, check_vjp, t32, to_dev

pytestmark = pytest.mark.gpu

L = pytest.importorskip("differentiable_exact_budget_amd")


def run(r, k, t, g=None, **opts):
    rd = to_dev(r)
    o = L.default_options(**opts) if opts else None
    p, b, st = L.forward(rd, k, t, options=o, stats=True)
    grad = None
    if g is not None:
        grad = L.vjp(rd, to_dev(g), t, b).cpu().numpy()
    torch.cuda.synchronize()
    return p.cpu().numpy(), float(b.cpu().item()), st, grad


# ---------------------------------------------------------------------------
# full-sort path
# ---------------------------------------------------------------------------
def test_c1_small_solve(oracle_mod):
    r, g, cfg = workloads.config_inputs("C1")
    p, b, st, grad = run(r, cfg.k, cfg.t, g)
    assert st["path_taken"] == 1 and st["status"] == 0
    b_ref = check_forward(oracle_mod, r, cfg.k, cfg.t, p, b, label="C1")
    check_vjp(oracle_mod, r, g, cfg.t, b_ref, grad, label="C1")


@pytest.mark.parametrize("n,k,t", [(1, 0.3, 0.5), (2, 1.0, 0.1), (3, 2.5, 1.0), (17, 4.0, 0.05),
                                   (1000, 999.5, 0.01), (16384, 100.0, 0.01), (5, 0.001, 0.2),
                                   # k close to n: b below every score (the solve's below-range edge)
                                   (4096, 4095.9, 0.05), (10000, 9999.7, 0.02), (16384, 16383.5, 0.1)])
def test_small_solve_edges(oracle_mod, n, k, t):
    rng = np.random.default_rng(n)
    r = rng.standard_normal(n).astype(np.float32)
    g = rng.standard_normal(n).astype(np.float32)
    p, b, st, grad = run(r, k, t, g)
    b_ref = check_forward(oracle_mod, r, k, t, p, b, label=f"n={n}")
    check_vjp(oracle_mod, r, g, t, b_ref, grad, label=f"n={n}")
    if k > n - 0.5:
        assert b_ref < float(r.min())  # the case is the below-range edge


def test_small_solve_ties_and_zero_temperature(oracle_mod):
    r = np.array([0.5, 0.5, 0.5, -1.0, 2.0, 2.0, 0.0, -0.0], dtype=np.float32)
    for k in (0.5, 1.0, 2.0, 3.0, 4.5, 7.9):
        for t in (0.01, 0.3, 3.0):
            p, b, st, _ = run(r, k, t)
            check_forward(oracle_mod, r, k, t, p, b, label=f"ties k={k} t={t}")
    r = np.random.default_rng(3).permutation(np.arange(20, dtype=np.float32))
    p, b, st, _ = run(r, 5.0, 0.01)
    assert abs(b - 14.5) <= 1e-6
    assert np.max(np.abs(p - (r >= 15))) <= 1e-6


# 16385 keys: 5 tiles, so a wave scans several digits; 2^20 keys: 256 tiles, a
# workgroup per CU; 2^20 + 1: one tile more than the CUs, the split passes
@pytest.mark.parametrize("n", [1, 2, 17, 4096, 16384, 16385, 65537, 300_001, 1 << 20, (1 << 20) + 1])
def test_sort_bit_exact(oracle_mod, n):
    rng = np.random.default_rng(100 + n)
    r = rng.standard_normal(n).astype(np.float32)
    if n > 8:
        r[::7] = r[1]            # ties
        r[3] = -0.0
        r[5] = 0.0
        r[6] = np.float32(-1e-40)  # subnormal
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    rc = L.lib().lapsum_test_sort(to_dev(r).data_ptr(), n, out.data_ptr(), None)
    assert rc == 0
    got = out.cpu().numpy()
    ref = oracle_mod.sort_keys(r)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_sort_forms_alternate(oracle_mod):
    """Large inputs take the split radix passes (counts, scan, scatter), small
    ones the one-kernel passes (epoch-tagged count and offset words); the split
    passes leave data in the region the one-kernel passes read, which must be
    cleared in between.  Sorts of both kinds, alternating on one workspace, all
    bit-exact."""
    for n in (2_500_001, 300_001, 4_000_000, 65_537):
        r = np.random.default_rng(n).standard_normal(n).astype(np.float32)
        r[::5] = r[2]
        out = torch.empty(n, dtype=torch.float32, device="cuda")
        assert L.lib().lapsum_test_sort(to_dev(r).data_ptr(), n, out.data_ptr(), None) == 0
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), oracle_mod.sort_keys(r).view(np.uint32)), n


@pytest.mark.parametrize("form", [1, 2])
@pytest.mark.parametrize("n", [16385, 300_001, 1 << 20])
def test_sort_form_bit_exact(oracle_mod, n, form):
    """Every form of the multi-workgroup passes gives the same keys: 1 the
    one-kernel passes in their look-back design (what a sort runs while
    another sort holds the device's resident-pass lock), 2 the split passes."""
    rng = np.random.default_rng(300 + n)
    r = rng.standard_normal(n).astype(np.float32)
    r[::9] = r[4]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    assert L.lib().lapsum_test_sort_form(to_dev(r).data_ptr(), n, out.data_ptr(), form, None) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint32), oracle_mod.sort_keys(r).view(np.uint32))
    assert L.lib().lapsum_test_sort_form(to_dev(r).data_ptr(), n, out.data_ptr(), 3, None) != 0


def test_full_path_concurrent_streams():
    """Full-sort solves on two streams at once: at most one of them holds the
    resident-pass lock and the other runs the look-back passes; both must
    give the single-stream result bit for bit, on every repetition."""
    r, g, cfg = workloads.config_inputs("C2")
    rd = to_dev(r)
    opt = L.default_options(path=L.PATH_FULL)
    p_ref, b_ref = L.forward(rd, cfg.k, cfg.t, options=opt)
    torch.cuda.synchronize()
    p_ref, b_ref = p_ref.cpu().numpy(), b_ref.cpu().numpy()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(5):
        outs = []
        for s in streams:
            with torch.cuda.stream(s):
                outs.append(L.forward(rd, cfg.k, cfg.t, options=opt))
        torch.cuda.synchronize()
        for p, b in outs:
            assert np.array_equal(b.cpu().numpy().view(np.uint64), b_ref.view(np.uint64)), rep
            assert np.array_equal(p.cpu().numpy().view(np.uint32), p_ref.view(np.uint32)), rep


@pytest.mark.parametrize("n,dist", [(16385, "normal"), (200_000, "student_t3"), (1_000_000, "normal")])
def test_full_sort_path(oracle_mod, n, dist):
    r = workloads.scores(dist, n, 7 + n)
    g = workloads.upstream(n, 8 + n)
    k, t = 200.0, 0.05
    p, b, st, grad = run(r, k, t, g, path=L.PATH_FULL)
    assert st["path_taken"] == 1 and st["status"] == 0
    b_ref = check_forward(oracle_mod, r, k, t, p, b, label=f"full n={n}")
    check_vjp(oracle_mod, r, g, t, b_ref, grad, label=f"full n={n}")


def test_c2_full_path(oracle_mod):
    r, g, cfg = workloads.config_inputs("C2")
    p, b, st, grad = run(r, cfg.k, cfg.t, g)
    assert st["path_taken"] == 1
    b_ref = check_forward(oracle_mod, r, cfg.k, cfg.t, p, b, label="C2")
    check_vjp(oracle_mod, r, g, cfg.t, b_ref, grad, label="C2")


# ---------------------------------------------------------------------------
# bracketing stages
# ---------------------------------------------------------------------------
def test_sample_matches_oracle(oracle_mod):
    r, _, _ = workloads.config_inputs("C3", 100_000)
    s, t, seed = 12650, 0.01, 0x5EED
    x = torch.empty(s, dtype=torch.float32, device="cuda")
    idx = torch.empty(s, dtype=torch.int64, device="cuda")
    rc = L.lib().lapsum_test_sample(to_dev(r).data_ptr(), r.size, t, seed, s, x.data_ptr(), idx.data_ptr(), None)
    assert rc == 0
    oi, ox = oracle_mod.sample(r, t32(t), seed, s)
    assert np.array_equal(idx.cpu().numpy(), oi), "Philox index stream must be bit-exact"
    gx = x.cpu().numpy()
    ulps = np.abs(gx.view(np.int32).astype(np.int64) - ox.view(np.int32).astype(np.int64))
    assert ulps.max() <= 1, f"noised sample differs by {ulps.max()} ulp"


def test_select_order_statistics():
    rng = np.random.default_rng(5)
    for s in (1, 2, 100, 12650, 40000):
        x = rng.standard_normal(s).astype(np.float32)
        xs = np.sort(x)
        for l, h in ((1, s), (0, s + 1), (max(1, s // 3), max(1, (2 * s) // 3)), (s, s)):
            aL = L._binding.ctypes.c_float()
            aR = L._binding.ctypes.c_float()
            nb = L._binding.ctypes.c_int32()
            rc = L.lib().lapsum_test_select(to_dev(x).data_ptr(), s, l, h, L._binding.ctypes.byref(aL),
                                            L._binding.ctypes.byref(aR), L._binding.ctypes.byref(nb), None)
            assert rc == 0
            eL = -np.inf if l < 1 else xs[l - 1]
            eR = np.inf if h > s else xs[h - 1]
            assert aL.value == eL and aR.value == eR, (s, l, h, aL.value, eL, aR.value, eR)
            assert 1 <= nb.value <= 1024


# Samples built so that the select's three ways to its order statistics all
# run: the window the sample histogram names (keys spread over many 12-bit
# bins), the select's own subsample window (every key in one 12-bit bin, so
# the histogram's window is the whole sample) and the radix select (every key
# in one 16-bit bin too), plus ties.  Each must give x_(l) and x_(h) exactly.
SELECT_SAMPLES = {
    "spread": lambda rng, s: rng.standard_normal(s) * 3.0,
    "one_12bit_bin": lambda rng, s: 1.0 + rng.uniform(0.0, 0.1249, s),
    "one_16bit_bin": lambda rng, s: 1.0 + rng.uniform(0.0, 0.0078, s),
    "ties": lambda rng, s: rng.integers(0, 7, s).astype(np.float64),
    "negative_cluster": lambda rng, s: -2.0 - rng.exponential(0.05, s),
}


@pytest.mark.parametrize("kind", sorted(SELECT_SAMPLES))
@pytest.mark.parametrize("s", [3000, 12650, 40000])
def test_select_window_forms(kind, s):
    rng = np.random.default_rng(1000 * sorted(SELECT_SAMPLES).index(kind) + s)
    x = SELECT_SAMPLES[kind](rng, s).astype(np.float32)
    xs = np.sort(x)
    for l, h in ((s - 40, s - 2), (s // 2, s // 2 + 30), (5, 60), (1, 1), (s, s), (0, 7), (s - 7, s + 1)):
        aL = L._binding.ctypes.c_float()
        aR = L._binding.ctypes.c_float()
        nb = L._binding.ctypes.c_int32()
        rc = L.lib().lapsum_test_select(to_dev(x).data_ptr(), s, l, h, L._binding.ctypes.byref(aL),
                                        L._binding.ctypes.byref(aR), L._binding.ctypes.byref(nb), None)
        assert rc == 0
        eL = -np.inf if l < 1 else xs[l - 1]
        eR = np.inf if h > s else xs[h - 1]
        assert aL.value == eL and aR.value == eR, (kind, s, l, h, aL.value, eL, aR.value, eR)
        assert 1 <= nb.value <= 1024


@pytest.mark.parametrize("aL,aR", [(1.0, 2.5), (-np.inf, -1.0), (2.0, np.inf), (0.3, 0.3001), (0.5, 0.5)])
def test_filter_band_bit_exact(oracle_mod, aL, aR):
    r, _, _ = workloads.config_inputs("C3", 400_003)
    t = 0.01
    ctypes = L._binding.ctypes
    counts = (ctypes.c_int64 * 3)()
    sums = (ctypes.c_double * 4)()
    msize = ctypes.c_int64()
    nbk = ctypes.c_int32()
    sizes = (ctypes.c_int64 * 1024)()
    cap = 400_003
    band = torch.empty(cap, dtype=torch.float32, device="cuda")
    rc = L.lib().lapsum_test_filter(to_dev(r).data_ptr(), r.size, t, float(np.float32(aL)), float(np.float32(aR)),
                                    counts, sums, band.data_ptr(), cap, ctypes.byref(msize), ctypes.byref(nbk),
                                    sizes, None)
    assert rc == 0
    ref = oracle_mod.bracket(r, t32(t), float(np.float32(aL)), float(np.float32(aR)))
    assert (counts[0], counts[1], counts[2]) == (ref["below"], ref["band"], ref["above"])
    if msize.value >= 0:
        got = band[: msize.value].cpu().numpy().astype(np.float64)
        # the band as a multiset is bit-exact; inside a bucket the order is free
        assert np.array_equal(np.sort(got), ref["band_values"]), "band must be bit-exact"
        # buckets are value-ordered: every score of a bucket <= every score of a later one
        assert 1 <= nbk.value <= 1024
        szs = [sizes[i] for i in range(nbk.value)]
        assert sum(szs) == msize.value
        prev_max, pos = -np.inf, 0
        for c in szs:
            if c:
                blk = got[pos:pos + c]
                assert blk.min() >= prev_max
                prev_max = blk.max()
                pos += c
    for i, key in enumerate(("S_L", "S_R", "B_L", "B_R")):
        assert abs(sums[i] - ref[key]) <= 1e-6 * max(ref[key], 1e-300) + 1e-300, (key, sums[i], ref[key])


# ---------------------------------------------------------------------------
# bracketing end to end (scaled-down configurations)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name,n", [("C3", 2_000_000), ("C4", 3_000_000), ("C5", 2_000_000)])
def test_bracket_path(oracle_mod, name, n):
    cfg = workloads.CONFIGS[name]
    r = workloads.scores(cfg.dist, n, 1000 + cfg.number, k=cfg.k * n / cfg.n)
    g = workloads.upstream(n, 2000 + cfg.number)
    k = cfg.k * n / cfg.n
    p, b, st, grad = run(r, k, cfg.t, g)
    assert st["status"] == 0
    assert st["path_taken"] in (2, 3)
    b_ref = check_forward(oracle_mod, r, k, cfg.t, p, b, label=name)
    check_vjp(oracle_mod, r, g, cfg.t, b_ref, grad, label=name)
    if st["path_taken"] == 2:
        # certification quantities agree with the oracle's direct sums
        ref = oracle_mod.bracket(r, t32(cfg.t), st["a_L"], st["a_R"], want_band=False)
        assert (st["count_below"], st["band_size"], st["count_above"]) == (ref["below"], ref["band"], ref["above"])
        if np.isfinite(st["a_L"]):
            assert abs(st["g_aL"] - ref["G_aL"]) <= 1e-6 * ref["G_aL"]
        if np.isfinite(st["a_R"]):
            assert abs(st["g_aR"] - ref["G_aR"]) <= 1e-6 * max(ref["G_aR"], 1.0)
        assert st["g_aL"] >= k > st["g_aR"]


def test_forced_fallback_and_widening(oracle_mod):
    r, g, cfg = workloads.config_inputs("C5", 1_500_000)
    k = 15000.0
    p, b, st, grad = run(r, k, cfg.t, g, path=L.PATH_FORCE_FALLBACK)
    assert st["path_taken"] == 3
    b_ref = check_forward(oracle_mod, r, k, cfg.t, p, b, label="forced fallback")
    check_vjp(oracle_mod, r, g, cfg.t, b_ref, grad, label="forced fallback")
    # zero margins: the first bracket has zero width and must be widened
    p, b, st, _ = run(r, k, cfg.t, path=L.PATH_BRACKET, margin_scale=0.0)
    assert st["widenings"] >= 1
    check_forward(oracle_mod, r, k, cfg.t, p, b, b_ref=b_ref, label="widened")
    # tiny buckets: nearly every bucket overflows; their scores are collected
    # by a second pass and the bracket is still solved (no full sort)
    p, b, st, _ = run(r, k, cfg.t, path=L.PATH_BRACKET, bucket_capacity=4)
    assert st["path_taken"] == 2
    check_forward(oracle_mod, r, k, cfg.t, p, b, b_ref=b_ref, label="overflow")


def test_overflow_collection_wide_band(oracle_mod):
    """A band holding most of the scores, with buckets far too small: every
    bucket overflows, and the collection pass's walk queues more band scores
    per wave than its LDS queue holds, so the rest go straight to their slots
    (the queue-overflow path).  Parity with the oracle; no full-sort
    fallback.  At 4M scores each of the pass's 4096 waves walks ~980 band
    scores against a 512-entry queue."""
    n = 4_000_000
    r = np.random.default_rng(91).standard_normal(n).astype(np.float32)
    k, t = float(n // 2), 0.05
    g = workloads.upstream(n, 92)
    p, b, st, grad = run(r, k, t, g, path=L.PATH_BRACKET, margin_scale=400.0, bucket_capacity=16, profile=1)
    assert st["status"] == 0 and st["path_taken"] == 2, st
    assert st["band_size"] > n // 2, st["band_size"]
    assert "heavy_collect" in [nm for nm, _ in st["kernels"]]
    b_ref = check_forward(oracle_mod, r, k, t, p, b, label="wide band, overflowed buckets")
    check_vjp(oracle_mod, r, g, t, b_ref, grad, label="wide band, overflowed buckets")


def test_deterministic(oracle_mod):
    r, _, cfg = workloads.config_inputs("C3", 2_000_000)
    p1, b1, _, _ = run(r, 2000.0, cfg.t)
    p2, b2, _, _ = run(r, 2000.0, cfg.t)
    assert b1 == b2 and np.array_equal(p1.view(np.uint32), p2.view(np.uint32))


# ---------------------------------------------------------------------------
# errors
# ---------------------------------------------------------------------------
def test_invalid_arguments():
    r = torch.zeros(8, device="cuda")
    for k, t in ((0.0, 1.0), (8.0, 1.0), (1.0, 0.0), (1.0, float("nan")), (float("inf"), 1.0)):
        with pytest.raises(L.LapsumError) as e:
            L.forward(r, k, t)
        assert e.value.code == 1


@pytest.mark.parametrize("n,bad", [(1000, np.nan), (2_000_000, np.nan), (2_000_000, np.inf), (50_000, -np.inf)])
def test_nonfinite_scores(n, bad):
    r = workloads.scores("normal", n, 3)
    r[n // 2] = bad
    rd = to_dev(r)
    if n > 1_000_000:
        # the bracketing path waits for its verdict and returns the error itself
        with pytest.raises(L.LapsumError) as e:
            L.forward(rd, 10.0, 0.1)
        assert e.value.code == 2
    else:
        # the full-sort path never blocks: without stats the call returns before
        # the device has looked, and b is NaN; with stats it waits and reports
        p, b = L.forward(rd, 10.0, 0.1)
        assert np.isnan(b.item())
    with pytest.raises(L.LapsumError) as e:
        L.forward(rd, 10.0, 0.1, stats=True)
    assert e.value.code == 2


@pytest.mark.parametrize("bad", [np.nan, -np.inf])
def test_nonfinite_scores_split_sort(bad):
    """Above 2^20 scores the full sort runs its split passes, whose first
    count pass looks for non-finite scores: b is NaN, a call with stats
    reports the error, and a finite call right after on the same workspace
    is not affected (the flag is not left behind)."""
    n = 2_000_000
    r = workloads.scores("normal", n, 5)
    good = r.copy()
    r[n // 3] = bad
    opt = L.default_options(path=L.PATH_FULL)
    p, b = L.forward(to_dev(r), 10.0, 0.1, options=opt)
    assert np.isnan(b.item())
    with pytest.raises(L.LapsumError) as e:
        L.forward(to_dev(r), 10.0, 0.1, options=opt, stats=True)
    assert e.value.code == 2
    p, b, st = L.forward(to_dev(good), 10.0, 0.1, options=opt, stats=True)
    assert st["status"] == 0 and np.isfinite(b.item())
    assert abs(p.double().sum().item() - 10.0) <= 1e-5 * 10.0


@pytest.mark.parametrize("frac", [0.25, 0.5])
def test_bracket_many_splitter_gaps(oracle_mod, frac):
    """Large budgets put hundreds of sample points inside the bracket, hence
    hundreds of splitter gaps: every gap must get its own buckets (no pile-up
    in one bucket, no overflow fallback)."""
    n = 2_000_000
    r = workloads.scores("normal", n, 77)
    g = workloads.upstream(n, 78)
    k = frac * n
    p, b, st, grad = run(r, k, 0.05, g)
    # before every gap had its own buckets, the scores above gap 255 piled
    # into one bucket, overflowed it and forced the full-sort fallback
    assert st["status"] == 0 and st["path_taken"] == 2, st["path_taken"]
    b_ref = check_forward(oracle_mod, r, k, 0.05, p, b, label=f"k={k}")
    check_vjp(oracle_mod, r, g, 0.05, b_ref, grad, label=f"k={k}")


@pytest.mark.parametrize("copies,k", [(20_000, 20_000.0), (60_000, 10_000.0), (60_000, 90_000.0), (3_000, 5_000.0),
                                      (60_000, None), (20_000, None)])
def test_bracket_tie_cluster(oracle_mod, copies, k):
    """A cluster of equal scores near the budget's quantile.  When the bracket
    takes it in, it overflows its bucket; the bracket stays certified (the
    filter's counts and sums are exact), the overflowed bucket's scores are
    collected by a second pass, and when the root lies in a bucket too large
    for LDS that bucket alone is sorted with the multi-workgroup sort.  k=None
    puts the root inside the cluster (k = #above + copies/2), which forces
    both.  Never a full-sort fallback."""
    n = 2_000_000
    rng = np.random.default_rng(copies + int(k or 1))
    r = rng.standard_normal(n).astype(np.float32)
    q = np.sort(r)[n - int(k or 50_000)]
    idx = rng.choice(n, copies, replace=False)
    r[idx] = q
    inside = k is None
    if inside:
        # just under G(q): b lies above q by less than q's fp32 spacing, so the
        # root interval starts at the cluster's last copy
        k = oracle_mod.budget_G(r, t32(0.01), float(q)) - 1e-3
    g = workloads.upstream(n, 79)
    p, b, st, grad = run(r, k, 0.01, g, profile=1)
    assert st["status"] == 0 and st["path_taken"] == 2, st
    names = [nm for nm, _ in st["kernels"]]
    if inside:
        assert "heavy_collect" in names, names
        if copies > 16384:
            info = {key: st[key] for key in ("a_L", "a_R", "band_size", "count_above", "buckets", "b")}
            assert "root_bucket_sort" in names, (names, info, float(q), k)
    b_ref = check_forward(oracle_mod, r, k, 0.01, p, b, label=f"cluster {copies}")
    check_vjp(oracle_mod, r, g, 0.01, b_ref, grad, label=f"cluster {copies}")


@pytest.mark.parametrize("n", [4093, 1_048_576, 1_048_576 + 4097])
def test_vjp_c_formed_in_apply_and_apart(oracle_mod, n):
    """The VJP's reduce leaves one partial per 4096 scores: up to 256 of them
    (n <= 2^20) the apply pass forms c itself, above that a kernel of its own
    does.  Both sides of that switch, and a size with a ragged tail, against
    the oracle; c and sum f from the stats against the oracle's sums."""
    r = workloads.scores("normal", n, 900 + n % 97)
    g = workloads.upstream(n, 901)
    t = 0.05
    b_ref, _ = oracle_mod.solve(r.astype(np.float64), 0.01 * n, t32(t))
    b = torch.tensor([b_ref], dtype=torch.float64, device="cuda")
    grad, st = L.vjp(to_dev(r), to_dev(g), t, b, stats=True)
    check_vjp(oracle_mod, r, g, t, b_ref, grad.cpu().numpy(), label=f"n={n}")
    r64, g64 = r.astype(np.float64), g.astype(np.float64)
    f = 0.5 * np.exp(-np.abs(r64 - b_ref) / t32(t))
    assert abs(st["vjp_c"] - (f * g64).sum() / f.sum()) <= 1e-6 * (np.abs(g64).max() + 1.0)
    assert abs(st["vjp_sum_f"] / f.sum() - 1.0) <= 1e-6
