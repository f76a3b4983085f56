"""Python view of the CPU fp64 oracle for the exact-budget LapSum operator.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
package never does.  It shares no code with the HIP library.

Every function takes scores as fp64 (fp32 scores are promoted exactly) and
returns fp64 results.  The definitions follow the Fast LapSum paper as
summarised on gist.science (section 2.1 for the operator and its VJP,
section 2.2 for the bracket bookkeeping) -- see ``lapsum_oracle.c``.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u32p = ctypes.POINTER(ctypes.c_uint32)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build_oracle
        build_oracle.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_get_threads.restype = ctypes.c_int
    lib.oracle_budget_G.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_double]
    lib.oracle_budget_G.restype = ctypes.c_double
    lib.oracle_budget_excess.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_double, ctypes.c_double]
    lib.oracle_budget_excess.restype = ctypes.c_double
    lib.oracle_solve.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_double, _dp,
                                 ctypes.POINTER(ctypes.c_int)]
    lib.oracle_solve.restype = ctypes.c_int
    lib.oracle_probs.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_double, _dp]
    lib.oracle_probs.restype = ctypes.c_double
    lib.oracle_vjp.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_double, ctypes.c_double, _dp, _dp, _dp]
    lib.oracle_vjp.restype = None
    lib.oracle_vjp_kt.argtypes = [_dp, _dp, ctypes.c_int64, ctypes.c_double, ctypes.c_double, _dp, _dp]
    lib.oracle_vjp_kt.restype = None
    lib.oracle_order_stats.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, _dp, _dp]
    lib.oracle_order_stats.restype = ctypes.c_int
    lib.oracle_hard_topk.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, _dp, _dp]
    lib.oracle_hard_topk.restype = ctypes.c_int64
    lib.oracle_dftopk.argtypes = [_dp, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, _dp, _dp]
    lib.oracle_dftopk.restype = ctypes.c_double
    lib.oracle_bracket.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                   _i64p, _dp, _dp, ctypes.c_int64]
    lib.oracle_bracket.restype = ctypes.c_int64
    lib.oracle_sort_keys.argtypes = [_fp, ctypes.c_int64, _fp]
    lib.oracle_sort_keys.restype = None
    lib.oracle_philox4x32_10.argtypes = [_u32p, _u32p, _u32p]
    lib.oracle_philox4x32_10.restype = None
    lib.oracle_sample.argtypes = [_dp, ctypes.c_int64, ctypes.c_double, ctypes.c_uint64, ctypes.c_int64,
                                  _i64p, _fp]
    lib.oracle_sample.restype = None
    lib.oracle_binomial_bounds.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_double, _i64p, _i64p]
    lib.oracle_binomial_bounds.restype = None
    lib.oracle_binomial_miss.argtypes = [ctypes.c_int64, ctypes.c_double, ctypes.c_int64, ctypes.c_int64]
    lib.oracle_binomial_miss.restype = ctypes.c_double
    _lib = lib
    return lib


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a, typ):
    return a.ctypes.data_as(typ)


def set_threads(nthreads: int) -> None:
    """Threads used by the chunked sums (0 = OpenMP default).  Results do
    not depend on it: chunks are fixed and combined in order."""
    _load().oracle_set_threads(int(nthreads))


def get_threads() -> int:
    return int(_load().oracle_get_threads())


def budget_G(r, t: float, b: float) -> float:
    """G(b) = sum_i F((r_i - b)/t), F the scale-1 Laplace CDF."""
    r = _f64(r)
    return float(_load().oracle_budget_G(_ptr(r, _dp), r.size, float(t), float(b)))


def budget_excess(r, t: float, b: float, k: float) -> float:
    """G(b) - k with the integer part of every F counted exactly."""
    r = _f64(r)
    return float(_load().oracle_budget_excess(_ptr(r, _dp), r.size, float(t), float(b), float(k)))


def solve(r, k: float, t: float):
    """Threshold b with G(b) = k, by bisection to fp64 exhaustion.
    Returns (b, iterations)."""
    r = _f64(r)
    b = ctypes.c_double(0.0)
    it = ctypes.c_int(0)
    rc = _load().oracle_solve(_ptr(r, _dp), r.size, float(k), float(t), ctypes.byref(b), ctypes.byref(it))
    if rc != 0:
        raise ValueError("oracle_solve: invalid arguments (need n >= 1, 0 < k < n, t > 0, finite scores)")
    return b.value, it.value


def probs(r, t: float, b: float):
    """p_i = F((r_i - b)/t) in fp64, and sum p."""
    r = _f64(r)
    p = np.empty_like(r)
    s = _load().oracle_probs(_ptr(r, _dp), r.size, float(t), float(b), _ptr(p, _dp))
    return p, float(s)


def vjp(r, g, t: float, b: float):
    """grad_j = (f_j/t)(g_j - c), c = sum g f / sum f.  Returns (grad, c, sum_f)."""
    r = _f64(r)
    g = _f64(g)
    assert r.shape == g.shape
    out = np.empty_like(r)
    c = ctypes.c_double(0.0)
    sf = ctypes.c_double(0.0)
    _load().oracle_vjp(_ptr(r, _dp), _ptr(g, _dp), r.size, float(t), float(b), _ptr(out, _dp),
                       ctypes.byref(c), ctypes.byref(sf))
    return out, c.value, sf.value


def forward(r, k: float, t: float):
    """Full oracle forward: (b, p, sum_p)."""
    b, _ = solve(r, k, t)
    p, s = probs(r, t, b)
    return b, p, s


def vjp_kt(r, g, t: float, b: float):
    """(dL/dk, dL/dt) for L = sum g_i p_i through the threshold b(k, t)."""
    r = _f64(r)
    g = _f64(g)
    dk = ctypes.c_double(0.0)
    dt = ctypes.c_double(0.0)
    _load().oracle_vjp_kt(_ptr(r, _dp), _ptr(g, _dp), r.size, float(t), float(b), ctypes.byref(dk), ctypes.byref(dt))
    return dk.value, dt.value


def order_stats(r, k: int):
    """(k-th largest, (k+1)-th largest) of r; the second is -inf when k = n."""
    r = _f64(r)
    a = ctypes.c_double(0.0)
    b = ctypes.c_double(0.0)
    if _load().oracle_order_stats(_ptr(r, _dp), r.size, int(k), ctypes.byref(a), ctypes.byref(b)) != 0:
        raise ValueError("k must be in [1, n]")
    return a.value, b.value


def hard_topk(r, k: int):
    """(mask, threshold, ones): mask_i = 1 where r_i >= the k-th largest."""
    r = _f64(r)
    m = np.empty(r.size)
    tau = ctypes.c_double(0.0)
    ones = _load().oracle_hard_topk(_ptr(r, _dp), r.size, int(k), _ptr(m, _dp), ctypes.byref(tau))
    if ones < 0:
        raise ValueError("k must be in [1, n]")
    return m, tau.value, int(ones)


def dftopk(r, k: int, t: float):
    """(p, b, sum p) of the DFTopK operator: b = midpoint of the k-th and
    (k+1)-th largest, p_i = F((r_i - b)/t)."""
    r = _f64(r)
    p = np.empty(r.size)
    b = ctypes.c_double(0.0)
    s = _load().oracle_dftopk(_ptr(r, _dp), r.size, int(k), float(t), _ptr(p, _dp), ctypes.byref(b))
    if s != s:
        raise ValueError("k must be in [1, n - 1]")
    return p, b.value, float(s)


def bracket(r, t: float, a_L: float, a_R: float, want_band: bool = True):
    """Bracket bookkeeping for [a_L, a_R).  Returns a dict with counts
    (below, band, above), sums S_L, S_R, B_L, B_R, the direct G(a_L), G(a_R)
    and (optionally) the ascending band values."""
    r = _f64(r)
    counts = np.zeros(3, dtype=np.int64)
    sums = np.zeros(6, dtype=np.float64)
    lib = _load()
    if want_band:
        # first pass for the size, second to fill
        m = lib.oracle_bracket(_ptr(r, _dp), r.size, float(t), float(a_L), float(a_R),
                               _ptr(counts, _i64p), _ptr(sums, _dp), None, 0)
        band = np.empty(max(int(m), 1), dtype=np.float64)
        lib.oracle_bracket(_ptr(r, _dp), r.size, float(t), float(a_L), float(a_R),
                           _ptr(counts, _i64p), _ptr(sums, _dp), _ptr(band, _dp), band.size)
        band = band[:m]
    else:
        lib.oracle_bracket(_ptr(r, _dp), r.size, float(t), float(a_L), float(a_R),
                           _ptr(counts, _i64p), _ptr(sums, _dp), None, 0)
        band = None
    return {
        "below": int(counts[0]), "band": int(counts[1]), "above": int(counts[2]),
        "S_L": float(sums[0]), "S_R": float(sums[1]), "B_L": float(sums[2]), "B_R": float(sums[3]),
        "G_aL": float(sums[4]), "G_aR": float(sums[5]), "band_values": band,
    }


def sort_keys(r):
    """Ascending fp32 keys with -0.0 read as +0.0 (qsort)."""
    r = np.ascontiguousarray(np.asarray(r, dtype=np.float32))
    out = np.empty_like(r)
    _load().oracle_sort_keys(_ptr(r, _fp), r.size, _ptr(out, _fp))
    return out


def philox4x32_10(ctr, key):
    """Philox4x32-10 block function (Salmon et al., SC'11)."""
    c = np.ascontiguousarray(np.asarray(ctr, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    assert c.size == 4 and k.size == 2
    out = np.zeros(4, dtype=np.uint32)
    _load().oracle_philox4x32_10(_ptr(c, _u32p), _ptr(k, _u32p), _ptr(out, _u32p))
    return out


def sample(r, t: float, seed: int, s: int):
    """The kernel-noised sample: (indices int64[s], x fp32[s])."""
    r = _f64(r)
    idx = np.empty(s, dtype=np.int64)
    x = np.empty(s, dtype=np.float32)
    _load().oracle_sample(_ptr(r, _dp), r.size, float(t), ctypes.c_uint64(seed & (2**64 - 1)), int(s),
                          _ptr(idx, _i64p), _ptr(x, _fp))
    return idx, x


def binomial_bounds(s: int, q: float, delta: float):
    """Order-statistic ranks (l, h) for Y ~ Bin(s, q): l = 0 means -inf,
    h = s + 1 means +inf."""
    l = ctypes.c_int64(0)
    h = ctypes.c_int64(0)
    _load().oracle_binomial_bounds(int(s), float(q), float(delta), ctypes.byref(l), ctypes.byref(h))
    return l.value, h.value


def binomial_miss(s: int, q: float, l: int, h: int) -> float:
    """P(Y <= l-1) + P(Y >= h) for Y ~ Bin(s, q)."""
    return float(_load().oracle_binomial_miss(int(s), float(q), int(l), int(h)))
