"""ctypes view of liblapsum.so (the C ABI in include/lapsum.h).

Argument marshalling only: every step of the solver runs in the HIP library.
torch is imported first so that the library binds to the HIP runtime torch
already loaded (one runtime per process, so torch's streams are valid here).
"""
import ctypes
import os

import torch  # noqa: F401  (must precede loading the HIP library)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblapsum.so")

MAX_TIMED = 24

PATH_AUTO, PATH_FULL, PATH_BRACKET, PATH_FORCE_FALLBACK = 0, 1, 2, 3

STATUS = {
    0: "ok",
    1: "invalid argument",
    2: "non-finite score",
    3: "out of device memory",
    4: "HIP runtime error",
    5: "internal consistency check failed",
}


class LapsumError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {STATUS.get(code, 'unknown status')} (status {code})")
        self.code = code


class Options(ctypes.Structure):
    _fields_ = [
        ("path", ctypes.c_int32),
        ("max_widen", ctypes.c_int32),
        ("seed", ctypes.c_uint64),
        ("sample_factor", ctypes.c_double),
        ("delta", ctypes.c_double),
        ("margin_scale", ctypes.c_double),
        ("auto_threshold", ctypes.c_int64),
        ("bucket_capacity", ctypes.c_int32),
        ("profile", ctypes.c_int32),
        ("cert_mode", ctypes.c_int32),
    ]


class Stats(ctypes.Structure):
    _fields_ = [
        ("status", ctypes.c_int32),
        ("path_taken", ctypes.c_int32),
        ("widenings", ctypes.c_int32),
        ("certified", ctypes.c_int32),
        ("count_below", ctypes.c_int64),
        ("band_size", ctypes.c_int64),
        ("count_above", ctypes.c_int64),
        ("sample_size", ctypes.c_int64),
        ("rank_lo", ctypes.c_int64),
        ("rank_hi", ctypes.c_int64),
        ("buckets", ctypes.c_int32),
        ("n_timed", ctypes.c_int32),
        ("a_L", ctypes.c_float),
        ("a_R", ctypes.c_float),
        ("g_aL", ctypes.c_double),
        ("g_aR", ctypes.c_double),
        ("g_aL_direct", ctypes.c_double),
        ("g_aR_direct", ctypes.c_double),
        ("sum_p", ctypes.c_double),
        ("b", ctypes.c_double),
        ("tail_S_L", ctypes.c_double),
        ("tail_S_R", ctypes.c_double),
        ("band_B_L", ctypes.c_double),
        ("band_B_R", ctypes.c_double),
        ("vjp_c", ctypes.c_double),
        ("vjp_sum_f", ctypes.c_double),
        ("kernel_ms", ctypes.c_float * MAX_TIMED),
        ("kernel_name", ctypes.c_char_p * MAX_TIMED),
    ]

    def as_dict(self) -> dict:
        d = {name: getattr(self, name) for name, _ in self._fields_ if name not in ("kernel_ms", "kernel_name")}
        d["kernels"] = [(self.kernel_name[i].decode(), float(self.kernel_ms[i])) for i in range(self.n_timed)]
        return d


_lib = None

EXPORTED = [
    "lapsum_default_options", "lapsum_status_string", "lapsum_forward", "lapsum_forward_ex", "lapsum_vjp",
    "lapsum_vjp_ex", "lapsum_vjp_kt", "lapsum_topk_threshold", "lapsum_hard_topk", "lapsum_dftopk",
    "lapsum_forward_batched", "lapsum_vjp_batched", "lapsum_forward_noalloc",
    "lapsum_release_workspaces", "lapsum_workspace_bytes",
    "lapsum_test_sort", "lapsum_test_sort_form", "lapsum_test_sample", "lapsum_test_select", "lapsum_test_filter",
    "lapsum_test_copy", "lapsum_test_read", "lapsum_test_binomial_ranks", "lapsum_test_inject_internal",
]


def lib():
    """Load liblapsum.so; raise if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                           "(python -c 'import __graft_entry__; __graft_entry__.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, f64, u64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_uint64
    L.lapsum_default_options.argtypes = [ctypes.POINTER(Options)]
    L.lapsum_default_options.restype = None
    L.lapsum_status_string.argtypes = [ctypes.c_int]
    L.lapsum_status_string.restype = ctypes.c_char_p
    L.lapsum_forward.argtypes = [vp, i64, f64, f32, vp, vp, vp]
    L.lapsum_forward.restype = ctypes.c_int
    L.lapsum_forward_ex.argtypes = [vp, i64, f64, f32, vp, vp, ctypes.POINTER(Options), ctypes.POINTER(Stats), vp]
    L.lapsum_forward_ex.restype = ctypes.c_int
    L.lapsum_vjp.argtypes = [vp, vp, vp, i64, f32, vp, vp, vp]
    L.lapsum_vjp.restype = ctypes.c_int
    L.lapsum_vjp_ex.argtypes = [vp, vp, vp, i64, f32, vp, vp, ctypes.POINTER(Options), ctypes.POINTER(Stats), vp]
    L.lapsum_vjp_ex.restype = ctypes.c_int
    L.lapsum_vjp_kt.argtypes = [vp, vp, i64, f32, vp, vp, vp, vp, ctypes.POINTER(Options), ctypes.POINTER(Stats), vp]
    L.lapsum_vjp_kt.restype = ctypes.c_int
    L.lapsum_topk_threshold.argtypes = [vp, i64, i64, vp, ctypes.POINTER(Options), ctypes.POINTER(Stats), vp]
    L.lapsum_topk_threshold.restype = ctypes.c_int
    L.lapsum_hard_topk.argtypes = [vp, i64, i64, vp, vp, ctypes.POINTER(Options), ctypes.POINTER(Stats), vp]
    L.lapsum_hard_topk.restype = ctypes.c_int
    L.lapsum_dftopk.argtypes = [vp, i64, i64, f32, vp, vp, ctypes.POINTER(Options), ctypes.POINTER(Stats), vp]
    L.lapsum_dftopk.restype = ctypes.c_int
    L.lapsum_forward_batched.argtypes = [vp, i64, i64, f64, vp, f32, vp, vp, vp]
    L.lapsum_forward_batched.restype = ctypes.c_int
    L.lapsum_vjp_batched.argtypes = [vp, vp, i64, i64, f32, vp, vp, vp]
    L.lapsum_vjp_batched.restype = ctypes.c_int
    L.lapsum_forward_noalloc.argtypes = [vp, i64, f64, f32, vp, vp, vp]
    L.lapsum_forward_noalloc.restype = ctypes.c_int
    L.lapsum_release_workspaces.argtypes = []
    L.lapsum_release_workspaces.restype = None
    L.lapsum_workspace_bytes.argtypes = [i64, ctypes.POINTER(Options)]
    L.lapsum_workspace_bytes.restype = ctypes.c_size_t
    L.lapsum_test_sort.argtypes = [vp, i64, vp, vp]
    L.lapsum_test_sort.restype = ctypes.c_int
    L.lapsum_test_sort_form.argtypes = [vp, i64, vp, ctypes.c_int32, vp]
    L.lapsum_test_sort_form.restype = ctypes.c_int
    L.lapsum_test_sample.argtypes = [vp, i64, f32, u64, i64, vp, vp, vp]
    L.lapsum_test_sample.restype = ctypes.c_int
    L.lapsum_test_select.argtypes = [vp, i64, i64, i64, ctypes.POINTER(f32), ctypes.POINTER(f32),
                                     ctypes.POINTER(ctypes.c_int32), vp]
    L.lapsum_test_select.restype = ctypes.c_int
    L.lapsum_test_filter.argtypes = [vp, i64, f32, f32, f32, ctypes.POINTER(i64), ctypes.POINTER(f64), vp, i64,
                                     ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(i64), vp]
    L.lapsum_test_filter.restype = ctypes.c_int
    L.lapsum_test_copy.argtypes = [vp, vp, i64, vp]
    L.lapsum_test_copy.restype = ctypes.c_int
    L.lapsum_test_read.argtypes = [vp, i64, vp, vp]
    L.lapsum_test_read.restype = ctypes.c_int
    L.lapsum_test_binomial_ranks.argtypes = [i64, f64, f64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.lapsum_test_binomial_ranks.restype = ctypes.c_int
    L.lapsum_test_inject_internal.argtypes = [vp]
    L.lapsum_test_inject_internal.restype = ctypes.c_int
    _lib = L
    return L


def default_options(**overrides) -> Options:
    o = Options()
    lib().lapsum_default_options(ctypes.byref(o))
    for k, v in overrides.items():
        if not hasattr(o, k):
            raise KeyError(f"unknown option {k!r}")
        setattr(o, k, v)
    return o
