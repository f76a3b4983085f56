"""GPU parity at the full sizes of the bracketing workloads.

Workloads: C3 (10^7 Student-t), C4 (10^8 mixture), and C5 (10^7 with a
cluster of 10^5 tied scores at the quantile); C5 and C4 also forced onto the
full-sort fallback, and C4 with the certification as a pass of its own.  Each runs in the launch configuration bench.py times:
default options, inputs resident on the device, one stream.

The oracle solves each whole input in fp64 in a few seconds on the host's
cores, so every output element is compared, not a sample.  Where the bracket
was certified, its bookkeeping (counts, and G at both ends) is compared with
the oracle's direct sums over all n.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_helpers import check_forward, check_vjp, t32, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

L = pytest.importorskip("differentiable_exact_budget_amd")

CASES = [("C3", None), ("C4", None), ("C5", None), ("C5", "fallback"), ("C4", "fallback"), ("C4", "cert")]


@pytest.mark.parametrize("name,mode", CASES,
                         ids=["C3", "C4", "C5", "C5-forced-fallback", "C4-forced-fallback", "C4-certification-pass"])
def test_full_size(oracle_mod, name, mode):
    print(f"\nfull-size {name} {mode or 'auto'}", flush=True)
    r, g, cfg = workloads.config_inputs(name)
    rd, gd = to_dev(r), to_dev(g)
    if mode == "fallback":
        opts = L.default_options(path=L.PATH_FORCE_FALLBACK)
    elif mode == "cert":
        opts = L.default_options(cert_mode=1)
    else:
        opts = None
    p, b, st = L.forward(rd, cfg.k, cfg.t, options=opts, stats=True)
    grad = L.vjp(rd, gd, cfg.t, b)
    torch.cuda.synchronize()
    p_h, b_h, grad_h = p.cpu().numpy(), float(b.cpu().item()), grad.cpu().numpy()
    del rd, gd, p, grad
    torch.cuda.empty_cache()

    assert st["status"] == 0
    if mode == "fallback":
        assert st["path_taken"] == 3
    else:
        assert st["path_taken"] in (2, 3)
    if name == "C4" and mode in (None, "cert"):
        assert st["path_taken"] == 2 and st["certified"] == 1 and st["band_size"] > 0

    b_ref = check_forward(oracle_mod, r, cfg.k, cfg.t, p_h, b_h, label=name)
    check_vjp(oracle_mod, r, g, cfg.t, b_ref, grad_h, label=name)

    if st["path_taken"] == 2:
        ref = oracle_mod.bracket(r, t32(cfg.t), st["a_L"], st["a_R"], want_band=False)
        assert (st["count_below"], st["band_size"], st["count_above"]) == (ref["below"], ref["band"], ref["above"])
        if np.isfinite(st["a_L"]):
            assert abs(st["g_aL"] - ref["G_aL"]) <= 1e-6 * ref["G_aL"]
            assert ref["G_aL"] >= cfg.k
        if np.isfinite(st["a_R"]):
            assert abs(st["g_aR"] - ref["G_aR"]) <= 1e-6 * max(ref["G_aR"], 1.0)
            assert ref["G_aR"] < cfg.k
        if mode == "cert":  # the direct pass's sums against the oracle's
            assert abs(st["g_aL_direct"] - ref["G_aL"]) <= 1e-6 * ref["G_aL"]
            assert abs(st["g_aR_direct"] - ref["G_aR"]) <= 1e-6 * max(ref["G_aR"], 1.0)


def test_full_size_order_statistics(oracle_mod):
    """Hard top-k and DFTopK on the 10^8-score mixture, k = 10^5, in the launch
    configuration bench.py times."""
    print("\nfull-size C4 order statistics", flush=True)
    r, _, cfg = workloads.config_inputs("C4")
    rd = to_dev(r)
    k = int(cfg.k)
    mask, tau, st = L.hard_topk(rd, k, stats=True)
    p, b = L.dftopk(rd, k, cfg.t)
    torch.cuda.synchronize()
    assert st["status"] == 0 and st["path_taken"] == 2
    got = tau.cpu().numpy()
    m = mask.cpu().numpy()
    ph = p.cpu().numpy()
    bg = float(b.item())
    del rd, mask, p
    torch.cuda.empty_cache()
    r64 = r.astype(np.float64)
    mask_ref, tau_ref, _ = oracle_mod.hard_topk(r64, k)
    assert got[0] == tau_ref
    assert np.array_equal(m.astype(np.float64), mask_ref)
    p_ref, b_ref, s_ref = oracle_mod.dftopk(r64, k, t32(cfg.t))
    assert bg == b_ref and got[1] == 2.0 * b_ref - got[0]
    assert np.max(np.abs(ph.astype(np.float64) - p_ref)) <= 2e-6
    assert abs(float(ph.astype(np.float64).sum()) - s_ref) <= 1e-5 * k


def test_full_size_sort_bit_exact(oracle_mod):
    """The full sort at 10^8 keys (the C4 input): the radix sort the
    fallback runs, bit for bit against the oracle's sort."""
    print("\nfull-size sort of the C4 input", flush=True)
    r, _, _ = workloads.config_inputs("C4")
    rd = to_dev(r)
    out = torch.empty_like(rd)
    assert L.lib().lapsum_test_sort(rd.data_ptr(), r.size, out.data_ptr(), None) == 0
    got = out.cpu().numpy()
    del rd, out
    torch.cuda.empty_cache()
    ref = oracle_mod.sort_keys(r)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
