"""The integer kernels' arithmetic, modelled on the CPU (tests/kernel_model.py),
against the oracle on the workload distributions and on the edge inputs of
tests/edge_inputs.py: the design meets the per-output bound before any
kernel runs it."""
import numpy as np
import pytest

import checks
import edge_inputs
import kernel_model
from block_quantized_decode_q4_amd import synth


@pytest.mark.parametrize("case", edge_inputs.all_cases(), ids=lambda c: c.name)
def test_model_edge_inputs(oracle_mod, case):
    y_ref, bound = oracle_mod.gemv(case.w, case.x, case.n)
    y, _ = kernel_model.gemv(case.w, case.x, case.n)
    checks.assert_y(y, y_ref, bound, case.name, strict_kind=case.strict_kind)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_model_workload_distribution(oracle_mod, seed):
    n, k, m = 48, 4096, 3
    w, x = synth.make_inputs(n, k, m, seed=seed)
    y_ref, bound = oracle_mod.gemv(w, x, n)
    y, dirty = kernel_model.gemv(w, x, n)
    worst = checks.assert_y(y, y_ref, bound, "workload distribution")
    assert worst < 1e-6
    # N(0,1) x: about 0.4 % of sub-blocks hold an element below 2^-14 of
    # their largest |x| that the grid does not carry to 2^-17
    assert sum(dirty) <= 0.03 * m * k // 32


def test_model_certification_is_needed(oracle_mod):
    """Without the exact terms of uncertified elements (x rounded to the
    31-bit grid everywhere) the mixed-magnitude case breaks the bound: the
    check is what carries the guarantee, not the digit count."""
    case = edge_inputs.mixed_subblock(rest="normal")
    y_ref, bound = oracle_mod.gemv(case.w, case.x, case.n)
    rep = kernel_model.XRep(case.x[0])
    assert rep.dirty[0] and rep.dirty.sum() == 1
    # the grid value of every element, as a kernel without the check would use it
    v = np.ldexp(case.x[0].reshape(-1, 32).astype(np.float64), rep.sigma[:, None])
    xg = (np.rint(v) * np.ldexp(1.0, -rep.sigma)[:, None]).reshape(-1)
    wd = oracle_mod.dequant(case.w, case.n, case.k).astype(np.float64)
    err = np.abs(wd @ xg - y_ref[0])
    assert np.any(err > 1e-5 * bound[0])


def test_model_digits_and_grid():
    """xi = sum of the four digits * 256^l, |digit| <= 128, and the grid puts
    each sub-block's largest |x| in [2^29, 2^30)."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(4096) * np.exp2(rng.integers(-140, 120, 4096))).astype(np.float32)
    rep = kernel_model.XRep(x)
    assert np.all(np.abs(rep.digits) <= 128)
    rebuilt = (rep.digits * (256 ** np.arange(4))).sum(axis=-1)
    assert np.array_equal(rebuilt, rep.xi)
    # the grid of each sub-block: its largest |x| (certified or not) lands in
    # [2^29, 2^30); an uncertified element has xi = 0
    assert np.all(rep.xi[~rep.cert] == 0)
    v = np.ldexp(np.abs(rep.x).astype(np.float64), rep.sigma[:, None])
    top = np.rint(np.where(np.isfinite(v), v, 0)).max(axis=1)
    nz = top > 0
    assert np.all((top[nz] >= 2 ** 29 - 1) & (top[nz] <= 2 ** 30))
