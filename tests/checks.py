"""The acceptance rule for y, shared by the CPU-model tests and the GPU tests.

y (f32, from a kernel or a model of one) against the oracle's y_ref and
bound = sum |w||x| (both f64):
  * where y_ref is finite: |y - y_ref| <= 1e-5 * bound (a zero bound demands
    y = +-0).  NaN or an infinity in y fails, except an infinity of y_ref's
    sign when a value within the tolerance of y_ref rounds to it in f32
    (the exact result overflows f32);
  * where y_ref is NaN or +-inf: y must be NaN or +-inf too; with
    strict_kind, exactly the same (NaN for NaN, the same signed infinity).
"""
from __future__ import annotations

import numpy as np

TOL = 1e-5
# smallest magnitude that rounds to infinity in f32 (round to nearest even)
F32_OVERFLOW = 2.0 ** 128 - 2.0 ** 103


def y_violations(y, y_ref, bound, strict_kind=True):
    """Boolean mask of outputs that break the rule, and the worst
    |y - y_ref| / bound over the finite ones."""
    y = np.asarray(y)
    y_ref = np.asarray(y_ref, np.float64)
    bound = np.asarray(bound, np.float64)
    assert y.shape == y_ref.shape == bound.shape
    yd = y.astype(np.float64)
    ref_fin = np.isfinite(y_ref)
    y_fin = np.isfinite(yd)
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.abs(yd - y_ref)
        tol = TOL * bound
        ok_fin = y_fin & (err <= tol)
        ok_ovf = (~y_fin & ~np.isnan(yd) & (np.sign(yd) == np.sign(y_ref))
                  & (np.abs(y_ref) + tol >= F32_OVERFLOW))
        if strict_kind:
            same = (np.isnan(yd) & np.isnan(y_ref)) | (yd == y_ref)
        else:
            same = ~y_fin
        ok = np.where(ref_fin, ok_fin | ok_ovf, same)
        ratio = np.where(ref_fin & y_fin & (bound > 0), err / np.where(bound > 0, bound, 1.0), 0.0)
    return ~ok, float(ratio.max()) if ratio.size else 0.0


def assert_y(y, y_ref, bound, what, strict_kind=True):
    bad, worst = y_violations(y, y_ref, bound, strict_kind)
    if np.any(bad):
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError("%s: %d outputs break the rule, first %s: y=%r ref=%r bound=%r"
                             % (what, int(bad.sum()), i, np.asarray(y)[i], np.asarray(y_ref)[i],
                                np.asarray(bound)[i]))
    return worst
