"""Comparison of the HIP path's outputs with the oracle's, at the tolerances
the method's target states:

  * rotated binary32 values within 1e-5 of the token's max |y|;
  * scale within 1e-6 relative; zero-point within 1e-6 relative to
    max(|zero|, 1);
  * int4 codes bit-exact, except a code whose exact position (y - mn)/s lies
    within 1e-4 of a rounding boundary, which may differ by +-1, on at most
    1e-4 of the elements.

The oracle decides codes in binary32 (the kernel's precision); its scale and
zero-point are the binary64 definition.  Nothing computed by the HIP path is
fed to the oracle: both sides get the same generated inputs.
"""

from __future__ import annotations

import math

import numpy as np

import oracle as O

Y_TOL = 1e-5
SZ_TOL = 1e-6
BOUNDARY = 1e-4
MISMATCH_FRACTION = 1e-4


def expected(x_bits: np.ndarray, d: np.ndarray):
    """Oracle outputs for bf16 rows and sign vector d."""
    y = O.rotate(O.bf16_bits_to_f64(x_bits), d)
    q32, _, _ = O.quant_asym(y, "f32")
    _, s, z = O.quant_asym(y, "f64")
    pos = O.code_position(y, "f32")
    return {"y": y, "q": q32, "scale": s, "zero": z, "pos": pos}


def compare(exp: dict, codes_packed: np.ndarray, scale: np.ndarray, zero: np.ndarray,
            y_gpu: np.ndarray | None = None, label: str = "") -> dict:
    """Assert every tolerance; return statistics."""
    stats = {}
    y = exp["y"]
    if y_gpu is not None:
        ymax = np.abs(y).max(axis=1)
        ymax = np.where(ymax == 0, 1.0, ymax)
        err = np.abs(y_gpu.astype(np.float64) - y).max(axis=1) / ymax
        stats["y_rel_max"] = float(err.max())
        assert np.all(err <= Y_TOL), f"{label}: rotated values off by {err.max():.3e} of max|y|"
    s_err = np.abs(scale.astype(np.float64) - exp["scale"]) / exp["scale"]
    z_err = np.abs(zero.astype(np.float64) - exp["zero"]) / np.maximum(np.abs(exp["zero"]), 1.0)
    stats["scale_rel_max"] = float(s_err.max())
    stats["zero_rel_max"] = float(z_err.max())
    assert np.all(s_err <= SZ_TOL), f"{label}: scale rel err {s_err.max():.3e} at token {int(s_err.argmax())}"
    assert np.all(z_err <= SZ_TOL), f"{label}: zero rel err {z_err.max():.3e} at token {int(z_err.argmax())}"
    q = O.unpack_int4(codes_packed)
    assert q.shape == exp["q"].shape
    diff = q.astype(np.int16) - exp["q"].astype(np.int16)
    bad = diff != 0
    nbad = int(bad.sum())
    stats["code_mismatches"] = nbad
    stats["elements"] = int(q.size)
    if nbad:
        pos = exp["pos"][bad]
        dist = np.abs(pos - np.floor(pos) - 0.5)
        assert np.all(np.abs(diff[bad]) == 1), f"{label}: a code differs by more than 1"
        assert np.all(dist < BOUNDARY), f"{label}: code mismatch {dist.max():.3e} away from a boundary"
        # "at most 1e-4 of the elements", counted in whole elements (rounded up)
        assert nbad <= math.ceil(MISMATCH_FRACTION * q.size), f"{label}: {nbad} mismatches of {q.size}"
    return stats
