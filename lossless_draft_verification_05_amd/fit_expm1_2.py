"""Coefficients of the polynomial behind expm1_2 in csrc/sv_sample.hip.

expm1_2(x) = 2^x - 1 for x in [-1/2, 0] is evaluated as x * P(x), P of degree
4, whose coefficients are fitted here for the smallest maximum relative error
by Lawson's algorithm (iteratively reweighted least squares on Chebyshev
nodes, each weight multiplied by the current absolute error), then rounded to
fp32. Run: python -m lossless_draft_verification_05_amd.fit_expm1_2
"""
from __future__ import annotations

import math

import numpy as np

LO = -0.5
NCOEF = 5


def fit(lo: float = LO, ncoef: int = NCOEF, npts: int = 20001, iters: int = 80):
    """fp64 coefficients c_0..c_{n-1} of P with x * P(x) ~ 2^x - 1 on [lo, 0),
    and the fit's maximum relative error."""
    ln2 = math.log(2.0)
    x = (np.cos(np.pi * (np.arange(npts) + 0.5) / npts) * 0.5 + 0.5) * lo
    x = x[x < 0]
    f = np.expm1(x * ln2) / x
    w = np.ones_like(x)
    for _ in range(iters):
        A = np.vander(x, ncoef, increasing=True)
        W = np.sqrt(w) / np.abs(f)
        c, *_ = np.linalg.lstsq(A * W[:, None], f * W, rcond=None)
        err = np.abs(A @ c - f) / np.abs(f)
        w = w * err
        w /= w.sum()
    return c, float(err.max())


def coefficients_f32():
    c, _ = fit()
    return [np.float32(v) for v in c]


def fp32_eval(coef, x: np.ndarray) -> np.ndarray:
    """x * P(x) in Horner form, each step an fp32 fused multiply-add (emulated
    exactly in fp64 and rounded), the final product rounded to fp32."""
    x = np.asarray(x, dtype=np.float32)
    p = np.full_like(x, coef[-1])
    for k in range(len(coef) - 2, -1, -1):
        p = (p.astype(np.float64) * x.astype(np.float64) + np.float64(coef[k])).astype(np.float32)
    return (p.astype(np.float64) * x.astype(np.float64)).astype(np.float32)


if __name__ == "__main__":
    c32 = coefficients_f32()
    xs = np.linspace(LO, 0.0, 400001, dtype=np.float32)[:-1]
    ref = np.expm1(xs.astype(np.float64) * math.log(2.0))
    rel = np.abs(fp32_eval(c32, xs) - ref) / np.abs(ref)
    print("coefficients:", ", ".join(f"{float(v):.9e}f" for v in c32))
    print(f"max relative error in fp32: {rel.max():.3e} ({rel.max() / 2.0 ** -24:.2f} ulp)")
