"""Coefficients of the GEMM epilogue's GELU (``gelu_fast`` in csrc/moe_internal.h).

P(a) ~ log2 Phi(-a) on [0, 6]: a degree-7 least-squares fit on a Chebyshev basis
(200001 equispaced points), expanded in powers of a and rounded to fp32. Prints
the coefficients from a^7 down to a^0 (the kernel's Horner order) and the error
of the fp32 evaluation over [-12, 12].
"""
import numpy as np
from numpy.polynomial import chebyshev as ch
from scipy.special import log_ndtr, ndtr


def coefficients(deg: int = 7, amax: float = 6.0) -> np.ndarray:
    a = np.linspace(0.0, amax, 200001)
    f = log_ndtr(-a) / np.log(2.0)
    c = ch.chebfit(a * (2.0 / amax) - 1.0, f, deg)
    p = np.polynomial.Polynomial(ch.cheb2poly(c))(np.polynomial.Polynomial([-1.0, 2.0 / amax]))
    return p.coef.astype(np.float32)  # a^0 .. a^deg


def gelu_fp32(v: np.ndarray, coef: np.ndarray, amax: float = 6.0) -> np.ndarray:
    v = v.astype(np.float32)
    a = np.minimum(np.abs(v), np.float32(amax))
    p = np.full_like(a, coef[-1])
    for c in coef[-2::-1]:
        p = (p * a + c).astype(np.float32)
    vq = (v * np.exp2(p)).astype(np.float32)
    return np.where(v >= 0, v - vq, vq).astype(np.float32)


if __name__ == "__main__":
    coef = coefficients()
    for c in coef[::-1]:
        print(f"{float(c):.7e}f")
    v = np.linspace(-12.0, 12.0, 2000001).astype(np.float32)
    exact = v.astype(np.float64) * ndtr(v.astype(np.float64))
    err = np.abs(gelu_fp32(v, coef) - exact)
    big = np.abs(exact) > 1e-3
    print("max abs error", err.max(), "max rel error where |gelu| > 1e-3", (err[big] / np.abs(exact[big])).max())
