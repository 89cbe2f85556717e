"""The GEMM epilogue's GELU (gelu_fast in csrc/moe_internal.h) on the host: the
coefficients in the header are the ones gelu_fit.py computes, and the header's
fp32 evaluation order stays within its stated error of the exact erf GELU."""
from __future__ import annotations

import os
import re

import numpy as np
from scipy.special import ndtr

from combine_softmax_top_amd import gelu_fit

HDR = os.path.join(os.path.dirname(__file__), "..", "combine_softmax_top_amd", "csrc", "moe_internal.h")


def _header_coefficients() -> np.ndarray:
    src = open(HDR).read()
    body = src[src.index("float gelu_fast(float v)"):]
    body = body[: body.index("}")]
    first = re.search(r"float p = ([-+0-9.eE]+)f;", body).group(1)
    rest = re.findall(r"p = fmaf\(p, a, ([-+0-9.eE]+)f\);", body)
    return np.array([float(first)] + [float(x) for x in rest], np.float32)[::-1]  # a^0 .. a^7


def test_header_coefficients_match_the_fit():
    hdr = _header_coefficients()
    fit = gelu_fit.coefficients()
    assert hdr.shape == fit.shape == (8,)
    assert np.allclose(hdr, fit, rtol=2e-7, atol=0.0), (hdr, fit)


def test_fp32_evaluation_error_bounds():
    v = np.linspace(-12.0, 12.0, 480001).astype(np.float32)
    exact = v.astype(np.float64) * ndtr(v.astype(np.float64))
    got = gelu_fit.gelu_fp32(v, _header_coefficients()).astype(np.float64)
    err = np.abs(got - exact)
    assert err.max() <= 5e-7, err.max()
    big = np.abs(exact) > 1e-3
    assert (err[big] / np.abs(exact[big])).max() <= 9e-6
    assert err[np.abs(v) > 6].max() <= 2e-8
    # the special points: gelu(0) = 0 exactly, odd-even identity gelu(v) - gelu(-v) = v
    assert gelu_fit.gelu_fp32(np.zeros(1, np.float32), _header_coefficients())[0] == 0.0
    w = np.linspace(0.0, 6.0, 6001).astype(np.float32)
    hc = _header_coefficients()
    d = gelu_fit.gelu_fp32(w, hc).astype(np.float64) - gelu_fit.gelu_fp32(-w, hc).astype(np.float64)
    assert np.abs(d - w).max() <= 2e-6
