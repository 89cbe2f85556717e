"""Helpers of the GPU parity tests: moving arrays between numpy (oracle side) and
torch device tensors (HIP side), running the library's entry points, and the
tolerance rules.

Tolerances: routing indices, locations, needed, fill, C, slot map and the
encode buffer are compared bit for bit; gates within one fp32 ulp (both sides
compute the softmax in fp64 and round once; only the fp64 summation order
differs); decode given the same expert output bit for bit. Everything
downstream of a GEMM is compared in fp32 with max |got - want| <= 1e-4 for fp32
data, or max |got - want| <= 2e-2 RMS(want) for bf16 data, where each bf16
element may also differ by one bf16 ulp of its value (see check_close).
"""
from __future__ import annotations

import math
from typing import Dict

import numpy as np
import torch

import workloads as W
from tests.helpers import f32_of, np_of

TOL_F32_ABS = 1e-4
TOL_BF16_REL_RMS = 2e-2


def dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """numpy -> device tensor (uint16 arrays become bf16 bit patterns)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(a).to(device)


def host(t: torch.Tensor) -> np.ndarray:
    return np_of(t)


def inputs_np(inp: Dict[str, torch.Tensor]) -> Dict[str, np.ndarray]:
    return {k: np_of(v) for k, v in inp.items()}


def check_close(got: np.ndarray, want: np.ndarray, dtype: int, what: str, mag: np.ndarray = None,
                extra: np.ndarray = None) -> float:
    """The tolerance rule; returns the largest error / bound ratio (<= 1 passes).

    fp32 data: max |got - want| <= 1e-4.
    bf16 data: |got - want| <= 2e-2 RMS(want) + 2^-7 mag elementwise, where mag
    defaults to |want|. The first term is the max-abs-versus-RMS rule; the second
    is one bf16 ulp of the element (an ulp is at most 2^-7 of the value): both
    sides round their own fp32/fp64 result to bf16, and whenever the two
    unrounded values straddle a rounding boundary the stored values differ by
    one ulp, which at values several times the RMS exceeds 2e-2 RMS by itself.
    Sums of separately rounded bf16 terms (dx) pass mag = |want| + sum |term|.
    extra (elementwise, either dtype) widens the bound by the propagated effect of
    an upstream input that the two sides computed within tolerance of each other.
    """
    g = f32_of(got).astype(np.float64)
    w = f32_of(want).astype(np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    if g.size == 0:
        return 0.0
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    d = np.abs(g - w)
    diff = d.max()
    if dtype == W.DT_F32:
        if extra is not None:
            d = np.maximum(d - np.asarray(extra, np.float64), 0.0)
            diff = d.max()
        assert diff <= TOL_F32_ABS, f"{what}: max abs err {diff:.3e} > {TOL_F32_ABS}"
        return float(diff / TOL_F32_ABS)
    rms = math.sqrt((w ** 2).mean())
    if mag is None:
        mag = np.abs(w)
    bound = TOL_BF16_REL_RMS * rms + 2.0 ** -7 * np.asarray(mag, np.float64)
    if extra is not None:
        bound = bound + np.asarray(extra, np.float64)
    ratio = d / np.maximum(bound, 1e-300)
    i = np.unravel_index(np.argmax(ratio), d.shape)
    assert ratio[i] <= 1.0, (f"{what}: |err| {d[i]:.3e} exceeds 2e-2*rms + 2^-7*mag = {bound[i]:.3e} at {i} "
                             f"(got {g[i]:.6e} want {w[i]:.6e}, rms {rms:.3e}; max err/rms {diff / rms:.3e})")
    return float(ratio[i])


def check_gates(got: np.ndarray, want: np.ndarray, what="gates"):
    ulp = np.spacing(np.abs(want).astype(np.float32))
    bad = np.abs(got.astype(np.float64) - want.astype(np.float64)) > ulp
    assert not bad.any(), f"{what}: {bad.sum()} values differ by more than one ulp"


def shape_of(w: W.Workload):
    import combine_softmax_top_amd as moe
    return moe.Shape.of(w)


def gpu_route(w: W.Workload, logits: np.ndarray) -> Dict[str, np.ndarray]:
    """moe_route on the given fp32 logits; returns host arrays (slot map cut to E*C)."""
    import combine_softmax_top_amd as moe
    s = shape_of(w)
    b = moe.alloc_forward(s)
    lg = dev(np.ascontiguousarray(logits, dtype=np.float32))
    moe.moe_route(s, lg, b["idx"], b["loc"], b["gates"], b["needed"], b["fill"], b["capacity"], b["slot_route"],
                  b["ws"])
    torch.cuda.synchronize()
    C = int(b["capacity"].item())
    return dict(idx=host(b["idx"]), loc=host(b["loc"]), gates=host(b["gates"]), needed=host(b["needed"]),
                fill=host(b["fill"]), C=C, slot_route=host(b["slot_route"][: w.E * C]))


def compare_route(g: Dict, o: Dict, E: int):
    assert g["C"] == o["C"], (g["C"], o["C"])
    for k in ("idx", "loc", "needed", "fill"):
        assert np.array_equal(g[k], o[k]), k
    check_gates(g["gates"], o["gates"])
    # slot map: rows below fill are defined; compare those
    C = o["C"]
    so = o["slot_route"].reshape(E, C)
    sg = g["slot_route"].reshape(E, C)
    for e in range(E):
        f = int(o["fill"][e])
        assert np.array_equal(sg[e, :f], so[e, :f]), f"slot_route expert {e}"


# ------------------------------------------------------------------ gate backward tolerances
# dlogits, dWg and the auxiliary loss are fp32 on the GPU and fp64 in the oracle. The
# bounds below are 2^-16 of each element's magnitude scale (fp32 carries 2^-24; the
# reductions involved are short or tree-shaped), plus, where the two sides were fed
# upstream values that themselves agree only within tolerance (dgates computed from
# each side's own expert outputs), that difference carried through linearly.

def dlogits_bound(logits, idx, dgates, needed, k, S_total, alpha, dg_err=None):
    """Elementwise bound on |dlogits_gpu - dlogits_oracle| for the tokens given ([n, E])."""
    from scipy.special import softmax
    p = softmax(np.asarray(logits, np.float64), axis=1)
    n, E = p.shape
    g = np.zeros((n, E))
    for r in range(k):
        np.add.at(g, (np.arange(n), idx[r]), np.abs(np.asarray(dgates[r], np.float64)))
    if needed is not None and S_total > 0:
        g += alpha * E * (np.asarray(needed, np.float64) / (k * S_total)) / S_total
    scale = p * (g + (p * g).sum(axis=1, keepdims=True))
    tol = 2.0 ** -16 * scale + 2.0 ** -30 * max(float(scale.max(initial=0.0)), 1e-30)
    if dg_err is not None:
        # |d(dlogits_j)| <= p_j (|d g_j| + sum_i p_i |d g_i|) <= 2 p_j max |d g|
        tol = tol + 2.0 * p * np.asarray(dg_err, np.float64).max(axis=0)[:, None]
    return tol


def check_dlogits(got, want, logits, idx, dgates, needed, k, S_total, alpha, dg_err=None, what="dlogits"):
    tol = dlogits_bound(logits, idx, dgates, needed, k, S_total, alpha, dg_err)
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{what}: non-finite values"
    ratio = d / np.maximum(tol, 1e-300)
    i = np.unravel_index(np.argmax(ratio), d.shape) if d.size else None
    assert d.size == 0 or ratio[i] <= 1.0, (f"{what}: |err| {d[i]:.3e} > bound {tol[i]:.3e} at {i} "
                                            f"(got {got[i]:.6e} want {want[i]:.6e})")
    return tol


def check_dwg(got, want, x, dl, dtype, dl_err=None, what="dWg"):
    """|dWg_gpu - dWg_oracle| <= 2^-16 sum_s |x[s,m]| |dl[s,e]| (+ |x|^T dl_err)."""
    xa = np.abs(f32_of(x).astype(np.float64))
    mag = xa.T @ np.abs(np.asarray(dl, np.float64))
    tol = 2.0 ** -16 * mag + 1e-30
    if dl_err is not None:
        tol = tol + xa.T @ np.asarray(dl_err, np.float64)
    d = np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))
    assert np.isfinite(np.asarray(got, np.float64)).all(), f"{what}: non-finite values"
    if d.size == 0:
        return
    ratio = d / tol
    i = np.unravel_index(np.argmax(ratio), d.shape)
    assert ratio[i] <= 1.0, f"{what}: |err| {d[i]:.3e} > bound {tol[i]:.3e} at {i} (got {got[i]:.6e} want {want[i]:.6e})"


def dgates_err(dg_want, dtype):
    """Elementwise bound of the dgates tolerance rule (check_close) for these values."""
    w = np.asarray(dg_want, np.float64)
    if dtype == W.DT_F32:
        return np.full(w.shape, TOL_F32_ABS)
    rms = math.sqrt((w ** 2).mean()) if w.size else 0.0
    return TOL_BF16_REL_RMS * rms + 2.0 ** -7 * np.abs(w)
