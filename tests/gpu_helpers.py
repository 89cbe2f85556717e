"""Helpers of the GPU parity tests: moving arrays between numpy (oracle side) and
torch device tensors (HIP side), running the library's entry points, and the
tolerance rules.

Tolerances: routing indices, locations, needed, fill, C, slot map and the
encode buffer are compared bit for bit, given the same fp32 logits; gate
logits within an fp32 summation bound (check_logits); gates within one fp32 ulp
(both sides compute the softmax in fp64 and round once; only the fp64 summation
order differs); decode given the same expert output bit for bit. Everything
downstream of a GEMM is compared in fp32 with max |got - want| <= 1e-4 for fp32
data, or max |got - want| <= 2e-2 RMS(want) for bf16 data; a result stored in
bf16 may exceed that only by being the adjacent bf16 value (see check_close).
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


def _bf16_key(a: np.ndarray) -> np.ndarray:
    """Ordered integer key of bf16 bit patterns: adjacent values differ by 1 (+0 and -0 are both 0)."""
    a = a.astype(np.int64)
    return np.where(a & 0x8000, -(a & 0x7FFF), a)


def check_close(got: np.ndarray, want: np.ndarray, dtype: int, what: str, extra: np.ndarray = None) -> float:
    """The tolerance rule; returns the largest error / bound ratio over the elements held to
    the bound (<= 1 passes).

    fp32 data: max |got - want| <= 1e-4.
    bf16 data: max |got - want| <= 2e-2 RMS(want), every element. For results stored in
    bf16 (got and want both bf16 bit patterns) an element may exceed that only if got and
    want are adjacent bf16 values: the two sides round different unrounded values (their
    summation orders differ) and a rounding boundary lay between them. Those elements are
    counted and printed. Results stored in fp32 (weight and bias gradients, dgates) have no
    such exception.
    extra (elementwise, >= 0, either dtype): where an input of this result was computed by
    the two sides within tolerance of each other rather than bit-identically (MX codes of
    h, the expert outputs y feeding decode, dlogits feeding dx's gate share), the bound is
    widened by that input's bound or measured difference carried through linearly: bound =
    rule + extra; a bf16-stored element may then exceed the bound only by the final
    rounding, |got - want| <= extra + one bf16 ulp of the larger stored value.
    """
    g = f32_of(got).astype(np.float64)
    w = f32_of(want).astype(np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    if g.size == 0:
        return 0.0
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    d = np.abs(g - w)
    if dtype == W.DT_F32:
        if extra is not None:
            d = np.maximum(d - np.asarray(extra, np.float64), 0.0)
        diff = d.max()
        assert diff <= TOL_F32_ABS, f"{what}: max abs err {diff:.3e} > {TOL_F32_ABS}"
        return float(diff / TOL_F32_ABS)
    rms = math.sqrt((w ** 2).mean())
    bound = np.full(d.shape, TOL_BF16_REL_RMS * rms)
    if extra is not None:
        bound = bound + np.asarray(extra, np.float64)
    ratio = d / np.maximum(bound, 1e-300)
    over = ratio > 1.0
    nflip = 0
    if over.any() and got.dtype == np.uint16 and want.dtype == np.uint16:
        # one bf16 ulp of the larger of the two stored values: 2^(floor(log2 |v|) - 7)
        mx = np.maximum(np.abs(g), np.abs(w))
        ulp = np.ldexp(1.0, np.frexp(np.where(mx > 0, mx, 1.0))[1] - 8)
        if extra is None:
            flip = over & (np.abs(_bf16_key(got) - _bf16_key(want)) == 1)
        else:
            flip = over & (d <= np.asarray(extra, np.float64) + ulp)
        nflip = int(flip.sum())
        over &= ~flip
        ratio = np.where(flip, 0.0, ratio)
    i = np.unravel_index(np.argmax(ratio), d.shape)
    if nflip:
        print(f"[tolerance] {what}: {nflip} of {d.size} elements beyond 2e-2 RMS are one-ulp bf16 rounding flips",
              flush=True)
    assert not over.any(), (f"{what}: {int(over.sum())} elements exceed 2e-2*rms{' + extra' if extra is not None else ''}"
                            f"; worst |err| {d[i]:.3e} > {bound[i]:.3e} at {i} (got {g[i]:.6e} want {w[i]:.6e}, "
                            f"rms {rms:.3e})")
    return float(ratio[i])


def check_logits(got: np.ndarray, want: np.ndarray, x: np.ndarray, Wg: np.ndarray, what="logits") -> float:
    """GPU gate logits (fp32 accumulation, any summation order) against the oracle's plain
    fp64 sum rounded once. Bound per element: the fp32 summation bound gamma_M sum_m
    |x_m Wg[m, e]| (gamma_n = n u / (1 - n u), u = 2^-24, any order of n - 1 additions)
    plus half an fp32 ulp of the oracle's value and the fp64 sum's own error; and at most
    1e-5 absolute. Returns max |got - want|. Routing is then checked on the GPU's logits."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    if g.size == 0:
        return 0.0
    assert np.isfinite(g).all(), f"{what}: non-finite values"
    M = x.shape[1]
    u = 2.0 ** -24
    gam = M * u / (1.0 - M * u)
    absum = np.abs(f32_of(x).astype(np.float64)) @ np.abs(np.asarray(Wg, np.float64))
    bound = (gam + M * 2.0 ** -53) * absum + 0.5 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    d = np.abs(g - w)
    ratio = d / np.maximum(bound, 1e-300)
    i = np.unravel_index(np.argmax(ratio), d.shape)
    assert ratio[i] <= 1.0, f"{what}: |err| {d[i]:.3e} > fp32 summation bound {bound[i]:.3e} at {i}"
    assert d.max() <= 1e-5, f"{what}: max abs err {d.max():.3e} > 1e-5"
    return float(d.max())


def decode_extra(rt: Dict, rows: np.ndarray, y_got: np.ndarray, y_want: np.ndarray, tokens=None,
                 gated: bool = True) -> np.ndarray:
    """How far the two sides' expert outputs move the decode output: per token (all, or the
    listed ones) and column, the sum over its kept routes of |gate| * |y_got - y_want| at the
    route's buffer row. rows (sorted) lists the buffer rows of y_got / y_want (compact) and
    must hold every row the tokens read. Decode itself is bit-exact given the same y, so an
    end-to-end output differs from the oracle's by this plus its own rounding. gated=False:
    the same for the encode backward (dx sums the token's dbuf rows with unit weights)."""
    k, S = rt["idx"].shape
    C = rt["C"]
    toks = np.arange(S) if tokens is None else np.asarray(tokens, np.int64)
    rows = np.asarray(rows, np.int64)
    dy = np.abs(f32_of(y_got).astype(np.float64) - f32_of(y_want).astype(np.float64))
    out = np.zeros((len(toks), dy.shape[1]))
    for r in range(k):
        kept = rt["loc"][r, toks] < C
        slot = rt["idx"][r, toks].astype(np.int64) * C + rt["loc"][r, toks]
        t = np.nonzero(kept)[0]
        i = np.searchsorted(rows, slot[t])
        assert (i < len(rows)).all() and (rows[np.minimum(i, len(rows) - 1)] == slot[t]).all(), \
            "decode_extra: a token's row is missing"
        wgt = np.abs(rt["gates"][r, toks[t]].astype(np.float64)) if gated else np.ones(len(t))
        out[t] += wgt[:, None] * dy[i]
    return out


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
    """Elementwise bound of the dgates tolerance rule (check_close; dgates are stored in fp32)."""
    w = np.asarray(dg_want, np.float64)
    if dtype == W.DT_F32:
        return np.full(w.shape, TOL_F32_ABS)
    rms = math.sqrt((w ** 2).mean()) if w.size else 0.0
    return np.full(w.shape, TOL_BF16_REL_RMS * rms)
