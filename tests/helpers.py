"""Shared test helpers: tensor marshalling and the dense (one-hot einsum) forms of
dispatch and combine used as independent pins of the oracle's index path.

The dense forms follow the MoE training blog, part 3 section 3.5 (dispatch input
= einsum("TEC,TM->ECM", mask, input)) and DeepSpeed PR #8195 section 3 (the
dense [s, e, c] one-hot einsum the index path replaces). They are written with
numpy/torch library calls only and share nothing with the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W


def np_of(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor: bf16 as uint16 bit patterns, fp32 as float32."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32_of(a: np.ndarray) -> np.ndarray:
    """Exact fp32 values of a bf16 (uint16) or fp32 array."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def bf16_bits_of_f32(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 round-to-nearest-even through torch (a library conversion)."""
    return np_of(torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16))


def to_dtype_bits(a32: np.ndarray, dtype: int) -> np.ndarray:
    return a32.astype(np.float32) if dtype == W.DT_F32 else bf16_bits_of_f32(a32)


def onehot_mask(idx: np.ndarray, loc: np.ndarray, E: int, C: int) -> np.ndarray:
    """Per-route one-hot masks [k, S, E, C]: 1 where route (r, s) is kept at slot (e, c)."""
    k, S = idx.shape
    mask = np.zeros((k, S, E, C), np.float32)
    for r in range(k):
        for s in range(S):
            if loc[r, s] < C:
                mask[r, s, idx[r, s], loc[r, s]] = 1.0
    return mask


def dense_dispatch(x32: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """buf[e, c, m] = sum_s mask[s, e, c] * x[s, m] over the union of route masks, fp32."""
    m = mask.sum(axis=0)
    return np.einsum("sec,sm->ecm", m, x32.astype(np.float32))


def dense_combine(y32: np.ndarray, mask: np.ndarray, gates: np.ndarray) -> np.ndarray:
    """Per-route combine: out = sum over r (in route order, from +0) of
    einsum("sec,ecm->sm", gates[r] * mask[r], y) in fp32."""
    k = mask.shape[0]
    out = np.zeros((mask.shape[1], y32.shape[-1]), np.float32)
    for r in range(k):
        cw = mask[r] * gates[r][:, None, None].astype(np.float32)
        out = (out + np.einsum("sec,ecm->sm", cw, y32.astype(np.float32))).astype(np.float32)
    return out
