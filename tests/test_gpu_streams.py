"""Concurrent fused forwards on two streams, each with its own buffers (how bench.py runs
consecutive batches): the library keeps no state between calls, so every call must give
the one-stream results bit for bit, whatever the other stream runs at the same time."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import host, shape_of

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16", W.Workload("streams_gate_S1000_M256_E8_k2_H384", S=1000, M=256, E=8, k=2, H=384,
                        capacity_factor=1.25, logits="gate")),
    ("bf16", W.Workload("streams_drops_S777_M128_E16_k3_H256", S=777, M=128, E=16, k=3, H=256,
                        capacity_factor=-0.5, logits="zipf")),
    ("residual", W.Workload("streams_residual_S600_M256_E8_k1_H256", S=600, M=256, E=8, k=1, H=256,
                            capacity_factor=1.0, residual=True)),
    ("mxfp8", W.Workload("streams_mx_S700_M256_E8_k2_H512", S=700, M=256, E=8, k=2, H=512,
                         capacity_factor=1.25, logits="gate")),
]

ROUTE = ("idx", "loc", "gates", "needed", "fill", "capacity")


@pytest.mark.parametrize("kind,w", CASES, ids=lambda c: c if isinstance(c, str) else c.name)
def test_two_stream_batches_match_one_stream(kind, w):
    import combine_softmax_top_amd as moe
    print(f"[two streams] {kind} {w.name}", flush=True)
    s = shape_of(w)
    gate = w.logits == "gate"
    # two different batches (seeds), the same weights
    inps = [{k_: v.cuda() for k_, v in W.make_inputs(w, seed=sd).items()} for sd in (0, 1)]
    shared = ("W1", "b1", "W2", "b2", "Wg", "W1r", "b1r", "W2r", "b2r")
    for name in shared:
        if name in inps[0]:
            inps[1][name] = inps[0][name]
    if kind == "mxfp8":
        W1q = moe.mx_quantize_weights(inps[0]["W1"], moe.MOE_MX_FP8)
        W2q = moe.mx_quantize_weights(inps[0]["W2"], moe.MOE_MX_FP8)

    def alloc():
        if kind == "mxfp8":
            return moe.alloc_forward_mx(s, "cuda", gate_projection=gate)
        return moe.alloc_forward(s, "cuda", gate_projection=gate, residual=kind == "residual")

    def run(i, bufs, stream=None):
        d = inps[i]
        if kind == "mxfp8":
            moe.layer_forward_mx(s, moe.MOE_MX_FP8, d["x"], W1q, d.get("b1"), W2q, d.get("b2"),
                                 logits=d.get("logits"), Wg=d.get("Wg"), bufs=bufs, stream=stream)
            return
        res = {n: d.get(n) for n in ("W1r", "b1r", "W2r", "b2r")} if kind == "residual" else None
        moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                          Wg=d.get("Wg"), bufs=bufs, residual=res, stream=stream)

    def snapshot(b):
        out = {k_: host(b[k_]).copy() for k_ in ROUTE + ("out",)}
        C = int(out["capacity"][0])
        rows = np.concatenate([e * C + np.arange(f) for e, f in enumerate(out["fill"])]).astype(np.int64)
        out["y"] = host(b["y"])[rows].copy()  # y is written for filled rows only
        if kind == "residual":
            out["y_r"] = host(b["y_r"]).copy()
        return out

    ref = []
    for i in range(2):
        b = alloc()
        run(i, b)
        torch.cuda.synchronize()
        ref.append(snapshot(b))
    streams = [torch.cuda.Stream() for _ in range(2)]
    bufs = [alloc() for _ in range(2)]
    for _ in range(5):  # several rounds, the two streams' launches interleaved
        for i in range(2):
            run(i, bufs[i], streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        got = snapshot(bufs[i])
        for k_, want in ref[i].items():
            assert got[k_].tobytes() == want.tobytes(), f"batch {i}: {k_} differs"
