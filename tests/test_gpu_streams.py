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

SW = [
    W.Workload("streams_gate_S1000_M256_E8_k2_H384", S=1000, M=256, E=8, k=2, H=384, capacity_factor=1.25,
               logits="gate"),
    W.Workload("streams_drops_S777_M128_E16_k3_H256", S=777, M=128, E=16, k=3, H=256, capacity_factor=-0.5,
               logits="zipf"),
]

KEYS = ("idx", "loc", "gates", "needed", "fill", "capacity", "buf", "h", "y", "out")


@pytest.mark.parametrize("w", SW, ids=lambda w: w.name)
def test_two_stream_batches_match_one_stream(w):
    import combine_softmax_top_amd as moe
    print(f"[two streams] {w.name}", flush=True)
    s = shape_of(w)
    gate = w.logits == "gate"
    # two different batches (seeds), the same weights
    inps = [{k_: v.cuda() for k_, v in W.make_inputs(w, seed=sd).items()} for sd in (0, 1)]
    for b in inps[1:]:
        for name in ("W1", "b1", "W2", "b2", "Wg"):
            if name in inps[0]:
                b[name] = inps[0][name]

    def run(i, bufs, stream=None):
        d = inps[i]
        moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                          Wg=d.get("Wg"), bufs=bufs, stream=stream)

    ref = []
    for i in range(2):
        b = moe.alloc_forward(s, "cuda", gate_projection=gate)
        run(i, b)
        torch.cuda.synchronize()
        ref.append({k_: host(b[k_]).copy() for k_ in KEYS})
    streams = [torch.cuda.Stream() for _ in range(2)]
    bufs = [moe.alloc_forward(s, "cuda", gate_projection=gate) for _ in range(2)]
    for _ in range(5):  # several rounds, the two streams' launches interleaved
        for i in range(2):
            run(i, bufs[i], streams[i])
    torch.cuda.synchronize()
    for i in range(2):
        C = int(ref[i]["capacity"][0])
        fill = ref[i]["fill"]
        # buf is written for all E * C rows (padding rows are zeros); h and y only for filled rows
        rows = np.concatenate([e * C + np.arange(f) for e, f in enumerate(fill)]).astype(np.int64)
        for k_ in KEYS:
            got, want = host(bufs[i][k_]), ref[i][k_]
            if k_ == "buf":
                got, want = got[: w.E * C], want[: w.E * C]
            elif k_ in ("h", "y"):
                got, want = got[rows], want[rows]
            assert got.tobytes() == want.tobytes(), f"batch {i}: {k_} differs"
