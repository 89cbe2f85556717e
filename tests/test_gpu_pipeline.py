"""GPU checks of capacity-dimension pipelining: the expert FFN on slot windows of every
expert's capacity, and the pipelined layer forward (chunks on several streams), which
must give the fused forward's results bit for bit (same kernels, same per-element
summation order; only the split of the tile walk differs), and the oracle's within
tolerance."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import check_close, decode_extra, host, inputs_np, shape_of

pytestmark = pytest.mark.gpu

PW = [
    W.Workload("pipe_S1000_M256_E8_k2_H384", S=1000, M=256, E=8, k=2, H=384, capacity_factor=1.25),
    W.Workload("pipe_gate_S600_M1088_E4_k2_H1152", S=600, M=1088, E=4, k=2, H=1152, capacity_factor=1.0,
               logits="gate"),
    W.Workload("pipe_drops_S777_M128_E16_k3_H256", S=777, M=128, E=16, k=3, H=256, capacity_factor=-0.5,
               logits="zipf"),
]


@pytest.mark.parametrize("w", PW, ids=lambda w: w.name)
def test_ffn_windows_partition_the_ffn(w):
    import combine_softmax_top_amd as moe
    print(f"[ffn windows] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    b = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                          Wg=d.get("Wg"))
    torch.cuda.synchronize()
    C = int(b["capacity"].item())
    fill = host(b["fill"])
    rows = np.concatenate([e * C + np.arange(f) for e, f in enumerate(fill)]).astype(np.int64)
    ridx = torch.from_numpy(rows).cuda()
    y_ref = host(b["y"][ridx])
    for parts in (2, 3, 7):
        y2 = torch.zeros_like(b["y"])
        h2 = torch.zeros_like(b["h"])
        for a, e_ in moe.pipeline_windows(s, parts):
            moe.moe_expert_ffn_window(s, b["buf"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), b["fill"],
                                      b["capacity"], a, e_, None, h2, y2)
        torch.cuda.synchronize()
        assert np.array_equal(host(y2[ridx]).view(np.uint16), y_ref.view(np.uint16)), f"{parts} windows"
    # an empty window writes nothing; a window past the capacity neither
    y3 = torch.zeros_like(b["y"])
    moe.moe_expert_ffn_window(s, b["buf"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), b["fill"], b["capacity"],
                              5, 5, None, torch.zeros_like(b["h"]), y3)
    moe.moe_expert_ffn_window(s, b["buf"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), b["fill"], b["capacity"],
                              C + 3, C + 50, None, torch.zeros_like(b["h"]), y3)
    torch.cuda.synchronize()
    assert (host(y3).view(np.uint16) == 0).all()


@pytest.mark.parametrize("chunks,nstreams", [(1, 1), (2, 2), (3, 2), (4, 4), (8, 2)])
@pytest.mark.parametrize("w", PW, ids=lambda w: w.name)
def test_pipelined_forward_equals_fused(w, chunks, nstreams):
    import combine_softmax_top_amd as moe
    print(f"[pipelined forward] {w.name} chunks={chunks} streams={nstreams}", flush=True)
    inp = W.make_inputs(w, seed=0)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    ref = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                            Wg=d.get("Wg"))
    streams = [torch.cuda.Stream() for _ in range(nstreams)]
    events = [torch.cuda.Event() for _ in range(nstreams + 1)]
    for _ in range(2):  # twice: the buffers of the first call are overwritten in place
        b = moe.layer_forward_pipelined(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), chunks, streams,
                                        events, logits=d.get("logits"), Wg=d.get("Wg"))
    torch.cuda.synchronize()
    assert np.array_equal(host(b["out"]).view(np.uint16), host(ref["out"]).view(np.uint16))
    ni = inputs_np(inp)
    fw = oracle.layer_forward(ni, w.k, w.capacity_factor, w.act, w.dtype)
    rows = fw["rows"]
    check_close(host(b["out"]), fw["out"], w.dtype, "out",
                extra=decode_extra(fw["route"], rows, host(b["y"])[rows], fw["y"][rows]))
