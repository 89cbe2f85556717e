"""The forward that allocates nothing (moe_layer_forward_noalloc) against moe_layer_forward
with its own workspace: the same kernels, so every output must be bit-identical. Two calls
in a row on the one static scratch, the second with a smaller input; and the size limit."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_helpers import host, shape_of

pytestmark = pytest.mark.gpu

OUTS = ("idx", "loc", "gates", "needed", "fill", "capacity", "buf", "h", "y", "out", "logits")


def _run_both(w, seed):
    import combine_softmax_top_amd as moe
    print(f"[no-alloc forward] {w.name} seed={seed}", flush=True)
    s = shape_of(w)
    inp = {k: v.cuda() for k, v in W.make_inputs(w, seed=seed).items()}
    gate = w.logits == "gate"
    ref = moe.alloc_forward(s, training=True, gate_projection=gate)
    moe.layer_forward(s, inp["x"], inp["W1"], inp.get("b1"), inp["W2"], inp.get("b2"), logits=inp.get("logits"),
                      Wg=inp.get("Wg"), bufs=ref)
    got = moe.alloc_forward(s, training=True, gate_projection=gate)
    for k in OUTS:  # poison, so that anything not written shows
        if got.get(k) is not None:
            got[k].fill_(7 if got[k].dtype == torch.int32 else float("nan"))
    moe.moe_layer_forward_noalloc(s, inp["x"], inp.get("logits"), inp.get("Wg"), got["logits"], inp["W1"],
                                  inp.get("b1"), inp["W2"], inp.get("b2"), got["idx"], got["loc"], got["gates"],
                                  got["needed"], got["fill"], got["capacity"], got["slot_route"], got["buf"],
                                  got["pre"], got["h"], got["y"], got["out"])
    torch.cuda.synchronize()
    C = int(ref["capacity"].item())
    fill = host(ref["fill"])
    rows = np.concatenate([e * C + np.arange(f) for e, f in enumerate(fill)]).astype(np.int64)
    for k in OUTS:
        if ref.get(k) is None:
            continue
        a, b = host(ref[k]), host(got[k])
        if k in ("h", "y"):  # rows past fill are not written by either call
            a, b = a[rows], b[rows]
        if k == "buf":
            a, b = a[: w.E * C], b[: w.E * C]
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), k
    sr_a, sr_b = host(ref["slot_route"]), host(got["slot_route"])
    for e, f in enumerate(fill):
        assert np.array_equal(sr_a[e * C: e * C + f], sr_b[e * C: e * C + f]), "slot_route"


def test_noalloc_forward_twice_second_smaller():
    big = W.Workload("noalloc_S3000_E16_k4", S=3000, M=256, E=16, k=4, H=384, capacity_factor=-1.5, logits="zipf")
    small = W.Workload("noalloc_gate_S300_E8_k2", S=300, M=128, E=8, k=2, H=128, capacity_factor=1.25,
                       logits="gate")
    _run_both(big, 0)
    _run_both(small, 1)


def test_noalloc_forward_rejects_shapes_beyond_the_scratch():
    import combine_softmax_top_amd as moe
    # E * k * ceil(S / 64) = 512 * 32 * 65 counts > 1048576 (4 MiB): rejected before anything runs
    s = moe.Shape(S=64 * 65, M=64, E=512, k=32, H=64, capacity_factor=1.0)
    t = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_layer_forward_noalloc(s, t, t, None, None, t, t, t, t, t, t, t, t, t, t, t, t, t, t, t, t)
    assert ei.value.status == moe.MOE_EUNSUPPORTED
    assert "static scratch" in moe.moe_last_error()
