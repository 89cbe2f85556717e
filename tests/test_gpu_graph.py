"""The fused layer captured into a HIP graph (torch.cuda.CUDAGraph): the library enqueues only
kernels on the caller's stream (no allocation, memset or host synchronisation), so a captured
forward, or forward + backward, replays to the eager results bit for bit. Each case captures once
after an eager warm-up, then replays three times; before each replay the outputs are overwritten
with garbage and the token input is changed in place (eager work between replays), and every
replay is compared with an eager run on the same inputs in separate buffers."""
from __future__ import annotations

import pytest
import torch

import workloads as W
from tests.gpu_helpers import shape_of

pytestmark = pytest.mark.gpu

CASES = [
    ("train", W.Workload("graph_train_gate_S700_M256_E8_k2_H384", S=700, M=256, E=8, k=2, H=384,
                         capacity_factor=1.25, logits="gate", backward=True)),
    ("train_residual", W.Workload("graph_train_res_S500_M256_E4_k1_H256", S=500, M=256, E=4, k=1, H=256,
                                  capacity_factor=1.0, residual=True, backward=True)),
    ("forward", W.Workload("graph_fwd_zipf_S1000_M256_E16_k3_H256", S=1000, M=256, E=16, k=3, H=256,
                           capacity_factor=-0.5, logits="zipf")),
    ("blockfp8", W.Workload("graph_blk_S600_M256_E8_k2_H384", S=600, M=256, E=8, k=2, H=384,
                            capacity_factor=1.25, logits="gate")),
    ("mxfp8", W.Workload("graph_mx_S600_M256_E8_k2_H384", S=600, M=256, E=8, k=2, H=384,
                         capacity_factor=1.25, logits="gate")),
    # the NVFP4 weights' quantisation (fill, amax, codes, g) is captured with the forward
    ("nvfp4", W.Workload("graph_nv_S600_M256_E8_k2_H384", S=600, M=256, E=8, k=2, H=384,
                         capacity_factor=1.25, logits="gate")),
]
NV = ("W1c", "W1s", "W1g", "W2c", "W2s", "W2g")


def _outputs(kind, b, g):
    names = {"train": ["logits", "idx", "loc", "gates", "fill", "capacity", "buf", "pre", "h", "y", "out"],
             "train_residual": ["idx", "loc", "gates", "fill", "capacity", "buf", "pre", "h", "y", "pre_r", "h_r",
                                "y_r", "out"],
             "forward": ["idx", "loc", "gates", "fill", "capacity", "buf", "h", "y", "out"],
             "blockfp8": ["logits", "idx", "loc", "fill", "capacity", "buf_codes", "buf_scales", "h_codes",
                          "h_scales", "y", "out"],
             "mxfp8": ["logits", "idx", "loc", "fill", "capacity", "buf_codes", "buf_scales", "h_codes", "h_scales",
                       "y", "out"],
             "nvfp4": ["logits", "idx", "loc", "fill", "capacity", "buf", "h", "y", "out", *NV]}[kind]
    out = {n: b[n] for n in names}
    if g is not None:
        for n in ("dx", "dW1", "db1", "dW2", "db2", "dgates", "dlogits", "dWg", "aux_loss", "dW1r", "dW2r", "db1r",
                  "db2r"):
            if g.get(n) is not None:
                out[n] = g[n]
    return out


@pytest.mark.parametrize("kind,w", CASES, ids=lambda c: c if isinstance(c, str) else c.name)
def test_graph_replays_equal_eager(kind, w):
    import combine_softmax_top_amd as moe
    print(f"[graph] {kind} {w.name}", flush=True)
    s = shape_of(w)
    gate = w.logits == "gate"
    d = {k_: v.cuda() for k_, v in W.make_inputs(w, seed=0, with_dout=w.backward).items()}
    x2 = W.make_inputs(w, seed=1)["x"].cuda()
    res = {n: d.get(n) for n in ("W1r", "b1r", "W2r", "b2r")} if w.residual else None
    if kind == "blockfp8":
        W1q, W2q = moe.blockfp8_quantize_weights(d["W1"]), moe.blockfp8_quantize_weights(d["W2"])
    elif kind == "mxfp8":
        W1q, W2q = moe.mx_quantize_weights(d["W1"], moe.MOE_MX_FP8), moe.mx_quantize_weights(d["W2"], moe.MOE_MX_FP8)

    def alloc():
        if kind == "blockfp8":
            return moe.alloc_forward_blockfp8(s, gate_projection=gate), None
        if kind == "mxfp8":
            return moe.alloc_forward_mx(s, gate_projection=gate), None
        if kind == "nvfp4":
            b = moe.alloc_forward(s, gate_projection=gate)
            for n, (Wt, N, K) in zip(("W1", "W2"), ((d["W1"], w.H, w.M), (d["W2"], w.M, w.H))):
                b[n + "c"] = torch.empty(w.E, N, K // 2, dtype=torch.uint8, device="cuda")
                b[n + "s"] = torch.empty(w.E, N, K // 16, dtype=torch.uint8, device="cuda")
                b[n + "g"] = torch.empty(w.E, dtype=torch.float32, device="cuda")
            return b, None
        b = moe.alloc_forward(s, training=w.backward, gate_projection=gate, residual=w.residual)
        g = moe.alloc_backward(s, gate=True, gate_projection=gate, residual=w.residual) if w.backward else None
        return b, g

    def step(x, b, g):
        if kind == "blockfp8":
            moe.layer_forward_blockfp8(s, x, W1q, d.get("b1"), W2q, d.get("b2"), logits=d.get("logits"),
                                       Wg=d.get("Wg"), bufs=b)
            return
        if kind == "mxfp8":
            moe.layer_forward_mx(s, moe.MOE_MX_FP8, x, W1q, d.get("b1"), W2q, d.get("b2"), logits=d.get("logits"),
                                 Wg=d.get("Wg"), bufs=b)
            return
        if kind == "nvfp4":
            for n in ("W1", "W2"):
                moe.moe_nvfp4_quantize(d[n], w.E, b[n + "c"], b[n + "s"], b[n + "g"])
            moe.layer_forward_nvfp4(s, x, (b["W1c"], b["W1s"], b["W1g"]), d.get("b1"), (b["W2c"], b["W2s"], b["W2g"]),
                                    d.get("b2"), logits=d.get("logits"), Wg=d.get("Wg"), bufs=b)
            return
        moe.layer_forward(s, x, d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"), Wg=d.get("Wg"),
                          bufs=b, training=w.backward, residual=res)
        if g is not None:
            moe.layer_backward(s, b, d["dout"], d["W1"], d["W2"], grads=g,
                               logits=b["logits"] if gate else d["logits"], x=x, Wg=d.get("Wg"), residual=res)

    xg = d["x"].clone()  # the captured input, changed in place between replays
    bg, gg = alloc()
    step(xg, bg, gg)  # eager warm-up on the graph's buffers (first-call set-up happens here)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(xg, bg, gg)
    for rep, x in enumerate((d["x"], x2, d["x"])):
        xg.copy_(x)
        for t in _outputs(kind, bg, gg).values():
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7 if t.dtype != torch.uint8 else 0xAB)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        be, ge = alloc()
        step(x, be, ge)
        torch.cuda.synchronize()
        want = _outputs(kind, be, ge)
        got = _outputs(kind, bg, gg)
        C = int(want["capacity"].item())
        rows = w.E * C
        for n, t in want.items():
            a, b_ = got[n], t
            if n in ("buf", "pre", "h", "y", "buf_codes", "buf_scales", "h_codes", "h_scales"):
                a, b_ = a[:rows], b_[:rows]  # the filled part of the E * cmax buffers (padding rows of buf too)
                if n in ("pre", "h", "y", "h_codes", "h_scales"):
                    keep = torch.zeros(rows, dtype=torch.bool, device="cuda")
                    fill = want["fill"]
                    for e in range(w.E):
                        keep[e * C: e * C + int(fill[e])] = True
                    a, b_ = a[keep], b_[keep]  # products write only the filled rows
            assert torch.equal(a.contiguous().view(torch.uint8), b_.contiguous().view(torch.uint8)), (rep, n)
