"""GPU parity of Residual-MoE (a dense MLP branch every token passes through, added to
the MoE output in the decode's fp32 sum) against the CPU oracle: the dense branch on
its own, forward and backward, the residual decode bit for bit given the same inputs,
and the fused layer, forward and backward."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import (check_close, check_dlogits, check_logits, decode_extra, dev, dgates_err, host,
                               inputs_np, shape_of)
from tests.helpers import bf16_bits_of_f32, f32_of

pytestmark = pytest.mark.gpu

# (S, M, H, dtype, act, biases)
FFN_CASES = [
    (1, 64, 64, W.DT_BF16, W.ACT_GELU, True), (300, 256, 384, W.DT_BF16, W.ACT_GELU, True),
    (1000, 1088, 1152, W.DT_BF16, W.ACT_GELU, True), (517, 128, 192, W.DT_BF16, W.ACT_RELU, False),
    (200, 64, 128, W.DT_F32, W.ACT_GELU, True), (0, 64, 64, W.DT_BF16, W.ACT_GELU, True),
]


@pytest.mark.parametrize("S,M,H,dtype,act,bias", FFN_CASES, ids=lambda v: str(v))
def test_residual_ffn_matches_oracle(S, M, H, dtype, act, bias):
    import combine_softmax_top_amd as moe
    print(f"[residual ffn] S={S} M={M} H={H} dtype={dtype} act={act} bias={bias}", flush=True)
    w = W.Workload("res", S=S, M=M, E=2, k=1, H=H, capacity_factor=1.0, dtype=dtype, act=act, has_fc1_bias=bias,
                   has_fc2_bias=bias, residual=True)
    inp = W.make_inputs(w, seed=0)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    ws = torch.empty(max(1, moe.moe_workspace_size(s)), dtype=torch.uint8, device="cuda")
    pre_r = torch.empty(S, H, dtype=w.torch_dtype, device="cuda")
    h_r = torch.empty(S, H, dtype=w.torch_dtype, device="cuda")
    y_r = torch.empty(S, M, dtype=w.torch_dtype, device="cuda")
    moe.moe_residual_ffn(s, d["x"], d["W1r"], d.get("b1r"), d["W2r"], d.get("b2r"), pre_r, h_r, y_r, ws)
    torch.cuda.synchronize()
    ni = inputs_np(inp)
    p_o, h_o, y_o = oracle.residual_mlp(ni["x"], ni["W1r"], ni.get("b1r"), ni["W2r"], ni.get("b2r"), act, dtype,
                                        want_pre=True)
    check_close(host(pre_r), p_o, dtype, "pre_r")
    check_close(host(h_r), h_o, dtype, "h_r")
    check_close(host(y_r), y_o, dtype, "y_r")
    # without pre_r (inference) the branch's outputs are the same bits
    h2, y2 = torch.empty_like(h_r), torch.empty_like(y_r)
    moe.moe_residual_ffn(s, d["x"], d["W1r"], d.get("b1r"), d["W2r"], d.get("b2r"), None, h2, y2, ws)
    torch.cuda.synchronize()
    assert torch.equal(h2.view(torch.uint8), h_r.view(torch.uint8)) and torch.equal(y2.view(torch.uint8),
                                                                                    y_r.view(torch.uint8))


@pytest.mark.parametrize("S,M,H,dtype,act,bias", FFN_CASES, ids=lambda v: str(v))
def test_residual_backward_matches_oracle(S, M, H, dtype, act, bias):
    # the dense branch's backward on its own: dpre_r, dx_r (stored) and the fp32 weight and
    # bias gradients summed over every token
    import combine_softmax_top_amd as moe
    print(f"[residual backward] S={S} M={M} H={H} dtype={dtype} act={act} bias={bias}", flush=True)
    w = W.Workload("resb", S=S, M=M, E=2, k=1, H=H, capacity_factor=1.0, dtype=dtype, act=act, has_fc1_bias=bias,
                   has_fc2_bias=bias, residual=True)
    inp = W.make_inputs(w, seed=1, with_dout=True)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    dt = w.torch_dtype
    f32 = dict(dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, moe.moe_workspace_size(s)), dtype=torch.uint8, device="cuda")
    pre_r, h_r = torch.empty(S, H, dtype=dt, device="cuda"), torch.empty(S, H, dtype=dt, device="cuda")
    y_r = torch.empty(S, M, dtype=dt, device="cuda")
    moe.moe_residual_ffn(s, d["x"], d["W1r"], d.get("b1r"), d["W2r"], d.get("b2r"), pre_r, h_r, y_r, ws)
    dpre_r, dx_r = torch.empty(S, H, dtype=dt, device="cuda"), torch.empty(S, M, dtype=dt, device="cuda")
    # gradients start as NaN: the call must overwrite every element
    dW1r, dW2r = torch.full((H, M), float("nan"), **f32), torch.full((M, H), float("nan"), **f32)
    db1r = torch.full((H,), float("nan"), **f32) if bias else None
    db2r = torch.full((M,), float("nan"), **f32) if bias else None
    moe.moe_residual_backward(s, d["dout"], d["x"], pre_r, h_r, d["W1r"], d["W2r"], dpre_r, dx_r, dW1r, db1r, dW2r,
                              db2r, ws)
    torch.cuda.synchronize()
    if S == 0:
        for t in (dW1r, dW2r) + ((db1r, db2r) if bias else ()):
            assert (host(t) == 0).all()
        return
    ni = inputs_np(inp)
    rb = oracle.residual_backward(ni, act, dtype)
    check_close(host(dpre_r), rb["dpre_r"], dtype, "dpre_r")
    check_close(host(dx_r), rb["dx_r"], dtype, "dx_r")
    check_close(host(dW1r), rb["dW1r"], dtype, "dW1r")
    check_close(host(dW2r), rb["dW2r"], dtype, "dW2r")
    if bias:
        check_close(host(db1r), rb["db1r"], dtype, "db1r")
        check_close(host(db2r), rb["db2r"], dtype, "db2r")


@pytest.mark.parametrize("dtype", [W.DT_BF16, W.DT_F32])
@pytest.mark.parametrize("S,E,k,f", [(1000, 8, 1, 1.25), (777, 16, 2, 0.5), (64, 4, 1, 0.25)])
def test_decode_residual_bit_exact(S, E, k, f, dtype):
    # given the same expert outputs and dense-branch rows, the fp32 sum and its one rounding match exactly
    import combine_softmax_top_amd as moe
    M = 192
    w = W.Workload("dres", S=S, M=M, E=E, k=k, H=64, capacity_factor=f, dtype=dtype)
    logits = W.normal((S, E), 1, "logits").numpy()
    rt = oracle.route(logits, k, f)
    C = rt["C"]
    tdt = w.torch_dtype
    y = W.normal((E * C, M), 1, "W1").to(tdt)
    yr = W.normal((S, M), 1, "W2").to(tdt)
    want = oracle.decode(host(y), rt, E, dtype, yres=host(yr))
    s = shape_of(w)
    out = torch.empty(S, M, dtype=tdt, device="cuda")
    moe.moe_decode_residual(s, y.cuda(), dev(rt["gates"]), dev(rt["idx"]), dev(rt["loc"]),
                            torch.tensor([C], dtype=torch.int32, device="cuda"), yr.cuda(), out)
    torch.cuda.synchronize()
    assert np.array_equal(host(out).view(np.uint8), want.view(np.uint8))


RES = [
    W.Workload("res_gate_S500_E8_k1", S=500, M=256, E=8, k=1, H=384, capacity_factor=1.25, logits="gate",
               residual=True),
    W.Workload("res_drops_S300_E4_k1", S=300, M=128, E=4, k=1, H=128, capacity_factor=0.5, residual=True),
    W.Workload("res_k2_relu_nobias_S257_E6", S=257, M=64, E=6, k=2, H=192, capacity_factor=1.0, act=W.ACT_RELU,
               has_fc1_bias=False, has_fc2_bias=False, residual=True),
    W.Workload("res_f32_S200_E4_k1", S=200, M=64, E=4, k=1, H=128, capacity_factor=1.0, dtype=W.DT_F32,
               residual=True),
    W.Workload("res_bigtile_S600_M1088_E4_k1_H1152", S=600, M=1088, E=4, k=1, H=1152, capacity_factor=1.0,
               residual=True),
]


@pytest.mark.parametrize("w", RES, ids=lambda w: w.name)
def test_residual_layer_forward_matches_oracle(w):
    import combine_softmax_top_amd as moe
    print(f"[residual layer] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    res = {n: d.get(n) for n in ("W1r", "b1r", "W2r", "b2r")}
    b = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                          Wg=d.get("Wg"), residual=res)
    torch.cuda.synchronize()
    ni = inputs_np(inp)
    glog = None
    if w.logits == "gate":
        # the projection within its fp32 bound; the oracle routes on the GPU's logits
        glog = host(b["logits"])
        check_logits(glog, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    fw = oracle.layer_forward(ni, w.k, w.capacity_factor, w.act, w.dtype, logits=glog)
    rt = fw["route"]
    assert int(b["capacity"].item()) == rt["C"]
    assert np.array_equal(host(b["idx"]), rt["idx"]) and np.array_equal(host(b["loc"]), rt["loc"])
    yr_g = host(b["y_r"])
    check_close(yr_g, fw["y_r"], w.dtype, "y_r")
    # the end-to-end output: the two sides' y and y_r rows (each within tolerance) carried through decode
    rows = fw["rows"]
    extra = decode_extra(rt, rows, host(b["y"])[rows], fw["y"][rows])
    extra += np.abs(f32_of(yr_g).astype(np.float64) - f32_of(fw["y_r"]).astype(np.float64))
    check_close(host(b["out"]), fw["out"], w.dtype, "out", extra=extra)
    # given the GPU's own expert outputs and dense rows, the residual decode is exact
    want = oracle.decode(host(b["y"][: w.E * rt["C"]]), rt, w.E, w.dtype, yres=host(b["y_r"]))
    assert np.array_equal(host(b["out"]).view(np.uint8), want.view(np.uint8))
    dropped = np.nonzero((rt["loc"] >= rt["C"]).all(axis=0))[0]
    if len(dropped):
        assert np.array_equal(host(b["out"])[dropped].view(np.uint8), host(b["y_r"])[dropped].view(np.uint8))


@pytest.mark.parametrize("w", RES, ids=lambda w: w.name)
def test_residual_layer_backward_matches_oracle(w):
    # the fused training step of a Residual-MoE layer: the MoE backward, the dense branch's
    # backward, and dx = the kept dbuf rows (+ the gate share) + dx_r, rounded once
    import combine_softmax_top_amd as moe
    print(f"[residual layer backward] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=2, with_dout=True)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    gate = w.logits == "gate"
    res = {n: d.get(n) for n in ("W1r", "b1r", "W2r", "b2r")}
    b = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                          Wg=d.get("Wg"), training=True, residual=res)
    gr = moe.layer_backward(s, b, d["dout"], d["W1"], d["W2"], logits=b["logits"] if gate else None, x=d["x"],
                            Wg=d.get("Wg"), residual=res)
    torch.cuda.synchronize()
    ni = inputs_np(inp)
    glog = None
    if gate:
        glog = host(b["logits"])
        check_logits(glog, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    fw = oracle.layer_forward(ni, w.k, w.capacity_factor, w.act, w.dtype, logits=glog)
    bw = oracle.layer_backward(fw, ni, w.act, w.dtype, aux_coef=moe.AUX_COEF if gate else None)
    rt = fw["route"]
    check_close(host(b["pre_r"]), fw["pre_r"], w.dtype, "pre_r")
    for n in ("dpre_r", "dx_r", "dW1r", "dW2r") + (("db1r", "db2r") if w.has_fc1_bias else ()):
        check_close(host(gr[n]), bw[n], w.dtype, n)
    check_close(host(gr["dW1"]), bw["dW1"], w.dtype, "dW1")
    check_close(host(gr["dW2"]), bw["dW2"], w.dtype, "dW2")
    # dx: both sides' dbuf rows and dx_r rows (each within tolerance) carried through the sum
    rows = fw["rows"]
    extra = decode_extra(rt, rows, host(gr["dbuf"])[rows], bw["dbuf"], gated=False)
    extra += np.abs(f32_of(host(gr["dx_r"])).astype(np.float64) - f32_of(bw["dx_r"]).astype(np.float64))
    if gate:
        dg_err = dgates_err(bw["dgates"], w.dtype)
        dg_err[rt["loc"] >= rt["C"]] = 0.0
        dl_err = check_dlogits(host(gr["dlogits"]), bw["dlogits"], fw["logits"], rt["idx"], bw["dgates"],
                               rt["needed"], w.k, w.S, moe.AUX_COEF, dg_err=dg_err)
        extra += dl_err @ np.abs(ni["Wg"].astype(np.float64)).T
    check_close(host(gr["dx"]), bw["dx"], w.dtype, "dx", extra=extra)
    # given the GPU's own dbuf and dx_r rows (and no gate share), dx is their fp32 sum rounded once
    if not gate:
        dbuf = f32_of(host(gr["dbuf"])).astype(np.float32)
        want = np.zeros((w.S, w.M), np.float32)
        for r in range(w.k):
            kept = rt["loc"][r] < rt["C"]
            slot = rt["idx"][r].astype(np.int64) * rt["C"] + rt["loc"][r]
            want[kept] = want[kept] + dbuf[slot[kept]]
        want = want + f32_of(host(gr["dx_r"])).astype(np.float32)
        got = f32_of(host(gr["dx"]))
        if w.dtype == W.DT_F32:
            assert np.array_equal(got, want)
        else:
            assert np.array_equal(host(gr["dx"]).view(np.uint16), bf16_bits_of_f32(want))


def test_residual_layer_empty_input():
    # S = 0: the training step runs and overwrites every weight and bias gradient with zeros
    import combine_softmax_top_amd as moe
    w = W.Workload("res_empty", S=0, M=64, E=3, k=1, H=128, capacity_factor=1.0, residual=True)
    inp = W.make_inputs(w, seed=0, with_dout=True)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    res = {n: d.get(n) for n in ("W1r", "b1r", "W2r", "b2r")}
    b = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d["logits"], training=True,
                          residual=res)
    g = moe.alloc_backward(s, residual=True)
    for n in ("dW1", "dW2", "db1", "db2", "dW1r", "dW2r", "db1r", "db2r"):
        g[n].fill_(float("nan"))
    moe.layer_backward(s, b, d["dout"], d["W1"], d["W2"], grads=g, x=d["x"], residual=res)
    torch.cuda.synchronize()
    assert b["out"].numel() == 0 and g["dx"].numel() == 0
    for n in ("dW1", "dW2", "db1", "db2", "dW1r", "dW2r", "db1r", "db2r"):
        assert (host(g[n]) == 0).all(), n


def test_residual_backward_of_fully_dropped_tokens_is_the_dense_branch():
    # all logits tie, so every token picks expert 0 (ties go to the lower index) and capacity keeps
    # C of them; a token with no kept route gets dx = dx_r exactly (0 + dx_r rounds to dx_r), the
    # kept ones gain their dbuf rows
    import combine_softmax_top_amd as moe
    w = W.Workload("res_ties", S=256, M=128, E=4, k=1, H=128, capacity_factor=0.25, residual=True)
    inp = W.make_inputs(w, seed=3, with_dout=True)
    inp["logits"] = torch.zeros(w.S, w.E)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    res = {n: d.get(n) for n in ("W1r", "b1r", "W2r", "b2r")}
    b = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d["logits"], training=True,
                          residual=res)
    g = moe.layer_backward(s, b, d["dout"], d["W1"], d["W2"], x=d["x"], residual=res)
    torch.cuda.synchronize()
    loc = host(b["loc"])[0]
    C = int(b["capacity"].item())
    dropped = np.nonzero(loc >= C)[0]
    kept = np.nonzero(loc < C)[0]
    assert len(dropped) == w.S - C > 0
    dx, dxr = host(g["dx"]).view(np.uint16), host(g["dx_r"]).view(np.uint16)
    assert np.array_equal(dx[dropped], dxr[dropped])
    assert not np.array_equal(dx[kept], dxr[kept])
