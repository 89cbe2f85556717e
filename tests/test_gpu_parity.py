"""GPU parity of every step of the HIP path against the CPU oracle, at sizes the
oracle finishes in seconds (several tiles, ragged tails), plus edge cases.

Each step is checked twice: on its own, fed with the oracle's own upstream
results (so a failure names the step), and inside the fused layer call.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import (check_close, check_gates, check_logits, compare_route, decode_extra, dev, gpu_route, host,
                               inputs_np, shape_of)
from tests.helpers import f32_of

pytestmark = pytest.mark.gpu

MID = [
    W.Workload("mid_bf16_S1000_E8_k2", S=1000, M=256, E=8, k=2, H=384, capacity_factor=1.25),
    W.Workload("mid_zipf_S777_E64_k6_nobias", S=777, M=128, E=64, k=6, H=192, capacity_factor=-1.5,
               has_fc1_bias=False, has_fc2_bias=False, logits="zipf"),
    W.Workload("mid_f0_S640_E16_k3", S=640, M=192, E=16, k=3, H=256, capacity_factor=0.0),
    W.Workload("mid_gate_S500_E8_k2", S=500, M=256, E=8, k=2, H=128, capacity_factor=1.25, logits="gate"),
    W.Workload("mid_f32_relu_S300_E4_k1", S=300, M=64, E=4, k=1, H=128, capacity_factor=1.0, dtype=W.DT_F32,
               act=W.ACT_RELU),
    W.Workload("mid_f32_gelu_S333_E6_k2", S=333, M=128, E=6, k=2, H=192, capacity_factor=0.5, dtype=W.DT_F32),
    W.Workload("mid_relu_bf16_S257_E5_k5", S=257, M=64, E=5, k=5, H=64, capacity_factor=0.0, act=W.ACT_RELU),
    # K > 1024 in both products, so the forward GEMMs take their large-tile
    # configuration; ragged row tiles and a partial last column tile (1152, 1088)
    W.Workload("mid_bigtile_S600_M1088_E4_k2_H1152", S=600, M=1088, E=4, k=2, H=1152, capacity_factor=1.0),
]


def _oracle_forward(w, inp_np, logits=None):
    return oracle.layer_forward(inp_np, w.k, w.capacity_factor, w.act, w.dtype, logits=logits)


def _gpu_forward(w, inp, training=False):
    import combine_softmax_top_amd as moe
    s = shape_of(w)
    d = {k: v.cuda() for k, v in inp.items()}
    b = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                          Wg=d.get("Wg"), training=training)
    torch.cuda.synchronize()
    return b, d


# ------------------------------------------------------------------ routing

ROUTE_CASES = [
    (1, 1, 1.0, 100), (3, 2, 1.0, 65), (4, 1, 1.0, 256), (8, 2, 1.25, 4096), (16, 3, 0.0, 1000),
    (64, 6, -1.5, 3000), (100, 7, -0.7, 999), (128, 8, -2.0, 5000), (256, 4, 2.0, 700), (512, 32, -1.0, 640),
    (8, 8, 0.0, 63), (5, 3, 0.3, 1),
]


@pytest.mark.parametrize("E,k,f,S", ROUTE_CASES)
def test_route_bit_exact(E, k, f, S):
    rng = np.random.default_rng(E * 1000 + k)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    logits[: S // 10] = np.round(logits[: S // 10] * 2) / 2  # many exact ties
    if S > 3:
        logits[1] = 0.0
        logits[2, ::2] = -0.0
        logits[2, 1::2] = 0.0
    if E > 1 and S > 4:
        logits[3:, 0] += 1.0  # skew toward expert 0 so that f < 0 drops
    w = W.Workload("route", S=S, M=64, E=E, k=k, H=64, capacity_factor=f)
    g = gpu_route(w, logits)
    o = oracle.route(logits, k, f)
    compare_route(g, o, E)


def test_route_all_tokens_tied():
    S, E, k = 300, 8, 3
    logits = np.full((S, E), 0.25, np.float32)
    w = W.Workload("tied", S=S, M=64, E=E, k=k, H=64, capacity_factor=1.0)
    g = gpu_route(w, logits)
    o = oracle.route(logits, k, 1.0)
    compare_route(g, o, E)
    assert (g["idx"] == np.arange(k)[:, None]).all()
    assert g["fill"][:k].tolist() == [g["C"]] * k and (g["fill"][k:] == 0).all()


def test_route_empty_input():
    w = W.Workload("empty", S=0, M=64, E=4, k=2, H=64, capacity_factor=0.0)
    g = gpu_route(w, np.zeros((0, 4), np.float32))
    assert g["C"] == 1 and (g["needed"] == 0).all() and (g["fill"] == 0).all()


# Gate projection shapes: M from 64 to 4160 (one to three LDS passes of up to 2048
# rows of Wg), ragged token groups, E from 3 to 512 (expert groups of 8, the last one
# partial; E not a multiple of 4 stages Wg element by element), both dtypes.
GATE_CASES = [
    MID[3],
    W.GATED_BF16.replace(S=1024),
    W.Workload("gp_bf16_S33_M3072_E8", S=33, M=3072, E=8, k=2, H=64, capacity_factor=1.0, logits="gate"),
    W.Workload("gp_f32_S50_M2048_E3", S=50, M=2048, E=3, k=1, H=64, capacity_factor=1.0, dtype=W.DT_F32,
               logits="gate"),
    W.Workload("gp_f32_S45_M192_E300", S=45, M=192, E=300, k=3, H=64, capacity_factor=1.0, dtype=W.DT_F32,
               logits="gate"),
    W.Workload("gp_bf16_S37_M128_E512", S=37, M=128, E=512, k=2, H=64, capacity_factor=1.0, logits="gate"),
    W.Workload("gp_bf16_S5_M64_E200", S=5, M=64, E=200, k=4, H=64, capacity_factor=1.0, logits="gate"),
    # three passes: 2048, 2048 and 64 rows
    W.Workload("gp_bf16_S19_M4160_E4", S=19, M=4160, E=4, k=2, H=64, capacity_factor=1.0, logits="gate"),
    # E = 13: two expert groups (8 and 5), Wg staged element by element; two passes (2048 + 128)
    W.Workload("gp_bf16_S77_M2176_E13", S=77, M=2176, E=13, k=3, H=64, capacity_factor=1.0, logits="gate"),
    W.Workload("gp_f32_S29_M2112_E13", S=29, M=2112, E=13, k=2, H=64, capacity_factor=1.0, dtype=W.DT_F32,
               logits="gate"),
]


@pytest.mark.parametrize("w", GATE_CASES, ids=lambda w: w.name)
def test_gate_projection_within_fp32_bound(w):
    import combine_softmax_top_amd as moe
    inp = W.make_inputs(w, seed=3)
    x, Wg = host(inp["x"]), host(inp["Wg"])
    o = oracle.gate_logits(x, Wg, w.dtype)
    logits = torch.empty(w.S, w.E, dtype=torch.float32, device="cuda")
    moe.moe_gate_project(shape_of(w), inp["x"].cuda(), inp["Wg"].cuda(), logits)
    torch.cuda.synchronize()
    check_logits(host(logits), o, x, Wg)


# ------------------------------------------------------------------ stage by stage

@pytest.mark.parametrize("w", MID, ids=lambda w: w.name)
def test_encode_bit_exact_given_oracle_route(w):
    import combine_softmax_top_amd as moe
    inp = W.make_inputs(w, seed=1)
    ni = inputs_np(inp)
    logits = ni["logits"] if "logits" in ni else oracle.gate_logits(ni["x"], ni["Wg"], w.dtype)
    rt = oracle.route(logits, w.k, w.capacity_factor)
    want = oracle.encode(ni["x"], rt, w.E, w.dtype)
    s = shape_of(w)
    cmax = moe.moe_capacity_bound(s)
    buf = torch.full((w.E * cmax, w.M), float("nan"), dtype=w.torch_dtype, device="cuda")
    moe.moe_encode(s, inp["x"].cuda(), dev(rt["idx"]), dev(rt["loc"]), dev(rt["fill"]),
                   dev(np.array([rt["C"]], np.int32)), buf)
    torch.cuda.synchronize()
    got = host(buf[: w.E * rt["C"]])
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))
    # rows beyond E*C are untouched
    if w.E * cmax > w.E * rt["C"]:
        assert torch.isnan(buf[w.E * rt["C"]:].float()).all()


@pytest.mark.parametrize("w", MID, ids=lambda w: w.name)
def test_expert_ffn_given_oracle_buffer(w):
    import combine_softmax_top_amd as moe
    inp = W.make_inputs(w, seed=2)
    ni = inputs_np(inp)
    fw = _oracle_forward(w, ni)
    rt = fw["route"]
    s = shape_of(w)
    cmax = moe.moe_capacity_bound(s)
    C = rt["C"]
    buf = torch.zeros(w.E * cmax, w.M, dtype=w.torch_dtype, device="cuda")
    buf[: w.E * C] = dev(fw["buf"])
    h = torch.empty(w.E * cmax, w.H, dtype=w.torch_dtype, device="cuda")
    pre = torch.empty_like(h)
    y = torch.empty(w.E * cmax, w.M, dtype=w.torch_dtype, device="cuda")
    d = {k: v.cuda() for k, v in inp.items()}
    moe.moe_expert_ffn(s, buf, d["W1"], d.get("b1"), d["W2"], d.get("b2"), dev(rt["fill"]),
                       dev(np.array([C], np.int32)), pre, h, y)
    torch.cuda.synchronize()
    rows = fw["rows"]
    check_close(host(pre)[rows], fw["pre"][rows], w.dtype, "pre")
    check_close(host(h)[rows], fw["h"][rows], w.dtype, "h")
    check_close(host(y)[rows], fw["y"][rows], w.dtype, "y")


@pytest.mark.parametrize("w", MID, ids=lambda w: w.name)
def test_decode_bit_exact_given_oracle_expert_output(w):
    # decode does the oracle's arithmetic (fp32, route order, separate multiply and add)
    import combine_softmax_top_amd as moe
    rng = np.random.default_rng(5)
    inp = W.make_inputs(w, seed=4)
    ni = inputs_np(inp)
    logits = ni["logits"] if "logits" in ni else oracle.gate_logits(ni["x"], ni["Wg"], w.dtype)
    rt = oracle.route(logits, w.k, w.capacity_factor)
    C = rt["C"]
    y32 = rng.standard_normal((w.E * C, w.M)).astype(np.float32)
    y = y32 if w.dtype == W.DT_F32 else host(torch.from_numpy(y32).to(torch.bfloat16))
    want = oracle.decode(y, rt, w.E, w.dtype)
    out = torch.empty(w.S, w.M, dtype=w.torch_dtype, device="cuda")
    moe.moe_decode(shape_of(w), dev(y), dev(rt["gates"]), dev(rt["idx"]), dev(rt["loc"]),
                   dev(np.array([C], np.int32)), out)
    torch.cuda.synchronize()
    got = host(out)
    assert np.array_equal(got.view(np.uint8), want.view(np.uint8))


# ------------------------------------------------------------------ fused forward

@pytest.mark.parametrize("w", MID, ids=lambda w: w.name)
def test_layer_forward_matches_oracle(w):
    inp = W.make_inputs(w, seed=0)
    b, d = _gpu_forward(w, inp, training=True)
    ni = inputs_np(inp)
    logits = None
    if w.logits == "gate":
        logits = host(b["logits"])
        check_logits(logits, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    fw = _oracle_forward(w, ni, logits=logits)
    rt = fw["route"]
    C = int(b["capacity"].item())
    g = dict(idx=host(b["idx"]), loc=host(b["loc"]), gates=host(b["gates"]), needed=host(b["needed"]),
             fill=host(b["fill"]), C=C, slot_route=host(b["slot_route"][: w.E * C]))
    compare_route(g, rt, w.E)
    assert np.array_equal(host(b["buf"][: w.E * C]).view(np.uint8), fw["buf"].view(np.uint8))
    rows = fw["rows"]
    check_close(host(b["h"])[rows], fw["h"][rows], w.dtype, "h")
    check_close(host(b["pre"])[rows], fw["pre"][rows], w.dtype, "pre")
    yg = host(b["y"])[rows]
    check_close(yg, fw["y"][rows], w.dtype, "y")
    check_close(host(b["out"]), fw["out"], w.dtype, "out", extra=decode_extra(rt, rows, yg, fw["y"][rows]))


def test_layer_forward_is_deterministic():
    w = MID[1]
    inp = W.make_inputs(w, seed=7)
    b1, _ = _gpu_forward(w, inp)
    r1 = {k: host(v).copy() for k, v in b1.items() if v is not None and k not in ("ws", "h", "y", "slot_route", "buf")}
    b2, _ = _gpu_forward(w, inp)
    for k, v in r1.items():
        assert np.array_equal(host(b2[k]).view(np.uint8), v.view(np.uint8)), k


def test_layer_forward_empty_input():
    import combine_softmax_top_amd as moe
    w = W.Workload("empty", S=0, M=64, E=3, k=2, H=64, capacity_factor=1.0)
    inp = W.make_inputs(w, seed=0)
    b, _ = _gpu_forward(w, inp)
    assert int(b["capacity"].item()) == 1
    assert (host(b["buf"][:3]).view(np.uint16) == 0).all()
    assert b["out"].numel() == 0
    assert moe.moe_capacity_bound(shape_of(w)) == 1


def test_layer_forward_everything_dropped_but_capacity():
    # all tokens tie: experts 0..k-1 take C tokens each, the rest are dropped; dropped tokens give 0
    w = W.Workload("ties", S=256, M=64, E=4, k=2, H=64, capacity_factor=0.25)
    inp = W.make_inputs(w, seed=0)
    inp["logits"] = torch.zeros(w.S, w.E)
    b, d = _gpu_forward(w, inp)
    ni = inputs_np(inp)
    fw = _oracle_forward(w, ni)
    C = int(b["capacity"].item())
    assert C == fw["route"]["C"] == 32
    out = f32_of(host(b["out"]))
    assert (out[C:] == 0).all()
    rows = fw["rows"]
    check_close(host(b["out"]), fw["out"], w.dtype, "out",
                extra=decode_extra(fw["route"], rows, host(b["y"])[rows], fw["y"][rows]))


# ------------------------------------------------------------------ backward

BWD = [
    W.Workload("bwd_bf16_S512_E8_k4", S=512, M=128, E=8, k=4, H=192, capacity_factor=-2.0, logits="zipf",
               backward=True),
    W.Workload("bwd_bf16_relu_S300_E4_k2_nobias", S=300, M=64, E=4, k=2, H=128, capacity_factor=0.75,
               act=W.ACT_RELU, has_fc1_bias=False, has_fc2_bias=False, backward=True),
    W.Workload("bwd_f32_S200_E4_k2", S=200, M=64, E=4, k=2, H=128, capacity_factor=0.5, dtype=W.DT_F32,
               backward=True),
    W.Workload("bwd_f32_relu_S130_E3_k3", S=130, M=64, E=3, k=3, H=64, capacity_factor=0.0, dtype=W.DT_F32,
               act=W.ACT_RELU, backward=True),
    # K > 1024 in both backward data products (the large-tile configuration,
    # weights read n-contiguous), ragged row tiles, partial last column tiles
    W.Workload("bwd_bigtile_S300_M1088_E4_k2_H1152", S=300, M=1088, E=4, k=2, H=1152, capacity_factor=1.0,
               backward=True),
]


@pytest.mark.parametrize("w", BWD, ids=lambda w: w.name)
def test_layer_backward_matches_oracle(w):
    import combine_softmax_top_amd as moe
    inp = W.make_inputs(w, seed=0)
    b, d = _gpu_forward(w, inp, training=True)
    s = shape_of(w)
    gr = moe.layer_backward(s, b, d["dout"], d["W1"], d["W2"])
    torch.cuda.synchronize()
    ni = inputs_np(inp)
    fw = _oracle_forward(w, ni)
    bw = oracle.layer_backward(fw, ni, w.act, w.dtype)
    # dx sums the token's dbuf rows: the two sides' rows (each within tolerance) carried through
    rows = fw["rows"]
    check_close(host(gr["dx"]), bw["dx"], w.dtype, "dx",
                extra=decode_extra(fw["route"], rows, host(gr["dbuf"])[rows], bw["dbuf"], gated=False))
    check_close(host(gr["dgates"]), bw["dgates"], w.dtype, "dgates")
    check_close(host(gr["dW1"]), bw["dW1"], w.dtype, "dW1")
    check_close(host(gr["dW2"]), bw["dW2"], w.dtype, "dW2")
    if w.has_fc1_bias:
        check_close(host(gr["db1"]), bw["db1"], w.dtype, "db1")
    if w.has_fc2_bias:
        check_close(host(gr["db2"]), bw["db2"], w.dtype, "db2")
    # dropped routes have no gate gradient
    rt = fw["route"]
    assert (host(gr["dgates"])[rt["loc"] >= rt["C"]] == 0).all()
    # experts that received nothing get zero weight gradients
    for e in np.nonzero(rt["fill"] == 0)[0]:
        assert (host(gr["dW1"][e]) == 0).all() and (host(gr["dW2"][e]) == 0).all()


@pytest.mark.parametrize("w", BWD, ids=lambda w: w.name)
def test_backward_intermediates_match_oracle(w):
    # dy, dpre and dbuf on every filled row, through the stage entry points (the fused
    # backward lets dbuf reuse dy's memory): dy = g * dout rounded to the data type,
    # dpre = (dy W2) * act'(pre), dbuf = dpre W1
    import combine_softmax_top_amd as moe
    print(f"[backward intermediates] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    b, d = _gpu_forward(w, inp, training=True)
    s = shape_of(w)
    g = moe.alloc_backward(s)
    g["dbuf"] = torch.empty_like(g["dy"])
    moe.moe_decode_backward(s, d["dout"], b["y"], b["gates"], b["idx"], b["loc"], b["capacity"], g["dy"], g["dgates"])
    moe.moe_expert_fc2_backward_data(s, g["dy"], d["W2"], b["pre"], b["fill"], b["capacity"], g["dpre"])
    moe.moe_expert_fc1_backward_data(s, g["dpre"], d["W1"], b["fill"], b["capacity"], g["dbuf"])
    torch.cuda.synchronize()
    ni = inputs_np(inp)
    fw = _oracle_forward(w, ni)
    bw = oracle.layer_backward(fw, ni, w.act, w.dtype)
    rows = fw["rows"]
    assert len(rows) > 0
    check_close(host(g["dy"])[rows], bw["dy"], w.dtype, "dy rows")
    check_close(host(g["dpre"])[rows], bw["dpre"], w.dtype, "dpre rows")
    check_close(host(g["dbuf"])[rows], bw["dbuf"], w.dtype, "dbuf rows")


@pytest.mark.parametrize("w", [BWD[0], BWD[2], BWD[4]], ids=lambda w: w.name)
def test_backward_stages_equal_the_fused_backward(w):
    # the per-stage entry points run the fused backward's kernels: same bits
    import combine_softmax_top_amd as moe
    print(f"[backward stages] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=3)
    b, d = _gpu_forward(w, inp, training=True)
    s = shape_of(w)
    gr = moe.layer_backward(s, b, d["dout"], d["W1"], d["W2"])
    g = moe.alloc_backward(s)
    g["dbuf"] = torch.empty_like(g["dy"])
    moe.moe_decode_backward(s, d["dout"], b["y"], b["gates"], b["idx"], b["loc"], b["capacity"], g["dy"], g["dgates"])
    moe.moe_expert_fc2_weight_grad(s, g["dy"], b["h"], b["fill"], b["capacity"], g["dW2"], g["db2"])
    moe.moe_expert_fc2_backward_data(s, g["dy"], d["W2"], b["pre"], b["fill"], b["capacity"], g["dpre"])
    moe.moe_expert_fc1_backward_data(s, g["dpre"], d["W1"], b["fill"], b["capacity"], g["dbuf"])
    moe.moe_expert_fc1_weight_grad(s, g["dpre"], b["buf"], b["fill"], b["capacity"], g["dW1"], g["db1"])
    moe.moe_encode_backward(s, g["dbuf"], b["idx"], b["loc"], b["capacity"], g["dx"])
    torch.cuda.synchronize()
    for n in ("dx", "dgates", "dW1", "dW2", "db1", "db2"):
        assert torch.equal(gr[n].view(torch.int16) if gr[n].dtype == torch.bfloat16 else gr[n].view(torch.int32),
                           g[n].view(torch.int16) if g[n].dtype == torch.bfloat16 else g[n].view(torch.int32)), n
