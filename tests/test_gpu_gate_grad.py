"""GPU parity of the gate backward (dlogits through the softmax, the auxiliary
load-balance loss, dWg and dx's gate share) against the CPU oracle.

Each entry point is checked on its own with identical inputs on both sides
(seeded logits, the oracle's routes, seeded upstream dgates), at sizes that
span several blocks with ragged tails and every lane-group shape of the kernel
(E from 1 to 512), and inside the fused backward, where the two sides' dgates
agree only within tolerance and that difference is carried into the bounds.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import (check_close, check_dlogits, check_dwg, check_logits, decode_extra, dev, dgates_err, host,
                               inputs_np, shape_of)
from tests.helpers import f32_of

pytestmark = pytest.mark.gpu

AUX_REL = 2.0 ** -16

# (S, E, k, alpha, aux term on)
GB_CASES = [
    (1, 1, 1, 0.01, True), (63, 3, 2, 0.01, True), (64, 8, 2, 0.01, True), (65, 8, 2, 0.0, True),
    (1000, 16, 3, 0.01, True), (777, 64, 6, 0.5, True), (300, 100, 7, 0.01, True), (513, 128, 8, 0.01, True),
    (200, 300, 4, 0.01, True), (130, 512, 32, 0.01, True), (4096, 8, 2, 0.01, True), (50, 5, 5, 0.0, False),
    (0, 8, 2, 0.01, True),
]


def _gb_inputs(S, E, k, seed=0):
    logits = W.normal((S, E), seed, "logits").numpy()
    idx, _ = oracle.softmax_topk(logits, k)
    _, needed = oracle.locations(idx, E)
    dgates = W.normal((k, S), seed, "dgates").numpy()
    return logits, idx, needed, dgates


@pytest.mark.parametrize("S,E,k,alpha,aux", GB_CASES, ids=lambda v: str(v))
def test_gate_backward_matches_oracle(S, E, k, alpha, aux):
    import combine_softmax_top_amd as moe
    print(f"[gate backward] S={S} E={E} k={k} alpha={alpha} aux={aux}", flush=True)
    s = moe.Shape(S=S, M=64, E=E, k=k, H=64, capacity_factor=1.0)
    logits, idx, needed, dgates = _gb_inputs(S, E, k)
    nd = needed if aux else None
    dl_o, aux_o = oracle.gate_backward(logits, idx, dgates, nd, alpha)
    ws = torch.empty(max(1, moe.moe_workspace_size(s)), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        dl = torch.full((S, E), float("nan"), device="cuda")
        al = torch.full((1,), float("nan"), device="cuda")
        moe.moe_gate_backward(s, dev(logits), dev(idx), dev(dgates), dev(needed) if aux else None, alpha, dl, al, ws)
        torch.cuda.synchronize()
        outs.append((host(dl), host(al)))
    (dl_g, al_g), (dl_g2, al_g2) = outs
    assert np.array_equal(dl_g.view(np.uint32), dl_g2.view(np.uint32)), "dlogits not reproducible"
    assert al_g.view(np.uint32)[0] == al_g2.view(np.uint32)[0], "aux loss not reproducible"
    check_dlogits(dl_g, dl_o, logits, idx, dgates, nd, k, S, alpha)
    assert abs(float(al_g[0]) - aux_o) <= AUX_REL * abs(aux_o) + 1e-30, (float(al_g[0]), aux_o)
    if S > 0:
        assert np.abs(dl_g.astype(np.float64).sum(axis=1)).max() <= 1e-5 * max(np.abs(dl_g).max(), 1e-30) * E


def test_gate_backward_balanced_uniform_is_zero():
    # all logits equal and routing perfectly balanced: l_aux = alpha and, with dgates 0, no gradient
    import combine_softmax_top_amd as moe
    S, E, k = 256, 8, 2
    s = moe.Shape(S=S, M=64, E=E, k=k, H=64, capacity_factor=1.0)
    logits = np.zeros((S, E), np.float32)
    idx = np.stack([(2 * np.arange(S)) % E, (2 * np.arange(S) + 1) % E]).astype(np.int32)
    _, needed = oracle.locations(idx, E)
    ws = torch.empty(max(1, moe.moe_workspace_size(s)), dtype=torch.uint8, device="cuda")
    dl = torch.empty(S, E, device="cuda")
    al = torch.empty(1, device="cuda")
    moe.moe_gate_backward(s, dev(logits), dev(idx), torch.zeros(k, S, device="cuda"), dev(needed), 0.01, dl, al, ws)
    torch.cuda.synchronize()
    assert abs(float(host(al)[0]) - 0.01) <= 1e-8
    assert np.abs(host(dl)).max() <= 1e-12


# (S, M, E, dtype)
WG_CASES = [
    (0, 64, 8, W.DT_BF16), (1, 64, 3, W.DT_F32), (100, 192, 17, W.DT_BF16), (1000, 256, 8, W.DT_BF16),
    (4096, 1024, 8, W.DT_BF16), (333, 512, 64, W.DT_F32), (2000, 128, 300, W.DT_BF16), (65, 256, 512, W.DT_BF16),
    (129, 320, 16, W.DT_F32),
]


@pytest.mark.parametrize("S,M,E,dtype", WG_CASES, ids=lambda v: str(v))
def test_gate_weight_grad_matches_oracle(S, M, E, dtype):
    import combine_softmax_top_amd as moe
    print(f"[dWg] S={S} M={M} E={E} dtype={dtype}", flush=True)
    s = moe.Shape(S=S, M=M, E=E, k=1, H=64, capacity_factor=1.0, dtype=dtype)
    tdt = torch.float32 if dtype == W.DT_F32 else torch.bfloat16
    x = W.normal((S, M), 0, "x").to(tdt)
    dl = W.normal((S, E), 0, "logits")  # any fp32 [S, E] serves as the upstream dlogits
    xn, dln = host(x), dl.numpy()
    want = oracle.gate_weight_grad(xn, dln.astype(np.float64), dtype)
    ws = torch.empty(max(1, moe.moe_workspace_size(s)), dtype=torch.uint8, device="cuda")
    got = torch.full((M, E), float("nan"), device="cuda")
    moe.moe_gate_weight_grad(s, x.cuda(), dl.cuda(), got, ws)
    torch.cuda.synchronize()
    g = host(got)
    if S == 0:
        assert (g == 0).all()
    check_dwg(g, want, xn, dln, dtype)
    got2 = torch.empty(M, E, device="cuda")
    moe.moe_gate_weight_grad(s, x.cuda(), dl.cuda(), got2, ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(got2).view(np.uint32), g.view(np.uint32)), "dWg not reproducible"


GBWD = [
    W.Workload("gbwd_bf16_S500_E8_k2", S=500, M=256, E=8, k=2, H=128, capacity_factor=1.25, logits="gate",
               backward=True),
    W.Workload("gbwd_f32_S200_E4_k2_drops", S=200, M=64, E=4, k=2, H=128, capacity_factor=0.5, dtype=W.DT_F32,
               logits="gate", backward=True),
    W.Workload("gbwd_bigtile_S300_M1088_E4_k2_H1152", S=300, M=1088, E=4, k=2, H=1152, capacity_factor=1.0,
               logits="gate", backward=True),
    W.Workload("gbwd_relu_S257_E20_k3", S=257, M=192, E=20, k=3, H=64, capacity_factor=-0.8, act=W.ACT_RELU,
               logits="gate", backward=True),
    # logits given (no projection): dlogits and the loss only, dx without a gate share
    W.Workload("gbwd_logits_zipf_S512_E8_k4", S=512, M=128, E=8, k=4, H=192, capacity_factor=-2.0, logits="zipf",
               backward=True),
]


@pytest.mark.parametrize("w", GBWD, ids=lambda w: w.name)
def test_layer_backward_with_gate_matches_oracle(w):
    import combine_softmax_top_amd as moe
    print(f"[layer backward with gate] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    gate = w.logits == "gate"
    b = moe.layer_forward(s, d["x"], d["W1"], d.get("b1"), d["W2"], d.get("b2"), logits=d.get("logits"),
                          Wg=d.get("Wg"), training=True)
    gr = moe.layer_backward(s, b, d["dout"], d["W1"], d["W2"], logits=b["logits"] if gate else d["logits"],
                            x=d["x"], Wg=d.get("Wg"))
    torch.cuda.synchronize()
    ni = inputs_np(inp)
    glog = None
    if gate:
        # the projection within its fp32 bound; the oracle routes on the GPU's logits
        glog = host(b["logits"])
        check_logits(glog, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    fw = oracle.layer_forward(ni, w.k, w.capacity_factor, w.act, w.dtype, logits=glog)
    bw = oracle.layer_backward(fw, ni, w.act, w.dtype, aux_coef=moe.AUX_COEF)
    rt = fw["route"]
    logits = fw["logits"]
    check_close(host(gr["dgates"]), bw["dgates"], w.dtype, "dgates")
    dg_err = dgates_err(bw["dgates"], w.dtype)
    dg_err[rt["loc"] >= rt["C"]] = 0.0  # dropped routes: 0 on both sides
    dl_err = check_dlogits(host(gr["dlogits"]), bw["dlogits"], logits, rt["idx"], bw["dgates"], rt["needed"], w.k,
                           w.S, moe.AUX_COEF, dg_err=dg_err)
    aux_g = float(host(gr["aux_loss"])[0])
    assert abs(aux_g - bw["aux_loss"]) <= AUX_REL * abs(bw["aux_loss"]), (aux_g, bw["aux_loss"])
    # dx sums the token's dbuf rows: the two sides' rows (each within tolerance) carried through
    rows = fw["rows"]
    extra = decode_extra(rt, rows, host(gr["dbuf"])[rows], bw["dbuf"], gated=False)
    if gate:
        check_dwg(host(gr["dWg"]), bw["dWg"], ni["x"], bw["dlogits"], w.dtype, dl_err=dl_err)
        # dx's gate share: the dlogits bound carried through |Wg|^T
        extra += dl_err @ np.abs(ni["Wg"].astype(np.float64)).T
    check_close(host(gr["dx"]), bw["dx"], w.dtype, "dx", extra=extra)
    check_close(host(gr["dW1"]), bw["dW1"], w.dtype, "dW1")
    check_close(host(gr["dW2"]), bw["dW2"], w.dtype, "dW2")
