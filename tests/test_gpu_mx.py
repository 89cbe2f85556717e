"""GPU parity of the MX (OCP microscaling) low-precision experts against the CPU oracle.

MX quantisation takes its decisions (shared exponent, element codes) from the same
inputs on both sides, so the quantiser and the MX encode are compared bit for bit.
The expert FFN's h is quantised from fp32 values that the two sides reach by
different summation orders (and the hardware's fp8 accumulation drops low-order
bits of small products, about 1e-4 of the sum of magnitudes), so its codes may
differ by one step where a value sits at a rounding boundary: they are checked to
agree almost everywhere, and y and the layer output are compared with the bf16
tolerance rule.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import check_close, check_logits, compare_route, decode_extra, dev, host, inputs_np, shape_of

pytestmark = pytest.mark.gpu

FMTS = [oracle.MX_FP8, oracle.MX_FP4]


def _mx_source(rows, K, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(rows, K, generator=g) * torch.exp(torch.empty(rows, 1).uniform_(-8, 8, generator=g))
    if rows > 2:
        a[0, :32] = 0.0
        a[1, :32] = 0.0
        a[1, 3] = -0.0
        a[2, 32:64] = 2.0 ** 5
    return a.to(torch.float32 if dtype == W.DT_F32 else torch.bfloat16)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16])
@pytest.mark.parametrize("rows,K", [(300, 256), (7, 64), (1, 32), (0, 128), (513, 1088)])
def test_mx_quantize_bit_exact(fmt, dtype, rows, K):
    import combine_softmax_top_amd as moe
    print(f"[mx quantize] fmt={fmt} dtype={dtype} rows={rows} K={K}", flush=True)
    a = _mx_source(rows, K, dtype, 3 + rows)
    want_c, want_s = oracle.mx_quantize(host(a), fmt, dtype)
    codes, scales = moe.mx_alloc((rows, K), fmt)
    moe.moe_mx_quantize(fmt, a.cuda(), codes, scales, dtype=dtype)
    torch.cuda.synchronize()
    assert np.array_equal(host(codes), want_c), "codes"
    assert np.array_equal(host(scales), want_s), "scales"


MXW = [
    W.Workload("mx_S1000_M256_E8_k2_H384", S=1000, M=256, E=8, k=2, H=384, capacity_factor=1.25),
    W.Workload("mx_S777_M128_E16_k3_H256_f0", S=777, M=128, E=16, k=3, H=256, capacity_factor=0.0),
    W.Workload("mx_relu_nobias_S300_M384_E4_k1_H640", S=300, M=384, E=4, k=1, H=640, capacity_factor=0.75,
               act=W.ACT_RELU, has_fc1_bias=False, has_fc2_bias=False),
    W.Workload("mx_gate_S600_M1024_E4_k2_H1152", S=600, M=1024, E=4, k=2, H=1152, capacity_factor=1.0,
               logits="gate"),
]


def _oracle_mx(w, ni, wfmt, logits=None):
    """The oracle's routing, encode and MX operands; a gate-projected workload routes on the given
    (GPU-exported) logits."""
    if logits is None:
        logits = ni["logits"] if "logits" in ni else oracle.gate_logits(ni["x"], ni["Wg"], w.dtype)
    rt = oracle.route(logits, w.k, w.capacity_factor)
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    bufq = oracle.mx_quantize(buf, oracle.MX_FP8, w.dtype)
    W1q = oracle.mx_quantize(ni["W1"], wfmt, w.dtype)
    W2q = oracle.mx_quantize(ni["W2"], wfmt, w.dtype)
    return logits, rt, bufq, W1q, W2q


@pytest.mark.parametrize("w", MXW, ids=lambda w: w.name)
def test_encode_mx_bit_exact(w):
    import combine_softmax_top_amd as moe
    print(f"[mx encode] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    ni = inputs_np(inp)
    logits, rt, bufq, _, _ = _oracle_mx(w, ni, oracle.MX_FP8)
    s = shape_of(w)
    C = rt["C"]
    b = moe.alloc_forward_mx(s)
    moe.moe_route(s, dev(logits), b["idx"], b["loc"], b["gates"], b["needed"], b["fill"], b["capacity"],
                  b["slot_route"], b["ws"])
    moe.moe_encode_mx(s, inp["x"].cuda(), b["idx"], b["loc"], b["fill"], b["capacity"], b["buf_codes"],
                      b["buf_scales"])
    torch.cuda.synchronize()
    assert int(b["capacity"].item()) == C
    assert np.array_equal(host(b["buf_codes"][: w.E * C]), bufq[0]), "buffer codes"
    assert np.array_equal(host(b["buf_scales"][: w.E * C]), bufq[1]), "buffer scales"


# The hardware's fp8 accumulation error, relative to the sum of the products' magnitudes
# (measured up to 2.2e-4 on random operands; 2^-11 = 4.9e-4 leaves room).
MFMA_FP8_REL = 2.0 ** -11


def _pre_slack(bufq, W1q, rows, C, wfmt, act):
    """Bound on |pre_gpu - pre_oracle| per h element, carried through the activation (slope
    <= 1.13 for GELU, 1 for ReLU): MFMA_FP8_REL * sum_m |x_m| |w_m|."""
    x = np.abs(oracle.mx_dequantize(bufq[0][rows], bufq[1][rows], oracle.MX_FP8))  # [n, M]
    w1 = np.abs(oracle.mx_dequantize(W1q[0], W1q[1], wfmt))                         # [E, H, M]
    e = np.asarray(rows) // C
    out = np.empty((len(rows), w1.shape[1]))
    for i in range(len(rows)):
        out[i] = w1[e[i]] @ x[i]
    return MFMA_FP8_REL * (1.13 if act == W.ACT_GELU else 1.0) * out


def _check_h(hc_g, hs_g, hq_o, what, slack):
    """h quantised on both sides from fp32 values that differ by at most `slack` (the fp8
    accumulation error): the codes agree almost everywhere, and the dequantised values differ
    by at most one quantisation step of the coarser block scale plus that slack. Returns
    |deq(h_gpu) - deq(h_oracle)| for the bound on y."""
    hc_o, hs_o = hq_o
    same_s = (hs_g == hs_o).mean()
    same_c = (hc_g == hc_o).mean()
    assert same_s >= 0.99 and same_c >= 0.99, f"{what}: scales agree {same_s:.5f}, codes {same_c:.5f}"
    dg = oracle.mx_dequantize(hc_g, hs_g, oracle.MX_FP8)
    do = oracle.mx_dequantize(hc_o, hs_o, oracle.MX_FP8)
    dh = np.abs(dg - do)
    # one E4M3 step of a value v is at most 2^-3 |v| (normal range) or the subnormal step 2^-9 X
    X = np.repeat(2.0 ** (np.maximum(hs_g, hs_o).astype(np.float64) - 127), 32, axis=-1)
    step = np.maximum(2.0 ** -3 * np.maximum(np.abs(dg), np.abs(do)), 2.0 ** -9 * X)
    bad = dh > step * (1 + 1e-12) + 2 * slack
    assert not bad.any(), (f"{what}: {bad.sum()} values differ by more than one quantisation step plus the "
                           f"accumulation slack (worst excess {(dh - step - 2 * slack).max():.3e})")
    return dh


def _y_extra(dh, rows, C, W2q, wfmt):
    """|dh| . |W2[e]|^T per row: how far the two sides' different h quantisations move y."""
    w2 = np.abs(oracle.mx_dequantize(W2q[0], W2q[1], wfmt))  # [E, M, H]
    e = np.asarray(rows) // C
    out = np.empty((len(rows), w2.shape[1]))
    for i in range(len(rows)):
        out[i] = w2[e[i]] @ dh[i]
    return out


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("w", MXW, ids=lambda w: w.name)
def test_expert_ffn_mx_matches_oracle(w, wfmt):
    import combine_softmax_top_amd as moe
    print(f"[mx ffn] {w.name} wfmt={wfmt}", flush=True)
    inp = W.make_inputs(w, seed=0)
    ni = inputs_np(inp)
    logits, rt, bufq, W1q, W2q = _oracle_mx(w, ni, wfmt)
    s = shape_of(w)
    C = rt["C"]
    cmax = moe.moe_capacity_bound(s)
    # the oracle's quantised operands on both sides (the quantiser is compared bit for bit above)
    bc = torch.zeros(w.E * cmax, w.M, dtype=torch.uint8)
    bs = torch.zeros(w.E * cmax, w.M // 32, dtype=torch.uint8)
    bc[: w.E * C] = torch.from_numpy(bufq[0])
    bs[: w.E * C] = torch.from_numpy(bufq[1])
    hc, hs = moe.mx_alloc((w.E * cmax, w.H), oracle.MX_FP8)
    y = torch.empty(w.E * cmax, w.M, dtype=torch.bfloat16, device="cuda")
    gq1 = tuple(torch.from_numpy(t).cuda() for t in W1q)
    gq2 = tuple(torch.from_numpy(t).cuda() for t in W2q)
    fill = dev(rt["fill"])
    cap = torch.tensor([C], dtype=torch.int32, device="cuda")
    b1g = inp["b1"].cuda() if "b1" in inp else None
    b2g = inp["b2"].cuda() if "b2" in inp else None
    moe.moe_expert_ffn_mx(s, wfmt, bc.cuda(), bs.cuda(), gq1, b1g, gq2, b2g, fill, cap, hc, hs, y)
    torch.cuda.synchronize()
    rows = oracle.filled_rows(rt)
    b1 = ni.get("b1")
    b2 = ni.get("b2")
    hq_o, y_o = oracle.expert_rows_mx(bufq, W1q, b1, W2q, b2, rows, C, w.act, wfmt, want_hq=True)
    ridx = torch.from_numpy(rows).cuda()
    dh = _check_h(host(hc[ridx]), host(hs[ridx]), hq_o, "h", _pre_slack(bufq, W1q, rows, C, wfmt, w.act))
    check_close(host(y[ridx]), y_o, w.dtype, "y", extra=_y_extra(dh, rows, C, W2q, wfmt))


@pytest.mark.parametrize("wfmt", FMTS)
@pytest.mark.parametrize("w", MXW, ids=lambda w: w.name)
def test_layer_forward_mx_matches_oracle(w, wfmt):
    import combine_softmax_top_amd as moe
    print(f"[mx layer] {w.name} wfmt={wfmt}", flush=True)
    inp = W.make_inputs(w, seed=0)
    ni = inputs_np(inp)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    W1g = moe.mx_quantize_weights(d["W1"], wfmt)
    W2g = moe.mx_quantize_weights(d["W2"], wfmt)
    b = moe.layer_forward_mx(s, wfmt, d["x"], W1g, d.get("b1"), W2g, d.get("b2"), logits=d.get("logits"),
                             Wg=d.get("Wg"))
    torch.cuda.synchronize()
    glog = None
    if "Wg" in ni:  # the projection within its fp32 bound; the oracle routes on the GPU's logits
        glog = host(b["logits"])
        check_logits(glog, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    logits, rt, bufq, W1q, W2q = _oracle_mx(w, ni, wfmt, logits=glog)
    assert np.array_equal(host(W1g[0]), W1q[0]) and np.array_equal(host(W1g[1]), W1q[1])
    C = rt["C"]
    g = dict(idx=host(b["idx"]), loc=host(b["loc"]), gates=host(b["gates"]), needed=host(b["needed"]),
             fill=host(b["fill"]), C=int(b["capacity"].item()), slot_route=host(b["slot_route"][: w.E * C]))
    compare_route(g, rt, w.E)
    rows = oracle.filled_rows(rt)
    hq_o, y_o = oracle.expert_rows_mx(bufq, W1q, ni.get("b1"), W2q, ni.get("b2"), rows, C, w.act, wfmt,
                                      want_hq=True)
    ridx = torch.from_numpy(rows).cuda()
    dh = _check_h(host(b["h_codes"][ridx]), host(b["h_scales"][ridx]), hq_o, "h",
                  _pre_slack(bufq, W1q, rows, C, wfmt, w.act))
    ey = _y_extra(dh, rows, C, W2q, wfmt)
    yg = host(b["y"][ridx])
    check_close(yg, y_o, w.dtype, "y", extra=ey)
    y_full = np.zeros((w.E * C, w.M), np.uint16)
    y_full[rows] = y_o
    out_o = oracle.decode(y_full, rt, w.E, w.dtype)
    check_close(host(b["out"]), out_o, w.dtype, "out", extra=decode_extra(rt, rows, yg, y_o))


@pytest.mark.parametrize("wfmt", FMTS)
def test_mx_full_size_gated_layer(wfmt):
    # the gated workload's layer with MX experts, sampled rows and tokens
    import combine_softmax_top_amd as moe
    w = W.GATED_BF16
    print(f"[mx full size] {w.name} wfmt={wfmt}", flush=True)
    rng = np.random.default_rng(77)
    inp = W.make_inputs(w, seed=0, device="cuda")
    s = shape_of(w)
    W1g = moe.mx_quantize_weights(inp["W1"], wfmt)
    W2g = moe.mx_quantize_weights(inp["W2"], wfmt)
    b = moe.layer_forward_mx(s, wfmt, inp["x"], W1g, inp["b1"], W2g, inp["b2"], Wg=inp["Wg"])
    torch.cuda.synchronize()
    ni = {k_: host(v) for k_, v in inp.items()}
    logits = host(b["logits"])
    check_logits(logits, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    rt = oracle.route(logits, w.k, w.capacity_factor)
    C = rt["C"]
    W1q = (host(W1g[0]), host(W1g[1]))
    W2q = (host(W2g[0]), host(W2g[1]))
    wq1 = oracle.mx_quantize(ni["W1"][:2], wfmt, w.dtype)  # spot check of the weight quantisation
    assert np.array_equal(W1q[0][:2], wq1[0]) and np.array_equal(W1q[1][:2], wq1[1])
    toks = np.sort(rng.choice(w.S, size=48, replace=False))
    rows = sorted({int(rt["idx"][r, t]) * C + int(rt["loc"][r, t]) for r in range(w.k) for t in toks
                   if rt["loc"][r, t] < C})
    rows = np.asarray(rows, np.int64)
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    bufq = oracle.mx_quantize(buf, oracle.MX_FP8, w.dtype)
    hq_o, y_o = oracle.expert_rows_mx(bufq, W1q, ni["b1"], W2q, ni["b2"], rows, C, w.act, wfmt, want_hq=True)
    ridx = torch.from_numpy(rows).cuda()
    dh = _check_h(host(b["h_codes"][ridx]), host(b["h_scales"][ridx]), hq_o, "h (sampled rows)",
                  _pre_slack(bufq, W1q, rows, C, wfmt, w.act))
    ey = _y_extra(dh, rows, C, W2q, wfmt)
    yg = host(b["y"][ridx])
    check_close(yg, y_o, w.dtype, "y (sampled rows)", extra=ey)
    y_full = np.zeros((w.E * C, w.M), np.uint16)
    y_full[rows] = y_o
    out_o = oracle.decode(y_full, rt, w.E, w.dtype, tokens=toks)
    eo = decode_extra(rt, rows, yg, y_o, tokens=toks)
    check_close(host(b["out"][torch.from_numpy(toks).cuda()]), out_o, w.dtype, "out (sampled tokens)", extra=eo)
