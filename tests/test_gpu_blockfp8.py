"""GPU parity of the block-wise FP8 experts (E4M3 codes, fp32 scales per 128 x 128 weight block
and per 1 x 128 token block) against the CPU oracle.

The quantiser and the encode take their decisions (amax, the fp32 scale, the codes) from the same
inputs on both sides, so they are compared bit for bit. The expert FFN's h is quantised from fp32
values that the two sides reach by different summation orders (and the hardware's fp8
accumulation drops low-order bits of small products), so its scales differ by that much and its
codes may differ by one step at a rounding boundary: the codes must agree almost everywhere and
the dequantised values within one step plus the accumulation bound; y and the layer output follow
the bf16 tolerance rule with the h differences carried through W2.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import check_close, check_logits, compare_route, decode_extra, dev, host, inputs_np, shape_of
from tests.test_gpu_mx import MFMA_FP8_REL, MXW

pytestmark = pytest.mark.gpu


def _source(rows, K, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(rows, K, generator=g) * torch.exp(torch.empty(rows, 1).uniform_(-8, 8, generator=g))
    if rows >= 128:
        a[:128, :128] = 0.0          # an all-zero block (both block shapes)
        a[3, 5] = -0.0
    if rows >= 256 and K >= 256:
        a[130, 128:256] = 2.0 ** 5   # every element at amax
        a[131, 128:256] = -(2.0 ** 5)
    return a.to(torch.float32 if dtype == W.DT_F32 else torch.bfloat16)


@pytest.mark.parametrize("brows", [1, 128])
@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16])
@pytest.mark.parametrize("rows,K", [(384, 256), (128, 128), (0, 128), (640, 1152)])
def test_blockfp8_quantize_bit_exact(brows, dtype, rows, K):
    import combine_softmax_top_amd as moe
    print(f"[blockfp8 quantize] brows={brows} dtype={dtype} rows={rows} K={K}", flush=True)
    a = _source(rows, K, dtype, 5 + rows)
    want_c, want_s = oracle.blockfp8_quantize(host(a), brows, dtype)
    codes, scales = moe.blockfp8_alloc((rows, K), brows)
    moe.moe_blockfp8_quantize(a.cuda(), brows, codes, scales, dtype=dtype)
    torch.cuda.synchronize()
    assert np.array_equal(host(codes), want_c), "codes"
    assert np.array_equal(host(scales).view(np.uint32), want_s.view(np.uint32)), "scales"


def test_blockfp8_quantize_rows_of_one():
    # 1 x 128 blocks of a single row, and odd row counts
    import combine_softmax_top_amd as moe
    for rows in (1, 7):
        a = _source(rows, 384, W.DT_BF16, 11)
        want_c, want_s = oracle.blockfp8_quantize(host(a), 1, W.DT_BF16)
        codes, scales = moe.blockfp8_alloc((rows, 384), 1)
        moe.moe_blockfp8_quantize(a.cuda(), 1, codes, scales)
        torch.cuda.synchronize()
        assert np.array_equal(host(codes), want_c) and np.array_equal(host(scales), want_s)


def _oracle_blk(w, ni, logits=None):
    """The oracle's routing, encode and block-FP8 operands; a gate-projected workload routes on
    the given (GPU-exported) logits."""
    if logits is None:
        logits = ni["logits"] if "logits" in ni else oracle.gate_logits(ni["x"], ni["Wg"], w.dtype)
    rt = oracle.route(logits, w.k, w.capacity_factor)
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    bufq = oracle.blockfp8_quantize(buf, 1, w.dtype)
    W1q = oracle.blockfp8_quantize(ni["W1"], oracle.BLOCK, w.dtype)
    W2q = oracle.blockfp8_quantize(ni["W2"], oracle.BLOCK, w.dtype)
    return logits, rt, bufq, W1q, W2q


@pytest.mark.parametrize("w", MXW, ids=lambda w: w.name)
def test_encode_blockfp8_bit_exact(w):
    import combine_softmax_top_amd as moe
    print(f"[blockfp8 encode] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    ni = inputs_np(inp)
    logits, rt, bufq, _, _ = _oracle_blk(w, ni)
    s = shape_of(w)
    C = rt["C"]
    b = moe.alloc_forward_blockfp8(s)
    moe.moe_route(s, dev(logits), b["idx"], b["loc"], b["gates"], b["needed"], b["fill"], b["capacity"],
                  b["slot_route"], b["ws"])
    moe.moe_encode_blockfp8(s, inp["x"].cuda(), b["idx"], b["loc"], b["fill"], b["capacity"], b["buf_codes"],
                            b["buf_scales"])
    torch.cuda.synchronize()
    assert int(b["capacity"].item()) == C
    assert np.array_equal(host(b["buf_codes"][: w.E * C]), bufq[0]), "buffer codes"
    assert np.array_equal(host(b["buf_scales"][: w.E * C]).view(np.uint32), bufq[1].view(np.uint32)), "scales"


def _pre_slack(bufq, W1q, rows, C, act):
    """Bound on |pre_gpu - pre_oracle| per h element, carried through the activation (slope <= 1.13
    for GELU, 1 for ReLU): the fp8 accumulation within each block plus the fp32 rescales,
    (MFMA_FP8_REL + 2^-20) * sum_m |x_m| |w_m|."""
    x = np.abs(oracle.blockfp8_dequantize(bufq[0][rows], bufq[1][rows], 1))
    w1 = np.abs(oracle.blockfp8_dequantize(W1q[0], W1q[1], oracle.BLOCK))  # [E, H, M]
    e = np.asarray(rows) // C
    out = np.empty((len(rows), w1.shape[1]))
    for i in range(len(rows)):
        out[i] = w1[e[i]] @ x[i]
    return (MFMA_FP8_REL + 2.0 ** -20) * (1.13 if act == W.ACT_GELU else 1.0) * out


def _check_h(hc_g, hs_g, hq_o, what, slack):
    """h quantised on both sides from fp32 values within `slack` of each other: the block scales
    agree to the amax's slack, the codes almost everywhere, the dequantised values within one E4M3
    step plus twice the slack plus the scales' difference times the largest code. Returns
    |deq(h_gpu) - deq(h_oracle)| for the bound on y."""
    hc_o, hs_o = hq_o
    blk_slack = slack.reshape(slack.shape[0], -1, 128).max(axis=2)
    ds = np.abs(hs_g.astype(np.float64) - hs_o.astype(np.float64))
    assert (ds <= blk_slack / 448.0 * 1.01 + 2.0 ** -23 * np.abs(hs_o)).all(), f"{what}: scales"
    same_c = (hc_g == hc_o).mean()
    assert same_c >= 0.98, f"{what}: codes agree {same_c:.5f}"
    dg = oracle.blockfp8_dequantize(hc_g, hs_g, 1)
    do = oracle.blockfp8_dequantize(hc_o, hs_o, 1)
    dh = np.abs(dg - do)
    smax = np.repeat(np.maximum(hs_g, hs_o).astype(np.float64), 128, axis=-1)
    step = np.maximum(2.0 ** -3 * np.maximum(np.abs(dg), np.abs(do)), 2.0 ** -9 * smax)
    bound = step * (1 + 1e-12) + 2 * slack + 448.0 * np.repeat(ds, 128, axis=-1)
    bad = dh > bound
    assert not bad.any(), f"{what}: {bad.sum()} values beyond one step (worst excess {(dh - bound).max():.3e})"
    return dh


def _y_extra(dh, rows, C, W2q):
    w2 = np.abs(oracle.blockfp8_dequantize(W2q[0], W2q[1], oracle.BLOCK))  # [E, M, H]
    e = np.asarray(rows) // C
    out = np.empty((len(rows), w2.shape[1]))
    for i in range(len(rows)):
        out[i] = w2[e[i]] @ dh[i]
    return out


@pytest.mark.parametrize("w", MXW, ids=lambda w: w.name)
def test_expert_ffn_blockfp8_matches_oracle(w):
    import combine_softmax_top_amd as moe
    print(f"[blockfp8 ffn] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    ni = inputs_np(inp)
    logits, rt, bufq, W1q, W2q = _oracle_blk(w, ni)
    s = shape_of(w)
    C = rt["C"]
    cmax = moe.moe_capacity_bound(s)
    # the oracle's quantised operands on both sides (the quantiser is compared bit for bit above)
    bc = torch.zeros(w.E * cmax, w.M, dtype=torch.uint8)
    bs = torch.zeros(w.E * cmax, w.M // 128, dtype=torch.float32)
    bc[: w.E * C] = torch.from_numpy(bufq[0])
    bs[: w.E * C] = torch.from_numpy(bufq[1])
    hc, hs = moe.blockfp8_alloc((w.E * cmax, w.H), 1)
    y = torch.empty(w.E * cmax, w.M, dtype=torch.bfloat16, device="cuda")
    gq1 = tuple(torch.from_numpy(t).cuda() for t in W1q)
    gq2 = tuple(torch.from_numpy(t).cuda() for t in W2q)
    fill = dev(rt["fill"])
    cap = torch.tensor([C], dtype=torch.int32, device="cuda")
    b1g = inp["b1"].cuda() if "b1" in inp else None
    b2g = inp["b2"].cuda() if "b2" in inp else None
    moe.moe_expert_ffn_blockfp8(s, bc.cuda(), bs.cuda(), gq1, b1g, gq2, b2g, fill, cap, hc, hs, y)
    torch.cuda.synchronize()
    rows = oracle.filled_rows(rt)
    hq_o, y_o = oracle.expert_rows_blockfp8(bufq, W1q, ni.get("b1"), W2q, ni.get("b2"), rows, C, w.act,
                                            want_hq=True)
    ridx = torch.from_numpy(rows).cuda()
    dh = _check_h(host(hc[ridx]), host(hs[ridx]), hq_o, "h", _pre_slack(bufq, W1q, rows, C, w.act))
    check_close(host(y[ridx]), y_o, w.dtype, "y", extra=_y_extra(dh, rows, C, W2q))
    # the two halves as calls of their own give the same bits
    hc2, hs2 = moe.blockfp8_alloc((w.E * cmax, w.H), 1)
    y2 = torch.empty_like(y)
    moe.moe_expert_fc1_blockfp8(s, bc.cuda(), bs.cuda(), gq1, b1g, fill, cap, hc2, hs2)
    moe.moe_expert_fc2_blockfp8(s, hc2, hs2, gq2, b2g, fill, cap, y2)
    torch.cuda.synchronize()
    assert torch.equal(hc2[ridx], hc[ridx]) and torch.equal(hs2[ridx], hs[ridx])
    assert torch.equal(y2[ridx].view(torch.int16), y[ridx].view(torch.int16))


@pytest.mark.parametrize("w", MXW, ids=lambda w: w.name)
def test_layer_forward_blockfp8_matches_oracle(w):
    import combine_softmax_top_amd as moe
    print(f"[blockfp8 layer] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    ni = inputs_np(inp)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    W1g = moe.blockfp8_quantize_weights(d["W1"])
    W2g = moe.blockfp8_quantize_weights(d["W2"])
    b = moe.layer_forward_blockfp8(s, d["x"], W1g, d.get("b1"), W2g, d.get("b2"), logits=d.get("logits"),
                                   Wg=d.get("Wg"))
    torch.cuda.synchronize()
    glog = None
    if "Wg" in ni:  # the projection within its fp32 bound; the oracle routes on the GPU's logits
        glog = host(b["logits"])
        check_logits(glog, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    logits, rt, bufq, W1q, W2q = _oracle_blk(w, ni, logits=glog)
    assert np.array_equal(host(W1g[0]), W1q[0]) and np.array_equal(host(W1g[1]), W1q[1])
    assert np.array_equal(host(W2g[0]), W2q[0]) and np.array_equal(host(W2g[1]), W2q[1])
    C = rt["C"]
    g = dict(idx=host(b["idx"]), loc=host(b["loc"]), gates=host(b["gates"]), needed=host(b["needed"]),
             fill=host(b["fill"]), C=int(b["capacity"].item()), slot_route=host(b["slot_route"][: w.E * C]))
    compare_route(g, rt, w.E)
    assert np.array_equal(host(b["buf_codes"][: w.E * C]), bufq[0])
    rows = oracle.filled_rows(rt)
    hq_o, y_o = oracle.expert_rows_blockfp8(bufq, W1q, ni.get("b1"), W2q, ni.get("b2"), rows, C, w.act,
                                            want_hq=True)
    ridx = torch.from_numpy(rows).cuda()
    dh = _check_h(host(b["h_codes"][ridx]), host(b["h_scales"][ridx]), hq_o, "h",
                  _pre_slack(bufq, W1q, rows, C, w.act))
    yg = host(b["y"][ridx])
    check_close(yg, y_o, w.dtype, "y", extra=_y_extra(dh, rows, C, W2q))
    y_full = np.zeros((w.E * C, w.M), np.uint16)
    y_full[rows] = y_o
    out_o = oracle.decode(y_full, rt, w.E, w.dtype)
    check_close(host(b["out"]), out_o, w.dtype, "out", extra=decode_extra(rt, rows, yg, y_o))


def test_blockfp8_full_size_gated_layer():
    # the gated workload's layer with block-FP8 experts, sampled rows and tokens
    import combine_softmax_top_amd as moe
    w = W.GATED_BF16
    print(f"[blockfp8 full size] {w.name}", flush=True)
    rng = np.random.default_rng(78)
    inp = W.make_inputs(w, seed=0, device="cuda")
    s = shape_of(w)
    W1g = moe.blockfp8_quantize_weights(inp["W1"])
    W2g = moe.blockfp8_quantize_weights(inp["W2"])
    b = moe.layer_forward_blockfp8(s, inp["x"], W1g, inp["b1"], W2g, inp["b2"], Wg=inp["Wg"])
    torch.cuda.synchronize()
    ni = {k_: host(v) for k_, v in inp.items()}
    logits = host(b["logits"])
    check_logits(logits, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    rt = oracle.route(logits, w.k, w.capacity_factor)
    C = rt["C"]
    W1q = (host(W1g[0]), host(W1g[1]))
    W2q = (host(W2g[0]), host(W2g[1]))
    wq1 = oracle.blockfp8_quantize(ni["W1"][:1], oracle.BLOCK, w.dtype)  # spot check of the weights
    assert np.array_equal(W1q[0][:1], wq1[0]) and np.array_equal(W1q[1][:1], wq1[1])
    toks = np.sort(rng.choice(w.S, size=48, replace=False))
    rows = np.asarray(sorted({int(rt["idx"][r, t]) * C + int(rt["loc"][r, t]) for r in range(w.k) for t in toks
                              if rt["loc"][r, t] < C}), np.int64)
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    bufq = oracle.blockfp8_quantize(buf, 1, w.dtype)
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(b["buf_codes"][ridx]), bufq[0][rows])
    hq_o, y_o = oracle.expert_rows_blockfp8(bufq, W1q, ni["b1"], W2q, ni["b2"], rows, C, w.act, want_hq=True)
    dh = _check_h(host(b["h_codes"][ridx]), host(b["h_scales"][ridx]), hq_o, "h (sampled rows)",
                  _pre_slack(bufq, W1q, rows, C, w.act))
    yg = host(b["y"][ridx])
    check_close(yg, y_o, w.dtype, "y (sampled rows)", extra=_y_extra(dh, rows, C, W2q))
    y_full = np.zeros((w.E * C, w.M), np.uint16)
    y_full[rows] = y_o
    out_o = oracle.decode(y_full, rt, w.E, w.dtype, tokens=toks)
    eo = decode_extra(rt, rows, yg, y_o, tokens=toks)
    check_close(host(b["out"][torch.from_numpy(toks).cuda()]), out_o, w.dtype, "out (sampled tokens)", extra=eo)


def test_layer_forward_blockfp8_empty_input():
    # S = 0: every expert buffer row is padding (codes 0, scale 0) and nothing else is written
    import combine_softmax_top_amd as moe
    w = W.Workload("blk_empty", S=0, M=256, E=3, k=2, H=128, capacity_factor=1.0)
    inp = W.make_inputs(w, seed=0)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    W1g = moe.blockfp8_quantize_weights(d["W1"])
    W2g = moe.blockfp8_quantize_weights(d["W2"])
    bufs = moe.alloc_forward_blockfp8(s)
    bufs["buf_codes"].fill_(0xAB)
    bufs["buf_scales"].fill_(1.0)
    b = moe.layer_forward_blockfp8(s, d["x"], W1g, d.get("b1"), W2g, d.get("b2"), logits=d["logits"], bufs=bufs)
    torch.cuda.synchronize()
    assert int(b["capacity"].item()) == 1 and b["out"].numel() == 0
    assert (host(b["buf_codes"][:3]) == 0).all() and (host(b["buf_scales"][:3]) == 0).all()
