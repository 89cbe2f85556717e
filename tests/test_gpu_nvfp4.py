"""GPU parity of the NVFP4 experts (weight-only: E2M1 weights in 16-value blocks with E4M3 block
scales and an fp32 scale per expert matrix, bf16 tokens) against the CPU oracle.

The quantiser takes every decision (the tensor's amax and g, each block's E4M3 scale, the E2M1
codes) from the same inputs in the same fp32 operations on both sides, so it is compared bit for
bit. The expert FFN multiplies bf16 tokens by the weights' exact values (each is a bf16 number),
so it follows the bf16 FFN's tolerance rule against the oracle's fp64 sums.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_helpers import host

pytestmark = pytest.mark.gpu


def _source(T, R, K, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(T, R, K, generator=g) * torch.exp(torch.empty(T, R, 1).uniform_(-6, 6, generator=g))
    if R >= 4 and K >= 32:
        a[0, 1, :16] = 0.0                 # an all-zero block
        a[0, 2, 16:32] = 0.0; a[0, 2, 20] = -0.0
        a[0, 3, :16] = 2.0 ** 3            # every element at the block's amax
    if T >= 2:
        a[1] *= 1e-30                      # a tensor of tiny values
    if T >= 3:
        a[2] = 0.0                         # an all-zero tensor: g = 0
    return a.to(torch.float32 if dtype == W.DT_F32 else torch.bfloat16)


@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16])
@pytest.mark.parametrize("T,R,K", [(3, 40, 64), (1, 1, 16), (4, 96, 1024), (2, 0, 32), (8, 256, 512)])
def test_nvfp4_quantize_bit_exact(dtype, T, R, K):
    import combine_softmax_top_amd as moe
    print(f"[nvfp4 quantize] dtype={dtype} T={T} R={R} K={K}", flush=True)
    a = _source(T, R, K, dtype, 3 + T * R + K)
    want_c, want_s, want_g = oracle.nvfp4_quantize(host(a), dtype)
    codes = torch.empty(T, R, K // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(T, R, K // 16, dtype=torch.uint8, device="cuda")
    g = torch.empty(T, dtype=torch.float32, device="cuda")
    moe.moe_nvfp4_quantize(a.cuda(), T, codes, scales, g, dtype=dtype)
    torch.cuda.synchronize()
    if R == 0:
        return
    assert np.array_equal(host(g).view(np.uint32), want_g.view(np.uint32)), "g"
    assert np.array_equal(host(scales), want_s), "scales"
    assert np.array_equal(host(codes), want_c), "codes"


from tests.gpu_helpers import check_close, check_logits, compare_route, decode_extra, dev, inputs_np, shape_of  # noqa: E402

NVW = [
    W.Workload("nv_S1000_M256_E8_k2_H384", S=1000, M=256, E=8, k=2, H=384, capacity_factor=1.25),
    W.Workload("nv_S129_M64_E3_k2_H192", S=129, M=64, E=3, k=2, H=192, capacity_factor=1.0),
    W.Workload("nv_relu_nobias_S300_M384_E4_k1_H640", S=300, M=384, E=4, k=1, H=640, capacity_factor=0.75,
               act=W.ACT_RELU, has_fc1_bias=False, has_fc2_bias=False),
    W.Workload("nv_gate_S600_M1024_E4_k2_H1152", S=600, M=1024, E=4, k=2, H=1152, capacity_factor=1.0,
               logits="gate"),
]


def _oracle_nv(w, ni, logits=None):
    """The oracle's routing, encode and NVFP4 weights; a gate-projected workload routes on the
    given (GPU-exported) logits."""
    if logits is None:
        logits = ni["logits"] if "logits" in ni else oracle.gate_logits(ni["x"], ni["Wg"], w.dtype)
    rt = oracle.route(logits, w.k, w.capacity_factor)
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    return logits, rt, buf, oracle.nvfp4_quantize(ni["W1"], w.dtype), oracle.nvfp4_quantize(ni["W2"], w.dtype)


@pytest.mark.parametrize("w", NVW, ids=lambda w: w.name)
def test_expert_ffn_nvfp4_matches_oracle(w):
    import combine_softmax_top_amd as moe
    print(f"[nvfp4 ffn] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=1)
    ni = inputs_np(inp)
    _, rt, buf_o, W1q, W2q = _oracle_nv(w, ni)
    s = shape_of(w)
    C = rt["C"]
    cmax = moe.moe_capacity_bound(s)
    buf = torch.zeros(w.E * cmax, w.M, dtype=torch.bfloat16, device="cuda")
    buf[: w.E * C] = dev(buf_o)
    gq1 = tuple(torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in W1q)
    gq2 = tuple(torch.from_numpy(np.ascontiguousarray(t)).cuda() for t in W2q)
    pre = torch.empty(w.E * cmax, w.H, dtype=torch.bfloat16, device="cuda")
    h = torch.empty_like(pre)
    y = torch.empty(w.E * cmax, w.M, dtype=torch.bfloat16, device="cuda")
    fill = dev(rt["fill"])
    cap = torch.tensor([C], dtype=torch.int32, device="cuda")
    b1g = inp["b1"].cuda() if "b1" in inp else None
    b2g = inp["b2"].cuda() if "b2" in inp else None
    moe.moe_expert_ffn_nvfp4(s, buf, gq1, b1g, gq2, b2g, fill, cap, pre, h, y)
    torch.cuda.synchronize()
    rows = oracle.filled_rows(rt)
    pre_o, h_o, y_o = oracle.expert_rows_nvfp4(buf_o, W1q, ni.get("b1"), W2q, ni.get("b2"), rows, C, w.act)
    ridx = torch.from_numpy(rows).cuda()
    check_close(host(pre[ridx]), pre_o, w.dtype, "pre")
    check_close(host(h[ridx]), h_o, w.dtype, "h")
    check_close(host(y[ridx]), y_o, w.dtype, "y")
    # the two halves as calls of their own give the same bits
    h2 = torch.empty_like(h)
    y2 = torch.empty_like(y)
    moe.moe_expert_fc1_nvfp4(s, buf, gq1, b1g, fill, cap, None, h2)
    moe.moe_expert_fc2_nvfp4(s, h2, gq2, b2g, fill, cap, y2)
    torch.cuda.synchronize()
    assert torch.equal(h2[ridx].view(torch.int16), h[ridx].view(torch.int16))
    assert torch.equal(y2[ridx].view(torch.int16), y[ridx].view(torch.int16))


@pytest.mark.parametrize("w", NVW, ids=lambda w: w.name)
def test_layer_forward_nvfp4_matches_oracle(w):
    import combine_softmax_top_amd as moe
    print(f"[nvfp4 layer] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=0)
    ni = inputs_np(inp)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    W1g = moe.nvfp4_quantize_weights(d["W1"])
    W2g = moe.nvfp4_quantize_weights(d["W2"])
    b = moe.layer_forward_nvfp4(s, d["x"], W1g, d.get("b1"), W2g, d.get("b2"), logits=d.get("logits"),
                                Wg=d.get("Wg"))
    torch.cuda.synchronize()
    glog = None
    if "Wg" in ni:  # the projection within its fp32 bound; the oracle routes on the GPU's logits
        glog = host(b["logits"])
        check_logits(glog, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    _, rt, buf_o, W1q, W2q = _oracle_nv(w, ni, logits=glog)
    for got, want in zip(W1g + W2g, W1q + W2q):
        assert np.array_equal(host(got).reshape(-1).view(np.uint8), np.ascontiguousarray(want).reshape(-1).view(np.uint8))
    C = rt["C"]
    g = dict(idx=host(b["idx"]), loc=host(b["loc"]), gates=host(b["gates"]), needed=host(b["needed"]),
             fill=host(b["fill"]), C=int(b["capacity"].item()), slot_route=host(b["slot_route"][: w.E * C]))
    compare_route(g, rt, w.E)
    assert np.array_equal(host(b["buf"][: w.E * C]), buf_o)
    rows = oracle.filled_rows(rt)
    _, h_o, y_o = oracle.expert_rows_nvfp4(buf_o, W1q, ni.get("b1"), W2q, ni.get("b2"), rows, C, w.act)
    ridx = torch.from_numpy(rows).cuda()
    check_close(host(b["h"][ridx]), h_o, w.dtype, "h")
    yg = host(b["y"][ridx])
    check_close(yg, y_o, w.dtype, "y")
    y_full = np.zeros((w.E * C, w.M), np.uint16)
    y_full[rows] = y_o
    out_o = oracle.decode(y_full, rt, w.E, w.dtype)
    check_close(host(b["out"]), out_o, w.dtype, "out", extra=decode_extra(rt, rows, yg, y_o))


# The gated workload's layer (S=4096, M=1024, E=8, k=2, H=4096) with NVFP4 experts, and the
# same layer with H=1536: the products' tile choice takes 192 x 256 tiles for the first
# (fc1 and fc2) and 256 x 256 tiles for the second's fc1.
FULL = [W.GATED_BF16, W.GATED_BF16.replace(name="gated_bf16_S4096_M1024_E8_k2_H1536", H=1536)]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_nvfp4_full_size_gated_layer(w):
    # sampled rows and tokens
    import combine_softmax_top_amd as moe
    print(f"[nvfp4 full size] {w.name}", flush=True)
    rng = np.random.default_rng(79)
    inp = W.make_inputs(w, seed=0, device="cuda")
    s = shape_of(w)
    W1g = moe.nvfp4_quantize_weights(inp["W1"])
    W2g = moe.nvfp4_quantize_weights(inp["W2"])
    b = moe.layer_forward_nvfp4(s, inp["x"], W1g, inp["b1"], W2g, inp["b2"], Wg=inp["Wg"])
    torch.cuda.synchronize()
    ni = {k_: host(v) for k_, v in inp.items()}
    logits = host(b["logits"])
    check_logits(logits, oracle.gate_logits(ni["x"], ni["Wg"], w.dtype), ni["x"], ni["Wg"])
    rt = oracle.route(logits, w.k, w.capacity_factor)
    C = rt["C"]
    W1q = tuple(host(t) for t in W1g)
    W2q = tuple(host(t) for t in W2g)
    wq1 = oracle.nvfp4_quantize(ni["W1"][:1], w.dtype)  # spot check of the weights (expert 0)
    assert np.array_equal(W1q[0][:1], wq1[0]) and np.array_equal(W1q[1][:1], wq1[1])
    assert W1q[2][0].view(np.uint32) == wq1[2].view(np.uint32)[0]
    toks = np.sort(rng.choice(w.S, size=48, replace=False))
    rows = np.asarray(sorted({int(rt["idx"][r, t]) * C + int(rt["loc"][r, t]) for r in range(w.k) for t in toks
                              if rt["loc"][r, t] < C}), np.int64)
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    ridx = torch.from_numpy(rows).cuda()
    assert np.array_equal(host(b["buf"][ridx]), buf[rows])
    _, h_o, y_o = oracle.expert_rows_nvfp4(buf, W1q, ni["b1"], W2q, ni["b2"], rows, C, w.act)
    check_close(host(b["h"][ridx]), h_o, w.dtype, "h (sampled rows)")
    yg = host(b["y"][ridx])
    check_close(yg, y_o, w.dtype, "y (sampled rows)")
    y_full = np.zeros((w.E * C, w.M), np.uint16)
    y_full[rows] = y_o
    out_o = oracle.decode(y_full, rt, w.E, w.dtype, tokens=toks)
    eo = decode_extra(rt, rows, yg, y_o, tokens=toks)
    check_close(host(b["out"][torch.from_numpy(toks).cuda()]), out_o, w.dtype, "out (sampled tokens)", extra=eo)


def test_layer_forward_nvfp4_empty_input():
    # S = 0: every expert buffer row is padding (zeros) and nothing else is written
    import combine_softmax_top_amd as moe
    w = W.Workload("nv_empty", S=0, M=256, E=3, k=2, H=128, capacity_factor=1.0)
    inp = W.make_inputs(w, seed=0)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    W1g = moe.nvfp4_quantize_weights(d["W1"])
    W2g = moe.nvfp4_quantize_weights(d["W2"])
    bufs = moe.alloc_forward(s)
    bufs["buf"].fill_(7.0)
    b = moe.layer_forward_nvfp4(s, d["x"], W1g, d.get("b1"), W2g, d.get("b2"), logits=d["logits"], bufs=bufs)
    torch.cuda.synchronize()
    assert int(b["capacity"].item()) == 1 and b["out"].numel() == 0
    assert (host(b["buf"][:3]).view(np.uint16) == 0).all()


def test_layer_forward_nvfp4_idle_experts():
    # 16 experts for 24 top-1 tokens: most experts get no row, the others a partial tile
    import combine_softmax_top_amd as moe
    w = W.Workload("nv_idle_S24_M64_E16_k1_H128", S=24, M=64, E=16, k=1, H=128, capacity_factor=1.0)
    print(f"[nvfp4 idle experts] {w.name}", flush=True)
    inp = W.make_inputs(w, seed=3)
    ni = inputs_np(inp)
    s = shape_of(w)
    d = {k_: v.cuda() for k_, v in inp.items()}
    W1g = moe.nvfp4_quantize_weights(d["W1"])
    W2g = moe.nvfp4_quantize_weights(d["W2"])
    b = moe.layer_forward_nvfp4(s, d["x"], W1g, d.get("b1"), W2g, d.get("b2"), logits=d["logits"])
    torch.cuda.synchronize()
    _, rt, buf_o, W1q, W2q = _oracle_nv(w, ni)
    assert (rt["fill"] == 0).sum() >= 4
    C = rt["C"]
    rows = oracle.filled_rows(rt)
    _, h_o, y_o = oracle.expert_rows_nvfp4(buf_o, W1q, ni.get("b1"), W2q, ni.get("b2"), rows, C, w.act)
    ridx = torch.from_numpy(rows).cuda()
    check_close(host(b["h"][ridx]), h_o, w.dtype, "h")
    yg = host(b["y"][ridx])
    check_close(yg, y_o, w.dtype, "y")
    y_full = np.zeros((w.E * C, w.M), np.uint16)
    y_full[rows] = y_o
    out_o = oracle.decode(y_full, rt, w.E, w.dtype)
    check_close(host(b["out"]), out_o, w.dtype, "out", extra=decode_extra(rt, rows, yg, y_o))
