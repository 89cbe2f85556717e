"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test ties one oracle function to something other than itself: a hand-derived
value from the pages' statements, a closed form, a library routine on a special
case, an invariant, or brute force on tiny inputs. The pages print no worked
numeric example for this path, so there are no printed values to pin to.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import workloads as W
from tests.helpers import (bf16_bits_of_f32, dense_combine, dense_dispatch, f32_of, np_of, onehot_mask,
                           to_dtype_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- scalar roundings

def test_bf16_rounding_single_rounding_and_ties():
    # ties go to even: 1 + 2^-8 is halfway between 1 and 1 + 2^-7
    assert oracle.f64_to_bf16(1.0 + 2 ** -8) == 0x3F80
    assert oracle.f64_to_bf16(1.0 + 3 * 2 ** -8) == 0x3F82
    # just above the tie by less than half an fp32 ulp: a double rounding through fp32
    # would land on the tie and go down; a single rounding goes up.
    assert oracle.f64_to_bf16(1.0 + 2 ** -8 + 2 ** -30) == 0x3F81
    assert oracle.f64_to_bf16(-(1.0 + 2 ** -8 + 2 ** -30)) == 0xBF81
    # on fp32-representable values it equals torch's fp32 -> bf16 conversion
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    want = bf16_bits_of_f32(v)
    got = np.array([oracle.f64_to_bf16(float(a)) for a in v], np.uint16)
    assert np.array_equal(got, want)


def test_activation_matches_library():
    v = np.linspace(-6, 6, 241)
    t = torch.from_numpy(v).requires_grad_(True)
    g = torch.nn.functional.gelu(t)  # exact erf form
    (dg,) = torch.autograd.grad(g.sum(), t)
    g = g.detach()
    for i, a in enumerate(v):
        assert oracle.act(W.ACT_GELU, a) == pytest.approx(float(g[i]), abs=1e-15)
        assert oracle.act_grad(W.ACT_GELU, a) == pytest.approx(float(dg[i]), abs=1e-14)
        assert oracle.act(W.ACT_RELU, a) == max(a, 0.0)
        assert oracle.act_grad(W.ACT_RELU, a) == (1.0 if a > 0 else 0.0)


# ---------------------------------------------------------------- gate projection

def _gate_case(x_vals, w_vals):
    """One token, one expert: x (exactly representable in bf16) and the Wg column."""
    x = bf16_bits_of_f32(np.asarray(x_vals, np.float32)[None, :])
    Wg = np.asarray(w_vals, np.float32)[:, None]
    return x, Wg


def test_gate_logits_sum_in_increasing_m():
    # The plain definition: one fp64 sum over m from 0 upward, rounded once. The
    # products are +2^30 at m = 0, 2^-23 at m = 64..126 (63 terms) and -2^30 at
    # m = 128, all others 0; the exact sum is 63 * 2^-23. Summed upward, each
    # 2^-23 is half an fp64 ulp of 2^30 and rounds away (ties to even), giving 0.
    # Other orders give other values: downward, -2^30 + 63 * 2^-23 is exact
    # (ulp 2^-23 just below 2^30 in magnitude), giving 63 * 2^-23; chunks of 64
    # combined pairwise give 2^-17.
    M = 192
    xv = np.zeros(M, np.float32)
    wv = np.zeros(M, np.float32)
    xv[0], wv[0] = 2.0 ** 15, 2.0 ** 15
    xv[64:127], wv[64:127] = 2.0 ** -8, 2.0 ** -15
    xv[128], wv[128] = -(2.0 ** 15), 2.0 ** 15
    x, Wg = _gate_case(xv, wv)
    assert oracle.gate_logits(x, Wg, W.DT_BF16)[0, 0] == np.float32(0.0)
    # the same terms with the two large ones swapped in position sum to the exact value
    xv[0], xv[128] = -xv[0], -xv[128]
    x, Wg = _gate_case(xv, wv)
    assert oracle.gate_logits(x, Wg, W.DT_BF16)[0, 0] == np.float32(63 * 2.0 ** -23)


def test_gate_logits_one_hot_weights_select_inputs():
    # Wg[m][e] = 1 iff m == e: every logit is one input element, whatever the order.
    rng = np.random.default_rng(7)
    S, M, E = 6, 4160, 5
    x = bf16_bits_of_f32(rng.standard_normal((S, M)).astype(np.float32))
    Wg = np.zeros((M, E), np.float32)
    for e in range(E):
        Wg[e * 997, e] = 1.0
    got = oracle.gate_logits(x, Wg, W.DT_BF16)
    assert np.array_equal(got, f32_of(x)[:, [e * 997 for e in range(E)]])


def test_gate_logits_within_error_bound_of_exact_sum():
    # The fp64 sum differs from the exact sum by far less than half an fp32
    # ulp of typical logits, so the fp32 result is the exact sum rounded, except
    # (rarely) next to a rounding boundary: allow one fp32 ulp.
    import math
    rng = np.random.default_rng(11)
    S, M, E = 4, 1024, 3
    x = bf16_bits_of_f32(rng.standard_normal((S, M)).astype(np.float32))
    Wg = (rng.standard_normal((M, E)) * 0.02).astype(np.float32)
    got = oracle.gate_logits(x, Wg, W.DT_BF16)
    xf = f32_of(x).astype(np.float64)
    for s in range(S):
        for e in range(E):
            exact = np.float32(math.fsum(xf[s] * Wg[:, e].astype(np.float64)))
            assert abs(int(got[s, e].view(np.int32)) - int(exact.view(np.int32))) <= 1


def test_gate_logits_exact_products_and_fp32_rounding():
    # bf16 x times fp32 Wg: each product is exact in fp64; the sum of few terms is too.
    rng = np.random.default_rng(1)
    x32 = rng.standard_normal((5, 16)).astype(np.float32)
    x = bf16_bits_of_f32(x32)
    Wg = (rng.standard_normal((16, 3)) * 0.02).astype(np.float32)
    got = oracle.gate_logits(x, Wg, W.DT_BF16)
    want = (f32_of(x).astype(np.float64) @ Wg.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------- capacity

def test_capacity_golden_cases():
    with open(os.path.join(GOLDEN, "capacity_cases.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        if "needed" in c:
            needed = np.array(c["needed"], np.int32)
        else:
            needed = np.zeros(c["E"], np.int32)
            needed[0] = c["needed_hot"]
        assert oracle.capacity(c["S"], c["E"], c["k"], c["f"], needed) == c["C"], c["why"]


@pytest.mark.parametrize("w", W.WORKLOADS, ids=lambda w: w.name)
def test_capacity_bound_of_workloads(w):
    # f > 0: the bound is the capacity itself; f <= 0: the capacity never exceeds it.
    needed = np.full(w.E, w.S, np.int32)  # the largest any expert can need
    C = oracle.capacity(w.S, w.E, w.k, w.capacity_factor, needed)
    assert C == W.capacity_bound(w)
    if w.capacity_factor > 0:
        assert C == math.ceil(w.k * w.S * w.capacity_factor / w.E)


def test_capacity_closed_forms_of_named_workloads():
    assert W.capacity_bound(W.TINY_F32) == 64
    assert W.capacity_bound(W.GATED_BF16) == 1280
    assert W.capacity_bound(W.FINE_BF16) == 2304
    assert W.capacity_bound(W.LARGE_BF16) == 4096


# ---------------------------------------------------------------- softmax top-k

def _brute_topk(logits: np.ndarray, k: int):
    """Brute force: lexicographic sort by (-logit, expert) and fp64 softmax (scipy)."""
    S, E = logits.shape
    idx = np.empty((k, S), np.int32)
    gates = np.empty((k, S), np.float32)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    for s in range(S):
        order = np.lexsort((np.arange(E), -logits[s].astype(np.float64)))
        idx[:, s] = order[:k]
        gates[:, s] = p[s, order[:k]].astype(np.float32)
    return idx, gates, p


@pytest.mark.parametrize("E,k", [(4, 1), (8, 2), (16, 3), (64, 6), (128, 8), (5, 5), (1, 1)])
def test_topk_against_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    S = 300
    logits = rng.standard_normal((S, E)).astype(np.float32)
    # inject exact ties, +0/-0 pairs and an all-equal token
    logits[0, :] = 0.5
    if E > 1:
        logits[1, :] = 0.0
        logits[1, ::2] = -0.0
        logits[2, E - 1] = logits[2, 0]
        logits[3, :] = np.float32(-1.0)
        logits[3, E // 2] = np.float32(2.0)
    for s in range(4, S, 7):  # quantised rows: many ties
        logits[s] = np.round(logits[s] * 2) / 2
    idx, gates = oracle.softmax_topk(logits, k)
    bidx, bgates, p = _brute_topk(logits, k)
    assert np.array_equal(idx, bidx)
    # fp64 softmax rounded once to fp32: equal up to one fp32 ulp (exp/sum libm differences)
    assert np.allclose(gates, bgates, rtol=2.5e-7, atol=0)
    # invariants: distinct experts, non-increasing gates, probabilities sum to one
    for s in range(S):
        assert len(set(idx[:, s].tolist())) == k
    assert (np.diff(gates, axis=0) <= 0).all()
    assert np.allclose(p.sum(axis=1), 1.0, atol=1e-12)
    # all-equal token: lowest indices first, each prob 1/E
    assert idx[:, 0].tolist() == list(range(k))
    assert np.allclose(gates[:, 0], 1.0 / E, rtol=1e-7)


def test_topk_rejects_non_finite():
    logits = np.zeros((2, 4), np.float32)
    logits[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.softmax_topk(logits, 1)


# ---------------------------------------------------------------- locations

def test_locations_brute_force_tiny():
    rng = np.random.default_rng(3)
    for (S, E, k) in [(9, 3, 2), (17, 4, 3), (1, 2, 2), (12, 5, 1)]:
        logits = rng.standard_normal((S, E)).astype(np.float32)
        idx, _ = oracle.softmax_topk(logits, k)
        loc, needed = oracle.locations(idx, E)
        routes = [(r, s) for r in range(k) for s in range(S)]  # route-major, then token
        for i, (r, s) in enumerate(routes):
            earlier = sum(1 for (r2, s2) in routes[:i] if idx[r2, s2] == idx[r, s])
            assert loc[r, s] == earlier
        assert needed.tolist() == [int((idx == e).sum()) for e in range(E)]


@pytest.mark.parametrize("w", [W.TINY_F32, W.FINE_BF16.replace(S=2048)], ids=lambda w: w.name)
def test_route_invariants(w):
    inp = W.make_inputs(w, seed=1)
    rt = oracle.route(np_of(inp["logits"]), w.k, w.capacity_factor)
    k, S = rt["idx"].shape
    C = rt["C"]
    assert rt["needed"].sum() == k * S
    for e in range(w.E):
        locs = np.sort(rt["loc"][rt["idx"] == e])
        assert np.array_equal(locs, np.arange(rt["needed"][e]))
        assert rt["fill"][e] == min(rt["needed"][e], C)
    kept = rt["loc"] < C
    assert kept.sum() == rt["fill"].sum()
    # slot_route is a bijection from kept routes onto filled rows, -1 on padding
    slot = rt["slot_route"].reshape(w.E, C)
    for e in range(w.E):
        assert (slot[e, :rt["fill"][e]] >= 0).all() and (slot[e, rt["fill"][e]:] == -1).all()
    q = slot[slot >= 0]
    assert len(np.unique(q)) == kept.sum()
    assert kept.reshape(-1)[q].all()
    r, s = q // S, q % S
    assert np.array_equal(rt["idx"][r, s] * C + rt["loc"][r, s], np.nonzero(slot.reshape(-1) >= 0)[0])


def test_factor_zero_keeps_every_route():
    w = W.DSPR_BF16.replace(S=1024, M=64, H=64)
    inp = W.make_inputs(w, seed=2)
    rt = oracle.route(np_of(inp["logits"]), w.k, 0.0)
    assert rt["C"] == rt["needed"].max()
    assert (rt["loc"] < rt["C"]).all()
    assert rt["fill"].sum() == w.k * w.S


def test_negative_factor_drops_on_hot_experts():
    w = W.FINE_BF16.replace(S=4096)
    inp = W.make_inputs(w, seed=0)
    rt = oracle.route(np_of(inp["logits"]), w.k, w.capacity_factor)
    bound = math.ceil(w.k * w.S * 1.5 / w.E)
    assert rt["C"] == min(bound, rt["needed"].max())
    assert rt["needed"].max() > bound  # the Zipf skew overloads expert 0
    dropped = (rt["loc"] >= rt["C"]).sum()
    assert dropped == (rt["needed"] - rt["fill"]).sum() > 0


# ---------------------------------------------------------------- encode / decode == dense einsum

DENSE_CASES = [(k, f) for k in (1, 2, 3) for f in (1.0, 0.5, 0.0, -0.5, -1.0)]


@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16], ids=["f32", "bf16"])
@pytest.mark.parametrize("k,f", DENSE_CASES)
def test_index_path_equals_dense_einsum(dtype, k, f):
    S, M, E = 40, 16, 4
    rng = np.random.default_rng(100 * k + int(10 * f) + dtype)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    x = to_dtype_bits(rng.standard_normal((S, M)).astype(np.float32), dtype)
    rt = oracle.route(logits, k, f)
    C = rt["C"]
    buf = oracle.encode(x, rt, E, dtype)
    mask = onehot_mask(rt["idx"], rt["loc"], E, C)
    dense_buf = dense_dispatch(f32_of(x), mask).reshape(E * C, M)
    assert np.array_equal(f32_of(buf), dense_buf)
    # padding rows are +0 bit patterns
    pad = np.ones(E * C, bool)
    pad[oracle.filled_rows(rt)] = False
    assert (buf[pad].view(np.uint16 if dtype == W.DT_BF16 else np.uint32) == 0).all()
    # combine: per-route dense form equals the index decode exactly
    y = to_dtype_bits(rng.standard_normal((E * C, M)).astype(np.float32), dtype)
    out = oracle.decode(y, rt, E, dtype)
    dense_out = dense_combine(f32_of(y).reshape(E, C, M), mask, rt["gates"])
    assert np.array_equal(out, to_dtype_bits(dense_out, dtype))


@pytest.mark.parametrize("S,E,k", [(1, 3, 2), (7, 1, 1), (13, 4, 4), (0, 4, 1)])
def test_index_path_edge_cases(S, E, k):
    M = 8
    rng = np.random.default_rng(S + E + k)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    x = rng.standard_normal((S, M)).astype(np.float32)
    rt = oracle.route(logits, k, 0.0 if S else 1.0)
    C = rt["C"]
    buf = oracle.encode(x, rt, E, W.DT_F32)
    mask = onehot_mask(rt["idx"], rt["loc"], E, C)
    assert np.array_equal(buf, dense_dispatch(x, mask).reshape(E * C, M))
    y = rng.standard_normal((E * C, M)).astype(np.float32)
    out = oracle.decode(y, rt, E, W.DT_F32)
    assert np.array_equal(out, dense_combine(y.reshape(E, C, M), mask, rt["gates"]))
    if k == E and S:
        # every expert chosen by every token: gates are the full softmax, summing to one
        assert np.allclose(rt["gates"].astype(np.float64).sum(axis=0), 1.0, atol=1e-6)


# ---------------------------------------------------------------- expert FFN

def _torch_mlp(x64, W1, b1, W2, b2, act):
    pre = x64 @ W1.T + (b1 if b1 is not None else 0)
    h = torch.nn.functional.gelu(pre) if act == W.ACT_GELU else torch.relu(pre)
    return h @ W2.T + (b2 if b2 is not None else 0)


@pytest.mark.parametrize("act", [W.ACT_GELU, W.ACT_RELU], ids=["gelu", "relu"])
def test_single_expert_top1_is_dense_mlp(act):
    # E=1, k=1, f=0: every gate is 1 and C = S, so the layer is a dense MLP.
    w = W.Workload("mlp", S=33, M=32, E=1, k=1, H=48, capacity_factor=0.0, dtype=W.DT_F32, act=act)
    inp = {k_: np_of(v) for k_, v in W.make_inputs(w, seed=4).items()}
    fw = oracle.layer_forward(inp, w.k, w.capacity_factor, act, W.DT_F32)
    assert fw["route"]["C"] == w.S and np.all(fw["route"]["gates"] == 1.0)
    t = {k_: torch.from_numpy(v).double() for k_, v in inp.items()}
    ref = _torch_mlp(t["x"], t["W1"][0], t["b1"][0], t["W2"][0], t["b2"][0], act).numpy()
    # h is rounded to fp32 before fc2, y rounded to fp32: relative error ~ 1e-7
    assert np.allclose(fw["out"], ref, rtol=2e-6, atol=1e-7)


def test_identical_experts_closed_form():
    # All experts share weights and nothing is dropped (f = 0): out[s] = (sum_r g_r) * MLP(x[s]).
    # With k = E the gates sum to one and out = MLP(x).
    S, M, E, H = 24, 16, 3, 32
    rng = np.random.default_rng(5)
    W1 = np.repeat((rng.standard_normal((1, H, M)) * 0.2).astype(np.float32), E, 0)
    W2 = np.repeat((rng.standard_normal((1, M, H)) * 0.2).astype(np.float32), E, 0)
    b1 = np.repeat((rng.standard_normal((1, H)) * 0.2).astype(np.float32), E, 0)
    b2 = np.repeat((rng.standard_normal((1, M)) * 0.2).astype(np.float32), E, 0)
    x = rng.standard_normal((S, M)).astype(np.float32)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    ref = _torch_mlp(torch.from_numpy(x).double(), torch.from_numpy(W1[0]).double(),
                     torch.from_numpy(b1[0]).double(), torch.from_numpy(W2[0]).double(),
                     torch.from_numpy(b2[0]).double(), W.ACT_GELU).numpy()
    for k in (1, 2, 3):
        inp = dict(x=x, W1=W1, W2=W2, b1=b1, b2=b2)
        fw = oracle.layer_forward(inp, k, 0.0, W.ACT_GELU, W.DT_F32, logits=logits)
        gsum = fw["route"]["gates"].astype(np.float64).sum(axis=0)
        assert np.allclose(fw["out"], gsum[:, None] * ref, rtol=1e-5, atol=1e-6)
        if k == E:
            assert np.allclose(fw["out"], ref, rtol=1e-5, atol=1e-6)


def test_bf16_ffn_within_rounding_of_fp64_mlp():
    w = W.Workload("mlp16", S=20, M=64, E=1, k=1, H=64, capacity_factor=0.0)
    inp = {k_: np_of(v) for k_, v in W.make_inputs(w, seed=6).items()}
    fw = oracle.layer_forward(inp, 1, 0.0, W.ACT_GELU, W.DT_BF16)
    t = {k_: torch.from_numpy(f32_of(v)).double() for k_, v in inp.items() if k_ != "logits"}
    ref = _torch_mlp(t["x"], t["W1"][0], t["b1"][0], t["W2"][0], t["b2"][0], W.ACT_GELU).numpy()
    got = f32_of(fw["out"]).astype(np.float64)
    rms = np.sqrt((ref ** 2).mean())
    assert np.abs(got - ref).max() / rms < 2e-2  # bf16 h and y: ~2^-8 relative each


# ---------------------------------------------------------------- backward

def _dense_layer_torch(x, logits_route, W1, b1, W2, b2, act, E, C, idx, loc, gates):
    """Dense (one-hot) formulation in fp64 torch: dispatch einsum, per-expert MLP by bmm,
    per-route gate-weighted combine einsum."""
    k, S = idx.shape
    mask = torch.from_numpy(onehot_mask(idx, loc, E, C)).double()  # [k,S,E,C]
    buf = torch.einsum("sec,sm->ecm", mask.sum(0), x)
    pre = torch.bmm(buf, W1.transpose(1, 2).contiguous()) + b1[:, None, :]
    h = torch.nn.functional.gelu(pre) if act == W.ACT_GELU else torch.relu(pre)
    y = torch.bmm(h, W2.transpose(1, 2).contiguous()) + b2[:, None, :]
    out = torch.zeros(S, x.shape[1], dtype=torch.float64)
    for r in range(k):
        out = out + torch.einsum("sec,ecm->sm", gates[r][:, None, None] * mask[r], y)
    return out


@pytest.mark.parametrize("act,k,f", [(W.ACT_GELU, 2, 0.0), (W.ACT_GELU, 3, -0.5), (W.ACT_RELU, 2, 0.75)])
def test_backward_matches_autograd_of_dense_layer(act, k, f):
    S, M, E, H = 16, 8, 3, 10
    rng = np.random.default_rng(7 + k)
    x = rng.standard_normal((S, M)).astype(np.float32)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    W1 = (rng.standard_normal((E, H, M)) * 0.3).astype(np.float32)
    W2 = (rng.standard_normal((E, M, H)) * 0.3).astype(np.float32)
    b1 = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    b2 = (rng.standard_normal((E, M)) * 0.3).astype(np.float32)
    dout = rng.standard_normal((S, M)).astype(np.float32)
    inp = dict(x=x, W1=W1, W2=W2, b1=b1, b2=b2, dout=dout)
    fw = oracle.layer_forward(inp, k, f, act, W.DT_F32, logits=logits)
    bw = oracle.layer_backward(fw, inp, act, W.DT_F32)
    rt = fw["route"]
    tt = {n: torch.from_numpy(v).double().requires_grad_(True) for n, v in inp.items() if n != "dout"}
    g = torch.from_numpy(rt["gates"]).double().requires_grad_(True)
    out = _dense_layer_torch(tt["x"], logits, tt["W1"], tt["b1"], tt["W2"], tt["b2"], act, E, rt["C"],
                             rt["idx"], rt["loc"], g)
    assert np.allclose(fw["out"], out.detach().numpy(), rtol=1e-5, atol=1e-6)
    grads = torch.autograd.grad((out * torch.from_numpy(dout).double()).sum(),
                                [tt["x"], tt["W1"], tt["b1"], tt["W2"], tt["b2"], g])
    names = ["dx", "dW1", "db1", "dW2", "db2", "dgates"]
    for n, ref in zip(names, grads):
        ref = ref.numpy()
        got = bw[n].astype(np.float64)
        scale = max(np.abs(ref).max(), 1e-30)
        assert np.abs(got - ref).max() / scale < 2e-6, n
    # dropped routes get no gate gradient
    assert (bw["dgates"][rt["loc"] >= rt["C"]] == 0).all()


def _bf16_rne_f64(t: torch.Tensor) -> torch.Tensor:
    """fp64 values rounded once to bf16 (to nearest, ties to even), as fp64: the 52-bit
    significand is rounded at its 7th bit by integer arithmetic on the bit pattern
    (values inside the bf16 normal range, and zero)."""
    a = t.detach().contiguous().numpy().copy()
    u = a.view(np.int64)
    sign = u & np.int64(-0x8000000000000000)
    mag = u & np.int64(0x7FFFFFFFFFFFFFFF)
    lsb = (mag >> 45) & 1
    mag = (mag + (np.int64(1) << 44) - 1 + lsb) & ~((np.int64(1) << 45) - 1)
    return torch.from_numpy((sign | mag).view(np.float64).copy())


class _RoundGradBF16(torch.autograd.Function):
    """Identity forward; the gradient passing back is rounded to bf16 (a bf16 store)."""
    @staticmethod
    def forward(ctx, t):
        return t.clone()

    @staticmethod
    def backward(ctx, g):
        return _bf16_rne_f64(g)


class _RoundGradF32BF16(torch.autograd.Function):
    """Identity forward; the gradient passing back is rounded to fp32, then to bf16."""
    @staticmethod
    def forward(ctx, t):
        return t.clone()

    @staticmethod
    def backward(ctx, g):
        return _bf16_rne_f64(g.float().double())


class _StoreBF16(torch.autograd.Function):
    """Forward rounds to bf16 (a stored activation); the gradient passes unchanged."""
    @staticmethod
    def forward(ctx, t):
        return _bf16_rne_f64(t)

    @staticmethod
    def backward(ctx, g):
        return g


class _ActAtStoredPre(torch.autograd.Function):
    """act(pre) on the unrounded pre-activation; its derivative taken by torch at the
    pre-activation as stored in bf16."""
    @staticmethod
    def forward(ctx, pre, act):
        ctx.act = act
        ctx.save_for_backward(_bf16_rne_f64(pre))
        return torch.nn.functional.gelu(pre) if act == W.ACT_GELU else torch.relu(pre)

    @staticmethod
    def backward(ctx, g):
        (ps,) = ctx.saved_tensors
        with torch.enable_grad():
            p = ps.clone().requires_grad_(True)
            a = torch.nn.functional.gelu(p) if ctx.act == W.ACT_GELU else torch.relu(p)
            (d,) = torch.autograd.grad(a, p, g)
        return d, None


@pytest.mark.parametrize("act,k,f", [(W.ACT_GELU, 2, 0.0), (W.ACT_GELU, 3, -0.75), (W.ACT_RELU, 2, 0.5)])
def test_bf16_backward_rounding_points_match_autograd(act, k, f):
    # fp64 autograd of the dense one-hot layer with bf16 stores inserted where the
    # layer stores bf16: the forward's h and y (values), the pre-activation the
    # backward reads, and the gradients dy (an fp32 product, then bf16), dpre and
    # dbuf; dx is the fp64 sum of a token's dbuf rows rounded once. The oracle's
    # dy, dpre and dbuf must equal these bit for bit, dx too, and its fp32 weight
    # and bias gradients must be the fp64 sums rounded to fp32 (within one fp32
    # ulp: only the fp64 summation order differs). A missing or doubled rounding
    # at any of these points, or act' taken at the unrounded pre, changes a
    # share of the bf16 values or the weight gradients by ~2^-9 relative.
    S, M, E, H = 24, 16, 3, 24
    w = W.Workload("bf16bwd", S=S, M=M, E=E, k=k, H=H, capacity_factor=f, act=act, backward=True)
    inp = {n: np_of(v) for n, v in W.make_inputs(w, seed=5).items()}
    # larger weights than the workloads' 0.02, so that pre-activations spread over GELU's curve
    for n in ("W1", "W2", "b1", "b2"):
        inp[n] = bf16_bits_of_f32(f32_of(inp[n]) * 15.0)
    fw = oracle.layer_forward(inp, k, f, act, W.DT_BF16)
    bw = oracle.layer_backward(fw, inp, act, W.DT_BF16)
    rt = fw["route"]
    C = rt["C"]
    t = {n: torch.from_numpy(f32_of(v).astype(np.float64)) for n, v in inp.items()}
    for n in ("x", "W1", "b1", "W2", "b2"):
        t[n].requires_grad_(True)
    mask = torch.from_numpy(onehot_mask(rt["idx"], rt["loc"], E, C)).double()
    gates = torch.from_numpy(rt["gates"].astype(np.float64))
    buf = torch.einsum("sec,sm->ecm", mask.sum(0), t["x"])
    buf.retain_grad()
    pre = torch.bmm(_RoundGradBF16.apply(buf), t["W1"].transpose(1, 2).contiguous()) + t["b1"][:, None, :]
    pre.retain_grad()
    h = _StoreBF16.apply(_ActAtStoredPre.apply(_RoundGradBF16.apply(pre), act))
    y = _StoreBF16.apply(torch.bmm(h, t["W2"].transpose(1, 2).contiguous()) + t["b2"][:, None, :])
    y.retain_grad()
    yr = _RoundGradF32BF16.apply(y)
    out = torch.zeros(S, M, dtype=torch.float64)
    for r in range(k):
        out = out + torch.einsum("sec,ecm->sm", gates[r][:, None, None] * mask[r], yr)
    (out * t["dout"]).sum().backward()
    rows = fw["rows"]
    assert len(rows) > 20
    # the oracle's [E*C] row numbering is the dense [E, C] flattening
    flat = lambda g, n: g.reshape(E * C, n)[torch.from_numpy(rows)]  # noqa: E731
    for name, want, got in (("dy", flat(y.grad, M), bw["dy"]), ("dpre", flat(pre.grad, H), bw["dpre"]),
                            ("dbuf", flat(buf.grad, M), bw["dbuf"])):
        assert np.array_equal(f32_of(got).astype(np.float64), want.numpy()), name
    assert np.array_equal(f32_of(bw["dx"]).astype(np.float64), _bf16_rne_f64(t["x"].grad).numpy()), "dx"
    for name, ref in (("dW1", t["W1"].grad), ("db1", t["b1"].grad), ("dW2", t["W2"].grad), ("db2", t["b2"].grad)):
        ref32 = ref.numpy().astype(np.float32)
        d = np.abs(bw[name].view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
        assert d.max() <= 1, (name, int(d.max()))


def test_dy_is_the_fp32_product_rounded_to_bf16():
    # dy = gate * dout is fp32 arithmetic whose result is stored in bf16: two roundings.
    # Constructed case where they differ from one rounding of the exact product: the
    # gate g (fp32) and dout d = 1 + 2^-7 (bf16) give g d just above the bf16 midpoint
    # 1 + 2^-8 by less than half an fp32 ulp; fp32 rounds it onto the midpoint, which
    # then goes to the even neighbour 1, where one rounding would give 1 + 2^-7.
    from fractions import Fraction
    d = 1.0 + 2.0 ** -7
    g0 = np.float32((1.0 + 2.0 ** -8) / d)
    g = None
    for step in range(-8, 9):
        c = np.nextafter(g0, np.float32(2.0 if step > 0 else 0.0), dtype=np.float32) if step else g0
        for _ in range(abs(step) - 1):
            c = np.nextafter(c, np.float32(2.0 if step > 0 else 0.0), dtype=np.float32)
        p = Fraction(float(c)) * Fraction(d)
        if np.float32(float(p)) == np.float32(1.0 + 2.0 ** -8) and p > Fraction(1) + Fraction(1, 256):
            g = c
            break
    assert g is not None
    S, M, E, H = 4, 8, 2, 8
    w = W.Workload("dy", S=S, M=M, E=E, k=1, H=H, capacity_factor=0.0, backward=True)
    inp = {n: np_of(v) for n, v in W.make_inputs(w, seed=1).items()}
    dout = f32_of(inp["dout"]).copy()
    dout[:, 0] = d
    inp["dout"] = bf16_bits_of_f32(dout)
    fw = oracle.layer_forward(inp, 1, 0.0, w.act, W.DT_BF16)
    fw["route"]["gates"][:] = g
    routes, dy, _, _ = oracle.backward_rows(fw, inp, fw["rows"], w.act, W.DT_BF16, want_dpre=False,
                                            want_dbuf=False)
    assert len(routes) == S
    assert (f32_of(dy[:, 0]) == 1.0).all(), f32_of(dy[:, 0])


def test_encode_decode_adjoint_identities():
    # <encode(x), B> = <x, K0(B)> and <decode(y, g), D> = <y, K1'(D, g)>, the K0/K1 duality.
    S, M, E, k = 30, 8, 4, 2
    rng = np.random.default_rng(11)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    rt = oracle.route(logits, k, 0.75)
    C = rt["C"]
    x = rng.standard_normal((S, M)).astype(np.float32)
    B = rng.standard_normal((E * C, M)).astype(np.float32)
    rows = oracle.filled_rows(rt)
    routes = rt["slot_route"][rows]
    lhs = (oracle.encode(x, rt, E, W.DT_F32).astype(np.float64) * B).sum()
    K0B = oracle.dx_tokens(routes, B[rows], np.arange(S), S, k, W.DT_F32).astype(np.float64)
    assert lhs == pytest.approx((x.astype(np.float64) * K0B).sum(), rel=1e-6)
    y = rng.standard_normal((E * C, M)).astype(np.float32)
    D = rng.standard_normal((S, M)).astype(np.float32)
    lhs2 = (oracle.decode(y, rt, E, W.DT_F32).astype(np.float64) * D).sum()
    # K1'(D, g): row slot of route (r, s) gets g[r][s] * D[s]
    K1D = np.zeros((E * C, M))
    for q in routes:
        r, s = divmod(int(q), S)
        K1D[rt["idx"][r, s] * C + rt["loc"][r, s]] = rt["gates"][r, s] * D[s].astype(np.float64)
    assert lhs2 == pytest.approx((y.astype(np.float64) * K1D).sum(), rel=1e-6)


def test_backward_columns_equal_backward_rows():
    # the column-subset helper used to sample large layers computes the same elements
    w = W.Workload("cols", S=96, M=64, E=3, k=2, H=64, capacity_factor=0.0, backward=True)
    inp = {k_: np_of(v) for k_, v in W.make_inputs(w, seed=9).items()}
    fw = oracle.layer_forward(inp, w.k, w.capacity_factor, w.act, w.dtype)
    rows = fw["rows"]
    _, dy, dpre, _ = oracle.backward_rows(fw, inp, rows, w.act, w.dtype)
    cols = np.arange(w.H, dtype=np.int32)[::3]
    _, dy2, hv2, dpre2 = oracle.backward_cols(fw["route"], fw["buf"], inp, rows, cols, w.act, w.dtype)
    assert np.array_equal(dy, dy2)
    assert np.array_equal(dpre[:, cols], dpre2)
    assert np.array_equal(fw["h"][rows][:, cols], hv2)


# ---------------------------------------------------------------- gate backward

def _aux_loss_torch(p, needed, k, alpha):
    """Load-balance loss as a function of the probabilities: alpha * E * sum_e f_e * mean_s p[s, e],
    f_e = needed[e] / (k S) held constant."""
    S, E = p.shape
    f = torch.from_numpy(np.asarray(needed, np.float64)) / (k * S)
    return alpha * E * (f * p.mean(dim=0)).sum()


def _gate_loss_torch(logits64, idx, dgates, needed, k, alpha):
    """Scalar whose gradient the gate backward computes: sum over routes of dgates * p at the
    route's expert, plus the auxiliary loss."""
    p = torch.softmax(logits64, dim=1)
    sel = p.gather(1, torch.from_numpy(idx.T.astype(np.int64)))  # [S, k]
    loss = (sel * torch.from_numpy(dgates.T.astype(np.float64))).sum()
    if needed is not None:
        loss = loss + _aux_loss_torch(p, needed, k, alpha)
    return loss


@pytest.mark.parametrize("S,E,k,alpha", [(7, 5, 2, 0.01), (9, 8, 1, 0.0), (6, 3, 3, 0.3), (11, 64, 4, 0.01)])
def test_gate_backward_matches_autograd_of_softmax_and_aux_loss(S, E, k, alpha):
    rng = np.random.default_rng(100 + S)
    logits = (rng.standard_normal((S, E)) * 2).astype(np.float32)
    idx, _ = oracle.softmax_topk(logits, k)
    _, needed = oracle.locations(idx, E)
    dgates = rng.standard_normal((k, S)).astype(np.float32)
    dl, aux = oracle.gate_backward(logits, idx, dgates, needed, alpha)
    lt = torch.from_numpy(logits.astype(np.float64)).requires_grad_(True)
    loss = _gate_loss_torch(lt, idx, dgates, needed, k, alpha)
    (ref,) = torch.autograd.grad(loss, lt)
    ref = ref.numpy()
    assert np.abs(dl - ref).max() <= 1e-13 * max(np.abs(ref).max(), 1.0)
    p = torch.softmax(torch.from_numpy(logits.astype(np.float64)), 1)
    assert aux == pytest.approx(float(_aux_loss_torch(p, needed, k, alpha)), rel=1e-13, abs=1e-300)


def test_gate_backward_central_differences():
    # a derivative the oracle does not compute analytically: central differences of the scalar
    S, E, k, alpha = 5, 6, 2, 0.05
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    idx, _ = oracle.softmax_topk(logits, k)
    _, needed = oracle.locations(idx, E)
    dgates = rng.standard_normal((k, S)).astype(np.float32)
    dl, _ = oracle.gate_backward(logits, idx, dgates, needed, alpha)

    def loss(l64):
        z = np.exp(l64 - l64.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        v = sum(float(dgates[r, s]) * p[s, idx[r, s]] for r in range(k) for s in range(S))
        f = needed / (k * S)
        return v + alpha * E * float((f * p.mean(axis=0)).sum())

    base = logits.astype(np.float64)
    h = 1e-5
    for s in range(S):
        for e in range(E):
            a, b = base.copy(), base.copy()
            a[s, e] += h
            b[s, e] -= h
            fd = (loss(a) - loss(b)) / (2 * h)
            assert dl[s, e] == pytest.approx(fd, abs=1e-9)


def test_gate_backward_invariants_and_closed_forms():
    S, E, k = 8, 4, 2
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    idx, _ = oracle.softmax_topk(logits, k)
    _, needed = oracle.locations(idx, E)
    dgates = rng.standard_normal((k, S)).astype(np.float32)
    dl, _ = oracle.gate_backward(logits, idx, dgates, needed, 0.01)
    # softmax is invariant to adding a constant to a token's logits: each row sums to 0
    assert np.abs(dl.sum(axis=1)).max() <= 1e-15 * np.abs(dl).max() * E
    # only the routed entries carry upstream gradient: with alpha = 0 and dgates at one route,
    # dlogits = dg * p_i * (onehot_i - p)
    one = np.zeros_like(dgates)
    one[0, 3] = 2.5
    dl1, aux0 = oracle.gate_backward(logits, idx, one, needed, 0.0)
    p = scipy.special.softmax(logits.astype(np.float64), axis=1)
    i = idx[0, 3]
    want = np.zeros((S, E))
    want[3] = 2.5 * p[3, i] * ((np.arange(E) == i) - p[3])
    assert np.abs(dl1 - want).max() <= 1e-15
    assert aux0 == 0.0
    # balanced routing at uniform probabilities: l_aux = alpha exactly, and no gradient at all
    flat = np.zeros((S, E), np.float32)
    fidx = np.array([[(2 * s) % E for s in range(S)], [(2 * s + 1) % E for s in range(S)]], np.int32)
    _, fneed = oracle.locations(fidx, E)
    assert (fneed == k * S // E).all()
    dlf, auxf = oracle.gate_backward(flat, fidx, np.zeros((k, S), np.float32), fneed, 0.01)
    assert auxf == pytest.approx(0.01, rel=1e-15)
    assert np.abs(dlf).max() <= 1e-18
    # every route on one expert with (almost) all the probability: l_aux -> alpha * E
    peaked = np.full((S, E), -60.0, np.float32)
    peaked[:, 1] = 60.0
    pidx = np.full((1, S), 1, np.int32)
    _, pneed = oracle.locations(pidx, E)
    _, auxp = oracle.gate_backward(peaked, pidx, np.zeros((1, S), np.float32), pneed, 0.01)
    assert auxp == pytest.approx(0.01 * E, rel=1e-12)
    # no token: no loss
    _, aux_e = oracle.gate_backward(np.zeros((0, E), np.float32), np.zeros((k, 0), np.int32),
                                    np.zeros((k, 0), np.float32), np.zeros(E, np.int32), 0.01)
    assert aux_e == 0.0


@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16])
def test_gate_projection_gradients_match_autograd(dtype):
    # x . Wg exact in fp32 (small integers times multiples of 2^-6), so the oracle's fp32 logits
    # equal the fp64 ones and autograd of the fp64 composite pins dWg and dx's gate share tightly
    S, M, E, k, alpha = 12, 16, 5, 2, 0.01
    rng = np.random.default_rng(21)
    x32 = rng.integers(-4, 5, (S, M)).astype(np.float32)
    Wg = (rng.integers(-64, 65, (M, E)) / 64.0).astype(np.float32)
    x = to_dtype_bits(x32, dtype)
    logits = oracle.gate_logits(x, Wg, dtype)
    assert np.array_equal(logits, (x32.astype(np.float64) @ Wg.astype(np.float64)).astype(np.float32))
    idx, _ = oracle.softmax_topk(logits, k)
    _, needed = oracle.locations(idx, E)
    dgates = rng.standard_normal((k, S)).astype(np.float32)
    dl, _ = oracle.gate_backward(logits, idx, dgates, needed, alpha)
    dWg = oracle.gate_weight_grad(x, dl, dtype)
    no_routes = np.zeros((0,), np.int64)
    dx = oracle.dx_tokens(no_routes, np.zeros((0, M), oracle.elem_dtype(dtype)), np.arange(S), S, k, dtype,
                          dlogits=dl, Wg=Wg)
    xt = torch.from_numpy(x32.astype(np.float64)).requires_grad_(True)
    wt = torch.from_numpy(Wg.astype(np.float64)).requires_grad_(True)
    loss = _gate_loss_torch(xt @ wt, idx, dgates, needed, k, alpha)
    rx, rw = (t.numpy() for t in torch.autograd.grad(loss, [xt, wt]))
    assert np.abs(dWg - rw).max() <= 1e-13 * max(np.abs(rw).max(), 1.0)
    # dx is stored once in the data type: within half an ulp of the fp64 gradient
    got = f32_of(dx).astype(np.float64)
    ulp = np.spacing(np.abs(rx).astype(np.float32)).astype(np.float64)
    if dtype == W.DT_BF16:
        ulp = ulp * 2 ** 16  # bf16 keeps 16 fewer fraction bits than fp32
    assert (np.abs(got - rx) <= 0.5 * ulp + 1e-12 * np.abs(rx).max()).all()


def test_layer_backward_with_gate_matches_autograd():
    # the whole training backward: gates from softmax(x . Wg) and the auxiliary loss
    S, M, E, k, H, f, act, alpha = 16, 8, 3, 2, 10, 0.75, W.ACT_GELU, 0.01
    rng = np.random.default_rng(31)
    x = rng.standard_normal((S, M)).astype(np.float32)
    Wg = rng.standard_normal((M, E)).astype(np.float32)
    W1 = (rng.standard_normal((E, H, M)) * 0.3).astype(np.float32)
    W2 = (rng.standard_normal((E, M, H)) * 0.3).astype(np.float32)
    b1 = (rng.standard_normal((E, H)) * 0.3).astype(np.float32)
    b2 = (rng.standard_normal((E, M)) * 0.3).astype(np.float32)
    dout = rng.standard_normal((S, M)).astype(np.float32)
    inp = dict(x=x, Wg=Wg, W1=W1, W2=W2, b1=b1, b2=b2, dout=dout)
    fw = oracle.layer_forward(inp, k, f, act, W.DT_F32)
    bw = oracle.layer_backward(fw, inp, act, W.DT_F32, aux_coef=alpha)
    rt = fw["route"]
    assert (rt["loc"] >= rt["C"]).any(), "the case should drop routes"
    tt = {n: torch.from_numpy(v).double().requires_grad_(True) for n, v in inp.items() if n != "dout"}
    logits64 = tt["x"] @ tt["Wg"]
    p = torch.softmax(logits64, 1)
    gates = p.gather(1, torch.from_numpy(rt["idx"].T.astype(np.int64))).T  # [k, S]
    out = _dense_layer_torch(tt["x"], None, tt["W1"], tt["b1"], tt["W2"], tt["b2"], act, E, rt["C"],
                             rt["idx"], rt["loc"], gates)
    loss = (out * torch.from_numpy(dout).double()).sum() + _aux_loss_torch(p, rt["needed"], k, alpha)
    grads = torch.autograd.grad(loss, [tt["x"], tt["Wg"], logits64])
    for n, ref in zip(["dx", "dWg", "dlogits"], grads):
        ref = ref.numpy()
        got = bw[n].astype(np.float64)
        assert np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30) < 2e-6, n
    assert bw["aux_loss"] == pytest.approx(float(_aux_loss_torch(p.detach(), rt["needed"], k, alpha)), rel=1e-6)


# ---------------------------------------------------------------- Residual-MoE

def _res_inputs(S, M, E, H, dtype, seed):
    w = W.Workload("res", S=S, M=M, E=E, k=1, H=H, capacity_factor=1.0, dtype=dtype, residual=True)
    return {k_: np_of(v) for k_, v in W.make_inputs(w, seed=seed).items()}


@pytest.mark.parametrize("act", [W.ACT_GELU, W.ACT_RELU])
def test_residual_single_expert_is_sum_of_two_mlps(act):
    # E = 1, k = 1, f = 0: every token's gate is softmax over one logit = 1 and nothing drops, so
    # the layer is MLP_expert(x) + MLP_dense(x), each rounded to fp32 once, then their sum once
    S, M, H = 40, 16, 24
    inp = _res_inputs(S, M, 1, H, W.DT_F32, 3)
    fw = oracle.layer_forward(inp, 1, 0.0, act, W.DT_F32)
    x64 = torch.from_numpy(inp["x"]).double()
    e = _torch_mlp(x64, *(torch.from_numpy(inp[n][0]).double() for n in ("W1", "b1", "W2", "b2")), act)
    r = _torch_mlp(x64, *(torch.from_numpy(inp[n]).double() for n in ("W1r", "b1r", "W2r", "b2r")), act)
    want = (e + r).numpy()
    got = fw["out"].astype(np.float64)
    assert np.abs(got - want).max() <= 4 * np.spacing(np.abs(want).astype(np.float32)).max()
    assert np.abs(fw["y_r"].astype(np.float64) - r.numpy()).max() <= 2e-6 * np.abs(r.numpy()).max()


def test_residual_branch_is_the_whole_output_of_dropped_tokens():
    # ties send every token to the same experts; capacity keeps a few, and a token whose routes
    # are all dropped gets exactly the dense branch's output (0 + y_r rounds to y_r)
    S, M, E, H = 64, 16, 4, 16
    for dtype in (W.DT_F32, W.DT_BF16):
        inp = _res_inputs(S, M, E, H, dtype, 5)
        logits = np.zeros((S, E), np.float32)
        fw = oracle.layer_forward(inp, 1, 0.25, W.ACT_GELU, dtype, logits=logits)
        rt = fw["route"]
        dropped = np.nonzero(rt["loc"][0] >= rt["C"])[0]
        assert len(dropped) == S - rt["C"] > 0
        assert np.array_equal(fw["out"][dropped], fw["y_r"][dropped])
        # kept tokens: the MoE branch is there too
        kept = np.nonzero(rt["loc"][0] < rt["C"])[0]
        assert not np.array_equal(fw["out"][kept], fw["y_r"][kept])


def test_residual_branch_ignores_routing():
    # the dense branch sees every token the same way whatever the gate does
    S, M, E, H = 48, 16, 4, 32
    inp = _res_inputs(S, M, E, H, W.DT_BF16, 9)
    a = oracle.layer_forward(inp, 1, 1.0, W.ACT_GELU, W.DT_BF16,
                             logits=np.random.default_rng(1).standard_normal((S, E)).astype(np.float32))
    b = oracle.layer_forward(inp, 1, 0.5, W.ACT_GELU, W.DT_BF16,
                             logits=np.random.default_rng(2).standard_normal((S, E)).astype(np.float32))
    assert np.array_equal(a["y_r"], b["y_r"])
    x64 = torch.from_numpy(f32_of(inp["x"])).double()
    r = _torch_mlp(x64, *(torch.from_numpy(f32_of(inp[n])).double() for n in ("W1r", "b1r", "W2r", "b2r")),
                   W.ACT_GELU).numpy()
    # h_r and y_r are bf16: within a few bf16 ulps of the fp64 MLP
    assert np.abs(f32_of(a["y_r"]) - r).max() <= 2 ** -6 * np.abs(r).max()


@pytest.mark.parametrize("act,k,f,bias", [(W.ACT_GELU, 1, 1.0, True), (W.ACT_RELU, 2, 0.5, False),
                                          (W.ACT_GELU, 2, 0.0, True)])
def test_residual_backward_matches_autograd_of_the_two_branches(act, k, f, bias):
    # fp32 data: out = (one-hot MoE layer) + (dense MLP) in fp64 torch; autograd gives every
    # gradient, the dense branch's own and dx through both branches
    S, M, E, H = 20, 8, 3, 12
    rng = np.random.default_rng(11 + k)
    r = lambda *shape: (rng.standard_normal(shape) * 0.4).astype(np.float32)  # noqa: E731
    inp = dict(x=r(S, M) * 2.5, W1=r(E, H, M), W2=r(E, M, H), W1r=r(H, M), W2r=r(M, H), dout=r(S, M) * 2.5)
    if bias:
        inp.update(b1=r(E, H), b2=r(E, M), b1r=r(H), b2r=r(M))
    logits = rng.standard_normal((S, E)).astype(np.float32)
    fw = oracle.layer_forward(inp, k, f, act, W.DT_F32, logits=logits)
    bw = oracle.layer_backward(fw, inp, act, W.DT_F32)
    rt = fw["route"]
    tt = {n: torch.from_numpy(v).double().requires_grad_(True) for n, v in inp.items() if n != "dout"}
    zero = lambda shape: torch.zeros(shape, dtype=torch.float64)  # noqa: E731
    g = torch.from_numpy(rt["gates"]).double()
    moe_out = _dense_layer_torch(tt["x"], logits, tt["W1"], tt.get("b1", zero((E, H))), tt["W2"],
                                 tt.get("b2", zero((E, M))), act, E, rt["C"], rt["idx"], rt["loc"], g)
    dense = _torch_mlp(tt["x"], tt["W1r"], tt.get("b1r"), tt["W2r"], tt.get("b2r"), act)
    out = moe_out + dense
    assert np.allclose(fw["out"], out.detach().numpy(), rtol=1e-5, atol=1e-6)
    names = ["x", "W1r", "W2r"] + (["b1r", "b2r"] if bias else [])
    grads = torch.autograd.grad((out * torch.from_numpy(inp["dout"]).double()).sum(), [tt[n] for n in names])
    for n, ref in zip(names, grads):
        ref = ref.numpy()
        got = bw["dx" if n == "x" else "d" + n].astype(np.float64)
        assert np.abs(got - ref).max() / max(np.abs(ref).max(), 1e-30) < 2e-6, n
    # the dense branch's input gradient on its own: dpre_r W1r
    xd = tt["x"].detach().clone().requires_grad_(True)
    d_only = _torch_mlp(xd, *(tt[n].detach() if n in tt else None for n in ("W1r", "b1r", "W2r", "b2r")), act)
    (ref,) = torch.autograd.grad((d_only * torch.from_numpy(inp["dout"]).double()).sum(), [xd])
    assert np.abs(bw["dx_r"] - ref.numpy()).max() / np.abs(ref.numpy()).max() < 2e-6


@pytest.mark.parametrize("act", [W.ACT_GELU, W.ACT_RELU])
def test_residual_bf16_backward_rounding_points_match_autograd(act):
    # bf16 data: fp64 autograd of the dense branch with bf16 stores where the branch stores
    # bf16 (pre_r as read by the backward, h_r, y_r; the gradients dpre_r and dx_r), and dx
    # as the fp64 sum of the token's dbuf rows and its dx_r row rounded once. The oracle's
    # dpre_r and dx_r must equal these bit for bit, dx too, and its fp32 weight and bias
    # gradients the fp64 sums rounded to fp32 (within one ulp: the summation order differs).
    S, M, E, H = 24, 16, 3, 24
    w = W.Workload("resbwd", S=S, M=M, E=E, k=2, H=H, capacity_factor=1.0, act=act, residual=True, backward=True)
    inp = {n: np_of(v) for n, v in W.make_inputs(w, seed=8).items()}
    for n in ("W1", "W2", "b1", "b2", "W1r", "W2r", "b1r", "b2r"):
        inp[n] = bf16_bits_of_f32(f32_of(inp[n]) * 15.0)
    fw = oracle.layer_forward(inp, 2, 1.0, act, W.DT_BF16)
    bw = oracle.layer_backward(fw, inp, act, W.DT_BF16)
    t = {n: torch.from_numpy(f32_of(v).astype(np.float64)) for n, v in inp.items()}
    for n in ("x", "W1r", "b1r", "W2r", "b2r"):
        t[n].requires_grad_(True)
    xr = _RoundGradBF16.apply(t["x"])
    pre = xr @ t["W1r"].T + t["b1r"]
    pre.retain_grad()
    h = _StoreBF16.apply(_ActAtStoredPre.apply(_RoundGradBF16.apply(pre), act))
    y = _StoreBF16.apply(h @ t["W2r"].T + t["b2r"])
    (y * t["dout"]).sum().backward()
    assert np.array_equal(f32_of(bw["dpre_r"]).astype(np.float64), _bf16_rne_f64(pre.grad).numpy()), "dpre_r"
    assert np.array_equal(f32_of(bw["dx_r"]).astype(np.float64), _bf16_rne_f64(t["x"].grad).numpy()), "dx_r"
    for name, ref in (("dW1r", t["W1r"].grad), ("db1r", t["b1r"].grad), ("dW2r", t["W2r"].grad),
                      ("db2r", t["b2r"].grad)):
        ref32 = ref.numpy().astype(np.float32)
        d = np.abs(bw[name].view(np.int32).astype(np.int64) - ref32.view(np.int32).astype(np.int64))
        assert d.max() <= 1, (name, int(d.max()))
    # dx: the MoE branch's dbuf rows (fp64 sum) plus dx_r, rounded once
    rt = fw["route"]
    want = np.zeros((S, M))
    for i, q in enumerate(bw["routes"]):
        want[int(q) % S] += f32_of(bw["dbuf"][i])
    want += f32_of(bw["dx_r"])
    assert np.array_equal(f32_of(bw["dx"]).astype(np.float64), _bf16_rne_f64(torch.from_numpy(want)).numpy())
    assert (rt["loc"] >= rt["C"]).any()  # some routes dropped: those tokens' dx has the dense share only


def test_residual_backward_columns_equal_backward_rows():
    # the column-sampled weight gradients of the dense branch (for large layers) are the full
    # ones restricted to those columns, bit for bit: the same per-element definitions
    S, M, H = 37, 16, 40
    for dtype in (W.DT_F32, W.DT_BF16):
        w = W.Workload("rescols", S=S, M=M, E=2, k=1, H=H, capacity_factor=1.0, dtype=dtype, residual=True,
                       backward=True)
        inp = {n: np_of(v) for n, v in W.make_inputs(w, seed=4).items()}
        full = oracle.residual_backward(inp, W.ACT_GELU, dtype)
        hcols = np.array([0, 7, 21, 39], np.int32)
        dW1c, db1c, dW2c, db2c = oracle.residual_backward_cols(inp, hcols, W.ACT_GELU, dtype)
        assert np.array_equal(dW1c, full["dW1r"][hcols]) and np.array_equal(db1c, full["db1r"][hcols])
        assert np.array_equal(dW2c, full["dW2r"][:, hcols]) and np.array_equal(db2c, full["db2r"])


# ---------------------------------------------------------------- MX (microscaling) experts

def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2  # S.1111.111 only
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e2m1_values_from_the_element_formula():
    # E2M1: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is subnormal (m/2)
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        v = (m / 2.0) if e == 0 else 2.0 ** (e - 1) * (1 + m / 2.0)
        assert oracle.e2m1_value(c) == (-v if s else v)
        assert math.copysign(1.0, oracle.e2m1_value(c)) == (-1.0 if s else 1.0)


def _mx_elem_values(fmt):
    if fmt == oracle.MX_FP8:
        return np.array([oracle.e4m3_value(c) for c in range(127)])  # finite magnitudes, by code
    return np.array([oracle.e2m1_value(c) for c in range(8)])


def _mx_codes_of(codes, fmt, K):
    if fmt == oracle.MX_FP8:
        return codes.astype(np.int64)
    lo, hi = (codes & 15).astype(np.int64), (codes >> 4).astype(np.int64)
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (K,))


@pytest.mark.parametrize("fmt", [oracle.MX_FP8, oracle.MX_FP4])
@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16])
def test_mx_quantize_against_brute_force(fmt, dtype):
    rng = np.random.default_rng(40 + fmt)
    rows, K = 24, 128
    a = rng.standard_normal((rows, K)) * np.exp(rng.uniform(-12, 12, (rows, 1)))
    a[0, :32] = 0.0                      # an all-zero block
    a[1, :32] = 0.0; a[1, 5] = -0.0      # and one with a negative zero
    a[2, 32:64] = 2.0 ** 5               # amax a power of two
    a[3, :32] = 1.9 * 2.0 ** 3           # saturating block (v / X = 1.9 * 2^emax)
    a = to_dtype_bits(a.astype(np.float32), dtype)
    v = f32_of(a).astype(np.float64)
    codes, scales = oracle.mx_quantize(a, fmt, dtype)
    emax = 8 if fmt == oracle.MX_FP8 else 2
    mags = _mx_elem_values(fmt)
    cds = _mx_codes_of(codes, fmt, K)
    sign_bit = 0x80 if fmt == oracle.MX_FP8 else 0x8
    for r in range(rows):
        for b in range(K // 32):
            blk = v[r, 32 * b:32 * b + 32]
            amax = np.abs(blk).max()
            e = (np.frexp(amax)[1] - 1 - emax) if amax > 0 else -127
            assert int(scales[r, b]) == e + 127, (r, b)
            q = np.abs(blk) / 2.0 ** e
            d = np.abs(mags[None, :] - q[:, None])
            best = d.min(axis=1)
            for i in range(32):
                c = int(cds[r, 32 * b + i])
                mag = c & (sign_bit - 1)
                assert d[i, mag] == best[i], (r, b, i)  # nearest (saturating: only finite codes exist)
                ties = np.nonzero(d[i] == best[i])[0]
                if len(ties) > 1:
                    assert mag % 2 == 0  # ties to the even code
                assert bool(c & sign_bit) == bool(np.signbit(blk[i]))
    # dequantised values: X * element
    deq = oracle.mx_dequantize(codes, scales, fmt)
    assert deq[0, :32].tolist() == [0.0] * 32 and np.signbit(deq[1, 5])
    assert np.all(np.abs(deq[3, :32]) == (448.0 * 2 ** -5 if fmt == oracle.MX_FP8 else 6.0 * 2 ** 1))


def test_mx_fp8_elements_match_torch_cast():
    # where no saturation is needed, the element codes equal torch's round-to-nearest fp32 -> e4m3 cast
    rng = np.random.default_rng(44)
    a = (rng.standard_normal((16, 256)) * 3).astype(np.float32)
    codes, scales = oracle.mx_quantize(a, oracle.MX_FP8, W.DT_F32)
    X = np.repeat(2.0 ** (scales.astype(np.float64) - 127), 32, axis=1)
    q = (a / X).astype(np.float32)
    ok = np.abs(q) <= 448
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert ok.mean() > 0.9 and np.array_equal(codes[ok], ref[ok])


def _representable(rng, shape, fmt):
    """Values whose MX quantisation is exact: per 32-block, a random element set times 2^s with the
    block's largest magnitude in the format's top binade (so the shared scale is 2^s exactly)."""
    if fmt == oracle.MX_FP8:
        pool = np.arange(-14, 15, dtype=np.float64)  # 32 v is representable for |v| <= 14; amax >= 8
        top = np.array([8.0, 9.0, 10.0, 12.0, 14.0])
    else:
        pool = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6, -0.5, -1, -1.5, -2, -3, -4, -6], np.float64)
        top = np.array([4.0, 6.0, -4.0, -6.0])
    v = rng.choice(pool, size=shape)
    blocks = v.reshape(-1, 32)
    blocks[:, 0] = rng.choice(top, size=blocks.shape[0])
    scale = 2.0 ** rng.integers(-3, 3, size=(blocks.shape[0], 1))
    return (blocks * scale).reshape(shape)


@pytest.mark.parametrize("wfmt", [oracle.MX_FP8, oracle.MX_FP4])
def test_mx_ffn_on_exact_operands_matches_torch(wfmt):
    # operands that quantise exactly: fc1's pre-activation is the exact product sum, h is
    # act(pre) rounded to fp32 and MX-quantised, and y = deq(hq) . W2^T + b2 rounded to bf16
    rng = np.random.default_rng(50 + wfmt)
    E, C, M, H = 2, 3, 64, 96
    x = _representable(rng, (E * C, M), oracle.MX_FP8)
    W1 = _representable(rng, (E, H, M), wfmt)
    W2 = _representable(rng, (E, M, H), wfmt)
    b1 = bf16_bits_of_f32(rng.standard_normal((E, H)).astype(np.float32))
    b2 = bf16_bits_of_f32(rng.standard_normal((E, M)).astype(np.float32))
    bufq = oracle.mx_quantize(x.astype(np.float32), oracle.MX_FP8, W.DT_F32)
    W1q = oracle.mx_quantize(W1.astype(np.float32), wfmt, W.DT_F32)
    W2q = oracle.mx_quantize(W2.astype(np.float32), wfmt, W.DT_F32)
    assert np.array_equal(oracle.mx_dequantize(*bufq, oracle.MX_FP8), x)
    assert np.array_equal(oracle.mx_dequantize(*W1q, wfmt), W1)
    rows = np.arange(E * C)
    hq, y = oracle.expert_rows_mx(bufq, W1q, b1, W2q, b2, rows, C, W.ACT_GELU, wfmt, want_hq=True)
    for r in rows:
        e = r // C
        pre = torch.from_numpy(x[r]) @ torch.from_numpy(W1[e]).T + torch.from_numpy(f32_of(b1[e]).astype(np.float64))
        h32 = torch.nn.functional.gelu(pre).to(torch.float32).numpy()
        hc, hs = oracle.mx_quantize(h32[None], oracle.MX_FP8, W.DT_F32)
        assert np.array_equal(hc[0], hq[0][r]) and np.array_equal(hs[0], hq[1][r])
        hd = oracle.mx_dequantize(hc, hs, oracle.MX_FP8)[0]
        yr = torch.from_numpy(hd) @ torch.from_numpy(W2[e]).T + torch.from_numpy(f32_of(b2[e]).astype(np.float64))
        assert np.array_equal(y[r], bf16_bits_of_f32(yr.numpy().astype(np.float32))) or \
            np.abs(f32_of(y[r]) - yr.numpy()).max() <= 2 ** -8 * np.abs(yr.numpy()).max()


# ---------------------------------------------------------------- block-wise FP8 experts

@pytest.mark.parametrize("brows", [1, 128])
@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16])
def test_blockfp8_quantize_against_brute_force(brows, dtype):
    # per block of brows x 128: s = amax / 448 in fp32, codes = the E4M3 value nearest to v / s
    # (fp32 quotient; ties to the even code; only finite codes, so beyond 448 saturates), sign
    # kept; an all-zero block has s = 0 and codes 0
    rng = np.random.default_rng(60 + brows)
    rows, K = 256, 384
    a = rng.standard_normal((rows, K)) * np.exp(rng.uniform(-10, 10, (rows, 1)))
    a[:, :128] *= np.exp(rng.uniform(-6, 6, (rows, 1)))  # blocks of very different ranges
    if brows == 1:
        a[0, :128] = 0.0                        # an all-zero block
        a[1, :128] = 0.0; a[1, 5] = -0.0        # and one with a negative zero
        a[2, 128:256] = 3.0; a[2, 130] = -3.0   # every element at amax: codes +-448
        a[3, :128] = 1e-3; a[3, 0] = 50.0       # small elements: subnormal E4M3 codes
    else:
        a[:128, :128] = 0.0; a[7, 9] = -0.0
        a[128:, 256:] = 1e-2; a[200, 300] = -9.0
    a = to_dtype_bits(a.astype(np.float32), dtype)
    v = f32_of(a).astype(np.float32)
    codes, scales = oracle.blockfp8_quantize(a, brows, dtype)
    assert codes.shape == (rows, K) and scales.shape == (rows // brows, K // 128)
    mags = np.array([oracle.e4m3_value(c) for c in range(127)])
    blk = v.reshape(rows // brows, brows, K // 128, 128)
    amax = np.abs(blk).max(axis=(1, 3)).astype(np.float32)
    s = amax / np.float32(448.0)
    assert s.dtype == np.float32 and np.array_equal(scales, s)
    sfull = np.repeat(np.repeat(s, brows, axis=0), 128, axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(sfull > 0, v / np.where(sfull > 0, sfull, 1), 0).astype(np.float32)
    d = np.abs(mags[None, :] - np.abs(q).reshape(-1, 1).astype(np.float64))
    best = d.min(axis=1)
    c = codes.reshape(-1).astype(np.int64)
    mag = c & 0x7F
    assert np.array_equal(d[np.arange(len(c)), mag], best)
    ties = (d == best[:, None]).sum(axis=1) > 1
    assert (mag[ties] % 2 == 0).all()
    zero_blk = (sfull == 0).reshape(-1)
    assert (c[zero_blk] == 0).all() and zero_blk.any()
    assert np.array_equal((c[~zero_blk] & 0x80) != 0, np.signbit(q.reshape(-1)[~zero_blk]))
    if brows == 1:
        assert set(np.unique(codes[2, 128:256])) == {0x7E, 0xFE}  # +-448
        assert (codes[3, 1:128] < 8).all() and (codes[3, 1:128] > 0).all()  # subnormal codes
    deq = oracle.blockfp8_dequantize(codes, scales, brows)
    assert np.array_equal(deq, np.array([oracle.e4m3_value(x) for x in range(256)])[codes] * sfull.astype(np.float64))


def test_blockfp8_elements_match_torch_cast():
    # the element codes equal torch's round-to-nearest fp32 -> e4m3 cast of the fp32 quotient
    rng = np.random.default_rng(61)
    a = (rng.standard_normal((64, 256)) * 5).astype(np.float32)
    codes, scales = oracle.blockfp8_quantize(a, 1, W.DT_F32)
    q = (a / np.repeat(scales, 128, axis=1)).astype(np.float32)
    ok = np.abs(q) <= 448
    ref = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert ok.mean() > 0.99 and np.array_equal(codes[ok], ref[ok])


def _blk_representable(rng, shape, brows):
    """Values whose block-FP8 quantisation is exact: integers -14..14 (all E4M3 values) times 2^j
    per block, with one element of each block +-448 * 2^j, so that s = 2^j exactly."""
    v = rng.integers(-14, 15, size=shape).astype(np.float64)
    R, K = shape[-2], shape[-1]
    lead = v.reshape(-1, R // brows, brows, K // 128, 128)
    nb = lead.shape[0] * lead.shape[1] * lead.shape[3]
    j = rng.integers(-4, 3, size=(lead.shape[0], lead.shape[1], 1, lead.shape[3], 1)).astype(np.float64)
    lead[:, :, 0, :, 0] = rng.choice([448.0, -448.0], size=(lead.shape[0], lead.shape[1], lead.shape[3]))
    assert nb > 0
    return (lead * 2.0 ** j).reshape(shape)


def test_blockfp8_ffn_on_exact_operands_matches_torch():
    # operands that quantise exactly: fc1's pre-activation is the exact product sum, h is
    # act(pre) rounded to fp32 and block-quantised (1 x 128), y = deq(hq) . W2^T + b2 in bf16
    rng = np.random.default_rng(62)
    E, C, M, H = 2, 3, 128, 256
    x = _blk_representable(rng, (E * C, M), 1)
    W1 = _blk_representable(rng, (E, H, M), 128) * 2.0 ** -12
    W2 = _blk_representable(rng, (E, M, H), 128) * 2.0 ** -12
    b1 = bf16_bits_of_f32(rng.standard_normal((E, H)).astype(np.float32))
    b2 = bf16_bits_of_f32(rng.standard_normal((E, M)).astype(np.float32))
    bufq = oracle.blockfp8_quantize(x.astype(np.float32), 1, W.DT_F32)
    W1q = oracle.blockfp8_quantize(W1.astype(np.float32), 128, W.DT_F32)
    W2q = oracle.blockfp8_quantize(W2.astype(np.float32), 128, W.DT_F32)
    assert np.array_equal(oracle.blockfp8_dequantize(*bufq, 1), x)
    assert np.array_equal(oracle.blockfp8_dequantize(*W1q, 128), W1)
    assert np.array_equal(oracle.blockfp8_dequantize(*W2q, 128), W2)
    rows = np.arange(E * C)
    hq, y = oracle.expert_rows_blockfp8(bufq, W1q, b1, W2q, b2, rows, C, W.ACT_GELU, want_hq=True)
    for r in rows:
        e = r // C
        pre = torch.from_numpy(x[r]) @ torch.from_numpy(W1[e]).T + torch.from_numpy(f32_of(b1[e]).astype(np.float64))
        h32 = torch.nn.functional.gelu(pre).to(torch.float32).numpy()
        hc, hs = oracle.blockfp8_quantize(h32[None], 1, W.DT_F32)
        assert np.array_equal(hc[0], hq[0][r]) and np.array_equal(hs[0], hq[1][r])
        hd = oracle.blockfp8_dequantize(hc, hs, 1)[0]
        yr = torch.from_numpy(hd) @ torch.from_numpy(W2[e]).T + torch.from_numpy(f32_of(b2[e]).astype(np.float64))
        assert np.abs(f32_of(y[r]) - yr.numpy()).max() <= 2 ** -8 * np.abs(yr.numpy()).max()


# ---------------------------------------------------------------- NVFP4 experts (weights)

_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _nvfp4_codes_of(codes, K):
    lo, hi = (codes & 15).astype(np.int64), (codes >> 4).astype(np.int64)
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[:-1] + (K,))


def test_nvfp4_worked_codes():
    # One tensor of four 16-value blocks, g fixed at 2^-4 by a block whose amax is 2688 g
    # (scale code 448 = 0x7E). Hand-derived codes (E2M1 magnitudes 0,.5,1,1.5,2,3,4,6 = codes
    # 0..7, ties to the even code; E4M3 1.0 = 0x38, 1.125 = 0x39, 448 = 0x7E):
    g = 2.0 ** -4
    t = np.zeros((1, 64))
    t[0, :16] = 0.0; t[0, 0] = 2688 * g; t[0, 1] = -6 * 448 * g          # block 0: sd = 448
    # block 1: sd = 1 (amax 6 g); x = v / g hits every E2M1 midpoint
    x1 = [6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.75, -5.0, 0.2, 0.3, 4.9, 5.1, -0.0, 1.0]
    t[0, 16:32] = np.array(x1) * g
    want1 = [7, 0, 2, 2, 4, 4, 6, 6, 8 | 2, 8 | 6, 0, 1, 6, 7, 8, 2]
    # block 2: amax = 6.375 g, d = 1.0625 (a tie between 1.0 and 1.125 -> the even code 0x38),
    # so v / g = 6.375 saturates to 6 and 3.1875 rounds to 3
    t[0, 32:48] = np.array([6.375, 3.1875] + [0.0] * 14) * g
    want2 = [7, 5] + [0] * 14
    # block 3: amax = 6.1875 g, d = 1.03125 -> E4M3 1.0 (0x38); 6.1875 saturates to 6
    t[0, 48:64] = np.array([-6.1875, 1.5] + [0.0] * 14) * g
    want3 = [8 | 7, 3] + [0] * 14
    codes, scales, gq = oracle.nvfp4_quantize(t.astype(np.float32)[None], W.DT_F32)
    assert float(gq[0]) == g
    assert scales[0, 0].tolist() == [0x7E, 0x38, 0x38, 0x38]
    c = _nvfp4_codes_of(codes[0], 64)[0]
    assert c[:2].tolist() == [7, 8 | 7]
    assert c[16:32].tolist() == want1 and c[32:48].tolist() == want2 and c[48:64].tolist() == want3
    deq = oracle.nvfp4_dequantize(codes, scales, gq)[0, 0]
    assert deq[17] == 0.0 and deq[18] == g and deq[32] == 6 * g and deq[48] == -6 * g
    assert np.signbit(deq[30])  # -0 keeps its sign


def test_nvfp4_zero_tensor_and_zero_block():
    a = np.zeros((2, 4, 32), np.float32)
    a[1, 0, :16] = 1.0; a[1, 2, 16:] = -0.0
    codes, scales, g = oracle.nvfp4_quantize(a, W.DT_F32)
    assert g[0] == 0.0 and not codes[0].any() and not scales[0].any()
    assert g[1] == np.float32(1.0) / np.float32(2688.0)
    assert not codes[1, 2].any() and not scales[1, 2].any()  # an all-zero block: scale 0, codes 0
    # every element at amax: scale code 448 (0x7E), codes 6 (7); value 6 * 448 * g, g = fl(1 / 2688)
    assert (scales[1, 0, 0] == 0x7E) and (_nvfp4_codes_of(codes[1, 0], 32)[:16] == 7).all()
    assert (oracle.nvfp4_dequantize(codes, scales, g)[1, 0, :16] == 2688.0 * np.float64(g[1])).all()


@pytest.mark.parametrize("dtype", [W.DT_F32, W.DT_BF16])
def test_nvfp4_quantize_against_brute_force(dtype):
    # g = amax_t / 2688 (fp32); per block d = (amax_b / 6) / g rounded to the nearest E4M3 value
    # (ties even); elements: the E2M1 value nearest to v / (sd * g) (fp32 product and quotient)
    rng = np.random.default_rng(70)
    T, R, K = 3, 16, 64
    a = rng.standard_normal((T, R, K)) * np.exp(rng.uniform(-6, 6, (T, R, 1)))
    a[0, 3, :16] = 0.0
    a[1] *= 1e-3
    a = to_dtype_bits(a.astype(np.float32), dtype)
    v = f32_of(a).astype(np.float32)
    codes, scales, g = oracle.nvfp4_quantize(a, dtype)
    amax_t = np.abs(v).reshape(T, -1).max(axis=1)
    assert np.array_equal(g, (amax_t / np.float32(2688.0)).astype(np.float32))
    e4 = np.array([oracle.e4m3_value(c) for c in range(127)])
    blk = v.reshape(T, R, K // 16, 16)
    amax_b = np.abs(blk).max(axis=3)
    d = ((amax_b / np.float32(6.0)).astype(np.float32) / g[:, None, None]).astype(np.float32)
    dist = np.abs(e4[None, :] - d.reshape(-1, 1).astype(np.float64))
    q = scales.reshape(-1).astype(np.int64)
    assert np.array_equal(dist[np.arange(len(q)), q], dist.min(axis=1))
    tie = (dist == dist.min(axis=1)[:, None]).sum(axis=1) > 1
    assert (q[tie] % 2 == 0).all()
    sd = e4[q].reshape(T, R, K // 16).astype(np.float32)
    den = (sd * g[:, None, None]).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        x = np.where(den[..., None] > 0, blk / np.where(den > 0, den, 1)[..., None], 0).astype(np.float32)
    c = _nvfp4_codes_of(codes, K).reshape(T, R, K // 16, 16)
    dd = np.abs(_E2M1[None, :] - np.abs(x).reshape(-1, 1).astype(np.float64))
    mag = (c & 7).reshape(-1)
    assert np.array_equal(dd[np.arange(len(mag)), mag], dd.min(axis=1))
    tie = (dd == dd.min(axis=1)[:, None]).sum(axis=1) > 1
    assert (mag[tie] % 2 == 0).all()
    nz = (den > 0)[..., None].repeat(16, axis=-1).reshape(-1)
    assert (c.reshape(-1)[~nz] == 0).all() and (~nz).any()
    assert np.array_equal((c.reshape(-1)[nz] & 8) != 0, np.signbit(x.reshape(-1)[nz]))
    deq = oracle.nvfp4_dequantize(codes, scales, g)
    sgn = np.where((c & 8) != 0, -1.0, 1.0)
    want = sgn * _E2M1[c & 7] * sd[..., None].astype(np.float64) * g[:, None, None, None].astype(np.float64)
    assert np.array_equal(deq, want.reshape(T, R, K))


def _nvfp4_representable(rng, shape, lg):
    """Values whose NVFP4 quantisation is exact, per tensor of the leading dimension: g = 2^lg,
    16-blocks of E2M1 values times an E4M3 scale sd, each block holding +-6 sd (so d = sd
    exactly), and the tensor's first block sd = 448 (so g = amax_t / 2688)."""
    T, R, K = shape
    pool = np.concatenate([_E2M1, -_E2M1[1:]])
    v = rng.choice(pool, size=(T, R, K // 16, 16))
    v[..., 0] = rng.choice([6.0, -6.0], size=v.shape[:-1])
    sd = rng.choice([0.25, 0.375, 0.5, 0.75, 1.0, 1.25, 1.875, 2.0, 3.5, 8.0], size=(T, R, K // 16, 1))
    sd[:, 0, 0, 0] = 448.0
    return (v * sd * 2.0 ** lg).reshape(shape)


def test_nvfp4_ffn_matches_torch_and_the_bf16_ffn():
    # W4A16: the weights' exact values against bf16 tokens; where those values are themselves
    # bf16 numbers the FFN must be the bf16 expert FFN's, and both match a torch fp64 reference
    rng = np.random.default_rng(71)
    E, C, M, H = 2, 3, 64, 96
    W1 = _nvfp4_representable(rng, (E, H, M), -12)
    W2 = _nvfp4_representable(rng, (E, M, H), -11)
    W1q = oracle.nvfp4_quantize(W1.astype(np.float32), W.DT_F32)
    W2q = oracle.nvfp4_quantize(W2.astype(np.float32), W.DT_F32)
    assert np.array_equal(oracle.nvfp4_dequantize(*W1q), W1) and np.array_equal(oracle.nvfp4_dequantize(*W2q), W2)
    x = bf16_bits_of_f32(rng.standard_normal((E * C, M)).astype(np.float32))
    b1 = bf16_bits_of_f32(rng.standard_normal((E, H)).astype(np.float32))
    b2 = bf16_bits_of_f32(rng.standard_normal((E, M)).astype(np.float32))
    rows = np.arange(E * C)
    pre, h, y = oracle.expert_rows_nvfp4(x, W1q, b1, W2q, b2, rows, C, W.ACT_GELU)
    W1b, W2b = bf16_bits_of_f32(W1.astype(np.float32)), bf16_bits_of_f32(W2.astype(np.float32))
    assert np.array_equal(f32_of(W1b).astype(np.float64), W1)
    ref = oracle.expert_rows(x, W1b, b1, W2b, b2, rows, C, W.ACT_GELU, W.DT_BF16, want_pre=True, want_h=True)
    assert np.array_equal(pre, ref[0]) and np.array_equal(h, ref[1]) and np.array_equal(y, ref[2])
    for r in rows:
        e = r // C
        p64 = torch.from_numpy(f32_of(x[r]).astype(np.float64)) @ torch.from_numpy(W1[e]).T \
            + torch.from_numpy(f32_of(b1[e]).astype(np.float64))
        assert np.abs(f32_of(pre[r]) - p64.numpy()).max() <= 2 ** -8 * np.abs(p64.numpy()).max()
