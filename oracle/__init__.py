"""CPU oracle of the single-GPU MoE layer (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It wraps the plain C oracle in ``moe_oracle.c`` (built with gcc,
no GPU code, nothing shared with the HIP library) with numpy marshalling.

bf16 arrays travel as ``np.uint16`` bit patterns, fp32 arrays as ``np.float32``.
Route tables are route-major [k, S] (route r = 0 is the largest gate).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

DT_F32 = 0
DT_BF16 = 1

_c_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_c_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_c_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_c_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fused multiply-add, fp64 accumulation as written)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-std=c99", "-D_GNU_SOURCE", "-Wall", "-shared", "-fPIC",
                               SRC, "-o", tmp, "-lm"])
        os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        vp, i32, i64, d = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        L.oracle_num_threads.argtypes = []; L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_f64_to_bf16.argtypes = [d]; L.oracle_f64_to_bf16.restype = ctypes.c_uint16
        L.oracle_act.argtypes = [ctypes.c_int, d]; L.oracle_act.restype = d
        L.oracle_act_grad.argtypes = [ctypes.c_int, d]; L.oracle_act_grad.restype = d
        L.oracle_gate_logits.argtypes = [i32, i32, i32, ctypes.c_int, vp, _c_f32p, _c_f32p]
        L.oracle_gate_logits.restype = None
        L.oracle_softmax_topk.argtypes = [i32, i32, i32, _c_f32p, _c_i32p, _c_f32p]
        L.oracle_softmax_topk.restype = ctypes.c_int
        L.oracle_locations.argtypes = [i32, i32, i32, _c_i32p, _c_i32p, _c_i32p]
        L.oracle_locations.restype = None
        L.oracle_capacity.argtypes = [i32, i32, i32, d, _c_i32p]
        L.oracle_capacity.restype = i32
        L.oracle_route.argtypes = [i32, i32, i32, d, _c_f32p, _c_i32p, _c_f32p, _c_i32p, _c_i32p,
                                   _c_i32p, vp]
        L.oracle_route.restype = i32
        L.oracle_encode.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, vp, _c_i32p, _c_i32p, vp]
        L.oracle_encode.restype = None
        L.oracle_expert_rows.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                         vp, vp, i64, _c_i64p, vp, vp, vp]
        L.oracle_expert_rows.restype = None
        L.oracle_decode.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, vp, _c_f32p, _c_i32p,
                                    _c_i32p, i64, vp, vp, vp]
        L.oracle_decode.restype = None
        L.oracle_backward_rows.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp,
                                           vp, vp, vp, _c_f32p, vp, i64, _c_i64p, _c_i32p, vp, vp, vp]
        L.oracle_backward_rows.restype = None
        L.oracle_backward_cols.argtypes = [i32, i32, i32, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp, vp,
                                           _c_f32p, vp, i64, _c_i64p, _c_i32p, i32, _c_i32p, vp, vp, vp]
        L.oracle_backward_cols.restype = None
        L.oracle_weight_grads.argtypes = [i32, i32, ctypes.c_int, i64, vp, vp, vp, vp, _c_f32p,
                                          _c_f32p, _c_f32p, _c_f32p]
        L.oracle_weight_grads.restype = None
        L.oracle_dgates.argtypes = [i32, i32, ctypes.c_int, i64, _c_i32p, vp, vp, _c_f32p]
        L.oracle_dgates.restype = None
        L.oracle_dx.argtypes = [i32, i32, ctypes.c_int, vp, i64, _c_i64p, i32, vp, vp, vp, vp]
        L.oracle_dx.restype = None
        u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
        L.oracle_e4m3_value.argtypes = [ctypes.c_int]; L.oracle_e4m3_value.restype = d
        L.oracle_e2m1_value.argtypes = [ctypes.c_int]; L.oracle_e2m1_value.restype = d
        L.oracle_mx_quantize.argtypes = [ctypes.c_int, i64, i32, ctypes.c_int, vp, u8p, u8p]
        L.oracle_mx_quantize.restype = None
        L.oracle_mx_dequantize.argtypes = [ctypes.c_int, i64, i32, u8p, u8p, _c_f64p]
        L.oracle_mx_dequantize.restype = None
        L.oracle_expert_rows_mx.argtypes = [i32, i32, i32, ctypes.c_int, ctypes.c_int, u8p, u8p, u8p, u8p, vp, u8p,
                                            u8p, vp, i64, _c_i64p, vp, vp, vp]
        L.oracle_expert_rows_mx.restype = None
        L.oracle_blockfp8_quantize.argtypes = [i64, i32, i32, ctypes.c_int, vp, u8p, _c_f32p]
        L.oracle_blockfp8_quantize.restype = None
        L.oracle_blockfp8_dequantize.argtypes = [i64, i32, i32, u8p, _c_f32p, _c_f64p]
        L.oracle_blockfp8_dequantize.restype = None
        L.oracle_expert_rows_blockfp8.argtypes = [i32, i32, i32, ctypes.c_int, u8p, _c_f32p, u8p, _c_f32p, vp, u8p,
                                                  _c_f32p, vp, i64, _c_i64p, vp, vp, vp]
        L.oracle_expert_rows_blockfp8.restype = None
        L.oracle_nvfp4_quantize.argtypes = [i64, i32, i32, ctypes.c_int, vp, u8p, u8p, _c_f32p]
        L.oracle_nvfp4_quantize.restype = None
        L.oracle_nvfp4_dequantize.argtypes = [i64, i32, i32, u8p, u8p, _c_f32p, _c_f64p]
        L.oracle_nvfp4_dequantize.restype = None
        L.oracle_expert_rows_nvfp4.argtypes = [i32, i32, i32, ctypes.c_int, vp, u8p, u8p, _c_f32p, vp, u8p, u8p,
                                               _c_f32p, vp, i64, _c_i64p, vp, vp, vp]
        L.oracle_expert_rows_nvfp4.restype = None
        L.oracle_gate_backward.argtypes = [i32, i32, i32, d, _c_f32p, _c_i32p, _c_f32p, vp, _c_f64p, _c_f64p]
        L.oracle_gate_backward.restype = None
        L.oracle_gate_weight_grad.argtypes = [i32, i32, i32, ctypes.c_int, vp, _c_f64p, _c_f64p]
        L.oracle_gate_weight_grad.restype = None
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers

def elem_dtype(dtype: int):
    return np.float32 if dtype == DT_F32 else np.uint16


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _check(a: np.ndarray, dtype: int, shape=None) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == elem_dtype(dtype), (a.dtype, dtype)
    if shape is not None:
        assert a.shape == tuple(shape), (a.shape, shape)
    return a


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (a.astype(np.uint32) << 16).view(np.float32)


def to_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    return a.astype(np.float64) if dtype == DT_F32 else bf16_to_f32(a).astype(np.float64)


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def f64_to_bf16(v: float) -> int:
    return int(lib().oracle_f64_to_bf16(float(v)))


def act(a: int, v: float) -> float:
    return lib().oracle_act(a, float(v))


def act_grad(a: int, v: float) -> float:
    return lib().oracle_act_grad(a, float(v))


# ------------------------------------------------------------------ gating

def gate_logits(x: np.ndarray, Wg: np.ndarray, dtype: int) -> np.ndarray:
    S, M = x.shape
    E = Wg.shape[1]
    x = _check(x, dtype)
    Wg = np.ascontiguousarray(Wg, dtype=np.float32)
    out = np.empty((S, E), np.float32)
    lib().oracle_gate_logits(S, M, E, dtype, _ptr(x), Wg, out)
    return out


def softmax_topk(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    S, E = logits.shape
    idx = np.empty((k, S), np.int32)
    gates = np.empty((k, S), np.float32)
    if lib().oracle_softmax_topk(S, E, k, logits, idx, gates) != 0:
        raise ValueError("non-finite logit")
    return idx, gates


def locations(idx: np.ndarray, E: int):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    k, S = idx.shape
    loc = np.empty((k, S), np.int32)
    needed = np.empty((E,), np.int32)
    lib().oracle_locations(S, E, k, idx, loc, needed)
    return loc, needed


def capacity(S: int, E: int, k: int, f: float, needed: np.ndarray) -> int:
    return int(lib().oracle_capacity(S, E, k, float(f), np.ascontiguousarray(needed, dtype=np.int32)))


def route(logits: np.ndarray, k: int, f: float, with_slots: bool = True) -> Dict[str, np.ndarray]:
    """Softmax top-k, locations, capacity, fill and the slot -> route map."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    S, E = logits.shape
    idx = np.empty((k, S), np.int32)
    gates = np.empty((k, S), np.float32)
    loc = np.empty((k, S), np.int32)
    needed = np.empty((E,), np.int32)
    fill = np.empty((E,), np.int32)
    # slot_route needs C, which is only known afterwards: route twice (cheap).
    C = lib().oracle_route(S, E, k, float(f), logits, idx, gates, loc, needed, fill, None)
    if C < 0:
        raise ValueError("non-finite logit")
    out = dict(idx=idx, gates=gates, loc=loc, needed=needed, fill=fill, C=int(C))
    if with_slots:
        slot = np.empty((E * C,), np.int32)
        lib().oracle_route(S, E, k, float(f), logits, idx, gates, loc, needed, fill, _ptr(slot))
        out["slot_route"] = slot
    return out


# ------------------------------------------------------------------ encode / FFN / decode

def encode(x: np.ndarray, rt: Dict, E: int, dtype: int) -> np.ndarray:
    x = _check(x, dtype)
    S, M = x.shape
    k = rt["idx"].shape[0]
    C = rt["C"]
    buf = np.empty((E * C, M), elem_dtype(dtype))
    lib().oracle_encode(S, M, E, k, C, dtype, _ptr(x), rt["idx"], rt["loc"], _ptr(buf))
    return buf


def expert_rows(buf, W1, b1, W2, b2, rows: Sequence[int], C: int, act_kind: int, dtype: int,
                want_pre: bool = False, want_h: bool = False):
    """Expert FFN for the listed buffer rows (row = e*C + j). Returns (pre, h, y), compact."""
    buf = _check(buf, dtype)
    W1 = _check(W1, dtype)
    W2 = _check(W2, dtype)
    E, H, M = W1.shape
    b1 = None if b1 is None else _check(b1, dtype, (E, H))
    b2 = None if b2 is None else _check(b2, dtype, (E, M))
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    et = elem_dtype(dtype)
    pre = np.empty((n, H), et) if want_pre else None
    h = np.empty((n, H), et) if want_h else None
    y = np.empty((n, M), et)
    lib().oracle_expert_rows(M, H, E, C, dtype, act_kind, _ptr(buf), _ptr(W1), _ptr(b1), _ptr(W2),
                             _ptr(b2), n, rows, _ptr(pre), _ptr(h), _ptr(y))
    return pre, h, y


def filled_rows(rt: Dict) -> np.ndarray:
    """Buffer rows e*C + j with j < fill[e], in expert order."""
    C = rt["C"]
    return np.concatenate([e * C + np.arange(f, dtype=np.int64) for e, f in enumerate(rt["fill"])]
                          or [np.zeros(0, np.int64)]).astype(np.int64)


def decode(y: np.ndarray, rt: Dict, E: int, dtype: int, tokens: Optional[Sequence[int]] = None,
           yres: Optional[np.ndarray] = None) -> np.ndarray:
    """Gate-weighted combine; y is the [E*C, M] expert output (only kept rows are read).
    yres: the Residual-MoE dense branch's output [S, M] (only the listed tokens' rows are read)."""
    y = _check(y, dtype)
    M = y.shape[1]
    k, S = rt["idx"].shape
    C = rt["C"]
    if tokens is None:
        n, tok = S, None
    else:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
        n = tok.shape[0]
    out = np.empty((n, M), elem_dtype(dtype))
    yr = None if yres is None else _check(yres, dtype, (S, M))
    lib().oracle_decode(S, M, E, k, C, dtype, _ptr(y), rt["gates"], rt["idx"], rt["loc"], n,
                        _ptr(tok), _ptr(yr), _ptr(out))
    return out


def residual_mlp(x: np.ndarray, W1r, b1r, W2r, b2r, act_kind: int, dtype: int, tokens=None, want_pre=False):
    """Residual-MoE's dense branch: the FFN of the experts' form, with its own weights
    (W1r [H, M], W2r [M, H]), over the listed tokens (all by default). Returns (h, y) compact,
    or (pre, h, y) with want_pre (the stored pre-activation the backward reads)."""
    S = x.shape[0]
    tok = np.arange(S, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    pre, h, y = expert_rows(x, W1r[None], None if b1r is None else b1r[None], W2r[None],
                            None if b2r is None else b2r[None], tok, S, act_kind, dtype, want_pre=want_pre,
                            want_h=True)
    return (pre, h, y) if want_pre else (h, y)


def residual_backward(inp: Dict[str, np.ndarray], act_kind: int, dtype: int, h_r: Optional[np.ndarray] = None,
                      tokens=None, want_wgrad: bool = True) -> Dict[str, np.ndarray]:
    """Backward of Residual-MoE's dense branch for the layer's upstream gradient inp["dout"]
    (the branch's output adds to the layer output, so its output gradient is dout): the
    experts' per-row backward with the branch as one expert over the S token rows and every
    gate 1, so dy = dout; dpre_r and dx_r (= the row backward's dbuf) for the listed tokens
    (all by default), compact. With want_wgrad (all tokens) also dW1r, db1r, dW2r, db2r (fp32)
    from h_r (the forward's; recomputed when not given)."""
    x = _check(inp["x"], dtype)
    S, M = x.shape
    dout = _check(inp["dout"], dtype, (S, M))
    W1r, W2r = inp["W1r"], inp["W2r"]
    H = W1r.shape[0]
    b1r = inp.get("b1r")
    tok = np.arange(S, dtype=np.int64) if tokens is None else np.ascontiguousarray(np.asarray(tokens, np.int64))
    n = tok.shape[0]
    et = elem_dtype(dtype)
    dpre = np.empty((n, H), et)
    dxr = np.empty((n, M), et)
    ones = np.ones((S,), np.float32)
    lib().oracle_backward_rows(S, M, H, 1, max(S, 1), dtype, act_kind, _ptr(x), _ptr(_check(W1r[None], dtype)),
                               _ptr(None if b1r is None else _check(b1r[None], dtype)),
                               _ptr(_check(W2r[None], dtype)), ones, _ptr(dout), n, tok,
                               np.ascontiguousarray(tok.astype(np.int32)), None, _ptr(dpre), _ptr(dxr))
    out = dict(dpre_r=dpre, dx_r=dxr)
    if want_wgrad:
        assert tokens is None, "the weight gradients sum over every token"
        if h_r is None:
            h_r, _ = residual_mlp(x, W1r, b1r, W2r, inp.get("b2r"), act_kind, dtype)
        out["dW1r"], out["db1r"], out["dW2r"], out["db2r"] = weight_grads(dout, h_r, dpre, x, dtype)
    return out


def residual_backward_cols(inp: Dict[str, np.ndarray], hcols, act_kind: int, dtype: int):
    """The dense branch's weight and bias gradients on the listed hidden columns, summed over
    every token (for sampling large layers): (dW1r[hcols], db1r[hcols], dW2r[:, hcols], db2r),
    fp32. The branch is one expert over the S token rows with every gate 1 (dy = dout)."""
    x = inp["x"]
    S = x.shape[0]
    rt = dict(C=max(S, 1), idx=np.zeros((1, S), np.int32), gates=np.ones((1, S), np.float32),
              slot_route=np.arange(S, dtype=np.int32))
    one = dict(W1=inp["W1r"][None], W2=inp["W2r"][None], dout=inp["dout"])
    if inp.get("b1r") is not None:
        one["b1"] = inp["b1r"][None]
    _, dy, hv, dpre = backward_cols(rt, x, one, np.arange(S), hcols, act_kind, dtype)
    return weight_grads(dy, hv, dpre, x, dtype)


def layer_forward(inp: Dict[str, np.ndarray], k: int, f: float, act_kind: int, dtype: int,
                  logits: Optional[np.ndarray] = None) -> Dict:
    """The whole forward for small shapes: returns route tables, buf, pre, h, y (full E*C rows,
    padding rows of pre/h/y left zero) and out. With the Residual-MoE weights in inp (W1r, W2r,
    and b1r/b2r when the biases are on) also pre_r, h_r, y_r and out = MoE output + y_r."""
    x = inp["x"]
    if logits is None:
        logits = inp["logits"] if "logits" in inp else gate_logits(x, inp["Wg"], dtype)
    E = inp["W1"].shape[0]
    rt = route(logits, k, f)
    buf = encode(x, rt, E, dtype)
    rows = filled_rows(rt)
    pre_r, h_r, y_r = expert_rows(buf, inp["W1"], inp.get("b1"), inp["W2"], inp.get("b2"), rows,
                                  rt["C"], act_kind, dtype, want_pre=True, want_h=True)
    H = inp["W1"].shape[1]
    M = x.shape[1]
    et = elem_dtype(dtype)
    pre = np.zeros((E * rt["C"], H), et); pre[rows] = pre_r
    h = np.zeros((E * rt["C"], H), et); h[rows] = h_r
    y = np.zeros((E * rt["C"], M), et); y[rows] = y_r
    res = {}
    if "W1r" in inp:
        res["pre_r"], res["h_r"], res["y_r"] = residual_mlp(x, inp["W1r"], inp.get("b1r"), inp["W2r"], inp.get("b2r"),
                                                            act_kind, dtype, want_pre=True)
    out = decode(y, rt, E, dtype, yres=res.get("y_r"))
    return dict(logits=logits, route=rt, buf=buf, pre=pre, h=h, y=y, out=out, rows=rows, **res)


# ------------------------------------------------------------------ backward

def backward_rows(fw: Dict, inp: Dict, rows: np.ndarray, act_kind: int, dtype: int,
                  want_dy=True, want_dpre=True, want_dbuf=True):
    """Per-row backward (dy, dpre, dbuf) for kept buffer rows, compact outputs."""
    rt = fw["route"]
    C = rt["C"]
    k, S = rt["idx"].shape
    W1, W2 = inp["W1"], inp["W2"]
    E, H, M = W1.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    routes = np.ascontiguousarray(rt["slot_route"][rows].astype(np.int32))
    assert (routes >= 0).all(), "backward rows must be filled rows"
    n = rows.shape[0]
    et = elem_dtype(dtype)
    dy = np.empty((n, M), et) if want_dy else None
    dpre = np.empty((n, H), et) if want_dpre else None
    dbuf = np.empty((n, M), et) if want_dbuf else None
    b1 = inp.get("b1")
    lib().oracle_backward_rows(S, M, H, E, C, dtype, act_kind, _ptr(fw["buf"]), _ptr(W1), _ptr(b1),
                               _ptr(W2), rt["gates"].reshape(-1).copy(), _ptr(_check(inp["dout"], dtype)),
                               n, rows, routes, _ptr(dy), _ptr(dpre), _ptr(dbuf))
    return routes, dy, dpre, dbuf


def backward_cols(rt: Dict, buf: np.ndarray, inp: Dict, rows, hcols, act_kind: int, dtype: int):
    """dy rows, h columns and dpre columns of the listed kept rows (selected hidden columns)."""
    C = rt["C"]
    k, S = rt["idx"].shape
    W1, W2 = _check(inp["W1"], dtype), _check(inp["W2"], dtype)
    E, H, M = W1.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    routes = np.ascontiguousarray(rt["slot_route"][rows].astype(np.int32))
    assert (routes >= 0).all()
    hcols = np.ascontiguousarray(np.asarray(hcols, dtype=np.int32))
    n, nc = rows.shape[0], hcols.shape[0]
    et = elem_dtype(dtype)
    dy = np.empty((n, M), et)
    hv = np.empty((n, nc), et)
    dpre = np.empty((n, nc), et)
    lib().oracle_backward_cols(S, M, H, C, dtype, act_kind, _ptr(_check(buf, dtype)), _ptr(W1),
                               _ptr(inp.get("b1")), _ptr(W2), rt["gates"].reshape(-1).copy(),
                               _ptr(_check(inp["dout"], dtype)), n, rows, routes, nc, hcols, _ptr(dy), _ptr(hv),
                               _ptr(dpre))
    return routes, dy, hv, dpre


def weight_grads(dy, hv, dpre, bufrows, dtype: int):
    n, M = dy.shape
    H = hv.shape[1]
    dW1 = np.empty((H, M), np.float32); db1 = np.empty((H,), np.float32)
    dW2 = np.empty((M, H), np.float32); db2 = np.empty((M,), np.float32)
    lib().oracle_weight_grads(M, H, dtype, n, _ptr(np.ascontiguousarray(dy)), _ptr(np.ascontiguousarray(hv)),
                              _ptr(np.ascontiguousarray(dpre)), _ptr(np.ascontiguousarray(bufrows)),
                              dW1, db1, dW2, db2)
    return dW1, db1, dW2, db2


def dgates(routes: np.ndarray, dout: np.ndarray, yrows: np.ndarray, S: int, dtype: int) -> np.ndarray:
    routes = np.ascontiguousarray(routes, dtype=np.int32)
    n = routes.shape[0]
    M = dout.shape[1]
    dg = np.empty((n,), np.float32)
    lib().oracle_dgates(S, M, dtype, n, routes, _ptr(_check(dout, dtype)),
                        _ptr(np.ascontiguousarray(yrows)), dg)
    return dg


def dx_tokens(routes: np.ndarray, dbufrows: np.ndarray, tokens: Sequence[int], S: int, k: int,
              dtype: int, dlogits: Optional[np.ndarray] = None, Wg: Optional[np.ndarray] = None,
              res: Optional[np.ndarray] = None) -> np.ndarray:
    """dx of the listed tokens from the dbuf rows of kept routes (routes[i] = r*S + s), plus
    dlogits[token] . Wg^T when the gate projection's gradient (fp64 dlogits [S,E]) is given,
    plus the Residual-MoE dense branch's dx_r rows (res, [S, M] in the data type) when given."""
    routes = np.asarray(routes, dtype=np.int64)
    tok = np.asarray(tokens, dtype=np.int64)
    pos = {int(t): i for i, t in enumerate(tok)}
    table = np.full((tok.shape[0], k), -1, np.int64)
    for i, q in enumerate(routes):
        t = pos.get(int(q % S))
        if t is not None:
            table[t, int(q // S)] = i
    M = dbufrows.shape[1]
    out = np.empty((tok.shape[0], M), elem_dtype(dtype))
    E, dl, wg = 0, None, None
    if dlogits is not None:
        E = dlogits.shape[1]
        dl = np.ascontiguousarray(np.asarray(dlogits, np.float64)[tok])
        wg = np.ascontiguousarray(Wg, dtype=np.float32)
        assert wg.shape == (M, E)
    rr = None if res is None else np.ascontiguousarray(_check(res, dtype, (S, M))[tok])
    lib().oracle_dx(M, k, dtype, _ptr(np.ascontiguousarray(dbufrows)), tok.shape[0],
                    np.ascontiguousarray(table), E, _ptr(dl), _ptr(wg), _ptr(rr), _ptr(out))
    return out


# ------------------------------------------------------------------ gate backward

def gate_backward(logits: np.ndarray, idx: np.ndarray, dgates: np.ndarray, needed: Optional[np.ndarray],
                  alpha: float):
    """dlogits (fp64 [S,E]) through the softmax, and the auxiliary load-balance loss (fp64)."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    S, E = logits.shape
    k = idx.shape[0]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    dgates = np.ascontiguousarray(dgates, dtype=np.float32)
    assert idx.shape == (k, S) and dgates.shape == (k, S)
    nd = None if needed is None else np.ascontiguousarray(needed, dtype=np.int32)
    dl = np.empty((S, E), np.float64)
    aux = np.zeros((1,), np.float64)
    lib().oracle_gate_backward(S, E, k, float(alpha), logits, idx, dgates, _ptr(nd), dl, aux)
    return dl, float(aux[0])


def gate_weight_grad(x: np.ndarray, dlogits: np.ndarray, dtype: int) -> np.ndarray:
    """dWg = x^T . dlogits (fp64 [M,E])."""
    x = _check(x, dtype)
    S, M = x.shape
    dl = np.ascontiguousarray(dlogits, dtype=np.float64)
    E = dl.shape[1]
    out = np.empty((M, E), np.float64)
    lib().oracle_gate_weight_grad(S, M, E, dtype, _ptr(x), dl, out)
    return out


def layer_backward(fw: Dict, inp: Dict, act_kind: int, dtype: int, aux_coef: Optional[float] = None
                   ) -> Dict[str, np.ndarray]:
    """The whole backward for small shapes: dx, dW1, db1, dW2, db2 (fp32) and dgates [k,S]
    (0 for dropped routes). With aux_coef given, also the gate backward: dlogits (fp64) and
    aux_loss from the forward's logits, and, when the logits were projected (inp has Wg),
    dWg (fp64) and the gate projection's share of dx. With the Residual-MoE weights in inp
    (W1r, W2r), also the dense branch's dpre_r, dx_r, dW1r, db1r, dW2r, db2r, and dx_r is
    added to dx."""
    rt = fw["route"]
    C = rt["C"]
    k, S = rt["idx"].shape
    E, H, M = inp["W1"].shape
    rows = fw["rows"]
    routes, dy, dpre, dbuf = backward_rows(fw, inp, rows, act_kind, dtype)
    dW1 = np.zeros((E, H, M), np.float32); db1 = np.zeros((E, H), np.float32)
    dW2 = np.zeros((E, M, H), np.float32); db2 = np.zeros((E, M), np.float32)
    start = 0
    for e in range(E):
        n = int(rt["fill"][e])
        sl = slice(start, start + n)
        dW1[e], db1[e], dW2[e], db2[e] = weight_grads(dy[sl], fw["h"][rows[sl]], dpre[sl],
                                                      fw["buf"][rows[sl]], dtype)
        start += n
    dg = np.zeros((k * S,), np.float32)
    dg[routes] = dgates(routes, inp["dout"], fw["y"][rows], S, dtype)
    dg = dg.reshape(k, S)
    out = dict(dW1=dW1, db1=db1, dW2=dW2, db2=db2, dgates=dg, dy=dy, dpre=dpre, dbuf=dbuf, routes=routes)
    dl = Wg = None
    if aux_coef is not None:
        dl, out["aux_loss"] = gate_backward(fw["logits"], rt["idx"], dg, rt["needed"], aux_coef)
        out["dlogits"] = dl
        if "Wg" in inp:
            Wg = inp["Wg"]
            out["dWg"] = gate_weight_grad(inp["x"], dl, dtype)
        else:
            dl = None
    dxr = None
    if "W1r" in inp:
        rb = residual_backward(inp, act_kind, dtype, h_r=fw.get("h_r"))
        out.update(rb)
        dxr = rb["dx_r"]
    out["dx"] = dx_tokens(routes, dbuf, np.arange(S), S, k, dtype, dlogits=dl, Wg=Wg, res=dxr)
    return out


# ------------------------------------------------------------------ MX (microscaling) experts

MX_FP8 = 0  # MXFP8: E4M3 elements, one byte each
MX_FP4 = 1  # MXFP4: E2M1 elements, two per byte (even index in the low nibble)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(int(code))


def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(int(code))


def mx_row_bytes(K: int, fmt: int) -> int:
    return K if fmt == MX_FP8 else K // 2


def mx_quantize(a: np.ndarray, fmt: int, dtype: int):
    """MX quantisation along the last dimension (a multiple of 32) of a data-type array:
    returns (codes uint8 [..., row bytes], scales uint8 [..., K/32])."""
    a = _check(a, dtype)
    K = a.shape[-1]
    assert K % 32 == 0
    rows = int(np.prod(a.shape[:-1], dtype=np.int64))
    codes = np.zeros(a.shape[:-1] + (mx_row_bytes(K, fmt),), np.uint8)
    scales = np.zeros(a.shape[:-1] + (K // 32,), np.uint8)
    lib().oracle_mx_quantize(fmt, rows, K, dtype, _ptr(a), codes, scales)
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, fmt: int) -> np.ndarray:
    K = scales.shape[-1] * 32
    rows = int(np.prod(scales.shape[:-1], dtype=np.int64))
    out = np.empty(scales.shape[:-1] + (K,), np.float64)
    lib().oracle_mx_dequantize(fmt, rows, K, np.ascontiguousarray(codes), np.ascontiguousarray(scales), out)
    return out


def expert_rows_mx(bufq, W1q, b1, W2q, b2, rows: Sequence[int], C: int, act_kind: int, wfmt: int,
                   want_hq: bool = False):
    """MX expert FFN for the listed buffer rows: bufq = (codes, scales) MXFP8 [E*C, M];
    W1q = (codes, scales) [E, H, M] and W2q [E, M, H] in format wfmt; biases bf16 or None.
    Returns (h codes, h scales) when asked and y (bf16, compact [n, M])."""
    bc, bs = (np.ascontiguousarray(t) for t in bufq)
    w1c, w1s = (np.ascontiguousarray(t) for t in W1q)
    w2c, w2s = (np.ascontiguousarray(t) for t in W2q)
    E, H = w1s.shape[0], w1s.shape[1]
    M = w2s.shape[1]
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    hc = np.empty((n, H), np.uint8) if want_hq else None
    hs = np.empty((n, H // 32), np.uint8) if want_hq else None
    y = np.empty((n, M), np.uint16)
    b1 = None if b1 is None else _check(b1, DT_BF16, (E, H))
    b2 = None if b2 is None else _check(b2, DT_BF16, (E, M))
    lib().oracle_expert_rows_mx(M, H, C, act_kind, wfmt, bc, bs, w1c, w1s, _ptr(b1), w2c, w2s, _ptr(b2), n, rows,
                                _ptr(hc), _ptr(hs), _ptr(y))
    return ((hc, hs) if want_hq else None), y


# ------------------------------------------------------------------ block-wise FP8 experts

BLOCK = 128  # block edge: 128 x 128 weight blocks, 1 x 128 activation blocks


def blockfp8_quantize(a: np.ndarray, brows: int, dtype: int):
    """Block-wise FP8 quantisation of a data-type array along its last dimension (a multiple of
    128) in blocks of brows (1 or 128) rows x 128: returns (codes uint8, same shape as a; scales
    fp32 [..., rows / brows, K / 128] over the last two dimensions, or [..., K / 128] for
    brows = 1)."""
    a = _check(a, dtype)
    K = a.shape[-1]
    assert K % BLOCK == 0 and brows in (1, BLOCK)
    rows = int(np.prod(a.shape[:-1], dtype=np.int64))
    assert rows % brows == 0
    codes = np.zeros(a.shape, np.uint8)
    if brows == 1:
        sshape = a.shape[:-1] + (K // BLOCK,)
    else:
        assert a.shape[-2] % brows == 0
        sshape = a.shape[:-2] + (a.shape[-2] // brows, K // BLOCK)
    scales = np.zeros(sshape, np.float32)
    lib().oracle_blockfp8_quantize(rows, K, brows, dtype, _ptr(a), codes, scales)
    return codes, scales


def blockfp8_dequantize(codes: np.ndarray, scales: np.ndarray, brows: int) -> np.ndarray:
    """Exact values (fp64, the shape of codes) of a block-FP8 array."""
    K = codes.shape[-1]
    rows = int(np.prod(codes.shape[:-1], dtype=np.int64))
    out = np.empty(codes.shape, np.float64)
    lib().oracle_blockfp8_dequantize(rows, K, brows, np.ascontiguousarray(codes),
                                     np.ascontiguousarray(scales, dtype=np.float32), out)
    return out


def expert_rows_blockfp8(bufq, W1q, b1, W2q, b2, rows: Sequence[int], C: int, act_kind: int, want_hq: bool = False):
    """Block-FP8 expert FFN for the listed buffer rows: bufq = (codes [E*C, M], scales [E*C, M/128]);
    W1q = (codes [E, H, M], scales [E, H/128, M/128]) and W2q likewise [E, M, H]; biases bf16 or None.
    Returns (h codes, h scales) when asked and y (bf16, compact [n, M])."""
    bc, bs = np.ascontiguousarray(bufq[0]), np.ascontiguousarray(bufq[1], dtype=np.float32)
    w1c, w1s = np.ascontiguousarray(W1q[0]), np.ascontiguousarray(W1q[1], dtype=np.float32)
    w2c, w2s = np.ascontiguousarray(W2q[0]), np.ascontiguousarray(W2q[1], dtype=np.float32)
    E, H, M = w1c.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    hc = np.empty((n, H), np.uint8) if want_hq else None
    hs = np.empty((n, H // BLOCK), np.float32) if want_hq else None
    y = np.empty((n, M), np.uint16)
    b1 = None if b1 is None else _check(b1, DT_BF16, (E, H))
    b2 = None if b2 is None else _check(b2, DT_BF16, (E, M))
    lib().oracle_expert_rows_blockfp8(M, H, C, act_kind, bc, bs, w1c, w1s, _ptr(b1), w2c, w2s, _ptr(b2), n, rows,
                                      _ptr(hc), _ptr(hs), _ptr(y))
    return ((hc, hs) if want_hq else None), y


# ------------------------------------------------------------------ NVFP4 experts (weights)

NVFP4_BLOCK = 16  # values per E4M3-scaled block along the reduction dimension


def nvfp4_quantize(a: np.ndarray, dtype: int):
    """NVFP4 quantisation of a data-type array [..., rows, K] (K a multiple of 16), each matrix
    over the last two dimensions one tensor with its own fp32 scale: returns (codes uint8
    [..., rows, K/2], block scales uint8 (E4M3) [..., rows, K/16], g fp32 [...])."""
    a = _check(a, dtype)
    assert a.ndim >= 2
    K = a.shape[-1]
    assert K % NVFP4_BLOCK == 0
    lead = a.shape[:-2]
    nt = int(np.prod(lead, dtype=np.int64)) if lead else 1
    rows = nt * a.shape[-2]
    codes = np.zeros(a.shape[:-1] + (K // 2,), np.uint8)
    scales = np.zeros(a.shape[:-1] + (K // NVFP4_BLOCK,), np.uint8)
    g = np.zeros(lead if lead else (1,), np.float32)
    lib().oracle_nvfp4_quantize(rows, K, nt, dtype, _ptr(a), codes, scales, g)
    return codes, scales, (g if lead else g.reshape(()))


def nvfp4_dequantize(codes: np.ndarray, scales: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Exact values (fp64 [..., rows, K]) of an NVFP4 array from nvfp4_quantize."""
    K = scales.shape[-1] * NVFP4_BLOCK
    lead = scales.shape[:-2]
    nt = int(np.prod(lead, dtype=np.int64)) if lead else 1
    rows = nt * scales.shape[-2]
    out = np.empty(scales.shape[:-1] + (K,), np.float64)
    lib().oracle_nvfp4_dequantize(rows, K, nt, np.ascontiguousarray(codes), np.ascontiguousarray(scales),
                                  np.ascontiguousarray(np.asarray(g, np.float32).reshape(-1)), out)
    return out


def expert_rows_nvfp4(buf, W1q, b1, W2q, b2, rows: Sequence[int], C: int, act_kind: int):
    """Expert FFN with NVFP4 weights for the listed buffer rows: buf bf16 [E*C, M]; W1q = (codes
    [E, H, M/2], scales [E, H, M/16], g [E]) and W2q likewise [E, M, H]; biases bf16 or None.
    Returns pre, h (bf16 [n, H]) and y (bf16 [n, M]), compact per listed row."""
    w1c, w1s = np.ascontiguousarray(W1q[0]), np.ascontiguousarray(W1q[1])
    w2c, w2s = np.ascontiguousarray(W2q[0]), np.ascontiguousarray(W2q[1])
    g1 = np.ascontiguousarray(np.asarray(W1q[2], np.float32).reshape(-1))
    g2 = np.ascontiguousarray(np.asarray(W2q[2], np.float32).reshape(-1))
    E, H = w1s.shape[0], w1s.shape[1]
    M = w2s.shape[1]
    buf = _check(buf, DT_BF16)
    assert buf.shape[-1] == M
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n = rows.shape[0]
    pre = np.empty((n, H), np.uint16)
    h = np.empty((n, H), np.uint16)
    y = np.empty((n, M), np.uint16)
    b1 = None if b1 is None else _check(b1, DT_BF16, (E, H))
    b2 = None if b2 is None else _check(b2, DT_BF16, (E, M))
    lib().oracle_expert_rows_nvfp4(M, H, C, act_kind, _ptr(buf), w1c, w1s, g1, _ptr(b1), w2c, w2s, g2, _ptr(b2), n,
                                   rows, _ptr(pre), _ptr(h), _ptr(y))
    return pre, h, y
