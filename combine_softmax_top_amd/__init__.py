"""Python binding of the gfx950 MoE layer library (``libmoe.so``, C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. PyTorch supplies device memory and the stream. Each function has the
name of the C entry point it calls, takes torch tensors (or None for NULL), and
raises ``MoeError`` on a non-OK status. Nothing here computes any part of the
layer; if the library is missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Dict, Optional

import torch  # loads the HIP runtime that libmoe.so then binds to

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_ACT_RELU, MOE_ACT_GELU = 0, 1
MOE_MX_FP8, MOE_MX_FP4 = 0, 1

STATUS_NAMES = {0: "MOE_OK", -1: "MOE_EINVAL", -2: "MOE_EUNSUPPORTED", -3: "MOE_EWORKSPACE", -4: "MOE_EHIP"}


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class moe_shape(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("M", ctypes.c_int32), ("E", ctypes.c_int32), ("k", ctypes.c_int32),
                ("H", ctypes.c_int32), ("capacity_factor", ctypes.c_double), ("dtype", ctypes.c_int32),
                ("act", ctypes.c_int32), ("has_fc1_bias", ctypes.c_int32), ("has_fc2_bias", ctypes.c_int32)]


@dataclasses.dataclass(frozen=True)
class Shape:
    S: int
    M: int
    E: int
    k: int
    H: int
    capacity_factor: float
    dtype: int = MOE_DT_BF16
    act: int = MOE_ACT_GELU
    has_fc1_bias: bool = True
    has_fc2_bias: bool = True

    def c(self) -> moe_shape:
        return moe_shape(self.S, self.M, self.E, self.k, self.H, float(self.capacity_factor), self.dtype, self.act,
                         int(bool(self.has_fc1_bias)), int(bool(self.has_fc2_bias)))

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == MOE_DT_F32 else torch.bfloat16

    @staticmethod
    def of(w) -> "Shape":
        """From any object with the layer's fields (e.g. a workload description)."""
        return Shape(w.S, w.M, w.E, w.k, w.H, w.capacity_factor, w.dtype, w.act, w.has_fc1_bias, w.has_fc2_bias)


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m combine_softmax_top_amd.build` "
                      "(or __graft_entry__.build()); there is no fallback path")
_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_SP = ctypes.POINTER(moe_shape)
_SIGS = {
    "moe_validate": [_SP],
    "moe_capacity_bound": [_SP, ctypes.POINTER(ctypes.c_int32)],
    "moe_workspace_size": [_SP, ctypes.POINTER(ctypes.c_size_t)],
    "moe_gate_project": [_SP, _P, _P, _P, _P],
    "moe_route": [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_encode": [_SP, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_ffn": [_SP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_fc1": [_SP, _P, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_fc2": [_SP, _P, _P, _P, _P, _P, _P, _P],
    "moe_expert_ffn_window": [_SP] + [_P] * 7 + [ctypes.c_int32, ctypes.c_int32] + [_P] * 4,
    "moe_layer_forward_pipelined": [_SP] + [_P] * 21 + [ctypes.c_size_t, ctypes.c_int32, _P, ctypes.c_int32, _P, _P],
    "moe_decode": [_SP, _P, _P, _P, _P, _P, _P, _P],
    "moe_layer_forward": [_SP] + [_P] * 21 + [ctypes.c_size_t, _P],
    "moe_mx_quantize": [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P],
    "moe_encode_mx": [_SP] + [_P] * 8,
    "moe_expert_ffn_mx": [_SP, ctypes.c_int32] + [_P] * 14,
    "moe_layer_forward_mx": [_SP, ctypes.c_int32] + [_P] * 24 + [ctypes.c_size_t, _P],
    "moe_expert_fc1_mx": [_SP, ctypes.c_int32] + [_P] * 10,
    "moe_expert_fc2_mx": [_SP, ctypes.c_int32] + [_P] * 9,
    "moe_blockfp8_quantize": [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P],
    "moe_nvfp4_quantize": [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P, _P],
    "moe_expert_ffn_nvfp4": [_SP] + [_P] * 15,
    "moe_expert_fc1_nvfp4": [_SP] + [_P] * 10,
    "moe_expert_fc2_nvfp4": [_SP] + [_P] * 9,
    "moe_layer_forward_nvfp4": [_SP] + [_P] * 24 + [ctypes.c_size_t, _P],
    "moe_encode_blockfp8": [_SP] + [_P] * 8,
    "moe_expert_ffn_blockfp8": [_SP] + [_P] * 14,
    "moe_layer_forward_blockfp8": [_SP] + [_P] * 24 + [ctypes.c_size_t, _P],
    "moe_expert_fc1_blockfp8": [_SP] + [_P] * 10,
    "moe_expert_fc2_blockfp8": [_SP] + [_P] * 9,
    "moe_residual_ffn": [_SP] + [_P] * 9 + [ctypes.c_size_t, _P],
    "moe_residual_backward": [_SP] + [_P] * 13 + [ctypes.c_size_t, _P],
    "moe_decode_residual": [_SP] + [_P] * 8,
    "moe_residual_layer_forward": [_SP] + [_P] * 28 + [ctypes.c_size_t, _P],
    "moe_gate_backward": [_SP, _P, _P, _P, _P, ctypes.c_double, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_gate_weight_grad": [_SP, _P, _P, _P, _P, ctypes.c_size_t, _P],
    "moe_layer_backward": [_SP] + [_P] * 23 + [ctypes.c_double] + [_P] * 6 + [ctypes.c_size_t, _P],
    "moe_residual_layer_backward": [_SP] + [_P] * 23 + [ctypes.c_double] + [_P] * 16 + [ctypes.c_size_t, _P],
    "moe_decode_backward": [_SP] + [_P] * 9,
    "moe_expert_fc2_backward_data": [_SP] + [_P] * 7,
    "moe_expert_fc2_weight_grad": [_SP] + [_P] * 7,
    "moe_expert_fc1_backward_data": [_SP] + [_P] * 6,
    "moe_expert_fc1_weight_grad": [_SP] + [_P] * 7,
    "moe_encode_backward": [_SP] + [_P] * 6,
    "moe_layer_forward_noalloc": [_SP] + [_P] * 21,
}

# coefficient of the auxiliary load-balance loss in the MoE training blog's runs
AUX_COEF = 0.01
for _name, _args in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = ctypes.c_int
_lib.moe_last_error.argtypes = []
_lib.moe_last_error.restype = ctypes.c_char_p

EXPORTED = sorted(list(_SIGS) + ["moe_last_error"])


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, moe_last_error())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def moe_validate(shape: Shape) -> int:
    return _lib.moe_validate(ctypes.byref(shape.c()))


def moe_capacity_bound(shape: Shape) -> int:
    c = ctypes.c_int32()
    _check(_lib.moe_capacity_bound(ctypes.byref(shape.c()), ctypes.byref(c)))
    return c.value


def moe_workspace_size(shape: Shape) -> int:
    n = ctypes.c_size_t()
    _check(_lib.moe_workspace_size(ctypes.byref(shape.c()), ctypes.byref(n)))
    return n.value


def moe_gate_project(shape: Shape, x, Wg, logits, stream=None) -> None:
    _check(_lib.moe_gate_project(ctypes.byref(shape.c()), _ptr(x), _ptr(Wg), _ptr(logits), _stream(stream)))


def moe_route(shape: Shape, logits, idx, loc, gates, needed, fill, capacity, slot_route, ws, stream=None) -> None:
    _check(_lib.moe_route(ctypes.byref(shape.c()), _ptr(logits), _ptr(idx), _ptr(loc), _ptr(gates), _ptr(needed),
                          _ptr(fill), _ptr(capacity), _ptr(slot_route), _ptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_encode(shape: Shape, x, idx, loc, fill, capacity, buf, stream=None) -> None:
    _check(_lib.moe_encode(ctypes.byref(shape.c()), _ptr(x), _ptr(idx), _ptr(loc), _ptr(fill), _ptr(capacity),
                           _ptr(buf), _stream(stream)))


def moe_expert_ffn(shape: Shape, buf, W1, b1, W2, b2, fill, capacity, pre, h, y, stream=None) -> None:
    _check(_lib.moe_expert_ffn(ctypes.byref(shape.c()), _ptr(buf), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                               _ptr(fill), _ptr(capacity), _ptr(pre), _ptr(h), _ptr(y), _stream(stream)))


def moe_expert_fc1(shape: Shape, buf, W1, b1, fill, capacity, pre, h, stream=None) -> None:
    _check(_lib.moe_expert_fc1(ctypes.byref(shape.c()), _ptr(buf), _ptr(W1), _ptr(b1), _ptr(fill), _ptr(capacity),
                               _ptr(pre), _ptr(h), _stream(stream)))


def moe_expert_fc2(shape: Shape, h, W2, b2, fill, capacity, y, stream=None) -> None:
    _check(_lib.moe_expert_fc2(ctypes.byref(shape.c()), _ptr(h), _ptr(W2), _ptr(b2), _ptr(fill), _ptr(capacity),
                               _ptr(y), _stream(stream)))


def moe_expert_ffn_window(shape: Shape, buf, W1, b1, W2, b2, fill, capacity, slot_begin: int, slot_end: int, pre,
                          h, y, stream=None) -> None:
    _check(_lib.moe_expert_ffn_window(ctypes.byref(shape.c()), _ptr(buf), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                      _ptr(fill), _ptr(capacity), int(slot_begin), int(slot_end), _ptr(pre), _ptr(h),
                                      _ptr(y), _stream(stream)))


def pipeline_windows(shape: Shape, d: int):
    """The d slot windows [begin, end) that cut the host capacity bound into near-equal chunks."""
    cmax = moe_capacity_bound(shape)
    w = -(-cmax // d)
    return [(i * w, min(cmax, (i + 1) * w)) for i in range(d) if i * w < cmax]


def layer_forward_pipelined(shape: Shape, x, W1, b1, W2, b2, chunks: int, streams, events, logits=None, Wg=None,
                            bufs=None, stream=None):
    """moe_layer_forward_pipelined: the expert FFN in ``chunks`` capacity windows on the given torch
    streams (``events``: len(streams) + 1 torch events, created with default flags)."""
    if bufs is None:
        bufs = alloc_forward(shape, x.device, gate_projection=Wg is not None)
    for e_ in events:  # a torch event is created lazily, on its first record
        if e_.cuda_event == 0:
            e_.record()
    sp = (ctypes.c_void_p * len(streams))(*[st.cuda_stream for st in streams])
    ep = (ctypes.c_void_p * len(events))(*[e_.cuda_event for e_ in events])
    lo = bufs["logits"] if Wg is not None else None
    _check(_lib.moe_layer_forward_pipelined(
        ctypes.byref(shape.c()), _ptr(x), _ptr(logits), _ptr(Wg), _ptr(lo), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
        _ptr(bufs["idx"]), _ptr(bufs["loc"]), _ptr(bufs["gates"]), _ptr(bufs["needed"]), _ptr(bufs["fill"]),
        _ptr(bufs["capacity"]), _ptr(bufs["slot_route"]), _ptr(bufs["buf"]), _ptr(bufs["pre"]), _ptr(bufs["h"]),
        _ptr(bufs["y"]), _ptr(bufs["out"]), *_ws_args(bufs["ws"]), int(chunks), sp, len(streams), ep,
        _stream(stream)))
    return bufs


def moe_decode(shape: Shape, y, gates, idx, loc, capacity, out, stream=None) -> None:
    _check(_lib.moe_decode(ctypes.byref(shape.c()), _ptr(y), _ptr(gates), _ptr(idx), _ptr(loc), _ptr(capacity),
                           _ptr(out), _stream(stream)))


def _ws_args(ws):
    return _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size()


def moe_mx_quantize(fmt: int, src, codes, scales, dtype: int = None, stream=None) -> None:
    """MX-quantise the rows of ``src`` ([..., K], fp32 or bf16) into codes / scales (uint8)."""
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    if dtype is None:
        dtype = MOE_DT_F32 if src.dtype == torch.float32 else MOE_DT_BF16
    _check(_lib.moe_mx_quantize(fmt, rows, K, dtype, _ptr(src), _ptr(codes), _ptr(scales), _stream(stream)))


def mx_alloc(shape_rows_k, fmt: int, device="cuda"):
    """Empty (codes, scales) for an MX matrix of the given [..., K] shape."""
    *lead, K = shape_rows_k
    cb = K if fmt == MOE_MX_FP8 else K // 2
    return (torch.empty(*lead, cb, dtype=torch.uint8, device=device),
            torch.empty(*lead, K // 32, dtype=torch.uint8, device=device))


def mx_quantize_weights(W, fmt: int):
    """(codes, scales) of a weight tensor quantised along its last (input) dimension."""
    codes, scales = mx_alloc(tuple(W.shape), fmt, W.device)
    moe_mx_quantize(fmt, W, codes, scales)
    return codes, scales


def moe_encode_mx(shape: Shape, x, idx, loc, fill, capacity, buf_codes, buf_scales, stream=None) -> None:
    _check(_lib.moe_encode_mx(ctypes.byref(shape.c()), _ptr(x), _ptr(idx), _ptr(loc), _ptr(fill), _ptr(capacity),
                              _ptr(buf_codes), _ptr(buf_scales), _stream(stream)))


def moe_expert_ffn_mx(shape: Shape, wfmt: int, buf_codes, buf_scales, W1q, b1, W2q, b2, fill, capacity, h_codes,
                      h_scales, y, stream=None) -> None:
    _check(_lib.moe_expert_ffn_mx(ctypes.byref(shape.c()), wfmt, _ptr(buf_codes), _ptr(buf_scales), _ptr(W1q[0]),
                                  _ptr(W1q[1]), _ptr(b1), _ptr(W2q[0]), _ptr(W2q[1]), _ptr(b2), _ptr(fill),
                                  _ptr(capacity), _ptr(h_codes), _ptr(h_scales), _ptr(y), _stream(stream)))


def moe_expert_fc1_mx(shape: Shape, wfmt: int, buf_codes, buf_scales, W1q, b1, fill, capacity, h_codes, h_scales,
                      stream=None) -> None:
    _check(_lib.moe_expert_fc1_mx(ctypes.byref(shape.c()), wfmt, _ptr(buf_codes), _ptr(buf_scales), _ptr(W1q[0]),
                                  _ptr(W1q[1]), _ptr(b1), _ptr(fill), _ptr(capacity), _ptr(h_codes), _ptr(h_scales),
                                  _stream(stream)))


def moe_expert_fc2_mx(shape: Shape, wfmt: int, h_codes, h_scales, W2q, b2, fill, capacity, y, stream=None) -> None:
    _check(_lib.moe_expert_fc2_mx(ctypes.byref(shape.c()), wfmt, _ptr(h_codes), _ptr(h_scales), _ptr(W2q[0]),
                                  _ptr(W2q[1]), _ptr(b2), _ptr(fill), _ptr(capacity), _ptr(y), _stream(stream)))


def alloc_forward_mx(shape: Shape, device="cuda", gate_projection: bool = False) -> Dict[str, torch.Tensor]:
    """Buffers of the MX forward: the bf16 forward's route tables, out, y and workspace, with
    the expert buffer and h as MXFP8 codes and scales."""
    b = alloc_forward(shape, device, gate_projection=gate_projection)
    cmax = moe_capacity_bound(shape)
    S, M, E, H = shape.S, shape.M, shape.E, shape.H
    b["buf_codes"], b["buf_scales"] = mx_alloc((E * cmax, M), MOE_MX_FP8, device)
    b["h_codes"], b["h_scales"] = mx_alloc((E * cmax, H), MOE_MX_FP8, device)
    del b["buf"], b["h"]
    return b


def layer_forward_mx(shape: Shape, wfmt: int, x, W1q, b1, W2q, b2, logits=None, Wg=None, bufs=None, stream=None):
    """The fused MX forward (W1q, W2q = (codes, scales) from mx_quantize_weights)."""
    if bufs is None:
        bufs = alloc_forward_mx(shape, x.device, gate_projection=Wg is not None)
    lo = bufs["logits"] if Wg is not None else None
    _check(_lib.moe_layer_forward_mx(
        ctypes.byref(shape.c()), wfmt, _ptr(x), _ptr(logits), _ptr(Wg), _ptr(lo), _ptr(W1q[0]), _ptr(W1q[1]),
        _ptr(b1), _ptr(W2q[0]), _ptr(W2q[1]), _ptr(b2), _ptr(bufs["idx"]), _ptr(bufs["loc"]), _ptr(bufs["gates"]),
        _ptr(bufs["needed"]), _ptr(bufs["fill"]), _ptr(bufs["capacity"]), _ptr(bufs["slot_route"]),
        _ptr(bufs["buf_codes"]), _ptr(bufs["buf_scales"]), _ptr(bufs["h_codes"]), _ptr(bufs["h_scales"]),
        _ptr(bufs["y"]), _ptr(bufs["out"]), *_ws_args(bufs["ws"]), _stream(stream)))
    return bufs


# ---------------------------------------------------------------- block-wise FP8 experts

BLOCK = 128  # block edge: 128 x 128 weight blocks, 1 x 128 token blocks


def moe_blockfp8_quantize(src, brows: int, codes, scales, dtype: int = None, stream=None) -> None:
    """Block-FP8-quantise ``src`` ([..., K], fp32 or bf16, rows a multiple of brows) into codes
    (uint8, same shape) and scales (fp32, [rows / brows, K / 128])."""
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    if dtype is None:
        dtype = MOE_DT_F32 if src.dtype == torch.float32 else MOE_DT_BF16
    _check(_lib.moe_blockfp8_quantize(rows, K, brows, dtype, _ptr(src), _ptr(codes), _ptr(scales), _stream(stream)))


def blockfp8_alloc(shape_rows_k, brows: int, device="cuda"):
    """Empty (codes, scales) for a block-FP8 matrix of the given [..., R, K] shape: scales
    [..., R / brows, K / 128]."""
    *lead, R, K = shape_rows_k
    return (torch.empty(*lead, R, K, dtype=torch.uint8, device=device),
            torch.empty(*lead, R // brows, K // BLOCK, dtype=torch.float32, device=device))


def blockfp8_quantize_weights(W):
    """(codes, scales) of expert weights [E, N, K] in 128 x 128 blocks along the input dimension."""
    codes, scales = blockfp8_alloc(tuple(W.shape), BLOCK, W.device)
    moe_blockfp8_quantize(W, BLOCK, codes, scales)
    return codes, scales


def moe_encode_blockfp8(shape: Shape, x, idx, loc, fill, capacity, buf_codes, buf_scales, stream=None) -> None:
    _check(_lib.moe_encode_blockfp8(ctypes.byref(shape.c()), _ptr(x), _ptr(idx), _ptr(loc), _ptr(fill),
                                    _ptr(capacity), _ptr(buf_codes), _ptr(buf_scales), _stream(stream)))


def moe_expert_ffn_blockfp8(shape: Shape, buf_codes, buf_scales, W1q, b1, W2q, b2, fill, capacity, h_codes, h_scales,
                            y, stream=None) -> None:
    _check(_lib.moe_expert_ffn_blockfp8(ctypes.byref(shape.c()), _ptr(buf_codes), _ptr(buf_scales), _ptr(W1q[0]),
                                        _ptr(W1q[1]), _ptr(b1), _ptr(W2q[0]), _ptr(W2q[1]), _ptr(b2), _ptr(fill),
                                        _ptr(capacity), _ptr(h_codes), _ptr(h_scales), _ptr(y), _stream(stream)))


def moe_expert_fc1_blockfp8(shape: Shape, buf_codes, buf_scales, W1q, b1, fill, capacity, h_codes, h_scales,
                            stream=None) -> None:
    _check(_lib.moe_expert_fc1_blockfp8(ctypes.byref(shape.c()), _ptr(buf_codes), _ptr(buf_scales), _ptr(W1q[0]),
                                        _ptr(W1q[1]), _ptr(b1), _ptr(fill), _ptr(capacity), _ptr(h_codes),
                                        _ptr(h_scales), _stream(stream)))


def moe_expert_fc2_blockfp8(shape: Shape, h_codes, h_scales, W2q, b2, fill, capacity, y, stream=None) -> None:
    _check(_lib.moe_expert_fc2_blockfp8(ctypes.byref(shape.c()), _ptr(h_codes), _ptr(h_scales), _ptr(W2q[0]),
                                        _ptr(W2q[1]), _ptr(b2), _ptr(fill), _ptr(capacity), _ptr(y), _stream(stream)))


def alloc_forward_blockfp8(shape: Shape, device="cuda", gate_projection: bool = False) -> Dict[str, torch.Tensor]:
    """Buffers of the block-FP8 forward: the bf16 forward's route tables, out, y and workspace,
    with the expert buffer and h as E4M3 codes and fp32 scales per 128 features."""
    b = alloc_forward(shape, device, gate_projection=gate_projection)
    cmax = moe_capacity_bound(shape)
    M, E, H = shape.M, shape.E, shape.H
    b["buf_codes"], b["buf_scales"] = blockfp8_alloc((E * cmax, M), 1, device)
    b["h_codes"], b["h_scales"] = blockfp8_alloc((E * cmax, H), 1, device)
    del b["buf"], b["h"]
    return b


def layer_forward_blockfp8(shape: Shape, x, W1q, b1, W2q, b2, logits=None, Wg=None, bufs=None, stream=None):
    """The fused block-FP8 forward (W1q, W2q = (codes, scales) from blockfp8_quantize_weights)."""
    if bufs is None:
        bufs = alloc_forward_blockfp8(shape, x.device, gate_projection=Wg is not None)
    lo = bufs["logits"] if Wg is not None else None
    _check(_lib.moe_layer_forward_blockfp8(
        ctypes.byref(shape.c()), _ptr(x), _ptr(logits), _ptr(Wg), _ptr(lo), _ptr(W1q[0]), _ptr(W1q[1]),
        _ptr(b1), _ptr(W2q[0]), _ptr(W2q[1]), _ptr(b2), _ptr(bufs["idx"]), _ptr(bufs["loc"]), _ptr(bufs["gates"]),
        _ptr(bufs["needed"]), _ptr(bufs["fill"]), _ptr(bufs["capacity"]), _ptr(bufs["slot_route"]),
        _ptr(bufs["buf_codes"]), _ptr(bufs["buf_scales"]), _ptr(bufs["h_codes"]), _ptr(bufs["h_scales"]),
        _ptr(bufs["y"]), _ptr(bufs["out"]), *_ws_args(bufs["ws"]), _stream(stream)))
    return bufs


def moe_residual_ffn(shape: Shape, x, W1r, b1r, W2r, b2r, pre_r, h_r, y_r, ws, stream=None) -> None:
    _check(_lib.moe_residual_ffn(ctypes.byref(shape.c()), _ptr(x), _ptr(W1r), _ptr(b1r), _ptr(W2r), _ptr(b2r),
                                 _ptr(pre_r), _ptr(h_r), _ptr(y_r), *_ws_args(ws), _stream(stream)))


def moe_residual_backward(shape: Shape, dout, x, pre_r, h_r, W1r, W2r, dpre_r, dx_r, dW1r, db1r, dW2r, db2r, ws,
                          stream=None) -> None:
    _check(_lib.moe_residual_backward(ctypes.byref(shape.c()), _ptr(dout), _ptr(x), _ptr(pre_r), _ptr(h_r),
                                      _ptr(W1r), _ptr(W2r), _ptr(dpre_r), _ptr(dx_r), _ptr(dW1r), _ptr(db1r),
                                      _ptr(dW2r), _ptr(db2r), *_ws_args(ws), _stream(stream)))


def moe_decode_residual(shape: Shape, y, gates, idx, loc, capacity, y_r, out, stream=None) -> None:
    _check(_lib.moe_decode_residual(ctypes.byref(shape.c()), _ptr(y), _ptr(gates), _ptr(idx), _ptr(loc),
                                    _ptr(capacity), _ptr(y_r), _ptr(out), _stream(stream)))


def moe_residual_layer_forward(shape: Shape, x, logits_in, Wg, logits_out, W1, b1, W2, b2, W1r, b1r, W2r, b2r,
                               idx, loc, gates, needed, fill, capacity, slot_route, buf, pre, h, y, pre_r, h_r, y_r,
                               out, ws, stream=None) -> None:
    _check(_lib.moe_residual_layer_forward(
        ctypes.byref(shape.c()), _ptr(x), _ptr(logits_in), _ptr(Wg), _ptr(logits_out), _ptr(W1), _ptr(b1), _ptr(W2),
        _ptr(b2), _ptr(W1r), _ptr(b1r), _ptr(W2r), _ptr(b2r), _ptr(idx), _ptr(loc), _ptr(gates), _ptr(needed),
        _ptr(fill), _ptr(capacity), _ptr(slot_route), _ptr(buf), _ptr(pre), _ptr(h), _ptr(y), _ptr(pre_r), _ptr(h_r),
        _ptr(y_r), _ptr(out), *_ws_args(ws), _stream(stream)))


def moe_gate_backward(shape: Shape, logits, idx, dgates, needed, aux_coef, dlogits, aux_loss, ws,
                      stream=None) -> None:
    _check(_lib.moe_gate_backward(ctypes.byref(shape.c()), _ptr(logits), _ptr(idx), _ptr(dgates), _ptr(needed),
                                  float(aux_coef), _ptr(dlogits), _ptr(aux_loss), *_ws_args(ws), _stream(stream)))


def moe_gate_weight_grad(shape: Shape, x, dlogits, dWg, ws, stream=None) -> None:
    _check(_lib.moe_gate_weight_grad(ctypes.byref(shape.c()), _ptr(x), _ptr(dlogits), _ptr(dWg), *_ws_args(ws),
                                     _stream(stream)))


def moe_layer_forward(shape: Shape, x, logits_in, Wg, logits_out, W1, b1, W2, b2, idx, loc, gates, needed, fill,
                      capacity, slot_route, buf, pre, h, y, out, ws, stream=None) -> None:
    _check(_lib.moe_layer_forward(
        ctypes.byref(shape.c()), _ptr(x), _ptr(logits_in), _ptr(Wg), _ptr(logits_out), _ptr(W1), _ptr(b1), _ptr(W2),
        _ptr(b2), _ptr(idx), _ptr(loc), _ptr(gates), _ptr(needed), _ptr(fill), _ptr(capacity), _ptr(slot_route),
        _ptr(buf), _ptr(pre), _ptr(h), _ptr(y), _ptr(out), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), _stream(stream)))


def moe_layer_forward_noalloc(shape: Shape, x, logits_in, Wg, logits_out, W1, b1, W2, b2, idx, loc, gates, needed,
                              fill, capacity, slot_route, buf, pre, h, y, out, stream=None) -> None:
    _check(_lib.moe_layer_forward_noalloc(
        ctypes.byref(shape.c()), _ptr(x), _ptr(logits_in), _ptr(Wg), _ptr(logits_out), _ptr(W1), _ptr(b1), _ptr(W2),
        _ptr(b2), _ptr(idx), _ptr(loc), _ptr(gates), _ptr(needed), _ptr(fill), _ptr(capacity), _ptr(slot_route),
        _ptr(buf), _ptr(pre), _ptr(h), _ptr(y), _ptr(out), _stream(stream)))


def moe_layer_backward(shape: Shape, dout, buf, pre, h, y, gates, idx, loc, fill, capacity, W1, W2, dy, dpre, dbuf,
                       dx, dW1, db1, dW2, db2, dgates, logits=None, needed=None, aux_coef=0.0, x=None, Wg=None,
                       dlogits=None, dWg=None, aux_loss=None, ws=None, stream=None) -> None:
    _check(_lib.moe_layer_backward(
        ctypes.byref(shape.c()), _ptr(dout), _ptr(buf), _ptr(pre), _ptr(h), _ptr(y), _ptr(gates), _ptr(idx),
        _ptr(loc), _ptr(fill), _ptr(capacity), _ptr(W1), _ptr(W2), _ptr(dy), _ptr(dpre), _ptr(dbuf), _ptr(dx),
        _ptr(dW1), _ptr(db1), _ptr(dW2), _ptr(db2), _ptr(dgates), _ptr(logits), _ptr(needed), float(aux_coef),
        _ptr(x), _ptr(Wg), _ptr(dlogits), _ptr(dWg), _ptr(aux_loss), *_ws_args(ws), _stream(stream)))


def moe_residual_layer_backward(shape: Shape, dout, buf, pre, h, y, gates, idx, loc, fill, capacity, W1, W2, dy, dpre,
                                dbuf, dx, dW1, db1, dW2, db2, dgates, W1r, W2r, pre_r, h_r, dpre_r, dx_r, dW1r, db1r,
                                dW2r, db2r, ws, logits=None, needed=None, aux_coef=0.0, x=None, Wg=None,
                                dlogits=None, dWg=None, aux_loss=None, stream=None) -> None:
    _check(_lib.moe_residual_layer_backward(
        ctypes.byref(shape.c()), _ptr(dout), _ptr(buf), _ptr(pre), _ptr(h), _ptr(y), _ptr(gates), _ptr(idx),
        _ptr(loc), _ptr(fill), _ptr(capacity), _ptr(W1), _ptr(W2), _ptr(dy), _ptr(dpre), _ptr(dbuf), _ptr(dx),
        _ptr(dW1), _ptr(db1), _ptr(dW2), _ptr(db2), _ptr(dgates), _ptr(logits), _ptr(needed), float(aux_coef),
        _ptr(x), _ptr(Wg), _ptr(dlogits), _ptr(dWg), _ptr(aux_loss), _ptr(W1r), _ptr(W2r), _ptr(pre_r), _ptr(h_r),
        _ptr(dpre_r), _ptr(dx_r), _ptr(dW1r), _ptr(db1r), _ptr(dW2r), _ptr(db2r), *_ws_args(ws), _stream(stream)))


def moe_decode_backward(shape: Shape, dout, y, gates, idx, loc, capacity, dy, dgates, stream=None) -> None:
    _check(_lib.moe_decode_backward(ctypes.byref(shape.c()), _ptr(dout), _ptr(y), _ptr(gates), _ptr(idx), _ptr(loc),
                                    _ptr(capacity), _ptr(dy), _ptr(dgates), _stream(stream)))


def moe_expert_fc2_backward_data(shape: Shape, dy, W2, pre, fill, capacity, dpre, stream=None) -> None:
    _check(_lib.moe_expert_fc2_backward_data(ctypes.byref(shape.c()), _ptr(dy), _ptr(W2), _ptr(pre), _ptr(fill),
                                             _ptr(capacity), _ptr(dpre), _stream(stream)))


def moe_expert_fc2_weight_grad(shape: Shape, dy, h, fill, capacity, dW2, db2, stream=None) -> None:
    _check(_lib.moe_expert_fc2_weight_grad(ctypes.byref(shape.c()), _ptr(dy), _ptr(h), _ptr(fill), _ptr(capacity),
                                           _ptr(dW2), _ptr(db2), _stream(stream)))


def moe_expert_fc1_backward_data(shape: Shape, dpre, W1, fill, capacity, dbuf, stream=None) -> None:
    _check(_lib.moe_expert_fc1_backward_data(ctypes.byref(shape.c()), _ptr(dpre), _ptr(W1), _ptr(fill),
                                             _ptr(capacity), _ptr(dbuf), _stream(stream)))


def moe_expert_fc1_weight_grad(shape: Shape, dpre, buf, fill, capacity, dW1, db1, stream=None) -> None:
    _check(_lib.moe_expert_fc1_weight_grad(ctypes.byref(shape.c()), _ptr(dpre), _ptr(buf), _ptr(fill),
                                           _ptr(capacity), _ptr(dW1), _ptr(db1), _stream(stream)))


def moe_encode_backward(shape: Shape, dbuf, idx, loc, capacity, dx, stream=None) -> None:
    _check(_lib.moe_encode_backward(ctypes.byref(shape.c()), _ptr(dbuf), _ptr(idx), _ptr(loc), _ptr(capacity),
                                    _ptr(dx), _stream(stream)))


# ---------------------------------------------------------------- buffers

def alloc_forward(shape: Shape, device="cuda", training: bool = False,
                  gate_projection: bool = False, residual: bool = False) -> Dict[str, torch.Tensor]:
    """Allocate every output and scratch buffer the forward writes, sized with the host
    capacity bound (torch.empty: contents undefined until the library writes them);
    residual adds the dense branch's h_r [S, H] and y_r [S, M] (and pre_r [S, H] when training)."""
    S, M, E, k, H = shape.S, shape.M, shape.E, shape.k, shape.H
    cmax = moe_capacity_bound(shape)
    dt = shape.torch_dtype
    i32 = dict(dtype=torch.int32, device=device)
    bufs = dict(
        idx=torch.empty(k, S, **i32), loc=torch.empty(k, S, **i32),
        gates=torch.empty(k, S, dtype=torch.float32, device=device),
        needed=torch.empty(E, **i32), fill=torch.empty(E, **i32), capacity=torch.empty(1, **i32),
        slot_route=torch.empty(E * cmax, **i32),
        buf=torch.empty(E * cmax, M, dtype=dt, device=device),
        h=torch.empty(E * cmax, H, dtype=dt, device=device),
        y=torch.empty(E * cmax, M, dtype=dt, device=device),
        out=torch.empty(S, M, dtype=dt, device=device),
        ws=torch.empty(max(1, moe_workspace_size(shape)), dtype=torch.uint8, device=device),
    )
    bufs["pre"] = torch.empty(E * cmax, H, dtype=dt, device=device) if training else None
    bufs["logits"] = torch.empty(S, E, dtype=torch.float32, device=device) if gate_projection else None
    bufs["h_r"] = torch.empty(S, H, dtype=dt, device=device) if residual else None
    bufs["y_r"] = torch.empty(S, M, dtype=dt, device=device) if residual else None
    bufs["pre_r"] = torch.empty(S, H, dtype=dt, device=device) if residual and training else None
    return bufs


def layer_forward(shape: Shape, x, W1, b1, W2, b2, logits=None, Wg=None, bufs=None, training=False,
                  residual=None, stream=None):
    """Run the fused forward into ``bufs`` (allocated if None) and return them. ``residual``:
    the Residual-MoE dense branch's weights as a dict W1r, b1r, W2r, b2r (biases may be None)."""
    if bufs is None:
        bufs = alloc_forward(shape, x.device, training=training, gate_projection=Wg is not None,
                             residual=residual is not None)
    lo = bufs["logits"] if Wg is not None else None
    if residual is None:
        moe_layer_forward(shape, x, logits, Wg, lo, W1, b1, W2, b2,
                          bufs["idx"], bufs["loc"], bufs["gates"], bufs["needed"], bufs["fill"], bufs["capacity"],
                          bufs["slot_route"], bufs["buf"], bufs["pre"], bufs["h"], bufs["y"], bufs["out"], bufs["ws"],
                          stream)
    else:
        moe_residual_layer_forward(shape, x, logits, Wg, lo, W1, b1, W2, b2, residual["W1r"], residual.get("b1r"),
                                   residual["W2r"], residual.get("b2r"), bufs["idx"], bufs["loc"], bufs["gates"],
                                   bufs["needed"], bufs["fill"], bufs["capacity"], bufs["slot_route"], bufs["buf"],
                                   bufs["pre"], bufs["h"], bufs["y"], bufs["pre_r"], bufs["h_r"], bufs["y_r"],
                                   bufs["out"], bufs["ws"], stream)
    return bufs


def alloc_backward(shape: Shape, device="cuda", gate: bool = False,
                   gate_projection: bool = False, residual: bool = False) -> Dict[str, torch.Tensor]:
    """Gradient buffers; gate adds dlogits and aux_loss, gate_projection also dWg; residual the
    dense branch's dpre_r, dx_r and its weight and bias gradients."""
    S, M, E, k, H = shape.S, shape.M, shape.E, shape.k, shape.H
    cmax = moe_capacity_bound(shape)
    dt = shape.torch_dtype
    f32 = dict(dtype=torch.float32, device=device)
    dyb = torch.empty(E * cmax, M, dtype=dt, device=device)
    res = {}
    if residual:
        res = dict(dpre_r=torch.empty(S, H, dtype=dt, device=device), dx_r=torch.empty(S, M, dtype=dt, device=device),
                   dW1r=torch.empty(H, M, **f32), dW2r=torch.empty(M, H, **f32),
                   db1r=torch.empty(H, **f32) if shape.has_fc1_bias else None,
                   db2r=torch.empty(M, **f32) if shape.has_fc2_bias else None)
    return dict(**res,
        dlogits=torch.empty(S, E, **f32) if gate or gate_projection else None,
        aux_loss=torch.empty(1, **f32) if gate or gate_projection else None,
        dWg=torch.empty(M, E, **f32) if gate_projection else None,
        dy=dyb, dbuf=dyb,  # dbuf reuses dy's memory (allowed by the ABI)
        dpre=torch.empty(E * cmax, H, dtype=dt, device=device),
        dx=torch.empty(S, M, dtype=dt, device=device),
        dW1=torch.empty(E, H, M, **f32), dW2=torch.empty(E, M, H, **f32),
        db1=torch.empty(E, H, **f32) if shape.has_fc1_bias else None,
        db2=torch.empty(E, M, **f32) if shape.has_fc2_bias else None,
        dgates=torch.empty(k, S, **f32),
    )


def layer_backward(shape: Shape, fw: Dict[str, torch.Tensor], dout, W1, W2, grads=None, logits=None, x=None,
                   Wg=None, aux_coef=AUX_COEF, residual=None, stream=None):
    """The fused backward into ``grads`` (allocated if None). With ``logits`` (the forward's;
    ``fw["logits"]`` for a projected gate) it includes the gate backward and the auxiliary
    load-balance loss of coefficient ``aux_coef``; with ``Wg`` and ``x`` also dWg and the gate
    projection's share of dx. ``residual``: the Residual-MoE dense branch's weights (a dict with
    W1r and W2r; ``fw`` from a training forward with the branch, ``x`` required): adds its
    backward, and its dx_r to dx."""
    if grads is None:
        grads = alloc_backward(shape, dout.device, gate=logits is not None, gate_projection=Wg is not None,
                               residual=residual is not None)
    gate = logits is not None
    if residual is not None:
        moe_residual_layer_backward(
            shape, dout, fw["buf"], fw["pre"], fw["h"], fw["y"], fw["gates"], fw["idx"], fw["loc"], fw["fill"],
            fw["capacity"], W1, W2, grads["dy"], grads["dpre"], grads["dbuf"], grads["dx"], grads["dW1"], grads["db1"],
            grads["dW2"], grads["db2"], grads["dgates"], residual["W1r"], residual["W2r"], fw["pre_r"], fw["h_r"],
            grads["dpre_r"], grads["dx_r"], grads["dW1r"], grads["db1r"], grads["dW2r"], grads["db2r"], fw["ws"],
            logits=logits, needed=fw["needed"] if gate else None, aux_coef=aux_coef if gate else 0.0, x=x, Wg=Wg,
            dlogits=grads["dlogits"] if gate else None, dWg=grads["dWg"] if Wg is not None else None,
            aux_loss=grads["aux_loss"] if gate else None, stream=stream)
        return grads
    moe_layer_backward(shape, dout, fw["buf"], fw["pre"], fw["h"], fw["y"], fw["gates"], fw["idx"], fw["loc"],
                       fw["fill"], fw["capacity"], W1, W2, grads["dy"], grads["dpre"], grads["dbuf"], grads["dx"],
                       grads["dW1"], grads["db1"], grads["dW2"], grads["db2"], grads["dgates"],
                       logits=logits, needed=fw["needed"] if gate else None, aux_coef=aux_coef if gate else 0.0,
                       x=x if Wg is not None else None, Wg=Wg,
                       dlogits=grads["dlogits"] if gate else None, dWg=grads["dWg"] if Wg is not None else None,
                       aux_loss=grads["aux_loss"] if gate else None, ws=fw["ws"] if gate else None, stream=stream)
    return grads


# ---------------------------------------------------------------- NVFP4 experts (weights)

NVFP4_BLOCK = 16  # values per E4M3-scaled block along the reduction dimension


def moe_nvfp4_quantize(src, ntensor: int, codes, scales, g, dtype: int = None, stream=None) -> None:
    """NVFP4-quantise ``src`` ([..., K], fp32 or bf16, K a multiple of 16) as ntensor tensors of
    consecutive rows into codes (uint8 [rows, K/2]), scales (uint8 E4M3 [rows, K/16]) and g (fp32
    [ntensor])."""
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    if dtype is None:
        dtype = MOE_DT_F32 if src.dtype == torch.float32 else MOE_DT_BF16
    _check(_lib.moe_nvfp4_quantize(rows, K, ntensor, dtype, _ptr(src), _ptr(codes), _ptr(scales), _ptr(g),
                                   _stream(stream)))


def nvfp4_quantize_weights(W):
    """(codes [E, N, K/2], scales [E, N, K/16], g [E]) of expert weights W [E, N, K], one tensor
    (one fp32 scale) per expert."""
    E, N, K = W.shape
    codes = torch.empty(E, N, K // 2, dtype=torch.uint8, device=W.device)
    scales = torch.empty(E, N, K // NVFP4_BLOCK, dtype=torch.uint8, device=W.device)
    g = torch.empty(E, dtype=torch.float32, device=W.device)
    moe_nvfp4_quantize(W, E, codes, scales, g)
    return codes, scales, g


def moe_expert_ffn_nvfp4(shape: Shape, buf, W1q, b1, W2q, b2, fill, capacity, pre, h, y, stream=None) -> None:
    """Expert FFN with NVFP4 weights W1q, W2q = (codes, scales, g) from nvfp4_quantize_weights."""
    _check(_lib.moe_expert_ffn_nvfp4(ctypes.byref(shape.c()), _ptr(buf), _ptr(W1q[0]), _ptr(W1q[1]), _ptr(W1q[2]),
                                     _ptr(b1), _ptr(W2q[0]), _ptr(W2q[1]), _ptr(W2q[2]), _ptr(b2), _ptr(fill),
                                     _ptr(capacity), _ptr(pre), _ptr(h), _ptr(y), _stream(stream)))


def moe_expert_fc1_nvfp4(shape: Shape, buf, W1q, b1, fill, capacity, pre, h, stream=None) -> None:
    _check(_lib.moe_expert_fc1_nvfp4(ctypes.byref(shape.c()), _ptr(buf), _ptr(W1q[0]), _ptr(W1q[1]), _ptr(W1q[2]),
                                     _ptr(b1), _ptr(fill), _ptr(capacity), _ptr(pre), _ptr(h), _stream(stream)))


def moe_expert_fc2_nvfp4(shape: Shape, h, W2q, b2, fill, capacity, y, stream=None) -> None:
    _check(_lib.moe_expert_fc2_nvfp4(ctypes.byref(shape.c()), _ptr(h), _ptr(W2q[0]), _ptr(W2q[1]), _ptr(W2q[2]),
                                     _ptr(b2), _ptr(fill), _ptr(capacity), _ptr(y), _stream(stream)))


def layer_forward_nvfp4(shape: Shape, x, W1q, b1, W2q, b2, logits=None, Wg=None, bufs=None, stream=None):
    """The fused forward (inference) with NVFP4 experts into ``bufs`` (alloc_forward's, allocated
    if None)."""
    if bufs is None:
        bufs = alloc_forward(shape, x.device, gate_projection=Wg is not None)
    lo = bufs["logits"] if Wg is not None else None
    _check(_lib.moe_layer_forward_nvfp4(
        ctypes.byref(shape.c()), _ptr(x), _ptr(logits), _ptr(Wg), _ptr(lo), _ptr(W1q[0]), _ptr(W1q[1]), _ptr(W1q[2]),
        _ptr(b1), _ptr(W2q[0]), _ptr(W2q[1]), _ptr(W2q[2]), _ptr(b2), _ptr(bufs["idx"]), _ptr(bufs["loc"]),
        _ptr(bufs["gates"]), _ptr(bufs["needed"]), _ptr(bufs["fill"]), _ptr(bufs["capacity"]),
        _ptr(bufs["slot_route"]), _ptr(bufs["buf"]), _ptr(bufs["h"]), _ptr(bufs["y"]), _ptr(bufs["out"]),
        *_ws_args(bufs["ws"]), _stream(stream)))
    return bufs
