"""The C ABI without a GPU: the library loads, exports every entry point the
header declares, and its host-side checks behave as documented (nothing here
launches a kernel)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def moe():
    import combine_softmax_top_amd as m
    return m


def _declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"^\s*(?:moe_status|const char \*)\s*(moe_\w+)\s*\(", text, re.M)))


def odd_ptr():
    return ctypes.c_void_p(0x1008)  # 8-byte aligned only, never dereferenced


def test_every_declared_symbol_is_exported(moe):
    names = _declared()
    assert len(names) == 46, names
    lib = ctypes.CDLL(moe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert names == moe.EXPORTED


def test_binding_arity_matches_header(moe):
    # every prototype's parameter count equals the argument count the binding declares
    with open(os.path.join(ROOT, "include", "moe.h")) as fh:
        text = fh.read()
    protos = re.findall(r"^\s*(?:moe_status|const char \*)\s*(moe_\w+)\s*\(([^;]*?)\);", text, re.M | re.S)
    assert len(protos) == len(_declared())
    for name, params in protos:
        n = 0 if params.strip() in ("", "void") else params.count(",") + 1
        if name == "moe_last_error":
            assert n == 0
            continue
        assert n == len(moe._SIGS[name]), (name, n, len(moe._SIGS[name]))


def test_shape_struct_layout_matches_header(moe):
    # int32 S, M, E, k, H; (4 bytes padding); double; int32 x4
    assert ctypes.sizeof(moe.moe_shape) == 48
    assert moe.moe_shape.capacity_factor.offset == 24


@pytest.mark.parametrize("w", W.WORKLOADS, ids=lambda w: w.name)
def test_capacity_bound_and_workspace(moe, w):
    s = moe.Shape.of(w)
    assert moe.moe_validate(s) == moe.MOE_OK
    assert moe.moe_capacity_bound(s) == W.capacity_bound(w)
    tiles = (w.S + 63) // 64
    assert moe.moe_workspace_size(s) >= 4 * w.E * w.k * tiles


def test_validation_errors(moe):
    ok = moe.Shape(S=64, M=64, E=4, k=2, H=64, capacity_factor=1.0)
    assert moe.moe_validate(ok) == moe.MOE_OK
    bad = [
        (dict(k=5), moe.MOE_EINVAL),            # k > E
        (dict(k=0), moe.MOE_EINVAL),
        (dict(S=-1), moe.MOE_EINVAL),
        (dict(M=0), moe.MOE_EINVAL),
        (dict(dtype=7), moe.MOE_EINVAL),
        (dict(act=9), moe.MOE_EINVAL),
        (dict(capacity_factor=float("nan")), moe.MOE_EINVAL),
        (dict(M=96), moe.MOE_EUNSUPPORTED),      # not a multiple of 64
        (dict(H=100), moe.MOE_EUNSUPPORTED),
        (dict(E=600, k=2), moe.MOE_EUNSUPPORTED),
        (dict(E=64, k=33), moe.MOE_EUNSUPPORTED),
    ]
    import dataclasses
    for change, want in bad:
        s = dataclasses.replace(ok, **change)
        assert moe.moe_validate(s) == want, change
        assert moe.moe_last_error() != ""
    lib = ctypes.CDLL(moe.LIB_PATH)
    lib.moe_validate.argtypes = [ctypes.c_void_p]
    assert lib.moe_validate(None) == moe.MOE_EINVAL


def test_entry_points_reject_before_enqueueing(moe):
    # Every failing check returns before any HIP call, so these run without a GPU.
    s = moe.Shape(S=64, M=64, E=4, k=2, H=64, capacity_factor=1.0)
    c = s.c()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: checks fail first
    lib = moe._lib
    st = lib.moe_route(ctypes.byref(c), None, fake, fake, fake, fake, fake, fake, None, fake, 16, None)
    assert st == moe.MOE_EINVAL  # logits NULL
    st = lib.moe_route(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake, None, fake, 1, None)
    assert st == moe.MOE_EWORKSPACE and "workspace" in moe.moe_last_error()
    st = lib.moe_expert_ffn(ctypes.byref(c), fake, fake, None, fake, fake, fake, fake, None, fake, fake, None)
    assert st == moe.MOE_EINVAL and "b1" in moe.moe_last_error()  # biases on, b1 missing
    st = lib.moe_layer_forward(ctypes.byref(c), fake, fake, fake, fake, *([fake] * 17), 1 << 20, None)
    assert st == moe.MOE_EINVAL  # both logits and Wg given
    st = lib.moe_layer_backward(ctypes.byref(c), *([None] * 23), 0.0, *([None] * 6), 0, None)
    assert st == moe.MOE_EINVAL
    # gate backward argument checks
    st = lib.moe_gate_backward(ctypes.byref(c), fake, fake, fake, None, 0.01, fake, None, fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL and "needed" in moe.moe_last_error()  # aux term without needed
    st = lib.moe_gate_backward(ctypes.byref(c), fake, fake, fake, fake, float("nan"), fake, None, fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL and "aux_coef" in moe.moe_last_error()
    st = lib.moe_gate_backward(ctypes.byref(c), fake, fake, fake, fake, 0.01, fake, fake, fake, 0, None)
    assert st == moe.MOE_EWORKSPACE
    st = lib.moe_gate_weight_grad(ctypes.byref(c), None, fake, fake, fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL  # x NULL with S > 0
    st = lib.moe_gate_weight_grad(ctypes.byref(c), fake, fake, odd_ptr(), fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL and "aligned" in moe.moe_last_error()
    # layer backward: Wg without dWg, and the gate backward without logits
    full = [fake] * 21
    st = lib.moe_layer_backward(ctypes.byref(c), *full[:21], fake, None, 0.0, fake, fake, fake, None, None,
                                fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL and "dWg" in moe.moe_last_error()
    st = lib.moe_layer_backward(ctypes.byref(c), *full[:21], None, None, 0.0, None, None, fake, None, None,
                                None, 0, None)
    assert st == moe.MOE_EINVAL and "logits" in moe.moe_last_error()
    # Residual-MoE backward: the dense branch alone, and inside the layer backward
    st = lib.moe_residual_backward(ctypes.byref(c), fake, fake, fake, fake, None, fake, fake, fake, fake, None, fake,
                                   None, fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL and "W1r" in moe.moe_last_error()
    st = lib.moe_residual_backward(ctypes.byref(c), fake, fake, fake, fake, fake, fake, fake, fake, fake, None, fake,
                                   None, fake, 1, None)
    assert st == moe.MOE_EWORKSPACE
    # NVFP4 experts take bf16 tokens and every weight part
    c32 = moe.Shape(S=64, M=64, E=4, k=2, H=64, capacity_factor=1.0, dtype=moe.MOE_DT_F32).c()
    st = lib.moe_expert_ffn_nvfp4(ctypes.byref(c32), *([fake] * 14), None)
    assert st == moe.MOE_EUNSUPPORTED and "bf16" in moe.moe_last_error()
    st = lib.moe_expert_fc1_nvfp4(ctypes.byref(c), fake, fake, None, fake, fake, fake, fake, None, fake, None)
    assert st == moe.MOE_EINVAL and "W1" in moe.moe_last_error()
    st = lib.moe_layer_forward_nvfp4(ctypes.byref(c), fake, fake, None, None, fake, fake, None, *([fake] * 17),
                                     1 << 20, None)
    assert st == moe.MOE_EINVAL and "scales" in moe.moe_last_error()
    # NVFP4 quantisation: K a multiple of 16, ntensor dividing rows, 16-byte aligned buffers
    st = lib.moe_nvfp4_quantize(64, 24, 1, moe.MOE_DT_BF16, fake, fake, fake, fake, None)
    assert st == moe.MOE_EINVAL and "16" in moe.moe_last_error()
    st = lib.moe_nvfp4_quantize(64, 32, 3, moe.MOE_DT_BF16, fake, fake, fake, fake, None)
    assert st == moe.MOE_EINVAL and "ntensor" in moe.moe_last_error()
    st = lib.moe_nvfp4_quantize(64, 32, 2, moe.MOE_DT_BF16, fake, fake, odd_ptr(), fake, None)
    assert st == moe.MOE_EINVAL and "aligned" in moe.moe_last_error()
    other = ctypes.c_void_p(0x2000)
    res = [fake, fake, fake, fake, fake, other, fake, None, fake, None]  # W1r .. db2r (dx_r distinct from dx)
    st = lib.moe_residual_layer_backward(ctypes.byref(c), *full[:21], None, None, 0.0, fake, None, None, None, None,
                                         *res, None, 0, None)
    assert st == moe.MOE_EWORKSPACE  # the dense branch always needs the workspace
    dx = full[15]
    same = res[:5] + [dx] + res[6:]  # dx_r aliasing dx
    st = lib.moe_residual_layer_backward(ctypes.byref(c), *full[:21], None, None, 0.0, fake, None, None, None, None,
                                         *same, fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL and "dx_r" in moe.moe_last_error()
    st = lib.moe_residual_layer_backward(ctypes.byref(c), *full[:21], None, None, 0.0, None, None, None, None, None,
                                         *res, fake, 1 << 20, None)
    assert st == moe.MOE_EINVAL and "x" in moe.moe_last_error()  # the dense branch reads x
    with pytest.raises(moe.MoeError):
        moe._check(lib.moe_decode(ctypes.byref(c), None, None, None, None, None, None, None))
    odd = odd_ptr()
    st = lib.moe_encode(ctypes.byref(c), odd, fake, fake, fake, fake, fake, None)
    assert st == moe.MOE_EINVAL and "aligned" in moe.moe_last_error()
    st = lib.moe_expert_fc2(ctypes.byref(c), fake, fake, fake, fake, fake, odd, None)
    assert st == moe.MOE_EINVAL and "aligned" in moe.moe_last_error()


def test_noalloc_forward_rejects_before_enqueueing(moe):
    # beyond the static scratch (E*k*ceil(S/64) = 512*32*65 counts > 4 MiB): rejected on the
    # host, before the device is touched
    s = moe.Shape(S=64 * 65, M=64, E=512, k=32, H=64, capacity_factor=1.0)
    fake = ctypes.c_void_p(0x1000)
    st = moe._lib.moe_layer_forward_noalloc(ctypes.byref(s.c()), fake, fake, None, None, *([fake] * 16), None)
    assert st == moe.MOE_EUNSUPPORTED and "static scratch" in moe.moe_last_error()
    st = moe._lib.moe_layer_forward_noalloc(None, *([fake] * 20), None)
    assert st == moe.MOE_EINVAL
