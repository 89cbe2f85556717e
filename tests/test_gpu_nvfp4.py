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
