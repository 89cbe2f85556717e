"""Seeded synthetic inputs for the single-GPU MoE layer, and the named workloads.

This module holds no arithmetic of the method: it only draws inputs. Both the
HIP path (through its tests and the benchmark) and the CPU oracle read the same
tensors drawn here, so the two sides always see identical bits.

Recipe (the pages' workloads are trained models on datasets, so seeded random
tensors of the same shapes stand in for them):
  * every tensor has its own torch generator, seeded with seed*1000 + tensor id
    (x=1, logits=2, Wg=3, W1=4, b1=5, W2=6, b2=7, dout=8, dgates=9, W1r=10,
    b1r=11, W2r=12, b2r=13; dgates is an upstream gate gradient [k,S] for tests
    of the gate backward on its own; W1r..b2r are the Residual-MoE dense MLP);
  * x ~ N(0,1); logits ~ N(0,1) fp32; Wg, W1, b1, W2, b2, W1r, b1r, W2r, b2r ~
    N(0, 0.02) (0.02 is the standard deviation); dout ~ N(0,1); dgates ~ N(0,1)
    fp32;
  * draws are fp32, then rounded to bf16 (round to nearest even) when the
    workload's dtype is bf16; logits, Wg and gates stay fp32;
  * the skewed workloads add a per-expert bias b_e = 2 (e+1)^-1.1 to every
    token's logits (a Zipf(1.1) law, expert 0 hottest), summed in fp64 and
    rounded once to fp32.

Workload shapes follow the Tutel configuration knobs (k, capacity_factor,
model_dim, experts, hidden size per expert, fc bias flags) described on the
Tutel catalogue page's "key configuration" table and FAQ. The S=8192, M=2048,
E=16, k=3 workload is the shape benchmarked in DeepSpeed PR #8195 ("Results").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

DT_F32 = 0
DT_BF16 = 1
ACT_RELU = 0
ACT_GELU = 1

TENSOR_IDS = {"x": 1, "logits": 2, "Wg": 3, "W1": 4, "b1": 5, "W2": 6, "b2": 7, "dout": 8, "dgates": 9,
              "W1r": 10, "b1r": 11, "W2r": 12, "b2r": 13}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    S: int
    M: int
    E: int
    k: int
    H: int
    capacity_factor: float
    dtype: int = DT_BF16
    act: int = ACT_GELU
    has_fc1_bias: bool = True
    has_fc2_bias: bool = True
    logits: str = "normal"  # "normal" | "gate" (x @ Wg) | "zipf" (normal + Zipf(1.1) bias x2)
    backward: bool = False
    residual: bool = False  # Residual-MoE: a dense MLP branch added to the MoE output
    mx: str = ""  # "mxfp8" / "mxfp4": experts with MX-quantised weights (tokens and h in MXFP8);
    #               "blockfp8": block-wise FP8 experts (weights, tokens and h);
    #               "nvfp4": NVFP4 weights only (tokens and h bf16)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == DT_F32 else torch.bfloat16

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == DT_F32 else 2


# The workloads, smallest first.
TINY_F32 = Workload("tiny_f32_S256_M64_E4_k1_H128", S=256, M=64, E=4, k=1, H=128,
                    capacity_factor=1.0, dtype=DT_F32, act=ACT_RELU)
GATED_BF16 = Workload("gated_bf16_S4096_M1024_E8_k2_H4096", S=4096, M=1024, E=8, k=2, H=4096,
                      capacity_factor=1.25, logits="gate")
# the same layer trained: forward + backward, gate backward and load-balance loss included
GATED_TRAIN_BF16 = GATED_BF16.replace(name="gated_train_bf16_S4096_M1024_E8_k2_H4096", backward=True)
# Residual-MoE at the same size: top-1 expert plus the dense MLP branch (the MoE training
# blog's PR-MoE layers use top-1 gating with the residual branch)
RESIDUAL_BF16 = Workload("residual_bf16_S4096_M1024_E8_k1_H4096", S=4096, M=1024, E=8, k=1, H=4096,
                         capacity_factor=1.25, logits="gate", residual=True)
# ... trained: forward + backward of both branches, gate backward included
RESIDUAL_TRAIN_BF16 = RESIDUAL_BF16.replace(name="residual_train_bf16_S4096_M1024_E8_k1_H4096", backward=True)
DSPR_BF16 = Workload("dspr_bf16_S8192_M2048_E16_k3_H8192", S=8192, M=2048, E=16, k=3, H=8192,
                     capacity_factor=0.0)
FINE_BF16 = Workload("fine_bf16_S16384_M2048_E64_k6_H1408", S=16384, M=2048, E=64, k=6, H=1408,
                     capacity_factor=-1.5, has_fc1_bias=False, has_fc2_bias=False, logits="zipf")
LARGE_BF16 = Workload("large_bf16_S32768_M4096_E128_k8_H1536", S=32768, M=4096, E=128, k=8, H=1536,
                      capacity_factor=-2.0, logits="zipf", backward=True)

# the gated layer with MX low-precision experts (the weights quantised from the same bf16 draws)
GATED_MXFP8 = GATED_BF16.replace(name="gated_mxfp8_S4096_M1024_E8_k2_H4096", mx="mxfp8")
GATED_MXFP4 = GATED_BF16.replace(name="gated_mxfp4_S4096_M1024_E8_k2_H4096", mx="mxfp4")
DSPR_MXFP8 = Workload("dspr_mxfp8_S8192_M2048_E16_k3_H8192", S=8192, M=2048, E=16, k=3, H=8192,
                      capacity_factor=0.0, mx="mxfp8")
# ... and with block-wise FP8 experts (fp32 scales per 128 x 128 weight block, 1 x 128 token block)
GATED_BLOCKFP8 = GATED_BF16.replace(name="gated_blockfp8_S4096_M1024_E8_k2_H4096", mx="blockfp8")
DSPR_BLOCKFP8 = DSPR_MXFP8.replace(name="dspr_blockfp8_S8192_M2048_E16_k3_H8192", mx="blockfp8")
# ... and with NVFP4 weights (weight-only: E2M1 in 16-value blocks with E4M3 scales, bf16 tokens)
GATED_NVFP4 = GATED_BF16.replace(name="gated_nvfp4_S4096_M1024_E8_k2_H4096", mx="nvfp4")
DSPR_NVFP4 = DSPR_MXFP8.replace(name="dspr_nvfp4_S8192_M2048_E16_k3_H8192", mx="nvfp4")

WORKLOADS = [TINY_F32, GATED_BF16, GATED_TRAIN_BF16, RESIDUAL_BF16, RESIDUAL_TRAIN_BF16, DSPR_BF16, FINE_BF16,
             LARGE_BF16]
# MX workloads are measured by bench.py and checked by the MX parity tests
MX_WORKLOADS = [GATED_MXFP8, GATED_MXFP4, DSPR_MXFP8, GATED_BLOCKFP8, DSPR_BLOCKFP8, GATED_NVFP4, DSPR_NVFP4]
BY_NAME = {w.name: w for w in WORKLOADS + MX_WORKLOADS}


def _gen(seed: int, tensor: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + TENSOR_IDS[tensor])
    return g


def normal(shape, seed: int, tensor: str, std: float = 1.0, device="cpu") -> torch.Tensor:
    """fp32 N(0, std^2) draw from the tensor's own generator."""
    t = torch.randn(*shape, generator=_gen(seed, tensor, device), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def zipf_bias(E: int) -> torch.Tensor:
    """Per-expert logit bias 2 (e+1)^-1.1, fp64."""
    e = torch.arange(E, dtype=torch.float64)
    return 2.0 * torch.pow(e + 1.0, -1.1)


def make_inputs(w: Workload, seed: int = 0, device="cpu", with_dout: Optional[bool] = None) -> Dict[str, torch.Tensor]:
    """Draw every input tensor of workload ``w`` on ``device``.

    Returns a dict with x [S,M], W1 [E,H,M], W2 [E,M,H], b1 [E,H] / b2 [E,M]
    (absent when the bias is off), and either logits [S,E] fp32 or Wg [M,E]
    fp32 (gate-projected workloads), the dense branch W1r [H,M], W2r [M,H],
    b1r [H], b2r [M] for Residual-MoE workloads, plus dout [S,M] when a
    backward is asked.
    """
    dt = w.torch_dtype
    out: Dict[str, torch.Tensor] = {}
    out["x"] = normal((w.S, w.M), seed, "x", device=device).to(dt)
    if w.logits == "gate":
        out["Wg"] = normal((w.M, w.E), seed, "Wg", 0.02, device=device)
    else:
        z = normal((w.S, w.E), seed, "logits", device=device)
        if w.logits == "zipf":
            z = (z.double() + zipf_bias(w.E).to(device)).float()
        out["logits"] = z
    out["W1"] = normal((w.E, w.H, w.M), seed, "W1", 0.02, device=device).to(dt)
    out["W2"] = normal((w.E, w.M, w.H), seed, "W2", 0.02, device=device).to(dt)
    if w.has_fc1_bias:
        out["b1"] = normal((w.E, w.H), seed, "b1", 0.02, device=device).to(dt)
    if w.has_fc2_bias:
        out["b2"] = normal((w.E, w.M), seed, "b2", 0.02, device=device).to(dt)
    if w.residual:
        out["W1r"] = normal((w.H, w.M), seed, "W1r", 0.02, device=device).to(dt)
        out["W2r"] = normal((w.M, w.H), seed, "W2r", 0.02, device=device).to(dt)
        if w.has_fc1_bias:
            out["b1r"] = normal((w.H,), seed, "b1r", 0.02, device=device).to(dt)
        if w.has_fc2_bias:
            out["b2r"] = normal((w.M,), seed, "b2r", 0.02, device=device).to(dt)
    if with_dout if with_dout is not None else w.backward:
        out["dout"] = normal((w.S, w.M), seed, "dout", device=device).to(dt)
    return out


def capacity_bound(w: Workload) -> int:
    """Host-known upper bound on the capacity C of a workload.

    f > 0 fixes C = ceil(k S f / E); f = 0 bounds C by S (top-k experts of a
    token are distinct, so no expert can receive more than S routes); f < 0
    bounds C by min(ceil(k S |f| / E), S). C is at least 1.
    """
    f = w.capacity_factor
    if f > 0:
        return max(1, math.ceil((w.k * w.S * f) / w.E))
    if f == 0:
        return max(1, w.S)
    return max(1, min(math.ceil((w.k * w.S * -f) / w.E), w.S))
