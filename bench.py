"""Benchmark of the single-GPU MoE layer on MI355X.

One step = one pass of the whole layer over one batch of synthetic input that is
already resident in HBM. The default workload is the largest one that fits one
GPU: S=32768 tokens, M=4096, E=128 experts, top-8, H=1536, bf16, Zipf-skewed
logits, capacity_factor -2.0, forward + backward. Its step is route -> encode ->
fc1 -> fc2 -> decode, then the backward: decode backward (dy, dgates), the gate
backward (dlogits through the softmax and the 0.01 load-balance loss), the four
expert products (dpre with the activation gradient, dW2, dbuf, dW1) and the
encode backward (dx). Gate-projected workloads add the projection (and dWg and
dx's gate share in training); Residual-MoE workloads add the dense branch (and
its backward in training); MX and block-FP8 workloads run their experts on the
fp8 MFMA. The timed region is exactly --steps calls of the fused C-ABI entry
points (moe_layer_forward, moe_layer_backward, or their variants), bracketed by
synchronisations; `value` is tokens per second of that one-stream loop. Forward
workloads also report consecutive batches alternating over two streams
(`multi_stream`), and --graph the step captured in a HIP graph and replayed
(`graph`); neither is `value`.

A second loop times each stage through its own C-ABI entry point (one kernel
each, except route and the gate backward) with HIP events on the stream the
library launches on, and reports it against its roofline: the bytes or flops the
method must move or compute per launch over the stage's average time. HBM-bound
stages run each launch after a 512 MiB buffer fill, so that their operands come
from HBM, not from L2 or the Infinity Cache, each launch bracketed by events of
its own (the interval includes its dispatch); MFMA-bound stages run in
back-to-back batches. `roofline` is the slowest single-kernel
stage. The CPU oracle is timed on a bounded sample of the same workload.

Prints one JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec on 1 MI355X; encode/decode HBM GB/s; FFN MFMA util"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFS = 2500.0  # dense bf16 MFMA
MFMA_FP8_PEAK_TFS = 5000.0   # dense fp8 MFMA (MX experts: the token operand is always MXFP8)
FP32_VECTOR_PEAK_TFS = 157.3
DEFAULT_WORKLOAD = "large_bf16_S32768_M4096_E128_k8_H1536"
FLUSH_MIB = 512


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="workload name (see workloads.py); default: the S=32768 forward + backward layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle's sample")
    ap.add_argument("--stage-reps", type=int, default=0,
                    help="launches per stage in the stage timing (0: about 2 s of GPU time per stage, 3..50)")
    ap.add_argument("--pipeline-chunks", type=int, default=0, metavar="D",
                    help="run the expert FFN in D capacity chunks on --pipeline-streams streams "
                         "(bf16 forward workloads; 0 = the fused forward)")
    ap.add_argument("--pipeline-streams", type=int, default=2)
    ap.add_argument("--batch-streams", type=int, default=0, metavar="N",
                    help="forward workloads: also time consecutive batches alternating over N streams, each stream "
                         "with its own buffers (reported as multi_stream; 0: 2 for forward workloads, off otherwise)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once in a HIP graph and replayed (reported as 'graph')")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB each (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


# HBM traffic of the dominant kernel comes from two counter runs (FETCH_SIZE, then
# WRITE_SIZE) recorded in profiles/traffic_<stage>_<workload>.md together with the
# sha256 of the sources that define that stage's kernel; it is reported only while
# those sources are unchanged.
GEMM_STAGES = {"fc1", "fc2", "fc2_bwd_data", "fc2_wgrad", "fc1_bwd_data", "fc1_wgrad"}
GEMM_SOURCES = ("combine_softmax_top_amd/csrc/gemm.hip", "combine_softmax_top_amd/csrc/moe_internal.h")
ROW_SOURCES = ("combine_softmax_top_amd/csrc/dispatch.hip", "combine_softmax_top_amd/csrc/moe_internal.h")


def sources_sha256(stage):
    import hashlib
    h = hashlib.sha256()
    for rel in (GEMM_SOURCES if stage in GEMM_STAGES else ROW_SOURCES):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(stage, workload):
    """Bytes per launch from the committed counter summary, or None if absent or stale."""
    path = os.path.join(ROOT, "profiles", f"traffic_{stage}_{workload}.md")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^- ([a-z_0-9]+): `?([^`\s]+)`?", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("sources_sha256") != sources_sha256(stage) or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def copy_calibration(mib):
    import torch
    a = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps(dict(copy_bytes_read=a.numel() * 4, copy_bytes_written=a.numel() * 4, launches=3)))


def fp8_tokens(w):
    """Whether the workload's experts quantise the tokens and run 8-bit products (MX, block FP8);
    NVFP4 experts are weight-only, on bf16 products."""
    return w.mx in ("mxfp8", "mxfp4", "blockfp8")


def algorithmic(w, C, kept):
    """Bytes (or flops) each stage must move (or compute), per launch, and its bound."""
    b = w.elem_bytes
    S, M, E, k, H = w.S, w.M, w.E, w.k, w.H
    prod = 2 * M * H * kept  # one expert product over the filled rows
    st = {
        "route": ("bytes", 4 * S * E + 12 * k * S + 4 * kept + 8 * E),
        # MX encode writes one code byte per value plus a scale byte per 32 (block FP8: 4 bytes per 128)
        "encode": ("bytes", S * M * b + (E * C * M * 33 // 32 if fp8_tokens(w) else E * C * M * b) + 8 * k * S),
        "fc1": ("flops", prod),
        "fc2": ("flops", prod),
        "decode": ("bytes", kept * M * b + S * M * b + 12 * k * S + (S * M * b if w.residual else 0)),
    }
    if w.residual:
        st["res_ffn"] = ("flops", 4 * M * H * S)  # the dense branch: fc1 and fc2 over all S tokens
    if w.logits == "gate":
        st["gate"] = ("bytes", S * M * b + 4 * M * E + 4 * S * E)
    if w.backward:
        # K1' and K2: read dout and the kept y rows, write the kept dy rows and dgates
        st["decode_bwd"] = ("bytes", S * M * b + 2 * kept * M * b + 16 * k * S)
        st["fc2_bwd_data"] = ("flops", prod)  # dpre = (dy W2) * act'(pre)
        st["fc2_wgrad"] = ("flops", prod)     # dW2 = dy^T h
        st["fc1_bwd_data"] = ("flops", prod)  # dbuf = dpre W1
        st["fc1_wgrad"] = ("flops", prod)     # dW1 = dpre^T buf
        # K0: read the kept dbuf rows, write dx
        st["encode_bwd"] = ("bytes", kept * M * b + S * M * b + 8 * k * S)
        if w.residual:
            st["res_bwd"] = ("flops", 8 * M * H * S)  # the dense branch's four backward products
        # gate backward: read logits, idx, dgates, needed; write dlogits
        st["gate_bwd"] = ("bytes", 8 * S * E + 8 * k * S + 4 * E)
        if w.logits == "gate":
            st["gate_wgrad"] = ("bytes", S * M * b + 4 * S * E + 4 * M * E)  # dWg = x^T dlogits
    return st


# stages that are one kernel launch (candidates for the dominant kernel)
SINGLE_KERNEL = {"gate", "encode", "fc1", "fc2", "decode", "decode_bwd", "fc2_bwd_data", "fc2_wgrad",
                 "fc1_bwd_data", "fc1_wgrad", "encode_bwd"}


def roofline_of(kind, amount, ms, dtype_bf16=True, mx=False):
    if kind == "bytes":
        ach = amount / (ms * 1e-3) / 1e9
        return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4))
    ach = amount / (ms * 1e-3) / 1e12
    peak = MFMA_FP8_PEAK_TFS if mx else (MFMA_BF16_PEAK_TFS if dtype_bf16 else FP32_VECTOR_PEAK_TFS)
    return dict(bound="mfma" if dtype_bf16 else "alu", achieved=round(ach, 2), peak=peak, unit="TFLOP/s",
                frac=round(ach / peak, 4))


def host_info():
    model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return dict(cpu_model=model, nproc=os.cpu_count(), affinity_cores=len(os.sched_getaffinity(0)))


def cpu_baseline(w, inp, budget_s):
    """Time the CPU oracle on a bounded sample of the workload; returns the cpu_baseline object.

    Routing, encode and decode run on every token. The expert FFN (and for training
    workloads its backward: the per-row backward, dgates, the weight gradients and dx)
    runs on the kept routes of a seeded sample of tokens, sized to about budget_s, and
    each stage's time is scaled linearly to the whole workload (rows, or tokens for dx).
    """
    import numpy as np
    import oracle
    from tests.helpers import np_of
    ni = {k: np_of(v) for k, v in inp.items()}
    t, scaled = {}, {}
    t0 = time.perf_counter()
    logits = oracle.gate_logits(ni["x"], ni["Wg"], w.dtype) if w.logits == "gate" else ni["logits"]
    t["gate"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    rt = oracle.route(logits, w.k, w.capacity_factor)
    t["route"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    t["encode"] = time.perf_counter() - t0
    C = rt["C"]
    kept_rows = oracle.filled_rows(rt)
    kept = len(kept_rows)
    rng = np.random.default_rng(0)
    order = rng.permutation(w.S)

    def rows_of(toks):
        r = [int(rt["idx"][q, s]) * C + int(rt["loc"][q, s]) for s in toks for q in range(w.k)
             if rt["loc"][q, s] < C]
        return np.asarray(sorted(r), np.int64)

    if w.mx == "blockfp8":
        t0 = time.perf_counter()
        bufq = oracle.blockfp8_quantize(buf, 1, w.dtype)
        t["encode"] += time.perf_counter() - t0
        W1q = oracle.blockfp8_quantize(ni["W1"], oracle.BLOCK, w.dtype)
        W2q = oracle.blockfp8_quantize(ni["W2"], oracle.BLOCK, w.dtype)

        def ffn(rs):
            return None, oracle.expert_rows_blockfp8(bufq, W1q, ni.get("b1"), W2q, ni.get("b2"), rs, C, w.act)[1]
    elif w.mx == "nvfp4":
        W1q = oracle.nvfp4_quantize(ni["W1"], w.dtype)
        W2q = oracle.nvfp4_quantize(ni["W2"], w.dtype)

        def ffn(rs):
            _, h, y = oracle.expert_rows_nvfp4(buf, W1q, ni.get("b1"), W2q, ni.get("b2"), rs, C, w.act)
            return h, y
    elif w.mx:
        wf = oracle.MX_FP8 if w.mx == "mxfp8" else oracle.MX_FP4
        t0 = time.perf_counter()
        bufq = oracle.mx_quantize(buf, oracle.MX_FP8, w.dtype)
        t["encode"] += time.perf_counter() - t0
        W1q = oracle.mx_quantize(ni["W1"], wf, w.dtype)
        W2q = oracle.mx_quantize(ni["W2"], wf, w.dtype)

        def ffn(rs):
            return None, oracle.expert_rows_mx(bufq, W1q, ni.get("b1"), W2q, ni.get("b2"), rs, C, w.act, wf)[1]
    else:
        def ffn(rs):
            _, h, y = oracle.expert_rows(buf, ni["W1"], ni.get("b1"), ni["W2"], ni.get("b2"), rs, C, w.act, w.dtype,
                                         want_h=True)
            return h, y

    def sample_pass(toks, timings):
        rs = rows_of(toks)
        t0 = time.perf_counter()
        h, y = ffn(rs)
        timings["ffn"] = time.perf_counter() - t0
        if w.backward:
            fw = dict(route=rt, buf=buf)
            t0 = time.perf_counter()
            q, dy, dpre, dbuf = oracle.backward_rows(fw, ni, rs, w.act, w.dtype)
            timings["ffn_bwd_rows"] = time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.dgates(q, ni["dout"], y, w.S, w.dtype)
            timings["dgates"] = time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.dx_tokens(q, dbuf, toks, w.S, w.k, w.dtype)
            timings["dx"] = time.perf_counter() - t0
        if w.residual:
            t0 = time.perf_counter()
            oracle.residual_mlp(ni["x"], ni["W1r"], ni.get("b1r"), ni["W2r"], ni.get("b2r"), w.act, w.dtype,
                                tokens=toks)
            timings["res_ffn"] = time.perf_counter() - t0
            if w.backward:
                t0 = time.perf_counter()
                oracle.residual_backward(ni, w.act, w.dtype, tokens=toks, want_wgrad=False)
                timings["res_bwd_rows"] = time.perf_counter() - t0
        return len(rs), y

    # probe on a few tokens, then a sample sized to the budget
    probe = {}
    n_probe = max(1, min(w.S, 4))
    nr, _ = sample_pass(order[:n_probe], probe)
    per_token = sum(probe.values()) / n_probe
    # a tenth of the budget goes to the weight gradients below
    ntok = int(min(w.S, max(n_probe, 0.9 * budget_s / max(per_token, 1e-9))))
    toks = np.sort(order[:ntok])
    samp = {}
    nrows, ys = sample_pass(toks, samp)
    row_scale = kept / max(1, nrows)
    for name, v in samp.items():
        scaled[name] = v * (w.S / ntok if name in ("dx", "res_ffn", "res_bwd_rows") else row_scale)
    nw = 0
    if w.backward and kept > 0:
        # weight gradients: a fixed cost per expert (its M x H outputs) plus one per row, so
        # they are timed on enough rows of one expert (the fullest) for the fixed part to be
        # small, and scaled by rows: kept rows over all experts
        e_w = int(np.argmax(rt["fill"]))
        nw = int(min(48, rt["fill"][e_w]))
        wr = e_w * C + np.arange(nw, dtype=np.int64)
        _, dyw, dprew, _ = oracle.backward_rows(dict(route=rt, buf=buf), ni, wr, w.act, w.dtype, want_dbuf=False)
        hw, _ = ffn(wr)
        t0 = time.perf_counter()
        oracle.weight_grads(dyw, hw, dprew, buf[wr], w.dtype)
        samp["wgrad"] = time.perf_counter() - t0
        scaled["wgrad"] = samp["wgrad"] * kept / nw
        if w.residual:
            # the dense branch's weight gradients: one row per token, timed on the first nw tokens
            xs = {n: ni[n][:nw] for n in ("x", "dout")}
            hr, _ = oracle.residual_mlp(xs["x"], ni["W1r"], ni.get("b1r"), ni["W2r"], ni.get("b2r"), w.act, w.dtype)
            dpr = oracle.residual_backward(dict(ni, **xs), w.act, w.dtype, want_wgrad=False)["dpre_r"]
            t0 = time.perf_counter()
            oracle.weight_grads(xs["dout"], hr, dpr, xs["x"], w.dtype)
            samp["res_wgrad"] = time.perf_counter() - t0
            scaled["res_wgrad"] = samp["res_wgrad"] * w.S / nw
    rs = rows_of(toks)
    y = np.zeros((w.E * C, w.M), ys.dtype)  # decode's cost does not depend on the values
    y[rs] = ys
    t0 = time.perf_counter()
    oracle.decode(y, rt, w.E, w.dtype)
    t["decode"] = time.perf_counter() - t0
    if w.backward:
        dg = np.zeros((w.k, w.S), np.float32)
        t0 = time.perf_counter()
        oracle.gate_backward(logits, rt["idx"], dg, rt["needed"], 0.01)
        t["gate_bwd"] = time.perf_counter() - t0
    total = sum(t.values()) + sum(scaled.values())
    what = "forward + backward" if w.backward else "forward"
    return dict(value=round(w.S / total, 2), unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=(f"{what}; gate/route/encode/decode{'/gate backward' if w.backward else ''} on all {w.S} "
                        f"tokens; expert FFN{' and its backward (rows, dgates, dx)' if w.backward else ''}"
                        f" on the {nrows} kept routes of {ntok} seeded random tokens"
                        + (f", weight gradients on {nw} rows of one expert" if w.backward else "")
                        + (f"; the Residual-MoE dense branch{' and its backward rows' if w.backward else ''} on the "
                           f"same tokens" + (f", its weight gradients on {nw} tokens" if w.backward else "")
                           if w.residual else "")
                        + f" ({sum(samp.values()):.1f} s), scaled linearly to all {kept} kept routes "
                        f"({w.S} tokens for dx{' and the dense branch' if w.residual else ''})"),
                seconds={**{k: round(v, 3) for k, v in t.items()}, **{k: round(v, 2) for k, v in scaled.items()}},
                sample_seconds={k: round(v, 3) for k, v in samp.items()},
                host=host_info())


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the MoE layer (routing, encode, the experts' GEMMs, decode and "
              f"their backward on one GPU, no collectives): --gpus {args.gpus} is not supported, run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    import torch
    import combine_softmax_top_amd as moe
    import workloads as W

    w = W.BY_NAME[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] workload {w.name}: generating inputs on the GPU")
    inp = W.make_inputs(w, seed=0, device=dev)
    s = moe.Shape.of(w)
    gate = w.logits == "gate"
    mxf = {"mxfp8": moe.MOE_MX_FP8, "mxfp4": moe.MOE_MX_FP4}.get(w.mx)
    blk = w.mx == "blockfp8"
    nv = w.mx == "nvfp4"

    def alloc_lowp():
        if nv:
            return moe.alloc_forward(s, dev, gate_projection=gate)
        return (moe.alloc_forward_blockfp8(s, dev, gate_projection=gate) if blk else
                moe.alloc_forward_mx(s, dev, gate_projection=gate))

    if mxf is not None or blk or nv:
        bufs = alloc_lowp()
    else:
        bufs = moe.alloc_forward(s, dev, training=w.backward, gate_projection=gate, residual=w.residual)
    res = {n: inp.get(n) for n in ("W1r", "b1r", "W2r", "b2r")} if w.residual else None
    grads = None
    if w.backward:
        grads = moe.alloc_backward(s, dev, gate=True, gate_projection=gate, residual=w.residual)
        grads["dbuf"] = torch.empty_like(grads["dy"])  # its own memory, so each stage can be timed alone
    x, W1, W2, b1, b2 = inp["x"], inp["W1"], inp["W2"], inp.get("b1"), inp.get("b2")
    logits_in, Wg = (None, inp["Wg"]) if gate else (inp["logits"], None)
    # the training step's backward includes the gate: dlogits, the load-balance loss, and with a
    # projected gate dWg and dx's gate share
    logits_bwd = bufs["logits"] if gate else logits_in

    def backward():
        moe.layer_backward(s, bufs, inp["dout"], W1, W2, grads=grads, logits=logits_bwd, x=x, Wg=Wg, residual=res)

    if mxf is not None or blk or nv:
        # low-precision experts: the weights are quantised once, outside the timed region (offline)
        if nv:
            W1q, W2q = moe.nvfp4_quantize_weights(W1), moe.nvfp4_quantize_weights(W2)
        elif blk:
            W1q, W2q = moe.blockfp8_quantize_weights(W1), moe.blockfp8_quantize_weights(W2)
        else:
            W1q, W2q = moe.mx_quantize_weights(W1, mxf), moe.mx_quantize_weights(W2, mxf)
        torch.cuda.synchronize()

    pipe = args.pipeline_chunks > 0
    if pipe:
        assert not w.mx and not w.residual and not w.backward and w.dtype == W.DT_BF16, \
            "--pipeline-chunks applies to the bf16 forward workloads"
        pstreams = [torch.cuda.Stream() for _ in range(args.pipeline_streams)]
        pevents = [torch.cuda.Event() for _ in range(args.pipeline_streams + 1)]

    nb = args.batch_streams if args.batch_streams > 0 else (1 if (w.backward or pipe) else 2)
    bsets, bstreams = [bufs], [None]
    if nb > 1:
        assert not w.backward and not pipe, "--batch-streams applies to the forward workloads"
        for _ in range(nb - 1):
            bsets.append(alloc_lowp() if w.mx else
                         moe.alloc_forward(s, dev, gate_projection=gate, residual=w.residual))
        bstreams = [torch.cuda.Stream() for _ in range(nb)]
    counter = [0]

    def step(multi=False):
        i = counter[0] % nb if multi else 0
        counter[0] += 1
        b, st = bsets[i], bstreams[i] if multi else None
        if nv:
            moe.layer_forward_nvfp4(s, x, W1q, b1, W2q, b2, logits=logits_in, Wg=Wg, bufs=b, stream=st)
            return
        if blk:
            moe.layer_forward_blockfp8(s, x, W1q, b1, W2q, b2, logits=logits_in, Wg=Wg, bufs=b, stream=st)
            return
        if mxf is not None:
            moe.layer_forward_mx(s, mxf, x, W1q, b1, W2q, b2, logits=logits_in, Wg=Wg, bufs=b, stream=st)
            return
        if pipe:
            moe.layer_forward_pipelined(s, x, W1, b1, W2, b2, args.pipeline_chunks, pstreams, pevents,
                                        logits=logits_in, Wg=Wg, bufs=bufs)
            return
        moe.layer_forward(s, x, W1, b1, W2, b2, logits=logits_in, Wg=Wg, bufs=b, residual=res, stream=st)
        if w.backward:
            backward()

    def timed_loop(multi):
        for _ in range(args.warmup):
            step(multi)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(multi)
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    # ---- the timed region: --steps fused steps on one stream
    elapsed = timed_loop(False)
    ms_per_step = elapsed * 1e3 / max(1, args.steps)
    value = w.S * args.steps / elapsed
    log(f"[bench] {args.steps} steps after {args.warmup} warm-up: {ms_per_step:.4f} ms/step, {value:.4g} tokens/s")
    multi = None
    if nb > 1:
        e2 = timed_loop(True)
        multi = dict(streams=nb, value=round(w.S * args.steps / e2, 1),
                     ms_per_step=round(e2 * 1e3 / max(1, args.steps), 5))
        log(f"[bench] the same steps alternating over {nb} streams: {multi['ms_per_step']:.4f} ms/step, "
            f"{multi['value']:.4g} tokens/s")

    graph = None
    if args.graph and not pipe:
        # the same one-stream step captured once (after the eager steps above) and replayed
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(False)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        eg = time.perf_counter() - t0
        graph = dict(value=round(w.S * args.steps / eg, 1), ms_per_step=round(eg * 1e3 / max(1, args.steps), 5))
        log(f"[bench] the same step replayed from a HIP graph: {graph['ms_per_step']:.4f} ms/step, "
            f"{graph['value']:.4g} tokens/s")

    C = int(bufs["capacity"].item())
    kept = int(bufs["fill"].sum().item())
    log(f"[bench] C={C}, kept={kept}")

    # ---- per-stage timing through each stage's own entry point, on the library's stream
    stream = torch.cuda.current_stream()
    lg = bufs["logits"] if gate else logits_in
    b = bufs
    alg = algorithmic(w, C, kept)
    stage_fns = []
    if gate:
        stage_fns.append(("gate", lambda: moe.moe_gate_project(s, x, Wg, lg)))
    stage_fns.append(("route", lambda: moe.moe_route(s, lg, b["idx"], b["loc"], b["gates"], b["needed"], b["fill"],
                                                     b["capacity"], b["slot_route"], b["ws"])))
    if nv:
        stage_fns += [
            ("encode", lambda: moe.moe_encode(s, x, b["idx"], b["loc"], b["fill"], b["capacity"], b["buf"])),
            ("fc1", lambda: moe.moe_expert_fc1_nvfp4(s, b["buf"], W1q, b1, b["fill"], b["capacity"], None, b["h"])),
            ("fc2", lambda: moe.moe_expert_fc2_nvfp4(s, b["h"], W2q, b2, b["fill"], b["capacity"], b["y"])),
        ]
    elif blk:
        stage_fns += [
            ("encode", lambda: moe.moe_encode_blockfp8(s, x, b["idx"], b["loc"], b["fill"], b["capacity"],
                                                       b["buf_codes"], b["buf_scales"])),
            ("fc1", lambda: moe.moe_expert_fc1_blockfp8(s, b["buf_codes"], b["buf_scales"], W1q, b1, b["fill"],
                                                        b["capacity"], b["h_codes"], b["h_scales"])),
            ("fc2", lambda: moe.moe_expert_fc2_blockfp8(s, b["h_codes"], b["h_scales"], W2q, b2, b["fill"],
                                                        b["capacity"], b["y"])),
        ]
    elif mxf is not None:
        stage_fns += [
            ("encode", lambda: moe.moe_encode_mx(s, x, b["idx"], b["loc"], b["fill"], b["capacity"], b["buf_codes"],
                                                 b["buf_scales"])),
            ("fc1", lambda: moe.moe_expert_fc1_mx(s, mxf, b["buf_codes"], b["buf_scales"], W1q, b1, b["fill"],
                                                  b["capacity"], b["h_codes"], b["h_scales"])),
            ("fc2", lambda: moe.moe_expert_fc2_mx(s, mxf, b["h_codes"], b["h_scales"], W2q, b2, b["fill"],
                                                  b["capacity"], b["y"])),
        ]
    else:
        stage_fns += [
            ("encode", lambda: moe.moe_encode(s, x, b["idx"], b["loc"], b["fill"], b["capacity"], b["buf"])),
            ("fc1", lambda: moe.moe_expert_fc1(s, b["buf"], W1, b1, b["fill"], b["capacity"], b["pre"], b["h"])),
            ("fc2", lambda: moe.moe_expert_fc2(s, b["h"], W2, b2, b["fill"], b["capacity"], b["y"])),
        ]
    if w.residual:
        stage_fns.append(("res_ffn", lambda: moe.moe_residual_ffn(s, x, res["W1r"], res["b1r"], res["W2r"], res["b2r"],
                                                                  b["pre_r"], b["h_r"], b["y_r"], b["ws"])))
        stage_fns.append(("decode", lambda: moe.moe_decode_residual(s, b["y"], b["gates"], b["idx"], b["loc"],
                                                                    b["capacity"], b["y_r"], b["out"])))
    else:
        stage_fns.append(("decode", lambda: moe.moe_decode(s, b["y"], b["gates"], b["idx"], b["loc"], b["capacity"],
                                                           b["out"])))
    if w.backward:
        g = grads
        stage_fns += [
            ("decode_bwd", lambda: moe.moe_decode_backward(s, inp["dout"], b["y"], b["gates"], b["idx"], b["loc"],
                                                           b["capacity"], g["dy"], g["dgates"])),
            ("gate_bwd", lambda: moe.moe_gate_backward(s, lg, b["idx"], g["dgates"], b["needed"], moe.AUX_COEF,
                                                       g["dlogits"], g["aux_loss"], b["ws"])),
            ("fc2_wgrad", lambda: moe.moe_expert_fc2_weight_grad(s, g["dy"], b["h"], b["fill"], b["capacity"],
                                                                 g["dW2"], g["db2"])),
            ("fc2_bwd_data", lambda: moe.moe_expert_fc2_backward_data(s, g["dy"], W2, b["pre"], b["fill"],
                                                                      b["capacity"], g["dpre"])),
            ("fc1_bwd_data", lambda: moe.moe_expert_fc1_backward_data(s, g["dpre"], W1, b["fill"], b["capacity"],
                                                                      g["dbuf"])),
            ("fc1_wgrad", lambda: moe.moe_expert_fc1_weight_grad(s, g["dpre"], b["buf"], b["fill"], b["capacity"],
                                                                 g["dW1"], g["db1"])),
            ("encode_bwd", lambda: moe.moe_encode_backward(s, g["dbuf"], b["idx"], b["loc"], b["capacity"], g["dx"])),
        ]
        if gate:
            stage_fns.append(("gate_wgrad", lambda: moe.moe_gate_weight_grad(s, x, g["dlogits"], g["dWg"], b["ws"])))
        if w.residual:
            stage_fns.append(("res_bwd", lambda: moe.moe_residual_backward(
                s, inp["dout"], x, b["pre_r"], b["h_r"], res["W1r"], res["W2r"], g["dpre_r"], g["dx_r"], g["dW1r"],
                g["db1r"], g["dW2r"], g["db2r"], b["ws"])))

    flush = torch.empty(FLUSH_MIB * 2 ** 20 // 4, dtype=torch.float32, device=dev)
    # bf16 matmuls enqueued ahead of a batch keep the GPU busy while the host enqueues it,
    # so the events bracket kernel time, not host gaps
    fa = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    fb = torch.randn(4096, 4096, device=dev, dtype=torch.bfloat16)
    torch.mm(fa, fb)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(4):
        torch.mm(fa, fb)
    c1.record(stream)
    torch.cuda.synchronize()
    filler_ms = max(c0.elapsed_time(c1) / 4, 1e-3)

    stages = {}
    for name, fn in stage_fns:
        kind, amount = alg[name]
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3  # bounds one call (host + device)
        reps = args.stage_reps or max(3, min(50, int(2000.0 / max(host_ms, 1e-3))))
        flushed = kind == "bytes"

        def batch(body, n):
            # fillers keep the GPU busy while the host enqueues the batch
            for _ in range(min(200, int((2.0 * host_ms * n + 0.5) / filler_ms) + 1)):
                torch.mm(fa, fb)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(n):
                body()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)

        if flushed:
            # each launch after a fill that evicts L2 and the Infinity Cache, so that its
            # operands come from HBM, bracketed by events of its own (the pairs are queued
            # behind fillers, so no host gap falls between a fill and its launch; the
            # interval includes the launch's dispatch). A batch of (fill, launch) pairs
            # minus a batch of fills was tried first: for launches of a few microseconds it
            # read up to 30x the kernel's traced duration.
            def flushed_total(n):
                for _ in range(min(200, int((2.0 * (host_ms + 0.1) * n + 0.5) / filler_ms) + 1)):
                    torch.mm(fa, fb)
                evs = []
                for _ in range(n):
                    flush.fill_(1.0)
                    a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record(stream)
                    fn()
                    z.record(stream)
                    evs.append((a, z))
                torch.cuda.synchronize()
                return sum(a.elapsed_time(z) for a, z in evs)

            n = max(5, min(reps, 20))
            ms = max(sum(flushed_total(n) for _ in range(3)) / (3 * n), 1e-6)
            reps = 3 * n
        else:
            ms = batch(fn, reps) / reps
        r = roofline_of(kind, amount, ms, w.dtype == W.DT_BF16, mx=fp8_tokens(w) and name in ("fc1", "fc2"))
        r["ms"] = round(ms, 5)
        r["launches"] = reps
        r["timing"] = "after a 512 MiB fill each, per-launch events" if flushed else "back-to-back batch"
        r["algorithmic_" + kind] = amount
        stages[name] = r
        log(f"[bench] stage {name:13s} {ms:9.4f} ms  {r['achieved']:10.2f} {r['unit']}  "
            f"({100 * r['frac']:.1f}% of peak; {r['timing']}, {reps} launches)")
    del flush
    dominant = max((n for n in stages if n in SINGLE_KERNEL), key=lambda n: stages[n]["ms"])
    d = stages[dominant]
    roofline = dict(kernel=dominant, bound=d["bound"], achieved=d["achieved"], peak=d["peak"], unit=d["unit"],
                    frac=d["frac"], traffic=recorded_traffic(dominant, w.name))
    log(f"[bench] dominant kernel: {dominant} ({d['ms']:.4f} ms, {100 * d['frac']:.1f}% of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, inp, args.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value']} tokens/s on {cpu['cores']} threads ({cpu['host']}): "
            f"{cpu['sample']}")

    line = dict(
        metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=(w.mx + "/bf16") if w.mx else ("bf16" if w.dtype == W.DT_BF16 else "f32"), data="synthetic",
        config=dict(workload=w.name, S=w.S, M=w.M, E=w.E, k=w.k, H=w.H, capacity_factor=w.capacity_factor,
                    act="gelu" if w.act == W.ACT_GELU else "relu", biases=[w.has_fc1_bias, w.has_fc2_bias],
                    logits=w.logits, backward=w.backward, C=C, kept_routes=kept, parallelism="single-gpu",
                    aux_coef=moe.AUX_COEF if w.backward else None, residual=w.residual, mx=w.mx or None,
                    pipeline=dict(chunks=args.pipeline_chunks, streams=args.pipeline_streams) if pipe else None),
        roofline=roofline, stages=stages, cpu_baseline=cpu, multi_stream=multi, graph=graph,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
