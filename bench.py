"""Benchmark of the single-GPU MoE layer on MI355X.

One step = one pass of the whole layer over one batch of synthetic input that is
already resident in HBM: for the default workload (S=4096 tokens, M=1024, E=8
experts, top-2, H=4096, bf16, logits projected from x by an fp32 gate matrix,
capacity_factor 1.25) that is gate projection -> route -> encode -> fc1 -> fc2
-> decode (Residual-MoE workloads add the dense MLP branch over all tokens,
summed into decode); workloads with a backward add the backward of decode, FFN, encode
and the gate (dlogits through the softmax, the 0.01 load-balance loss, and for
a projected gate dWg and the projection's share of dx). The timed region is exactly --steps calls of the fused C-ABI entry
points, bracketed by synchronisations. Forward workloads run consecutive batches on two streams by
default, each stream with its own buffers (--batch-streams): a batch's short routing, encode and
decode launches then overlap the neighbouring batch's expert products, which leave CUs idle in their
last round. The same steps run one after another on one stream are timed too (single_stream).

A second timed loop records HIP events around each stage on the stream the
library launches on, to report each stage against its roofline (bytes or flops
the method must move or compute per launch, over the stage's average time).
The CPU oracle is timed on a bounded sample of the same workload as a baseline.

Prints one JSON line on stdout; diagnostics go to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # a step of the default workload is ~0.25 ms: 1000 timed steps keep the GPU at
    # its steady clocks for about a quarter second (20 steps measured the ramp)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="gated_bf16_S4096_M1024_E8_k2_H4096",
                    help="workload name (see workloads.py); default: the S=4096 gate-projected bf16 layer")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle FFN sample")
    ap.add_argument("--pipeline-chunks", type=int, default=0, metavar="D",
                    help="run the expert FFN in D capacity chunks on --pipeline-streams streams "
                         "(bf16 forward workloads; 0 = the fused forward)")
    ap.add_argument("--pipeline-streams", type=int, default=2)
    ap.add_argument("--batch-streams", type=int, default=0, metavar="N",
                    help="consecutive batches alternate over N streams, each stream with its own buffers, so that "
                         "one batch's routing, encode and decode overlap the neighbouring batches' expert products; "
                         "0 (default): 2 for forward workloads, 1 for training and pipelined runs. With N > 1 the "
                         "same steps are also timed on one stream and reported as single_stream")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB each (the reference kernel that scales the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


# HBM traffic of the dominant kernel comes from two counter runs (FETCH_SIZE, then
# WRITE_SIZE) recorded in profiles/traffic_<stage>_<workload>.md together with the
# sha256 of the kernel sources they were taken on; it is reported only while those
# sources are unchanged.
TRAFFIC_SOURCES = ("combine_softmax_top_amd/csrc/gemm.hip", "combine_softmax_top_amd/csrc/moe_internal.h")


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:
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
    if fields.get("sources_sha256") != sources_sha256() or "traffic_bytes_per_launch" not in fields:
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


def algorithmic(w, C, kept):
    """Bytes (or flops) each stage must move (or compute), per launch."""
    b = w.elem_bytes
    S, M, E, k, H = w.S, w.M, w.E, w.k, w.H
    st = {
        "route": ("bytes", 4 * S * E + 12 * k * S + 4 * kept + 8 * E),
        # MX encode writes one code byte per value plus a scale byte per 32
        "encode": ("bytes", S * M * b + (E * C * M * 33 // 32 if w.mx else E * C * M * b) + 8 * k * S),
        "fc1": ("flops", 2 * M * H * kept),
        "fc2": ("flops", 2 * M * H * kept),
        "decode": ("bytes", kept * M * b + S * M * b + 12 * k * S + (S * M * b if w.residual else 0)),
    }
    if w.residual:
        # the dense branch: fc1 and fc2 over all S tokens
        st["res_ffn"] = ("flops", 4 * M * H * S)
    if w.logits == "gate":
        st["gate"] = ("bytes", S * M * b + 4 * M * E + 4 * S * E)
    if w.backward:
        # dy/dgates: read dout and kept y rows, write kept dy rows; dx: read kept dbuf rows, write dx;
        # GEMMs: dh, dW2, dbuf, dW1 (2*M*H*kept flops each)
        st["backward"] = ("flops", 8 * M * H * kept)
        # gate backward: read logits, idx, dgates, needed; write dlogits
        st["gate_bwd"] = ("bytes", 8 * S * E + 8 * k * S + 4 * E)
        if w.logits == "gate":
            # dWg = x^T dlogits: read x and dlogits, write dWg
            st["gate_wgrad"] = ("bytes", S * M * b + 4 * S * E + 4 * M * E)
    return st


def roofline_of(kind, amount, ms, dtype_bf16=True, mx=False):
    if kind == "bytes":
        ach = amount / (ms * 1e-3) / 1e9
        return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(ach / HBM_PEAK_GBS, 4))
    ach = amount / (ms * 1e-3) / 1e12
    peak = MFMA_FP8_PEAK_TFS if mx else (MFMA_BF16_PEAK_TFS if dtype_bf16 else FP32_VECTOR_PEAK_TFS)
    return dict(bound="mfma" if dtype_bf16 else "alu", achieved=round(ach, 2), peak=peak, unit="TFLOP/s",
                frac=round(ach / peak, 4))


def cpu_baseline(w, inp, C_gpu, budget_s):
    """Time the CPU oracle on a bounded sample of the workload; returns the cpu_baseline object."""
    import numpy as np
    import oracle
    from tests.helpers import np_of
    ni = {k: np_of(v) for k, v in inp.items()}
    t = {}
    t0 = time.perf_counter()
    if w.logits == "gate":
        logits = oracle.gate_logits(ni["x"], ni["Wg"], w.dtype)
    else:
        logits = ni["logits"]
    t["gate"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    rt = oracle.route(logits, w.k, w.capacity_factor, with_slots=False)
    t["route"] = time.perf_counter() - t0
    assert rt["C"] == C_gpu, (rt["C"], C_gpu)
    t0 = time.perf_counter()
    buf = oracle.encode(ni["x"], rt, w.E, w.dtype)
    t["encode"] = time.perf_counter() - t0
    rows = oracle.filled_rows(rt)
    kept = len(rows)
    if w.mx:
        # MX experts: the token rows are quantised in the encode (timed with it), the weights offline
        wf = oracle.MX_FP8 if w.mx == "mxfp8" else oracle.MX_FP4
        t0 = time.perf_counter()
        bufq = oracle.mx_quantize(buf, oracle.MX_FP8, w.dtype)
        t["encode"] += time.perf_counter() - t0
        W1q = oracle.mx_quantize(ni["W1"], wf, w.dtype)
        W2q = oracle.mx_quantize(ni["W2"], wf, w.dtype)

        def ffn(rs):
            return None, None, oracle.expert_rows_mx(bufq, W1q, ni.get("b1"), W2q, ni.get("b2"), rs, rt["C"], w.act,
                                                     wf)[1]
    else:
        def ffn(rs):
            return oracle.expert_rows(buf, ni["W1"], ni.get("b1"), ni["W2"], ni.get("b2"), rs, rt["C"], w.act,
                                      w.dtype)
    # FFN on an evenly strided sample of the filled rows, sized to about budget_s
    probe = rows[:: max(1, kept // 16)][:16]
    t0 = time.perf_counter()
    ffn(probe)
    per_row = (time.perf_counter() - t0) / max(1, len(probe))
    n = int(min(kept, max(16, budget_s / max(per_row, 1e-9))))
    sample = rows[:: max(1, kept // n)][:n]
    t0 = time.perf_counter()
    _, _, ys = ffn(sample)
    t_sample = time.perf_counter() - t0
    t["ffn"] = t_sample / len(sample) * kept
    y = np.zeros((w.E * rt["C"], w.M), ys.dtype)  # decode's cost does not depend on the values
    y[sample] = ys
    t0 = time.perf_counter()
    oracle.decode(y, rt, w.E, w.dtype)
    t["decode"] = time.perf_counter() - t0
    total = sum(t.values())
    return dict(value=round(w.S / total, 2), unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample=(f"gate/route/encode/decode on all {w.S} tokens; expert FFN on {len(sample)} of the {kept} "
                        f"filled rows (evenly strided, {t_sample:.1f}s), scaled linearly to all filled rows; "
                        f"forward only"),
                seconds={k: round(v, 3) for k, v in t.items()})


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the layer: --gpus {args.gpus} is not supported "
              "(the layer here runs on one GPU, with no collectives; run with --gpus 1)", file=sys.stderr)
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
    if mxf is not None:
        bufs = moe.alloc_forward_mx(s, dev, gate_projection=gate)
    else:
        bufs = moe.alloc_forward(s, dev, training=w.backward, gate_projection=gate, residual=w.residual)
    res = {n: inp.get(n) for n in ("W1r", "b1r", "W2r", "b2r")} if w.residual else None
    grads = moe.alloc_backward(s, dev, gate=True, gate_projection=gate) if w.backward else None
    x, W1, W2, b1, b2 = inp["x"], inp["W1"], inp["W2"], inp.get("b1"), inp.get("b2")
    logits_in, Wg = (None, inp["Wg"]) if gate else (inp["logits"], None)
    # the training step's backward includes the gate: dlogits, the load-balance loss, and with a
    # projected gate dWg and dx's gate share
    logits_bwd = bufs["logits"] if gate else logits_in

    def backward():
        moe.layer_backward(s, bufs, inp["dout"], W1, W2, grads=grads, logits=logits_bwd, x=x, Wg=Wg)

    if mxf is not None:
        # MX experts: the weights are quantised once, outside the timed region (offline)
        W1q = moe.mx_quantize_weights(W1, mxf)
        W2q = moe.mx_quantize_weights(W2, mxf)
        torch.cuda.synchronize()

    pipe = args.pipeline_chunks > 0
    if pipe:
        assert mxf is None and not w.residual and not w.backward and w.dtype == W.DT_BF16, \
            "--pipeline-chunks applies to the bf16 forward workloads"
        pstreams = [torch.cuda.Stream() for _ in range(args.pipeline_streams)]
        pevents = [torch.cuda.Event() for _ in range(args.pipeline_streams + 1)]

    nb = args.batch_streams if args.batch_streams > 0 else (1 if (w.backward or pipe) else 2)
    bsets, bstreams = [bufs], [None]
    if nb > 1:
        assert not w.backward and not pipe, "--batch-streams applies to the forward workloads"
        for _ in range(nb - 1):
            bsets.append(moe.alloc_forward_mx(s, dev, gate_projection=gate) if mxf is not None else
                         moe.alloc_forward(s, dev, gate_projection=gate, residual=w.residual))
        bstreams = [torch.cuda.Stream() for _ in range(nb)]
    counter = [0]

    def step(one_stream=False):
        i = 0 if one_stream else counter[0] % nb
        counter[0] += 1
        b, st = bsets[i], bstreams[i]
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

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / max(1, args.steps)
    value = w.S * args.steps / elapsed
    single = None
    if nb > 1:
        # the same steps, one after another on one stream
        for _ in range(args.warmup):
            step(one_stream=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(one_stream=True)
        torch.cuda.synchronize()
        e1 = time.perf_counter() - t0
        single = dict(value=round(w.S * args.steps / e1, 1), ms_per_step=round(e1 * 1e3 / max(1, args.steps), 5))
        log(f"[bench] {nb} streams: {ms_per_step:.4f} ms/step; one stream: {single['ms_per_step']:.4f} ms/step, "
            f"{single['value']:.4g} tokens/s")

    C = int(bufs["capacity"].item())
    kept = int(bufs["fill"].sum().item())
    log(f"[bench] {ms_per_step:.4f} ms/step, {value:.4g} tokens/s; C={C}, kept={kept}")

    # ---- per-stage HIP-event timing on the library's stream
    stream = torch.cuda.current_stream()
    names = (["gate"] if gate else []) + ["route", "encode", "fc1", "fc2"] + (["res_ffn"] if w.residual else []) + [
        "decode"] + (
        ["backward", "gate_bwd"] + (["gate_wgrad"] if gate else []) if w.backward else [])
    ev = {n: [] for n in names}
    lg = bufs["logits"] if gate else logits_in
    b = bufs

    # Each stage is timed over a batch of back-to-back launches between two events.
    # bf16 matmuls enqueued ahead of the first event keep the GPU busy while the
    # host enqueues the batch, so the events bracket kernel time, not host gaps.
    # Every stage is idempotent (same inputs, same outputs).
    fa = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    fb = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    torch.mm(fa, fb)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(4):
        torch.mm(fa, fb)
    c1.record(stream)
    torch.cuda.synchronize()
    filler_ms = max(c0.elapsed_time(c1) / 4, 1e-3)

    def stage_batch(name, fn, reps):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        host_ms = (time.perf_counter() - t0) * 1e3  # bounds one call's host time
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        for _ in range(min(200, int((2.0 * host_ms * reps + 0.5) / filler_ms) + 1)):
            torch.mm(fa, fb)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        ev[name].append((e0, e1, reps))

    stage_fns = []
    if gate:
        stage_fns.append(("gate", lambda: moe.moe_gate_project(s, x, Wg, lg)))
    stage_fns.append(("route", lambda: moe.moe_route(s, lg, b["idx"], b["loc"], b["gates"], b["needed"], b["fill"],
                                                     b["capacity"], b["slot_route"], b["ws"])))
    if mxf is not None:
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
                                                                  b["h_r"], b["y_r"], b["ws"])))
        stage_fns.append(("decode", lambda: moe.moe_decode_residual(s, b["y"], b["gates"], b["idx"], b["loc"],
                                                                    b["capacity"], b["y_r"], b["out"])))
    else:
        stage_fns.append(("decode", lambda: moe.moe_decode(s, b["y"], b["gates"], b["idx"], b["loc"], b["capacity"],
                                                           b["out"])))
    if w.backward:
        stage_fns.append(("backward", backward))
        stage_fns.append(("gate_bwd", lambda: moe.moe_gate_backward(s, lg, b["idx"], grads["dgates"], b["needed"],
                                                                    moe.AUX_COEF, grads["dlogits"],
                                                                    grads["aux_loss"], b["ws"])))
        if gate:
            stage_fns.append(("gate_wgrad", lambda: moe.moe_gate_weight_grad(s, x, grads["dlogits"], grads["dWg"],
                                                                             b["ws"])))
    reps = max(1, min(50, args.steps))
    rounds = max(1, min(10, args.steps // reps))
    for rd in range(rounds):
        for name, fn in stage_fns:
            stage_batch(name, fn, reps)
        torch.cuda.synchronize()
        log(f"[bench] stage timing round {rd + 1}/{rounds} done ({reps} launches per stage)")
    torch.cuda.synchronize()
    alg = algorithmic(w, C, kept)
    stages = {}
    for n in names:
        ms = sum(e0.elapsed_time(e1) for e0, e1, r in ev[n]) / sum(r for _, _, r in ev[n])
        kind, amount = alg[n]
        r = roofline_of(kind, amount, ms, w.dtype == W.DT_BF16, mx=bool(w.mx) and n in ("fc1", "fc2"))
        r["ms"] = round(ms, 5)
        r["algorithmic_" + kind] = amount
        stages[n] = r
        log(f"[bench] stage {n:9s} {ms:9.4f} ms  {r['achieved']:10.2f} {r['unit']}  ({100 * r['frac']:.1f}% of peak)")
    # one-kernel stages only (the fused backward and the dense branch are several launches)
    dominant = max((n for n in names if n not in ("backward", "res_ffn")), key=lambda n: stages[n]["ms"])
    d = stages[dominant]
    roofline = dict(kernel=dominant, bound=d["bound"], achieved=d["achieved"], peak=d["peak"], unit=d["unit"],
                    frac=d["frac"], traffic=recorded_traffic(dominant, w.name))

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        cpu = cpu_baseline(w, inp, C, args.cpu_seconds)
        log(f"[bench] cpu baseline {cpu['value']} tokens/s on {cpu['cores']} threads: {cpu['sample']}")

    line = dict(
        metric=METRIC, value=round(value, 1), unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms_per_step, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=(w.mx + "/bf16") if w.mx else ("bf16" if w.dtype == W.DT_BF16 else "f32"), data="synthetic",
        config=dict(workload=w.name, S=w.S, M=w.M, E=w.E, k=w.k, H=w.H, capacity_factor=w.capacity_factor,
                    act="gelu" if w.act == W.ACT_GELU else "relu", biases=[w.has_fc1_bias, w.has_fc2_bias],
                    logits=w.logits, backward=w.backward, C=C, kept_routes=kept, parallelism="single-gpu",
                    aux_coef=moe.AUX_COEF if w.backward else None, residual=w.residual, mx=w.mx or None,
                    pipeline=dict(chunks=args.pipeline_chunks, streams=args.pipeline_streams) if pipe else None,
                    batch_streams=nb if nb > 1 else None),
        roofline=roofline, stages=stages, cpu_baseline=cpu, single_stream=single,
    )
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
