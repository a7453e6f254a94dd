#!/usr/bin/env python3
"""Benchmark of the GDN-2 chunkwise operator (forward + gate-aware backward) on one MI355X.

One step = forward + gate-aware backward (gdn2_chunk_bwd_factors, gdn2_chunk_fwd_factored,
gdn2_chunk_bwd_reverse, gdn2_chunk_bwd_grads: the staged form of gdn2_chunk_fwd +
gdn2_chunk_bwd in which the key-side chunk operands are formed once and the backward
reuses the forward's chunk states; on shapes where gdn2_chunk_sweeps runs the two sweeps
as one launch, that entry replaces the middle two) over one batch of the
forward/backward workload B=8, T=2048, H=16, dk=dv=128 (bf16 q/k/v, fp32
gates, decay and state; the 2K x 8 training shape of the Gated DeltaNet-2
pages).  Inputs are seeded synthetic tensors (linear_attention_sequence_gdn2_amd.inputs)
already resident in HBM when the timed region starts.

Prints one JSON line (rank 0):
  value        tokens/s of whole steps (tokens = B*T per step)
  roofline     for the dominant kernel: algorithmic bytes per launch / its
               average launch time (HIP events on the stream it runs on),
               against MI355X HBM3E 8 TB/s
  cpu_baseline the fp64 oracle (fwd + bwd) timed on the host's cores on a
               bounded sample of the same workload
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WORKLOAD = "fwd_bf16_B8H16T2048d128"
HBM_PEAK_GBS = 8000.0
# algorithmic HBM bytes per token-head (bf16 q/k/v, fp32 gates, o and gradients):
#   forward : q,k,v 3*256 + log_alpha,b,w 3*512 + o 512              = 2816
#   backward: q,k,v 768 + gates 1536 + dO 512 + six gradients 6*512  = 5888
FWD_BYTES_PER_TOKHEAD = 2816
BWD_BYTES_PER_TOKHEAD = 5888
# per-kernel algorithmic bytes per token-head of the four launches of a step:
#   adjoint factors     : q,k 512 + log_alpha,b 1024
#                         + factors (128*128 + 64*128)*4 / 64 tokens = 1536
#                         + chunk operand record 180736 / 64 tokens = 2824      -> 5896
#   forward sweep       : record operands it reads (Kt, Qt split, Et hi, T, P,
#                         gamma: 115200 / 64 tokens) 1800 + v 256 + w 512
#                         + o 512 + chunk states 1024                           -> 4104
#   reverse sweep       : factors 1536 + dO 512 + dstates 1024                  -> 3072
#   chunk gradients     : q,k,v 768 + b,w 1024 + dO 512 + states, dstates 2048
#                         + record (Kt, Et split, T, P^T, G, gamma: 131584 / 64)
#                         2056 + dq,dk,dv,dlog_alpha,db,dw 3072                 -> 9480
# with the gates given as bf16 logits each pass reads 1536 -> 768 gate bytes per token-head
GATE_BYTES_SAVED_PER_TOKHEAD = 768
LOGIT_WORKLOAD = "logits_bf16_B8H16T2048d128"
# with all three gates given per token ([B,T,H] fp32) each gate read, and each gate
# gradient written, moves 12 instead of 1536 bytes per token-head
TOKEN_GATE_BYTES_SAVED_PER_TOKHEAD = 1536 - 12
TOKEN_WORKLOAD = "gdn_token_bf16_B8H16T2048d128"
FWD_SWEEP_BYTES_PER_TOKHEAD = 4104
# the inference forward on shapes with a 64-column value tile per CU: two launches
#   forward-only records: q,k 512 + log_alpha,b 1024 + the record operands the sweep
#                         reads (115200 / 64 tokens) 1800                        -> 3336
#   sweep (o, S_final)  : record operands 1800 + v 256 + w 512 + o 512           -> 3080
FWD_RECORDS_BYTES_PER_TOKHEAD = 3336
FWD_INFER_SWEEP_BYTES_PER_TOKHEAD = 3080
BWD_FACTORS_BYTES_PER_TOKHEAD = 5896
BWD_REVERSE_BYTES_PER_TOKHEAD = 3072
BWD_GRADS_BYTES_PER_TOKHEAD = 9480


def _kernel_sources_digest():
    """Digest of the device code (the .hip sources and the headers they include); the host-side
    C-ABI file does not change what a kernel reads or writes."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_attention_sequence_gdn2_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if not name.endswith((".hip", ".h")):
            continue
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key, launches_bytes):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE/WRITE_SIZE, if the
    committed counter summary was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_digest") != _kernel_sources_digest():
        return None
    k = rec.get("kernels", {}).get(kernel_key)
    if not k or k.get("workload") != WORKLOAD:
        return None
    return k.get("hbm_bytes_per_launch")


def cpu_baseline(wl, sample_batches):
    import numpy as np  # noqa: F401
    import oracle
    from linear_attention_sequence_gdn2_amd.inputs import make_workload
    x = make_workload(wl, B=sample_batches, grads=True)
    nthreads = oracle.default_threads()
    args = [x["q32"], x["k32"], x["v32"], x["log_alpha"], x["b"], x["w"], x["S0"]]
    args = [oracle._f64(t) for t in args]
    dO = oracle._f64(x["dO"])
    dsf = oracle._f64(x["dS_final"])
    t0 = time.perf_counter()
    oracle.fwd(*args, nthreads=nthreads)
    oracle.bwd(*args, dO, dsf, nthreads=nthreads)
    dt = time.perf_counter() - t0
    tokens = sample_batches * wl.T
    return {"value": tokens / dt, "unit": "tokens/s", "cores": min(nthreads, sample_batches * wl.H),
            "kind": "oracle",
            "sample": "fp64 token-by-token oracle, fwd + bwd, B=%d of %d batches (T=%d, H=%d, d=%d), %.1f s"
                      % (sample_batches, wl.B, wl.T, wl.H, wl.dk, dt)}


def decode_bench(dev, B=64, H=16, dk=128, dv=128, iters=100):
    """The recurrent step (gdn2_step) on a decode batch: one token per (batch, head), the
    state read and written in place.  Bytes per step are the state (2*dk*dv*4 per head)
    plus the token vectors."""
    import torch
    import linear_attention_sequence_gdn2_amd as gdn2
    g = torch.Generator(device="cpu").manual_seed(4242)
    q = torch.nn.functional.normalize(torch.randn(B, H, dk, generator=g), dim=-1).to(torch.bfloat16).to(dev)
    k = torch.nn.functional.normalize(torch.randn(B, H, dk, generator=g), dim=-1).to(torch.bfloat16).to(dev)
    v = torch.randn(B, H, dv, generator=g).to(torch.bfloat16).to(dev)
    la = torch.nn.functional.logsigmoid(torch.randn(B, H, dk, generator=g) + 3.0).to(dev)
    b = torch.sigmoid(torch.randn(B, H, dk, generator=g)).to(dev)
    w = torch.sigmoid(torch.randn(B, H, dv, generator=g)).to(dev)
    S = (0.02 * torch.randn(B, H, dk, dv, generator=g)).to(dev)
    for _ in range(5):
        gdn2.step(q, k, v, la, b, w, S, in_place=True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        gdn2.step(q, k, v, la, b, w, S, in_place=True)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    nbytes = B * H * (2 * dk * dv * 4 + (2 * dk + dv) * 2 + (2 * dk + dv) * 4 + dv * 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"entry": "gdn2_step", "B": B, "H": H, "dk": dk, "dv": dv, "qkv": "bf16", "us_per_step": round(us, 2),
            "tokens_per_s": round(B / (us * 1e-6), 1), "algorithmic_bytes": nbytes, "achieved_GBs": round(gbs, 1),
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


# MI355X dense bf16 MFMA peak (TFLOP/s) and the forward's useful flops per token-head at
# dk = dv = 128, chunk C = 64 (the chunk equations, per chunk and head, / 64 tokens):
#   A = strictly-lower(Et Kt^T)  d C (C - 1)      = 516,096
#   P = lower(Qt Kt^T)           d C (C + 1)      = 532,480
#   T = (I + A)^-1               C^3 / 3          =  87,381
#   X = Z - Et S, Qt S, Kt^T U   3 x 2 C d^2      = 6,291,456
#   U = T X, P U                 2 x d C (C + 1)  = 1,064,960
#   -> 8,492,373 per chunk and head = 132,693 per token-head
MFMA_PEAK_TFLOPS = 2500.0
FWD_USEFUL_FLOPS_PER_TOKHEAD = 8492373 / 64


def _mfma_insts(kernel_key):
    """MFMA instructions per launch from the committed counter profile (SQ_INSTS_MFMA),
    if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("sources_digest") != _kernel_sources_digest():
        return None
    return rec.get("kernels", {}).get(kernel_key, {}).get("mfma_insts_per_launch")


def forward_bench(dev, wl, iters=20):
    """The inference forward gdn2_chunk_fwd (o and S_final) on the training shape, timed
    with HIP events.  At this shape it launches the forward-only chunk-record kernel, then
    the eight-wave sweep, with the records in a workspace; `hbm` counts the operator's own
    inputs and outputs, `hbm_with_records` adds the records written and read back."""
    import torch
    import linear_attention_sequence_gdn2_amd as gdn2
    from linear_attention_sequence_gdn2_amd.inputs import make_workload
    x = make_workload(wl)
    d = {k: x[k].to(dev) for k in ("q", "k", "v", "log_alpha", "b", "w")}
    args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"])
    for _ in range(3):
        gdn2.fwd(*args)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        gdn2.fwd(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    tokheads = wl.B * wl.T * wl.H
    state = wl.B * wl.H * wl.dk * wl.dv * 4
    nbytes = FWD_BYTES_PER_TOKHEAD * tokheads + state
    kbytes = (FWD_RECORDS_BYTES_PER_TOKHEAD + FWD_INFER_SWEEP_BYTES_PER_TOKHEAD) * tokheads + state
    gbs, kgbs = nbytes / (ms * 1e-3) / 1e9, kbytes / (ms * 1e-3) / 1e9
    tfl = FWD_USEFUL_FLOPS_PER_TOKHEAD * tokheads / (ms * 1e-3) / 1e12
    out = {"entry": "gdn2_chunk_fwd", "kernels": ["bwd_factors_kernel (forward-only records)", "fwd_sweep64_kernel"],
           "ms": round(ms, 4), "tokens_per_s": round(wl.B * wl.T / (ms * 1e-3), 1),
           "hbm": {"achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)},
           "hbm_with_records": {"achieved_GBs": round(kgbs, 1), "frac": round(kgbs / HBM_PEAK_GBS, 4)},
           "mfma_useful": {"achieved_TFLOPs": round(tfl, 1), "peak": MFMA_PEAK_TFLOPS,
                           "frac": round(tfl / MFMA_PEAK_TFLOPS, 4)}}
    i1, i2 = _mfma_insts("fwd_records_kernel"), _mfma_insts("fwd_infer_sweep_kernel")
    if i1 and i2:
        ex = (i1 + i2) * 16384 / (ms * 1e-3) / 1e12
        out["mfma_executed"] = {"achieved_TFLOPs": round(ex, 1), "frac": round(ex / MFMA_PEAK_TFLOPS, 4)}
    return out


# the other configurations of the operator, measured beside the headline: forward of the long
# sequence and of the per-token (KDA) gates, and the whole training step at B4 T4096
OTHER_FORWARD = ("long_bf16_B1H16T16384d128", "kda_bf16_B4H16T4096d128", "fwdbwd_bf16_B4H16T4096d128")
OTHER_STEP = ("fwdbwd_bf16_B4H16T4096d128",)


def _nbytes(*ts):
    return sum(t.numel() * t.element_size() for t in ts if t is not None)


def configs_bench(dev, timed_steps, iters=10, steps=10, warmup=3):
    """Forward (gdn2_chunk_fwd) and training-step times of the other configurations, HIP events.
    HBM fractions count the operator's own inputs and outputs (the tensors as given: bf16 q/k/v,
    fp32 gates, per-token gates where the workload has them)."""
    import torch
    import linear_attention_sequence_gdn2_amd as gdn2
    from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_workload
    res = {}
    for name in OTHER_FORWARD:
        wl = WORKLOADS[name]
        x = make_workload(wl, grads=name in OTHER_STEP)
        d = {k: (v.to(dev) if v is not None and hasattr(v, "to") else None) for k, v in x.items()
             if k in ("q", "k", "v", "log_alpha", "b", "w", "S0")}
        args = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
        o, sf = gdn2.fwd(*args)
        for _ in range(2):
            gdn2.fwd(*args)
        stream = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            gdn2.fwd(*args)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        io = _nbytes(*args, o, sf)
        r = {"B": wl.B, "T": wl.T, "H": wl.H, "dk": wl.dk, "dv": wl.dv,
             "forward_ms": round(ms, 4), "forward_tokens_per_s": round(wl.B * wl.T / (ms * 1e-3), 1),
             "forward_hbm_frac": round(io / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        if name in OTHER_STEP:
            wall, k_ms, step_ms = timed_steps(x, steps, warmup, wl=wl)
            # the backward reads the forward's inputs, dO and dS_final, and writes the seven fp32
            # gradients (dq, dk, dv in fp32 whatever the dtype of q, k, v)
            grads = 4 * (d["q"].numel() + d["k"].numel() + d["v"].numel()) + _nbytes(*args[3:6], sf)
            bwd_io = _nbytes(*args) + _nbytes(o, sf) + grads
            r.update({"step_ms": round(wall / steps * 1e3, 4),
                      "step_tokens_per_s": round(wl.B * wl.T / (wall / steps), 1),
                      "kernel_ms": [round(v, 4) for v in k_ms],
                      "sweeps_one_launch": gdn2.sweeps_fused(wl.B, wl.T, wl.H, wl.dk, wl.dv, d["q"].dtype),
                      "step_algorithmic_frac": round((io + bwd_io) / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)})
        res[name] = r
    return res


# output epilogue (RMS norm, weight, output gate) per token-head at dv = 128, bf16 gate and y:
#   forward : o 512 + g 256 + y 256                      = 1024
#   backward: o 512 + g 256 + dy 512 + dO 512 + dg 512   = 2304  (+ dweight partials per workgroup)
OUT_FWD_BYTES_PER_TOKHEAD = 1024
OUT_BWD_BYTES_PER_TOKHEAD = 2304


def output_bench(dev, wl, iters=20):
    """The output epilogue (gdn2_output_fwd / gdn2_output_bwd with dweight) on the
    operator's output shape of the training workload."""
    import torch
    import linear_attention_sequence_gdn2_amd as gdn2
    from linear_attention_sequence_gdn2_amd.inputs import make_output_inputs
    x = {k: v.to(dev) for k, v in make_output_inputs(wl.B, wl.T, wl.H, wl.dv, seed=4343, g_dtype="bf16").items()}
    ws = torch.empty(gdn2.output_bwd_workspace_bytes(wl.B, wl.T, wl.H, wl.dv), dtype=torch.uint8, device=dev)

    def fwd():
        return gdn2.output_fwd(x["o"], x["g"], x["weight"], 1e-6, out_dtype=torch.bfloat16)

    def bwd():
        return gdn2.output_bwd(x["o"], x["g"], x["weight"], 1e-6, x["dy"], workspace=ws)

    stream = torch.cuda.current_stream(dev)
    res = {}
    tokheads = wl.B * wl.T * wl.H
    for name, fn, per in (("fwd", fwd, OUT_FWD_BYTES_PER_TOKHEAD), ("bwd", bwd, OUT_BWD_BYTES_PER_TOKHEAD)):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        gbs = per * tokheads / (ms * 1e-3) / 1e9
        res[name] = {"entry": "gdn2_output_" + name, "ms": round(ms, 4), "algorithmic_bytes": per * tokheads,
                     "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
    res["shape"] = {"B": wl.B, "T": wl.T, "H": wl.H, "dv": wl.dv, "g": "bf16", "y": "bf16", "dy": "f32"}
    # a plain device copy of 512 MiB (read + write bytes / time): what a write-heavy stream reaches
    src = torch.empty(1 << 27, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    res["copy_reference_GBs"] = round(2 * src.numel() * 4 / (ms * 1e-3) / 1e9, 1)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the recurrent-step (decode) measurement")
    ap.add_argument("--no-logit-gates", action="store_true", help="skip the step with bf16 logit gates")
    ap.add_argument("--no-token-gates", action="store_true", help="skip the step with per-token gates")
    ap.add_argument("--no-output", action="store_true", help="skip the output epilogue measurement")
    ap.add_argument("--no-forward", action="store_true", help="skip the inference-forward measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the long-sequence, per-token-gate and B4 T4096 training measurements")
    ap.add_argument("--cpu-sample-batches", type=int, default=8)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (3 times), to calibrate "
                         "rocprofv3 FETCH_SIZE/WRITE_SIZE against known bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this operator benchmark runs on exactly one GPU; --gpus %d is not supported "
              "(multi-GPU sharding is design-only)." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import linear_attention_sequence_gdn2_amd as gdn2
    from linear_attention_sequence_gdn2_amd.inputs import WORKLOADS, make_workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.rand(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": 3}))
        return
    wl = WORKLOADS[WORKLOAD]
    stream = torch.cuda.current_stream(dev)
    nk = 4

    def timed_steps(x, steps, warmup, wl=wl):
        """Run `warmup` then `steps` training steps on the inputs x (of workload wl); returns
        (wall seconds, per-kernel event ms averaged over the steps, whole-step event ms)."""
        d = {k: (v.to(dev) if v is not None and hasattr(v, "to") else None)
             for k, v in x.items() if k in ("q", "k", "v", "log_alpha", "b", "w", "S0", "dO", "dS_final")}
        fargs = (d["q"], d["k"], d["v"], d["log_alpha"], d["b"], d["w"], d["S0"])
        sshape = gdn2.states_shape(wl.B, wl.T, wl.H, wl.dk, wl.dv)
        states = torch.empty(sshape, dtype=torch.float32, device=dev)
        dstates = torch.empty(sshape, dtype=torch.float32, device=dev)
        factors = torch.empty(gdn2.factors_bytes(wl.B, wl.T, wl.H, wl.dk, wl.dv), dtype=torch.uint8, device=dev)

        # One training step = four kernel launches:
        #   bwd_factors_kernel  (gdn2_chunk_bwd_factors: per-chunk adjoint factors R, Q2 and the
        #                        key-side chunk operands)
        #   fwd_sweep_kernel    (gdn2_chunk_fwd_factored: o, S_final and the chunk-start states)
        #   bwd_reverse_kernel  (gdn2_chunk_bwd_reverse: end-state gradient of every chunk, dS0)
        #   bwd_chunk_kernel    (gdn2_chunk_bwd_grads: dq, dk, dv, dlog_alpha, db, dw)
        # With few heads gdn2_chunk_sweeps runs the middle two as one launch (fwd_rev_sweep_kernel);
        # the step then calls it, and its time is the second entry of the breakdown (the third is 0).
        fused = gdn2.sweeps_fused(wl.B, wl.T, wl.H, wl.dk, wl.dv, d["q"].dtype)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            gdn2.bwd_factors(d["q"], d["k"], d["log_alpha"], d["b"], factors=factors)
            if ev is not None:
                ev[1].record(stream)
            if fused:
                o, sf, _, _, dS0 = gdn2.sweeps(factors, d["v"], d["w"], wl.dk, d["S0"], d["dO"], d["dS_final"],
                                               states=states, dstates=dstates)
                if ev is not None:
                    ev[2].record(stream)
            else:
                o, sf, _ = gdn2.fwd_factored(factors, d["v"], d["w"], wl.dk, d["S0"], states=states)
                if ev is not None:
                    ev[2].record(stream)
                _, dS0 = gdn2.bwd_reverse(factors, d["dO"], wl.dk, d["dS_final"], dstates=dstates)
            if ev is not None:
                ev[3].record(stream)
            g = gdn2.bwd_grads(*fargs[:6], d["dO"], states, dstates, factors)
            if ev is not None:
                ev[4].record(stream)
            return o, sf, g, dS0

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            step(evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        k_ms = [sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j in range(nk)]
        step_ms = sum(e[0].elapsed_time(e[nk]) for e in evs) / steps
        return wall, k_ms, step_ms

    wall, k_ms, step_ms = timed_steps(make_workload(wl, grads=True), args.steps, args.warmup)
    tokens = wl.B * wl.T
    tokheads = wl.B * wl.T * wl.H
    state_bytes = wl.B * wl.H * wl.dk * wl.dv * 4
    value = tokens / (wall / args.steps)

    # algorithmic bytes per launch of each kernel (per token-head figures times
    # B*T*H, plus per-sequence states), from the per-token-head constants above
    kernels = [
        ("bwd_factors_kernel", "gdn2_chunk_bwd_factors", BWD_FACTORS_BYTES_PER_TOKHEAD * tokheads),
        ("fwd_sweep_kernel", "gdn2_chunk_fwd_factored", FWD_SWEEP_BYTES_PER_TOKHEAD * tokheads + state_bytes),
        ("bwd_reverse_kernel", "gdn2_chunk_bwd_reverse", BWD_REVERSE_BYTES_PER_TOKHEAD * tokheads + 2 * state_bytes),
        ("bwd_chunk_kernel", "gdn2_chunk_bwd_grads", BWD_GRADS_BYTES_PER_TOKHEAD * tokheads),
    ]
    per_kernel = {}
    for (name, entry, nbytes), ms in zip(kernels, k_ms):
        gbs = nbytes / (ms * 1e-3) / 1e9
        per_kernel[name] = {"entry": entry, "launch_ms": round(ms, 4), "algorithmic_bytes": nbytes,
                            "achieved_GBs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}
        insts = _mfma_insts(name)
        if insts:   # executed bf16 MFMA (16x16x32: 16384 flops each), split operands included
            ex = insts * 16384 / (ms * 1e-3) / 1e12
            per_kernel[name]["mfma_executed_TFLOPs"] = round(ex, 1)
            per_kernel[name]["mfma_frac"] = round(ex / MFMA_PEAK_TFLOPS, 4)
    dom = max(range(nk), key=lambda j: k_ms[j])
    name, entry, nbytes = kernels[dom]
    achieved = nbytes / (k_ms[dom] * 1e-3) / 1e9
    roof = {"bound": "hbm", "kernel": name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": _traffic(name, nbytes),
            "algorithmic_bytes_per_launch": nbytes, "launch_ms": round(k_ms[dom], 4)}
    step_alg = (FWD_BYTES_PER_TOKHEAD + BWD_BYTES_PER_TOKHEAD) * tokheads
    out = {
        "metric": "GDN-2 chunk fwd+bwd tokens/s (H=16 dk=dv=128 B8xT2K)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "B": wl.B, "T": wl.T, "H": wl.H, "dk": wl.dk, "dv": wl.dv,
                   "chunk": 64, "seed": wl.seed, "qkv": "bf16", "gates_state_grads": "fp32",
                   "parallelism": "single-gpu"},
        "breakdown": {"kernels": per_kernel, "step_event_ms": round(step_ms, 4),
                      "fwd_tokens_per_s": round(tokens / ((k_ms[0] + k_ms[1]) * 1e-3), 1),
                      "step_algorithmic_frac": round(step_alg / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roof,
    }
    if not args.no_logit_gates:
        # the same step with the gates given as bf16 logits (activated in the kernels)
        lwl = WORKLOADS[LOGIT_WORKLOAD]
        lwall, lk_ms, lstep_ms = timed_steps(make_workload(lwl), args.steps, args.warmup)
        lalg = (FWD_BYTES_PER_TOKHEAD + BWD_BYTES_PER_TOKHEAD - 2 * GATE_BYTES_SAVED_PER_TOKHEAD) * tokheads
        out["breakdown"]["logit_gates_step"] = {
            "workload": LOGIT_WORKLOAD, "ms_per_step": round(lwall / args.steps * 1e3, 4),
            "tokens_per_s": round(tokens / (lwall / args.steps), 1),
            "kernel_ms": {kn[0]: round(ms, 4) for kn, ms in zip(kernels, lk_ms)},
            "step_event_ms": round(lstep_ms, 4),
            "step_algorithmic_frac": round(lalg / (lstep_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if not args.no_token_gates:
        # the same step with Gated DeltaNet's gates, one value per token ([B,T,H])
        twl = WORKLOADS[TOKEN_WORKLOAD]
        twall, tk_ms, tstep_ms = timed_steps(make_workload(twl), args.steps, args.warmup)
        talg = (FWD_BYTES_PER_TOKHEAD + BWD_BYTES_PER_TOKHEAD - 3 * TOKEN_GATE_BYTES_SAVED_PER_TOKHEAD) * tokheads
        out["breakdown"]["token_gates_step"] = {
            "workload": TOKEN_WORKLOAD, "ms_per_step": round(twall / args.steps * 1e3, 4),
            "tokens_per_s": round(tokens / (twall / args.steps), 1),
            "kernel_ms": {kn[0]: round(ms, 4) for kn, ms in zip(kernels, tk_ms)},
            "step_event_ms": round(tstep_ms, 4),
            "step_algorithmic_frac": round(talg / (tstep_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if not args.no_forward:
        out["breakdown"]["forward_only"] = forward_bench(dev, wl)
    if not args.no_configs:
        out["breakdown"]["other_configs"] = configs_bench(dev, timed_steps)
    if not args.no_output:
        out["breakdown"]["output_epilogue"] = output_bench(dev, wl)
    if not args.no_decode:
        out["breakdown"]["decode_step"] = decode_bench(dev)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_sample_batches)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
