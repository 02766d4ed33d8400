#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

Metric: chunk_kda fwd+bwd tokens/s at H16, D128, T8192 (packed sequences of
1024/2048/1024/4096 tokens, bf16 q/k/v, fp32 gate/beta/state), plus batched
decode sequence-steps/s at 64 sequences x H96 x d128, with roofline fractions.

A step is one kda_chunk_fwd + one kda_chunk_bwd over the packed batch (every
stage of both, each timed with HIP events on the launch stream).  Inputs are
synthetic (see kimi_delta_attention_amd/inputs.py) and resident in HBM before
the timed region; two input sets alternate so that the 256 MiB Infinity Cache
cannot serve one step from the previous one.

The headline `roofline` is the whole fwd+bwd step against its operator-level
bytes (every operator input and output crossing HBM once: 4,364 B per
token-head at d = 128 in bf16, plus the states), with each stage's share next
to the HBM bytes its kernel was counted moving.  The bytes this design's
kernels pass each other through the workspace are a labelled secondary figure.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

# MI355X published peaks (dense): HBM3E 8 TB/s; bf16 MFMA 2.5 PFLOP/s.
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0

HYBRID_CU = [0, 1024, 3072, 4096, 8192]
T_H, H_H, D_H = 8192, 16, 128


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


# ---------------------------------------------------------------- algorithmic work
# Per (chunk, head) slot of C = 64 rows: the HBM bytes each kernel must move in
# this design (every operand read once, every result written once; the
# per-chunk operands that one kernel hands to the next live in the workspace
# in bf16) and the flops of its MFMA-shaped products (triangular products at
# their triangular size).  elt is the byte size of q, k, v, o, dO and their
# gradients; intermediates are bf16.  Per-sequence terms (initial and final
# states) are added by stage_work().
C = 64


def _slot_terms(K, V, elt):
    e = 2
    tri = (C + 1) / 2
    qkv_in = C * (2 * K + V) * elt + 4 * C * K + 4 * C          # q, k, v, g, beta
    prep_out = e * (3 * C * K + C * V + 2 * C * C) + 4 * K      # QE, W, KD, U, TB, MS, GC
    prep_f = C * (2 * tri * K * 2 + 2 * tri * V) + C ** 3 / 3   # A, M, W, U; the solve
    return {
        "fwd.prep": (qkv_in + prep_out, prep_f),
        "fwd.state": (e * (3 * C * K + C * V + C * C) + 4 * K + C * V * elt, C * 6 * K * V + C * 2 * tri * V),
        "bwd.0": (qkv_in + prep_out + e * (C * K + 2 * C * C), prep_f),
        "bwd.1": (e * (2 * C * K + C * V) + 4 * K + e * K * V, C * 4 * K * V),
        "bwd.2": (e * (3 * C * K + C * C) + 4 * K + C * V * elt + e * K * V, C * (6 * K * V + 2 * tri * V)),
        "bwd.3": (e * (2 * C * K + 2 * C * C + 2 * K * V) + C * V * elt + C * V * elt
                  + e * (3 * C * K + 2 * C * C) + 4 * K,
                  C * (6 * K * V + 3 * 2 * tri * V)),
        "bwd.4": (C * 2 * K * elt + 4 * C * K + 4 * C + e * (4 * C * C + 3 * C * K) + 4 * K
                  + C * 2 * K * elt + 4 * C * K + 4 * C + 4 * (K + 1),
                  4 * C ** 3 + C * 4 * 2 * tri * K),
    }


def stage_work(slots, n_seq, H, K, V, elt, with_h0=False, keep=True):
    """{stage: (bytes, flops)} for one launch over `slots` (chunk, head) slots.
    With keep the forward's prep writes the backward's operands too (as bwd.0)
    and its state pass also stores each chunk's entry state (as bwd.1)."""
    terms = _slot_terms(K, V, elt)
    out = {k: (b * slots, f * slots) for k, (b, f) in terms.items()}
    st = n_seq * H * K * V * 4
    if keep:
        out["fwd.prep"] = out["bwd.0"]
        b, f = out["fwd.state"]
        out["fwd.state"] = (b + 2 * K * V * slots, f)
    b, f = out["fwd.state"]
    out["fwd.state"] = (b + st * (2 if with_h0 else 1), f)
    b, f = out["bwd.2"]
    out["bwd.2"] = (b + st * 2, f)  # d(final state) in, d(initial state) out
    return out


def stage_roofline(name, work, ms):
    """Roofline entry of one kernel: the bound is the one its algorithmic work hits first."""
    nbytes, flops = work
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    if t_hbm >= t_mfma:
        ach = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": name, "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
                "kernel_ms": ms}
    ach = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma", "kernel": name, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": ach / PEAK_BF16_TFLOPS, "algorithmic_bytes": nbytes, "algorithmic_flops": flops,
            "kernel_ms": ms}


# Whole-path figures per token-head at d = 128 (operator inputs and outputs
# only): forward 1,540 B and 141,013 flops; forward + backward 4,364 B and
# about 423 k flops (three times the forward, recomputation not counted).
PATH_FWD = (1540, 141013)
PATH_FWDBWD = (4364, 423039)


def path_shares(K, V, elt):
    """Operator-level HBM bytes per token-head of one fwd+bwd step, each operator
    input and output crossing HBM once, assigned to the stage that first reads
    or writes it: the prep reads q, k, v, g, beta; the state pass writes o; the
    reverse state pass reads dO; V-local reads v and writes dv; K-local reads q,
    k, g, beta again and writes dq, dk, dg, dbeta.  At K = V = 128 in bf16 these
    are 1,284 + 256 + 256 + 512 + 2,056 = 4,364 B."""
    return {
        "fwd.prep": (2 * K + V) * elt + 4 * K + 4,
        "fwd.state": V * elt,
        "bwd.2": V * elt,
        "bwd.3": 2 * V * elt,
        "bwd.4": 2 * K * elt + 4 * K + 4 + 2 * K * elt + 4 * K + 4,
    }


def path_roofline(stage_ms, step_ms, token_heads, K, V, elt, state_bytes, design):
    """Headline roofline of the whole fwd+bwd step against its operator-level
    bytes (path_shares per token-head, plus the final state written by the
    forward and d(initial state) written by the backward), over the measured
    step time.  Each stage carries its own share next to the counted HBM bytes
    of its kernel; the bytes this design's kernels hand each other through the
    workspace are the secondary `design_bytes` figure."""
    shares = path_shares(K, V, elt)
    per = {}
    total_share = 0
    traffic = 0.0
    for n, ms in stage_ms.items():
        share = shares.get(n, 0) * token_heads
        if n == "fwd.state":
            share += state_bytes
        if n == "bwd.2":
            share += state_bytes
        total_share += share
        tr = stored_traffic(n)
        traffic = None if (traffic is None or tr is None) else traffic + tr
        per[n] = {"kernel_ms": ms, "share_bytes": share, "share_frac": share / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "design_bytes": design[n][0],
                  "design_frac": design[n][0] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                  "traffic": tr, "traffic_ratio": None if tr is None else tr / share if share else None,
                  "mfma_util": stored_mfma_util(n)}
    ach = total_share / (step_ms * 1e-3) / 1e9
    return {"bound": "hbm", "kernel": "fwd+bwd path (every stage of kda_chunk_fwd + kda_chunk_bwd)",
            "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
            "traffic": traffic, "traffic_ratio": None if traffic is None else traffic / total_share,
            "algorithmic_bytes": total_share, "step_ms": step_ms,
            "stage_sum_ms": sum(stage_ms.values()), "stages": per}


def decode_bytes(N, H, D, W, x_elt):
    """State and conv state read + written once; x, g, beta, conv_w read; o written."""
    return (2 * N * H * D * D * 4 + 2 * N * 3 * H * D * W * 4 + N * 3 * H * D * x_elt + N * H * D * 4
            + N * H * 4 + 3 * H * D * W * 4 + N * H * D * 4)


def gate_bytes(rows, H, V, elt):
    """Output gate: o and g read, y written once (elt bytes each)."""
    return 3 * rows * H * V * elt


def gate_bwd_bytes(rows, H, V, elt):
    """Its reverse mode: o, g and dy read, dO and dg written once (elt bytes each)."""
    return 5 * rows * H * V * elt


def conv_bytes(rows, n_seq, H, D, W, elt):
    """x read once and q, k, v written once (elt bytes each); conv_w read; the
    conv state read and written once per sequence."""
    C = 3 * H * D
    return 2 * rows * C * elt + C * W * 4 + 2 * n_seq * C * W * 4


# ---------------------------------------------------------------- workloads
def make_hybrid(seed, device):
    from kimi_delta_attention_amd import inputs
    w = inputs.chunk_inputs(1, T_H, H_H, D_H, D_H, seed=seed, dtype=torch.bfloat16, cu_seqlens=HYBRID_CU,
                            with_grad_out=True)
    return w, {k: (v.to(device) if hasattr(v, "to") else v) for k, v in w.items()}


def chunk_op(d, with_bwd, keep=True):
    import kimi_delta_attention_amd as kda
    return kda.ChunkOp(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"], initial_state=None,
                       output_final_state=True, use_qk_l2norm_in_kernel=True, gate_mode=d["gate_mode"],
                       use_beta_sigmoid_in_kernel=d["use_beta_sigmoid"], lower_bound=d["lower_bound"],
                       cu_seqlens=d["cu_seqlens"], dO=d["dO"] if with_bwd else None,
                       keep_for_backward=with_bwd and keep)


def time_chunk(ops, steps, warmup, with_bwd, n_bwd_stages, keep=True):
    """Mean seconds per fwd(+bwd) step, timed over whole calls (host clock), mean
    ms per stage from a second run of the same steps stage by stage, and the
    mean ms per whole step from HIP events on the launch stream.  With keep the
    forward saves what the backward's stages 0 and 1 would recompute, and those
    stages (which then launch nothing) are not called."""
    stream = torch.cuda.current_stream()
    first = 2 if keep else 0
    bwd_stages = list(range(first, n_bwd_stages)) if with_bwd else []
    names = ["fwd.prep", "fwd.state"] + [f"bwd.{i}" for i in bwd_stages]

    def one(op, evs):
        k = 0
        for st in range(2):
            evs[k].record(stream)
            op.forward(stage=st)
            k += 1
        if with_bwd:
            for st in bwd_stages:
                evs[k].record(stream)
                op.backward(stage=st)
                k += 1
        evs[k].record(stream)

    def whole(op):
        op.forward()
        if with_bwd:
            op.backward()

    # the timed steps: whole kda_chunk_fwd / kda_chunk_bwd calls, as a caller makes them
    for i in range(warmup):
        whole(ops[i % len(ops)])
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(steps):
        whole(ops[i % len(ops)])
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = ev0.elapsed_time(ev1) / steps  # HIP events on the launch stream
    # then the same steps stage by stage, with events between the stages, for the breakdown
    for i in range(min(warmup, 2)):
        one(ops[i % len(ops)], [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)])
    all_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        one(ops[i % len(ops)], all_evs[i])
    torch.cuda.synchronize()
    per = {n: [] for n in names}
    for evs in all_evs:
        for j, n in enumerate(names):
            per[n].append(evs[j].elapsed_time(evs[j + 1]))
    return (t1 - t0) / steps, {n: sum(v) / len(v) for n, v in per.items()}, step_ms


def run_decode(steps, warmup, device):
    import kimi_delta_attention_amd as kda
    from kimi_delta_attention_amd import inputs
    shp = inputs.DECODE_SHAPE
    N, H, D, W = shp["N"], shp["H"], shp["D"], shp["W"]
    seed = inputs.SEEDS["decode"]
    init = inputs.decode_init(N, H, D, W, seed=seed)
    cw = init["conv_w"].to(device)
    cs = init["conv_state"].to(device)
    st = init["state"].to(device)
    n_in = min(16, steps + warmup)
    ins = []
    for t in range(n_in):
        s = inputs.decode_step_inputs(N, H, D, seed=seed, step=t)
        ins.append({k: v.to(device) for k, v in s.items()})
    o = torch.empty(N, H * D, device=device)
    stream = torch.cuda.current_stream()
    for t in range(warmup):
        s = ins[t % n_in]
        kda.recurrent_step(s["x"], cw, cs, s["g"], s["beta"], st, out=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for t in range(steps):
        s = ins[(warmup + t) % n_in]
        kda.recurrent_step(s["x"], cw, cs, s["g"], s["beta"], st, out=o)
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = e0.elapsed_time(e1) / steps  # back-to-back launches: the average launch duration
    wall = (t1 - t0) / steps
    algo = decode_bytes(N, H, D, W, 2)
    # the same steps with the full-rank output gate fused into the step
    gates = [inputs.gate_inputs(N, H, D, seed=seed + 10 + t)["g"].reshape(N, H * D).to(device) for t in range(2)]
    for t in range(warmup):
        s = ins[t % n_in]
        kda.recurrent_step(s["x"], cw, cs, s["g"], s["beta"], st, out=o, out_gate=gates[t % 2])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for t in range(steps):
        s = ins[(warmup + t) % n_in]
        kda.recurrent_step(s["x"], cw, cs, s["g"], s["beta"], st, out=o, out_gate=gates[t % 2])
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gk_ms = e0.elapsed_time(e1) / steps
    galgo = algo + N * H * D * 2
    gated = {"value": N * steps / (t1 - t0), "unit": "seq/s", "kernel_ms": gk_ms, "algorithmic_bytes": galgo,
             "frac": galgo / (gk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
             "workload": "the same decode steps with the full-rank output gate (bf16 gate input) fused"}
    return {
        "metric": "decode sequence-steps/s", "unit": "seq/s", "value": N / wall,
        "ms_per_step": wall * 1e3, "workload": f"decode N{N} H{H} d{D} conv{W} bf16 x, fp32 state",
        "roofline": {"bound": "hbm", "kernel": "decode_step_kernel", "achieved": algo / (kern_ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": algo / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": stored_traffic("decode", "decode"),
                     "algorithmic_bytes": algo, "kernel_ms": kern_ms,
                     "timing": f"{steps} back-to-back steps between two events (state {N * H * D * D * 4 >> 20} MiB, "
                               "above the Infinity Cache)"},
        "with_output_gate": gated,
    }


def run_prefill(steps, warmup, device):
    """Stateful prefill of the packed batch: the short conv from a conv state
    (kda_conv_prefill), then the chunk forward from a decode state with the
    final states out and the full-rank output gate (kda_chunk_fwd with
    out_gate; at these 64 chains the library gates o in place right after the
    state pass) -- the prime that hands over to decode.  The same prefill with
    the gate as a call of its own (kda_output_gate after the plain forward) is
    timed beside it for comparison."""
    import kimi_delta_attention_amd as kda
    from kimi_delta_attention_amd import inputs
    H, D, W = H_H, D_H, 4
    cu = torch.tensor(HYBRID_CU, dtype=torch.int32, device=device)
    n_seq = len(HYBRID_CU) - 1
    pre = inputs.prefill_inputs(T_H, H, D, seed=inputs.SEEDS["decode"] + 1)
    init = inputs.decode_init(n_seq, H, D, W, seed=inputs.SEEDS["decode"] + 2)
    x = pre["x"].to(device)
    g = pre["g"].to(device).reshape(1, T_H, H, D)
    beta = pre["beta"].to(device).reshape(1, T_H, H)
    cw = init["conv_w"].to(device)
    cs = init["conv_state"].to(device)
    st0 = init["state"].to(device)
    qkv = tuple(torch.empty(T_H, H, D, dtype=torch.bfloat16, device=device) for _ in range(3))
    g_out = inputs.gate_inputs(T_H, H, D, seed=inputs.SEEDS["decode"] + 3)["g"].to(device)
    y = torch.empty(T_H, H, D, dtype=torch.bfloat16, device=device)
    common = dict(initial_state=st0, output_final_state=True, use_qk_l2norm_in_kernel=True,
                  use_beta_sigmoid_in_kernel=True, cu_seqlens=cu)
    args = tuple(t.unsqueeze(0) for t in qkv) + (g, beta)
    fused = kda.ChunkOp(*args, out_gate=g_out.unsqueeze(0), **common)
    plain = kda.ChunkOp(*args, **common)
    stream = torch.cuda.current_stream()

    def conv():
        kda.conv_prefill(x, cw, H, D, conv_state=cs, cu_seqlens=cu, out=qkv)

    o = plain.o.reshape(T_H, H, D)

    def gate():
        kda.output_gate(o, g_out, out=y)

    for _ in range(warmup):
        conv()
        fused.forward()
        plain.forward()
        gate()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        conv()
        e[1].record(stream)
        fused.forward()
        e[2].record(stream)
        plain.forward()
        e[3].record(stream)
        gate()
        e[4].record(stream)
    torch.cuda.synchronize()
    conv_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    fwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    plain_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    gate_ms = sum(e[3].elapsed_time(e[4]) for e in ev) / steps
    algo = conv_bytes(T_H, n_seq, H, D, W, 2)
    galgo = gate_bytes(T_H, H, D, 2)
    gbalgo = gate_bwd_bytes(T_H, H, D, 2)

    # Each bandwidth kernel alone: back-to-back launches over R input/output
    # sets (R x 200 MB, above the 256 MiB Infinity Cache), so that no launch
    # finds the previous one's data cached and no event sits between launches.
    R = 4
    xs = [x] + [inputs.prefill_inputs(T_H, H, D, seed=inputs.SEEDS["decode"] + 20 + i)["x"].to(device)
                for i in range(R - 1)]
    css = [init["conv_state"].to(device) for _ in range(R)]
    outs = [qkv] + [tuple(torch.empty_like(qkv[0]) for _ in range(3)) for _ in range(R - 1)]
    gsets = []
    for i in range(R):
        gi = inputs.gate_inputs(T_H, H, D, seed=inputs.SEEDS["decode"] + 30 + i)
        gsets.append({k: gi[k].to(device) for k in ("o", "g", "dy")})
        gsets[-1].update(y=torch.empty_like(gsets[-1]["o"]), dO=torch.empty_like(gsets[-1]["o"]),
                         dg=torch.empty_like(gsets[-1]["g"]))
    n_loop = 8 * R
    conv_cold = time_rotating(lambda i: kda.conv_prefill(xs[i], cw, H, D, conv_state=css[i], cu_seqlens=cu,
                                                         out=outs[i]), R, n_loop, stream)
    gate_cold = time_rotating(lambda i: kda.output_gate(gsets[i]["o"], gsets[i]["g"], out=gsets[i]["y"]),
                              R, n_loop, stream)
    gbwd_cold = time_rotating(lambda i: kda.output_gate_bwd(gsets[i]["o"], gsets[i]["g"], gsets[i]["dy"],
                                                            out=(gsets[i]["dO"], gsets[i]["dg"])),
                              R, n_loop, stream)
    del xs, css, outs, gsets

    def roof(kernel, nbytes, ms, stage, pipe_ms):
        ach = nbytes / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "kernel": kernel, "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "algorithmic_bytes": nbytes, "kernel_ms": ms,
                "traffic": stored_traffic(stage, "prefill"),
                "timing": f"{n_loop} back-to-back launches over {R} rotating buffer sets",
                "in_pipeline_ms": pipe_ms}

    return {
        "metric": "stateful prefill tokens/s", "unit": "tokens/s",
        "value": T_H / ((conv_ms + fwd_ms) * 1e-3),
        "workload": f"conv{W} prefill + chunk forward from decode states with the output gate in the same call, packed "
                    f"1024/2048/1024/4096 (T{T_H}), H{H} d{D}, bf16 x/q/k/v/o/gate, fp32 states",
        "conv_ms": conv_ms, "chunk_fwd_gated_ms": fwd_ms,
        "conv_roofline": roof("conv_prefill_kernel", algo, conv_cold, "prefill.conv", conv_ms),
        "gate_roofline": roof("output_gate_kernel (forward)", galgo, gate_cold, "prefill.gate", gate_ms),
        "gate_bwd_roofline": roof("output_gate_kernel (reverse)", gbalgo, gbwd_cold, "prefill.gate_bwd", None),
        "unfused": {"value": T_H / ((conv_ms + plain_ms + gate_ms) * 1e-3), "chunk_fwd_ms": plain_ms,
                    "gate_ms": gate_ms,
                    "workload": "the same prefill with the plain forward and kda_output_gate as a call of its own"},
    }


def time_rotating(fn, R, n, stream):
    """Average duration (ms) of fn(i % R) over n back-to-back launches between two events."""
    for i in range(2 * R):
        fn(i % R)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(n):
        fn(i % R)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def hbm_ceiling(device, mib=1024, R=3, n=12):
    """What HBM sustains for a kernel with nothing to compute: the streaming copy
    and read of libkda_stream.so over R rotating mib-MiB buffers."""
    import ctypes
    from kimi_delta_attention_amd import build as kbuild
    lib = ctypes.CDLL(kbuild.STREAM_LIB)
    lib.kda_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.kda_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    nb = mib << 20
    src = [torch.ones(nb // 4, device=device) for _ in range(R)]
    dst = [torch.empty_like(t) for t in src]
    sink = torch.zeros(256, device=device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def call(f, *a):
        rc = f(*a)
        if rc:
            raise RuntimeError(f"stream calibration kernel failed ({rc})")

    t_copy = time_rotating(lambda i: call(lib.kda_stream_copy, src[i].data_ptr(), dst[i].data_ptr(), nb, sp),
                           R, n, stream)
    t_read = time_rotating(lambda i: call(lib.kda_stream_read, src[i].data_ptr(), sink.data_ptr(), nb, sp),
                           R, n, stream)
    del src, dst
    copy_gbs = 2 * nb / (t_copy * 1e-3) / 1e9
    read_gbs = nb / (t_read * 1e-3) / 1e9
    return {"copy_GBs": copy_gbs, "copy_frac": copy_gbs / PEAK_HBM_GBS, "read_GBs": read_gbs,
            "read_frac": read_gbs / PEAK_HBM_GBS,
            "what": f"streaming copy (nontemporal 16-byte loads and stores) and streaming read of {mib} MiB "
                    f"buffers, {R} rotating, {n} launches each"}


def cpu_baseline(host):
    """The oracle (fp64 token recurrence + BPTT) on the whole packed batch."""
    import oracle
    thr = oracle.default_threads()
    kw = dict(scale=host["scale"], use_qk_l2norm=True, gate_mode=host["gate_mode"], lower_bound=host["lower_bound"],
              use_beta_sigmoid=host["use_beta_sigmoid"], cu_seqlens=host["cu_seqlens"], threads=thr)
    t0 = time.perf_counter()
    oracle.chunk_fwd(host["q"], host["k"], host["v"], host["g"], host["beta"], **kw)
    oracle.chunk_bwd(host["q"], host["k"], host["v"], host["g"], host["beta"], host["dO"], **kw)
    dt = time.perf_counter() - t0
    return {"value": T_H / dt, "unit": "tokens/s", "cores": thr, "kind": "oracle",
            "sample": f"whole packed batch (T{T_H} H{H_H} d{D_H}, 4 sequences), fwd+bwd in fp64, {dt:.1f} s"}


def csrc_digest():
    """SHA-256 over the KDA kernel sources, to tell whether stored counter readings still apply
    (the calibration kernels of libkda_stream.so are not among them)."""
    import hashlib
    d = os.path.join(os.path.dirname(os.path.abspath(__file__)), "kimi_delta_attention_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".cpp")) and f != "stream_ceiling.hip":
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


# committed rocprofv3 summaries, one per leg (see the commands in their headers)
PROFILE_SUFFIX = {"chunk": "chunk_fwdbwd_T8192_H16_D128", "gated": "chunk_softplus_T8192_H16_D128",
                  "narrow": "chunk_narrow_B16_T2048_H8_K32_V64", "decode": "decode_N64_H96_D128",
                  "prefill": "prefill_T8192_H16_D128"}


def stored_traffic(stage, leg="chunk"):
    """HBM bytes per launch of `stage` from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary of `leg`, or None when there is none or the kernels changed since it was taken."""
    return _stored(f"hbm_traffic_{PROFILE_SUFFIX[leg]}.txt", f"hbm_bytes_per_launch[{stage}]")


def stored_mfma_util(stage, leg="chunk"):
    """MFMA busy fraction of `stage` from the committed rocprofv3 MFMA counter summary
    (SQ_VALU_MFMA_BUSY_CYCLES over the launch's cycles x 1,024 SIMDs), or None when
    there is none or the kernels changed since it was taken."""
    return _stored(f"mfma_util_{PROFILE_SUFFIX[leg]}.txt", f"mfma_util[{stage}]")


def _stored(name, key):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith((" ", "#", "|")):
                k, v = ln.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("csrc_sha256") != csrc_digest():
        return None
    v = kv.get(key)
    return float(v) if v else None


def copy_probe(mib, device):
    """A plain device copy of known size, so that a counter run can calibrate FETCH_SIZE / WRITE_SIZE."""
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device=device).fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    _log(f"copy probe: {mib} MiB read + {mib} MiB written per launch")
    del src, dst


def run_train(steps, warmup, device):
    """Forward + backward on the dense training shape B8 x T4096, H16, K=V=128 (bf16 q/k/v/dO, fp32
    g/beta/state), with an explicit zero initial state so that d(initial state) is produced."""
    from kimi_delta_attention_amd import inputs
    import kimi_delta_attention_amd as kda
    w = inputs.workload("train")
    d = {k: (v.to(device) if hasattr(v, "to") else v) for k, v in w.items()}
    B, T, H, K = d["q"].shape
    h0 = torch.zeros(B, H, K, K, dtype=torch.float32, device=device)
    op = kda.ChunkOp(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"], initial_state=h0,
                     output_final_state=True, use_qk_l2norm_in_kernel=True, gate_mode=d["gate_mode"],
                     use_beta_sigmoid_in_kernel=d["use_beta_sigmoid"], lower_bound=d["lower_bound"], dO=d["dO"],
                     keep_for_backward=True)
    sec, per_stage, _ = time_chunk([op], steps, warmup, True, _lib_stages())
    tokens = B * T
    fwd_ms = per_stage["fwd.prep"] + per_stage["fwd.state"]
    pb, pf = PATH_FWDBWD
    th = tokens * H
    return {"workload": f"chunk_kda fwd+bwd, dense B{B} x T{T}, H{H}, K=V={K}, bf16 q/k/v/dO, fp32 g/beta/state, "
                        "zero initial state passed, forward saves for backward",
            "tokens_per_s": tokens / sec, "ms_per_step": sec * 1e3,
            "fwd_tokens_per_s": tokens / (fwd_ms * 1e-3), "stages_ms": per_stage,
            "path_hbm_frac": pb * th / sec / 1e9 / PEAK_HBM_GBS,
            "path_mfma_frac": pf * th / sec / 1e12 / PEAK_BF16_TFLOPS}


def run_variant(B, T, H, K, V, cu, gate, steps, warmup, device, seed, what):
    """Forward + backward of another geometry or gate form, timed like the main
    step (forward saving for the backward, stages timed on the launch stream),
    two alternating input sets.  In-kernel gates also produce dA_log and
    d(dt_bias)."""
    from kimi_delta_attention_amd import inputs
    import kimi_delta_attention_amd as kda
    ops = []
    for sd in (seed, seed + 1000):
        w = inputs.chunk_inputs(B, T, H, K, V, seed=sd, dtype=torch.bfloat16, cu_seqlens=cu, gate_mode=gate,
                                beta_logits=gate != inputs.GATE_LOGDECAY, with_grad_out=True)
        d = {k: (v.to(device) if hasattr(v, "to") else v) for k, v in w.items()}
        ops.append(kda.ChunkOp(d["q"], d["k"], d["v"], d["g"], d["beta"], A_log=d["A_log"], dt_bias=d["dt_bias"],
                               scale=d["scale"], output_final_state=True, use_qk_l2norm_in_kernel=True,
                               gate_mode=gate, use_beta_sigmoid_in_kernel=d["use_beta_sigmoid"],
                               lower_bound=d["lower_bound"], cu_seqlens=d["cu_seqlens"], dO=d["dO"],
                               keep_for_backward=True))
    sec, per_stage, _ = time_chunk(ops, steps, warmup, True, _lib_stages())
    tokens = B * T if cu is None else cu[-1]
    leg = "narrow" if K != V else "gated"
    counted = {}
    for n, ms in per_stage.items():
        tr = stored_traffic(n, leg)
        counted[n] = {"kernel_ms": ms, "traffic": tr,
                      "traffic_frac": None if tr is None else tr / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                      "mfma_util": stored_mfma_util(n, leg)}
    return {"workload": what, "tokens_per_s": tokens / sec, "ms_per_step": sec * 1e3, "stages_ms": per_stage,
            "stages_counted": counted}


def run_leg(name, args, device):
    """One leg of the benchmark other than the main chunk step."""
    from kimi_delta_attention_amd import inputs
    try:
        if name == "train":
            _log("timing chunk path (dense B8 x T4096)")
            return run_train(max(args.steps // 2, 3), min(args.warmup, 3), device)
        if name == "gated":
            _log("timing chunk path (packed T8192) with the in-kernel softplus gate")
            return run_variant(1, T_H, H_H, D_H, D_H, HYBRID_CU, inputs.GATE_SOFTPLUS, max(args.steps // 2, 5),
                               min(args.warmup, 3), device, 1013,
                               "chunk_kda fwd+bwd, packed 1024/2048/1024/4096 (T8192), H16, K=V=128, bf16, "
                               "softplus gate and beta sigmoid in kernel, dA_log and d(dt_bias) produced")
        if name == "narrow":
            _log("timing chunk path, narrow-key geometry (K32, V64)")
            return run_variant(16, 2048, 8, 32, 64, None, inputs.GATE_SOFTPLUS, max(args.steps // 2, 5),
                               min(args.warmup, 3), device, 1015,
                               "chunk_kda fwd+bwd, dense B16 x T2048, H8, K=32, V=64 (the 300M model's "
                               "heads), bf16, softplus gate and beta sigmoid in kernel")
        if name == "decode":
            _log("timing decode")
            return run_decode(max(args.steps, 10), args.warmup, device)
        if name == "prefill":
            _log("timing stateful prefill")
            return run_prefill(max(args.steps // 2, 5), min(args.warmup, 3), device)
        if name == "ceiling":
            _log("timing the streaming copy and read (HBM ceiling)")
            return hbm_ceiling(device)
        raise ValueError(name)
    finally:
        torch.cuda.empty_cache()


def _lib_stages():
    from kimi_delta_attention_amd import _lib
    return _lib.load().kda_chunk_bwd_stages()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip the dense B8 x T4096 training shape")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the in-kernel gate and narrow-key (K32/V64) fwd+bwd legs")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--only", choices=["chunk", "train", "gated", "narrow", "decode", "prefill", "ceiling"],
                    help="run one leg alone and print its object (profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA operator needs no cross-GPU exchange and this build "
              "has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    from kimi_delta_attention_amd import _lib
    _lib.load()
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib, device)

    if args.only and args.only != "chunk":
        print(json.dumps({"leg": args.only, **run_leg(args.only, args, device)}), flush=True)
        return

    n_bwd = _lib_stages()
    _log("building inputs")
    host0, d0 = make_hybrid(1003, device)
    _, d1 = make_hybrid(2003, device)
    ops = [chunk_op(d0, True), chunk_op(d1, True)]
    _log("timing chunk path (packed T8192)")
    sec, per_stage, step_ms = time_chunk(ops, args.steps, args.warmup, True, n_bwd)
    del ops
    torch.cuda.empty_cache()
    _log("timing chunk path (packed T8192), backward recomputing the forward's operands")
    ops = [chunk_op(d0, True, keep=False), chunk_op(d1, True, keep=False)]
    sec_r, per_stage_r, _ = time_chunk(ops, args.steps, args.warmup, True, n_bwd, keep=False)
    tokens = T_H
    n_seq = len(HYBRID_CU) - 1
    # the inference forward (nothing saved) is the recomputing run's forward
    fwd_ms = per_stage_r["fwd.prep"] + per_stage_r["fwd.state"]
    slots = sum((HYBRID_CU[i + 1] - HYBRID_CU[i] + C - 1) // C for i in range(n_seq)) * H_H
    work = stage_work(slots, n_seq, H_H, D_H, D_H, 2)
    th = tokens * H_H
    # headline: the whole fwd+bwd step against its operator-level bytes (final
    # state written by the forward, d(initial state) by the backward)
    state_bytes = n_seq * H_H * D_H * D_H * 4
    roof = path_roofline(per_stage, step_ms, th, D_H, D_H, 2, state_bytes, work)
    # the slowest stage against the bytes this design moves through the workspace
    dom = max(per_stage, key=per_stage.get)
    slowest = stage_roofline(dom, work[dom], per_stage[dom])
    slowest["traffic"] = stored_traffic(dom)
    slowest["mfma_util"] = stored_mfma_util(dom)
    pb, pf = PATH_FWDBWD
    fb, ff = PATH_FWD
    roof["inference_fwd_mfma_frac"] = ff * th / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    line = {
        "metric": "chunk_kda fwd+bwd tokens/s (H16,D128,T8192) + decode seq/s; % MFMA/HBM peak",
        "value": tokens / sec,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "chunk_kda fwd+bwd, packed 1024/2048/1024/4096 (T8192), H16, K=V=128, "
                               "bf16 q/k/v, fp32 g/beta/state, l2norm in kernel, log-decay gate, "
                               "forward saves for backward",
                   "global_batch": n_seq, "seq_len": tokens, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "stages_ms": per_stage,
        "slowest_stage_design_bytes": slowest,
        "path_roofline": {"fwd+bwd_hbm_frac": pb * th / (step_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "fwd+bwd_mfma_frac": pf * th / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                          "inference_fwd_tokens_per_s": tokens / (fwd_ms * 1e-3),
                          "inference_fwd_hbm_frac": fb * th / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "inference_fwd_mfma_frac": ff * th / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS},
        "recompute": {"tokens_per_s": tokens / sec_r, "ms_per_step": sec_r * 1e3, "stages_ms": per_stage_r},
    }
    del ops, d0, d1
    torch.cuda.empty_cache()
    if args.only == "chunk":
        print(json.dumps({"leg": "chunk", **line}), flush=True)
        return
    if not args.no_train:
        line["train"] = run_leg("train", args, device)
    if not args.no_variants:
        line["gated"] = run_leg("gated", args, device)
        line["narrow_key"] = run_leg("narrow", args, device)
    if not args.no_decode:
        line["decode"] = run_leg("decode", args, device)
        line["roofline"]["decode_hbm_frac"] = line["decode"]["roofline"]["frac"]
        line["prefill"] = run_leg("prefill", args, device)
        ceil = run_leg("ceiling", args, device)
        line["hbm_ceiling"] = ceil
        for leg, key in ((line["decode"], "roofline"), (line["prefill"], "conv_roofline"),
                         (line["prefill"], "gate_roofline"), (line["prefill"], "gate_bwd_roofline")):
            leg[key]["frac_of_stream_copy"] = leg[key]["achieved"] / ceil["copy_GBs"]
    if not args.no_cpu_baseline:
        _log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(host0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
