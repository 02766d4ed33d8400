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
def chunk_fwd_bytes(tokens, H, K, V, elt, n_seq):
    """q, k, v and o in the input dtype, g fp32, beta fp32, final state fp32."""
    return tokens * H * (2 * K * elt + V * elt + K * 4 + 4 + V * elt) + n_seq * H * K * V * 4


def chunk_bwd_bytes(tokens, H, K, V, elt, n_seq):
    """Reads q, k, v, g, beta, dO; writes dq, dk, dv, dg, dbeta and d(initial state)."""
    reads = tokens * H * (2 * K * elt + V * elt + K * 4 + 4 + V * elt)
    writes = tokens * H * (2 * K * elt + V * elt + K * 4 + 4) + n_seq * H * K * V * 4
    return reads + writes


def decode_bytes(N, H, D, W, x_elt):
    """State and conv state read + written once; x, g, beta, conv_w read; o written."""
    return (2 * N * H * D * D * 4 + 2 * N * 3 * H * D * W * 4 + N * 3 * H * D * x_elt + N * H * D * 4
            + N * H * 4 + 3 * H * D * W * 4 + N * H * D * 4)


# Flops per token-head of the chunk form at C = 64 (triangular products at
# their triangular size): the three 2*d^2 state products and the intra-chunk
# part (A, M, the two products with T and the solve).
def chunk_flops_per_token_head(d, C=64):
    state = 3 * 2 * d * d
    tri = (C + 1) / 2
    intra = 2 * tri * d * 2 + 2 * tri * d * 2 + C * C / 3
    return state, intra


# ---------------------------------------------------------------- workloads
def make_hybrid(seed, device):
    from kimi_delta_attention_amd import inputs
    w = inputs.chunk_inputs(1, T_H, H_H, D_H, D_H, seed=seed, dtype=torch.bfloat16, cu_seqlens=HYBRID_CU,
                            with_grad_out=True)
    return w, {k: (v.to(device) if hasattr(v, "to") else v) for k, v in w.items()}


def chunk_op(d, with_bwd):
    import kimi_delta_attention_amd as kda
    return kda.ChunkOp(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"], initial_state=None,
                       output_final_state=True, use_qk_l2norm_in_kernel=True, gate_mode=d["gate_mode"],
                       use_beta_sigmoid_in_kernel=d["use_beta_sigmoid"], lower_bound=d["lower_bound"],
                       cu_seqlens=d["cu_seqlens"], dO=d["dO"] if with_bwd else None)


def _bwd_probe():
    # The backward entry point exists in every build; a build without the
    # backward kernels reports it through its stage count.
    from kimi_delta_attention_amd import _lib
    lib = _lib.load()
    return hasattr(lib, "kda_chunk_bwd_stage")


def time_chunk(ops, steps, warmup, with_bwd, n_bwd_stages):
    stream = torch.cuda.current_stream()
    names = ["fwd.prep", "fwd.state"] + ([f"bwd.{i}" for i in range(n_bwd_stages)] if with_bwd else [])

    def one(op, evs):
        k = 0
        for st in range(2):
            evs[k].record(stream)
            op.forward(stage=st)
            k += 1
        if with_bwd:
            for st in range(n_bwd_stages):
                evs[k].record(stream)
                op.backward(stage=st)
                k += 1
        evs[k].record(stream)

    for i in range(warmup):
        one(ops[i % len(ops)], [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)])
    torch.cuda.synchronize()
    all_evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(ops[i % len(ops)], all_evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = {n: [] for n in names}
    for evs in all_evs:
        for j, n in enumerate(names):
            per[n].append(evs[j].elapsed_time(evs[j + 1]))
    return (t1 - t0) / steps, {n: sum(v) / len(v) for n, v in per.items()}


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
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for t in range(steps):
        s = ins[(warmup + t) % n_in]
        evs[t].record(stream)
        kda.recurrent_step(s["x"], cw, cs, s["g"], s["beta"], st, out=o)
    evs[steps].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = sum(evs[t].elapsed_time(evs[t + 1]) for t in range(steps)) / steps
    wall = (t1 - t0) / steps
    algo = decode_bytes(N, H, D, W, 2)
    return {
        "metric": "decode sequence-steps/s", "unit": "seq/s", "value": N / wall,
        "ms_per_step": wall * 1e3, "workload": f"decode N{N} H{H} d{D} conv{W} bf16 x, fp32 state",
        "roofline": {"bound": "hbm", "kernel": "decode_step_kernel", "achieved": algo / (kern_ms * 1e-3) / 1e9,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": algo / (kern_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": None,
                     "algorithmic_bytes": algo, "kernel_ms": kern_ms},
    }


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


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the KDA operator needs no cross-GPU exchange and this build "
              "has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    device = torch.device("cuda", 0)
    torch.cuda.set_device(device)
    from kimi_delta_attention_amd import _lib
    _lib.load()

    with_bwd = _bwd_probe()
    n_bwd = 0
    if with_bwd:
        n_bwd = _lib.load().kda_chunk_bwd_stages()
    _log(f"building inputs (bwd={'yes' if with_bwd else 'no'})")
    host0, d0 = make_hybrid(1003, device)
    _, d1 = make_hybrid(2003, device)
    ops = [chunk_op(d0, with_bwd), chunk_op(d1, with_bwd)]
    _log("timing chunk path")
    sec, per_stage = time_chunk(ops, args.steps, args.warmup, with_bwd, n_bwd)
    tokens = T_H
    n_seq = len(HYBRID_CU) - 1
    fwd_ms = per_stage["fwd.prep"] + per_stage["fwd.state"]

    # dominant kernel: the stage with the largest mean duration
    dom = max(per_stage, key=per_stage.get)
    st_f, in_f = chunk_flops_per_token_head(D_H)
    th = tokens * H_H
    flops_of = {"fwd.prep": in_f * th, "fwd.state": st_f * th}
    roof = None
    if dom in flops_of:
        ach = flops_of[dom] / (per_stage[dom] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": ach / PEAK_BF16_TFLOPS, "traffic": None, "algorithmic_flops": flops_of[dom],
                "kernel_ms": per_stage[dom]}
    fb = chunk_fwd_bytes(tokens, H_H, D_H, D_H, 2, n_seq)
    line = {
        "metric": "chunk_kda fwd+bwd tokens/s (H16,D128,T8192) + decode seq/s; % MFMA/HBM peak",
        "value": tokens / sec if with_bwd else None,
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": sec * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "chunk_kda fwd+bwd, packed 1024/2048/1024/4096 (T8192), H16, K=V=128, "
                               "bf16 q/k/v, fp32 g/beta/state, l2norm in kernel, log-decay gate",
                   "global_batch": n_seq, "seq_len": tokens, "parallelism": "none (1 GPU)"},
        "stages_ms": per_stage,
        "fwd_tokens_per_s": tokens / (fwd_ms * 1e-3),
        "fwd_hbm_frac": fb / (fwd_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "roofline": roof,
    }
    del ops, d0, d1
    torch.cuda.empty_cache()
    if not args.no_decode:
        _log("timing decode")
        line["decode"] = run_decode(max(args.steps, 10), args.warmup, device)
    if not args.no_cpu_baseline:
        _log("cpu baseline (oracle)")
        line["cpu_baseline"] = cpu_baseline(host0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
