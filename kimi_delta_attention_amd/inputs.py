"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no part of the method's arithmetic: it only draws random
tensors with a CPU ``torch.Generator`` in a fixed order and rounds them to the
storage dtype (round-to-nearest-even for bfloat16).  The same host tensors are
given to the CPU oracle and uploaded to the GPU.

Workload recipes (shapes and distributions of the pages' workloads; the
second argument of N(0, s) is the standard deviation):

* ``fwd_small``   B1 T128 H2 K=V=32, fp32, log-decay g = -5*sigmoid(N(0,1)),
                  beta = sigmoid(N(0,1)), zero initial state.
* ``fwd_twin``    B4 T2048 H8 K=V=32, fp32, unbounded in-kernel gate from
                  x ~ N(0,1), dt_bias ~ N(0,0.1), A_log ~ U(0, ln 16); beta
                  logits N(0,1); initial state N(0,0.1).
* ``fwd_hybrid``  packed sequences 1024/2048/1024/4096 (T=8192), H16 K=V=128,
                  bf16 q/k/v, fp32 g and beta, zero initial state.
* ``train``       B8 T4096 H16 K=V=128, bf16, plus dO ~ N(0,1) in bf16.
* ``decode``      64 sequences, H96, D128, conv kernel 4; per step
                  x ~ N(0,1) bf16 [64, 3*96*128], g = -5*sigmoid(N(0,1)),
                  beta logits N(0,1); once: conv_w ~ N(0,0.5),
                  S0 ~ N(0,0.05), conv state ~ N(0,0.05).
"""
from __future__ import annotations

import math

import torch

GATE_LOGDECAY, GATE_SAFE, GATE_SOFTPLUS = 0, 1, 2

SEEDS = {"fwd_small": 1001, "fwd_twin": 1002, "fwd_hybrid": 1003, "train": 1004, "decode": 1005}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _n(gen, shape, std=1.0):
    return torch.randn(*shape, generator=gen, dtype=torch.float32) * std


def chunk_inputs(B, T, H, K, V, *, seed, dtype=torch.float32, gate_mode=GATE_LOGDECAY,
                 lower_bound=-5.0, beta_logits=False, h0_std=0.0, cu_seqlens=None,
                 with_grad_out=False, dfinal_std=0.0):
    """Random chunk-path inputs.

    Draw order: q, k, v, then the gate input, then beta, then (if the gate is
    computed in kernel) dt_bias and A_log, then the initial state, then dO and
    the final-state cotangent.  Returns a dict of CPU tensors and flags."""
    gen = _gen(seed)
    q = _n(gen, (B, T, H, K)).to(dtype)
    k = _n(gen, (B, T, H, K)).to(dtype)
    v = _n(gen, (B, T, H, V)).to(dtype)
    x = _n(gen, (B, T, H, K))
    if gate_mode == GATE_LOGDECAY:
        g = lower_bound * torch.sigmoid(x)  # a log-decay drawn in [lower_bound, 0]
    else:
        g = x  # raw gate input; the kernel applies the gate
    b = _n(gen, (B, T, H))
    beta = b if beta_logits else torch.sigmoid(b)
    A_log = dt_bias = None
    if gate_mode != GATE_LOGDECAY:
        dt_bias = _n(gen, (H * K,), 0.1)
        A_log = torch.rand(H, generator=gen, dtype=torch.float32) * math.log(16.0)
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    h0 = _n(gen, (N, H, K, V), h0_std) if h0_std > 0 else torch.zeros(N, H, K, V)
    out = dict(q=q, k=k, v=v, g=g.contiguous(), beta=beta.contiguous(), A_log=A_log,
               dt_bias=dt_bias, initial_state=h0,
               cu_seqlens=None if cu_seqlens is None else torch.tensor(cu_seqlens, dtype=torch.int32),
               gate_mode=gate_mode, use_qk_l2norm=True, use_beta_sigmoid=beta_logits,
               lower_bound=lower_bound if gate_mode != GATE_SOFTPLUS else None,
               scale=K ** -0.5)
    if with_grad_out:
        out["dO"] = _n(gen, (B, T, H, V)).to(dtype)
        out["d_final_state"] = _n(gen, (N, H, K, V), dfinal_std) if dfinal_std > 0 else None
    return out


def workload(name: str, **over):
    """The named workload's inputs (see the module docstring)."""
    s = SEEDS[name]
    if name == "fwd_small":
        return chunk_inputs(1, 128, 2, 32, 32, seed=s, **over)
    if name == "fwd_twin":
        return chunk_inputs(4, 2048, 8, 32, 32, seed=s, gate_mode=GATE_SOFTPLUS,
                            beta_logits=True, h0_std=0.1, **over)
    if name == "fwd_hybrid":
        return chunk_inputs(1, 8192, 16, 128, 128, seed=s, dtype=torch.bfloat16,
                            cu_seqlens=[0, 1024, 3072, 4096, 8192], **over)
    if name == "train":
        return chunk_inputs(8, 4096, 16, 128, 128, seed=s, dtype=torch.bfloat16,
                            with_grad_out=True, **over)
    raise KeyError(name)


DECODE_SHAPE = dict(N=64, H=96, D=128, W=4)


def decode_init(N, H, D, W, *, seed, state_std=0.05, conv_std=0.05, w_std=0.5):
    """Decode-path parameters and initial states: conv_w [3HD, W], conv state
    [N, 3HD, W] and recurrent state [N, H, D, D], all fp32."""
    gen = _gen(seed)
    CH = 3 * H * D
    conv_w = _n(gen, (CH, W), w_std)
    state = _n(gen, (N, H, D, D), state_std)
    conv_state = _n(gen, (N, CH, W), conv_std)
    return dict(conv_w=conv_w, state=state, conv_state=conv_state)


def prefill_inputs(rows, H, D, *, seed, dtype=torch.bfloat16, lower_bound=-5.0):
    """Prompt inputs of a stateful prefill, drawn like the decode steps: x
    [rows, 3HD] (pre-conv q|k|v), log-decay g [rows, HD], beta logits [rows, H]."""
    gen = _gen(seed)
    x = _n(gen, (rows, 3 * H * D)).to(dtype)
    g = lower_bound * torch.sigmoid(_n(gen, (rows, H * D)))
    beta = _n(gen, (rows, H))
    return dict(x=x, g=g.contiguous(), beta=beta)


def gate_inputs(rows, H, V, *, seed, dtype=torch.bfloat16, g_dtype=None):
    """Output-gate inputs: the attention output o, the gate input g and an
    upstream gradient dy, each [rows, H, V] ~ N(0, 1) (g in g_dtype, default dtype)."""
    gen = _gen(seed)
    o = _n(gen, (rows, H, V)).to(dtype)
    g = _n(gen, (rows, H, V)).to(g_dtype or dtype)
    dy = _n(gen, (rows, H, V)).to(dtype)
    return dict(o=o, g=g, dy=dy)


def decode_step_inputs(N, H, D, *, seed, step, dtype=torch.bfloat16, lower_bound=-5.0):
    """Per-step decode inputs: x [N, 3HD] (pre-conv q|k|v), log-decay g
    [N, HD] and beta logits [N, H].  Each step has its own generator seed."""
    gen = _gen(int(seed) * 1_000_003 + int(step) + 1)
    x = _n(gen, (N, 3 * H * D)).to(dtype)
    g = lower_bound * torch.sigmoid(_n(gen, (N, H * D)))
    beta = _n(gen, (N, H))
    return dict(x=x, g=g.contiguous(), beta=beta)
