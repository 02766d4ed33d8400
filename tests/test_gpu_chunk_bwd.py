"""GPU parity of kda_chunk_bwd against the oracle's hand-derived backward
(itself pinned by central finite differences in test_oracle.py)."""
import numpy as np
import pytest
import torch

import oracle
import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import inputs
from parity import check, dev, tol_for, nan_full

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]


def _gpu_bwd(w, **over):
    kw = dict(A_log=dev(w["A_log"]), dt_bias=dev(w["dt_bias"]), scale=w["scale"],
              initial_state=dev(w["initial_state"]), use_qk_l2norm_in_kernel=w["use_qk_l2norm"],
              gate_mode=w["gate_mode"], use_beta_sigmoid_in_kernel=w["use_beta_sigmoid"],
              lower_bound=w["lower_bound"], cu_seqlens=dev(w["cu_seqlens"]),
              d_final_state=dev(w.get("d_final_state")))
    kw.update(over)
    # gradients start as NaN, so that an element the kernels do not write fails the check
    B, T, H, K = w["q"].shape
    V = w["v"].shape[-1]
    N = B if w["cu_seqlens"] is None else len(w["cu_seqlens"]) - 1
    dt = w["q"].dtype
    pre = {"dq": nan_full((B, T, H, K), dt), "dk": nan_full((B, T, H, K), dt), "dv": nan_full((B, T, H, V), dt),
           "dg": nan_full((B, T, H, K), torch.float32), "dbeta": nan_full((B, T, H), torch.float32),
           "dh0": nan_full((N, H, K, V), torch.float32)}
    if w["gate_mode"] != inputs.GATE_LOGDECAY:
        pre["dA_log"] = nan_full((H,), torch.float32)
        pre["ddt_bias"] = nan_full((H * K,), torch.float32)
    kw.setdefault("out", pre)
    out = kda.chunk_kda_bwd(dev(w["q"]), dev(w["k"]), dev(w["v"]), dev(w["g"]), dev(w["beta"]), dev(w["dO"]), **kw)
    torch.cuda.synchronize()
    return out


def _oracle_bwd(w):
    return oracle.chunk_bwd(w["q"], w["k"], w["v"], w["g"], w["beta"], w["dO"], d_final_state=w.get("d_final_state"),
                            A_log=w["A_log"], dt_bias=w["dt_bias"], scale=w["scale"], initial_state=w["initial_state"],
                            use_qk_l2norm=w["use_qk_l2norm"], gate_mode=w["gate_mode"],
                            use_beta_sigmoid=w["use_beta_sigmoid"], lower_bound=w["lower_bound"],
                            cu_seqlens=w["cu_seqlens"])


def _compare(w, tag, names=NAMES):
    tol = tol_for(w["q"].dtype)
    print(f"{tag}: q{tuple(w['q'].shape)} {w['q'].dtype} gate={w['gate_mode']}", flush=True)
    g = _gpu_bwd(w)
    o = _oracle_bwd(w)
    for name in names:
        check(f"{tag} {name}", g[name], o[name], tol)
    if w["gate_mode"] != inputs.GATE_LOGDECAY:
        check(f"{tag} dA_log", g["dA_log"], o["dA_log"], tol)
        check(f"{tag} ddt_bias", g["ddt_bias"], o["ddt_bias"], tol)


@pytest.mark.parametrize("T", [1, 7, 63, 64, 65, 130])
@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 32, 32), (torch.float32, 64, 64), (torch.bfloat16, 32, 32),
                                       (torch.bfloat16, 64, 64), (torch.bfloat16, 128, 128),
                                       (torch.float32, 32, 64), (torch.bfloat16, 32, 64)])
def test_bwd_boundary_lengths(T, dtype, K, V):
    w = inputs.chunk_inputs(2, T, 2, K, V, seed=300 + T + K + V, dtype=dtype, h0_std=0.1, with_grad_out=True,
                            dfinal_std=0.1)
    _compare(w, f"T={T} K={K} V={V}")


@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 32, 32), (torch.float32, 64, 64), (torch.bfloat16, 64, 64),
                                       (torch.bfloat16, 128, 128), (torch.float32, 32, 64),
                                       (torch.bfloat16, 32, 64)])
def test_bwd_weak_decay(dtype, K, V):
    """Log-decay drawn in [-0.02, 0] per step (a chunk decays the state by about
    e^-0.6), with a final-state cotangent: the state gradient carries back
    through every chunk boundary, and the gate gradient's state-decay term
    (per key, the sum over the value columns of the entry state times the
    exit state's gradient, scaled by the chunk's total decay) is of the order
    of the rest of dg.  With the default [-5, 0] draw that term is scaled by
    about e^-160 in every whole chunk."""
    w = inputs.chunk_inputs(2, 320, 3, K, V, seed=600 + K + V, dtype=dtype, lower_bound=-0.02, h0_std=0.1,
                            with_grad_out=True, dfinal_std=0.1)
    _compare(w, f"weak decay K={K} V={V}")


@pytest.mark.parametrize("mode", [inputs.GATE_SAFE, inputs.GATE_SOFTPLUS])
@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 32, 32), (torch.bfloat16, 128, 128), (torch.bfloat16, 32, 64)])
def test_bwd_in_kernel_gates(mode, dtype, K, V):
    w = inputs.chunk_inputs(2, 150, 2, K, V, seed=17 + mode, dtype=dtype, gate_mode=mode, beta_logits=True,
                            h0_std=0.1, with_grad_out=True, dfinal_std=0.1)
    _compare(w, f"gate {mode}")


def test_bwd_small_fp32_workload():
    """B1 T128 H2 K=V=32 fp32 with an upstream dO and final-state cotangent."""
    w = inputs.chunk_inputs(1, 128, 2, 32, 32, seed=inputs.SEEDS["fwd_small"], with_grad_out=True, dfinal_std=0.1)
    _compare(w, "small")


def test_bwd_twin_fp32_unbounded_gate():
    """B4 T2048 H8 K=V=32 fp32, unbounded in-kernel gate, beta logits."""
    w = inputs.chunk_inputs(4, 2048, 8, 32, 32, seed=inputs.SEEDS["fwd_twin"], gate_mode=inputs.GATE_SOFTPLUS,
                            beta_logits=True, h0_std=0.1, with_grad_out=True, dfinal_std=0.1)
    _compare(w, "twin")


def test_bwd_varlen_empty_and_tiny():
    cu = [0, 0, 1, 66, 66, 130, 200]
    w = inputs.chunk_inputs(1, 200, 2, 64, 64, seed=23, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.2,
                            with_grad_out=True, dfinal_std=0.1)
    _compare(w, "varlen")


def test_bwd_train_geometry_whole_batch():
    """B8 T4096 H16 K=V=128 bf16 with dO ~ N(0,1), in the launch configuration
    the bench times: every gradient of all 128 (sequence, head) units against
    the oracle."""
    w = inputs.workload("train")
    print("train geometry: whole batch", flush=True)
    g = _gpu_bwd(w)
    o = _oracle_bwd(w)
    for name in NAMES:
        check(f"train {name}", g[name], o[name], 2e-2)


def test_bwd_narrow_key_geometry_whole_batch():
    """The narrow-key head geometry of the Primus 300M configuration (8 heads,
    key dim 32, value dim 64, T2048, its unbounded softplus gate in kernel and
    beta logits), bf16, 16 sequences of its micro-batch: every element of the
    forward and the backward (dA_log and d(dt_bias) included) against the
    oracle."""
    w = inputs.chunk_inputs(16, 2048, 8, 32, 64, seed=75, dtype=torch.bfloat16, gate_mode=inputs.GATE_SOFTPLUS,
                            beta_logits=True, with_grad_out=True)
    print("narrow-key geometry B16 T2048 H8 K32 V64: whole batch", flush=True)
    _compare(w, "narrow")
    kw = dict(A_log=dev(w["A_log"]), dt_bias=dev(w["dt_bias"]), scale=w["scale"],
              use_qk_l2norm_in_kernel=True, gate_mode=w["gate_mode"], use_beta_sigmoid_in_kernel=True)
    o_gpu, _ = kda.chunk_kda(dev(w["q"]), dev(w["k"]), dev(w["v"]), dev(w["g"]), dev(w["beta"]), **kw)
    torch.cuda.synchronize()
    of, _ = oracle.chunk_fwd(w["q"], w["k"], w["v"], w["g"], w["beta"], A_log=w["A_log"], dt_bias=w["dt_bias"],
                             scale=w["scale"], use_qk_l2norm=True, gate_mode=w["gate_mode"], use_beta_sigmoid=True)
    check("narrow o", o_gpu, of, 2e-2)


def test_bwd_hybrid_varlen_whole_batch():
    """Packed 1024/2048/1024/4096, H16 K=V=128 bf16, dO ~ N(0,1): every head."""
    w = inputs.chunk_inputs(1, 8192, 16, 128, 128, seed=inputs.SEEDS["fwd_hybrid"], dtype=torch.bfloat16,
                            cu_seqlens=[0, 1024, 3072, 4096, 8192], with_grad_out=True)
    print("hybrid backward: whole batch", flush=True)
    _compare(w, "hybrid")


def test_bwd_deterministic():
    w = inputs.chunk_inputs(2, 200, 2, 128, 128, seed=9, dtype=torch.bfloat16, with_grad_out=True)
    a = _gpu_bwd(w)
    b = _gpu_bwd(w)
    for name in NAMES:
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("case", ["bf16_128_varlen_tail", "f32_32_softplus_h0", "bf16_64_safe_dfinal",
                                  "bf16_32x64_softplus_varlen"])
def test_bwd_reuses_saved_forward(case):
    """A forward with keep_for_backward writes what the backward's first two
    stages compute; the backward with the flag skips them.  Same kernels, same
    inputs: o, the final state and every gradient are bit-identical to the
    recomputing path, which the other tests check against the oracle."""
    if case == "bf16_128_varlen_tail":
        w = inputs.chunk_inputs(1, 300, 2, 128, 128, seed=71, dtype=torch.bfloat16, cu_seqlens=[0, 100, 300],
                                with_grad_out=True, h0_std=0.1)
    elif case == "f32_32_softplus_h0":
        w = inputs.chunk_inputs(2, 130, 2, 32, 32, seed=72, gate_mode=inputs.GATE_SOFTPLUS, beta_logits=True,
                                h0_std=0.1, with_grad_out=True, dfinal_std=0.1)
    elif case == "bf16_64_safe_dfinal":
        w = inputs.chunk_inputs(2, 97, 2, 64, 64, seed=73, dtype=torch.bfloat16, gate_mode=inputs.GATE_SAFE,
                                with_grad_out=True, dfinal_std=0.1)
    else:
        w = inputs.chunk_inputs(1, 260, 2, 32, 64, seed=74, dtype=torch.bfloat16, gate_mode=inputs.GATE_SOFTPLUS,
                                beta_logits=True, cu_seqlens=[0, 0, 130, 260], with_grad_out=True, h0_std=0.1,
                                dfinal_std=0.1)
    print(f"saved-forward {case}", flush=True)
    kw = dict(A_log=dev(w["A_log"]), dt_bias=dev(w["dt_bias"]), scale=w["scale"],
              initial_state=dev(w["initial_state"]), use_qk_l2norm_in_kernel=True, gate_mode=w["gate_mode"],
              use_beta_sigmoid_in_kernel=w["use_beta_sigmoid"], lower_bound=w["lower_bound"],
              cu_seqlens=dev(w["cu_seqlens"]))
    q, k, v, g, beta, dO = (dev(w[n]) for n in ("q", "k", "v", "g", "beta", "dO"))
    nb = kda.chunk_bwd_workspace_bytes(q, k, v, g, beta, **kw)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    o0, s0 = kda.chunk_kda(q, k, v, g, beta, output_final_state=True, **kw)
    ref = kda.chunk_kda_bwd(q, k, v, g, beta, dO, d_final_state=dev(w["d_final_state"]), **kw)
    o1, s1 = kda.chunk_kda(q, k, v, g, beta, output_final_state=True, workspace=ws, keep_for_backward=True, **kw)
    got = kda.chunk_kda_bwd(q, k, v, g, beta, dO, d_final_state=dev(w["d_final_state"]), workspace=ws,
                            keep_for_backward=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(s0, s1)
    for name in NAMES + (["dA_log", "ddt_bias"] if w["gate_mode"] != inputs.GATE_LOGDECAY else []):
        assert torch.equal(ref[name], got[name]), name
    if case == "bf16_128_varlen_tail":
        o = _oracle_bwd(w)
        for name in NAMES:
            check(f"saved {name}", got[name], o[name], tol_for(w["q"].dtype))


@pytest.mark.parametrize("case", ["packed_h4", "dense_b17_h4"])
def test_bwd_many_chains_64_column_state_blocks(case):
    """K = V = 128 bf16 with 80 and 68 (sequence, head) chains, where the state
    passes run 64-column blocks: every gradient against the oracle, both from
    the recomputing backward and from a forward that saved for it (bit-identical)."""
    from test_gpu_chunk_fwd import many_chain_cu
    if case == "packed_h4":
        cu = many_chain_cu()
        w = inputs.chunk_inputs(1, cu[-1], 4, 128, 128, seed=83, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.1,
                                with_grad_out=True, dfinal_std=0.1)
    else:
        w = inputs.chunk_inputs(17, 150, 4, 128, 128, seed=84, dtype=torch.bfloat16, h0_std=0.1,
                                with_grad_out=True, dfinal_std=0.1)
    _compare(w, case)
    kw = dict(scale=w["scale"], initial_state=dev(w["initial_state"]), use_qk_l2norm_in_kernel=True,
              gate_mode=w["gate_mode"], lower_bound=w["lower_bound"], cu_seqlens=dev(w["cu_seqlens"]))
    q, k, v, g, beta, dO = (dev(w[n]) for n in ("q", "k", "v", "g", "beta", "dO"))
    ws = torch.empty(kda.chunk_bwd_workspace_bytes(q, k, v, g, beta, **kw), dtype=torch.uint8, device="cuda")
    ref = kda.chunk_kda_bwd(q, k, v, g, beta, dO, d_final_state=dev(w["d_final_state"]), **kw)
    kda.chunk_kda(q, k, v, g, beta, output_final_state=True, workspace=ws, keep_for_backward=True, **kw)
    got = kda.chunk_kda_bwd(q, k, v, g, beta, dO, d_final_state=dev(w["d_final_state"]), workspace=ws,
                            keep_for_backward=True, **kw)
    torch.cuda.synchronize()
    for name in NAMES:
        assert torch.equal(ref[name], got[name]), name


def test_bwd_many_short_sequences():
    """1,500 packed sequences of 0..70 tokens (more than the 1,024 the plan
    kernel's scan takes per round, empty ones among them), H2 K=V=32 bf16:
    the plan's chunk offsets and slot map, forward and backward, against the
    oracle."""
    gen = torch.Generator().manual_seed(61)
    lens = torch.randint(0, 71, (1500,), generator=gen)
    lens[::97] = 0
    cu = [0] + torch.cumsum(lens, 0).tolist()
    w = inputs.chunk_inputs(1, cu[-1], 2, 32, 32, seed=62, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.1,
                            with_grad_out=True, dfinal_std=0.1)
    print(f"many short: N={len(cu) - 1} T={cu[-1]}", flush=True)
    _compare(w, "many-short")
