"""GPU parity of kda_chunk_fwd against the CPU oracle (the token recurrence)."""
import numpy as np
import pytest
import torch

import oracle
import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import inputs
from parity import check, dev, tol_for, nan_full

pytestmark = pytest.mark.gpu


def _run_gpu(w, output_final_state=True, **over):
    kw = dict(A_log=dev(w["A_log"]), dt_bias=dev(w["dt_bias"]), scale=w["scale"],
              initial_state=dev(w["initial_state"]), output_final_state=output_final_state,
              use_qk_l2norm_in_kernel=w["use_qk_l2norm"], gate_mode=w["gate_mode"],
              use_beta_sigmoid_in_kernel=w["use_beta_sigmoid"], lower_bound=w["lower_bound"],
              cu_seqlens=dev(w["cu_seqlens"]))
    kw.update(over)
    # outputs start as NaN, so that an element the kernels do not write fails the check
    B, T, H, K = w["q"].shape
    V = w["v"].shape[-1]
    N = B if w["cu_seqlens"] is None else len(w["cu_seqlens"]) - 1
    kw.setdefault("out", nan_full((B, T, H, V), w["q"].dtype))
    if kw["output_final_state"]:
        kw.setdefault("final_state_out", nan_full((N, H, K, V), torch.float32))
    o, fs = kda.chunk_kda(dev(w["q"]), dev(w["k"]), dev(w["v"]), dev(w["g"]), dev(w["beta"]), **kw)
    torch.cuda.synchronize()
    return o, fs


def _run_oracle(w, **over):
    kw = dict(A_log=w["A_log"], dt_bias=w["dt_bias"], scale=w["scale"], initial_state=w["initial_state"],
              use_qk_l2norm=w["use_qk_l2norm"], gate_mode=w["gate_mode"],
              use_beta_sigmoid=w["use_beta_sigmoid"], lower_bound=w["lower_bound"],
              cu_seqlens=w["cu_seqlens"])
    kw.update(over)
    return oracle.chunk_fwd(w["q"], w["k"], w["v"], w["g"], w["beta"], **kw)


def _compare(w, tag):
    tol = tol_for(w["q"].dtype)
    print(f"{tag}: q{tuple(w['q'].shape)} {w['q'].dtype} gate={w['gate_mode']}", flush=True)
    o, fs = _run_gpu(w)
    oo, ofs = _run_oracle(w)
    check(f"{tag} o", o, oo, tol)
    check(f"{tag} final_state", fs, ofs, tol)


def test_fwd_small_fp32():
    """B1 T128 H2 K=V=32 fp32, log-decay -5*sigmoid(N), zero initial state."""
    _compare(inputs.workload("fwd_small"), "fwd_small")


def test_fwd_twin_fp32_unbounded_gate():
    """B4 T2048 H8 K=V=32 fp32 with the unbounded softplus gate in kernel (per-step
    decays reach about -54, so the pairwise diagonal path is exercised)."""
    _compare(inputs.workload("fwd_twin"), "fwd_twin")


def test_fwd_hybrid_bf16_varlen_whole_batch():
    """Packed 1024/2048/1024/4096, H16 K=V=128 bf16, in the launch configuration
    the bench times: every head of every sequence against the oracle."""
    w = inputs.workload("fwd_hybrid")
    print("fwd_hybrid: whole batch", flush=True)
    o, fs = _run_gpu(w)
    oo, ofs = _run_oracle(w)
    check("hybrid o", o, oo, 2e-2)
    check("hybrid final_state", fs, ofs, 2e-2)


@pytest.mark.parametrize("T", [1, 7, 63, 64, 65, 130])
@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 32, 32), (torch.float32, 64, 64), (torch.bfloat16, 32, 32),
                                       (torch.bfloat16, 64, 64), (torch.bfloat16, 128, 128),
                                       (torch.float32, 32, 64), (torch.bfloat16, 32, 64)])
def test_fwd_boundary_lengths(T, dtype, K, V):
    """Lengths straddling the 64-token chunk (memra gate 1 lengths), random initial state."""
    w = inputs.chunk_inputs(2, T, 3, K, V, seed=100 + T + K + V, dtype=dtype, h0_std=0.1)
    _compare(w, f"T={T} K={K} V={V}")


@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 32, 32), (torch.float32, 64, 64), (torch.bfloat16, 64, 64),
                                       (torch.bfloat16, 128, 128), (torch.bfloat16, 32, 64)])
def test_fwd_weak_decay(dtype, K, V):
    """Log-decay drawn in [-0.02, 0] per step: a chunk decays the state by about
    e^-0.6, so the state carries through every chunk boundary.  With the
    default [-5, 0] draw a chunk decays it by about e^-160, and only the first
    rows of a chunk see the state it enters with."""
    w = inputs.chunk_inputs(2, 320, 3, K, V, seed=500 + K + V, dtype=dtype, lower_bound=-0.02, h0_std=0.1)
    _compare(w, f"weak decay K={K} V={V}")


@pytest.mark.parametrize("mode", [inputs.GATE_SAFE, inputs.GATE_SOFTPLUS])
@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 32, 32), (torch.bfloat16, 128, 128), (torch.bfloat16, 32, 64)])
def test_fwd_in_kernel_gates(mode, dtype, K, V):
    w = inputs.chunk_inputs(1, 200, 2, K, V, seed=7 + mode, dtype=dtype, gate_mode=mode, beta_logits=True,
                            h0_std=0.1)
    _compare(w, f"gate {mode}")


def test_fwd_varlen_with_empty_and_tiny_sequences():
    cu = [0, 0, 1, 66, 66, 130, 200]
    w = inputs.chunk_inputs(1, 200, 2, 64, 64, seed=21, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.2)
    _compare(w, "varlen")


def test_fwd_more_sequences_than_the_plans_lds_offsets():
    """4,500 packed sequences of 0..12 tokens (above the 4,096 whose chunk
    offsets the plan kernel keeps in LDS for its slot search, so the search
    reads them from the workspace), H1 K=V=32 bf16."""
    gen = torch.Generator().manual_seed(71)
    lens = torch.randint(0, 13, (4500,), generator=gen)
    lens[::101] = 0
    cu = [0] + torch.cumsum(lens, 0).tolist()
    w = inputs.chunk_inputs(1, cu[-1], 1, 32, 32, seed=72, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.1)
    _compare(w, f"N={len(cu) - 1} T={cu[-1]}")


# Lengths of a packed batch with more (sequence, head) chains than four
# 32-column state blocks each can place on the chip at one workgroup per CU,
# so that the K = V = 128 state passes take 64-column blocks: empty, one-row,
# chunk-boundary and ragged sequences.
MANY_CHAIN_LENS = [0, 1, 63, 64, 65, 127, 130, 200, 7, 0, 129, 64, 3, 191, 66, 100, 1, 250, 64, 31]


def many_chain_cu():
    cu = [0]
    for n in MANY_CHAIN_LENS:
        cu.append(cu[-1] + n)
    return cu


@pytest.mark.parametrize("case", ["packed_h4", "dense_b17_h4"])
def test_fwd_many_chains_64_column_state_blocks(case):
    """K = V = 128 bf16 with 80 and 68 (sequence, head) chains: the state pass
    runs 64-column blocks (two per chain).  Ragged and empty packed sequences
    with an initial state; a dense batch with a tail chunk."""
    if case == "packed_h4":
        cu = many_chain_cu()
        w = inputs.chunk_inputs(1, cu[-1], 4, 128, 128, seed=81, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.1)
    else:
        w = inputs.chunk_inputs(17, 150, 4, 128, 128, seed=82, dtype=torch.bfloat16, h0_std=0.1)
    _compare(w, case)


def test_fwd_no_l2norm_and_plain_scale():
    w = inputs.chunk_inputs(1, 96, 2, 32, 32, seed=8)
    # unit-norm keys supplied by the caller, so the chunk form stays well conditioned
    w["q"] = w["q"] / w["q"].norm(dim=-1, keepdim=True)
    w["k"] = w["k"] / w["k"].norm(dim=-1, keepdim=True)
    w["use_qk_l2norm"] = False
    w["scale"] = 0.7
    _compare(w, "no-l2norm")


def test_fwd_split_call_equals_single_call():
    """memra gate 3 analogue on the GPU: two calls with the state carried over
    equal one call, for splits around the chunk boundary."""
    w = inputs.chunk_inputs(1, 130, 2, 128, 128, seed=33, dtype=torch.bfloat16)
    o, fs = _run_gpu(w)
    for split in [1, 2, 3, 63, 64, 65, 127]:
        a = {k: (v[:, :split] if k in ("q", "k", "v", "g", "beta") else v) for k, v in w.items()}
        b = {k: (v[:, split:] if k in ("q", "k", "v", "g", "beta") else v) for k, v in w.items()}
        oa, fa = _run_gpu(a)
        ob, fb = _run_gpu(b, initial_state=fa)
        check(f"split {split} o", torch.cat([oa, ob], 1), o.float().cpu().numpy(), 2e-2)
        check(f"split {split} state", fb, fs.cpu().numpy(), 2e-2)


def test_fwd_varlen_equals_separate_calls():
    cu = [0, 100, 164, 300]
    w = inputs.chunk_inputs(1, 300, 2, 64, 64, seed=44, dtype=torch.float32, cu_seqlens=cu, h0_std=0.1)
    o, fs = _run_gpu(w)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        s = {k: (v[:, a:b] if k in ("q", "k", "v", "g", "beta") else v) for k, v in w.items()}
        s["cu_seqlens"] = None
        s["initial_state"] = w["initial_state"][n:n + 1]
        on, fn = _run_gpu(s)
        check(f"seq {n} o", o[:, a:b], on.cpu().numpy(), 1e-5)
        check(f"seq {n} state", fs[n:n + 1], fn.cpu().numpy(), 1e-5)


def test_fwd_no_final_state_and_deterministic():
    w = inputs.chunk_inputs(2, 150, 2, 128, 128, seed=5, dtype=torch.bfloat16)
    o1, f1 = _run_gpu(w, output_final_state=False)
    o2, _ = _run_gpu(w, output_final_state=False)
    assert f1 is None
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("chunk_size", [1, 16, 32, 100])
def test_fwd_chunk_size_is_a_tiling_request(chunk_size):
    """Any chunk size >= 1 is accepted as a tiling request, as the api.py dispatch
    maps it to each backend's own tiling: these kernels always tile with 64 rows, so
    the result is bit-identical to the default request and matches the oracle."""
    w = inputs.chunk_inputs(1, 130, 2, 64, 64, seed=90 + chunk_size, dtype=torch.bfloat16, h0_std=0.1,
                            cu_seqlens=[0, 33, 130])
    o64, fs64 = _run_gpu(w)
    o, fs = _run_gpu(w, chunk_size=chunk_size)
    assert torch.equal(o, o64) and torch.equal(fs, fs64)
    oo, ofs = _run_oracle(w)
    check(f"chunk_size={chunk_size} o", o, oo, tol_for(w["q"].dtype))
    check(f"chunk_size={chunk_size} final_state", fs, ofs, tol_for(w["q"].dtype))
