"""GPU parity of the full-rank output gate (kda_output_gate, its reverse mode,
and the gate fused into kda_recurrent_step) against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import inputs
from parity import check, dev, tol_for, TOL_F32, nan_full

pytestmark = pytest.mark.gpu

DTYPES = [(torch.float32, torch.float32), (torch.bfloat16, torch.bfloat16),
          (torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)]


@pytest.mark.parametrize("o_dtype,g_dtype", DTYPES)
@pytest.mark.parametrize("V", [32, 64, 128, 256])
def test_output_gate_forward(o_dtype, g_dtype, V):
    # 37 rows x 3 heads: not a multiple of any workgroup's vector count
    rows, H = 37, 3
    print(f"output gate rows={rows} H={H} V={V} o={o_dtype} g={g_dtype}", flush=True)
    x = inputs.gate_inputs(rows, H, V, seed=50 + V, dtype=o_dtype, g_dtype=g_dtype)
    for eps in (1e-5, 0.3):
        y = kda.output_gate(dev(x["o"]), dev(x["g"]), eps=eps, out=nan_full(x["o"].shape, o_dtype))
        torch.cuda.synchronize()
        assert y.dtype == o_dtype
        want = oracle.output_gate(x["o"], x["g"], eps=eps)
        tol = TOL_F32 if o_dtype == g_dtype == torch.float32 else tol_for(torch.bfloat16)
        check(f"y eps={eps}", y, want, tol)


@pytest.mark.parametrize("o_dtype,g_dtype", DTYPES)
@pytest.mark.parametrize("V", [32, 128, 256])
def test_output_gate_backward(o_dtype, g_dtype, V):
    rows, H = 29, 2
    print(f"output gate bwd rows={rows} H={H} V={V} o={o_dtype} g={g_dtype}", flush=True)
    x = inputs.gate_inputs(rows, H, V, seed=60 + V, dtype=o_dtype, g_dtype=g_dtype)
    pre = (nan_full(x["o"].shape, o_dtype), nan_full(x["g"].shape, g_dtype))  # unwritten elements fail the check
    dO, dg = kda.output_gate_bwd(dev(x["o"]), dev(x["g"]), dev(x["dy"]), eps=0.3, out=pre)
    torch.cuda.synchronize()
    assert dO.dtype == o_dtype and dg.dtype == g_dtype
    want_dO, want_dg = oracle.output_gate_bwd(x["o"], x["g"], x["dy"], eps=0.3)
    tol = TOL_F32 if o_dtype == g_dtype == torch.float32 else tol_for(torch.bfloat16)
    check("dO", dO, want_dO, tol)
    check("dg", dg, want_dg, tol)


def test_output_gate_in_place_and_default_eps():
    rows, H, V = 50, 4, 128
    x = inputs.gate_inputs(rows, H, V, seed=70, dtype=torch.float32)
    o = dev(x["o"]).clone()
    y = kda.output_gate(o, dev(x["g"]), out=o)  # eps None: 1e-5
    torch.cuda.synchronize()
    assert y.data_ptr() == o.data_ptr()
    check("y in place", o, oracle.output_gate(x["o"], x["g"], eps=1e-5), TOL_F32)
    # a zero upstream gradient gives zero gradients
    dO, dg = kda.output_gate_bwd(dev(x["o"]), dev(x["g"]), torch.zeros_like(o))
    torch.cuda.synchronize()
    assert float(dO.abs().max()) == 0.0 and float(dg.abs().max()) == 0.0


def test_output_gate_empty_is_noop():
    o = torch.zeros(0, 2, 64, device="cuda")
    y = kda.output_gate(o, o.clone())
    dO, dg = kda.output_gate_bwd(o, o.clone(), o.clone())
    torch.cuda.synchronize()
    assert y.numel() == dO.numel() == dg.numel() == 0


def test_output_gate_packed_batch_geometry():
    # every element of the packed batch's output: 8192 rows, H16, V128, bf16
    rows, H, V = 8192, 16, 128
    print(f"output gate rows={rows} H={H} V={V} bf16", flush=True)
    x = inputs.gate_inputs(rows, H, V, seed=71, dtype=torch.bfloat16)
    o, g, dy = dev(x["o"]), dev(x["g"]), dev(x["dy"])
    y = kda.output_gate(o, g)
    dO, dg = kda.output_gate_bwd(o, g, dy)
    torch.cuda.synchronize()
    check("y", y, oracle.output_gate(x["o"], x["g"], eps=1e-5), tol_for(torch.bfloat16))
    want_dO, want_dg = oracle.output_gate_bwd(x["o"], x["g"], x["dy"], eps=1e-5)
    check("dO", dO, want_dO, tol_for(torch.bfloat16))
    check("dg", dg, want_dg, tol_for(torch.bfloat16))


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("x_dtype", [torch.float32, torch.bfloat16])
def test_decode_with_fused_output_gate(D, x_dtype):
    # the gated output of a decode step equals the oracle's step followed by its gate
    N, H, W, T = 3, 2, 4, 3
    init = inputs.decode_init(N, H, D, W, seed=80 + D)
    steps = [inputs.decode_step_inputs(N, H, D, seed=81, step=t) for t in range(T)]
    gates = [inputs.gate_inputs(N, H, D, seed=90 + t, dtype=x_dtype)["g"].reshape(N, H * D) for t in range(T)]
    print(f"decode + output gate N={N} H={H} D={D} x={x_dtype}", flush=True)
    cw = dev(init["conv_w"])
    cs = dev(init["conv_state"]).clone()
    st = dev(init["state"]).clone()
    ocs, ost = init["conv_state"], init["state"]
    for t, (s, gt) in enumerate(zip(steps, gates)):
        eps = 1e-5 if t == 0 else 0.2
        y = kda.recurrent_step(dev(s["x"].to(x_dtype)), cw, cs, dev(s["g"]), dev(s["beta"]), st,
                               out_gate=dev(gt), out_gate_eps=eps)
        torch.cuda.synchronize()
        o, ocs, ost = oracle.decode_step(s["x"].to(x_dtype), init["conv_w"], ocs, s["g"], s["beta"], ost)
        want = oracle.output_gate(o.reshape(N, H, D), gt.reshape(N, H, D), eps=eps).reshape(N, H * D)
        check(f"y[{t}]", y, want, TOL_F32)
    check("state", st, ost, TOL_F32)
    check("conv_state", cs, ocs, TOL_F32)


def _fused(w, gate, eps, **over):
    B, T, H, K = w["q"].shape
    V = w["v"].shape[-1]
    N = B if w["cu_seqlens"] is None else len(w["cu_seqlens"]) - 1
    kw = dict(A_log=dev(w["A_log"]), dt_bias=dev(w["dt_bias"]), scale=w["scale"],
              initial_state=dev(w["initial_state"]), output_final_state=True,
              use_qk_l2norm_in_kernel=w["use_qk_l2norm"], gate_mode=w["gate_mode"],
              use_beta_sigmoid_in_kernel=w["use_beta_sigmoid"], lower_bound=w["lower_bound"],
              cu_seqlens=dev(w["cu_seqlens"]), out_gate=dev(gate), out_gate_eps=eps,
              out=nan_full((B, T, H, V), w["q"].dtype), final_state_out=nan_full((N, H, K, V), torch.float32))
    kw.update(over)
    y, fs = kda.chunk_kda(dev(w["q"]), dev(w["k"]), dev(w["v"]), dev(w["g"]), dev(w["beta"]), **kw)
    torch.cuda.synchronize()
    oo, ofs = oracle.chunk_fwd(w["q"], w["k"], w["v"], w["g"], w["beta"], A_log=w["A_log"], dt_bias=w["dt_bias"],
                               scale=w["scale"], initial_state=w["initial_state"], use_qk_l2norm=w["use_qk_l2norm"],
                               gate_mode=w["gate_mode"], use_beta_sigmoid=w["use_beta_sigmoid"],
                               lower_bound=w["lower_bound"], cu_seqlens=w["cu_seqlens"])
    want = oracle.output_gate(oo, gate, eps=1e-5 if eps is None else eps)
    # the same kernels' plain output, gated by the oracle: isolates the epilogue
    kw_plain = dict(kw)
    for key in ("out_gate", "out_gate_eps", "out", "final_state_out"):
        kw_plain.pop(key)
    o_plain, _ = kda.chunk_kda(dev(w["q"]), dev(w["k"]), dev(w["v"]), dev(w["g"]), dev(w["beta"]), **kw_plain)
    torch.cuda.synchronize()
    on_plain = oracle.output_gate(o_plain.float().cpu().double().numpy(), gate, eps=1e-5 if eps is None else eps)
    return y, fs, want, ofs, on_plain, oo


def _check_gated(tag, y, want, on_plain, oo, tol):
    """The gated output against (1) the oracle's gate of the same kernels' plain
    output, elementwise at tol, and (2) the oracle's gate of the oracle's
    forward, with the forward's bar carried through the gate: the gate divides
    row i by rms_i(o), so an error e in o becomes at most about 2 e / rms_i in y;
    |y - y_ref| * rms_i(o_ref) / 2 must stay within tol * max|o_ref|."""
    check(f"{tag} y vs gate(plain o)", y, on_plain, tol)
    got = y.float().cpu().double().numpy()
    assert np.isfinite(got).all(), f"{tag}: non-finite values"
    rms = np.sqrt((oo ** 2).mean(axis=-1, keepdims=True) + 1e-5)
    scale = max(float(np.abs(oo).max()), 1e-6)
    md = float((np.abs(got - want) * rms / 2.0).max())
    print(f"  {tag} y vs gate(oracle o), forward-equivalent: rel {md / scale:.3e} (tol {tol:.0e})", flush=True)
    assert md <= tol * scale, f"{tag}: forward-equivalent error {md / scale:.3e} above {tol:.1e}"


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
@pytest.mark.parametrize("dtype,K,V", [(torch.float32, 32, 32), (torch.float32, 64, 64), (torch.bfloat16, 32, 32),
                                       (torch.bfloat16, 64, 64), (torch.bfloat16, 128, 128),
                                       (torch.float32, 32, 64), (torch.bfloat16, 32, 64)])
def test_chunk_fwd_fused_output_gate(T, dtype, K, V):
    """kda_chunk_fwd with out_gate: the output gate applied in the state pass
    equals the oracle's gate of the oracle's forward, at lengths around the
    64-row chunk, with a random initial state, every geometry and dtype."""
    w = inputs.chunk_inputs(2, T, 3, K, V, seed=500 + T + K + V, dtype=dtype, h0_std=0.1)
    g_dtype = torch.bfloat16 if (T % 2) else torch.float32
    gate = inputs.gate_inputs(2 * T, 3, V, seed=600 + T, dtype=g_dtype)["g"].reshape(2, T, 3, V)
    print(f"fused gate T={T} K={K} V={V} {dtype} gate {g_dtype}", flush=True)
    y, fs, want, ofs, on_plain, oo = _fused(w, gate, None)
    tol = tol_for(dtype)
    _check_gated("fused", y, want, on_plain, oo, tol)
    check("final_state", fs, ofs, tol)


@pytest.mark.parametrize("dtype,K,V,B,H", [(torch.bfloat16, 128, 128, 16, 16), (torch.bfloat16, 32, 64, 32, 8),
                                           (torch.float32, 64, 64, 16, 16)])
def test_chunk_fwd_output_gate_in_state_pass(dtype, K, V, B, H):
    """With at least 256 (sequence, head) chains the gate is applied inside the
    state pass, one workgroup per chain (below that, by a pass over o in the
    same call): the same bar, a ragged tail chunk, a random initial state."""
    T = 70
    w = inputs.chunk_inputs(B, T, H, K, V, seed=620 + K + V, dtype=dtype, h0_std=0.1)
    gate = inputs.gate_inputs(B * T, H, V, seed=621, dtype=torch.bfloat16)["g"].reshape(B, T, H, V)
    print(f"gate in state pass B{B} H{H} K={K} V={V} {dtype}", flush=True)
    y, fs, want, ofs, on_plain, oo = _fused(w, gate, None)
    tol = tol_for(dtype)
    _check_gated("in state pass", y, want, on_plain, oo, tol)
    check("final_state", fs, ofs, tol)


def test_chunk_fwd_fused_output_gate_packed_batch():
    """The packed 1024/2048/1024/4096 batch, H16 K=V=128 bf16 with a bf16 gate
    input: every element of the gated output, and empty and tiny sequences."""
    w = inputs.workload("fwd_hybrid")
    gate = inputs.gate_inputs(8192, 16, 128, seed=611, dtype=torch.bfloat16)["g"].reshape(1, 8192, 16, 128)
    print("fused gate packed T8192 H16", flush=True)
    y, fs, want, ofs, on_plain, oo = _fused(w, gate, 0.01)
    _check_gated("packed", y, want, on_plain, oo, tol_for(torch.bfloat16))
    check("final_state", fs, ofs, tol_for(torch.bfloat16))
    cu = [0, 0, 1, 66, 66, 130, 200]
    w = inputs.chunk_inputs(1, 200, 2, 128, 128, seed=612, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.2)
    gate = inputs.gate_inputs(200, 2, 128, seed=613, dtype=torch.float32)["g"].reshape(1, 200, 2, 128)
    y, fs, want, ofs, on_plain, oo = _fused(w, gate, None)
    _check_gated("varlen", y, want, on_plain, oo, tol_for(torch.bfloat16))
    check("final_state varlen", fs, ofs, tol_for(torch.bfloat16))


def test_chunk_fwd_fused_output_gate_refuses_saving():
    w = inputs.chunk_inputs(1, 64, 2, 64, 64, seed=614, dtype=torch.bfloat16)
    gate = torch.zeros(1, 64, 2, 64, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        kda.chunk_kda(dev(w["q"]), dev(w["k"]), dev(w["v"]), dev(w["g"]), dev(w["beta"]), out_gate=gate,
                      workspace=ws, keep_for_backward=True)
