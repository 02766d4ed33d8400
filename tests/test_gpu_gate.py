"""GPU parity of the full-rank output gate (kda_output_gate, its reverse mode,
and the gate fused into kda_recurrent_step) against the CPU oracle."""
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
