"""Robustness of the GPU path on inputs and buffers that parity cases do not
cover: a non-finite input stays inside its own (sequence, head) unit, and no
entry point writes outside its output tensors.

The finiteness-first form of the "memra-engine kda_fixture_gpu.rs" page's
`check` is applied to every unit that the poisoned token cannot reach: those
units must be finite and equal to the oracle."""
import numpy as np
import pytest
import torch

import oracle
import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import inputs
from parity import check, dev, tol_for

pytestmark = pytest.mark.gpu

CU = [0, 100, 230, 300]
POISON_SEQ, POISON_HEAD, POISON_ROW = 1, 1, 137  # row 137 lies in sequence 1 (rows 100..229)


def _blank_unit(x, seq, head, cu, per_row=True):
    """x with the (sequence, head) unit's entries set to zero: rows of `seq`
    (per_row tensors [1, T, H, ...]) or the unit's state ([N, H, ...])."""
    x = np.array(x, dtype=np.float64, copy=True)
    if per_row:
        x[:, cu[seq]:cu[seq + 1], head] = 0.0
    else:
        x[seq, head] = 0.0
    return x


def _gpu_np(t):
    return t.detach().float().cpu().double().numpy()


@pytest.mark.parametrize("where", ["q", "v", "g", "beta", "dO"])
def test_nan_token_stays_in_its_unit(where):
    """One token of one packed sequence carries NaN in one input (q, v, the
    gate, beta or the upstream gradient).  The calls return, and every other
    (sequence, head) unit's outputs and gradients are finite and equal to the
    oracle's."""
    w = inputs.chunk_inputs(1, CU[-1], 3, 64, 64, seed=121, dtype=torch.bfloat16, cu_seqlens=CU, h0_std=0.1,
                            with_grad_out=True, dfinal_std=0.1)
    if where == "beta":
        w["beta"][0, POISON_ROW, POISON_HEAD] = float("nan")
    else:
        w[where][0, POISON_ROW, POISON_HEAD, :5] = float("nan")
    print(f"NaN in {where} at row {POISON_ROW} head {POISON_HEAD}", flush=True)
    kw = dict(scale=w["scale"], initial_state=dev(w["initial_state"]), use_qk_l2norm_in_kernel=True,
              lower_bound=w["lower_bound"], cu_seqlens=dev(w["cu_seqlens"]), gate_mode=w["gate_mode"])
    q, k, v, g, beta, dO = (dev(w[n]) for n in ("q", "k", "v", "g", "beta", "dO"))
    o, fs = kda.chunk_kda(q, k, v, g, beta, output_final_state=True, **kw)
    gr = kda.chunk_kda_bwd(q, k, v, g, beta, dO, d_final_state=dev(w["d_final_state"]), **kw)
    torch.cuda.synchronize()
    okw = dict(scale=w["scale"], initial_state=w["initial_state"], use_qk_l2norm=True, gate_mode=w["gate_mode"],
               lower_bound=w["lower_bound"], cu_seqlens=w["cu_seqlens"])
    with np.errstate(invalid="ignore"):
        oo, ofs = oracle.chunk_fwd(w["q"], w["k"], w["v"], w["g"], w["beta"], **okw)
        og = oracle.chunk_bwd(w["q"], w["k"], w["v"], w["g"], w["beta"], w["dO"],
                              d_final_state=w["d_final_state"], **okw)
    tol = tol_for(torch.bfloat16)
    s, h = POISON_SEQ, POISON_HEAD
    check("o (other units)", _blank_unit(_gpu_np(o), s, h, CU), _blank_unit(oo, s, h, CU), tol)
    check("final state (other units)", _blank_unit(_gpu_np(fs), s, h, CU, False),
          _blank_unit(ofs, s, h, CU, False), tol)
    for name in ("dq", "dk", "dv", "dg", "dbeta"):
        check(f"{name} (other units)", _blank_unit(_gpu_np(gr[name]), s, h, CU), _blank_unit(og[name], s, h, CU),
              tol)
    check("dh0 (other units)", _blank_unit(_gpu_np(gr["dh0"]), s, h, CU, False),
          _blank_unit(og["dh0"], s, h, CU, False), tol)
    # the poisoned unit's outputs after the token are not finite (the NaN propagates)
    if where != "dO":
        assert not np.isfinite(_gpu_np(o)[0, POISON_ROW:CU[s + 1], h]).all()


PAD = 256  # guard elements on each side: a multiple of 8, so views stay 16-byte aligned
SENTINEL = 12288.0  # exact in bf16 and fp32


def _guarded(shape, dtype):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * PAD,), SENTINEL, dtype=dtype, device="cuda")
    return buf, buf[PAD:PAD + n].view(*shape)


def _guards_intact(name, buf):
    g = torch.cat([buf[:PAD], buf[-PAD:]]).float().cpu()
    assert bool((g == SENTINEL).all()), f"{name}: an entry point wrote outside its output tensor"


def test_outputs_are_not_overrun():
    """Every output of the chunk forward and backward, the decode step, the
    conv prefill and the output gate, placed between guard bands of a sentinel
    value: after the calls the guards are unchanged and the outputs match the
    oracle (ragged packed lengths, so that tail chunks and partial rows are
    exercised)."""
    cu = [0, 1, 66, 130, 197]
    T, H, K, V = cu[-1], 2, 128, 128
    w = inputs.chunk_inputs(1, T, H, K, V, seed=131, dtype=torch.bfloat16, cu_seqlens=cu, h0_std=0.1,
                            with_grad_out=True, dfinal_std=0.1)
    N = len(cu) - 1
    kw = dict(scale=w["scale"], initial_state=dev(w["initial_state"]), use_qk_l2norm_in_kernel=True,
              lower_bound=w["lower_bound"], cu_seqlens=dev(w["cu_seqlens"]), gate_mode=w["gate_mode"])
    q, k, v, g, beta, dO = (dev(w[n]) for n in ("q", "k", "v", "g", "beta", "dO"))
    bo, o = _guarded((1, T, H, V), torch.bfloat16)
    bfs, fs = _guarded((N, H, K, V), torch.float32)
    kda.chunk_kda(q, k, v, g, beta, output_final_state=True, out=o, final_state_out=fs, **kw)
    shapes = {"dq": ((1, T, H, K), torch.bfloat16), "dk": ((1, T, H, K), torch.bfloat16),
              "dv": ((1, T, H, V), torch.bfloat16), "dg": ((1, T, H, K), torch.float32),
              "dbeta": ((1, T, H), torch.float32), "dh0": ((N, H, K, V), torch.float32)}
    bufs, outs = {}, {}
    for name, (shape, dt) in shapes.items():
        bufs[name], outs[name] = _guarded(shape, dt)
    kda.chunk_kda_bwd(q, k, v, g, beta, dO, d_final_state=dev(w["d_final_state"]), out=outs, **kw)
    torch.cuda.synchronize()
    _guards_intact("o", bo)
    _guards_intact("final_state", bfs)
    for name in shapes:
        _guards_intact(name, bufs[name])
    okw = dict(scale=w["scale"], initial_state=w["initial_state"], use_qk_l2norm=True, gate_mode=w["gate_mode"],
               lower_bound=w["lower_bound"], cu_seqlens=w["cu_seqlens"])
    oo, ofs = oracle.chunk_fwd(w["q"], w["k"], w["v"], w["g"], w["beta"], **okw)
    og = oracle.chunk_bwd(w["q"], w["k"], w["v"], w["g"], w["beta"], w["dO"], d_final_state=w["d_final_state"],
                          **okw)
    tol = tol_for(torch.bfloat16)
    check("o", o, oo, tol)
    check("final_state", fs, ofs, tol)
    for name in shapes:
        check(name, outs[name], og[name], tol)

    # decode step (fp32 output) and the gated output
    Nd, Hd, D, W = 3, 2, 128, 4
    init = inputs.decode_init(Nd, Hd, D, W, seed=132)
    st_in = inputs.decode_step_inputs(Nd, Hd, D, seed=132, step=0)
    cs, s = dev(init["conv_state"]).clone(), dev(init["state"]).clone()
    bdo, do_ = _guarded((Nd, Hd * D), torch.float32)
    kda.recurrent_step(dev(st_in["x"]), dev(init["conv_w"]), cs, dev(st_in["g"]), dev(st_in["beta"]), s, out=do_)
    torch.cuda.synchronize()
    _guards_intact("decode o", bdo)
    o_ref, _, _ = oracle.decode_step(st_in["x"], init["conv_w"], init["conv_state"], st_in["g"], st_in["beta"],
                                     init["state"])
    check("decode o", do_, o_ref, 1e-4)

    # conv prefill (q, k, v outputs) and the output gate with its reverse mode
    x = inputs.prefill_inputs(T, H, K, seed=133)["x"]
    cinit = inputs.decode_init(N, H, K, W, seed=134)
    qkv_bufs, qkv = zip(*(_guarded((T, H, K), torch.bfloat16) for _ in range(3)))
    kda.conv_prefill(dev(x), dev(cinit["conv_w"]), H, K, conv_state=dev(cinit["conv_state"]).clone(),
                     cu_seqlens=dev(w["cu_seqlens"]), out=tuple(qkv))
    gi = inputs.gate_inputs(T, H, V, seed=135)
    by, y = _guarded((T, H, V), torch.bfloat16)
    kda.output_gate(dev(gi["o"]), dev(gi["g"]), out=y)
    bdo2, dO2 = _guarded((T, H, V), torch.bfloat16)
    bdg2, dg2 = _guarded((T, H, V), torch.bfloat16)
    kda.output_gate_bwd(dev(gi["o"]), dev(gi["g"]), dev(gi["dy"]), out=(dO2, dg2))
    torch.cuda.synchronize()
    for name, b in zip("qkv", qkv_bufs):
        _guards_intact(f"conv prefill {name}", b)
    _guards_intact("output gate y", by)
    _guards_intact("output gate dO", bdo2)
    _guards_intact("output gate dg", bdg2)
    y_ref, _ = oracle.conv_prefill(x, cinit["conv_w"], cinit["conv_state"], cu_seqlens=np.array(cu, np.int32))
    HK = H * K
    for i, name in enumerate("qkv"):
        check(f"conv {name}", qkv[i].reshape(T, HK), y_ref[:, i * HK:(i + 1) * HK], tol)
    check("gate y", y, oracle.output_gate(gi["o"], gi["g"]), tol)
    rdO, rdg = oracle.output_gate_bwd(gi["o"], gi["g"], gi["dy"])
    check("gate dO", dO2, rdO, tol)
    check("gate dg", dg2, rdg, tol)
