"""GPU parity of kda_recurrent_step against the CPU oracle's decode step."""
import numpy as np
import pytest
import torch

import oracle
import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import inputs
from parity import check, dev, TOL_F32, nan_full

pytestmark = pytest.mark.gpu


def _gpu_steps(init, steps, N, H, D, x_dtype, **kw):
    cw = dev(init["conv_w"])
    cs = dev(init["conv_state"]).clone()
    st = dev(init["state"]).clone()
    outs = []
    for s in steps:
        # the output starts as NaN, so that an element the kernel does not write fails the check
        o = kda.recurrent_step(dev(s["x"].to(x_dtype)), cw, cs, dev(s["g"]), dev(s["beta"]), st,
                               out=nan_full((N, H * D), torch.float32), **kw)
        outs.append(o.clone())
    torch.cuda.synchronize()
    return outs, cs, st


def _oracle_steps(init, steps, x_dtype, **kw):
    cs = init["conv_state"]
    st = init["state"]
    outs = []
    for s in steps:
        o, cs, st = oracle.decode_step(s["x"].to(x_dtype), init["conv_w"], cs, s["g"], s["beta"], st, **kw)
        outs.append(o)
    return outs, cs, st


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("x_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("W", [4, 3])
def test_decode_small(D, x_dtype, W):
    N, H, T = 3, 2, 5
    init = inputs.decode_init(N, H, D, W, seed=11 + D + W)
    steps = [inputs.decode_step_inputs(N, H, D, seed=5, step=t) for t in range(T)]
    print(f"decode N={N} H={H} D={D} W={W} x={x_dtype}", flush=True)
    go, gcs, gst = _gpu_steps(init, steps, N, H, D, x_dtype)
    oo, ocs, ost = _oracle_steps(init, steps, x_dtype)
    for t in range(T):
        check(f"o[{t}]", go[t], oo[t], TOL_F32)
    check("state", gst, ost, TOL_F32)
    check("conv_state", gcs, ocs, TOL_F32)


@pytest.mark.parametrize("mode", [kda.KDA_GATE_SAFE, kda.KDA_GATE_SOFTPLUS])
def test_decode_gate_modes_and_flags(mode):
    N, H, D, W = 2, 3, 64, 4
    init = inputs.decode_init(N, H, D, W, seed=3)
    steps = [inputs.decode_step_inputs(N, H, D, seed=9, step=t) for t in range(3)]
    gen = torch.Generator().manual_seed(4)
    A_log = torch.rand(H, generator=gen) * np.log(16.0)
    dt = torch.randn(H * D, generator=gen) * 0.1
    lb = -5.0 if mode == kda.KDA_GATE_SAFE else None
    for st_ in steps:  # raw gate inputs for the in-kernel gate
        st_["g"] = torch.randn(N, H * D, generator=gen)
    kw_gpu = dict(gate_mode=mode, A_log=dev(A_log), dt_bias=dev(dt), lower_bound=lb, scale=0.3)
    kw_or = dict(gate_mode=mode, A_log=A_log, dt_bias=dt, lower_bound=lb, scale=0.3)
    go, gcs, gst = _gpu_steps(init, steps, N, H, D, torch.float32, **kw_gpu)
    oo, ocs, ost = _oracle_steps(init, steps, torch.float32, **kw_or)
    for t in range(3):
        check(f"o[{t}]", go[t], oo[t], TOL_F32)
    check("state", gst, ost, TOL_F32)
    # beta as a value and no normalisation
    go, _, gst = _gpu_steps(init, steps[:1], N, H, D, torch.float32, use_beta_sigmoid=False,
                            use_qk_l2norm=False, **kw_gpu)
    oo, _, ost = _oracle_steps(init, steps[:1], torch.float32, use_beta_sigmoid=False,
                               use_qk_l2norm=False, **kw_or)
    check("o/noflags", go[0], oo[0], TOL_F32)
    check("state/noflags", gst, ost, TOL_F32)


def test_decode_production_geometry_whole_batch():
    """64 sequences x 96 heads x d128, 256 consecutive steps in place, in the
    launch configuration the bench times: after every 32 steps the outputs,
    recurrent states and conv states of all 6,144 (sequence, head) units are
    compared with the oracle, which steps the whole batch in place alongside."""
    shp = inputs.DECODE_SHAPE
    N, H, D, W = shp["N"], shp["H"], shp["D"], shp["W"]
    seed = inputs.SEEDS["decode"]
    init = inputs.decode_init(N, H, D, W, seed=seed)
    ocs = init["conv_state"].double().numpy().copy()
    ost = init["state"].double().numpy().copy()
    cw = dev(init["conv_w"])
    cs = dev(init["conv_state"])
    st = dev(init["state"])
    o = nan_full((N, H * D), torch.float32)
    print("decode production geometry: 256 steps, whole batch", flush=True)
    for t in range(256):
        s = inputs.decode_step_inputs(N, H, D, seed=seed, step=t)
        if (t + 1) % 32 == 0:
            o.fill_(float("nan"))
        kda.recurrent_step(dev(s["x"]), cw, cs, dev(s["g"]), dev(s["beta"]), st, out=o)
        oo, _, _ = oracle.decode_step(s["x"], init["conv_w"], ocs, s["g"], s["beta"], ost, inplace=True)
        if (t + 1) % 32 == 0:
            torch.cuda.synchronize()
            check(f"o step {t + 1}", o, oo, TOL_F32)
            check(f"state step {t + 1}", st, ost, TOL_F32)
            check(f"conv state step {t + 1}", cs, ocs, TOL_F32)
            print(f"  step {t + 1} ok", flush=True)


def test_decode_slot_indexed_states():
    """Sequences resume from slots of a state pool (the prefix-hit restore of the
    kda.rs page's test prefix_hit_wrong_slot_diverges): the right slots give the
    oracle's steps from those states, other slots stay untouched, the wrong slot
    diverges, and a slot outside the pool is refused by the kernel."""
    S, N, H, D, W, T = 5, 3, 2, 64, 4, 3
    init = inputs.decode_init(S, H, D, W, seed=21)
    steps = [inputs.decode_step_inputs(N, H, D, seed=22, step=t) for t in range(T)]
    slots = [3, 0, 4]
    print(f"decode slots S={S} N={N} H={H} D={D} slots={slots}", flush=True)
    cw = dev(init["conv_w"])
    cs = dev(init["conv_state"]).clone()
    st = dev(init["state"]).clone()
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    outs = []
    for s in steps:
        outs.append(kda.recurrent_step(dev(s["x"]), cw, cs, dev(s["g"]), dev(s["beta"]), st,
                                       state_slots=sl).clone())
    torch.cuda.synchronize()
    ocs, ost = init["conv_state"][slots], init["state"][slots]
    for t, s in enumerate(steps):
        o, ocs, ost = oracle.decode_step(s["x"], init["conv_w"], ocs, s["g"], s["beta"], ost)
        check(f"o[{t}]", outs[t], o, TOL_F32)
    check("state slots", st[slots], ost, TOL_F32)
    check("conv_state slots", cs[slots], ocs, TOL_F32)
    for u in (1, 2):  # not in the map: bit-identical
        assert torch.equal(st[u].cpu(), init["state"][u]) and torch.equal(cs[u].cpu(), init["conv_state"][u])

    # the wrong slot for sequence 0 (its neighbour's state) gives a different output
    cs2 = dev(init["conv_state"]).clone()
    st2 = dev(init["state"]).clone()
    wrong = torch.tensor([0, 3, 4], dtype=torch.int32, device="cuda")
    o_wrong = kda.recurrent_step(dev(steps[0]["x"]), cw, cs2, dev(steps[0]["g"]), dev(steps[0]["beta"]), st2,
                                 state_slots=wrong)
    torch.cuda.synchronize()
    assert float((o_wrong[0] - outs[0][0]).abs().max()) > 1e-3

    # a slot outside the pool: NaN output for that sequence, its neighbours as usual
    cs3 = dev(init["conv_state"]).clone()
    st3 = dev(init["state"]).clone()
    bad = torch.tensor([S + 2, 0, 4], dtype=torch.int32, device="cuda")
    o_bad = kda.recurrent_step(dev(steps[0]["x"]), cw, cs3, dev(steps[0]["g"]), dev(steps[0]["beta"]), st3,
                               state_slots=bad)
    torch.cuda.synchronize()
    assert torch.isnan(o_bad[0]).all()
    assert torch.equal(o_bad[1:], outs[0][1:])
    for u in (1, 2, 3):
        assert torch.equal(st3[u].cpu(), init["state"][u]) and torch.equal(cs3[u].cpu(), init["conv_state"][u])
