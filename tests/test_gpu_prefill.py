"""GPU parity of the stateful prefill: kda_conv_prefill against the oracle,
and the prime -> decode hand-off through kda_chunk_fwd and kda_recurrent_step
(the "memra-engine kda_fixture_gpu.rs" page: GATE 2, decode after a stateful
prefill equals one full pass; GATE 3, a prompt primed in two stateful pieces
equals one prime)."""
import numpy as np
import pytest
import torch

import oracle
import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import inputs
from parity import check, dev, TOL_F32, TOL_BF16, nan_full

pytestmark = pytest.mark.gpu


def _cu(lens):
    return torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)


@pytest.mark.parametrize("x_dtype,y_dtype", [(torch.float32, torch.float32), (torch.bfloat16, torch.bfloat16),
                                             (torch.bfloat16, torch.float32), (torch.float32, torch.bfloat16)])
@pytest.mark.parametrize("W", [4, 2, 8])
def test_conv_prefill_packed(x_dtype, y_dtype, W):
    # ragged lengths: empty, shorter than the window, and across the 32-row blocks
    H, D = 2, 64
    lens = [0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 130]
    cu = _cu(lens)
    T, N, HD = int(cu[-1]), len(lens), H * D
    print(f"conv prefill packed lens={lens} H={H} D={D} W={W} x={x_dtype} y={y_dtype}", flush=True)
    x = inputs.prefill_inputs(T, H, D, seed=31 + W, dtype=x_dtype)["x"]
    init = inputs.decode_init(N, H, D, W, seed=32 + W)
    cs = dev(init["conv_state"]).clone()
    pre = tuple(nan_full((T, H, D), y_dtype) for _ in range(3))  # unwritten elements fail the check
    q, k, v = kda.conv_prefill(dev(x), dev(init["conv_w"]), H, D, conv_state=cs, cu_seqlens=dev(cu),
                               out_dtype=y_dtype, out=pre)
    torch.cuda.synchronize()
    y_ref, cs_ref = oracle.conv_prefill(x, init["conv_w"], init["conv_state"], cu_seqlens=cu.numpy())
    tol = TOL_BF16 if y_dtype == torch.bfloat16 else TOL_F32
    check("q", q.reshape(T, HD), y_ref[:, :HD], tol)
    check("k", k.reshape(T, HD), y_ref[:, HD:2 * HD], tol)
    check("v", v.reshape(T, HD), y_ref[:, 2 * HD:], tol)
    check("conv_state", cs, cs_ref, TOL_F32)


@pytest.mark.parametrize("D", [32, 128])
def test_conv_prefill_dense_without_state(D):
    B, T, H, W = 2, 100, 3, 4
    print(f"conv prefill dense B={B} T={T} H={H} D={D}", flush=True)
    x = inputs.prefill_inputs(B * T, H, D, seed=41, dtype=torch.bfloat16)["x"].reshape(B, T, 3 * H * D)
    init = inputs.decode_init(B, H, D, W, seed=42)
    q, k, v = kda.conv_prefill(dev(x), dev(init["conv_w"]), H, D)
    torch.cuda.synchronize()
    y_ref, none = oracle.conv_prefill(x, init["conv_w"])
    assert none is None
    HD = H * D
    check("q", q.reshape(B, T, HD), y_ref[..., :HD], TOL_BF16)
    check("k", k.reshape(B, T, HD), y_ref[..., HD:2 * HD], TOL_BF16)
    check("v", v.reshape(B, T, HD), y_ref[..., 2 * HD:], TOL_BF16)


def test_conv_prefill_packed_batch_geometry():
    # the packed batch of the chunk benchmark: 1024/2048/1024/4096 rows, H16, d128
    H, D, W = 16, 128, 4
    lens = [1024, 2048, 1024, 4096]
    cu = _cu(lens)
    T, N, HD = int(cu[-1]), len(lens), H * D
    print(f"conv prefill packed T={T} H={H} D={D}", flush=True)
    x = inputs.prefill_inputs(T, H, D, seed=43, dtype=torch.bfloat16)["x"]
    init = inputs.decode_init(N, H, D, W, seed=44)
    cs = dev(init["conv_state"]).clone()
    q, k, v = kda.conv_prefill(dev(x), dev(init["conv_w"]), H, D, conv_state=cs, cu_seqlens=dev(cu))
    torch.cuda.synchronize()
    y_ref, cs_ref = oracle.conv_prefill(x, init["conv_w"], init["conv_state"], cu_seqlens=cu.numpy())
    check("q", q.reshape(T, HD), y_ref[:, :HD], TOL_BF16)
    check("k", k.reshape(T, HD), y_ref[:, HD:2 * HD], TOL_BF16)
    check("v", v.reshape(T, HD), y_ref[:, 2 * HD:], TOL_BF16)
    check("conv_state", cs, cs_ref, TOL_F32)


def _oracle_decode_all(init, pre, dec, lens, H, D):
    """Oracle truth: every token of each sequence through the decode step."""
    cu = np.concatenate([[0], np.cumsum(lens)])
    outs, css, sts = [], [], []
    for n, L in enumerate(lens):
        cs = init["conv_state"][n:n + 1]
        st = init["state"][n:n + 1]
        on = []
        for r in range(cu[n], cu[n] + L):
            o, cs, st = oracle.decode_step(pre["x"][r:r + 1], init["conv_w"], cs, pre["g"][r:r + 1],
                                           pre["beta"][r:r + 1], st)
            on.append(o[0])
        for s in dec:
            o, cs, st = oracle.decode_step(s["x"][n:n + 1], init["conv_w"], cs, s["g"][n:n + 1],
                                           s["beta"][n:n + 1], st)
            on.append(o[0])
        outs.append(np.stack(on) if on else np.zeros((0, H * D)))
        css.append(cs[0])
        sts.append(st[0])
    return outs, np.stack(css), np.stack(sts)


def _gpu_prime(x, g, beta, conv_w, cs, state, cu, H, D, dtype):
    """Stateful prime of packed prompts: conv prefill, then the chunk forward
    from the decode state; conv state in place, returns (o [T, H*D], final state)."""
    T = x.shape[0]
    q, k, v = kda.conv_prefill(x, conv_w, H, D, conv_state=cs, cu_seqlens=cu, out_dtype=dtype)
    o, fs = kda.chunk_kda(q.unsqueeze(0), k.unsqueeze(0), v.unsqueeze(0), g.reshape(1, T, H, D),
                          beta.reshape(1, T, H), initial_state=state, output_final_state=True,
                          use_qk_l2norm_in_kernel=True, use_beta_sigmoid_in_kernel=True, cu_seqlens=cu)
    return o.reshape(T, H * D), fs


@pytest.mark.parametrize("dtype,D", [(torch.float32, 32), (torch.bfloat16, 128)])
def test_prime_then_decode_equals_decode(dtype, D):
    # GATE 2: prime each prompt statefully, step three more tokens through decode;
    # outputs, recurrent state and conv state equal decoding every token
    H, W, steps = 2, 4, 3
    lens = [1, 7, 64, 65]
    cu = _cu(lens)
    T, N = int(cu[-1]), len(lens)
    print(f"prime+decode lens={lens} H={H} D={D} dtype={dtype}", flush=True)
    init = inputs.decode_init(N, H, D, W, seed=51)
    pre = inputs.prefill_inputs(T, H, D, seed=52, dtype=dtype)
    dec = [inputs.decode_step_inputs(N, H, D, seed=53, step=t, dtype=dtype) for t in range(steps)]
    cw = dev(init["conv_w"])
    cs = dev(init["conv_state"]).clone()
    o_p, st = _gpu_prime(dev(pre["x"]), dev(pre["g"]), dev(pre["beta"]), cw, cs, dev(init["state"]), dev(cu),
                         H, D, dtype)
    o_d = []
    for s in dec:
        o_d.append(kda.recurrent_step(dev(s["x"]), cw, cs, dev(s["g"]), dev(s["beta"]), st).clone())
    torch.cuda.synchronize()
    outs, cs_ref, st_ref = _oracle_decode_all(init, pre, dec, lens, H, D)
    tol = TOL_BF16 if dtype == torch.bfloat16 else TOL_F32
    for n, L in enumerate(lens):
        check(f"prime o[{n}]", o_p[int(cu[n]):int(cu[n + 1])], outs[n][:L], tol)
        for t in range(steps):
            check(f"decode o[{n}][{t}]", o_d[t][n], outs[n][L + t], tol)
    check("state", st, st_ref, tol)
    check("conv_state", cs, cs_ref, TOL_F32)


@pytest.mark.parametrize("split", [1, 2, 3, 31, 33, 63, 64, 65, 127])
def test_two_piece_prime_equals_one(split):
    # GATE 3: one 130-token prompt primed in two stateful pieces equals a single prime
    H, D, W, total = 2, 32, 4, 130
    print(f"two-piece prime split={split}/{total - split}", flush=True)
    init = inputs.decode_init(1, H, D, W, seed=61)
    pre = inputs.prefill_inputs(total, H, D, seed=62, dtype=torch.float32)
    cw = dev(init["conv_w"])
    cs = dev(init["conv_state"]).clone()
    st = dev(init["state"])
    got = []
    start = 0
    for L in (split, total - split):
        rows = slice(start, start + L)
        o, st = _gpu_prime(dev(pre["x"][rows]), dev(pre["g"][rows]), dev(pre["beta"][rows]), cw, cs, st,
                           dev(_cu([L])), H, D, torch.float32)
        got.append(o)
        start += L
    torch.cuda.synchronize()
    outs, cs_ref, st_ref = _oracle_decode_all(init, pre, [], [total], H, D)
    check("o", torch.cat(got), outs[0], TOL_F32)
    check("state", st, st_ref, TOL_F32)
    check("conv_state", cs, cs_ref, TOL_F32)
