"""Pins of the CPU oracle against what the pages and the mathematics fix.

Nothing here compares the oracle with itself: each check is a hand-worked
value, a closed form, an invariant, an independent second derivation
(chunkwise vs token recurrence) or central finite differences.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from kimi_delta_attention_amd import inputs

LN2 = math.log(2.0)


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _num(x):
    if x == "-ln2":
        return -LN2
    return float(x)


# ---------------------------------------------------------------- recurrence
def _three_token_arrays(fx, q3=None):
    toks = fx["tokens"]
    T = len(toks)
    q = np.array([[t["q"] for t in toks]], dtype=np.float64).reshape(1, T, 1, 2)
    if q3 is not None:
        q[0, 2, 0] = q3
    k = np.array([[t["k"] for t in toks]], dtype=np.float64).reshape(1, T, 1, 2)
    v = np.array([[t["v"] for t in toks]], dtype=np.float64).reshape(1, T, 1, 2)
    g = np.array([[[_num(x) for x in t["g"]] for t in toks]]).reshape(1, T, 1, 2)
    beta = np.array([[t["beta"] for t in toks]]).reshape(1, T, 1)
    return q, k, v, g, beta


def test_three_token_hand_example(golden_dir):
    fx = _load(golden_dir, "three_token_recurrence.json")
    q, k, v, g, beta = _three_token_arrays(fx)
    o, S = oracle.chunk_fwd(q, k, v, g, beta, scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], fx["expected"]["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], fx["expected"]["final_state"], rtol=0, atol=1e-14)
    q, k, v, g, beta = _three_token_arrays(fx, q3=[0.6, 0.8])
    o, _ = oracle.chunk_fwd(q, k, v, g, beta, scale=1.0)
    np.testing.assert_allclose(o[0, 2, 0], fx["expected"]["o3_when_q3_equals_k3"], atol=1e-14)


@pytest.mark.parametrize("C", [1, 2, 3])
def test_three_token_chunked_form(golden_dir, C):
    fx = _load(golden_dir, "three_token_recurrence.json")
    q, k, v, g, beta = _three_token_arrays(fx)
    o, S = oracle.chunk_fwd_chunked(q, k, v, g, beta, chunk_size=C, scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], fx["expected"]["o"], atol=1e-14)
    np.testing.assert_allclose(S[0, 0], fx["expected"]["final_state"], atol=1e-14)


def test_single_token_closed_form():
    # From a zero state one token gives S1 = beta k^ v^T and o1 = s beta (q^.k^) v.
    rng = np.random.default_rng(7)
    K, V = 5, 3
    q, k = rng.normal(size=(1, 1, 1, K)), rng.normal(size=(1, 1, 1, K))
    v = rng.normal(size=(1, 1, 1, V))
    g = -rng.uniform(0, 3, size=(1, 1, 1, K))
    beta = np.array([[[0.3]]])
    s = 0.7
    o, S = oracle.chunk_fwd(q, k, v, g, beta, scale=s, use_qk_l2norm=True)
    qn = q[0, 0, 0] / math.sqrt((q ** 2).sum() + 1e-6)
    kn = k[0, 0, 0] / math.sqrt((k ** 2).sum() + 1e-6)
    np.testing.assert_allclose(S[0, 0], 0.3 * np.outer(kn, v[0, 0, 0]), rtol=1e-13)
    np.testing.assert_allclose(o[0, 0, 0], s * 0.3 * (qn @ kn) * v[0, 0, 0], rtol=1e-13)


def test_beta_zero_only_decays():
    # beta = 0: no writes, S_t = diag(exp(G_t)) S0 and o_t = s (diag(exp(G_t)) S0)^T q^_t.
    rng = np.random.default_rng(11)
    T, K, V = 9, 4, 3
    q, k = rng.normal(size=(1, T, 1, K)), rng.normal(size=(1, T, 1, K))
    v = rng.normal(size=(1, T, 1, V))
    g = -rng.uniform(0, 1, size=(1, T, 1, K))
    beta = np.zeros((1, T, 1))
    S0 = rng.normal(size=(1, 1, K, V))
    o, S = oracle.chunk_fwd(q, k, v, g, beta, scale=0.5, initial_state=S0, use_qk_l2norm=True)
    G = np.cumsum(g[0, :, 0], axis=0)
    for t in range(T):
        St = np.exp(G[t])[:, None] * S0[0, 0]
        qn = q[0, t, 0] / math.sqrt((q[0, t, 0] ** 2).sum() + 1e-6)
        np.testing.assert_allclose(o[0, t, 0], 0.5 * St.T @ qn, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(S[0, 0], np.exp(G[-1])[:, None] * S0[0, 0], rtol=1e-12)


def test_orthonormal_keys_overwrite():
    # g = 0, beta = 1, k_t = e_t: the write replaces what k_t reads, so row t of S is v_t,
    # and reading with q_t = k_t returns v_t exactly.
    T = K = 6
    V = 4
    rng = np.random.default_rng(3)
    k = np.eye(K)[None, :, None, :]
    v = rng.normal(size=(1, T, 1, V))
    S0 = rng.normal(size=(1, 1, K, V))
    o, S = oracle.chunk_fwd(k, k, v, np.zeros((1, T, 1, K)), np.ones((1, T, 1)), scale=1.0,
                            initial_state=S0)
    np.testing.assert_allclose(S[0, 0], v[0, :, 0], atol=1e-14)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], atol=1e-14)


def test_l2norm_epsilon():
    x = np.array([[0.6, 0.8]])
    np.testing.assert_allclose(oracle.l2norm(x), x / math.sqrt(1.0 + 1e-6), rtol=1e-15)


def test_decay_on_key_axis_not_value_axis():
    # One channel of decay hits one ROW of S (key index), never a column.
    S0 = np.arange(6, dtype=np.float64).reshape(1, 1, 2, 3) + 1
    g = np.array([[[[-LN2, 0.0]]]])
    z = np.zeros((1, 1, 1, 2))
    _, S = oracle.chunk_fwd(z, z, np.zeros((1, 1, 1, 3)), g, np.zeros((1, 1, 1)),
                            initial_state=S0, scale=1.0)
    np.testing.assert_allclose(S[0, 0], [[0.5, 1.0, 1.5], [4.0, 5.0, 6.0]], atol=1e-15)


# ---------------------------------------------------------------- prologue
def test_gate_values(golden_dir):
    fx = _load(golden_dir, "gate_values.json")
    x = np.array(fx["x"])
    sp = oracle.gate(x, gate_mode=oracle.GATE_SOFTPLUS, A_log=fx["A_log"], dt_bias=fx["dt_bias"])
    sf = oracle.gate(x, gate_mode=oracle.GATE_SAFE, A_log=fx["A_log"], dt_bias=fx["dt_bias"],
                     lower_bound=fx["lower_bound"])
    np.testing.assert_allclose(sp[0], fx["expected_softplus"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(sf[0], fx["expected_safe"], rtol=0, atol=1e-14)
    assert abs(sf[0, 0] - sp[0, 0]) > 0.1  # the bounded gate must differ from the unbounded one
    # A_log scales the rate: exp(A_log) multiplies the softplus (unbounded) and the logit (safe).
    sp2 = oracle.gate(x, gate_mode=oracle.GATE_SOFTPLUS, A_log=[math.log(3.0)], dt_bias=fx["dt_bias"])
    np.testing.assert_allclose(sp2, 3.0 * sp, rtol=1e-14)
    sf2 = oracle.gate(x, gate_mode=oracle.GATE_SAFE, A_log=[math.log(3.0)], dt_bias=fx["dt_bias"],
                      lower_bound=-5.0)
    z = x[0] + np.array(fx["dt_bias"])
    np.testing.assert_allclose(sf2[0], -5.0 / (1.0 + np.exp(-3.0 * z)), rtol=1e-14)
    # Large inputs: the stable softplus neither overflows nor loses the linear tail.
    big = oracle.gate(np.array([[800.0, -800.0]]), gate_mode=oracle.GATE_SOFTPLUS, A_log=[0.0])
    np.testing.assert_allclose(big[0], [-800.0, 0.0], atol=1e-300)


def test_beta_sigmoid_in_kernel():
    # Logit 0 means beta 0.5, and it still writes (kda.rs test beta_zero_is_sigmoid_half_not_zero).
    q = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    k = q.copy()
    v = np.array([1.0, 0.5]).reshape(1, 1, 1, 2)
    g = np.full((1, 1, 1, 2), -1.0)
    o0, _ = oracle.chunk_fwd(q, k, v, g, np.zeros((1, 1, 1)), use_qk_l2norm=True, use_beta_sigmoid=True)
    kn = 1.0 / math.sqrt(1.0 + 1e-6)
    np.testing.assert_allclose(o0[0, 0, 0], (2 ** -0.5) * 0.5 * kn * kn * v[0, 0, 0], rtol=1e-14)
    o20, _ = oracle.chunk_fwd(q, k, v, g, np.full((1, 1, 1), 20.0), use_qk_l2norm=True,
                              use_beta_sigmoid=True)
    assert np.abs(o20 - o0).max() > 1e-3


def test_missing_gate_params_raise():
    z = np.zeros((1, 2, 1, 2))
    with pytest.raises(ValueError):
        oracle.chunk_fwd(z, z, z, z, np.zeros((1, 2, 1)), gate_mode=oracle.GATE_SOFTPLUS)
    with pytest.raises(ValueError):
        oracle.chunk_fwd(z, z, z, z, np.zeros((1, 2, 1)), gate_mode=oracle.GATE_SAFE, A_log=[0.0])


# ---------------------------------------------------------------- chunkwise form
def _rand_problem(seed, B=1, T=13, H=2, K=4, V=3, gate_mode=oracle.GATE_LOGDECAY, cu=None,
                  beta_logits=False, h0=True):
    rng = np.random.default_rng(seed)
    q, k = rng.normal(size=(B, T, H, K)), rng.normal(size=(B, T, H, K))
    v = rng.normal(size=(B, T, H, V))
    if gate_mode == oracle.GATE_LOGDECAY:
        g = -5.0 / (1.0 + np.exp(-rng.normal(size=(B, T, H, K))))
    else:
        g = rng.normal(size=(B, T, H, K)) * 2.0
    beta = rng.normal(size=(B, T, H))
    if not beta_logits:
        beta = 1.0 / (1.0 + np.exp(-beta))
    N = B if cu is None else len(cu) - 1
    kw = dict(use_qk_l2norm=True, gate_mode=gate_mode, use_beta_sigmoid=beta_logits,
              initial_state=rng.normal(size=(N, H, K, V)) * 0.3 if h0 else None,
              cu_seqlens=None if cu is None else np.array(cu, dtype=np.int32), scale=0.61)
    if gate_mode != oracle.GATE_LOGDECAY:
        kw["A_log"] = rng.uniform(0, math.log(16), size=H)
        kw["dt_bias"] = rng.normal(size=H * K) * 0.1
    if gate_mode == oracle.GATE_SAFE:
        kw["lower_bound"] = -5.0
    return (q, k, v, g, beta), kw


@pytest.mark.parametrize("C", [1, 2, 4, 5, 16, 64])
@pytest.mark.parametrize("mode", [oracle.GATE_LOGDECAY, oracle.GATE_SAFE, oracle.GATE_SOFTPLUS])
def test_chunked_form_equals_recurrence(C, mode):
    args, kw = _rand_problem(100 + C + 7 * mode, T=13, gate_mode=mode, beta_logits=(mode == 2))
    o1, S1 = oracle.chunk_fwd(*args, **kw)
    o2, S2 = oracle.chunk_fwd_chunked(*args, chunk_size=C, **kw)
    np.testing.assert_allclose(o2, o1, rtol=1e-11, atol=1e-12 * np.abs(o1).max())
    np.testing.assert_allclose(S2, S1, rtol=1e-11, atol=1e-12 * np.abs(S1).max())


def test_chunked_form_varlen_long():
    args, kw = _rand_problem(5, T=200, H=1, K=8, V=6, cu=[0, 1, 64, 65, 130, 200])
    o1, S1 = oracle.chunk_fwd(*args, **kw)
    o2, S2 = oracle.chunk_fwd_chunked(*args, chunk_size=64, **kw)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12 * np.abs(o1).max())
    np.testing.assert_allclose(S2, S1, rtol=1e-10, atol=1e-12 * np.abs(S1).max())


def test_varlen_equals_separate_calls():
    cu = [0, 7, 7, 70, 130]
    args, kw = _rand_problem(9, T=130, cu=cu)
    o, S = oracle.chunk_fwd(*args, **kw)
    q, k, v, g, beta = args
    for n in range(len(cu) - 1):
        a, b = cu[n], cu[n + 1]
        sub = [x[:, a:b] for x in (q, k, v, g, beta)]
        kw1 = dict(kw, cu_seqlens=None, initial_state=kw["initial_state"][n:n + 1])
        if b > a:
            o1, S1 = oracle.chunk_fwd(*sub, **kw1)
            np.testing.assert_array_equal(o[:, a:b], o1)
        else:
            S1 = kw1["initial_state"]  # empty sequence: final state = initial state
        np.testing.assert_array_equal(S[n], S1[0])


@pytest.mark.parametrize("split", [1, 2, 3, 63, 64, 65, 127])
def test_split_call_equals_single_call(split):
    # memra gate 3 analogue: two calls with the state carried equal one call.
    args, kw = _rand_problem(21, T=130, H=1, K=4, V=4)
    o, S = oracle.chunk_fwd(*args, **kw)
    a1 = [x[:, :split] for x in args]
    a2 = [x[:, split:] for x in args]
    oa, Sa = oracle.chunk_fwd(*a1, **kw)
    ob, Sb = oracle.chunk_fwd(*a2, **dict(kw, initial_state=Sa))
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(Sb, S, rtol=1e-13, atol=1e-15)


def test_thread_count_does_not_change_results():
    args, kw = _rand_problem(31, B=3, T=40, H=3)
    o1, S1 = oracle.chunk_fwd(*args, threads=1, **kw)
    o8, S8 = oracle.chunk_fwd(*args, threads=8, **kw)
    np.testing.assert_array_equal(o1, o8)
    np.testing.assert_array_equal(S1, S8)


# ---------------------------------------------------------------- backward
def _loss(args, kw, dO, dSf):
    o, S = oracle.chunk_fwd(*args, **kw)
    return float((o * dO).sum() + (S * dSf).sum())


@pytest.mark.parametrize("mode,beta_logits,K,V", [(oracle.GATE_LOGDECAY, False, 8, 8),
                                                  (oracle.GATE_SAFE, True, 8, 8),
                                                  (oracle.GATE_SOFTPLUS, True, 8, 8),
                                                  (oracle.GATE_LOGDECAY, False, 4, 6)])
def test_backward_matches_finite_differences(mode, beta_logits, K, V):
    B, T, H = 1, 16, 1
    args, kw = _rand_problem(77 + mode, B=B, T=T, H=H, K=K, V=V, gate_mode=mode,
                             beta_logits=beta_logits)
    rng = np.random.default_rng(5)
    dO = rng.normal(size=(B, T, H, V))
    dSf = rng.normal(size=(B, H, K, V))
    gr = oracle.chunk_bwd(*args, dO, d_final_state=dSf, **kw)
    eps = 1e-6
    names = ["dq", "dk", "dv", "dg", "dbeta"]
    for idx, name in enumerate(names):
        base = [a.copy() for a in args]
        num = np.zeros_like(base[idx])
        flat = num.reshape(-1)
        for j in range(flat.size):
            plus = [a.copy() for a in base]
            minus = [a.copy() for a in base]
            plus[idx].reshape(-1)[j] += eps
            minus[idx].reshape(-1)[j] -= eps
            flat[j] = (_loss(plus, kw, dO, dSf) - _loss(minus, kw, dO, dSf)) / (2 * eps)
        scale = np.abs(num).max()
        np.testing.assert_allclose(gr[name], num, rtol=0, atol=1e-6 * scale, err_msg=name)
    # initial state, and the gate parameters
    extra = {"dh0": "initial_state"}
    if mode != oracle.GATE_LOGDECAY:
        extra.update({"dA_log": "A_log", "ddt_bias": "dt_bias"})
    for gname, key in extra.items():
        base = np.array(kw[key], dtype=np.float64)
        num = np.zeros_like(base)
        for j in range(base.size):
            p = base.copy()
            m = base.copy()
            p.reshape(-1)[j] += eps
            m.reshape(-1)[j] -= eps
            num.reshape(-1)[j] = (_loss(args, dict(kw, **{key: p}), dO, dSf)
                                  - _loss(args, dict(kw, **{key: m}), dO, dSf)) / (2 * eps)
        np.testing.assert_allclose(np.asarray(gr[gname]).reshape(num.shape), num, rtol=0,
                                   atol=1e-6 * np.abs(num).max(), err_msg=gname)


def test_backward_varlen_and_zero_cotangent_state():
    # packed sequences: the gradient of each sequence is the one of a separate call
    cu = [0, 5, 70, 80]
    args, kw = _rand_problem(41, T=80, H=1, K=4, V=3, cu=cu)
    rng = np.random.default_rng(1)
    dO = rng.normal(size=(1, 80, 1, 3))
    gr = oracle.chunk_bwd(*args, dO, **kw)
    for n in range(3):
        a, b = cu[n], cu[n + 1]
        sub = [x[:, a:b] for x in args]
        g1 = oracle.chunk_bwd(*sub, dO[:, a:b], **dict(kw, cu_seqlens=None,
                                                         initial_state=kw["initial_state"][n:n + 1]))
        for name in ["dq", "dk", "dv", "dg", "dbeta"]:
            np.testing.assert_allclose(gr[name][:, a:b], g1[name], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(gr["dh0"][n], g1["dh0"][0], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- decode
def _tiny_decode_problem():
    H, D, W = 1, 2, 4
    return H, D, W


def test_conv_window_advances(golden_dir):
    fx = _load(golden_dir, "conv_window.json")
    H, D, W = fx["H"], fx["D"], fx["W"]
    CH = 3 * H * D
    cs = np.zeros((1, CH, W))
    st = np.zeros((1, H, D, D))
    w = np.ones((CH, W))
    for t in fx["tokens"]:
        x = np.full((1, CH), t)
        o, cs, st = oracle.decode_step(x, w, cs, np.full((1, H * D), -1.0), np.zeros((1, H)), st)
        np.testing.assert_array_equal(cs[0, :, -1], x[0])  # the newest slot is the current token
    np.testing.assert_array_equal(cs[0], np.tile(fx["expected_window"], (CH, 1)))
    # the post-conv v channel reaches the recurrence: with S0 = 0 and one more token the
    # output is s * sigmoid(beta) * (q^.k^) * SiLU(conv), here with all channels equal.
    cs2 = cs.copy()
    cs2[0, :, :] = [0.0, 1.0, 2.0, 3.0]
    o, cs3, st3 = oracle.decode_step(np.full((1, CH), 4.0), w, cs2, np.zeros((1, H * D)),
                                     np.zeros((1, H)), np.zeros((1, H, D, D)))
    y = fx["expected_conv_out_after_4"]
    qn = np.full(D, y) / math.sqrt(D * y * y + 1e-6)
    expect = (D ** -0.5) * 0.5 * (qn @ qn) * y
    np.testing.assert_allclose(o[0], expect, rtol=1e-13)


def test_prefix_hit_wrong_slot_diverges():
    # kda.rs test prefix_hit_wrong_slot_diverges: restoring the snapshot taken after the real
    # prefix reproduces sequential decode; the snapshot of a shorter prefix does not.
    H, D, W = 1, 2, 4
    CH = 3 * H * D
    w = np.full((CH, W), 0.25)
    kw = dict(gate_mode=oracle.GATE_SAFE, A_log=np.array([-1.0]), dt_bias=np.zeros(2),
              lower_bound=-5.0)
    gx = np.array([[0.1, -0.2]])
    beta = np.array([[0.5]])
    cs, st = np.zeros((1, CH, W)), np.zeros((1, H, D, D))
    snaps = []
    for t in range(2):
        _, cs, st = oracle.decode_step(np.full((1, CH), (t + 1) * 0.1), w, cs, gx, beta, st, **kw)
        snaps.append((cs.copy(), st.copy()))
    x3 = np.full((1, CH), 0.4)
    y_seq, cs_seq, _ = oracle.decode_step(x3, w, cs, gx, beta, st, **kw)
    y_hit, cs_hit, _ = oracle.decode_step(x3, w, snaps[1][0], gx, beta, snaps[1][1], **kw)
    np.testing.assert_array_equal(y_hit, y_seq)
    np.testing.assert_array_equal(cs_hit, cs_seq)
    y_wrong, _, _ = oracle.decode_step(x3, w, snaps[0][0], gx, beta, snaps[0][1], **kw)
    assert np.abs(y_wrong - y_hit).max() > 1e-4


def test_decode_sequence_equals_chunk_forward_on_conv_output():
    # memra gate 2 analogue for the core: stepping T tokens through decode equals the chunk
    # forward of the same conv outputs, gate and beta, from the same initial state.
    rng = np.random.default_rng(12)
    N, H, D, W, T = 2, 2, 4, 4, 9
    CH = 3 * H * D
    w = rng.normal(size=(CH, W)) * 0.5
    cs0 = rng.normal(size=(N, CH, W)) * 0.05
    st0 = rng.normal(size=(N, H, D, D)) * 0.05
    xs = rng.normal(size=(T, N, CH))
    gs = -5.0 / (1.0 + np.exp(-rng.normal(size=(T, N, H * D))))
    bs = rng.normal(size=(T, N, H))
    cs, st = cs0.copy(), st0.copy()
    outs = []
    for t in range(T):
        o, cs, st = oracle.decode_step(xs[t], w, cs, gs[t], bs[t], st)
        outs.append(o)
    # conv outputs by explicit causal depthwise convolution over the history window
    hist = np.concatenate([np.transpose(cs0, (0, 2, 1))[:, 1:], np.transpose(xs, (1, 0, 2))], axis=1)
    y = np.zeros((N, T, CH))
    for t in range(T):
        win = hist[:, t:t + W]  # oldest -> newest
        a = np.einsum("nwc,cw->nc", win, w)
        y[:, t] = a / (1.0 + np.exp(-a))
    q = y[..., :H * D].reshape(N, T, H, D)
    k = y[..., H * D:2 * H * D].reshape(N, T, H, D)
    v = y[..., 2 * H * D:].reshape(N, T, H, D)
    g = np.transpose(gs, (1, 0, 2)).reshape(N, T, H, D)
    b = np.transpose(bs, (1, 0, 2))
    o_ref, S_ref = oracle.chunk_fwd(q, k, v, g, b, initial_state=st0, use_qk_l2norm=True,
                                    use_beta_sigmoid=True)
    np.testing.assert_allclose(np.stack(outs, 1).reshape(N, T, H, D), o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(st, S_ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- conv prefill
def _silu(a):
    from scipy.special import expit
    return a * expit(a)


def test_conv_prefill_is_causal_convolution():
    # the stateful prime is the textbook causal depthwise convolution (np.convolve)
    # of each channel's input extended by its W-1 history samples; the state left
    # behind is the last W samples of history ++ input
    rng = np.random.default_rng(21)
    C, W = 6, 4
    w = rng.normal(size=(C, W))
    lens = [0, 1, 2, 3, 7, 12]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = rng.normal(size=(int(cu[-1]), C))
    s0 = rng.normal(size=(len(lens), C, W))
    y, s1 = oracle.conv_prefill(x, w, s0, cu_seqlens=cu)
    for n, L in enumerate(lens):
        rows = slice(int(cu[n]), int(cu[n + 1]))
        for c in range(C):
            full = np.concatenate([s0[n, c], x[rows, c]])
            np.testing.assert_array_equal(s1[n, c], full[-W:])
            if L == 0:
                continue
            ref = np.convolve(full[1:], w[c, ::-1], mode="valid")  # ref[t] = sum_j w[c, j] full[1 + t + j]
            np.testing.assert_allclose(y[rows, c], _silu(ref), rtol=1e-13, atol=1e-14)
    # no state: a zero history, and the dense layout gives the same rows
    yz, none = oracle.conv_prefill(x[None, :7], w)
    assert none is None
    for c in range(C):
        ref = np.convolve(np.concatenate([np.zeros(W - 1), x[:7, c]]), w[c, ::-1], mode="valid")
        np.testing.assert_allclose(yz[0, :, c], _silu(ref), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("split", [0, 1, 2, 3, 5, 9])
def test_conv_prefill_state_carry_split(split):
    # memra GATE 3 analogue: one sequence primed in two stateful pieces equals a
    # single prime, including pieces shorter than the window
    rng = np.random.default_rng(22)
    C, W, T = 5, 4, 9
    w = rng.normal(size=(C, W))
    x = rng.normal(size=(1, T, C))
    s0 = rng.normal(size=(1, C, W))
    y, s = oracle.conv_prefill(x, w, s0)
    y1, sa = oracle.conv_prefill(x[:, :split], w, s0)
    y2, sb = oracle.conv_prefill(x[:, split:], w, sa)
    np.testing.assert_array_equal(np.concatenate([y1, y2], axis=1), y)
    np.testing.assert_array_equal(sb, s)


def test_conv_prefill_then_decode_equals_all_decode():
    # memra GATE 2 analogue: prime t0 tokens (conv prefill, then the chunk forward
    # from the decode state), then decode the rest; outputs and both states equal
    # decoding every token
    rng = np.random.default_rng(23)
    N, H, D, W, T, t0 = 2, 2, 4, 4, 8, 5
    CH = 3 * H * D
    w = rng.normal(size=(CH, W)) * 0.5
    cs0 = rng.normal(size=(N, CH, W)) * 0.05
    st0 = rng.normal(size=(N, H, D, D)) * 0.05
    xs = rng.normal(size=(N, T, CH))
    gs = -5.0 / (1.0 + np.exp(-rng.normal(size=(N, T, H * D))))
    bs = rng.normal(size=(N, T, H))
    cs, st, outs = cs0.copy(), st0.copy(), []
    for t in range(T):
        o, cs, st = oracle.decode_step(xs[:, t], w, cs, gs[:, t], bs[:, t], st)
        outs.append(o)
    o_all = np.stack(outs, 1)
    y, cs1 = oracle.conv_prefill(xs[:, :t0], w, cs0)
    q = y[..., :H * D].reshape(N, t0, H, D)
    k = y[..., H * D:2 * H * D].reshape(N, t0, H, D)
    v = y[..., 2 * H * D:].reshape(N, t0, H, D)
    o_p, st1 = oracle.chunk_fwd(q, k, v, gs[:, :t0].reshape(N, t0, H, D), bs[:, :t0], initial_state=st0,
                                use_qk_l2norm=True, use_beta_sigmoid=True)
    np.testing.assert_allclose(o_p.reshape(N, t0, H * D), o_all[:, :t0], rtol=1e-12, atol=1e-14)
    outs = []
    for t in range(t0, T):
        o, cs1, st1 = oracle.decode_step(xs[:, t], w, cs1, gs[:, t], bs[:, t], st1)
        outs.append(o)
    np.testing.assert_allclose(np.stack(outs, 1), o_all[:, t0:], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(cs1, cs)
    np.testing.assert_allclose(st1, st, rtol=1e-12, atol=1e-14)


def test_shared_input_recipes_have_stated_shapes():
    w = inputs.workload("fwd_small")
    assert tuple(w["q"].shape) == (1, 128, 2, 32) and w["q"].dtype.is_floating_point
    assert float(w["g"].max()) <= 0.0 and float(w["g"].min()) >= -5.0
    d = inputs.decode_step_inputs(2, 3, 4, seed=1, step=0)
    assert tuple(d["x"].shape) == (2, 36)


# ---------------------------------------------------------------- output gate
# [kda.rs] full_rank_output_gate: per head, sigmoid(g) * o / sqrt(mean(o^2) + eps).

def test_output_gate_hand_worked_vector():
    # o = (3, 4): mean of squares 12.5; with eps = 0, r = 1/sqrt(12.5).
    # g = (0, ln 3): sigmoid = (1/2, 3/4).
    y = oracle.output_gate(np.array([[3.0, 4.0]]), np.array([[0.0, math.log(3.0)]]), eps=0.0)
    r = 1.0 / math.sqrt(12.5)
    np.testing.assert_allclose(y, [[0.5 * 3.0 * r, 0.75 * 4.0 * r]], rtol=1e-15)


def test_output_gate_constant_row_closed_form():
    # a row of one value c: y[v] = sigmoid(g[v]) * c / sqrt(c^2 + eps)
    c, eps, V = -2.5, 1e-5, 8
    g = np.linspace(-3, 3, V)
    y = oracle.output_gate(np.full((1, V), c), g[None, :], eps=eps)
    want = [1.0 / (1.0 + math.exp(-gv)) * c / math.sqrt(c * c + eps) for gv in g]
    np.testing.assert_allclose(y[0], want, rtol=1e-14)


def test_output_gate_is_per_head_and_scale_free():
    rng = np.random.default_rng(5)
    o = rng.standard_normal((3, 2, 16))
    g = rng.standard_normal((3, 2, 16))
    y = oracle.output_gate(o, g, eps=0.0)
    # with eps = 0 the norm removes any positive scale of a head's vector
    o2 = o.copy()
    o2[:, 1] *= 7.0
    y2 = oracle.output_gate(o2, g, eps=0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-13, atol=1e-15)
    # changing head 1 leaves head 0 alone: the norm does not mix heads
    o3 = o.copy()
    o3[:, 1] = rng.standard_normal((3, 16))
    y3 = oracle.output_gate(o3, g, eps=1e-5)
    np.testing.assert_array_equal(y3[:, 0], oracle.output_gate(o, g, eps=1e-5)[:, 0])


def test_output_gate_open_gate_is_rms_norm():
    # g -> +inf opens the gate: mean(y^2) = ms / (ms + eps)
    rng = np.random.default_rng(6)
    o = 0.01 * rng.standard_normal((4, 32))
    eps = 1e-5
    y = oracle.output_gate(o, np.full_like(o, 60.0), eps=eps)
    ms = (o ** 2).mean(axis=1)
    np.testing.assert_allclose((y ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-12)


def test_output_gate_bwd_central_differences():
    rng = np.random.default_rng(7)
    o = rng.standard_normal((3, 2, 8))
    g = rng.standard_normal((3, 2, 8))
    dy = rng.standard_normal((3, 2, 8))
    eps, h = 0.3, 1e-6  # a large eps keeps both terms of dO of similar size
    dO, dg = oracle.output_gate_bwd(o, g, dy, eps=eps)
    loss = lambda oo, gg: float((dy * oracle.output_gate(oo, gg, eps=eps)).sum())
    for idx in [(0, 0, 0), (1, 1, 3), (2, 0, 7), (2, 1, 5)]:
        e = np.zeros_like(o)
        e[idx] = h
        fd_o = (loss(o + e, g) - loss(o - e, g)) / (2 * h)
        fd_g = (loss(o, g + e) - loss(o, g - e)) / (2 * h)
        assert abs(fd_o - dO[idx]) < 1e-8 * max(1.0, abs(fd_o)), (idx, fd_o, dO[idx])
        assert abs(fd_g - dg[idx]) < 1e-8 * max(1.0, abs(fd_g)), (idx, fd_g, dg[idx])


def test_output_gate_bwd_is_orthogonal_to_o_at_zero_eps():
    # scaling o does not change y when eps = 0, so the gradient has no component along o
    rng = np.random.default_rng(8)
    o = rng.standard_normal((5, 64))
    g = rng.standard_normal((5, 64))
    dy = rng.standard_normal((5, 64))
    dO, _ = oracle.output_gate_bwd(o, g, dy, eps=0.0)
    np.testing.assert_allclose((dO * o).sum(axis=1), 0.0, atol=1e-12)
