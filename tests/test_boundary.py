"""CPU checks of the C ABI: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before launching anything.
Every call here fails validation, so no kernel is ever launched."""
import ctypes
import os
import re

import pytest

from kimi_delta_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from kimi_delta_attention_amd import build
        build.build()
    return _lib.load()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w ]+?\*?\s*\b(kda_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    for s in range(6):
        assert lib.kda_status_string(s)
    assert lib.kda_version() >= 10000


FAKE = 0x10000  # an aligned non-null address; never dereferenced because validation fails first


def _args(**over):
    a = _lib.ChunkArgs()
    a.B, a.T, a.H, a.K, a.V = 1, 64, 2, 32, 32
    a.qkv_dtype = _lib.KDA_F32
    for f in ("q", "k", "v", "g", "beta", "o"):
        setattr(a, f, FAKE)
    a.scale = float("nan")
    a.lower_bound = float("nan")
    a.gate_mode = _lib.KDA_GATE_LOGDECAY
    a.chunk_size = 64
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(chunk_size=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(chunk_size=-64), _lib.KDA_ERR_INVALID_ARG),
    (dict(K=48, V=48), _lib.KDA_ERR_UNSUPPORTED),
    (dict(K=64, V=32), _lib.KDA_ERR_UNSUPPORTED),              # only the narrow-key pair 32/64 is built
    (dict(K=64, V=128), _lib.KDA_ERR_UNSUPPORTED),
    (dict(K=128, V=128), _lib.KDA_ERR_UNSUPPORTED),           # fp32 at K = 128
    (dict(qkv_dtype=7), _lib.KDA_ERR_UNSUPPORTED),
    (dict(H=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(T=-1), _lib.KDA_ERR_INVALID_ARG),
    (dict(q=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(q=FAKE + 4), _lib.KDA_ERR_INVALID_ARG),             # misaligned
    (dict(gate_mode=5), _lib.KDA_ERR_INVALID_ARG),
    (dict(use_qk_l2norm=3), _lib.KDA_ERR_INVALID_ARG),
    (dict(gate_mode=_lib.KDA_GATE_SOFTPLUS), _lib.KDA_ERR_MISSING_PARAM),
    (dict(gate_mode=_lib.KDA_GATE_SAFE, A_log=FAKE), _lib.KDA_ERR_MISSING_PARAM),
    (dict(output_final_state=1), _lib.KDA_ERR_INVALID_ARG),
    (dict(cu_seqlens=FAKE, B=2, N=2), _lib.KDA_ERR_INVALID_ARG),
    (dict(keep_for_backward=2), _lib.KDA_ERR_INVALID_ARG),
    (dict(), _lib.KDA_ERR_WORKSPACE),                         # workspace required, none given
])
def test_chunk_fwd_rejects_before_launch(lib, over, status):
    a = _args(**over)
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == status


def test_workspace_query_is_host_only(lib):
    a = _args()
    need = lib.kda_chunk_fwd_workspace(ctypes.byref(a))
    assert need > 0
    a.workspace = FAKE
    a.workspace_bytes = need - 1
    assert lib.kda_chunk_fwd(ctypes.byref(a)) == _lib.KDA_ERR_WORKSPACE
    bad = _args(chunk_size=0)
    assert lib.kda_chunk_fwd_workspace(ctypes.byref(bad)) == 0


def test_keep_for_backward_needs_the_backward_workspace(lib):
    # the saving forward writes the backward's layout, so it asks for (and
    # checks against) the backward's workspace size
    a = _args()
    need_fwd = lib.kda_chunk_fwd_workspace(ctypes.byref(a))
    need_bwd = lib.kda_chunk_bwd_workspace(ctypes.byref(a))
    assert need_bwd > need_fwd > 0
    k = _args(keep_for_backward=1)
    assert lib.kda_chunk_fwd_workspace(ctypes.byref(k)) == need_bwd
    k.workspace = FAKE
    k.workspace_bytes = need_fwd
    assert lib.kda_chunk_fwd(ctypes.byref(k)) == _lib.KDA_ERR_WORKSPACE


def test_chunk_bwd_rejects_before_launch(lib):
    a = _args()
    g = _lib.ChunkGrads()
    assert lib.kda_chunk_bwd(ctypes.byref(a), None) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_chunk_bwd(ctypes.byref(a), ctypes.byref(g)) == _lib.KDA_ERR_INVALID_ARG  # no dO
    for f in ("dO", "dq", "dk", "dv", "dg", "dbeta"):
        setattr(g, f, FAKE)
    g.dA_log = FAKE  # only meaningful for the in-kernel gate
    assert lib.kda_chunk_bwd(ctypes.byref(a), ctypes.byref(g)) == _lib.KDA_ERR_INVALID_ARG


def _step(**over):
    s = _lib.StepArgs()
    s.N, s.H, s.D, s.W = 2, 2, 128, 4
    s.x_dtype = _lib.KDA_BF16
    for f in ("x_qkv", "conv_w", "conv_state", "g", "beta", "state", "o"):
        setattr(s, f, FAKE)
    s.lower_bound = float("nan")
    s.scale = float("nan")
    s.use_qk_l2norm = s.use_beta_sigmoid = 1
    for k, v in over.items():
        setattr(s, k, v)
    return s


@pytest.mark.parametrize("over,status", [
    (dict(D=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(W=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(W=9), _lib.KDA_ERR_INVALID_ARG),
    (dict(x_dtype=3), _lib.KDA_ERR_UNSUPPORTED),
    (dict(state=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(state=FAKE + 8), _lib.KDA_ERR_INVALID_ARG),
    (dict(gate_mode=_lib.KDA_GATE_SAFE, A_log=FAKE), _lib.KDA_ERR_MISSING_PARAM),
    (dict(gate_mode=_lib.KDA_GATE_SOFTPLUS), _lib.KDA_ERR_MISSING_PARAM),
])
def test_recurrent_step_rejects_before_launch(lib, over, status):
    s = _step(**over)
    assert lib.kda_recurrent_step(ctypes.byref(s)) == status


def test_recurrent_step_empty_batch_is_noop(lib):
    s = _step(N=0)
    assert lib.kda_recurrent_step(ctypes.byref(s)) == _lib.KDA_OK


def _conv(**over):
    a = _lib.ConvArgs()
    a.B, a.T, a.H, a.D, a.W = 2, 100, 2, 128, 4
    a.N = 0
    a.x_dtype = a.y_dtype = _lib.KDA_BF16
    for f in ("x_qkv", "conv_w", "conv_state", "q", "k", "v"):
        setattr(a, f, FAKE)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(D=96), _lib.KDA_ERR_UNSUPPORTED),
    (dict(W=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(W=9), _lib.KDA_ERR_INVALID_ARG),
    (dict(B=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(T=-1), _lib.KDA_ERR_INVALID_ARG),
    (dict(x_dtype=3), _lib.KDA_ERR_UNSUPPORTED),
    (dict(y_dtype=3), _lib.KDA_ERR_UNSUPPORTED),
    (dict(conv_w=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(q=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(x_qkv=FAKE + 8), _lib.KDA_ERR_INVALID_ARG),
    (dict(conv_state=FAKE + 4), _lib.KDA_ERR_INVALID_ARG),
    (dict(cu_seqlens=FAKE, B=2, N=2), _lib.KDA_ERR_INVALID_ARG),  # packed input needs B = 1
    (dict(cu_seqlens=FAKE, B=1, N=0), _lib.KDA_ERR_INVALID_ARG),
])
def test_conv_prefill_rejects_before_launch(lib, over, status):
    a = _conv(**over)
    assert lib.kda_conv_prefill(ctypes.byref(a)) == status


def test_python_binding_rejects_host_tensors():
    import torch
    import kimi_delta_attention_amd as kda
    x = torch.zeros(1, 4, 1, 32)
    with pytest.raises(ValueError):
        kda.chunk_kda(x, x, x, x, torch.zeros(1, 4, 1))


def _gate(**over):
    a = _lib.GateArgs()
    a.rows, a.H, a.V = 4, 2, 128
    a.o_dtype = a.g_dtype = _lib.KDA_BF16
    a.eps = float("nan")
    for f in ("o", "g", "y"):
        setattr(a, f, FAKE)
    for k, v in over.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("over,status", [
    (dict(V=48), _lib.KDA_ERR_UNSUPPORTED),
    (dict(V=512), _lib.KDA_ERR_UNSUPPORTED),
    (dict(o_dtype=3), _lib.KDA_ERR_UNSUPPORTED),
    (dict(g_dtype=3), _lib.KDA_ERR_UNSUPPORTED),
    (dict(rows=-1), _lib.KDA_ERR_INVALID_ARG),
    (dict(H=0), _lib.KDA_ERR_INVALID_ARG),
    (dict(eps=-1e-5), _lib.KDA_ERR_INVALID_ARG),
    (dict(y=None), _lib.KDA_ERR_INVALID_ARG),
    (dict(o=FAKE + 8), _lib.KDA_ERR_INVALID_ARG),
])
def test_output_gate_rejects_before_launch(lib, over, status):
    a = _gate(**over)
    assert lib.kda_output_gate(ctypes.byref(a)) == status


def test_output_gate_bwd_rejects_before_launch(lib):
    a = _gate()
    assert lib.kda_output_gate_bwd(ctypes.byref(a), None, FAKE, FAKE) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_output_gate_bwd(ctypes.byref(a), FAKE, FAKE + 4, FAKE) == _lib.KDA_ERR_INVALID_ARG
    assert lib.kda_output_gate_bwd(ctypes.byref(_gate(eps=-1.0)), FAKE, FAKE, FAKE) == _lib.KDA_ERR_INVALID_ARG


def test_output_gate_empty_is_noop(lib):
    # no rows: nothing to read, nothing launched, null pointers allowed
    a = _gate(rows=0, o=None, g=None, y=None)
    assert lib.kda_output_gate(ctypes.byref(a)) == _lib.KDA_OK
    assert lib.kda_output_gate_bwd(ctypes.byref(a), None, None, None) == _lib.KDA_OK


def test_recurrent_step_rejects_negative_gate_eps(lib):
    s = _step(out_gate=FAKE, out_gate_eps=-0.5)
    assert lib.kda_recurrent_step(ctypes.byref(s)) == _lib.KDA_ERR_INVALID_ARG


def test_recurrent_step_slot_map_needs_a_pool_size(lib):
    s = _step(state_slots=FAKE, n_slots=0)
    assert lib.kda_recurrent_step(ctypes.byref(s)) == _lib.KDA_ERR_INVALID_ARG
