"""kda_chunk_fwd_noalloc, called through the C ABI, against kda_chunk_fwd on
the same inputs: two calls in a row on one GPU (the second smaller, so that
it runs over what the first left in the library's scratch array), each equal
to the caller-workspace forward and to the oracle; and a call whose
workspace would exceed the array, refused before any launch."""
import ctypes

import pytest
import torch

import oracle
import kimi_delta_attention_amd as kda
from kimi_delta_attention_amd import _lib, inputs
from parity import check, dev, nan_full

pytestmark = pytest.mark.gpu


def _pair(w):
    kw = dict(A_log=dev(w["A_log"]), dt_bias=dev(w["dt_bias"]), scale=w["scale"],
              initial_state=dev(w["initial_state"]), output_final_state=True,
              use_qk_l2norm_in_kernel=True, gate_mode=w["gate_mode"],
              use_beta_sigmoid_in_kernel=w["use_beta_sigmoid"], lower_bound=w["lower_bound"],
              cu_seqlens=dev(w["cu_seqlens"]))
    q, k, v, g, beta = (dev(w[n]) for n in ("q", "k", "v", "g", "beta"))
    B, T, H, K = w["q"].shape
    V = w["v"].shape[-1]
    N = B if w["cu_seqlens"] is None else len(w["cu_seqlens"]) - 1
    ref_o, ref_s = kda.chunk_kda(q, k, v, g, beta, **kw)
    o, s = kda.chunk_kda_noalloc(q, k, v, g, beta, out=nan_full((B, T, H, V), w["q"].dtype),
                                 final_state_out=nan_full((N, H, K, V), torch.float32), **kw)
    torch.cuda.synchronize()
    return (o, s), (ref_o, ref_s), kw


def test_noalloc_forward_two_calls_then_smaller():
    big = inputs.chunk_inputs(1, 4096, 8, 128, 128, seed=141, dtype=torch.bfloat16,
                              cu_seqlens=[0, 1000, 3100, 4096], h0_std=0.1)
    small = inputs.chunk_inputs(2, 130, 3, 64, 64, seed=142, dtype=torch.bfloat16, h0_std=0.1,
                                gate_mode=inputs.GATE_SOFTPLUS, beta_logits=True)
    for tag, w in (("first (packed T4096 H8 K=V=128)", big), ("second (B2 T130 H3 K=V=64, softplus gate)", small)):
        print(f"noalloc {tag}", flush=True)
        (o, s), (ro, rs), _ = _pair(w)
        assert torch.equal(o, ro), tag
        assert torch.equal(s, rs), tag
        oo, os_ = oracle.chunk_fwd(w["q"], w["k"], w["v"], w["g"], w["beta"], A_log=w["A_log"],
                                   dt_bias=w["dt_bias"], scale=w["scale"], initial_state=w["initial_state"],
                                   use_qk_l2norm=True, gate_mode=w["gate_mode"],
                                   use_beta_sigmoid=w["use_beta_sigmoid"], lower_bound=w["lower_bound"],
                                   cu_seqlens=w["cu_seqlens"])
        check(f"{tag} o", o, oo, 2e-2)
        check(f"{tag} final_state", s, os_, 2e-2)


def test_noalloc_refuses_oversized_and_saving_calls():
    """A problem whose forward workspace exceeds the array is refused with
    KDA_ERR_WORKSPACE, and keep_for_backward with KDA_ERR_INVALID_ARG; neither
    launches anything (the device pointers are never dereferenced)."""
    lib = _lib.load()
    a = _lib.ChunkArgs()
    a.B, a.T, a.H, a.K, a.V = 1, 1 << 15, 64, 128, 128
    a.qkv_dtype = _lib.KDA_BF16
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: the call fails validation on the host
    a.q = a.k = a.v = a.g = a.beta = a.o = fake
    a.scale = float("nan")
    a.lower_bound = float("nan")
    a.chunk_size = 64
    assert lib.kda_chunk_fwd_workspace(ctypes.byref(a)) > _lib.KDA_NOALLOC_SCRATCH_BYTES
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(a)) == _lib.KDA_ERR_WORKSPACE
    a.T = 64
    a.keep_for_backward = 1
    assert lib.kda_chunk_fwd_noalloc(ctypes.byref(a)) == _lib.KDA_ERR_INVALID_ARG
