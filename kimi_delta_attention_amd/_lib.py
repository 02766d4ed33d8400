"""ctypes mirror of include/kda.h and the loader of the in-tree ``libkda.so``.

There is no fallback: if the library is missing or fails to load, every call
raises.  The library is built by ``kimi_delta_attention_amd.build`` (or
``__graft_entry__.build()``).
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_MISSING_PARAM, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(6)
KDA_F32, KDA_BF16 = 0, 1
KDA_GATE_LOGDECAY, KDA_GATE_SAFE, KDA_GATE_SOFTPLUS = 0, 1, 2

_vp = ctypes.c_void_p

# Size of the library's own device scratch used by kda_chunk_fwd_noalloc.
KDA_NOALLOC_SCRATCH_BYTES = 192 << 20


class ChunkArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("K", ctypes.c_int), ("V", ctypes.c_int),
        ("cu_seqlens", _vp), ("N", ctypes.c_int),
        ("qkv_dtype", ctypes.c_int),
        ("q", _vp), ("k", _vp), ("v", _vp), ("g", _vp), ("beta", _vp),
        ("A_log", _vp), ("dt_bias", _vp),
        ("scale", ctypes.c_float), ("lower_bound", ctypes.c_float),
        ("gate_mode", ctypes.c_int), ("use_qk_l2norm", ctypes.c_int), ("use_beta_sigmoid", ctypes.c_int),
        ("chunk_size", ctypes.c_int),
        ("initial_state", _vp), ("output_final_state", ctypes.c_int),
        ("o", _vp), ("final_state", _vp),
        ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
        ("stream", _vp),
        ("keep_for_backward", ctypes.c_int),
        ("out_gate", _vp), ("out_gate_dtype", ctypes.c_int), ("out_gate_eps", ctypes.c_float),
    ]


class ChunkGrads(ctypes.Structure):
    _fields_ = [
        ("dO", _vp), ("d_final_state", _vp),
        ("dq", _vp), ("dk", _vp), ("dv", _vp),
        ("dg", _vp), ("dbeta", _vp), ("d_initial_state", _vp),
        ("dA_log", _vp), ("ddt_bias", _vp),
    ]


class StepArgs(ctypes.Structure):
    _fields_ = [
        ("N", ctypes.c_int), ("H", ctypes.c_int), ("D", ctypes.c_int), ("W", ctypes.c_int),
        ("x_dtype", ctypes.c_int),
        ("x_qkv", _vp), ("conv_w", _vp), ("conv_state", _vp),
        ("g", _vp), ("beta", _vp), ("A_log", _vp), ("dt_bias", _vp),
        ("lower_bound", ctypes.c_float), ("gate_mode", ctypes.c_int),
        ("use_qk_l2norm", ctypes.c_int), ("use_beta_sigmoid", ctypes.c_int),
        ("scale", ctypes.c_float),
        ("state", _vp), ("o", _vp),
        ("stream", _vp),
        ("out_gate", _vp), ("out_gate_eps", ctypes.c_float),
        ("state_slots", _vp), ("n_slots", ctypes.c_int),
    ]


class ConvArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int), ("T", ctypes.c_int), ("H", ctypes.c_int), ("D", ctypes.c_int), ("W", ctypes.c_int),
        ("cu_seqlens", _vp), ("N", ctypes.c_int),
        ("x_dtype", ctypes.c_int),
        ("x_qkv", _vp), ("conv_w", _vp), ("conv_state", _vp),
        ("y_dtype", ctypes.c_int),
        ("q", _vp), ("k", _vp), ("v", _vp),
        ("stream", _vp),
    ]


class GateArgs(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int), ("H", ctypes.c_int), ("V", ctypes.c_int),
        ("o_dtype", ctypes.c_int), ("g_dtype", ctypes.c_int),
        ("eps", ctypes.c_float),
        ("o", _vp), ("g", _vp), ("y", _vp),
        ("stream", _vp),
    ]


# Every symbol include/kda.h declares.
EXPORTS = ["kda_chunk_fwd", "kda_chunk_fwd_noalloc", "kda_chunk_fwd_stage", "kda_chunk_fwd_workspace", "kda_chunk_bwd",
           "kda_chunk_bwd_stage", "kda_chunk_bwd_stages", "kda_chunk_bwd_workspace", "kda_recurrent_step",
           "kda_conv_prefill", "kda_output_gate", "kda_output_gate_bwd", "kda_status_string", "kda_version"]

_lib = None


def load(path: str = LIB_PATH):
    """Load libkda.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m kimi_delta_attention_amd.build` "
                           "(the KDA operators have no fallback path)")
    lib = ctypes.CDLL(path)
    CA = ctypes.POINTER(ChunkArgs)
    lib.kda_chunk_fwd.argtypes = [CA]
    lib.kda_chunk_fwd.restype = ctypes.c_int
    lib.kda_chunk_fwd_noalloc.argtypes = [CA]
    lib.kda_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.kda_chunk_fwd_stage.argtypes = [CA, ctypes.c_int]
    lib.kda_chunk_fwd_stage.restype = ctypes.c_int
    lib.kda_chunk_fwd_workspace.argtypes = [CA]
    lib.kda_chunk_fwd_workspace.restype = ctypes.c_size_t
    lib.kda_chunk_bwd.argtypes = [CA, ctypes.POINTER(ChunkGrads)]
    lib.kda_chunk_bwd.restype = ctypes.c_int
    lib.kda_chunk_bwd_stage.argtypes = [CA, ctypes.POINTER(ChunkGrads), ctypes.c_int]
    lib.kda_chunk_bwd_stage.restype = ctypes.c_int
    lib.kda_chunk_bwd_stages.argtypes = []
    lib.kda_chunk_bwd_stages.restype = ctypes.c_int
    lib.kda_chunk_bwd_workspace.argtypes = [CA]
    lib.kda_chunk_bwd_workspace.restype = ctypes.c_size_t
    lib.kda_recurrent_step.argtypes = [ctypes.POINTER(StepArgs)]
    lib.kda_recurrent_step.restype = ctypes.c_int
    lib.kda_conv_prefill.argtypes = [ctypes.POINTER(ConvArgs)]
    lib.kda_conv_prefill.restype = ctypes.c_int
    lib.kda_output_gate.argtypes = [ctypes.POINTER(GateArgs)]
    lib.kda_output_gate.restype = ctypes.c_int
    lib.kda_output_gate_bwd.argtypes = [ctypes.POINTER(GateArgs), _vp, _vp, _vp]
    lib.kda_output_gate_bwd.restype = ctypes.c_int
    lib.kda_status_string.argtypes = [ctypes.c_int]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_version.argtypes = []
    lib.kda_version.restype = ctypes.c_int
    _lib = lib
    return lib


class KDAError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {load().kda_status_string(status).decode()} (status {status})")


def check(status: int, what: str):
    if status == KDA_OK:
        return
    if status in (KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_MISSING_PARAM, KDA_ERR_WORKSPACE):
        err = KDAError(status, what)
        raise ValueError(str(err))
    raise KDAError(status, what)
