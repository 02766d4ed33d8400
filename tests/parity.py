"""Shared helpers of the GPU parity tests (no method arithmetic here).

Tolerance form of the memra-engine kda_fixture_gpu.rs page (`check`): every
value finite, then max|got - want| <= TOL * max|want| with the scale floored
at 1e-6.  TOL is 1e-4 for the fp32 path and 2e-2 for bf16 inputs."""
import numpy as np
import torch

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def tol_for(dtype):
    return TOL_BF16 if dtype == torch.bfloat16 else TOL_F32


def check(name, got, want, tol):
    got = got.detach().float().cpu().double().numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{name}: shape {got.shape} vs {want.shape}"
    assert np.isfinite(got).all(), f"{name}: non-finite values in the GPU result"
    scale = max(float(np.abs(want).max()) if want.size else 0.0, 1e-6)
    md = float(np.abs(got - want).max()) if want.size else 0.0
    print(f"  {name}: rel {md / scale:.3e} (tol {tol:.0e})", flush=True)
    assert md <= tol * scale, f"{name}: maxdiff {md:.3e} scale {scale:.3e} rel {md / scale:.3e} tol {tol:.1e}"
    return md / scale


def dev(x, device="cuda"):
    return None if x is None else x.to(device).contiguous()


def nan_full(shape, dtype, device="cuda"):
    """An output buffer filled with NaN before a GPU call, so that any element
    the kernels fail to write fails the finiteness check."""
    return torch.full(tuple(shape), float("nan"), dtype=dtype, device=device)
