"""Helpers shared by the GPU parity tests: move synthetic inputs to the GPU and
compare with the oracle.  Imports torch lazily."""

import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def require_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    import gqa_attention_attn_amd as G
    G.lib()   # raises if the HIP library is not built: no fallback
    return torch


def dev(x, dtype, device="cuda"):
    """numpy float32 (bf16-exact for bf16) -> torch device tensor of dtype."""
    import torch
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(device=device).to(dtype)


def ints(x, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to(device)


def compare(got, ref, atol, what=""):
    """Element-wise |got - ref| <= atol; returns the max error (logged)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    log(f"  {what}: max|err| = {mx:.3e} (atol {atol:g}, n = {err.size})")
    assert mx <= atol, f"{what}: max abs error {mx} > {atol}"
    return mx
