"""Helpers for the GPU parity tests (host <-> device marshalling and metrics)."""
import sys

import numpy as np

from oracle import bf16_bits_to_f64

# Tolerances for bf16 outputs against the unrounded fp64 oracle.
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def log(msg: str) -> None:
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def device():
    import torch
    return torch.device("cuda:0")


def to_dev(arr: np.ndarray):
    """Host array -> device tensor.  uint16 arrays become bf16 tensors (same bits)."""
    import torch
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device()).view(torch.bfloat16)
    return torch.from_numpy(a).to(device())


def bits(t) -> np.ndarray:
    """Device bf16 tensor -> host uint16 bit patterns."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def compare(gpu_bits: np.ndarray, ref: np.ndarray, name: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    got = bf16_bits_to_f64(gpu_bits)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite GPU output"
    err = np.abs(got - ref)
    mx, mn = float(err.max()), float(err.mean())
    rel_l2 = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    log(f"{name}: max_abs={mx:.3e} mean_abs={mn:.3e} rel_l2={rel_l2:.3e}")
    assert mx <= max_abs, f"{name}: max abs err {mx} > {max_abs}"
    assert mn <= mean_abs, f"{name}: mean abs err {mn} > {mean_abs}"
    return mx, mn, rel_l2
