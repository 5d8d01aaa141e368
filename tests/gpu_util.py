"""Helpers shared by the GPU parity tests (no method arithmetic here)."""

from __future__ import annotations

import sys

import numpy as np
import torch

TOL = 2e-2          # per-output bound: max|gpu - ref| <= TOL * max|ref|
LOSS_RTOL = 1e-3    # scalar-loss relative error bound


def dev(x):
    """numpy int array or synth.Bf16 -> cuda tensor with identical bits."""
    if hasattr(x, "bits"):
        return x.torch("cuda")
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(gpu - ref))) if ref.size else 0.0
    return err / scale if scale > 0 else err


def assert_close(gpu, ref, name, tol=TOL):
    gpu = np.asarray(gpu, np.float64)
    assert np.all(np.isfinite(gpu)), f"{name}: non-finite output"
    e = rel_err(gpu, ref)
    print(f"  {name}: max|err|/max|ref| = {e:.3e}", flush=True)
    assert e <= tol, f"{name}: max|err|/max|ref| = {e:.3e} > {tol}"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def padded(rows, cols, dtype, pad_rows=3, pad_cols=8, fill=None):
    """A cuda buffer with canary padding; returns (full, view)."""
    full = torch.empty((rows + pad_rows, cols + pad_cols), dtype=dtype, device="cuda")
    if fill is None:
        fill = 12345.0 if dtype == torch.float32 else -1024.0
    full.fill_(fill)
    return full, full[:rows, :cols]


def canary_intact(full, rows, cols, fill=None):
    if fill is None:
        fill = 12345.0 if full.dtype == torch.float32 else -1024.0
    f = full.float()
    return bool(torch.all(f[rows:, :] == fill)) and bool(torch.all(f[:, cols:] == fill))
