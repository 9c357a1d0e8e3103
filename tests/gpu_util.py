"""Test-side helpers: layout decoding of the library's tiled buffers and the tolerance rule.

Nothing here computes any part of the decode step; it only reorders bytes to compare them.
"""
import math
import sys

import numpy as np
import pytest
import torch

# element index inside a block held by group g, slot e (P_g = {4g..4g+3, 4g+16..4g+19})
P = np.array([[4 * g + e if e < 4 else 4 * g + 16 + (e - 4) for e in range(8)] for g in range(4)])

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X")


def say(*a):
    """Print and flush (names the case before each GPU step)."""
    print(*a, flush=True)
    sys.stdout.flush()


def untile_act(qs: torch.Tensor, d: torch.Tensor, B: int, k: int):
    """Codes [B, k] (int8) and scales [B, k/32] of the tiled activation layout."""
    NQ = math.ceil(k / 128)
    a = qs.detach().cpu().numpy().reshape(B, NQ, 4, 4, 8)          # [b][q][g][j][e]
    codes = np.zeros((B, NQ * 4, 32), dtype=np.int8)
    for g in range(4):
        for e in range(8):
            codes[:, :, P[g, e]] = a[:, :, g, :, e].reshape(B, NQ * 4)
    sc = d.detach().cpu().numpy().reshape(B, NQ * 4)
    return codes.reshape(B, NQ * 128)[:, :k], sc[:, : k // 32], codes[:, k // 32:], sc[:, k // 32:]


def assert_close_rows(gpu, ref, rel=2e-3, what=""):
    """Per output row: |gpu - ref| <= rel * max(|ref_i|, rms(ref_row)) for every element."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    g2 = gpu.reshape(-1, gpu.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    scale = np.maximum(np.abs(r2), rms)
    err = np.abs(g2 - r2) / np.where(scale == 0, 1.0, scale)
    worst = float(err.max()) if err.size else 0.0
    assert np.all(np.isfinite(g2)), f"{what}: non-finite GPU values"
    assert worst <= rel, f"{what}: worst scaled error {worst:.3e} > {rel:.1e}"
    return worst
