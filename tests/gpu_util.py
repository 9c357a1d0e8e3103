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


def untile_codes(qs: np.ndarray, k: int) -> np.ndarray:
    """int8 codes [R, k] of R activation rows in the tiled layout (rows of NQ * 128 bytes)."""
    NQ = math.ceil(k / 128)
    R = qs.shape[0]
    a = np.asarray(qs).reshape(R, NQ, 4, 4, 8)                       # [r][q][g][j][e]
    codes = np.zeros((R, NQ * 4, 32), dtype=np.int8)
    for g in range(4):
        for e in range(8):
            codes[:, :, P[g, e]] = a[:, :, g, :, e].reshape(R, NQ * 4)
    return codes.reshape(R, NQ * 128)[:, :k]


def row_errors(gpu, ref):
    """(normwise, elementwise) relative errors per row: ||g - r||_2 / ||r||_2 and
    max_i |g_i - r_i| / max(|r_i|, rms(r))."""
    g2 = np.asarray(gpu, dtype=np.float64).reshape(-1, np.shape(gpu)[-1])
    r2 = np.asarray(ref, dtype=np.float64).reshape(-1, np.shape(ref)[-1])
    d = g2 - r2
    nrm = np.sqrt(np.sum(r2 * r2, axis=1))
    normwise = np.sqrt(np.sum(d * d, axis=1)) / np.where(nrm == 0, 1.0, nrm)
    rms = np.sqrt(np.mean(r2 * r2, axis=1, keepdims=True))
    scale = np.maximum(np.abs(r2), rms)
    elem = np.max(np.abs(d) / np.where(scale == 0, 1.0, scale), axis=1)
    return normwise, elem


def assert_close_rows(gpu, ref, rel=2e-3, what="", elem_rel=None):
    """Kernel-level bar: every element |g_i - r_i| <= rel * max(|r_i|, rms(row)).

    With ``elem_rel`` given (whole-step bar): per row ||g - r|| / ||r|| <= rel and every
    element within elem_rel * max(|r_i|, rms(row)).  Returns the worst normwise error."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    normwise, elem = row_errors(gpu, ref)
    if elem_rel is None:
        worst = float(elem.max()) if elem.size else 0.0
        assert worst <= rel, f"{what}: worst scaled error {worst:.3e} > {rel:.1e}"
        return worst
    say(f"  {what}: normwise max {normwise.max():.3e}, elementwise max {elem.max():.3e}")
    assert normwise.max() <= rel, f"{what}: normwise relative error {normwise.max():.3e} > {rel:.1e}"
    assert elem.max() <= elem_rel, f"{what}: elementwise scaled error {elem.max():.3e} > {elem_rel:.1e}"
    return float(normwise.max())
