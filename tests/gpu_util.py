"""Helpers for GPU parity tests: case banners, tolerances and comparisons."""

from __future__ import annotations

import sys

import numpy as np
import torch

# bf16 gate: elementwise |gpu - ref| <= ATOL + RTOL*|ref| (the stated "2e-2
# abs and 1e-2 rel"), plus relative L2 <= REL_L2 per sequence so an output
# that collapses to zero cannot pass at long context, where |O| itself is
# below 2e-2.
BF16_ATOL = 2e-2
BF16_RTOL = 1e-2
BF16_REL_L2 = 1e-2
F32_ATOL = 1e-5
LSE_ATOL_BF16 = 1e-3
LSE_ATOL_F32 = 1e-5


def banner(*parts):
    """Name the case on stdout before its GPU step (flushed)."""
    print("CASE:", *parts, flush=True)
    sys.stdout.flush()


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def check_bf16(gpu: np.ndarray, ref: np.ndarray, what: str, rel_l2=True):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = np.abs(gpu - ref)
    bound = BF16_ATOL + BF16_RTOL * np.abs(ref)
    worst = float(np.max(err - bound))
    assert worst <= 0.0, (f"{what}: elementwise gate exceeded by {worst:.3e} "
                          f"(max abs err {float(err.max()):.3e})")
    if rel_l2:
        rl = float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))
        assert rl <= BF16_REL_L2, f"{what}: relative L2 {rl:.3e} > {BF16_REL_L2}"
        return rl
    return None


def check_f32(gpu, ref, what, atol=F32_ATOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, f"{what}: shape {gpu.shape} vs {ref.shape}"
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU output"
    err = float(np.max(np.abs(gpu - ref)))
    assert err <= atol, f"{what}: max abs error {err:.3e} > {atol}"
    return err


def check_lse(gpu, ref, what, atol):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = float(np.max(np.abs(gpu - ref)))
    assert err <= atol, f"{what}: lse max abs error {err:.3e} > {atol}"
    return err
