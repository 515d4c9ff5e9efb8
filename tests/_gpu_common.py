"""Shared helpers for the GPU parity tests (tolerances, transfers, printing)."""
import sys

import numpy as np
import torch

# Tolerances for outputs compared with the float64 oracle.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
FP32_MAX_ABS = 1e-5
# LSE (natural log): the row's top scores carry the 16-bit operand rounding
# directly; same absolute bound as the outputs.
BF16_LSE_ABS = 2e-2
FP32_LSE_ABS = 1e-5


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(a: np.ndarray, dtype=torch.bfloat16) -> torch.Tensor:
    """Host float32 array (bf16-exact when dtype is bf16) -> contiguous device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(dtype).cuda().contiguous()


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def errs(gpu: np.ndarray, ref: np.ndarray):
    d = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    return float(d.max()), float(d.mean())


def assert_bf16_close(gpu, ref, what=""):
    mx, mn = errs(gpu, ref)
    note(f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert mx <= BF16_MAX_ABS and mn <= BF16_MEAN_ABS, (what, mx, mn)


def assert_f32_close(gpu, ref, what="", tol=FP32_MAX_ABS):
    mx, mn = errs(gpu, ref)
    note(f"{what}: max-abs {mx:.3e} mean-abs {mn:.3e}")
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite output"
    assert mx <= tol, (what, mx, mn)
