"""Helpers shared by the GPU parity tests: layout marshalling and error metrics."""
import math
import sys

import numpy as np
import torch


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_nthwc(x_ncthw: torch.Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    """[1, C, T, H, W] CPU tensor -> [1, T, H, W, C] contiguous device tensor (marshalled on the CPU)."""
    return x_ncthw.permute(0, 2, 3, 4, 1).contiguous().to(dtype).to("cuda")


def from_dev_nthwc(y: torch.Tensor) -> np.ndarray:
    """[1, T, H, W, C] device tensor -> [C, T, H, W] float32 numpy."""
    return y[0].float().cpu().permute(3, 0, 1, 2).contiguous().numpy()


def rel_max(got: np.ndarray, ref: np.ndarray) -> float:
    """Normwise max relative error: max|got - ref| / max|ref|."""
    return float(np.abs(got.astype(np.float64) - ref).max() / max(np.abs(ref).max(), 1e-30))


def psnr(got: np.ndarray, ref: np.ndarray) -> float:
    """10 log10(R^2 / MSE) with R the reference's range (max - min), MSE in double."""
    ref = ref.astype(np.float64)
    mse = float(((got.astype(np.float64) - ref) ** 2).mean())
    rng = float(ref.max() - ref.min())
    return math.inf if mse == 0 else 10.0 * math.log10(rng * rng / mse)


def bf16_elementwise_ok(got: np.ndarray, ref: np.ndarray, ulps: float = 2.0, floor: float = 1e-4):
    """|got - ref| <= ulps * 2^-9 * |ref| + floor * max|ref|: one bf16 rounding of the result (half
    an ulp, 2^-9 relative), with a margin for a rounding flipped by fp32 summation order, plus a
    floor for the fp32 accumulation error of long sums. Returns (ok, worst ratio)."""
    ref64 = ref.astype(np.float64)
    bound = ulps * 2.0 ** -9 * np.abs(ref64) + floor * np.abs(ref64).max()
    ratio = np.abs(got.astype(np.float64) - ref64) / bound
    return bool((ratio <= 1.0).all()), float(ratio.max())
