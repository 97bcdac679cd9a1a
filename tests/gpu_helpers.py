"""Glue for GPU parity tests: device tensors -> host arrays the oracle accepts, tolerance checks.

Nothing here computes any part of the layer.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from workloads import bf16_bits


def host(t: torch.Tensor) -> np.ndarray:
    """bf16 -> raw uint16 bits (the oracle decodes them exactly); other dtypes -> numpy."""
    if t.dtype == torch.bfloat16:
        return bf16_bits(t)
    return t.detach().cpu().numpy()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 value of a device tensor (bf16 via its bits)."""
    if t.dtype == torch.bfloat16:
        return (bf16_bits(t).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


class LazyExperts:
    """routed[e] -> (W_gate[e], W_up[e], W_down[e]) copied to the host on demand."""

    def __init__(self, wg, wu, wd):
        self.w = (wg, wu, wd)

    def __len__(self):
        return self.w[0].shape[0]

    def __getitem__(self, e):
        return tuple(host(w[e]) for w in self.w)


def max_rel(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max|gpu - ref| / max|ref| (the bf16 output gate)."""
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-300))


def frob_rel(gpu: np.ndarray, ref: np.ndarray) -> float:
    """||gpu - ref||_F / ||ref||_F (the FP8 output gate)."""
    return float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300))


def row_frob_max(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over rows r of ||gpu_r - ref_r|| / ||ref_r|| (a wrong or missing row fails it even
    where the whole-tensor norm would hide it)."""
    num = np.linalg.norm(gpu - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    return float(np.max(num / den)) if num.size else 0.0


def near_ties(s, bias, K: int, thr: float = 1e-6) -> np.ndarray:
    """Tokens whose selection or its order is decided by keys closer than thr.

    Sorted float64 keys s + b: any adjacent gap among the first K+1 below thr.
    """
    key = np.asarray(s, np.float64) + np.asarray(bias, np.float64)[None, :]
    top = -np.sort(-key, axis=1)[:, : K + 1]
    gaps = -np.diff(top, axis=1)
    return np.nonzero((gaps < thr).any(axis=1))[0]


def report(name: str, **vals):
    """One line of measured errors in the test log."""
    print(f"[parity] {name}: " + ", ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                          for k, v in vals.items()), file=sys.stderr, flush=True)
