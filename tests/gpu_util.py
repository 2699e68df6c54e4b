"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as O


def say(*a):
    """Print and flush, so that a GPU run names its case before each step."""
    print(*a, flush=True)
    sys.stdout.flush()


def host(t) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def rel_rms_err(got, want) -> tuple[float, float]:
    """(max |got - want| / rms(want), rms(want))."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(w * w)))
    if rms == 0.0:
        return float(np.max(np.abs(g - w))) if g.size else 0.0, 0.0
    return float(np.max(np.abs(g - w)) / rms) if g.size else 0.0, rms


def assert_rel(got, want, rtol, what=""):
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    den = np.maximum(np.abs(w), 1e-30)
    err = float(np.max(np.abs(g - w) / den)) if g.size else 0.0
    assert err <= rtol, f"{what}: max relative error {err:.3e} > {rtol:.1e}"
    return err


def bf16_floor(y_ref) -> float:
    """Rounding floor: max |bf16(y) - y| / rms(y) of the oracle's own output."""
    return rel_rms_err(O.bf16_round(y_ref), y_ref)[0]


def err_beyond_bf16_output(got, want) -> float:
    """max over elements of (|got - want| - half a bf16 ulp of got) / rms(want),
    floored at 0: the error of a bf16 output beyond its own final rounding.
    A bf16 value y = bf16_RNE(s) of an exact-arithmetic-free sum s satisfies
    |y - s| <= 2^(floor(log2 |y|) - 8), so this bounds |s - want| / rms, the
    arithmetic error before the output is rounded."""
    g = np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    rms = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
    a = np.abs(g)
    half = np.where(a >= 2.0 ** -126, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -126))) - 8), 2.0 ** -134)
    half = np.where(a == 0, 0.0, half)
    beyond = np.maximum(np.abs(g - w) - half, 0.0)
    if not g.size:
        return 0.0
    return float(beyond.max() / rms) if rms > 0 else float(beyond.max())


def sample_tokens(T: int, n: int, seed: int = 0) -> np.ndarray:
    if n >= T:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(T, n, replace=False))
