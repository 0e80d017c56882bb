"""Shared test helpers: device transfer and the output comparison rule.

Comparison of attention outputs (bf16 / fp16) with the oracle, given
identical quantized inputs:
  err = |o_kernel - o_oracle_rounded| over every valid element;
  pass iff mean(err) <= 2e-3 and every err <= 2e-2, except that where one
  output ulp at |o_oracle| is already larger than 2e-2 (|o| >= 4 for bf16,
  >= 32 for fp16) an element may instead be off by at most one ulp.
The ulp clause exists because there the absolute bound is finer than the
output format can represent; the literal max error is always reported.
"""
from __future__ import annotations

import numpy as np

MAX_ABS = 2e-2
MEAN_ABS = 2e-3
# lse (natural log) bound: 1e-3 absolute plus a relative term.  gfx950's fp8
# MFMA sums its 128 products with about 2^-12.7 relative precision (measured
# worst case 1.45e-4 of the sum of |products|), so logits -- and the lse of
# rows dominated by large logits -- carry a relative error of that order.
LSE_ABS = 1e-3
LSE_REL = 4e-4


def to_dev(x, torch_dtype=None):
    import torch
    if x.dtype == np.uint16 and torch_dtype is None:
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    elif x.dtype == np.uint8:
        t = torch.from_numpy(np.ascontiguousarray(x))
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    if torch_dtype is not None:
        t = t.view(torch_dtype)
    return t.cuda()


def from_dev_bits(t) -> np.ndarray:
    """A bf16 / fp16 tensor -> uint16 bit patterns on the host."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def dev_u8(t) -> np.ndarray:
    import torch
    return t.detach().view(torch.uint8).cpu().numpy()


def decode_out(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def ulp_at(x: np.ndarray, dtype: str) -> np.ndarray:
    frac, emin = (7, -126) if dtype == "bf16" else (10, -14)
    _, ex = np.frexp(np.abs(x))
    return np.exp2(np.maximum(ex - 1, emin) - frac).astype(np.float64)


def compare_outputs(got: np.ndarray, want_rounded: np.ndarray, want_exact: np.ndarray,
                    dtype: str, label: str = "") -> dict:
    """Apply the rule above; returns the statistics and raises AssertionError on failure."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - want_rounded)
    assert np.all(np.isfinite(got)), f"{label}: non-finite outputs"
    ulp = ulp_at(want_exact, dtype)
    big = err > MAX_ABS
    ulp_ok = (ulp > MAX_ABS) & (err <= ulp * (1 + 1e-12))
    stats = {
        "n": int(err.size), "max_abs": float(err.max(initial=0.0)), "mean_abs": float(err.mean()) if err.size else 0.0,
        "n_over_2e-2": int(big.sum()), "n_ulp_clause": int((big & ulp_ok).sum()),
        "max_ulps": float((err / ulp).max(initial=0.0)),
    }
    assert stats["mean_abs"] <= MEAN_ABS, f"{label}: mean abs err {stats}"
    assert not np.any(big & ~ulp_ok), f"{label}: max abs err {stats}"
    return stats


def compare_lse(got: np.ndarray, want: np.ndarray, label: str = "") -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)), f"{label}: lse finiteness differs"
    assert np.all(got[~fin] == want[~fin]), f"{label}: -inf rows differ"
    err = np.abs(got[fin] - want[fin])
    tol = LSE_ABS + LSE_REL * np.abs(want[fin])
    assert np.all(err <= tol), f"{label}: lse max err {err.max()} (worst ratio to bound {(err / tol).max():.3g})"
    return float(err.max(initial=0.0))
