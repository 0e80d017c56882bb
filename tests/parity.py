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
# lse (natural log) bound: 1e-3 absolute plus a relative term.  The absolute
# part covers the fp16 rounding of the P that the row sums are taken over
# (at most 2^-12 relative in l, 2.4e-4 in ln l).  Every default path sums
# QK^T exactly up to fp32 accumulation (int8 MFMA; fp8 and int8 codes widened
# to fp16 / bf16 for f16 / bf16 MFMA), so its relative term only covers the
# fp32 roundings of m and ln 2 at very large logits: LSE_REL = 1e-5.
# The opt-in fp8-MFMA QK mode (ATTNQ_Q_FP8_PER_HEAD_MFMA8) does not sum its
# 128 products in full fp32: tests/test_gpu_mfma_accum.py measures the error
# of q . k against exact host sums and asserts it stays within 2^-11.5 of
# sum_d |q_d k_d|.  Its logits -- and the lse of rows dominated by large
# logits, where sum |q_d k_d| is close to |lse| -- carry a relative error of
# that order: LSE_REL_MFMA8 = 4e-4, that bound with a margin of 1.16.
LSE_ABS = 1e-3
LSE_REL = 1e-5
LSE_REL_MFMA8 = 4e-4


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


def compare_lse(got: np.ndarray, want: np.ndarray, label: str = "", rel: float = LSE_REL) -> float:
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    fin = np.isfinite(want)
    assert np.array_equal(fin, np.isfinite(got)), f"{label}: lse finiteness differs"
    assert np.all(got[~fin] == want[~fin]), f"{label}: -inf rows differ"
    err = np.abs(got[fin] - want[fin])
    tol = LSE_ABS + rel * np.abs(want[fin])
    assert np.all(err <= tol), f"{label}: lse max err {err.max()} (worst ratio to bound {(err / tol).max():.3g})"
    return float(err.max(initial=0.0))
