"""Number formats of the path, in fp64 numpy (oracle: test infrastructure only).

FP8 is OCP E4M3 "fn" (the aiter page's fp8 Q/K/V; the Ascend page's
FLOAT8_E4M3): exponent bias 7, 3 mantissa bits, no infinities, S.1111.111 is
NaN, the largest finite magnitude is 448 (S.1111.110), subnormals are
m * 2^-9.  The descale convention amax/448 used with these codes only fits
the "fn" variant (the "fnuz" variant tops out at 240).

Reading taken where the pages are silent (quantizer arithmetic): the value
to encode is v = fp32(x) / fp32(scale) (one IEEE fp32 division); NaN encodes
as 0x7F; |v| is clamped to 448; rounding is to nearest, ties to even, on the
e4m3 grid; the sign is kept, so a negative value that rounds to zero gives
0x80.  INT8 codes are rint(v) (ties to even) clamped to [-127, 127].

Outputs of the attention steps are bf16 or fp16, rounded once, to nearest
even, directly from the fp64 result.

Pins (tests/test_oracle_numerics.py): closed-form codes; agreement with
torch's float8_e4m3fn cast on clamped inputs (a library routine); a
nearest-grid-point search over all 256 codes (oracle.brute); torch's
bf16 / fp16 casts on fp32 inputs; hand-placed ties between grid points.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN = 0x7F


def e4m3fn_decode_table() -> np.ndarray:
    """fp64 value of each of the 256 codes (NaN for 0x7F / 0xFF)."""
    c = np.arange(256)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * mag
    val[(c & 0x7F) == 0x7F] = np.nan
    return val


_E4M3_TABLE = e4m3fn_decode_table()


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3fn_encode(v32: np.ndarray) -> np.ndarray:
    """Encode fp32 values (already divided by their scale) as e4m3fn codes."""
    v32 = np.asarray(v32, dtype=np.float32)
    nan = np.isnan(v32)
    neg = np.signbit(v32)
    a = np.minimum(np.abs(v32.astype(np.float64)), E4M3_MAX)
    a = np.where(nan, 0.0, a)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e_unb = np.maximum(ex - 1, -6)           # binade; below 2^-6 the quantum is fixed
    quantum = np.exp2((e_unb - 3).astype(np.float64))
    r = np.rint(a / quantum) * quantum        # exact scaling; rint = ties to even
    # encode the rounded magnitude r (0 <= r <= 448, on the grid)
    _, ex2 = np.frexp(r)
    e2 = ex2 - 1
    sub = r < 2.0 ** -6
    exp_field = np.where(sub, 0, e2 + 7)
    mant = np.where(sub, r / 2.0 ** -9, (r / np.exp2(e2.astype(np.float64)) - 1.0) * 8.0)
    code = (exp_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(r == 0, 0, code)
    code = code | np.where(neg, 0x80, 0)
    code = np.where(nan, E4M3_NAN, code)
    return code.astype(np.uint8)


def int8_encode(v32: np.ndarray) -> np.ndarray:
    """rint (ties to even) of fp32 values, clamped to [-127, 127]."""
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    return np.clip(np.rint(v), -127, 127).astype(np.int8)


def _round_binary(x: np.ndarray, frac_bits: int, emin: int, max_finite: float) -> np.ndarray:
    """Round fp64 values to a binary format with ``frac_bits`` fraction bits
    and minimum normal exponent ``emin`` (ties to even); overflow -> inf."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    fin = np.isfinite(a)
    a0 = np.where(fin, a, 0.0)
    _, ex = np.frexp(a0)
    e = np.maximum(ex - 1, emin)
    q = np.exp2((e - frac_bits).astype(np.float64))
    r = np.rint(a0 / q) * q
    r = np.where(r > max_finite, np.inf, r)
    r = np.where(fin, r, a)
    return np.copysign(r, x)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 value (ties to even), returned as fp64."""
    return _round_binary(x, 7, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127)


def round_fp16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest fp16 value (ties to even), returned as fp64."""
    return _round_binary(x, 10, -14, 65504.0)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns (uint16), one rounding from fp64."""
    r = round_bf16(x).astype(np.float32)      # exact: r is on the bf16 grid
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def to_fp16(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp16 array, one rounding from fp64."""
    return round_fp16(x).astype(np.float16)   # exact: r is on the fp16 grid


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)
