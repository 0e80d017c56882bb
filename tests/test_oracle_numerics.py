"""Pins of oracle.numerics: encoders and output rounding (CPU only)."""
import os

import numpy as np
import pytest
import torch

from oracle import brute
from oracle.numerics import (e4m3fn_decode, e4m3fn_encode, int8_encode, round_bf16,
                             round_fp16, to_bf16_bits, to_fp16, bf16_bits_to_f64)

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_closed_form.txt")


def _golden():
    out = []
    for line in open(GOLD):
        line = line.split("#")[0].strip()
        if not line:
            continue
        tok = line.split()
        v = float.fromhex(tok[0]) if "0x" in tok[0] else float(tok[0])
        out.append((v, int(tok[1], 16)))
    return out


def test_e4m3fn_closed_form_fixture():
    cases = _golden()
    assert len(cases) >= 15
    vals = np.array([v for v, _ in cases], np.float32)
    want = np.array([c for _, c in cases], np.uint8)
    got = e4m3fn_encode(vals)
    assert [hex(x) for x in got] == [hex(x) for x in want]
    # the scalar nearest-grid search agrees on every fixture line
    assert [brute.e4m3fn_encode_search(float(v)) for v in vals] == list(want)


def test_e4m3fn_nan():
    assert e4m3fn_encode(np.array([np.nan], np.float32))[0] == 0x7F
    assert np.isnan(e4m3fn_decode(np.array([0x7F, 0xFF])).astype(float)).all()


def test_e4m3fn_decode_table_against_bitfields():
    for c in range(256):
        a, b = e4m3fn_decode(np.array([c]))[0], brute.e4m3fn_value(c)
        assert (np.isnan(a) and np.isnan(b)) or a == b, c


def test_e4m3fn_roundtrip_all_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = e4m3fn_decode(codes).astype(np.float32)
    assert np.array_equal(e4m3fn_encode(vals), codes)


def _grid_midpoints():
    pos = np.unique(np.abs(e4m3fn_decode(np.arange(0x7F))))
    mids = (pos[1:] + pos[:-1]) / 2
    eps = np.array([-1, 0, 1], np.float64)
    pts = []
    for m in mids:
        m32 = np.float32(m)
        pts += [np.nextafter(m32, np.float32(-1)), m32, np.nextafter(m32, np.float32(1000))]
    del eps
    pts = np.array(pts, np.float32)
    return np.concatenate([pts, -pts, pos.astype(np.float32), -pos.astype(np.float32)])


def test_e4m3fn_vs_torch_cast_on_clamped_inputs():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.standard_normal(400_000).astype(np.float32) * np.float32(60),
        (rng.standard_normal(200_000) * 2.0 ** rng.integers(-14, 9, 200_000)).astype(np.float32),
        _grid_midpoints(),
    ])
    x = np.clip(x, -448, 448).astype(np.float32)
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = e4m3fn_encode(x)
    assert np.array_equal(ours, lib)


def test_e4m3fn_vs_exhaustive_search():
    rng = np.random.default_rng(6)
    x = np.concatenate([_grid_midpoints()[::3],
                        (rng.standard_normal(1500) * 2.0 ** rng.integers(-12, 9, 1500)).astype(np.float32),
                        np.array([600.0, -1e30, 1e-40, -1e-40], np.float32)])
    got = e4m3fn_encode(x)
    want = np.array([brute.e4m3fn_encode_search(float(v)) for v in x], np.uint8)
    assert np.array_equal(got, want)


def test_e4m3fn_half_ulp_bound():
    rng = np.random.default_rng(7)
    x = np.clip(rng.standard_normal(100_000) * 100, -448, 448).astype(np.float32)
    r = e4m3fn_decode(e4m3fn_encode(x))
    a = np.abs(x.astype(np.float64))
    _, ex = np.frexp(a)
    ulp = np.exp2(np.maximum(ex - 1, -6) - 3.0)
    assert np.all(np.abs(r - x) <= ulp / 2)


def test_int8_encode_ties_and_clamp():
    v = np.array([2.5, 3.5, -2.5, -3.5, 0.5, 1.5, 126.5, 127.4, 300.0, -300.0, -0.4], np.float32)
    assert list(int8_encode(v)) == [2, 4, -2, -4, 0, 2, 126, 127, 127, -127, 0]


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
def test_16bit_rounding_vs_torch(fmt):
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(300_000) * 2.0 ** rng.integers(-30, 20, 300_000)).astype(np.float32)
    if fmt == "fp16":
        x = x[np.abs(x) < 60000]
        lib = torch.from_numpy(x).to(torch.float16).numpy()
        ours = to_fp16(x.astype(np.float64))
        assert np.array_equal(ours.view(np.uint16), lib.view(np.uint16))
    else:
        lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        ours = to_bf16_bits(x.astype(np.float64))
        assert np.array_equal(ours, lib)


def test_16bit_ties_from_fp64():
    # exact midpoints (fp64) round to the even neighbour
    one = 1.0
    assert round_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0
    assert round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == one + 2 * 2.0 ** -7
    assert round_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == one + 2.0 ** -7
    assert round_fp16(np.array([one + 2.0 ** -11]))[0] == 1.0
    assert round_fp16(np.array([one + 3 * 2.0 ** -11]))[0] == one + 2 * 2.0 ** -10
    # single rounding from fp64: a value just above an fp32-representable tie
    # must not be double-rounded through fp32
    v = one + 2.0 ** -8 + 2.0 ** -30
    assert round_bf16(np.array([v]))[0] == one + 2.0 ** -7
    assert round_fp16(np.array([65519.0, 65520.0]))[1] == np.inf
    assert round_fp16(np.array([65519.0]))[0] == 65504.0
    assert round_fp16(np.array([2.0 ** -25, 3 * 2.0 ** -25]))[0] == 0.0
    assert round_fp16(np.array([3 * 2.0 ** -25]))[0] == 2 * 2.0 ** -24
    assert bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
