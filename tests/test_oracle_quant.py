"""Pins of oracle.quant: per-head FP8, per-block INT8, V transpose/permute (CPU)."""
import numpy as np
import pytest

import gen
from oracle import brute
from oracle.quant import (as_f32, quant_fp8_per_head, quant_fp8_per_channel, quant_int8_per_block,
                          v_permute, v_unpermute, perm_pi, s_pad, fp8_descale)
from oracle.numerics import e4m3fn_decode


def _tiny(seed, lens, h, d, dtype="bf16"):
    rng = np.random.default_rng(seed)
    t = int(sum(lens))
    x = (rng.standard_normal((t, h, d)) * 3).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    if dtype == "bf16":
        return gen.bf16_bits(x), cu
    return x.astype(np.float16), cu


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fp8_per_head_vs_brute(dtype):
    x, cu = _tiny(1, [3, 5, 1], 3, 8, dtype)
    codes, ds = quant_fp8_per_head(x, dtype)
    bc, bds = brute.quant_fp8_per_head(as_f32(x, dtype))
    assert np.array_equal(ds.view(np.uint32), bds.view(np.uint32))
    assert np.array_equal(codes, bc)


def test_fp8_descale_is_amax_over_448_and_zero_head():
    x, _ = _tiny(2, [4], 3, 8)
    x[:, 1, :] = 0                       # bf16 +0 everywhere in head 1
    codes, ds = quant_fp8_per_head(x, "bf16")
    a = np.abs(as_f32(x, "bf16"))
    for h in (0, 2):
        assert ds[h] == np.float32(a[:, h].max()) / np.float32(448)
        # the amax element encodes to the largest finite code
        assert np.abs(e4m3fn_decode(codes[:, h])).max() == 448.0
    assert ds[1] == 1.0 and not codes[:, 1].any()
    # a supplied amax gives the same result as the reduction
    c2, d2 = quant_fp8_per_head(x, "bf16", amax_in=a.max(axis=(0, 2)))
    assert np.array_equal(c2, codes) and np.array_equal(d2, ds)
    assert fp8_descale(np.array([0.0, 448.0]))[1] == 1.0


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fp8_per_channel_vs_brute(dtype):
    x, cu = _tiny(5, [3, 5, 0, 1], 2, 4, dtype)
    codes, ds = quant_fp8_per_channel(x, dtype, cu)
    bc, bds = brute.quant_fp8_per_channel(as_f32(x, dtype), cu)
    assert ds.shape == (4, 2, 4)
    assert np.array_equal(ds.view(np.uint32), bds.view(np.uint32))
    assert np.array_equal(codes, bc)
    assert (ds[2] == 1.0).all()                  # the empty sequence
    from oracle.attention import dequant_fp8_per_channel
    deq = dequant_fp8_per_channel(codes, ds, cu)
    seq_of = np.repeat(np.arange(4), np.diff(cu))
    for i, h, c in np.ndindex(*codes.shape):
        assert deq[i, h, c] == brute.e4m3fn_value(int(bc[i, h, c])) * float(bds[seq_of[i], h, c])


def test_fp8_per_channel_reduces_to_per_head_when_channel_maxima_agree():
    # one sequence whose channels of a head share one amax (token 0 holds
    # +-A in every channel): each channel descale is the head's, and so are the codes
    x, cu = _tiny(6, [40], 3, 8, "fp16")
    x32 = as_f32(x, "fp16")
    amax = np.abs(x32).max(axis=(0, 2)) * 2
    signs = np.where(np.arange(8) % 2 == 0, 1.0, -1.0)
    x = x32.copy()
    x[0] = amax[:, None] * signs[None, :]
    x = x.astype(np.float16)
    c1, d1 = quant_fp8_per_channel(x, "fp16", cu)
    c0, d0 = quant_fp8_per_head(x, "fp16")
    assert np.array_equal(d1[0], np.repeat(d0[:, None], 8, axis=1))
    assert np.array_equal(c1, c0)


def test_fp8_per_channel_keeps_a_small_channel_that_per_head_flushes():
    # head 0: channel 0 ~ 1000 N(0,1), channel 1 ~ 0.004 N(0,1).  With the
    # head's descale (about amax/448 = 8) channel 1 lands below half of
    # e4m3's smallest subnormal 2^-9 and mostly encodes to 0; with its own
    # descale every value is a normal e4m3 number (relative error <= 2^-4)
    # or a subnormal well below the channel's magnitude
    from oracle.attention import dequant_fp8_per_head, dequant_fp8_per_channel
    rng = np.random.default_rng(7)
    x = np.zeros((256, 1, 2), np.float32)
    x[:, 0, 0] = rng.standard_normal(256) * 1000
    x[:, 0, 1] = rng.standard_normal(256) * 0.004
    x = x.astype(np.float16)
    cu = np.array([0, 256], np.int32)
    v = as_f32(x, "fp16").astype(np.float64)[:, 0, 1]
    ph = dequant_fp8_per_head(*quant_fp8_per_head(x, "fp16"))[:, 0, 1]
    pc = dequant_fp8_per_channel(*quant_fp8_per_channel(x, "fp16", cu), cu)[:, 0, 1]
    assert (ph == 0).mean() > 0.5
    assert np.abs(ph - v).mean() > 0.5 * np.abs(v).mean()
    assert np.abs(pc - v).mean() < 2.0 ** -4 * np.abs(v).mean()


def test_int8_per_block_vs_brute():
    x, cu = _tiny(3, [5, 11, 0, 7], 2, 4, "fp16")
    codes, sc = quant_int8_per_block(x, "fp16", cu, max_seqlen=11, block_tokens=4)
    bc, bsc = brute.quant_int8_per_block(as_f32(x, "fp16"), cu, 4)
    assert np.array_equal(codes, bc)
    nblk = sc.shape[2]
    assert nblk == 3
    for b in range(4):
        L = cu[b + 1] - cu[b]
        for h in range(2):
            for j in range(nblk):
                if j * 4 < L:
                    assert sc[b, h, j] == bsc[(b, h, j)]
                else:
                    assert sc[b, h, j] == 0.0


def test_int8_blocks_restart_at_each_sequence():
    # one large value at token 2 of sequence 1 must only inflate that
    # sequence's block 0, whatever the global token index is
    lens = [6, 6]
    x = np.ones((12, 1, 2), np.float16)
    x[6 + 2, 0, 0] = 100
    cu = np.array([0, 6, 12], np.int32)
    _, sc = quant_int8_per_block(x, "fp16", cu, 6, block_tokens=4)
    assert sc[0, 0, 0] == np.float32(1) / np.float32(127)
    assert sc[0, 0, 1] == np.float32(1) / np.float32(127)
    assert sc[1, 0, 0] == np.float32(100) / np.float32(127)
    assert sc[1, 0, 1] == np.float32(1) / np.float32(127)


def test_pi_definition_and_bijection():
    p = perm_pi(np.arange(32))
    assert sorted(p.tolist()) == list(range(32))
    # lane group g of an operand reads stored positions 8g..8g+7, which hold
    # tokens 4g..4g+3 and 16+4g..16+4g+3
    for g in range(4):
        toks = [j for j in range(32) if 8 * g <= p[j] < 8 * g + 8]
        assert sorted(toks) == [4 * g + r for r in range(4)] + [16 + 4 * g + r for r in range(4)]
    assert p[0] == 0 and p[17] == 5 and p[4] == 8 and p[31] == 31 and p[16] == 4


@pytest.mark.parametrize("fp8", [False, True, "per_channel"])
def test_v_permute_inverse_and_padding(fp8):
    lens = [37, 64, 1]
    x, cu = _tiny(4, lens, 2, 8, "bf16")
    out, ds = v_permute(x, "bf16", cu, max(lens), fp8=bool(fp8), per_channel=fp8 == "per_channel")
    assert out.shape == (3, 2, 8, s_pad(64)) and s_pad(64) == 128
    rec = v_unpermute(out, lens)
    if fp8 == "per_channel":
        ref, d1 = quant_fp8_per_channel(x, "bf16", cu)
        assert np.array_equal(ds, d1) and ds.shape == (3, 2, 8)
    else:
        ref = quant_fp8_per_head(x, "bf16")[0] if fp8 else x
    for b in range(3):
        assert np.array_equal(rec[b], ref[cu[b]:cu[b + 1]])
    # explicit placement: token 17 of sequence 0, head 1, channel 3
    assert out[0, 1, 3, 5] == ref[17, 1, 3]
    assert out[1, 0, 2, 32 + 8] == ref[37 + 32 + 4, 0, 2]
    # padding is +0
    pos_of = (np.arange(128) // 32) * 32 + perm_pi(np.arange(128) % 32)
    for b, L in enumerate(lens):
        pad = np.setdiff1d(np.arange(128), pos_of[:L])
        assert not out[b][:, :, pad].any()


# ---------------------------------------------------------------------------
# K smoothing (per-sequence, per-channel mean subtracted before int8 quant)
# ---------------------------------------------------------------------------
def _sage_small(seed=31, lens=(300, 1, 0, 129)):
    return gen.sage_inputs(seed, list(lens), 4, 2, 64)


def test_channel_mean_vs_exact_rationals():
    from fractions import Fraction
    from oracle.quant import channel_mean_fp16
    x = _sage_small()
    k, cu = x["k"], x["cu_seqlens"]
    m = channel_mean_fp16(k, cu)
    rng = np.random.default_rng(0)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for h, c in zip(rng.integers(0, 2, 6), rng.integers(0, 64, 6)):
            if s1 == s0:
                assert m[b, h, c] == 0.0
                continue
            exact = sum(Fraction(float(v)) for v in k[s0:s1, h, c].astype(np.float64)) / (s1 - s0)
            got = Fraction(float(m[b, h, c]))
            # two roundings after an exact sum: within one fp32 ulp of the exact mean
            ulp = Fraction(float(np.spacing(np.float32(abs(float(exact)) or 1e-30))))
            assert abs(got - exact) <= ulp


def test_channel_mean_independent_of_token_order_and_exact_on_constants():
    from oracle.quant import channel_mean_fp16
    x = _sage_small(32, (257,))
    k, cu = x["k"], x["cu_seqlens"]
    perm = np.random.default_rng(1).permutation(257)
    assert np.array_equal(channel_mean_fp16(k, cu).view(np.uint32), channel_mean_fp16(k[perm], cu).view(np.uint32))
    const = np.full((5, 1, 64), np.float16(-3.140625), np.float16)
    assert np.all(channel_mean_fp16(const, np.array([0, 5], np.int32)) == np.float32(-3.140625))


def test_smoothing_shrinks_int8_error_with_channel_offsets():
    from oracle.quant import smooth_quant_k
    from oracle.attention import dequant_int8_per_block
    x = gen.sage_inputs(33, [700, 400], 4, 2, 128, offset_frac=0.05, offset_sd=4.0)
    k, cu = x["k"], x["cu_seqlens"]
    k32 = as_f32(k, "fp16").astype(np.float64)
    c0, s0 = quant_int8_per_block(k, "fp16", cu, 700)
    c1, s1, mean = smooth_quant_k(k, cu, 700)
    e0 = np.abs(dequant_int8_per_block(c0, s0, cu) - k32).mean()
    back = dequant_int8_per_block(c1, s1, cu)
    for b in range(2):
        back[cu[b]:cu[b + 1]] += mean[b][None].astype(np.float64)
    e1 = np.abs(back - k32).mean()
    assert e1 < 0.8 * e0, (e0, e1)
