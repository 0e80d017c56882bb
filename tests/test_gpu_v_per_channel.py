"""GPU parity of fp8 V with one descale per (sequence, kv head, channel)
through the C ABI: descales and codes (1-byte and fp16-valued) bit-exact
against the oracle, and the prefill with per-channel V within the comparison
rule -- int8 per-block Q/K (Q quantized inside the prefill, K plain or
smoothed) and fp8 per-head Q/K, with V as codes and as their fp16 values."""
import math

import numpy as np
import pytest

import gen
from oracle.attention import (dequant_fp8_per_channel, dequant_fp8_per_head, dequant_int8_per_block,
                              prefill_varlen)
from oracle.numerics import e4m3fn_decode, to_fp16
from oracle.quant import (as_f32, quant_fp8_per_channel, quant_fp8_per_head, quant_int8_per_block,
                          smooth_quant_k, v_permute, s_pad)
from tests.parity import to_dev, from_dev_bits, dev_u8, decode_out, compare_outputs, compare_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _v_channels(seed, lens, h, d, dtype, extreme=True):
    """V whose channels differ in magnitude by up to ~e^12 (the largest of
    a head N(0,1)), one all-zero channel and, with extreme, one token holding
    the format's largest finite value."""
    rng = np.random.default_rng(seed)
    t = int(sum(lens))
    x = rng.standard_normal((t, h, d)).astype(np.float32)
    f = np.exp(rng.normal(0.0, 2.0, size=(1, h, d)))
    x *= (f / f.max(axis=2, keepdims=True)).astype(np.float32)
    x[:, 0, 1] = 0.0
    if t and extreme:
        x[t // 2, h - 1, d - 1] = 65504.0 if dtype == "fp16" else 3.0e38
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    if dtype == "bf16":
        return gen.bf16_bits(x), cu
    return np.clip(x, -65504, 65504).astype(np.float16), cu


@pytest.mark.parametrize("wide", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("lens", [[300, 1, 0, 129], [1100]])
def test_v_permute_per_channel_bit_exact(lens, dtype, d, wide):
    import paged_kv_amd as A
    h = 3
    v, cu = _v_channels(91, lens, h, d, dtype)
    mx = max(lens)
    b, sp = len(lens), s_pad(mx)
    out = torch.empty((b, h, d, sp), dtype=torch.float16 if wide else torch.uint8, device="cuda")
    ds = torch.empty((b, h, d), dtype=torch.float32, device="cuda")
    out.fill_(7) if not wide else out.fill_(1.0)   # every position must be written
    A.attn_quant_v_permute(to_dev(v), A.BF16 if dtype == "bf16" else A.FP16, to_dev(cu), b, mx, int(cu[-1]), h, d,
                           A.Q_FP8_PER_CHANNEL_WIDE if wide else A.Q_FP8_PER_CHANNEL, None, out, ds)
    torch.cuda.synchronize()
    ref, rds = v_permute(v, dtype, cu, mx, fp8=True, per_channel=True)
    assert np.array_equal(ds.cpu().numpy().view(np.uint32), rds.view(np.uint32))
    if wide:
        assert np.array_equal(from_dev_bits(out), to_fp16(e4m3fn_decode(ref)).view(np.uint16))
    else:
        assert np.array_equal(dev_u8(out), ref)


def _ref_out(qd, kd, vd, cu, sm, causal, dtype):
    return prefill_varlen(qd, kd, vd, cu, cu, sm, causal, dtype)


@pytest.mark.parametrize("smooth", [False, True])
@pytest.mark.parametrize("causal", [True, False])
def test_sage_prefill_with_per_channel_v(causal, smooth):
    from paged_kv_amd.pipeline import SagePrefill
    x = gen.sage_inputs(92, [700, 129, 1, 0, 64], 8, 2, 128, offset_frac=0.05, offset_sd=4.0, v_channel_sd=2.0)
    cu = x["cu_seqlens"]
    mx = int(np.diff(cu).max())
    sm = 128 ** -0.5
    p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), mx, sm, causal=causal,
                    want_lse=True, smooth_k=smooth, v_fp8_per_channel=True)
    p.run()
    torch.cuda.synchronize()
    vc, vs = quant_fp8_per_channel(x["v"], "fp16", cu)
    assert np.array_equal(p.vs.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    vperm, _ = v_permute(x["v"], "fp16", cu, mx, fp8=True, per_channel=True)
    assert np.array_equal(from_dev_bits(p.vp), to_fp16(e4m3fn_decode(vperm)).view(np.uint16))
    qc, qs = quant_int8_per_block(x["q"], "fp16", cu, mx)
    if smooth:
        kc, ks, _ = smooth_quant_k(x["k"], cu, mx)
    else:
        kc, ks = quant_int8_per_block(x["k"], "fp16", cu, mx)
    ref = _ref_out(dequant_int8_per_block(qc, qs, cu), dequant_int8_per_block(kc, ks, cu),
                   dequant_fp8_per_channel(vc, vs, cu), cu, sm, causal, "fp16")
    label = f"sage v-chan causal={causal} smooth={smooth}"
    compare_outputs(decode_out(from_dev_bits(p.o), "fp16"), ref["o"], ref["o_exact"], "fp16", label)
    compare_lse(p.lse.cpu().numpy(), ref["lse"], label)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("qk", ["fp8", "int8_raw_q"])
def test_prefill_one_byte_v_per_channel(qk, d):
    """V as 1-byte e4m3fn codes with per-channel descales (the prefill widens
    them itself), under both Q/K forms."""
    import paged_kv_amd as A
    lens = [1, 0, 128, 129, 300]
    h, hkv = 4, 2
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    t, b, mx = int(cu[-1]), len(lens), max(lens)
    rng = np.random.default_rng(93)
    q32 = rng.standard_normal((t, h, d)).astype(np.float32)
    k32 = rng.standard_normal((t, hkv, d)).astype(np.float32)
    v, _ = _v_channels(94, lens, hkv, d, "fp16", extreme=False)
    sm = 1 / math.sqrt(d)
    dcu = to_dev(cu)
    vp = torch.empty((b, hkv, d, s_pad(mx)), dtype=torch.uint8, device="cuda")
    vs = torch.empty((b, hkv, d), dtype=torch.float32, device="cuda")
    A.attn_quant_v_permute(to_dev(v), A.FP16, dcu, b, mx, t, hkv, d, A.Q_FP8_PER_CHANNEL, None, vp, vs)
    o = torch.empty((t, h, d), dtype=torch.float16, device="cuda")
    lse = torch.empty((h, t), dtype=torch.float32, device="cuda")
    nblk = (mx + 127) // 128
    if qk == "fp8":
        q, k = q32.astype(np.float16), k32.astype(np.float16)
        qc, kc = torch.empty((t, h, d), dtype=torch.uint8, device="cuda"), torch.empty((t, hkv, d), dtype=torch.uint8, device="cuda")
        qs, ks = torch.empty(h, dtype=torch.float32, device="cuda"), torch.empty(hkv, dtype=torch.float32, device="cuda")
        A.attn_quant_qk(to_dev(q), A.FP16, dcu, b, mx, t, h, d, A.Q_FP8_PER_HEAD, 128, None, qc, qs)
        A.attn_quant_qk(to_dev(k), A.FP16, dcu, b, mx, t, hkv, d, A.Q_FP8_PER_HEAD, 128, None, kc, ks)
        A.attn_prefill_varlen(qc, kc, vp, A.FP8E4M3, A.FP8E4M3, qs, ks, vs, A.Q_FP8_PER_CHANNEL, A.Q_FP8_PER_HEAD,
                              dcu, dcu, b, mx, mx, t, t, h, hkv, d, sm, True, o, A.FP16, lse)
        rq, rqs = quant_fp8_per_head(q, "fp16")
        rk, rks = quant_fp8_per_head(k, "fp16")
        qd, kd = dequant_fp8_per_head(rq, rqs), dequant_fp8_per_head(rk, rks)
    else:
        q, k = q32.astype(np.float16), k32.astype(np.float16)
        kc = torch.empty((t, hkv, d), dtype=torch.int8, device="cuda")
        qs = torch.empty((b, h, nblk), dtype=torch.float32, device="cuda")
        ks = torch.empty((b, hkv, nblk), dtype=torch.float32, device="cuda")
        A.attn_quant_qk(to_dev(k), A.FP16, dcu, b, mx, t, hkv, d, A.Q_INT8_PER_BLOCK, 128, None, kc, ks)
        A.attn_prefill_varlen(to_dev(q), kc, vp, A.FP16, A.FP8E4M3, qs, ks, vs, A.Q_FP8_PER_CHANNEL,
                              A.Q_INT8_PER_BLOCK_RAW_Q, dcu, dcu, b, mx, mx, t, t, h, hkv, d, sm, True, o, A.FP16, lse)
        rq, rqs = quant_int8_per_block(q, "fp16", cu, mx)
        rk, rks = quant_int8_per_block(k, "fp16", cu, mx)
        qd, kd = dequant_int8_per_block(rq, rqs, cu), dequant_int8_per_block(rk, rks, cu)
    torch.cuda.synchronize()
    vc, rvs = quant_fp8_per_channel(v, "fp16", cu)
    assert np.array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32))
    ref = _ref_out(qd, kd, dequant_fp8_per_channel(vc, rvs, cu), cu, sm, True, "fp16")
    label = f"1-byte v-chan qk={qk} d={d}"
    compare_outputs(decode_out(from_dev_bits(o), "fp16"), ref["o"], ref["o_exact"], "fp16", label)
    compare_lse(lse.cpu().numpy(), ref["lse"], label)


def test_config2_per_channel_v_and_smoothing_sampled():
    """The SageAttention workload at full size with both refinements on:
    descales and smoothed K codes bit-exact everywhere, outputs on sampled
    rows of every sequence against the oracle."""
    from paged_kv_amd.pipeline import SagePrefill
    x = gen.config2()
    cu = x["cu_seqlens"]
    mx = int(np.diff(cu).max())
    sm = x["sm_scale"]
    p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), mx, sm, causal=True,
                    want_lse=True, smooth_k=True, v_fp8_per_channel=True)
    p.run()
    torch.cuda.synchronize()
    kc, ks, km = smooth_quant_k(x["k"], cu, mx)
    vc, vs = quant_fp8_per_channel(x["v"], "fp16", cu)
    assert np.array_equal(p.kc.cpu().numpy(), kc)
    assert np.array_equal(p.ks.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(p.vs.cpu().numpy().view(np.uint32), vs.view(np.uint32))
    qc, qs = quant_int8_per_block(x["q"], "fp16", cu, mx)
    got_all = decode_out(from_dev_bits(p.o), "fp16")
    lse_all = p.lse.cpu().numpy()
    rng = np.random.default_rng(5)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        one = np.array([0, L], np.int32)
        qd = dequant_int8_per_block(qc[s0:s1], qs[b:b + 1], one)
        kd = dequant_int8_per_block(kc[s0:s1], ks[b:b + 1], one)
        vd = dequant_fp8_per_channel(vc[s0:s1], vs[b:b + 1], one)
        idx = np.array(sorted({0, L - 1, 127, 128} | set(rng.integers(0, L, 10).tolist())))
        rows = [(0, h, idx) for h in rng.choice(32, 3, replace=False)]
        for (_, h, ii, o_ex, o_r, l) in prefill_varlen(qd, kd, vd, one, one, sm, True, "fp16", rows=rows):
            compare_outputs(got_all[s0 + ii, h], o_r, o_ex, "fp16", f"c2 refined b={b} h={h}")
            compare_lse(lse_all[h, s0 + ii], l, f"c2 refined b={b} h={h}")
