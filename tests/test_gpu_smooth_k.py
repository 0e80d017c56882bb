"""GPU parity of SageAttention's K smoothing through the C ABI: per-channel
means, int8 codes and block scales of K - mean bit-exact against the oracle;
the prefill on smoothed K within the comparison rule; smoothing keeps the
output of the unquantized attention and brings the quantized output closer
to it on data with channel offsets."""
import numpy as np
import pytest

import gen
from oracle.attention import dequant_int8_per_block, prefill_varlen
from oracle.quant import quant_int8_per_block, smooth_quant_k, as_f32
from tests.parity import to_dev, from_dev_bits, decode_out, compare_outputs, compare_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _flow(x, smooth, causal=True):
    from paged_kv_amd.pipeline import SagePrefill
    cu = x["cu_seqlens"]
    mx = int(np.diff(cu).max())
    p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), mx, x["sm_scale"],
                    causal=causal, want_lse=True, smooth_k=smooth)
    p.run()
    torch.cuda.synchronize()
    return p, mx


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("lens", [[300, 1, 0, 129], [4096]])
def test_smooth_codes_scales_means_bit_exact(d, lens):
    x = gen.sage_inputs(81, lens, 8, 2, d, offset_frac=0.05, offset_sd=4.0)
    x["sm_scale"] = d ** -0.5
    p, mx = _flow(x, True)
    kc, ks, km = smooth_quant_k(x["k"], x["cu_seqlens"], mx)
    assert np.array_equal(p.kmean.cpu().numpy().view(np.uint32), km.view(np.uint32))
    assert np.array_equal(p.kc.cpu().numpy(), kc)
    assert np.array_equal(p.ks.cpu().numpy().view(np.uint32), ks.view(np.uint32))


@pytest.mark.parametrize("causal", [True, False])
def test_smooth_prefill_parity(causal):
    x = gen.sage_inputs(82, [700, 129, 64], 8, 2, 128, offset_frac=0.05, offset_sd=4.0)
    x["sm_scale"] = 128 ** -0.5
    p, mx = _flow(x, True, causal)
    cu = x["cu_seqlens"]
    qc, qs = quant_int8_per_block(x["q"], "fp16", cu, mx)
    kc, ks, km = smooth_quant_k(x["k"], cu, mx)
    ref = prefill_varlen(dequant_int8_per_block(qc, qs, cu), dequant_int8_per_block(kc, ks, cu),
                         as_f32(x["v"], "fp16").astype(np.float64), cu, cu, x["sm_scale"], causal, "fp16")
    got = decode_out(from_dev_bits(p.o), "fp16")
    compare_outputs(got, ref["o"], ref["o_exact"], "fp16", f"smooth causal={causal}")
    compare_lse(p.lse.cpu().numpy(), ref["lse"], f"smooth causal={causal}")


def test_smoothing_brings_the_output_closer_to_unquantized_attention():
    """The config-2 workload's own data (1% offset channels): mean error of
    the int8 flow against fp64 attention on the unquantized inputs, with and
    without smoothing, on sampled rows."""
    x = gen.config2()
    cu = x["cu_seqlens"]
    errs = {}
    for smooth in (False, True):
        p, mx = _flow(x, smooth)
        got = decode_out(from_dev_bits(p.o), "fp16")
        rng = np.random.default_rng(3)
        e = []
        for b in range(len(cu) - 1):
            s0, s1 = int(cu[b]), int(cu[b + 1])
            one = np.array([0, s1 - s0], np.int32)
            qd = as_f32(x["q"][s0:s1], "fp16").astype(np.float64)
            kd = as_f32(x["k"][s0:s1], "fp16").astype(np.float64)
            vd = as_f32(x["v"][s0:s1], "fp16").astype(np.float64)
            idx = np.unique(rng.integers(0, s1 - s0, 16))
            for h in (0, 13, 31):
                for (_, _, _, o_ex, _, _) in prefill_varlen(qd, kd, vd, one, one, x["sm_scale"], True, "fp16",
                                                             rows=[(0, h, idx)]):
                    e.append(np.abs(got[s0 + idx, h] - o_ex).mean())
        errs[smooth] = float(np.mean(e))
        del p
    print("mean |o - o_unquantized|: plain", errs[False], "smoothed", errs[True])
    assert errs[True] < errs[False]
