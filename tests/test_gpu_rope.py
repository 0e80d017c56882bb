"""GPU parity of attn_append_kv_rope: rotated Q/K, cache bytes and fused amax bit-exact."""
import numpy as np
import pytest

import gen
from oracle.rope import append_kv_rope
from oracle.quant import quant_fp8_per_head
from tests.parity import to_dev, from_dev_bits, dev_u8

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _case(seed, lens, before, hq, hkv, d, ps, dtype="bf16"):
    x = gen.long_prefill_inputs(seed, lens, hq, hkv, d, ps, outlier_p=0.001, kv_len_before=before,
                                spare_frac=0.25)
    if dtype == "fp16":
        for n in ("q", "k", "v"):
            x[n] = (x[n].astype(np.uint32) << 16).view(np.float32).astype(np.float16).view(np.uint16)
    return x


def _run(x, kc_np, vc_np, dtype):
    import paged_kv_amd as pk
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
    q, k, v = (to_dev(x[n], tdt) for n in ("q", "k", "v"))
    kc, vc = to_dev(kc_np, tdt), to_dev(vc_np, tdt)
    hq, hkv, d = x["hq"], x["hkv"], x["d"]
    amax = [torch.full((h,), -1.0, dtype=torch.float32, device="cuda") for h in (hq, hkv, hkv)]
    cs = x["rope_cos_sin"]
    pk.attn_append_kv_rope(q, k, v, pk.BF16 if dtype == "bf16" else pk.FP16, to_dev(x["cu_seqlens"]),
                           to_dev(x["kv_len_before"]), len(x["seqlens"]), q.shape[0], hq, hkv, d,
                           to_dev(cs), cs.shape[0], kc, vc, to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                           kc.shape[0], x["page_size"], *amax)
    torch.cuda.synchronize()
    return (from_dev_bits(q), from_dev_bits(k), from_dev_bits(kc), from_dev_bits(vc),
            *[a.cpu().numpy() for a in amax])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("lens,before,ps", [([37, 64], [0, 0], 16), ([5, 100, 1], [3, 0, 70], 64),
                                            ([300], [17], 32)])
def test_append_rope_bit_exact(dtype, lens, before, ps):
    hq, hkv, d = 8, 2, 128
    x = _case(21, lens, before, hq, hkv, d, ps, dtype)
    pool = x["num_pages"]
    kc = np.full((pool, ps, hkv, d), 0x7FC0, np.uint16)
    vc = kc.copy()
    got = _run(x, kc, vc, dtype)
    ref = append_kv_rope(x["q"] if dtype == "bf16" else x["q"].view(np.float16),
                         x["k"] if dtype == "bf16" else x["k"].view(np.float16),
                         x["v"] if dtype == "bf16" else x["v"].view(np.float16), dtype,
                         x["cu_seqlens"], x["kv_len_before"], x["rope_cos_sin"],
                         kc if dtype == "bf16" else kc.view(np.float16),
                         vc if dtype == "bf16" else vc.view(np.float16),
                         x["kv_indptr"], x["kv_indices"], ps)
    for i, name in enumerate(["q", "k", "k_cache", "v_cache"]):
        assert np.array_equal(got[i], np.asarray(ref[i]).view(np.uint16)), name
    for i, name in enumerate(["amax_q", "amax_k", "amax_v"]):
        assert np.array_equal(got[4 + i].view(np.uint32), ref[4 + i].view(np.uint32)), name


def test_fused_amax_feeds_fp8_quant():
    """append -> quant_qk(amax_in) gives the same codes as quant_qk's own reduction."""
    import paged_kv_amd as pk
    x = _case(3, [257, 64], [0, 5], 4, 4, 128, 64)
    kc = np.zeros((x["num_pages"], 64, 4, 128), np.uint16)
    q, k, _, _, aq, ak, av = _run(x, kc, kc.copy(), "bf16")
    for arr, am in ((q, aq), (k, ak)):
        dq = to_dev(arr)
        codes = torch.empty(dq.shape, dtype=torch.uint8, device="cuda")
        sc = torch.empty(4, dtype=torch.float32, device="cuda")
        pk.attn_quant_qk(dq, pk.BF16, None, 2, 0, dq.shape[0], 4, 128, pk.Q_FP8_PER_HEAD, 128,
                         to_dev(am), codes, sc)
        torch.cuda.synchronize()
        rc, rd = quant_fp8_per_head(arr, "bf16")
        assert np.array_equal(sc.cpu().numpy().view(np.uint32), rd.view(np.uint32))
        assert np.array_equal(dev_u8(codes), rc)


def test_chunked_append_equals_one_shot_on_gpu():
    hq, hkv, d, ps = 4, 2, 64, 16
    x = _case(8, [40], [0], hq, hkv, d, ps)
    pool = x["num_pages"]
    kc = np.full((pool, ps, hkv, d), 0x7FC0, np.uint16)
    one = _run(x, kc, kc.copy(), "bf16")
    a = dict(x)
    a.update(q=x["q"][:15], k=x["k"][:15], v=x["v"][:15], cu_seqlens=np.array([0, 15], np.int32),
             kv_len_before=np.array([0], np.int32), seqlens=np.array([15]))
    ra = _run(a, kc, kc.copy(), "bf16")
    b = dict(x)
    b.update(q=x["q"][15:], k=x["k"][15:], v=x["v"][15:], cu_seqlens=np.array([0, 25], np.int32),
             kv_len_before=np.array([15], np.int32), seqlens=np.array([25]))
    rb = _run(b, ra[2], ra[3], "bf16")
    assert np.array_equal(rb[2], one[2]) and np.array_equal(rb[3], one[3])
    assert np.array_equal(np.concatenate([ra[0], rb[0]]), one[0])
