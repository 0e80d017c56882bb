"""GPU parity of the prefill against a paged 16-bit cache through the C ABI:
the page gather bit-exact, the quantized inputs bit-exact, outputs within the
comparison rule against the oracle (pages read into the ragged layout, fp8
per-head quantization, the prefill with the chunk's queries aligned to the
end of their sequence's keys)."""
import numpy as np
import pytest

import gen
from oracle.attention import dequant_fp8_per_head, prefill_varlen, ragged_from_pages
from oracle.quant import quant_fp8_per_head
from tests.parity import to_dev, from_dev_bits, dev_u8, decode_out, compare_outputs, compare_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(x, causal=True):
    from paged_kv_amd.pipeline import PagedPrefill
    p = PagedPrefill(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["kv_indptr"]),
                     to_dev(x["kv_indices"]), to_dev(x["kv_last_page_len"]), to_dev(x["cu_q"]),
                     to_dev(x["cu_k"]), x["max_q"], x["max_k"], x["sm_scale"], causal=causal, want_lse=True)
    p.run()
    torch.cuda.synchronize()
    return p


def _refs(x):
    kg = ragged_from_pages(x["k_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_k"])
    vg = ragged_from_pages(x["v_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_k"])
    qc, qs = quant_fp8_per_head(x["q"], "bf16")
    kc, ks = quant_fp8_per_head(kg, "bf16")
    vc, vs = quant_fp8_per_head(vg, "bf16")
    return kg, vg, (qc, qs, kc, ks, vc, vs)


def _check(x, causal=True, label=""):
    p = _run(x, causal)
    kg, vg, (qc, qs, kc, ks, vc, vs) = _refs(x)
    assert np.array_equal(from_dev_bits(p.kg), kg) and np.array_equal(from_dev_bits(p.vg), vg)
    assert np.array_equal(dev_u8(p.qc), qc) and np.array_equal(dev_u8(p.kc), kc)
    for a, b in ((p.qs, qs), (p.ks, ks), (p.vs, vs)):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.view(np.uint32))
    ref = prefill_varlen(dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kc, ks),
                         dequant_fp8_per_head(vc, vs), x["cu_q"], x["cu_k"], x["sm_scale"], causal, "bf16")
    got = decode_out(from_dev_bits(p.o), "bf16")
    stats = compare_outputs(got, ref["o"], ref["o_exact"], "bf16", label)
    compare_lse(p.lse.cpu().numpy(), ref["lse"], label)
    return p, stats


@pytest.mark.parametrize("page_size", [16, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_paged_prefill_ragged(page_size, causal):
    # chunks of 1..300 queries against 0..700 cached tokens, a sequence with no
    # query, one whose chunk is its whole history, ragged last pages
    x = gen.paged_prefill_inputs(71, [700, 129, 64, 300, 1], [300, 0, 64, 1, 1], 4, 2, 128, page_size)
    x["sm_scale"] = 128 ** -0.5
    _check(x, causal, f"ps={page_size} causal={causal}")


def test_paged_prefill_d64_gqa():
    x = gen.paged_prefill_inputs(72, [257, 1000], [257, 130], 8, 1, 64, 32)
    x["sm_scale"] = 0.125
    _check(x, True, "d64 gqa 8:1")


def test_gather_zero_fills_rows_past_the_cache():
    from paged_kv_amd import api as A
    x = gen.paged_prefill_inputs(73, [40, 5], [1, 1], 1, 2, 64, 16)
    cu = np.array([0, 48, 60], np.int32)  # 8 and 7 rows more than cached
    out = torch.full((60, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    A.attn_gather_paged_kv(to_dev(x["k_cache"]), 2, to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                           to_dev(x["kv_last_page_len"]), to_dev(cu), 2, 48, x["num_pages"], 16, 2, 64, out)
    torch.cuda.synchronize()
    ref = ragged_from_pages(x["k_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], cu)
    assert np.array_equal(from_dev_bits(out), ref)


def test_gather_fp8_codes_unchanged():
    from paged_kv_amd import api as A
    x = gen.paged_decode_inputs(74, [33, 0, 100], 4, 2, 128, page_size=16)
    lens = x["kv_lens"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    out = torch.empty((int(cu[-1]), 2, 128), dtype=torch.uint8, device="cuda")
    A.attn_gather_paged_kv(to_dev(x["k_cache"]), 1, to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                           to_dev(x["kv_last_page_len"]), to_dev(cu), 3, int(lens.max()), x["num_pages"], 16,
                           2, 128, out)
    torch.cuda.synchronize()
    ref = ragged_from_pages(x["k_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], cu)
    assert np.array_equal(dev_u8(out), ref)


def test_paged_prefill_workload_sampled():
    """The chunked-prefill workload at full size (B=4, kv_len U{8192..24576},
    2048-query chunks, 32/8 heads, D=128, page 64): gathered caches and
    codes bit-exact, sampled output rows of 3 heads per sequence against the
    oracle, every output finite."""
    x = gen.paged_prefill_workload()
    p = _run(x)
    kg, vg, (qc, qs, kc, ks, vc, vs) = _refs(x)
    assert np.array_equal(from_dev_bits(p.kg), kg) and np.array_equal(from_dev_bits(p.vg), vg)
    assert np.array_equal(dev_u8(p.qc), qc) and np.array_equal(dev_u8(p.kc), kc)
    assert torch.isfinite(p.o.float()).all()
    got = decode_out(from_dev_bits(p.o), "bf16")
    lse = p.lse.cpu().numpy()
    qd, kd, vd = dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kc, ks), dequant_fp8_per_head(vc, vs)
    rng = np.random.default_rng(6)
    cu_q = x["cu_q"]
    rows = []
    for b in range(len(cu_q) - 1):
        L = int(cu_q[b + 1] - cu_q[b])
        idx = np.unique(np.concatenate([[0, L - 1, 127, 128], rng.integers(0, L, 8)]))
        for h in rng.choice(32, 3, replace=False):
            rows.append((b, int(h), idx))
    for (b, h, idx, o_ex, o_r, l) in prefill_varlen(qd, kd, vd, cu_q, x["cu_k"], x["sm_scale"], True, "bf16",
                                                   rows=rows):
        s0 = int(cu_q[b])
        compare_outputs(got[s0 + idx, h], o_r, o_ex, "bf16", f"paged b={b} h={h}")
        compare_lse(lse[h, s0 + idx], l, f"paged b={b} h={h}")
