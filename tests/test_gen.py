"""Seeded generators: determinism and the structure the workloads need (CPU)."""
import numpy as np

import gen
from gen.configs import config2_lengths, config3_lengths


def _same(a, b):
    assert a.keys() == b.keys()
    for k in a:
        if isinstance(a[k], np.ndarray):
            assert np.array_equal(a[k], b[k]), k


def test_config1_deterministic_and_shaped():
    a, b = gen.config1(), gen.config1()
    _same(a, b)
    assert list(a["cu_seqlens"]) == [0, 37, 101]
    assert a["q"].shape == (101, 2, 64) and a["q"].dtype == np.uint16
    assert a["sm_scale"] == 0.125


def test_sage_offsets_structure():
    x = gen.sage_inputs(3, [40, 17], 4, 2, 32)
    assert x["q"].dtype == np.float16 and x["q"].shape == (57, 4, 32)
    assert len(x["q_offset_channels"]) == round(0.01 * 4 * 32)
    assert len(set(x["q_offset_channels"].tolist())) == len(x["q_offset_channels"])
    lens = config2_lengths()
    assert lens.size == 8 and lens.min() >= 512 and lens.max() <= 4096


def test_paged_decode_structure():
    x = gen.paged_decode_inputs(5, [5, 0, 33, 16], 4, 2, 8, page_size=16)
    ind, ptr = x["kv_indices"], x["kv_indptr"]
    assert list(np.diff(ptr)) == [1, 0, 3, 1]
    assert len(set(ind.tolist())) == ind.size and ind.max() < x["num_pages"]
    assert list(x["kv_last_page_len"]) == [5, 0, 1, 16]
    # slots past a sequence's end and spare pages hold NaN codes
    assert np.all(x["k_cache"][ind[0], 5:] == 0x7F)
    spare = np.setdiff1d(np.arange(x["num_pages"]), ind)
    assert spare.size > 0 and np.all(x["v_cache"][spare] == 0x7F)
    lens = config3_lengths()
    assert lens.size == 64 and lens.min() >= 1024 and lens.max() <= 32768


def test_sparse_mla_structure():
    x = gen.sparse_mla_inputs(7, 2, 1, 4, [100, 64], 16, 12, n_valid=10)
    idx = x["sparse_indices"]
    for b, L in enumerate([100, 64]):
        v = idx[b, 0, 0]
        assert np.all(v[:10] >= 0) and np.all(v[:10] < L) and len(set(v[:10].tolist())) == 10
        assert np.all(v[10:] == -1)
    rows = x["kv_cache"].reshape(-1, gen.MLA_ROW_BYTES)
    sel = set()
    for b in range(2):
        for i in idx[b, 0, 0, :10]:
            sel.add(int(x["block_table"][b][i // 16]) * 16 + int(i) % 16)
    other = np.array(sorted(set(range(rows.shape[0])) - sel))
    sc = rows[:, 640:656].copy().view(np.float32)
    assert np.all(np.isnan(sc[other])) and np.all(np.isfinite(sc[sorted(sel)]))
    assert np.all(sc[sorted(sel)] > 0)
    assert gen.MLA_ROW_BYTES == 656


def test_long_prefill_structure():
    x = gen.long_prefill_inputs(9, [100, 30], 4, 2, 16, 8, kv_len_before=[5, 0])
    assert x["rope_cos_sin"].shape[0] >= 105 and x["rope_cos_sin"].shape[1:] == (8, 2)
    assert list(np.diff(x["kv_indptr"])) == [14, 4]
    assert x["num_pages"] > 18
    # outliers: roughly 0.1% of elements are scaled by 20
    y = gen.prefill_fp8_inputs(1, [4000], 4, 4, 64, outlier_p=0.001)
    from oracle.numerics import bf16_bits_to_f32
    big = (np.abs(bf16_bits_to_f32(y["q"])) > 8).mean()
    assert 2e-4 < big < 2e-3
