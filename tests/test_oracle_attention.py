"""Pins of oracle.attention: brute force on tiny shapes plus invariants (CPU)."""
import math

import numpy as np
import pytest

import gen
from oracle import brute
from oracle.attention import (attend, prefill_varlen, decode_paged, sparse_mla_decode,
                              lse_merge, dequant_fp8_per_head, dequant_int8_per_block,
                              causal_visible, paged_kv_len)
from oracle.quant import quant_fp8_per_head, quant_int8_per_block


def _fp8_case(seed, lens_q, lens_k, hq, hkv, d):
    rng = np.random.default_rng(seed)
    tq, tk = sum(lens_q), sum(lens_k)
    q = gen.bf16_bits(rng.standard_normal((tq, hq, d)).astype(np.float32))
    k = gen.bf16_bits(rng.standard_normal((tk, hkv, d)).astype(np.float32))
    v = gen.bf16_bits(rng.standard_normal((tk, hkv, d)).astype(np.float32))
    qc, qs = quant_fp8_per_head(q, "bf16")
    kc, ks = quant_fp8_per_head(k, "bf16")
    vc, vs = quant_fp8_per_head(v, "bf16")
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    return (qc, qs, kc, ks, vc, vs), cu_q, cu_k


def _brute_dequant(codes, scale):
    out = np.zeros(codes.shape)
    for idx in np.ndindex(codes.shape):
        out[idx] = brute.e4m3fn_value(int(codes[idx])) * float(scale[idx[1]])
    return out


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("lens", [([3, 1, 0, 5], [3, 1, 0, 5]), ([2, 4], [5, 4]), ([4, 1], [2, 3])])
def test_prefill_vs_brute(causal, lens):
    (qc, qs, kc, ks, vc, vs), cu_q, cu_k = _fp8_case(1, lens[0], lens[1], 4, 2, 8)
    qd, kd, vd = dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kc, ks), dequant_fp8_per_head(vc, vs)
    assert np.array_equal(qd, _brute_dequant(qc, qs))
    assert np.array_equal(vd, _brute_dequant(vc, vs))
    scale = 1 / math.sqrt(8)
    res = prefill_varlen(qd, kd, vd, cu_q, cu_k, scale, causal)
    bo, bl = brute.prefill(qd, kd, vd, cu_q, cu_k, scale, causal)
    assert np.allclose(res["o_exact"], bo, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(res["lse"]))
    assert np.allclose(res["lse"][fin], bl[fin], rtol=1e-6)


def test_int8_block_dequant_vs_scalar():
    rng = np.random.default_rng(2)
    lens = [5, 3]
    x = rng.standard_normal((8, 2, 4)).astype(np.float16)
    cu = np.array([0, 5, 8], np.int32)
    codes, sc = quant_int8_per_block(x, "fp16", cu, 5, block_tokens=2)
    d = dequant_int8_per_block(codes, sc, cu, block_tokens=2)
    for t in range(8):
        b = 0 if t < 5 else 1
        j = (t - cu[b]) // 2
        for h in range(2):
            for c in range(4):
                assert d[t, h, c] == float(codes[t, h, c]) * float(sc[b, h, j])
    del lens


def test_one_visible_key_gives_that_row():
    (qc, qs, kc, ks, vc, vs), cu, _ = _fp8_case(3, [6], [6], 2, 2, 8)
    vd = dequant_fp8_per_head(vc, vs)
    res = prefill_varlen(dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kc, ks), vd, cu, cu, 0.3, True)
    assert np.array_equal(res["o_exact"][0], vd[0])


def test_constant_v_and_ones():
    rng = np.random.default_rng(4)
    qd, kd = rng.standard_normal((7, 2, 8)), rng.standard_normal((7, 1, 8))
    vd = np.full((7, 1, 8), 0.375)
    cu = np.array([0, 3, 7], np.int32)
    r = prefill_varlen(qd, kd, vd, cu, cu, 0.7, True)
    assert np.allclose(r["o_exact"], 0.375, rtol=0, atol=1e-15)
    r1 = prefill_varlen(qd, kd, np.ones_like(vd), cu, cu, 0.7, False)
    assert np.allclose(r1["o_exact"], 1.0, rtol=0, atol=1e-15)


def test_scale_zero_gives_mean_and_log_count():
    rng = np.random.default_rng(5)
    qd, kd, vd = rng.standard_normal((9, 1, 4)), rng.standard_normal((9, 1, 4)), rng.standard_normal((9, 1, 4))
    cu = np.array([0, 9], np.int32)
    r = prefill_varlen(qd, kd, vd, cu, cu, 0.0, True)
    for i in range(9):
        assert np.allclose(r["o_exact"][i, 0], vd[:i + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(r["lse"][0, i] - math.log(i + 1)) < 1e-6


def test_two_key_closed_form():
    q = np.array([[0.5, -1.0]])
    k = np.array([[1.0, 2.0], [-0.5, 0.25]])
    v = np.array([[1.0, 3.0], [-2.0, 5.0]])
    o, lse = attend(q, k, v, 0.8, np.array([2]))
    s0, s1 = 0.8 * q[0] @ k[0], 0.8 * q[0] @ k[1]
    dlt = s1 - s0
    want = (v[0] + math.exp(dlt) * v[1]) / (1 + math.exp(dlt))
    assert np.allclose(o[0], want, rtol=1e-14)
    assert abs(lse[0] - math.log(math.exp(s0) + math.exp(s1))) < 1e-14


def test_masked_future_garbage_has_no_effect():
    rng = np.random.default_rng(6)
    qd, kd, vd = rng.standard_normal((8, 2, 4)), rng.standard_normal((8, 1, 4)), rng.standard_normal((8, 1, 4))
    cu = np.array([0, 8], np.int32)
    base = prefill_varlen(qd, kd, vd, cu, cu, 0.5, True)["o_exact"]
    kd2, vd2 = kd.copy(), vd.copy()
    kd2[5:] = np.nan
    vd2[5:] = np.inf
    got = prefill_varlen(qd, kd2, vd2, cu, cu, 0.5, True)["o_exact"]
    # same sums up to summation order (BLAS vs per-row products)
    assert np.allclose(got[:5], base[:5], rtol=1e-13, atol=1e-15)


def test_bottom_right_causal_alignment():
    assert list(causal_visible(2, 5, True)) == [4, 5]
    assert list(causal_visible(4, 2, True)) == [0, 0, 1, 2]
    assert list(causal_visible(3, 3, True)) == [1, 2, 3]


# ---------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------
def _decode_case(seed=7, lens=(5, 0, 9, 4), ps=4, hq=4, hkv=2, d=8):
    return gen.paged_decode_inputs(seed, list(lens), hq, hkv, d, page_size=ps, spare_frac=0.5)


def _dec(x, scale=0.35, **kw):
    return decode_paged(x["q"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                        x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], scale, **kw)


def test_decode_vs_brute():
    x = _decode_case()
    r = _dec(x)
    bo, bl = brute.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                                x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], 0.35)
    assert np.allclose(r["o_exact"], bo, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isfinite(r["lse"]), np.isfinite(bl))
    assert not r["o_exact"][1].any() and np.all(np.isinf(r["lse"][1]))
    assert list(paged_kv_len(x["kv_indptr"], x["kv_last_page_len"], 4)) == [5, 0, 9, 4]
    assert not np.isnan(r["o_exact"]).any()


def test_decode_page_permutation_invariance():
    x = _decode_case(lens=(13, 7))
    r = _dec(x)
    rng = np.random.default_rng(0)
    p = rng.permutation(x["num_pages"])
    y = dict(x)
    inv = np.empty_like(p)
    inv[p] = np.arange(p.size)
    y["k_cache"] = x["k_cache"][p]
    y["v_cache"] = x["v_cache"][p]
    y["kv_indices"] = inv[x["kv_indices"]].astype(np.int32)
    assert np.array_equal(_dec(y)["o_exact"], r["o_exact"])


def test_decode_equals_dense_with_one_page():
    x = _decode_case(lens=(8,), ps=8, hq=2, hkv=2)
    r = _dec(x)
    page = x["kv_indices"][0]
    kd = dequant_fp8_per_head(x["k_cache"][page], x["k_scale"])
    vd = dequant_fp8_per_head(x["v_cache"][page], x["v_scale"])
    from oracle.numerics import bf16_bits_to_f64
    qd = bf16_bits_to_f64(x["q"])                  # [1, Hq, D] as a 1-token sequence
    d = prefill_varlen(qd, kd, vd, np.array([0, 1]), np.array([0, 8]), 0.35, True)
    assert np.allclose(d["o_exact"][0], r["o_exact"][0], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("last", [1, 4])
def test_decode_last_page_len_edges(last):
    lens = (4 * 2 + last,)
    x = _decode_case(lens=lens)
    r = _dec(x)
    bo, _ = brute.decode_paged(x["q"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                               x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], 0.35)
    assert np.allclose(r["o_exact"], bo, rtol=1e-12, atol=1e-12)


def test_split_then_merge_equals_unsplit():
    rng = np.random.default_rng(9)
    q, k, v = rng.standard_normal((3, 8)), rng.standard_normal((50, 8)), rng.standard_normal((50, 8))
    o, lse = attend(q, k, v, 0.4, np.full(3, 50))
    cuts = [0, 7, 7, 30, 50]                        # includes an empty chunk
    parts_o, parts_l = [], []
    for a, b in zip(cuts[:-1], cuts[1:]):
        po, pl = attend(q, k[a:b], v[a:b], 0.4, np.full(3, b - a))
        parts_o.append(po)
        parts_l.append(pl)
    mo, ml = lse_merge(np.stack(parts_o), np.stack(parts_l))
    assert np.allclose(mo, o, rtol=1e-13, atol=1e-14)
    assert np.allclose(ml, lse, rtol=1e-13)
    eo, el = lse_merge(np.zeros((2, 1, 4)), np.full((2, 1), -np.inf))
    assert not eo.any() and np.isinf(el).all()


# ---------------------------------------------------------------------------
# sparse MLA decode
# ---------------------------------------------------------------------------
def _mla_case(seed=10, batch=2, heads=2, kv_len=(40, 25), bs=16, topk=7, n_valid=5):
    x = gen.sparse_mla_inputs(seed, batch, 1, heads, list(kv_len), bs, topk, n_valid=n_valid,
                              spare_blocks=2)
    return x


def _mla(x, scale=1 / 24, idx=None):
    return sparse_mla_decode(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"],
                             x["sparse_indices"] if idx is None else idx, scale)


def test_mla_vs_brute_with_invalid_and_duplicate_indices():
    x = _mla_case()
    idx = x["sparse_indices"].copy()
    idx[0, 0, 0, 5] = idx[0, 0, 0, 1]           # a duplicate counts twice
    idx[1, 0, 0, 5] = 25                         # == kv_len -> invalid
    r = _mla(x, idx=idx)
    bo, bl = brute.sparse_mla(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"], idx, 1 / 24)
    assert np.allclose(r["o_exact"], bo, rtol=1e-11, atol=1e-12)
    assert np.allclose(r["lse"], bl, rtol=1e-6)
    assert not np.isnan(r["o_exact"]).any()


def test_mla_index_order_irrelevant():
    x = _mla_case()
    a = _mla(x)["o_exact"]
    idx = x["sparse_indices"].copy()
    idx[:, :, :, :5] = idx[:, :, :, :5][..., ::-1]
    assert np.allclose(_mla(x, idx=idx)["o_exact"], a, rtol=1e-13, atol=1e-15)


def test_mla_no_valid_index():
    x = _mla_case()
    idx = np.full_like(x["sparse_indices"], -1)
    r = _mla(x, idx=idx)
    assert not r["o_exact"].any() and np.isinf(r["lse"]).all()


def test_mla_all_tokens_equals_dense_mqa():
    x = gen.sparse_mla_inputs(12, 1, 1, 3, 32, 16, 32)
    r = _mla(x)
    # dense: all 32 tokens, decoded row by row
    from oracle.attention import mla_decode_row
    from oracle.numerics import bf16_bits_to_f64
    rows = x["kv_cache"].reshape(-1, 656)
    kn, kr = [], []
    for t in range(32):
        a, b = mla_decode_row(rows[x["block_table"][0][t // 16] * 16 + t % 16])
        kn.append(a)
        kr.append(b)
    kn, kr = np.array(kn), np.array(kr)
    q = bf16_bits_to_f64(x["q"])[0, 0]                 # [3, 576]
    logits = (q[:, :512] @ kn.T + q[:, 512:] @ kr.T) / 24
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(r["o_exact"][0, 0], p @ kn, rtol=1e-12, atol=1e-13)


def test_mla_unit_scales_zero_rope_is_plain_int8_attention():
    x = gen.sparse_mla_inputs(13, 1, 1, 2, 20, 16, 6)
    rows = x["kv_cache"].reshape(-1, 656)
    rows[:, 512:640] = 0
    rows[:, 640:656] = np.ones(4, np.float32).view(np.uint8)
    r = _mla(x, scale=0.01)
    idx = x["sparse_indices"][0, 0, 0]
    codes = np.array([rows[x["block_table"][0][i // 16] * 16 + i % 16, :512].view(np.int8) for i in idx], float)
    from oracle.numerics import bf16_bits_to_f64
    q = bf16_bits_to_f64(x["q"])[0, 0, :, :512]
    lg = 0.01 * q @ codes.T
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    assert np.allclose(r["o_exact"][0, 0], p @ codes, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------
# reading the paged cache into the ragged layout (prefill against pages)
# ---------------------------------------------------------------------------
def _page_walk(cache, kv_indptr, kv_indices, kv_last_page_len, b):
    """Tokens of sequence b by walking its pages in order, slot by slot."""
    ps = cache.shape[1]
    pages = list(kv_indices[kv_indptr[b]:kv_indptr[b + 1]])
    rows = []
    for j, pg in enumerate(pages):
        m = ps if j < len(pages) - 1 else int(kv_last_page_len[b])
        for s in range(m):
            rows.append(cache[pg, s])
    return np.array(rows, cache.dtype).reshape((-1,) + cache.shape[2:])


def test_ragged_from_pages_vs_page_walk():
    from oracle.attention import ragged_from_pages
    x = gen.paged_prefill_inputs(21, [5, 0, 9, 13], [2, 0, 9, 1], 2, 2, 8, page_size=4, spare_frac=0.5)
    for name in ("k_cache", "v_cache"):
        got = ragged_from_pages(x[name], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_k"])
        cu = x["cu_k"]
        for b in range(4):
            ref = _page_walk(x[name], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], b)
            assert np.array_equal(got[cu[b]:cu[b + 1]], ref)
        assert not np.any(got == 0x7FC0)  # no spare page or unused slot leaks in


def test_ragged_from_pages_rows_past_the_cache_are_zero():
    from oracle.attention import ragged_from_pages
    x = gen.paged_prefill_inputs(22, [6, 3], [1, 1], 1, 1, 4, page_size=4)
    cu = np.array([0, 8, 12], np.int32)  # 2 and 1 rows more than cached
    got = ragged_from_pages(x["k_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], cu)
    assert np.array_equal(got[0:6], _page_walk(x["k_cache"], x["kv_indptr"], x["kv_indices"],
                                               x["kv_last_page_len"], 0))
    assert not got[6:8].any() and not got[11:12].any()


def test_ragged_from_pages_returns_what_the_append_wrote():
    from oracle.attention import ragged_from_pages
    from oracle.rope import append_kv_rope
    x = gen.long_prefill_inputs(23, [7, 5, 12], 2, 2, 8, 4)
    shape = (x["num_pages"], 4, 2, 8)
    kc = np.full(shape, 0x7FC0, np.uint16)
    vc = np.full(shape, 0x7FC0, np.uint16)
    q_rot, k_rot, kc2, vc2 = append_kv_rope(x["q"], x["k"], x["v"], "bf16", x["cu_seqlens"], x["kv_len_before"],
                                            x["rope_cos_sin"], kc, vc, x["kv_indptr"], x["kv_indices"], 4)[:4]
    lens = np.diff(x["cu_seqlens"]) + x["kv_len_before"]
    npg = np.diff(x["kv_indptr"])
    last = (lens - (npg - 1) * 4).astype(np.int32)
    assert np.array_equal(ragged_from_pages(kc2, x["kv_indptr"], x["kv_indices"], last, x["cu_seqlens"]), k_rot)
    assert np.array_equal(ragged_from_pages(vc2, x["kv_indptr"], x["kv_indices"], last, x["cu_seqlens"]), x["v"])


def test_k_smoothing_leaves_softmax_output_unchanged():
    """Subtracting a per-sequence, per-channel mean from K moves every logit
    of a query by the same amount: O is unchanged, lse moves by sm * q . mean."""
    rng = np.random.default_rng(40)
    lens_q, lens_k = [5, 3], [9, 3]
    cu_q = np.array([0, 5, 8], np.int32)
    cu_k = np.array([0, 9, 12], np.int32)
    q = rng.standard_normal((8, 4, 16))
    k = rng.standard_normal((12, 2, 16)) + rng.standard_normal((1, 2, 16)) * 3
    v = rng.standard_normal((12, 2, 16))
    ks = k.copy()
    means = []
    for b in range(2):
        m = k[cu_k[b]:cu_k[b + 1]].mean(axis=0)
        ks[cu_k[b]:cu_k[b + 1]] -= m
        means.append(m)
    a = prefill_varlen(q, k, v, cu_q, cu_k, 0.3, True, "bf16")
    s = prefill_varlen(q, ks, v, cu_q, cu_k, 0.3, True, "bf16")
    assert np.abs(a["o_exact"] - s["o_exact"]).max() < 1e-12
    for b in range(2):
        for i in range(cu_q[b], cu_q[b + 1]):
            for h in range(4):
                shift = 0.3 * float(q[i, h] @ means[b][h // 2])
                assert abs(float(a["lse"][h, i]) - float(s["lse"][h, i]) - shift) < 1e-4


# ---------------------------------------------------------------------------
# sparse MLA variants: fp8 rows, block-wise sparsity, right-down causal mask
# ---------------------------------------------------------------------------
def _mla_var(x, idx=None, **kw):
    return sparse_mla_decode(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"],
                             x["sparse_indices"] if idx is None else idx, 1 / 24,
                             kv_dtype=x["kv_dtype"], sparse_block_size=x["sparse_block_size"], **kw)


@pytest.mark.parametrize("kv_dtype", ["int8", "fp8"])
@pytest.mark.parametrize("sbs", [1, 4])
@pytest.mark.parametrize("mode", [0, 3])
def test_mla_variants_vs_brute(kv_dtype, sbs, mode):
    x = gen.sparse_mla_inputs(21, 2, 3, 2, [40, 25], 16, 5, n_valid=4, spare_blocks=1,
                              kv_dtype=kv_dtype, sparse_block_size=sbs)
    idx = x["sparse_indices"].copy()
    idx[0, 1, 0, 4] = idx[0, 1, 0, 0]            # a duplicate entry counts twice
    r = _mla_var(x, idx, sparse_mode=mode)
    bo, bl = brute.sparse_mla(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"], idx, 1 / 24,
                              kv_dtype=kv_dtype, sparse_block_size=sbs, sparse_mode=mode)
    assert np.allclose(r["o_exact"], bo, rtol=1e-11, atol=1e-12)
    assert np.array_equal(np.isinf(r["lse"]), np.isinf(bl))
    fin = np.isfinite(bl)
    assert np.allclose(r["lse"][fin], bl[fin], rtol=1e-6)
    assert not np.isnan(r["o_exact"]).any()


def test_mla_block_sparse_is_its_token_expansion():
    # an entry e of block size 4 is the four token entries 4e .. 4e+3
    x = gen.sparse_mla_inputs(22, 2, 1, 2, [40, 25], 16, 4, n_valid=3, sparse_block_size=4)
    idx = x["sparse_indices"]
    tok = np.where(idx[..., None] >= 0, idx[..., None] * 4 + np.arange(4), -1).reshape(2, 1, 1, 16)
    a = _mla_var(x)
    y = dict(x, sparse_block_size=1)
    b = _mla_var(y, tok)
    assert np.array_equal(a["o_exact"], b["o_exact"]) and np.array_equal(a["lse"], b["lse"])


def test_mla_right_down_causal():
    x = gen.sparse_mla_inputs(23, 2, 4, 2, [40, 25], 16, 12, n_valid=10)
    kv = x["kv_lens"]
    full = _mla_var(x)
    causal = _mla_var(x, sparse_mode=3)
    for b in range(2):
        for s in range(4):
            # row s keeps exactly the tokens at or before kv_len - 4 + s
            idx = x["sparse_indices"].copy()
            row = idx[b, s, 0]
            row[row > kv[b] - 4 + s] = -1
            one = _mla_var(x, idx)
            assert np.array_equal(causal["o_exact"][b, s], one["o_exact"][b, s])
    # the last query row sees every token below kv_len: no mask
    assert np.array_equal(causal["o_exact"][:, 3], full["o_exact"][:, 3])
    # with one query row the mask removes nothing
    y = gen.sparse_mla_inputs(23, 2, 1, 2, [40, 25], 16, 12, n_valid=10)
    assert np.array_equal(_mla_var(y, sparse_mode=3)["o_exact"], _mla_var(y)["o_exact"])


def test_mla_fp8_row_decode():
    from oracle.attention import mla_decode_row
    x = gen.sparse_mla_inputs(24, 1, 1, 1, 16, 16, 16, kv_dtype="fp8")
    row = x["kv_cache"][x["block_table"][0][0], 3, 0]
    kn, kr = mla_decode_row(row, "fp8")
    sc = row[640:656].view(np.float32)
    for c in range(512):
        assert kn[c] == brute.e4m3fn_value(int(row[c])) * float(sc[c // 128])
    assert np.abs(kn).max() <= 3.75 * float(sc.max())


# ---------------------------------------------------------------------------
# paged prefill (fp8 pages)
# ---------------------------------------------------------------------------
def _paged_fp8(seed, kv, ql, ps=4, hq=4, hkv=2, d=8):
    return gen.paged_prefill_fp8_inputs(seed, list(kv), list(ql), hq, hkv, d, page_size=ps, spare_frac=0.5)


def _ppf(x, scale, causal, **kw):
    from oracle.attention import prefill_paged
    return prefill_paged(x["q"], x["q_scale"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                         x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_q"], scale, causal, **kw)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kv,ql", [((9, 0, 6, 4), (3, 0, 6, 1)), ((5, 8), (0, 2)), ((3,), (3,))])
def test_prefill_paged_vs_page_walk(causal, kv, ql):
    """The composition (pages -> ragged -> dequantize -> prefill_varlen)
    against a scalar walk over pages and slots with its own fp8 decoder;
    stale slots and spare pages hold NaN codes."""
    x = _paged_fp8(11, kv, ql)
    r = _ppf(x, 0.4, causal)
    bo, bl = brute.prefill_paged(x["q"], x["q_scale"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                                 x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_q"], 0.4, causal)
    assert np.allclose(r["o_exact"], bo, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isfinite(r["lse"]), np.isfinite(bl))
    fin = np.isfinite(bl)
    assert np.allclose(r["lse"][fin], bl[fin], rtol=1e-6)
    assert not np.isnan(r["o_exact"]).any()


def test_prefill_paged_last_query_is_the_decode():
    """One query per sequence at the last position sees every cached key:
    with a power-of-two q descale its dequantized value is a bf16 value, and
    the result is decode_paged's."""
    x = _paged_fp8(12, (9, 6, 4), (1, 1, 1))
    x["q_scale"] = np.full(x["q_scale"].shape, 0.5, np.float32)
    from oracle.numerics import e4m3fn_decode
    qv = e4m3fn_decode(x["q"]) * 0.5                  # [B, Hq, D], exact in bf16
    qbits = gen.bf16_bits(qv.astype(np.float32))
    r = _ppf(x, 0.3, True)
    dd = decode_paged(qbits, x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"], x["kv_indptr"],
                      x["kv_indices"], x["kv_last_page_len"], 0.3)
    assert np.allclose(r["o_exact"], dd["o_exact"], rtol=1e-13, atol=1e-14)
    assert np.allclose(r["lse"].T, dd["lse"], rtol=1e-7)
