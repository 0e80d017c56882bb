"""A NaN among the values the formula uses makes exactly the output rows that
use it NaN (o and lse), as in the fp64 oracle; every other row is unchanged.
One NaN code is planted in a used fp8 K entry of the prefill and of the paged
decode, and one NaN cache row is selected in the sparse MLA decode."""
import math

import numpy as np
import pytest

import gen
from oracle.attention import decode_paged, dequant_fp8_per_head, prefill_varlen, sparse_mla_decode
from oracle.quant import quant_fp8_per_head
from tests.parity import to_dev, dev_u8, from_dev_bits, decode_out, compare_outputs, compare_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _same_nan_rows_then_compare(got, lse, ref, label):
    """got [..., D], lse [...]: NaN rows must match the oracle's; the others
    follow the comparison rule."""
    nan_ref = np.isnan(ref["o_exact"]).any(axis=-1)
    assert nan_ref.any(), f"{label}: the planted NaN reached no row"
    assert np.array_equal(np.isnan(got).all(axis=-1), nan_ref), f"{label}: NaN rows differ"
    assert np.array_equal(np.isnan(got).any(axis=-1), nan_ref), f"{label}: partly NaN rows"
    assert np.array_equal(np.isnan(lse), nan_ref), f"{label}: NaN lse rows differ"
    ok = ~nan_ref
    compare_outputs(got[ok], ref["o"][ok], ref["o_exact"][ok], "bf16", label)
    compare_lse(lse[ok], ref["lse"][ok], label)


def test_nan_in_prefill_key():
    from paged_kv_amd.pipeline import Fp8Prefill
    lens = [300, 129]
    x = gen.prefill_fp8_inputs(81, lens, 4, 2, 128)
    cu = x["cu_seqlens"]
    p = Fp8Prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), max(lens), 1 / math.sqrt(128),
                   causal=True, want_lse=True)
    p.quantize()
    p.kc[100, 1, 7] = 0x7F          # token 100 of sequence 0, kv head 1: NaN code
    p.attend()
    torch.cuda.synchronize()
    qc, kc = dev_u8(p.qc), dev_u8(p.kc)
    qs, ks, vs = (t.cpu().numpy() for t in (p.qs, p.ks, p.vs))
    vc, _ = quant_fp8_per_head(x["v"], "bf16")
    ref = prefill_varlen(dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kc, ks), dequant_fp8_per_head(vc, vs),
                         cu, cu, 1 / math.sqrt(128), True, "bf16")
    got = decode_out(from_dev_bits(p.o), "bf16")
    lse = p.lse.cpu().numpy().T                       # [H, T] -> [T, H], as o's rows
    _same_nan_rows_then_compare(got, lse, dict(ref, lse=ref["lse"].T), "prefill NaN key")


def test_nan_in_decode_key():
    from paged_kv_amd.pipeline import PagedDecode
    x = gen.paged_decode_inputs(82, [700, 64, 2000], 16, 4, 128, page_size=16)
    kc = x["k_cache"].copy()
    b, tok = 2, 1500                                  # a used slot of sequence 2
    page = x["kv_indices"][x["kv_indptr"][b] + tok // 16]
    kc[page, tok % 16, 3, 5] = 0x7F                   # kv head 3
    p = PagedDecode(to_dev(x["q"]), to_dev(kc), to_dev(x["v_cache"]), to_dev(x["k_scale"]), to_dev(x["v_scale"]),
                    to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]), to_dev(x["kv_last_page_len"]),
                    x["max_kv_len"], 1 / math.sqrt(128), want_lse=True)
    p.run()
    torch.cuda.synchronize()
    ref = decode_paged(x["q"], kc, x["v_cache"], x["k_scale"], x["v_scale"], x["kv_indptr"], x["kv_indices"],
                       x["kv_last_page_len"], 1 / math.sqrt(128))
    _same_nan_rows_then_compare(decode_out(from_dev_bits(p.o), "bf16"), p.lse.cpu().numpy(), ref, "decode NaN key")


def test_nan_row_selected_in_sparse_mla():
    from paged_kv_amd.pipeline import SparseMlaDecode
    x = gen.sparse_mla_inputs(83, 2, 2, 16, [1200, 300], 64, 700, n_valid=650)
    rows = x["kv_cache"].reshape(-1, 656)
    nan_tok = next(t for t in range(1200)
                   if np.isnan(rows[x["block_table"][0][t // 64] * 64 + t % 64, 640:656].view(np.float32)).any())
    x["sparse_indices"][0, 1, 0, 600] = nan_tok       # row (0, 1) selects a NaN row in its second split
    p = SparseMlaDecode(to_dev(x["q"]), to_dev(x["kv_cache"]), to_dev(x["block_table"]), to_dev(x["kv_lens"]),
                        to_dev(x["sparse_indices"]), 1 / 24, want_lse=True)
    p.run()
    torch.cuda.synchronize()
    ref = sparse_mla_decode(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"], x["sparse_indices"], 1 / 24)
    _same_nan_rows_then_compare(decode_out(from_dev_bits(p.o), "bf16"), p.lse.cpu().numpy(), ref, "mla NaN row")
