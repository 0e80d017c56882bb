"""attn_decode_paged_noalloc (the paged decode for callers that cannot
allocate: its split partials live in the library's fixed scratch) against
attn_decode_paged with a caller workspace, through the C ABI: two calls in a
row, the second smaller, each identical bit for bit to the workspace call on
the same inputs (the same kernels run), and within the comparison rule of the
oracle; sizes past the scratch are rejected before anything runs."""
import numpy as np
import pytest

import gen
from oracle.attention import decode_paged
from tests.parity import compare_lse, compare_outputs, decode_out, from_dev_bits, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _inputs(x):
    return [to_dev(x[k]) for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "kv_indptr", "kv_indices",
                                   "kv_last_page_len")]


def _sizes(x):
    b, hq, d = x["q"].shape
    return b, x["num_pages"], x["page_size"], hq, x["hkv"], d, x["max_kv_len"]


def _with_workspace(x, sm):
    import paged_kv_amd.api as A
    b, npg, ps, hq, hkv, d, mkv = _sizes(x)
    need = A.attn_decode_paged_workspace_size(b, hq, d, mkv, ps)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    o = torch.empty((b, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((b, hq), dtype=torch.float32, device="cuda")
    A.attn_decode_paged(*_inputs(x), b, npg, ps, hq, hkv, d, mkv, sm, ws, need, o, lse)
    torch.cuda.synchronize()
    return from_dev_bits(o).copy(), lse.cpu().numpy().copy()


def _no_alloc(x, sm):
    import paged_kv_amd.api as A
    b, npg, ps, hq, hkv, d, mkv = _sizes(x)
    o = torch.full((b, hq, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((b, hq), float("nan"), dtype=torch.float32, device="cuda")
    A.attn_decode_paged_noalloc(*_inputs(x), b, npg, ps, hq, hkv, d, mkv, sm, o, lse)
    torch.cuda.synchronize()
    return from_dev_bits(o).copy(), lse.cpu().numpy().copy()


def _check(x, sm, label):
    o1, l1 = _no_alloc(x, sm)
    o2, l2 = _with_workspace(x, sm)
    assert np.array_equal(o1, o2), label
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), label
    ref = decode_paged(x["q"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"], x["kv_indptr"],
                       x["kv_indices"], x["kv_last_page_len"], sm)
    compare_outputs(decode_out(o1, "bf16"), ref["o"], ref["o_exact"], "bf16", label)
    compare_lse(l1, ref["lse"], label)


def test_no_alloc_decode_two_calls_second_smaller():
    big = gen.paged_decode_inputs(91, [3000, 17, 0, 1025, 6000, 511], 32, 8, 128, page_size=16)
    small = gen.paged_decode_inputs(92, [40, 700], 16, 4, 64, page_size=32)
    _check(big, 1 / 11.3, "first call")
    _check(small, 0.125, "second, smaller call")   # the scratch still holds the first call's partials


def test_no_alloc_decode_rejects_sizes_past_the_scratch():
    import paged_kv_amd.api as A
    x = gen.paged_decode_inputs(93, [64], 8, 8, 128)
    q, kc, vc, ks, vs, ip, ix, lpl = _inputs(x)
    o = torch.empty((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    # 128 q heads x (2^20 tokens / 512) chunks x 129 floats: 129 MiB of partials
    # (valid arguments otherwise: they are checked before the size)
    with pytest.raises(RuntimeError, match="scratch"):
        A.attn_decode_paged_noalloc(q, kc, vc, ks, vs, ip, ix, lpl, 1, x["num_pages"], 16, 128, 8, 128, 1 << 20,
                                    0.1, o, None)
