"""GPU parity of attn_prefill_paged: a prefill chunk whose kernel reads fp8
K/V pages itself (page ids per 64-key tile, rows by page offset), against
oracle.attention.prefill_paged (pages read into the ragged layout,
dequantized, the ragged prefill with the chunk aligned to the end of its
sequence).  Every cache carries NaN codes in its spare pages and in the
stale slots of each last page; none may reach an output.  The same inputs
through the ragged path (pages gathered on the host, V^T permuted as
attn_quant_v_permute documents) give bit-identical results: the kernels feed
the matrix instructions the same values in the same key order."""
import numpy as np
import pytest

import gen
from oracle.attention import paged_kv_len, prefill_paged, ragged_from_pages
from tests.parity import LSE_REL_MFMA8, compare_lse, compare_outputs, decode_out, from_dev_bits, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _attend(x, causal, mode=None, out="bf16", sm_scale=None):
    import paged_kv_amd.api as A
    mode = A.Q_FP8_PER_HEAD if mode is None else mode
    tq, hq, d = x["q"].shape
    b = len(x["cu_q"]) - 1
    max_kv = int(paged_kv_len(x["kv_indptr"], x["kv_last_page_len"], x["page_size"]).max(initial=0))
    o = torch.full((tq, hq, d), 7.0, dtype=torch.bfloat16 if out == "bf16" else torch.float16, device="cuda")
    lse = torch.full((hq, tq), 3.0, dtype=torch.float32, device="cuda")
    A.attn_prefill_paged(to_dev(x["q"]), to_dev(x["q_scale"]), mode, to_dev(x["k_cache"]), to_dev(x["v_cache"]),
                         to_dev(x["k_scale"]), to_dev(x["v_scale"]), to_dev(x["kv_indptr"]),
                         to_dev(x["kv_indices"]), to_dev(x["kv_last_page_len"]), to_dev(x["cu_q"]), b,
                         x["num_pages"], x["page_size"], int(x["max_q"]), max_kv, tq, hq, x["hkv"], d,
                         x["sm_scale"] if sm_scale is None else sm_scale, causal, o,
                         A.BF16 if out == "bf16" else A.FP16, lse)
    torch.cuda.synchronize()
    return o, lse


def _check(x, causal, label, mode=None, out="bf16", rel=None):
    o, lse = _attend(x, causal, mode, out)
    ref = prefill_paged(x["q"], x["q_scale"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                        x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], x["cu_q"], x["sm_scale"], causal,
                        out)
    got = decode_out(from_dev_bits(o), out)
    stats = compare_outputs(got, ref["o"], ref["o_exact"], out, label)
    compare_lse(lse.cpu().numpy(), ref["lse"], label, **({} if rel is None else {"rel": rel}))
    print(label, stats)
    return o, lse


@pytest.mark.parametrize("page_size", [16, 48, 64, 1024])
@pytest.mark.parametrize("causal", [True, False])
def test_paged_fp8_prefill_ragged(page_size, causal):
    # chunks of 1..300 queries against 1..700 cached tokens: a sequence
    # without queries, one whose chunk is its whole history, one query
    # against one key, ragged last pages
    x = gen.paged_prefill_fp8_inputs(81, [700, 129, 64, 300, 1], [300, 0, 64, 1, 1], 4, 2, 128, page_size)
    x["sm_scale"] = 128 ** -0.5
    _check(x, causal, f"ps={page_size} causal={causal}")


def test_paged_fp8_prefill_d64_gqa_fp16_out():
    x = gen.paged_prefill_fp8_inputs(82, [257, 1000, 65], [257, 130, 2], 8, 1, 64, 32)
    x["sm_scale"] = 0.125
    _check(x, True, "d64 gqa 8:1 fp16 out", out="fp16")


def test_paged_fp8_prefill_mfma8_mode():
    import paged_kv_amd.api as A
    x = gen.paged_prefill_fp8_inputs(83, [513, 90], [200, 90], 4, 4, 128, 16)
    x["sm_scale"] = 128 ** -0.5
    _check(x, True, "fp8 mfma qk", mode=A.Q_FP8_PER_HEAD_MFMA8, rel=LSE_REL_MFMA8)


def test_paged_fp8_prefill_queries_without_keys():
    """A sequence with queries and no page: its rows get o = 0, lse = -inf
    (the output is pre-filled with 7 and lse with 3)."""
    x = gen.paged_prefill_fp8_inputs(84, [40, 0], [5, 0], 2, 2, 128, 16)
    rng = np.random.default_rng(1)
    extra = gen.fp8_lut_codes(rng, (3, 2, 128))
    x["q"] = np.concatenate([x["q"], extra])
    x["cu_q"] = np.array([0, 5, 8], np.int32)
    x["max_q"] = 5
    x["sm_scale"] = 128 ** -0.5
    o, lse = _check(x, True, "no keys")
    assert torch.all(o[5:].float() == 0) and torch.all(torch.isneginf(lse[:, 5:]))


def _vperm_host(codes, cu_k, max_k):
    """fp8 codes [T, H, D] -> the permuted V^T layout [B, H, D, round_up(max_k, 128)]:
    token 32G + j of a sequence at position 32G + 8((j % 16) / 4) + 4(j / 16) + j % 4,
    zeros past its end."""
    b = len(cu_k) - 1
    _, h, d = codes.shape
    s_pad = (max_k + 127) // 128 * 128
    out = np.zeros((b, h, d, s_pad), np.uint8)
    for i in range(b):
        rows = codes[cu_k[i]:cu_k[i + 1]]
        for t in range(rows.shape[0]):
            j = t % 32
            pos = 32 * (t // 32) + 8 * ((j % 16) // 4) + 4 * (j // 16) + j % 4
            out[i, :, :, pos] = rows[t]
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_paged_equals_ragged_bit_exact(causal):
    import paged_kv_amd.api as A
    x = gen.paged_prefill_fp8_inputs(85, [700, 129, 300, 1], [300, 129, 1, 1], 4, 2, 128, 16)
    x["sm_scale"] = 128 ** -0.5
    o_p, lse_p = _attend(x, causal)
    lens = paged_kv_len(x["kv_indptr"], x["kv_last_page_len"], 16)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kc = ragged_from_pages(x["k_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], cu_k)
    vc = ragged_from_pages(x["v_cache"], x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], cu_k)
    max_k = int(lens.max())
    vp = _vperm_host(vc, cu_k, max_k)
    tq = x["q"].shape[0]
    o_r = torch.full((tq, 4, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse_r = torch.full((4, tq), 3.0, dtype=torch.float32, device="cuda")
    A.attn_prefill_varlen(to_dev(x["q"]), to_dev(kc), to_dev(vp), A.FP8E4M3, A.FP8E4M3, to_dev(x["q_scale"]),
                          to_dev(x["k_scale"]), to_dev(x["v_scale"]), A.Q_FP8_PER_HEAD, A.Q_FP8_PER_HEAD,
                          to_dev(x["cu_q"]), to_dev(cu_k), len(lens), int(x["max_q"]), max_k, tq, int(cu_k[-1]),
                          4, 2, 128, x["sm_scale"], causal, o_r, A.BF16, lse_r)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bits(o_p), from_dev_bits(o_r))
    assert np.array_equal(lse_p.cpu().numpy().view(np.uint32), lse_r.cpu().numpy().view(np.uint32))


def test_paged_fp8_prefill_workload_sampled():
    """The chunked-prefill workload over an fp8 cache at full size (B=4,
    kv_len U{8192..24576}, 2048-query chunks, 32/8 heads, D=128, page 64):
    every output finite, sampled rows of 3 heads per sequence against the
    oracle."""
    x = gen.paged_prefill_fp8_workload()
    o, lse = _attend(x, True)
    assert torch.isfinite(o.float()).all()
    got = decode_out(from_dev_bits(o), "bf16")
    lse = lse.cpu().numpy()
    rng = np.random.default_rng(7)
    cu_q = x["cu_q"]
    rows = []
    for b in range(len(cu_q) - 1):
        L = int(cu_q[b + 1] - cu_q[b])
        idx = np.unique(np.concatenate([[0, L - 1, 127, 128], rng.integers(0, L, 8)]))
        for h in rng.choice(32, 3, replace=False):
            rows.append((b, int(h), idx))
    res = prefill_paged(x["q"], x["q_scale"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"],
                        x["kv_indptr"], x["kv_indices"], x["kv_last_page_len"], cu_q, x["sm_scale"], True, "bf16",
                        rows=rows)
    for (b, h, idx, o_ex, o_r, l) in res:
        s0 = int(cu_q[b])
        compare_outputs(got[s0 + idx, h], o_r, o_ex, "bf16", f"paged fp8 b={b} h={h}")
        compare_lse(lse[h, s0 + idx], l, f"paged fp8 b={b} h={h}")
