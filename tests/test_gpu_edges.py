"""GPU parity at the edges of the boundary's contract, through the C ABI:

  * prefill with sm_scale = 0 (every visible key weighs the same: O is the
    mean of the visible V rows) and sm_scale < 0, and with negative
    descales, on causal ragged batches whose lengths are not multiples of
    the 64-key tile: the causal mask must hold for any sign of the scale;
  * the prefill that quantizes a 16-bit Q itself (INT8_PER_BLOCK_RAW_Q) with
    cu_seqlens_q != cu_seqlens_k: sequences with queries and no keys, and
    causal chunks with L_q much larger than L_k (query tiles that see no key);
  * the paged decode at head_dim 64;
  * the sparse MLA decode with tile scales from 1e-3 to 1e3 and with scores
    that rise by more than 10 log2 units along the index list (the lagging
    reference max moves many times).
"""
import math

import numpy as np
import pytest

import gen
from oracle.attention import (decode_paged, dequant_fp8_per_head, dequant_int8_per_block, prefill_varlen,
                              sparse_mla_decode)
from oracle.quant import as_f32, quant_fp8_per_head, quant_int8_per_block
from tests.parity import compare_lse, compare_outputs, decode_out, from_dev_bits, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _round_up(x, m):
    return (x + m - 1) // m * m


# ---------------------------------------------------------------------------
# prefill: scale of any sign
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("sm_scale", [0.0, -0.09, -1.3])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_prefill_scale_of_any_sign(sm_scale, causal):
    from paged_kv_amd.pipeline import Fp8Prefill
    lens = [37, 100, 1, 200, 65]
    x = gen.prefill_fp8_inputs(71, lens, 4, 2, 64, outlier_p=0.001)
    cu = x["cu_seqlens"]
    p = Fp8Prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), max(lens), sm_scale,
                   causal=causal, want_lse=True)
    p.run()
    torch.cuda.synchronize()
    qc, qs = quant_fp8_per_head(x["q"], "bf16")
    kc, ks = quant_fp8_per_head(x["k"], "bf16")
    vc, vs = quant_fp8_per_head(x["v"], "bf16")
    ref = prefill_varlen(dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kc, ks), dequant_fp8_per_head(vc, vs),
                         cu, cu, sm_scale, causal, "bf16")
    got = decode_out(from_dev_bits(p.o), "bf16")
    st = compare_outputs(got, ref["o"], ref["o_exact"], "bf16", f"fp8 sm_scale={sm_scale} causal={causal}")
    compare_lse(p.lse.cpu().numpy(), ref["lse"], f"fp8 sm_scale={sm_scale}")
    if sm_scale == 0.0:  # lse = ln(number of visible keys)
        vis = np.concatenate([np.arange(1, L + 1) if causal else np.full(L, L) for L in lens]).astype(np.float64)
        assert np.allclose(p.lse.cpu().numpy(), np.log(vis)[None, :], atol=1e-5, rtol=0)
    print("scale", sm_scale, causal, st)


@pytest.mark.parametrize("sm_scale", [0.0, -0.088])
def test_sage_prefill_scale_of_any_sign(sm_scale):
    from paged_kv_amd.pipeline import SagePrefill
    lens = [130, 1, 257, 63]
    x = gen.sage_inputs(72, lens, 8, 2, 128)
    cu = x["cu_seqlens"]
    mx = max(lens)
    p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), mx, sm_scale, causal=True,
                    want_lse=True)
    p.run()
    torch.cuda.synchronize()
    qc, qs = quant_int8_per_block(x["q"], "fp16", cu, mx)
    kc, ks = quant_int8_per_block(x["k"], "fp16", cu, mx)
    ref = prefill_varlen(dequant_int8_per_block(qc, qs, cu), dequant_int8_per_block(kc, ks, cu),
                         as_f32(x["v"], "fp16").astype(np.float64), cu, cu, sm_scale, True, "fp16")
    compare_outputs(decode_out(from_dev_bits(p.o), "fp16"), ref["o"], ref["o_exact"], "fp16",
                    f"sage sm_scale={sm_scale}")
    compare_lse(p.lse.cpu().numpy(), ref["lse"], f"sage sm_scale={sm_scale}")


def test_fp8_prefill_negative_descales():
    """Dequant(x, s) = x * s with s < 0 for some q heads (the fold of those
    heads is negative); the causal mask must still remove the future keys."""
    import paged_kv_amd.api as A
    from paged_kv_amd.pipeline import Fp8Prefill
    lens = [70, 129, 5]
    x = gen.prefill_fp8_inputs(73, lens, 4, 2, 128)
    cu = x["cu_seqlens"]
    p = Fp8Prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), max(lens), 0.11, causal=True,
                   want_lse=True)
    p.quantize()
    sign = torch.tensor([1.0, -1.0, -1.0, 1.0], device="cuda")
    qs_neg = (p.qs * sign).contiguous()
    A.attn_prefill_varlen(p.qc, p.kc, p.vp, A.FP8E4M3, A.FP16, qs_neg, p.ks, p.vs, A.Q_FP8_PER_HEAD,
                          A.Q_FP8_PER_HEAD, p.cu, p.cu, p.b, p.max_seqlen, p.max_seqlen, p.t, p.t, p.hq, p.hkv,
                          p.d, 0.11, True, p.o, A.BF16, p.lse)
    torch.cuda.synchronize()
    qc, qs = quant_fp8_per_head(x["q"], "bf16")
    kc, ks = quant_fp8_per_head(x["k"], "bf16")
    vc, vs = quant_fp8_per_head(x["v"], "bf16")
    ref = prefill_varlen(dequant_fp8_per_head(qc, qs * sign.cpu().numpy().astype(np.float32)),
                         dequant_fp8_per_head(kc, ks), dequant_fp8_per_head(vc, vs), cu, cu, 0.11, True, "bf16")
    compare_outputs(decode_out(from_dev_bits(p.o), "bf16"), ref["o"], ref["o_exact"], "bf16", "negative descales")
    compare_lse(p.lse.cpu().numpy(), ref["lse"], "negative descales")


# ---------------------------------------------------------------------------
# prefill quantizing a 16-bit Q itself, against keys of other lengths
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("q_dtype", ["fp16", "bf16"])
def test_raw_q_prefill_with_separate_key_lengths(causal, q_dtype):
    """cu_seqlens_q != cu_seqlens_k in the INT8_PER_BLOCK_RAW_Q mode: a
    sequence with queries and no keys; causal chunks with L_q >> L_k, whose
    first query tiles see no key at all (their workgroups never enter the
    tile loop); a sequence with keys and no queries; ragged tails."""
    import paged_kv_amd.api as A
    lq = [5, 130, 64, 200, 1, 0, 300]
    lk = [0, 300, 64, 10, 50, 7, 129]
    hq, hkv, d = 8, 2, 128
    xq = gen.sage_inputs(74, lq, hq, hkv, d)
    xk = gen.sage_inputs(75, lk, hq, hkv, d)
    q = xq["q"]
    if q_dtype == "bf16":
        q = (as_f32(q, "fp16").view(np.uint32) >> 16).astype(np.uint16)   # bf16 bit patterns
    k, v = xk["k"], xk["v"]
    cu_q, cu_k = xq["cu_seqlens"], xk["cu_seqlens"]
    B, mq, mk = len(lq), max(lq), max(lk)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    dq = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16 if q_dtype == "bf16" else torch.float16).cuda()
    dk, dv = to_dev(k), to_dev(v)
    dcq, dck = to_dev(cu_q), to_dev(cu_k)
    kc = torch.empty(k.shape, dtype=torch.int8, device="cuda")
    ks = torch.empty((B, hkv, (mk + 127) // 128), dtype=torch.float32, device="cuda")
    vp = torch.empty((B, hkv, d, _round_up(mk, 128)), dtype=torch.float16, device="cuda")
    A.attn_quant_qk(dk, A.FP16, dck, B, mk, tk, hkv, d, A.Q_INT8_PER_BLOCK, 128, None, kc, ks)
    A.attn_quant_v_permute(dv, A.FP16, dck, B, mk, tk, hkv, d, A.Q_NONE, None, vp, None)
    qs = torch.full((B, hq, (mq + 127) // 128), -1.0, dtype=torch.float32, device="cuda")
    o = torch.full((tq, hq, d), float("nan"), dtype=torch.float16, device="cuda")
    lse = torch.empty((hq, tq), dtype=torch.float32, device="cuda")
    A.attn_prefill_varlen(dq, kc, vp, A.BF16 if q_dtype == "bf16" else A.FP16, A.FP16, qs, ks, None,
                          A.Q_FP8_PER_HEAD, A.Q_INT8_PER_BLOCK_RAW_Q, dcq, dck, B, mq, mk, tq, tk, hq, hkv, d,
                          0.09, causal, o, A.FP16, lse)
    torch.cuda.synchronize()
    qcode, qsc = quant_int8_per_block(q, q_dtype, cu_q, mq)
    kcode, ksc = quant_int8_per_block(k, "fp16", cu_k, mk)
    assert np.array_equal(kc.cpu().numpy(), kcode)
    got_qs = qs.cpu().numpy()
    for b, L in enumerate(lq):  # the scale of every block that holds a query, nothing else
        nb = (L + 127) // 128
        assert np.array_equal(got_qs[b, :, :nb].view(np.uint32), qsc[b, :, :nb].view(np.uint32))
        assert np.all(got_qs[b, :, nb:] == -1.0)
    ref = prefill_varlen(dequant_int8_per_block(qcode, qsc, cu_q), dequant_int8_per_block(kcode, ksc, cu_k),
                         as_f32(v, "fp16").astype(np.float64), cu_q, cu_k, 0.09, causal, "fp16")
    compare_outputs(decode_out(from_dev_bits(o), "fp16"), ref["o"], ref["o_exact"], "fp16",
                    f"raw q {q_dtype} causal={causal}")
    compare_lse(lse.cpu().numpy(), ref["lse"], "raw q")
    # rows without a visible key: o = 0 exactly and lse = -inf
    none = ~np.isfinite(ref["lse"])
    assert none.any()
    assert np.all(np.isneginf(lse.cpu().numpy()[none]))


# ---------------------------------------------------------------------------
# paged decode at head_dim 64
# ---------------------------------------------------------------------------
def _decode(x, sm_scale, label):
    from paged_kv_amd.pipeline import PagedDecode
    p = PagedDecode(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["k_scale"]),
                    to_dev(x["v_scale"]), to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                    to_dev(x["kv_last_page_len"]), x["max_kv_len"], sm_scale, want_lse=True)
    p.run()
    torch.cuda.synchronize()
    ref = decode_paged(x["q"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"], x["kv_indptr"],
                       x["kv_indices"], x["kv_last_page_len"], 1 / 8 if sm_scale is None else sm_scale)
    st = compare_outputs(decode_out(from_dev_bits(p.o), "bf16"), ref["o"], ref["o_exact"], "bf16", label)
    compare_lse(p.lse.cpu().numpy(), ref["lse"], label)
    return st


@pytest.mark.parametrize("ps", [16, 32, 48, 1024])
def test_decode_head_dim_64(ps):
    x = gen.paged_decode_inputs(76, [5, 0, 33, 16, 600, 1, 1025, 511, 512, 513], 16, 4, 64, page_size=ps)
    _decode(x, 1 / 8, f"d64 ps={ps}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 1), (12, 4), (6, 3)])
def test_decode_head_dim_64_groups(hq, hkv):
    x = gen.paged_decode_inputs(77, [700, 64, 2000, 3], hq, hkv, 64, page_size=16)
    _decode(x, None, f"d64 {hq}/{hkv} default scale")   # None: the library's 1/sqrt(64)


# ---------------------------------------------------------------------------
# sparse MLA: tile scales over six decades, scores rising along the list
# ---------------------------------------------------------------------------
def _compare_wide_range(got, want_r, want_ex, label):
    """Outputs whose magnitude spans many decades (tile scales up to 1e3 make
    |O| up to ~1e5, where one bf16 ulp is 512): every element within
    max(2e-2, 2 bf16 ulps at the exact value) and the mean error relative to
    max(1, |O|) at most 2e-3.  (The absolute rule presumes |O| of order 1.)
    Two ulps: before the output's own rounding, a value passes two bf16
    roundings of at most half an ulp each -- P * tile scale as the PV operand
    and the split's partial O -- so 1.5 ulps of error can round to 2."""
    from tests.parity import ulp_at
    err = np.abs(np.asarray(got, np.float64) - want_r)
    bound = np.maximum(2e-2, 2 * ulp_at(want_ex, "bf16") * (1 + 1e-12))
    assert np.all(err <= bound), f"{label}: worst err / bound {(err / bound).max():.3g}"
    rel = float((err / np.maximum(1.0, np.abs(want_ex))).mean())
    assert rel <= 2e-3, f"{label}: mean relative err {rel:.3g}"
    return {"max_abs": float(err.max()), "max_over_bound": float((err / bound).max()), "mean_rel": rel,
            "max_abs_out": float(np.abs(want_ex).max())}


def _mla(x, sm_scale, kv_fp8, label, wide_range=False):
    from paged_kv_amd.pipeline import SparseMlaDecode
    p = SparseMlaDecode(to_dev(x["q"]), to_dev(x["kv_cache"]), to_dev(x["block_table"]), to_dev(x["kv_lens"]),
                        to_dev(x["sparse_indices"]), sm_scale, want_lse=True, kv_fp8=kv_fp8)
    p.run()
    torch.cuda.synchronize()
    ref = sparse_mla_decode(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"], x["sparse_indices"],
                            1 / 24 if sm_scale is None else sm_scale, kv_dtype="fp8" if kv_fp8 else "int8")
    got = decode_out(from_dev_bits(p.o), "bf16")
    assert np.all(np.isfinite(got)), label
    if wide_range:
        st = _compare_wide_range(got, ref["o"], ref["o_exact"], label)
    else:
        st = compare_outputs(got, ref["o"], ref["o_exact"], "bf16", label)
    compare_lse(p.lse.cpu().numpy(), ref["lse"], label)
    return st


def _selected_rows(x):
    """Physical cache rows of the used tokens, per (b, s): list of arrays in
    index-list order."""
    bs = x["block_size"]
    out = {}
    for b in range(x["batch"]):
        for s in range(x["s_q"]):
            idx = x["sparse_indices"][b, s, 0]
            idx = idx[(idx >= 0) & (idx < x["kv_lens"][b])].astype(np.int64)
            out[(b, s)] = x["block_table"][b][idx // bs].astype(np.int64) * bs + idx % bs
    return out


@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_mla_tile_scales_over_six_decades(kv):
    x = gen.sparse_mla_inputs(78, 3, 1, 32, [1000, 300, 2048], 64, 600, n_valid=550, kv_dtype=kv)
    rows = x["kv_cache"].reshape(-1, gen.MLA_ROW_BYTES)
    rng = np.random.default_rng(7)
    for r in np.unique(np.concatenate(list(_selected_rows(x).values()))):
        sc = (10.0 ** rng.uniform(-3.0, 3.0, size=4)).astype(np.float32)
        rows[r, gen.MLA_NOPE + 2 * gen.MLA_ROPE:] = sc.view(np.uint8)
    st = _mla(x, None, kv == "fp8", f"mla scales 1e-3..1e3 {kv}", wide_range=True)
    print("mla scales", kv, st)


@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_mla_scores_rising_along_the_index_list(kv):
    """The rope part of the u-th used token of each query row is set so that
    its logit grows by 40/24 nats (2.4 log2 units) per 32-index step: over
    the 600 indices the largest logit keeps overtaking the reference."""
    x = gen.sparse_mla_inputs(79, 2, 1, 16, [4096, 1500], 64, 600, kv_dtype=kv)
    rows = x["kv_cache"].reshape(-1, gen.MLA_ROW_BYTES)
    q = x["q"].copy()
    q[..., gen.MLA_NOPE] = 0x3F80          # q_rope[0] = 1.0 (bf16)
    x["q"] = q
    for (b, s), r in _selected_rows(x).items():
        rope = rows[r, gen.MLA_NOPE:gen.MLA_NOPE + 2 * gen.MLA_ROPE].view(np.uint16).copy()
        val = (40.0 / 32.0) * np.arange(r.size, dtype=np.float32)      # rope[0] grows along the list
        rope[:, 0] = (val.view(np.uint32) >> 16).astype(np.uint16)      # bf16 (truncated); the oracle reads these bytes
        rows[r, gen.MLA_NOPE:gen.MLA_NOPE + 2 * gen.MLA_ROPE] = rope.view(np.uint8)
    _mla(x, None, kv == "fp8", f"mla rising {kv}")
