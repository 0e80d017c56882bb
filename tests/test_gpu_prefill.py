"""GPU parity of the varlen prefill through the C ABI (fp8 and SageAttention
int8 flows): quantized inputs bit-exact, outputs within the comparison rule."""
import math

import numpy as np
import pytest

import gen
from oracle.attention import dequant_fp8_per_head, dequant_int8_per_block, prefill_varlen
from oracle.numerics import e4m3fn_decode, to_fp16
from oracle.quant import quant_fp8_per_head, quant_int8_per_block, v_permute, as_f32
from tests.parity import (LSE_REL, LSE_REL_MFMA8, compare_lse, compare_outputs, decode_out, dev_u8,
                          from_dev_bits, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _fp8_flow(x, sm_scale, causal=True, lse=True, wide_v=True, fp8_mma8=False):
    from paged_kv_amd.pipeline import Fp8Prefill
    cu = x["cu_seqlens"]
    mx = int(np.diff(cu).max()) if len(cu) > 1 else 0
    p = Fp8Prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), mx, sm_scale,
                   causal=causal, want_lse=lse, wide_v=wide_v, fp8_mma8=fp8_mma8)
    p.run()
    torch.cuda.synchronize()
    return p, mx


def _check_fp8(x, sm_scale, causal=True, label="", wide_v=True, fp8_mma8=False):
    p, mx = _fp8_flow(x, sm_scale, causal, wide_v=wide_v, fp8_mma8=fp8_mma8)
    cu = x["cu_seqlens"]
    qc, qs = quant_fp8_per_head(x["q"], "bf16")
    kc, ks = quant_fp8_per_head(x["k"], "bf16")
    vc, vs = quant_fp8_per_head(x["v"], "bf16")
    vperm, _ = v_permute(x["v"], "bf16", cu, mx, fp8=True)
    # quantized inputs are bit-exact
    assert np.array_equal(dev_u8(p.qc), qc) and np.array_equal(dev_u8(p.kc), kc)
    if wide_v:  # each code stored as its exact fp16 value
        assert np.array_equal(from_dev_bits(p.vp), to_fp16(e4m3fn_decode(vperm)).view(np.uint16))
    else:
        assert np.array_equal(dev_u8(p.vp), vperm)
    for a, b in ((p.qs, qs), (p.ks, ks), (p.vs, vs)):
        assert np.array_equal(a.cpu().numpy().view(np.uint32), b.view(np.uint32))
    ref = prefill_varlen(dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kc, ks),
                         dequant_fp8_per_head(vc, vs), cu, cu, sm_scale, causal, "bf16")
    got = decode_out(from_dev_bits(p.o), "bf16")
    stats = compare_outputs(got, ref["o"], ref["o_exact"], "bf16", label)
    compare_lse(p.lse.cpu().numpy(), ref["lse"], label, rel=LSE_REL_MFMA8 if fp8_mma8 else LSE_REL)
    return stats


@pytest.mark.parametrize("fp8_mma8", [False, True])
def test_config1_fp8_varlen(fp8_mma8):
    x = gen.config1()
    st = _check_fp8(x, x["sm_scale"], True, f"config1 mma8={fp8_mma8}", fp8_mma8=fp8_mma8)
    print("PARITY config1 (every row, fp8_mma8=%s):" % fp8_mma8, st)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("wide_v", [True, False])
@pytest.mark.parametrize("fp8_mma8", [False, True])
def test_fp8_ragged_edges(d, causal, wide_v, fp8_mma8):
    # empty, single-token, exactly one tile, one past a tile, long ragged;
    # V as fp8 codes and as their fp16 values; QK^T exact or on the fp8 MFMA
    lens = [1, 0, 128, 129, 64, 65, 300]
    x = gen.prefill_fp8_inputs(31, lens, 4, 2, d, outlier_p=0.001)
    _check_fp8(x, 1 / math.sqrt(d), causal, f"ragged d={d} causal={causal} wide_v={wide_v} mma8={fp8_mma8}",
               wide_v, fp8_mma8)


def test_fp8_gqa_8to1():
    x = gen.prefill_fp8_inputs(32, [513, 70], 8, 1, 128)
    _check_fp8(x, 1 / math.sqrt(128), True, "gqa8")


def test_fp8_deterministic():
    x = gen.prefill_fp8_inputs(33, [200, 90], 4, 4, 128)
    p, _ = _fp8_flow(x, 0.1)
    a = from_dev_bits(p.o).copy()
    p.run()
    torch.cuda.synchronize()
    assert np.array_equal(from_dev_bits(p.o), a)


def _sage_flow(x, sm_scale, causal=True, fuse_q=True):
    from paged_kv_amd.pipeline import SagePrefill
    cu = x["cu_seqlens"]
    mx = int(np.diff(cu).max())
    p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(cu), mx, sm_scale,
                    causal=causal, want_lse=True, fuse_q=fuse_q)
    p.run()
    torch.cuda.synchronize()
    return p, mx


def _sage_ref(x, mx, sm_scale, causal, rows=None, seqs=None):
    cu = x["cu_seqlens"]
    qc, qs = quant_int8_per_block(x["q"], "fp16", cu, mx)
    kc, ks = quant_int8_per_block(x["k"], "fp16", cu, mx)
    return qc, qs, kc, ks


def _qs_written(qs, cu):
    """Mask of the per-block scale entries that hold a query (the fused flow
    writes only those)."""
    m = np.zeros(qs.shape, bool)
    for b, L in enumerate(np.diff(cu)):
        m[b, :, :(int(L) + 127) // 128] = True
    return m


@pytest.mark.parametrize("fuse_q", [True, False])
@pytest.mark.parametrize("lens", [[130, 257, 1, 511], [64, 0, 700]])
def test_sage_int8_small(lens, fuse_q):
    x = gen.sage_inputs(41, lens, 8, 2, 128)
    sm = 1 / math.sqrt(128)
    p, mx = _sage_flow(x, sm, fuse_q=fuse_q)
    cu = x["cu_seqlens"]
    qc, qs, kc, ks = _sage_ref(x, mx, sm, True)
    assert np.array_equal(p.kc.cpu().numpy(), kc)
    if fuse_q:  # Q codes stay inside the prefill; its block scales are output
        w = _qs_written(qs, cu)
        assert np.array_equal(p.qs.cpu().numpy().view(np.uint32)[w], qs.view(np.uint32)[w])
    else:
        assert np.array_equal(p.qc.cpu().numpy(), qc)
        assert np.array_equal(p.qs.cpu().numpy().view(np.uint32), qs.view(np.uint32))
    vperm, _ = v_permute(x["v"], "fp16", cu, mx, fp8=False)
    assert np.array_equal(p.vp.cpu().numpy().view(np.uint16), vperm.view(np.uint16))
    ref = prefill_varlen(dequant_int8_per_block(qc, qs, cu), dequant_int8_per_block(kc, ks, cu),
                         as_f32(x["v"], "fp16").astype(np.float64), cu, cu, sm, True, "fp16")
    got = decode_out(from_dev_bits(p.o), "fp16")
    compare_outputs(got, ref["o"], ref["o_exact"], "fp16", f"sage {lens}")
    compare_lse(p.lse.cpu().numpy(), ref["lse"], "sage")


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("fuse_q", [True, False])
def test_sage_int8_block_scales_far_apart(causal, fuse_q, d):
    """K blocks of one sequence at magnitudes 2^-6 .. 2^6 in a shuffled order
    (the fold of a later tile can be far above or below the current
    reference's), one sequence at about 300x (a fold above 1: the kernel then
    takes the tile without its exact-reference bias) and one at 1e-3x: every
    case against the oracle."""
    lens = [1300, 700, 300, 129]
    x = gen.sage_inputs(47, lens, 8, 2, d)
    cu = x["cu_seqlens"]
    rng = np.random.default_rng(5)
    k = as_f32(x["k"], "fp16")
    q = as_f32(x["q"], "fp16")
    s0 = int(cu[0])
    nb = (lens[0] + 127) // 128
    f = 2.0 ** rng.permutation(np.linspace(-6, 6, nb))
    for j in range(nb):
        k[s0 + 128 * j:min(s0 + 128 * (j + 1), int(cu[1]))] *= f[j]
    q[cu[1]:cu[2]] *= 300.0
    k[cu[1]:cu[2]] *= 300.0
    q[cu[2]:cu[3]] *= 1e-3
    x["q"], x["k"] = q.astype(np.float16), k.astype(np.float16)
    assert np.isfinite(x["q"]).all() and np.isfinite(x["k"]).all()
    sm = 1 / math.sqrt(d)
    p, mx = _sage_flow(x, sm, causal=causal, fuse_q=fuse_q)
    qc, qs, kc, ks = _sage_ref(x, mx, sm, causal)
    ref = prefill_varlen(dequant_int8_per_block(qc, qs, cu), dequant_int8_per_block(kc, ks, cu),
                         as_f32(x["v"], "fp16").astype(np.float64), cu, cu, sm, causal, "fp16")
    got = decode_out(from_dev_bits(p.o), "fp16")
    stats = compare_outputs(got, ref["o"], ref["o_exact"], "fp16", f"sage scales d={d} causal={causal}")
    compare_lse(p.lse.cpu().numpy(), ref["lse"], "sage scales")
    print("sage block scales", d, causal, fuse_q, stats)


@pytest.mark.parametrize("case", ["config2", "d64_bf16", "ragged_gqa"])
def test_sage_fused_q_equals_separate_quant(case):
    """Quantizing Q inside the prefill gives bit-identical outputs, lse and
    block scales to attn_quant_qk followed by the prefill (same codes)."""
    from paged_kv_amd.pipeline import SagePrefill
    if case == "config2":
        x, sm = gen.config2(), 1 / math.sqrt(128)
    elif case == "d64_bf16":  # bf16 Q (and K), fp16 V
        x, sm = gen.sage_inputs(44, [300, 129, 1000], 4, 4, 64), 0.125
        for t in ("q", "k"):  # truncated to bf16 bit patterns
            x[t] = (as_f32(x[t], "fp16").view(np.uint32) >> 16).astype(np.uint16)
    else:
        x, sm = gen.sage_inputs(45, [1, 127, 128, 129, 383, 0, 2049], 12, 4, 128), 0.07
    cu = x["cu_seqlens"]
    mx = int(np.diff(cu).max())
    q, k, v = (to_dev(x[t]) for t in ("q", "k", "v"))
    outs = []
    for fuse in (True, False):
        p = SagePrefill(q, k, v, to_dev(cu), mx, sm, causal=True, want_lse=True, fuse_q=fuse)
        if fuse:
            p.qs.fill_(-1.0)
        p.run()
        torch.cuda.synchronize()
        outs.append((from_dev_bits(p.o).copy(), p.lse.cpu().numpy().copy(), p.qs.cpu().numpy().copy()))
    (o1, l1, s1), (o2, l2, s2) = outs
    w = _qs_written(s2, cu)
    assert np.array_equal(s1.view(np.uint32)[w], s2.view(np.uint32)[w])
    assert np.all(s1[~w] == -1.0)  # entries without a query are left alone
    assert np.array_equal(o1, o2)
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


def test_config2_full_size():
    """The SageAttention workload at full size (B=8, lens U{512..4096}, 32/8
    heads, D=128): codes and scales bit-exact everywhere, and every output
    row of every head against the oracle."""
    x = gen.config2()
    sm = x["sm_scale"]
    p, mx = _sage_flow(x, sm)
    cu = x["cu_seqlens"]
    qc, qs, kc, ks = _sage_ref(x, mx, sm, True)
    assert np.array_equal(p.kc.cpu().numpy(), kc)
    w = _qs_written(qs, cu)
    assert np.array_equal(p.qs.cpu().numpy().view(np.uint32)[w], qs.view(np.uint32)[w])
    assert np.array_equal(p.ks.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    ref = prefill_varlen(dequant_int8_per_block(qc, qs, cu), dequant_int8_per_block(kc, ks, cu),
                         as_f32(x["v"], "fp16").astype(np.float64), cu, cu, sm, True, "fp16")
    st = compare_outputs(decode_out(from_dev_bits(p.o), "fp16"), ref["o"], ref["o_exact"], "fp16", "config2")
    st["lse_max_err"] = compare_lse(p.lse.cpu().numpy(), ref["lse"], "config2")
    print("PARITY config2 (every row):", st)


def test_config5_full_size_four_heads():
    """Long fp8 prefill with RoPE + paged append at full size (S=32768, 64
    heads, D=128, 0.1% outliers x20, page 64): for 4 sampled heads the
    rotated Q/K, the cache rows, the fp8 codes/descales are bit-exact, and
    every output row of those heads matches the oracle; every output of
    every head is finite."""
    from oracle.rope import append_kv_rope
    from paged_kv_amd.pipeline import AppendRopeFp8Prefill
    x = gen.config5()
    S, H, D, ps = 32768, 64, 128, x["page_size"]
    kc = torch.zeros((x["num_pages"], ps, H, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    p = AppendRopeFp8Prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), to_dev(x["cu_seqlens"]),
                             to_dev(x["kv_len_before"]), S, to_dev(x["rope_cos_sin"]), kc, vc,
                             to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]), ps, x["sm_scale"],
                             want_lse=True)
    p.run()
    torch.cuda.synchronize()
    assert torch.isfinite(p.prefill.o.float()).all()
    rng = np.random.default_rng(5)
    hs = np.sort(rng.choice(H, 4, replace=False))
    sub = lambda a: np.ascontiguousarray(a[:, hs])
    ref = append_kv_rope(sub(x["q"]), sub(x["k"]), sub(x["v"]), "bf16", x["cu_seqlens"], x["kv_len_before"],
                         x["rope_cos_sin"], np.zeros((x["num_pages"], ps, 4, D), np.uint16),
                         np.zeros((x["num_pages"], ps, 4, D), np.uint16), x["kv_indptr"], x["kv_indices"], ps)
    q_rot, k_rot = ref[0], ref[1]
    assert np.array_equal(from_dev_bits(p.q[:, hs.tolist()]), q_rot)
    assert np.array_equal(from_dev_bits(p.k[:, hs.tolist()]), k_rot)
    assert np.array_equal(from_dev_bits(kc[:, :, hs.tolist()]), ref[2])
    assert np.array_equal(from_dev_bits(vc[:, :, hs.tolist()]), ref[3])
    qc, qs = quant_fp8_per_head(q_rot, "bf16")
    kq, ks = quant_fp8_per_head(k_rot, "bf16")
    vq, vs = quant_fp8_per_head(sub(x["v"]), "bf16")
    pf = p.prefill
    assert np.array_equal(dev_u8(pf.qc[:, hs.tolist()]), qc)
    assert np.array_equal(dev_u8(pf.kc[:, hs.tolist()]), kq)
    assert np.array_equal(pf.qs.cpu().numpy()[hs].view(np.uint32), qs.view(np.uint32))
    assert np.array_equal(pf.vs.cpu().numpy()[hs].view(np.uint32), vs.view(np.uint32))
    cu = x["cu_seqlens"]
    qd, kd, vd = dequant_fp8_per_head(qc, qs), dequant_fp8_per_head(kq, ks), dequant_fp8_per_head(vq, vs)
    got_all = decode_out(from_dev_bits(pf.o[:, hs.tolist()]), "bf16")
    lse_all = pf.lse.cpu().numpy()[hs]
    # every row of the 4 heads, in chunks of 1024 query rows; a chunk is
    # given only the keys its rows can see (causal: keys past the chunk's
    # last row are masked for all of them, and masked keys add exactly
    # nothing), chunks spread over a few threads
    from concurrent.futures import ThreadPoolExecutor
    from oracle.attention import attend
    from oracle.numerics import round_bf16
    o_ex = np.empty((S, 4, D))
    lse = np.empty((4, S), np.float32)

    def chunk(jc):
        j, c = jc
        e = c + 1024
        o, l = attend(qd[c:e, j], kd[:e, j], vd[:e, j], x["sm_scale"], np.arange(c, e) + 1)
        o_ex[c:e, j], lse[j, c:e] = o, l.astype(np.float32)

    with ThreadPoolExecutor(4) as ex:
        list(ex.map(chunk, [(j, c) for j in range(4) for c in range(0, S, 1024)]))
    o_r = round_bf16(o_ex)
    st = compare_outputs(got_all, o_r, o_ex, "bf16", f"c5 heads {hs.tolist()}")
    st["lse_max_err"] = compare_lse(lse_all, lse, "c5")
    print(f"PARITY config5 (every row of heads {hs.tolist()}):", st)
