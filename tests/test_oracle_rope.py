"""Pins of oracle.rope: rotation and paged append (CPU)."""
import numpy as np

import gen
from oracle import brute
from oracle.numerics import bf16_bits_to_f32, bf16_bits_to_f64
from oracle.rope import append_kv_rope, rotate


def _inputs(seed=11, lens=(5, 9), before=(0, 3), hq=4, hkv=2, d=8, ps=4):
    x = gen.long_prefill_inputs(seed, list(lens), hq, hkv, d, ps, outlier_p=0.0,
                                kv_len_before=list(before), spare_frac=0.5)
    pool = x["num_pages"]
    kc = np.full((pool, ps, hkv, d), 0x7FC0, np.uint16)
    vc = kc.copy()
    return x, kc, vc


def _run(x, kc, vc):
    return append_kv_rope(x["q"], x["k"], x["v"], "bf16", x["cu_seqlens"], x["kv_len_before"],
                          x["rope_cos_sin"], kc, vc, x["kv_indptr"], x["kv_indices"], x["page_size"])


def test_table_position_zero_is_identity():
    tab = gen.rope_cos_sin_table(4, 8)
    assert np.all(tab[0, :, 0] == 1) and np.all(tab[0, :, 1] == 0)
    x = np.random.default_rng(0).standard_normal((1, 3, 8)).astype(np.float32)
    assert np.array_equal(rotate(x, tab[:1]), x)


def test_rotation_vs_scalar_brute():
    x, kc, vc = _inputs()
    q_rot, k_rot, *_ = _run(x, kc, vc)
    pos = np.concatenate([np.arange(5), 3 + np.arange(9)])
    q32 = bf16_bits_to_f32(x["q"])
    for t in range(14):
        for h in range(4):
            y = brute.rope_token(q32[t, h], x["rope_cos_sin"][pos[t]])
            assert np.array_equal(bf16_bits_to_f32(q_rot[t, h]), bf16_bits_to_f32(gen.bf16_bits(y)))


def test_rotation_within_one_ulp_of_fp64_and_norm():
    x, kc, vc = _inputs(d=16, lens=(40,), before=(100,))
    q_rot, *_ = _run(x, kc, vc)
    pos = 100 + np.arange(40)
    inv = 10000.0 ** (-2.0 * np.arange(8) / 16)
    ang = pos[:, None] * inv[None]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    q = bf16_bits_to_f64(x["q"])
    y = np.concatenate([q[..., :8] * c - q[..., 8:] * s, q[..., 8:] * c + q[..., :8] * s], -1)
    got = bf16_bits_to_f64(q_rot)
    _, ex = np.frexp(np.abs(y))
    ulp = np.exp2(ex - 1 - 7.0)
    assert np.all(np.abs(got - y) <= ulp * 1.01 + 1e-30)
    # each (i, i + D/2) pair keeps its length (exact rotation in fp64)
    n0 = q[..., :8] ** 2 + q[..., 8:] ** 2
    n1 = y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=1e-12)


def test_relative_position_property_fp64():
    rng = np.random.default_rng(3)
    d = 16
    inv = 10000.0 ** (-2.0 * np.arange(d // 2) / d)
    q, k = rng.standard_normal(d), rng.standard_normal(d)

    def rot(v, p):
        c, s = np.cos(p * inv), np.sin(p * inv)
        return np.concatenate([v[:d // 2] * c - v[d // 2:] * s, v[d // 2:] * c + v[:d // 2] * s])
    a = rot(q, 7) @ rot(k, 3)
    b = rot(q, 104) @ rot(k, 100)
    assert abs(a - b) < 1e-12


def test_cache_placement_and_untouched_slots():
    x, kc, vc = _inputs()
    q_rot, k_rot, kc2, vc2, *_ = _run(x, kc, vc)
    ps = 4
    # sequence 1 token 0 has position 3 -> its page 0, slot 3
    page = x["kv_indices"][x["kv_indptr"][1] + 0]
    assert np.array_equal(kc2[page, 3], k_rot[5])
    assert np.array_equal(vc2[page, 3], x["v"][5])
    # sequence 1 token 6 -> position 9 -> its page 2, slot 1
    page = x["kv_indices"][x["kv_indptr"][1] + 2]
    assert np.array_equal(kc2[page, 1], k_rot[11])
    # slots before kv_len_before and spare pages stay untouched
    page0 = x["kv_indices"][x["kv_indptr"][1]]
    assert np.all(kc2[page0, :3] == 0x7FC0)
    used = set(x["kv_indices"].tolist())
    for p in range(x["num_pages"]):
        if p not in used:
            assert np.all(kc2[p] == 0x7FC0) and np.all(vc2[p] == 0x7FC0)
    del ps


def test_chunked_append_equals_one_shot():
    x, kc, vc = _inputs(lens=(10,), before=(0,))
    one = _run(x, kc, vc)
    # split the same 10 tokens into 4 + 6
    a = dict(x)
    a.update(q=x["q"][:4], k=x["k"][:4], v=x["v"][:4], cu_seqlens=np.array([0, 4], np.int32),
             kv_len_before=np.array([0], np.int32))
    ra = _run(a, kc, vc)
    b = dict(x)
    b.update(q=x["q"][4:], k=x["k"][4:], v=x["v"][4:], cu_seqlens=np.array([0, 6], np.int32),
             kv_len_before=np.array([4], np.int32))
    rb = _run(b, ra[2], ra[3])
    assert np.array_equal(rb[2], one[2]) and np.array_equal(rb[3], one[3])
    assert np.array_equal(np.concatenate([ra[0], rb[0]]), one[0])


def test_fused_amax_matches_rotated_values():
    x, kc, vc = _inputs()
    q_rot, k_rot, _, _, aq, ak, av = _run(x, kc, vc)
    assert np.array_equal(aq, np.abs(bf16_bits_to_f32(q_rot)).max(axis=(0, 2)))
    assert np.array_equal(ak, np.abs(bf16_bits_to_f32(k_rot)).max(axis=(0, 2)))
    assert np.array_equal(av, np.abs(bf16_bits_to_f32(x["v"])).max(axis=(0, 2)))
