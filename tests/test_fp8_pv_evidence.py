"""Whether the PV product could take P in fp8 (the fourth "next" row: fp8 PV
with error control), settled on the CPU with the c1 and c5 inputs.

The aiter page's fp8 attention hands fp8 V with its descale to the kernel;
the question is whether P itself may also be fp8.  This file simulates the
PV step of a tiled kernel on exact fp64 logits (the oracle's quantized Q/K/V,
so everything but P is as in the shipped path) and applies the comparison
rule to the result:

  fp16 P   p rounded to fp16 (what the prefill does)              -> holds
  fp8 P    p * 2^8 rounded to e4m3fn (RNE, saturating), / 2^8    -> fails
  mass-controlled fp8 P: a 64-key tile goes fp8 only while its mass is at
           most tau = 1/64 of the row's running sum, else fp16    -> fails (c5)

Every variant gets the exact row max (p <= 1, the best case for fp8) and
normalizes by the sum of its own rounded P.  The failing max-abs errors are
printed; the conclusion (PV stays fp16) is what the prefill implements.
"""
import numpy as np
import pytest

import gen
from oracle.attention import dequant_fp8_per_head
from oracle.numerics import e4m3fn_decode, e4m3fn_encode, round_bf16, round_fp16
from oracle.quant import quant_fp8_per_head
from tests.parity import compare_outputs

TAU = 1.0 / 64
TILE = 64


def _pv(s_row: np.ndarray, v: np.ndarray, variant: str) -> np.ndarray:
    """One query row: exact logits s_row [L] -> O [D] with P rounded as the
    variant says."""
    p = np.exp(s_row - s_row.max())                     # exact, <= 1
    p16 = round_fp16(p)
    if variant == "fp16":
        pr = p16
    elif variant == "fp8":
        pr = e4m3fn_decode(e4m3fn_encode((p * 256.0).astype(np.float32))) / 256.0
    elif variant == "tau":
        p8 = e4m3fn_decode(e4m3fn_encode((p * 256.0).astype(np.float32))) / 256.0
        pr = p16.copy()
        run = 0.0
        for t0 in range(0, p.size, TILE):
            t1 = min(p.size, t0 + TILE)
            mass = p[t0:t1].sum()
            if run > 0.0 and mass <= TAU * run:
                pr[t0:t1] = p8[t0:t1]
            run += mass
    else:
        raise ValueError(variant)
    return (pr @ v) / pr.sum()


def _rows(qd, kd, vd, sm_scale, rows, variant):
    """Causal rows of one head (L_q == L_k): list of (row index) -> O [n, D]."""
    out = np.empty((len(rows), vd.shape[1]))
    for n, i in enumerate(rows):
        s = sm_scale * (kd[: i + 1] @ qd[i])
        out[n] = _pv(s, vd[: i + 1], variant)
    return out


def _exact(qd, kd, vd, sm_scale, rows):
    out = np.empty((len(rows), vd.shape[1]))
    for n, i in enumerate(rows):
        s = sm_scale * (kd[: i + 1] @ qd[i])
        p = np.exp(s - s.max())
        out[n] = (p @ vd[: i + 1]) / p.sum()
    return out


def _verdict(got, exact, label):
    try:
        st = compare_outputs(round_bf16(got), round_bf16(exact), exact, "bf16", label)
        return True, st
    except AssertionError as e:
        err = np.abs(round_bf16(got) - round_bf16(exact))
        return False, {"max_abs": float(err.max()), "mean_abs": float(err.mean()), "why": str(e)[:60]}


def test_fp8_p_fails_on_config1():
    x = gen.config1()
    cu = x["cu_seqlens"]
    q = dequant_fp8_per_head(*quant_fp8_per_head(x["q"], "bf16"))
    k = dequant_fp8_per_head(*quant_fp8_per_head(x["k"], "bf16"))
    v = dequant_fp8_per_head(*quant_fp8_per_head(x["v"], "bf16"))
    res = {}
    for variant in ("fp16", "fp8", "tau"):
        got, ex = [], []
        for b in range(len(cu) - 1):
            s0, s1 = int(cu[b]), int(cu[b + 1])
            for h in range(2):
                rows = list(range(s1 - s0))
                got.append(_rows(q[s0:s1, h], k[s0:s1, h], v[s0:s1, h], x["sm_scale"], rows, variant))
                ex.append(_exact(q[s0:s1, h], k[s0:s1, h], v[s0:s1, h], x["sm_scale"], rows))
        res[variant] = _verdict(np.concatenate(got), np.concatenate(ex), f"c1 {variant}")
    print("config1:", res)
    assert res["fp16"][0], res["fp16"]
    assert not res["fp8"][0] and res["fp8"][1]["max_abs"] > 2e-2


@pytest.mark.slow
def test_fp8_p_fails_on_config5():
    """c5 inputs (S=32768, 0.1% outliers x20): RoPE and fp8 per-head
    quantization of 2 heads by the oracle, then 192 rows per head drawn at
    random (the last rows of the sequence among them: the most keys)."""
    from oracle.rope import append_kv_rope
    x = gen.config5()
    S, ps = 32768, x["page_size"]
    rng = np.random.default_rng(8)
    res = {v: [[], []] for v in ("fp16", "fp8", "tau")}
    for h in (0, 37):
        one = lambda a: np.ascontiguousarray(a[:, h:h + 1])
        zero = np.zeros((x["num_pages"], ps, 1, 128), np.uint16)
        r = append_kv_rope(one(x["q"]), one(x["k"]), one(x["v"]), "bf16", x["cu_seqlens"], x["kv_len_before"],
                           x["rope_cos_sin"], zero, zero.copy(), x["kv_indptr"], x["kv_indices"], ps)
        q = dequant_fp8_per_head(*quant_fp8_per_head(r[0], "bf16"))[:, 0]
        k = dequant_fp8_per_head(*quant_fp8_per_head(r[1], "bf16"))[:, 0]
        v = dequant_fp8_per_head(*quant_fp8_per_head(one(x["v"]), "bf16"))[:, 0]
        rows = sorted(set(rng.integers(0, S, size=176).tolist()) | set(range(S - 16, S)))
        ex = _exact(q, k, v, x["sm_scale"], rows)
        for variant in res:
            res[variant][0].append(_rows(q, k, v, x["sm_scale"], rows, variant))
            res[variant][1].append(ex)
    out = {v: _verdict(np.concatenate(g), np.concatenate(e), f"c5 {v}") for v, (g, e) in res.items()}
    print("config5:", out)
    assert out["fp16"][0], out["fp16"]
    assert not out["fp8"][0] and out["fp8"][1]["max_abs"] > 2e-2
    assert not out["tau"][0] and out["tau"][1]["max_abs"] > 2e-2
