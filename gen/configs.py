"""Seeded generators for the five workloads of the quantized-attention path.

Every generator takes an explicit seed and sizes, so the same function makes
the small parity cases and the full-size benchmark inputs.  The ``config*``
functions fix the sizes of the five named workloads:

  config1  tiny varlen causal FP8 prefill (B=2, lens 37/64, H=2, D=64)
  config2  SageAttention-style varlen INT8 prefill (B=8, lens U{512..4096},
           H_q=32, H_kv=8, D=128, 1% channels with an N(0, 4) offset)
  config3  paged FP8 decode (B=64, kv lens U{1024..32768}, page 16, H_q=32,
           H_kv=8, D=128, permuted page pool)
  config4  MLA-absorb sparse INT8 decode (B=32, 128 heads, 576-d queries,
           65536-token caches in 64-token blocks, 2048 distinct indices)
  config5  long causal FP8 prefill with RoPE + paged append (B=1, S=32768,
           H=64, D=128, 0.1% outliers x20, page 64)

Library casts (torch's bf16 / fp8-e4m3fn conversions) are used only to give
random draws their storage dtype; no quantizer of the method lives here.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "seed_for", "bf16_bits", "fp8_lut_codes",
    "prefill_fp8_inputs", "config1", "paged_prefill_fp8_inputs", "paged_prefill_fp8_workload",
    "sage_inputs", "config2",
    "paged_decode_inputs", "config3",
    "sparse_mla_inputs", "config4",
    "long_prefill_inputs", "config5", "rope_cos_sin_table",
    "paged_prefill_inputs", "paged_prefill_workload", "paged_prefill_workload_lengths",
    "MLA_ROW_BYTES", "MLA_NOPE", "MLA_ROPE", "MLA_TILE",
]

SEED_BASE = 1000

# Combined MLA cache row: 512 int8 nope codes | 64 bf16 rope values |
# 4 fp32 per-128-tile scales  (656 bytes per token).
MLA_NOPE = 512
MLA_ROPE = 64
MLA_TILE = 128
MLA_ROW_BYTES = MLA_NOPE + 2 * MLA_ROPE + 4 * (MLA_NOPE // MLA_TILE)

_CHUNK = 1 << 24


def seed_for(config_index: int) -> int:
    """Seed of workload ``config_index`` (1-based)."""
    return SEED_BASE + int(config_index)


def _torch():
    import torch  # local import: generators are usable without a GPU
    return torch


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Store float32 draws as bf16 (torch's round-to-nearest-even cast)."""
    torch = _torch()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for s in range(0, flat_in.size, _CHUNK):
        t = torch.from_numpy(flat_in[s:s + _CHUNK]).to(torch.bfloat16)
        flat_out[s:s + _CHUNK] = t.view(torch.int16).numpy().view(np.uint16)
    return out


def _normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - s)
        flat[s:s + n] = rng.standard_normal(n, dtype=np.float32)
    return out


def _cu(lens) -> np.ndarray:
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return cu


# ---------------------------------------------------------------------------
# fp8 codes with a normal-like value distribution
# ---------------------------------------------------------------------------
_LUT_CACHE: dict = {}


def _fp8_lut(spread: float) -> np.ndarray:
    """65536 e4m3fn codes at the normal quantiles (k+0.5)/65536, scaled so
    that ``spread`` standard deviations land on the largest finite code."""
    key = float(spread)
    if key not in _LUT_CACHE:
        from scipy.special import ndtri
        torch = _torch()
        p = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
        vals = np.clip(ndtri(p) * (448.0 / spread), -448.0, 448.0).astype(np.float32)
        codes = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        _LUT_CACHE[key] = codes.copy()
    return _LUT_CACHE[key]


def fp8_lut_codes(rng: np.random.Generator, shape, spread: float = 4.5) -> np.ndarray:
    """Random e4m3fn codes whose decoded values follow N(0, (448/spread)^2)."""
    lut = _fp8_lut(spread)
    out = np.empty(shape, dtype=np.uint8)
    flat = out.reshape(-1)
    for s in range(0, flat.size, _CHUNK):
        n = min(_CHUNK, flat.size - s)
        flat[s:s + n] = lut[rng.integers(0, 65536, size=n, dtype=np.uint16)]
    return out


# ---------------------------------------------------------------------------
# varlen FP8 prefill (config 1) and long prefill with append (config 5)
# ---------------------------------------------------------------------------
def _outliers(rng, x: np.ndarray, p: float, mult: float) -> None:
    """Multiply a Binomial(n, p) set of positions (drawn with replacement;
    a repeated position is scaled once) by ``mult`` in place."""
    if p <= 0:
        return
    flat = x.reshape(-1)
    n_out = rng.binomial(flat.size, p)
    idx = rng.integers(0, flat.size, size=n_out, dtype=np.int64)
    flat[idx] *= np.float32(mult)


def prefill_fp8_inputs(seed: int, seqlens, hq: int, hkv: int, d: int,
                       outlier_p: float = 0.0, outlier_mult: float = 20.0) -> dict:
    """bf16 Q/K/V of a varlen batch, N(0,1) with optional outliers.

    Returns cu_seqlens int32[B+1], q [T,hq,d], k/v [T,hkv,d] (bf16 bits)."""
    rng = np.random.default_rng(seed)
    cu = _cu(seqlens)
    t = int(cu[-1])
    out = {"cu_seqlens": cu, "seqlens": np.asarray(seqlens, dtype=np.int32),
           "hq": hq, "hkv": hkv, "d": d}
    for name, h in (("q", hq), ("k", hkv), ("v", hkv)):
        x = _normal_f32(rng, (t, h, d))
        _outliers(rng, x, outlier_p, outlier_mult)
        out[name] = bf16_bits(x)
    return out


def config1() -> dict:
    """Tiny varlen causal FP8 prefill: lens [37, 64], H=2, D=64, scale 1/8."""
    x = prefill_fp8_inputs(seed_for(1), [37, 64], 2, 2, 64)
    x.update(sm_scale=0.125, causal=True, name="c1_tiny_varlen_fp8")
    return x


def rope_cos_sin_table(max_pos: int, d: int, theta: float = 10000.0) -> np.ndarray:
    """Caller-side RoPE table fp32 [max_pos, d/2, 2] = (cos, sin) of
    p * theta^(-2i/d), evaluated in fp64 and stored in fp32."""
    half = d // 2
    inv_freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv_freq[None, :]
    tab = np.empty((max_pos, half, 2), dtype=np.float32)
    tab[:, :, 0] = np.cos(ang)
    tab[:, :, 1] = np.sin(ang)
    return tab


def long_prefill_inputs(seed: int, seqlens, hq: int, hkv: int, d: int,
                        page_size: int, outlier_p: float = 0.001,
                        outlier_mult: float = 20.0, theta: float = 10000.0,
                        kv_len_before=None, spare_frac: float = 0.05) -> dict:
    """Inputs of the RoPE + paged-append + FP8 prefill pipeline.

    New tokens of sequence b sit at positions kv_len_before[b] + i.  The page
    pool holds ceil((before+new)/page_size) pages per sequence plus
    ``spare_frac`` spare pages, in a random physical order; every pool byte
    starts as the bf16 NaN sentinel 0x7FC0 so that unwritten slots are
    recognisable."""
    x = prefill_fp8_inputs(seed, seqlens, hq, hkv, d, outlier_p, outlier_mult)
    rng = np.random.default_rng(seed + 7919)
    b = len(seqlens)
    before = np.zeros(b, np.int32) if kv_len_before is None else np.asarray(kv_len_before, np.int32)
    total = before.astype(np.int64) + np.asarray(seqlens, np.int64)
    npages = [(int(n) + page_size - 1) // page_size for n in total]
    used = int(sum(npages))
    pool = used + int(math.ceil(spare_frac * used))
    perm = rng.permutation(pool).astype(np.int32)
    indptr = _cu(npages)
    x.update(
        kv_len_before=before,
        kv_indptr=indptr,
        kv_indices=perm[:used].copy(),
        num_pages=pool,
        page_size=page_size,
        max_pos=int(total.max()) if b else 0,
        rope_cos_sin=rope_cos_sin_table(max(int(total.max()) if b else 1, 1), d, theta),
        cache_fill=np.uint16(0x7FC0),
    )
    return x


def config5() -> dict:
    """Long causal FP8 prefill with RoPE and paged append: S=32768, H=64."""
    x = long_prefill_inputs(seed_for(5), [32768], 64, 64, 128, 64)
    x.update(sm_scale=1.0 / math.sqrt(128.0), causal=True, name="c5_long_fp8_append")
    return x


# ---------------------------------------------------------------------------
# SageAttention-style INT8 prefill (config 2)
# ---------------------------------------------------------------------------
def sage_inputs(seed: int, seqlens, hq: int, hkv: int, d: int,
                offset_frac: float = 0.01, offset_sd: float = 2.0,
                v_channel_sd: float = 0.0) -> dict:
    """fp16 Q/K/V, N(0,1); in Q and in K (independently) round(frac*H*d)
    distinct (head, channel) pairs get one N(0, offset_sd^2) offset added to
    every token.  v_channel_sd > 0: every (head, channel) of V is multiplied
    by f = exp(N(0, v_channel_sd^2)) / (the largest f of its head), so the
    largest channel of a head stays N(0,1) and the others are smaller
    (drawn after everything else, so the other tensors do not change)."""
    rng = np.random.default_rng(seed)
    cu = _cu(seqlens)
    t = int(cu[-1])
    out = {"cu_seqlens": cu, "seqlens": np.asarray(seqlens, np.int32),
           "hq": hq, "hkv": hkv, "d": d}
    for name, h in (("q", hq), ("k", hkv)):
        x = _normal_f32(rng, (t, h, d))
        n_off = int(round(offset_frac * h * d))
        pairs = rng.choice(h * d, size=n_off, replace=False)
        offs = rng.normal(0.0, offset_sd, size=n_off).astype(np.float32)
        x.reshape(t, h * d)[:, pairs] += offs[None, :]
        out[name] = x.astype(np.float16)
        out[name + "_offset_channels"] = pairs.astype(np.int32)
    v = _normal_f32(rng, (t, hkv, d))
    if v_channel_sd > 0:
        f = np.exp(rng.normal(0.0, v_channel_sd, size=(1, hkv, d)))
        v *= (f / f.max(axis=2, keepdims=True)).astype(np.float32)
    out["v"] = v.astype(np.float16)
    return out


def config2_lengths(seed: int = None, batch: int = 8) -> np.ndarray:
    rng = np.random.default_rng(seed_for(2) if seed is None else seed)
    return rng.integers(512, 4097, size=batch).astype(np.int32)


def config2() -> dict:
    lens = config2_lengths()
    x = sage_inputs(seed_for(2) + 1, lens, 32, 8, 128)
    x.update(sm_scale=1.0 / math.sqrt(128.0), causal=True, block_tokens=128,
             name="c2_sage_int8_varlen")
    return x


# ---------------------------------------------------------------------------
# paged FP8 decode (config 3)
# ---------------------------------------------------------------------------
def paged_decode_inputs(seed: int, kv_lens, hq: int, hkv: int, d: int,
                        page_size: int = 16, spare_frac: float = 0.05,
                        spread: float = 4.5) -> dict:
    """bf16 queries [B,hq,d] and fp8 e4m3fn K/V page pools
    [num_pages, page_size, hkv, d] in NHD order.

    Pages of all sequences are a random permutation of the pool; spare pages
    and the slots past each sequence's end in its last page hold 0x7F (NaN),
    which must never reach an output.  Descales are positive fp32 per kv head.
    A sequence with kv_len 0 owns no page."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, np.int64)
    b = kv_lens.size
    npages = (kv_lens + page_size - 1) // page_size
    used = int(npages.sum())
    pool = used + int(math.ceil(spare_frac * used))
    perm = rng.permutation(pool).astype(np.int32)
    indptr = _cu(npages)
    last = np.where(kv_lens > 0, kv_lens - (npages - 1) * page_size, 0).astype(np.int32)
    q = bf16_bits(_normal_f32(rng, (b, hq, d)))
    caches = {}
    for name in ("k_cache", "v_cache"):
        c = fp8_lut_codes(rng, (pool, page_size, hkv, d), spread)
        c[perm[used:]] = 0x7F
        for i in range(b):
            if kv_lens[i] > 0 and last[i] < page_size:
                c[perm[indptr[i + 1] - 1], last[i]:] = 0x7F
        caches[name] = c
    k_descale = (rng.uniform(0.8, 1.2, size=hkv) * spread / 448.0).astype(np.float32)
    v_descale = (rng.uniform(0.8, 1.2, size=hkv) * spread / 448.0).astype(np.float32)
    return {
        "q": q, "k_cache": caches["k_cache"], "v_cache": caches["v_cache"],
        "k_scale": k_descale, "v_scale": v_descale,
        "kv_indptr": indptr, "kv_indices": perm[:used].copy(),
        "kv_last_page_len": last, "kv_lens": kv_lens.astype(np.int32),
        "num_pages": pool, "page_size": page_size, "hq": hq, "hkv": hkv, "d": d,
        "max_kv_len": int(kv_lens.max()) if b else 0,
    }


def config3_lengths(seed: int = None, batch: int = 64) -> np.ndarray:
    rng = np.random.default_rng(seed_for(3) if seed is None else seed)
    return rng.integers(1024, 32769, size=batch).astype(np.int32)


def config3() -> dict:
    x = paged_decode_inputs(seed_for(3) + 1, config3_lengths(), 32, 8, 128, 16)
    x.update(sm_scale=1.0 / math.sqrt(128.0), name="c3_paged_fp8_decode")
    return x


# ---------------------------------------------------------------------------
# MLA-absorb sparse INT8 decode (config 4)
# ---------------------------------------------------------------------------
def sparse_mla_inputs(seed: int, batch: int, s_q: int, heads: int, kv_len,
                      block_size: int, topk: int, n_valid=None,
                      spare_blocks: int = 0, kv_dtype: str = "int8",
                      sparse_block_size: int = 1) -> dict:
    """bf16 queries [B,S_q,H,576]; combined cache rows
    [num_blocks, block_size, 1, 656]; block_table [B, max_blocks];
    sparse_indices [B, S_q, 1, topk] with the n_valid (default topk) valid,
    distinct, unsorted indices first and -1 after.  An index names the
    sparse_block_size tokens [idx * sbs, idx * sbs + sbs) (sbs = 1: one token).

    Selected rows hold nope codes (int8: a rounded normal; fp8 e4m3: random
    sign, exponent field 0..8 and mantissa, so |value| <= 3.75), bf16 N(0,1)
    rope values and positive fp32 tile scales; every other row holds NaN
    rope values and NaN scales, which must never reach an output."""
    rng = np.random.default_rng(seed)
    kv_len = np.broadcast_to(np.asarray(kv_len, np.int64), (batch,)).copy()
    nblk = (kv_len + block_size - 1) // block_size
    max_blocks = int(nblk.max()) if batch else 0
    used = int(nblk.sum())
    nb = used + spare_blocks
    perm = rng.permutation(nb).astype(np.int32)
    table = np.full((batch, max(max_blocks, 1)), -1, np.int32)
    off = 0
    for b in range(batch):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += int(nblk[b])
    q = bf16_bits(_normal_f32(rng, (batch, s_q, heads, MLA_NOPE + MLA_ROPE)))
    # every row starts as the NaN template
    tmpl = np.zeros(MLA_ROW_BYTES, np.uint8)
    tmpl[:MLA_NOPE] = 0x7F
    tmpl[MLA_NOPE:MLA_NOPE + 2 * MLA_ROPE] = np.full(MLA_ROPE, 0x7FC0, np.uint16).view(np.uint8)
    tmpl[MLA_NOPE + 2 * MLA_ROPE:] = np.full(MLA_NOPE // MLA_TILE, 0x7FC00000, np.uint32).view(np.uint8)
    cache = np.empty((nb, block_size, 1, MLA_ROW_BYTES), np.uint8)
    cache[...] = tmpl
    nvalid = topk if n_valid is None else n_valid
    sbs = int(sparse_block_size)
    idx = np.full((batch, s_q, 1, topk), -1, np.int32)
    for b in range(batch):
        nsb = (int(kv_len[b]) + sbs - 1) // sbs       # sparse blocks holding a token
        for s in range(s_q):
            k = min(int(nvalid), nsb)
            if k > 0:
                idx[b, s, 0, :k] = rng.choice(nsb, size=k, replace=False)
    toks = []
    for b in range(batch):
        t = (idx[b][idx[b] >= 0].astype(np.int64)[:, None] * sbs + np.arange(sbs)[None, :]).ravel()
        t = t[t < kv_len[b]]
        toks.append(table[b][t // block_size].astype(np.int64) * block_size + t % block_size)
    sel = np.unique(np.concatenate(toks)) if batch else np.zeros(0, np.int64)
    rows = cache.reshape(nb * block_size, MLA_ROW_BYTES)
    n = sel.size
    if kv_dtype == "int8":
        codes = np.clip(np.rint(rng.standard_normal((n, MLA_NOPE)) * (127.0 / 3.5)), -127, 127).astype(np.int8)
        rope = bf16_bits(_normal_f32(rng, (n, MLA_ROPE)))
        scales = (rng.uniform(2.8, 4.2, size=(n, MLA_NOPE // MLA_TILE)) / 127.0).astype(np.float32)
    elif kv_dtype == "fp8":
        sign = rng.integers(0, 2, size=(n, MLA_NOPE)) << 7
        expo = rng.integers(0, 9, size=(n, MLA_NOPE)) << 3
        mant = rng.integers(0, 8, size=(n, MLA_NOPE))
        codes = (sign | expo | mant).astype(np.uint8)
        rope = bf16_bits(_normal_f32(rng, (n, MLA_ROPE)))
        scales = rng.uniform(0.5, 1.0, size=(n, MLA_NOPE // MLA_TILE)).astype(np.float32)
    else:
        raise ValueError(kv_dtype)
    rows[sel, :MLA_NOPE] = codes.view(np.uint8)
    rows[sel, MLA_NOPE:MLA_NOPE + 2 * MLA_ROPE] = rope.view(np.uint8)
    rows[sel, MLA_NOPE + 2 * MLA_ROPE:] = scales.view(np.uint8)
    return {
        "q": q, "kv_cache": cache, "block_table": table, "max_blocks_per_seq": table.shape[1],
        "kv_lens": kv_len.astype(np.int32), "sparse_indices": idx, "topk": topk,
        "batch": batch, "s_q": s_q, "heads": heads, "num_blocks": nb,
        "block_size": block_size, "kv_dtype": kv_dtype, "sparse_block_size": sbs,
    }


def config4() -> dict:
    x = sparse_mla_inputs(seed_for(4), 32, 1, 128, 65536, 64, 2048)
    x.update(sm_scale=1.0 / 24.0, name="c4_sparse_mla_int8")
    return x


# ---------------------------------------------------------------------------
# prefill chunk against a paged 16-bit cache (the paged prefill run mode)
# ---------------------------------------------------------------------------
def paged_prefill_inputs(seed: int, kv_lens, q_lens, hq: int, hkv: int, d: int,
                         page_size: int = 64, spare_frac: float = 0.05) -> dict:
    """A prefill chunk whose queries are the last q_lens[b] of kv_lens[b]
    tokens of sequence b, against bf16 K/V page pools [num_pages, page_size,
    hkv, d] (NHD) that already hold all kv_lens[b] tokens (the chunk's own
    keys included, as after the append step).  q: bf16 N(0,1) [sum q_lens,
    hq, d]; K and V: bf16 N(0,1).  Pages of all sequences are a random
    permutation of the pool; spare pages and the unused slots of each last
    page hold the bf16 NaN 0x7FC0, which must never reach an output.
    cu_q / cu_k are the ragged row offsets of the queries and of the keys."""
    rng = np.random.default_rng(seed)
    kv_lens = np.asarray(kv_lens, np.int64)
    q_lens = np.asarray(q_lens, np.int64)
    assert kv_lens.shape == q_lens.shape and np.all(q_lens <= kv_lens)
    b = kv_lens.size
    npages = (kv_lens + page_size - 1) // page_size
    used = int(npages.sum())
    pool = used + int(math.ceil(spare_frac * used))
    perm = rng.permutation(pool).astype(np.int32)
    indptr = _cu(npages)
    last = np.where(kv_lens > 0, kv_lens - (npages - 1) * page_size, 0).astype(np.int32)
    q = bf16_bits(_normal_f32(rng, (int(q_lens.sum()), hq, d)))
    caches = {}
    for name in ("k_cache", "v_cache"):
        c = np.full((pool, page_size, hkv, d), 0x7FC0, np.uint16)
        for i in range(b):
            n = int(kv_lens[i])
            if n == 0:
                continue
            rows = bf16_bits(_normal_f32(rng, (n, hkv, d)))
            pages = perm[indptr[i]:indptr[i + 1]]
            for j, pg in enumerate(pages):
                s0 = j * page_size
                m = min(page_size, n - s0)
                c[pg, :m] = rows[s0:s0 + m]
        caches[name] = c
    return {
        "q": q, "k_cache": caches["k_cache"], "v_cache": caches["v_cache"],
        "kv_indptr": indptr, "kv_indices": perm[:used].copy(), "kv_last_page_len": last,
        "kv_lens": kv_lens.astype(np.int32), "q_lens": q_lens.astype(np.int32),
        "cu_q": _cu(q_lens), "cu_k": _cu(kv_lens),
        "num_pages": pool, "page_size": page_size, "hq": hq, "hkv": hkv, "d": d,
        "max_q": int(q_lens.max()) if b else 0, "max_k": int(kv_lens.max()) if b else 0,
    }


def paged_prefill_fp8_inputs(seed: int, kv_lens, q_lens, hq: int, hkv: int, d: int,
                             page_size: int = 64, spare_frac: float = 0.05) -> dict:
    """A prefill chunk (the last q_lens[b] of kv_lens[b] positions of
    sequence b) against fp8 e4m3fn K/V page pools: the caches, page
    permutation, NaN spare pages and NaN stale slots of paged_decode_inputs,
    plus fp8 query codes [sum q_lens, hq, d] (the same normal-like code
    distribution) with positive per-head descales, and cu_q."""
    kv_lens = np.asarray(kv_lens, np.int64)
    q_lens = np.asarray(q_lens, np.int64)
    assert kv_lens.shape == q_lens.shape and np.all(q_lens <= kv_lens)
    x = paged_decode_inputs(seed, kv_lens, hq, hkv, d, page_size, spare_frac)
    rng = np.random.default_rng(seed + 7919)
    del x["q"]
    x["q"] = fp8_lut_codes(rng, (int(q_lens.sum()), hq, d))
    x["q_scale"] = (rng.uniform(0.8, 1.2, size=hq) * 4.5 / 448.0).astype(np.float32)
    x["q_lens"] = q_lens.astype(np.int32)
    x["cu_q"] = _cu(q_lens)
    x["max_q"] = int(q_lens.max()) if q_lens.size else 0
    return x


def paged_prefill_fp8_workload() -> dict:
    """The chunked-prefill workload (B=4 sequences of kv_len U{8192..24576},
    seeded, each with a 2048-token chunk at its end; 32 q / 8 kv heads,
    D=128, page size 64, causal) over an fp8 e4m3fn cache with per-head
    descales."""
    kv = paged_prefill_workload_lengths()
    x = paged_prefill_fp8_inputs(seed_for(6) + 2, kv, np.full(kv.size, 2048), 32, 8, 128, 64)
    x.update(sm_scale=1.0 / math.sqrt(128.0), name="chunked_prefill_paged_fp8")
    return x


def paged_prefill_workload_lengths(seed: int = None, batch: int = 4):
    rng = np.random.default_rng(seed_for(6) if seed is None else seed)
    return rng.integers(8192, 24577, size=batch).astype(np.int32)


def paged_prefill_workload() -> dict:
    """Chunked prefill against a paged bf16 cache: B=4 sequences of kv_len
    U{8192..24576} (seeded) whose last 2048 tokens are the new chunk, 32 q /
    8 kv heads, D=128, page size 64, causal."""
    kv = paged_prefill_workload_lengths()
    x = paged_prefill_inputs(seed_for(6) + 1, kv, np.full(kv.size, 2048), 32, 8, 128, 64)
    x.update(sm_scale=1.0 / math.sqrt(128.0), name="chunked_prefill_paged_bf16")
    return x
