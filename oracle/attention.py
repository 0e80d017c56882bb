"""Attention steps of the path as plain definitions (oracle: test infrastructure only).

The method computes O = softmax(scale * Dequant(Q) Dequant(K)^T + mask)
Dequant(V) (the Ascend "KvQuantSparseFlashAttention" formula, with
Dequant(x, s) = x * s).  Flash tiling, split-KV and sparse gathering all
reach exactly this result up to rounding order, so the oracle is the
definition itself: dequantize to fp64 and run an exact two-pass softmax
(row max first, then exp / sum / weighted sum).

Readings where the pages are silent or garbled:
  * causal masks are bottom-right aligned (the Ascend page's
    rightDownCausal): query i of a sequence with L_q queries and L_k keys
    sees key j iff j <= i + L_k - L_q (top-left when L_q == L_k);
  * grouped heads: q head h reads kv head h // (H_q / H_kv);
  * the default scale is 1 / sqrt(d_k) (aiter's softmax_scale=None; the
    Ascend scale_value); callers pass it explicitly;
  * lse is the natural-log log-sum-exp of the scaled logits (FlashInfer's
    maybe_lse); a row with no visible key has O = 0 and lse = -inf;
  * outputs are rounded once from fp64 to bf16 / fp16.

Functions:
  prefill_varlen     FlashInfer's ragged batch prefill / aiter's
                     flash_attn_func with fp8 or per-block int8 Q/K
  decode_paged       FlashInfer's batch decode over a paged KV cache
                     (indptr / indices / last_page_len), fp8 K/V with
                     per-head descales (aiter's paged fp8 flash_attn_with_kvcache)
  sparse_mla_decode  the Ascend operator: MLA-absorb, 656-byte combined rows
                     (int8 or fp8 e4m3 nope codes), per-token tile-128 scales,
                     block_table, sparse_indices, sparse_block_size, sparse_mode
                     0 or 3; sparse_mla_tokens states which tokens a query
                     row uses
  prefill_paged      a prefill chunk over a paged fp8 cache (FlashInfer's paged
                     prefill run; aiter's flash_attn_with_kvcache, fp8 cache)
  ragged_from_pages  a paged cache read back into the ragged [T, H, D] layout
  dequant_*          code * scale for fp8 per head / per channel and int8 per block
  lse_merge          combination of split partials (O_c, lse_c)

Pins (tests/test_oracle_attention.py): pure-Python brute force
(oracle.brute) on tiny random shapes, and invariants -- one visible key
gives that V row; constant V gives V; scale 0 gives the mean of the visible
V rows and lse = ln(n); V = 1 gives 1 (rows of P sum to 1); garbage in the
masked tail has no effect; the two-key closed form; split + merge equals
no split; page permutation invariance; sparse over all tokens equals dense;
block-sparse equals its token expansion; the right-down causal mode equals
mode 0 on the filtered indices; a page walk and the append round trip for
ragged_from_pages; K smoothing leaves the softmax output unchanged.
"""
from __future__ import annotations

import math

import numpy as np

from .numerics import (e4m3fn_decode, bf16_bits_to_f64, round_bf16, round_fp16,
                       to_bf16_bits, to_fp16)

MLA_NOPE, MLA_ROPE, MLA_TILE = 512, 64, 128
MLA_ROW = MLA_NOPE + 2 * MLA_ROPE + 4 * (MLA_NOPE // MLA_TILE)


# ---------------------------------------------------------------------------
# dequantization
# ---------------------------------------------------------------------------
def dequant_fp8_per_head(codes: np.ndarray, descale: np.ndarray) -> np.ndarray:
    """codes [T, H, D] uint8, descale [H] -> fp64 values code * descale."""
    return e4m3fn_decode(codes) * np.asarray(descale, np.float64)[None, :, None]


def dequant_fp8_per_channel(codes: np.ndarray, descale: np.ndarray, cu_seqlens) -> np.ndarray:
    """codes [T, H, D] uint8, descale [B, H, D] -> fp64 values code * descale
    of the token's sequence."""
    out = np.zeros(codes.shape, np.float64)
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        out[s0:s1] = e4m3fn_decode(codes[s0:s1]) * np.asarray(descale[b], np.float64)[None, :, :]
    return out


def dequant_int8_per_block(codes: np.ndarray, scales: np.ndarray, cu_seqlens,
                           block_tokens: int = 128) -> np.ndarray:
    """codes [T, H, D] int8, scales [B, H, nblk] -> fp64 values."""
    out = np.zeros(codes.shape, np.float64)
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        blk = np.arange(s1 - s0) // block_tokens
        sc = np.asarray(scales[b], np.float64)[:, blk].T        # [L, H]
        out[s0:s1] = codes[s0:s1].astype(np.float64) * sc[:, :, None]
    return out


# ---------------------------------------------------------------------------
# exact two-pass softmax attention
# ---------------------------------------------------------------------------
def attend(qd: np.ndarray, kd: np.ndarray, vd: np.ndarray, sm_scale: float,
           n_visible: np.ndarray):
    """qd [n, D], kd [L, Dk], vd [L, Dv] fp64; query r sees keys [0, n_visible[r]).

    Returns (O [n, Dv] fp64, lse [n] fp64)."""
    n, L = qd.shape[0], kd.shape[0]
    o = np.zeros((n, vd.shape[1]), np.float64)
    lse = np.full(n, -np.inf)
    if n == 0 or L == 0:
        return o, lse
    s = float(sm_scale) * (qd @ kd.T)                          # [n, L]
    vis = np.arange(L)[None, :] < np.asarray(n_visible)[:, None]
    s = np.where(vis, s, -np.inf)
    has = vis.any(axis=1)
    m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)     # pass 1: row max
    e = np.where(vis, np.exp(s - m[:, None]), 0.0)             # pass 2
    l = e.sum(axis=1)
    lsafe = np.where(has, l, 1.0)
    p = e / lsafe[:, None]
    if np.isfinite(vd).all():
        # invisible keys have p == 0 exactly, so they add exactly nothing
        o = p @ vd
    else:
        # a masked key must contribute nothing even if its V row is not
        # finite (0 * inf would be NaN): sum over each row's visible keys
        for r in range(n):
            nv = int(n_visible[r])
            if nv > 0:
                o[r] = p[r, :nv] @ vd[:nv]
    o = np.where(has[:, None], o, 0.0)
    lse = np.where(has, m + np.log(lsafe), -np.inf)
    return o, lse


def causal_visible(lq: int, lk: int, causal: bool) -> np.ndarray:
    i = np.arange(lq)
    if not causal:
        return np.full(lq, lk)
    return np.clip(i + lk - lq + 1, 0, lk)


def _round_out(o: np.ndarray, out_dtype: str):
    if out_dtype == "bf16":
        return round_bf16(o), to_bf16_bits(o)
    if out_dtype == "fp16":
        return round_fp16(o), to_fp16(o)
    raise ValueError(out_dtype)


def prefill_varlen(qd, kd, vd, cu_q, cu_k, sm_scale, causal, out_dtype="bf16",
                   rows=None):
    """Varlen batch prefill on dequantized fp64 Q [Tq,Hq,D], K/V [Tk,Hkv,D].

    ``rows`` (optional): a list of (b, h, row indices within sequence b)
    restricting the computation; the result then holds only those rows.

    Returns dict: o_exact fp64 [Tq,Hq,D], o (rounded, fp64), o_store
    (bf16 bits / fp16), lse fp32 [Hq, Tq]; or, with ``rows``, a list of
    (b, h, idx, o_exact, o, lse)."""
    tq, hq, d = qd.shape
    hkv = kd.shape[1]
    grp = hq // hkv
    nb = len(cu_q) - 1

    def one(b, h, idx):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        nvis = causal_visible(q1 - q0, k1 - k0, causal)[idx]
        return attend(qd[q0 + idx, h], kd[k0:k1, h // grp], vd[k0:k1, h // grp], sm_scale, nvis)

    if rows is not None:
        res = []
        for b, h, idx in rows:
            idx = np.asarray(idx, np.int64)
            o, lse = one(b, h, idx)
            res.append((b, h, idx, o, _round_out(o, out_dtype)[0], lse.astype(np.float32)))
        return res
    o_ex = np.zeros((tq, hq, vd.shape[2]), np.float64)
    lse = np.full((hq, tq), -np.inf)
    for b in range(nb):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        for h in range(hq):
            o, l = one(b, h, np.arange(q1 - q0))
            o_ex[q0:q1, h] = o
            lse[h, q0:q1] = l
    r, st = _round_out(o_ex, out_dtype)
    return {"o_exact": o_ex, "o": r, "o_store": st, "lse": lse.astype(np.float32)}


# ---------------------------------------------------------------------------
# paged decode
# ---------------------------------------------------------------------------
def paged_kv_len(kv_indptr, kv_last_page_len, page_size) -> np.ndarray:
    npg = np.diff(np.asarray(kv_indptr, np.int64))
    return np.where(npg > 0, (npg - 1) * page_size + np.asarray(kv_last_page_len, np.int64), 0)


def gather_pages(cache: np.ndarray, kv_indptr, kv_indices, b: int, kv_len: int) -> np.ndarray:
    """Tokens [0, kv_len) of sequence b from an NHD page pool -> [kv_len, H, D]."""
    ps = cache.shape[1]
    t = np.arange(kv_len)
    pages = np.asarray(kv_indices)[int(kv_indptr[b]) + t // ps]
    return cache[pages, t % ps]


def ragged_from_pages(cache: np.ndarray, kv_indptr, kv_indices, kv_last_page_len, cu_k) -> np.ndarray:
    """The paged cache read into the ragged layout a prefill attends to
    (FlashInfer's prefill against a paged KV cache: the pages hold each
    sequence's tokens in order, page kv_indices[kv_indptr[b] + i // page_size],
    slot i % page_size).  Row cu_k[b] + i is token i of sequence b for
    i < min(kv_len[b], cu_k[b+1] - cu_k[b]); rows past kv_len[b] are zero.
    cache [P, page_size, H, D] of any dtype -> [cu_k[-1], H, D]."""
    cu_k = np.asarray(cu_k, np.int64)
    ps = cache.shape[1]
    lens = paged_kv_len(kv_indptr, kv_last_page_len, ps)
    out = np.zeros((int(cu_k[-1]),) + cache.shape[2:], cache.dtype)
    for b in range(len(cu_k) - 1):
        n = int(cu_k[b + 1] - cu_k[b])
        m = min(n, int(lens[b]))
        if m > 0:
            out[cu_k[b]:cu_k[b] + m] = gather_pages(cache, kv_indptr, kv_indices, b, m)
    return out


def decode_paged(q_bits, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices,
                 kv_last_page_len, sm_scale, batches=None):
    """q bf16 bits [B, Hq, D]; fp8 caches [P, page_size, Hkv, D]; descales [Hkv].

    Returns dict with o_exact [B,Hq,D], o (bf16-rounded fp64), o_store (bits),
    lse fp32 [B, Hq] for the batches listed (default all; others stay 0/-inf)."""
    q = bf16_bits_to_f64(q_bits)
    nb, hq, d = q.shape
    hkv = k_cache.shape[2]
    grp = hq // hkv
    ps = k_cache.shape[1]
    lens = paged_kv_len(kv_indptr, kv_last_page_len, ps)
    o_ex = np.zeros((nb, hq, d))
    lse = np.full((nb, hq), -np.inf)
    for b in (range(nb) if batches is None else batches):
        L = int(lens[b])
        kd = dequant_fp8_per_head(gather_pages(k_cache, kv_indptr, kv_indices, b, L), k_scale)
        vd = dequant_fp8_per_head(gather_pages(v_cache, kv_indptr, kv_indices, b, L), v_scale)
        for h in range(hq):
            o, l = attend(q[b, h][None, :], kd[:, h // grp], vd[:, h // grp], sm_scale, np.array([L]))
            o_ex[b, h], lse[b, h] = o[0], l[0]
    r, st = _round_out(o_ex, "bf16")
    return {"o_exact": o_ex, "o": r, "o_store": st, "lse": lse.astype(np.float32)}


def prefill_paged(q_codes, q_scale, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices,
                  kv_last_page_len, cu_q, sm_scale, causal, out_dtype="bf16", rows=None):
    """A prefill chunk against a paged fp8 cache (FlashInfer's prefill over
    paged_kv_indptr / paged_kv_indices / paged_kv_last_page_len; aiter's
    flash_attn_with_kvcache with an fp8 e4m3 cache, a page table and
    descales): q_codes [Tq, Hq, D] e4m3fn with q_scale [Hq]; caches
    [P, page_size, Hkv, D] e4m3fn with k_scale / v_scale [Hkv].  Sequence b's
    keys are its kv_len[b] cached tokens (page kv_indices[kv_indptr[b] +
    t // page_size], slot t % page_size); its queries, rows cu_q[b] ..
    cu_q[b+1], are the last L_q of those positions (the bottom-right causal
    alignment of prefill_varlen).  The pages read into the ragged layout,
    dequantized, then prefill_varlen (same returns, ``rows`` as there)."""
    ps = k_cache.shape[1]
    lens = paged_kv_len(kv_indptr, kv_last_page_len, ps)
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    kd = dequant_fp8_per_head(ragged_from_pages(k_cache, kv_indptr, kv_indices, kv_last_page_len, cu_k), k_scale)
    vd = dequant_fp8_per_head(ragged_from_pages(v_cache, kv_indptr, kv_indices, kv_last_page_len, cu_k), v_scale)
    qd = dequant_fp8_per_head(q_codes, q_scale)
    return prefill_varlen(qd, kd, vd, cu_q, cu_k, sm_scale, causal, out_dtype, rows)


# ---------------------------------------------------------------------------
# sparse MLA-absorb decode
# ---------------------------------------------------------------------------
def mla_decode_row(row: np.ndarray, kv_dtype: str = "int8"):
    """One 656-byte cache row -> (k_nope fp64 [512], rope fp64 [64]); the
    nope codes are int8 or fp8 e4m3fn (Ascend "KvQuantSparseFlashAttention",
    parameter table: key in FLOAT8_E4M3 or INT8)."""
    if kv_dtype == "int8":
        codes = row[:MLA_NOPE].view(np.int8).astype(np.float64)
    elif kv_dtype == "fp8":
        codes = e4m3fn_decode(row[:MLA_NOPE])
    else:
        raise ValueError(kv_dtype)
    rope = bf16_bits_to_f64(row[MLA_NOPE:MLA_NOPE + 2 * MLA_ROPE].view(np.uint16))
    scales = row[MLA_NOPE + 2 * MLA_ROPE:MLA_ROW].view(np.float32).astype(np.float64)
    return codes * np.repeat(scales, MLA_TILE), rope


def sparse_mla_tokens(entries, kv_len: int, s: int, s_q: int, sparse_block_size: int = 1,
                      sparse_mode: int = 0) -> np.ndarray:
    """The token positions one query row attends to (Ascend
    "KvQuantSparseFlashAttention", parameters sparse_indices,
    sparse_block_size, sparse_mode).  Reading: an entry idx >= 0 names the
    sparse_block_size tokens [idx * sbs, idx * sbs + sbs) (tokens of a block
    share its selection); a token is used iff it is below kv_len and, with
    sparse_mode 3 (the lower triangle bounded by the line through the
    bottom-right corner), at most kv_len - s_q + s for query row s.  Negative
    entries are padding; every used occurrence is one softmax term."""
    ent = np.asarray(entries, np.int64)
    ent = ent[ent >= 0]
    tok = (ent[:, None] * sparse_block_size + np.arange(sparse_block_size)[None, :]).ravel()
    lim = kv_len if sparse_mode == 0 else kv_len - s_q + s + 1
    return tok[tok < lim]


def sparse_mla_decode(q_bits, kv_cache, block_table, kv_lens, sparse_indices, sm_scale,
                      batches=None, kv_dtype: str = "int8", sparse_block_size: int = 1,
                      sparse_mode: int = 0):
    """q bf16 bits [B, Sq, H, 576]; kv_cache uint8 [NB, bs, 1, 656];
    block_table [B, *]; kv_lens [B]; sparse_indices [B, Sq, 1, topk].

    The tokens of query row (b, s) are sparse_mla_tokens(...); every one is a
    softmax term.  K = [k_nope | rope] (576-d), V = k_nope (512-d).
    Returns o_exact [B,Sq,H,512], o, o_store, lse fp32 [B,Sq,H]."""
    if sparse_mode not in (0, 3):
        raise ValueError(sparse_mode)
    q = bf16_bits_to_f64(q_bits)
    nb, sq, h, _ = q.shape
    bs = kv_cache.shape[1]
    rows = kv_cache.reshape(-1, MLA_ROW)
    o_ex = np.zeros((nb, sq, h, MLA_NOPE))
    lse = np.full((nb, sq, h), -np.inf)
    for b in (range(nb) if batches is None else batches):
        for s in range(sq):
            idx = sparse_mla_tokens(sparse_indices[b, s, 0], int(kv_lens[b]), s, sq, sparse_block_size,
                                    sparse_mode)
            n = idx.size
            if n == 0:
                continue
            r = block_table[b][idx // bs].astype(np.int64) * bs + idx % bs
            kn = np.empty((n, MLA_NOPE))
            kr = np.empty((n, MLA_ROPE))
            for i in range(n):
                kn[i], kr[i] = mla_decode_row(rows[r[i]], kv_dtype)
            kd = np.concatenate([kn, kr], axis=1)               # [n, 576]
            o, l = attend(q[b, s], kd, kn, sm_scale, np.full(h, n))
            o_ex[b, s], lse[b, s] = o, l
    r_, st = _round_out(o_ex, "bf16")
    return {"o_exact": o_ex, "o": r_, "o_store": st, "lse": lse.astype(np.float32)}


# ---------------------------------------------------------------------------
# log-sum-exp merge of split partials
# ---------------------------------------------------------------------------
def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """o_parts [C, ..., D], lse_parts [C, ...] -> (O, lse).

    lse = ln sum_c exp(lse_c); O = sum_c exp(lse_c - lse) O_c; parts with
    lse_c = -inf weigh 0; if all are -inf, O = 0 and lse = -inf."""
    lp = np.asarray(lse_parts, np.float64)
    m = lp.max(axis=0)
    fin = np.isfinite(m)
    msafe = np.where(fin, m, 0.0)
    w = np.where(np.isfinite(lp), np.exp(lp - msafe[None]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(fin, msafe + np.log(np.where(fin, tot, 1.0)), -np.inf)
    wn = np.where(fin[None], w / np.where(fin, tot, 1.0)[None], 0.0)
    o = (wn[..., None] * np.asarray(o_parts, np.float64)).sum(axis=0)
    return o, lse


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)
