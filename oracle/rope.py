"""RoPE + paged KV-cache append (oracle: test infrastructure only).

PaddleNLP "Sage Attention Support Varlen & write kv cache BF16/FP16": the
new Q/K/V of a varlen batch get the rotary embedding and K/V are written
into a paged BF16/FP16 cache; the paging follows FlashInfer's
"[Refactor] Unify JIT/Customization/AOT mode" (paged_kv_indptr /
paged_kv_indices, page_size) and its rope_theta parameter.

Readings where the pages are silent:
  * rotate-half ("NeoX") RoPE; the caller supplies an fp32 table
    cos_sin[pos, i] = (cos, sin)(pos * theta^(-2 i / D)), i < D/2;
  * token i of sequence b has position kv_len_before[b] + i;
  * Q and K are rotated in place, V is not rotated;
  * arithmetic in fp32, each product and sum rounded separately:
        y[i]       = (x[i] * c[i]) - (x[i + D/2] * s[i])
        y[i + D/2] = (x[i + D/2] * c[i]) + (x[i] * s[i])
    then one round-to-nearest-even to the 16-bit storage type;
  * cache layout NHD [num_pages, page_size, H_kv, D]; position p of
    sequence b lives in page kv_indices[kv_indptr[b] + p // page_size],
    slot p % page_size;
  * the optional fused amax outputs are max |value| per head over the new
    rows of the rotated Q, rotated K and V, as stored (16-bit) -- exactly
    what a following per-head quantizer would compute.

Pins (tests/test_oracle_rope.py): position 0 is the identity; the fp32 path
stays within one 16-bit ulp of an fp64 rotation; the rotation preserves
each pair's norm; q.k depends only on the position difference (fp64);
appending in two chunks equals appending in one.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_to_f32, to_bf16_bits, to_fp16


def _load(x, dtype):
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    return np.asarray(x, np.float16).astype(np.float32)


def _store(y32, dtype):
    if dtype == "bf16":
        return to_bf16_bits(y32.astype(np.float64))
    return to_fp16(y32.astype(np.float64))


def rotate(x32: np.ndarray, cs: np.ndarray) -> np.ndarray:
    """x32 [N, H, D] fp32, cs [N, D/2, 2] fp32 -> rotated fp32 [N, H, D]."""
    half = x32.shape[-1] // 2
    c = cs[:, None, :, 0]
    s = cs[:, None, :, 1]
    x1, x2 = x32[..., :half], x32[..., half:]
    y = np.empty_like(x32)
    y[..., :half] = (x1 * c).astype(np.float32) - (x2 * s).astype(np.float32)
    y[..., half:] = (x2 * c).astype(np.float32) + (x1 * s).astype(np.float32)
    return y


def positions(cu_seqlens, kv_len_before) -> np.ndarray:
    t = int(cu_seqlens[-1])
    pos = np.zeros(t, np.int64)
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        pos[s0:s1] = int(kv_len_before[b]) + np.arange(s1 - s0)
    return pos


def append_kv_rope(q, k, v, dtype, cu_seqlens, kv_len_before, cos_sin,
                   k_cache, v_cache, kv_indptr, kv_indices, page_size):
    """Returns (q_rot, k_rot, k_cache', v_cache', amax_q, amax_k, amax_v).

    Inputs are not modified; the cache arrays returned are updated copies."""
    pos = positions(cu_seqlens, kv_len_before)
    cs = cos_sin[pos]
    q_rot = _store(rotate(_load(q, dtype), cs), dtype)
    k_rot = _store(rotate(_load(k, dtype), cs), dtype)
    kc, vc = k_cache.copy(), v_cache.copy()
    for b in range(len(cu_seqlens) - 1):
        s0, s1 = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
        for i in range(s1 - s0):
            p = int(kv_len_before[b]) + i
            page = int(kv_indices[int(kv_indptr[b]) + p // page_size])
            kc[page, p % page_size] = k_rot[s0 + i]
            vc[page, p % page_size] = v[s0 + i]

    def amax(a):
        a32 = np.abs(_load(a, dtype))
        return a32.max(axis=(0, 2)).astype(np.float32) if a32.shape[0] else np.zeros(a32.shape[1], np.float32)
    return q_rot, k_rot, kc, vc, amax(q_rot), amax(k_rot), amax(v)
