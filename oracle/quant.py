"""Quantizers of the path (oracle: test infrastructure only).

* ``quant_fp8_per_head`` -- fp8 Q/K/V with one fp32 descale per head
  (aiter "[Triton] FP8 with FA v3 API": the caller hands fp8 q, k, v plus
  their descales; the Ascend formula's Dequant(x, s) = x * s).  Reading: one
  descale per head over every row of the call, descale = amax / 448 with an
  IEEE fp32 division, amax = 0 -> descale 1.
* ``quant_int8_per_block`` -- SageAttention-style INT8 Q/K (PaddleNLP
  "Sage Attention Support Varlen", the varlen "quant qk" kernel).  Reading:
  one fp32 scale per (sequence, head, 128-token block counted from the
  sequence start), scale = amax / 127, codes rint(x / scale) clamped to
  [-127, 127]; no smoothing of K (the pages never mention it).
* ``v_permute`` -- the varlen "quant_transpose_permute v" step of the same
  page: V [T, H, D] -> V^T [B, H, D, S_pad], S_pad = round_up(max_seqlen,
  128), tokens reordered inside each 32-token group by ``pi`` (below), tail
  zero-filled, optionally fp8-encoded with per-head descales.  The pages do
  not state the permutation (it is tied to the attention kernel's operand
  layout); ours is defined here and, independently, in the HIP source.

Token permutation pi inside a 32-token group (j in [0, 32)):
    half = j // 16, g = (j % 16) // 4, r = j % 4  ->  pi(j) = 8 g + 4 half + r
so stored position p = 8 g + s holds token (s // 4) * 16 + 4 g + s % 4.

* ``quant_fp8_per_channel`` -- SageAttention's fp8 V with one descale per
  channel.  The pages give fp8 V only with per-head descales; reading: one
  descale per (sequence, kv head, channel), amax over the sequence's tokens,
  descale = amax / 448 (IEEE fp32), 1 where amax = 0 (so also for an empty
  sequence); codes as in ``quant_fp8_per_head``.  ``v_permute`` takes the
  same option.
* ``channel_mean_fp16`` / ``smooth_quant_k`` -- SageAttention's K smoothing
  before the int8 block quantization: subtract each sequence's per-channel
  mean of K (softmax-invariant).  Reading: exact sum, mean = fp32(fp64(S)/L),
  then codes of fp32(k) - mean.

Pins (tests/test_oracle_quant.py): amax and descale by exhaustive
comparison with a per-element Python max (per head and per channel); codes against the brute-force
nearest-grid encoder; block boundaries at sequence starts; pi is a
bijection and its inverse recovers V bit-exactly; padding is +0; the
channel mean against exact rational arithmetic, its independence of token
order and its exactness on constant channels; smoothing leaves fp64 attention
unchanged (test_oracle_attention.py) and shrinks the int8 error of K on data
with channel offsets.
"""
from __future__ import annotations

import numpy as np

from .numerics import e4m3fn_encode, int8_encode, bf16_bits_to_f32

PERM_GROUP = 32


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """bf16 bits (uint16) or fp16 array -> exact fp32 values ("f32": x as is)."""
    if dtype == "bf16":
        return bf16_bits_to_f32(x)
    if dtype == "fp16":
        return np.asarray(x, dtype=np.float16).astype(np.float32)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def fp8_descale(amax: np.ndarray) -> np.ndarray:
    """descale = fp32(amax) / fp32(448) (IEEE), 1.0 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float32)
    d = amax / np.float32(448.0)
    return np.where(amax == 0, np.float32(1.0), d).astype(np.float32)


def int8_scale(amax: np.ndarray) -> np.ndarray:
    amax = np.asarray(amax, dtype=np.float32)
    s = amax / np.float32(127.0)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def amax_per_head(x32: np.ndarray) -> np.ndarray:
    """max |x| over rows and channels, per head: x32 [T, H, D] -> [H]."""
    if x32.shape[0] == 0:
        return np.zeros(x32.shape[1], np.float32)
    return np.abs(x32).max(axis=(0, 2)).astype(np.float32)


def quant_fp8_per_head(x: np.ndarray, dtype: str, amax_in=None):
    """x [T, H, D] (bf16 bits or fp16) -> (codes uint8 [T,H,D], descale f32[H]).

    ``amax_in`` replaces the reduction when a previous step already produced
    the per-head amax of exactly these values."""
    x32 = as_f32(x, dtype)
    amax = amax_per_head(x32) if amax_in is None else np.asarray(amax_in, np.float32)
    ds = fp8_descale(amax)
    v = x32 / ds[None, :, None]               # fp32 IEEE division
    return e4m3fn_encode(v), ds


def quant_fp8_per_channel(x: np.ndarray, dtype: str, cu_seqlens):
    """x [T, H, D] -> (codes uint8 [T,H,D], descale f32 [B, H, D]): the
    descale of (b, h, c) is fp8_descale of max |x| over sequence b's tokens
    in channel c of head h."""
    x32 = as_f32(x, dtype)
    t, h, d = x32.shape
    cu = np.asarray(cu_seqlens, np.int64)
    b = len(cu) - 1
    codes = np.zeros((t, h, d), np.uint8)
    ds = np.ones((b, h, d), np.float32)
    for bi in range(b):
        s0, s1 = int(cu[bi]), int(cu[bi + 1])
        if s1 > s0:
            ds[bi] = fp8_descale(np.abs(x32[s0:s1]).max(axis=0))
            codes[s0:s1] = e4m3fn_encode(x32[s0:s1] / ds[bi][None, :, :])
    return codes, ds


def quant_int8_per_block(x: np.ndarray, dtype: str, cu_seqlens: np.ndarray,
                         max_seqlen: int, block_tokens: int = 128):
    """x [T, H, D] -> (codes int8 [T,H,D], scales f32 [B, H, ceil(max_seqlen/block)]).

    Block j of sequence b covers rows [cu[b] + j*bt, min(cu[b] + (j+1)*bt, cu[b+1])).
    Scale entries of blocks past a sequence's end are 0.  Rows outside
    [0, cu[B]) are left as 0 codes."""
    x32 = as_f32(x, dtype)
    t, h, d = x32.shape
    b = len(cu_seqlens) - 1
    nblk = (max_seqlen + block_tokens - 1) // block_tokens
    codes = np.zeros((t, h, d), np.int8)
    scales = np.zeros((b, h, nblk), np.float32)
    for bi in range(b):
        s0, s1 = int(cu_seqlens[bi]), int(cu_seqlens[bi + 1])
        for j in range((s1 - s0 + block_tokens - 1) // block_tokens):
            r0, r1 = s0 + j * block_tokens, min(s0 + (j + 1) * block_tokens, s1)
            blk = x32[r0:r1]                           # [rows, H, D]
            amax = np.abs(blk).max(axis=(0, 2)).astype(np.float32)
            sc = int8_scale(amax)
            scales[bi, :, j] = sc
            codes[r0:r1] = int8_encode(blk / sc[None, :, None])
    return codes, scales


def perm_pi(j: np.ndarray) -> np.ndarray:
    """Stored position of token j (0..31) inside its 32-token group."""
    j = np.asarray(j)
    half, g, r = j // 16, (j % 16) // 4, j % 4
    return 8 * g + 4 * half + r


def s_pad(max_seqlen: int) -> int:
    return ((int(max_seqlen) + 127) // 128) * 128


def v_permute(v: np.ndarray, dtype: str, cu_seqlens: np.ndarray, max_seqlen: int,
              fp8: bool, amax_in=None, per_channel: bool = False):
    """V [T, H, D] -> (v_out [B, H, D, S_pad], descale f32[H], [B, H, D] or None).

    v_out[b, h, d, 32*G + pi(j)] = enc(V[cu[b] + 32*G + j, h, d]) for tokens
    32*G + j < L_b, and the all-zero pattern (+0) past L_b.  enc is the
    e4m3fn code with the per-head descale (fp8=True), with the per-channel
    descale (fp8=True, per_channel=True), or the unchanged 16-bit pattern
    (fp8=False)."""
    t, h, d = v.shape
    b = len(cu_seqlens) - 1
    sp = s_pad(max_seqlen)
    if fp8:
        if per_channel:
            codes, ds = quant_fp8_per_channel(v, dtype, cu_seqlens)
        else:
            codes, ds = quant_fp8_per_head(v, dtype, amax_in)
        src = codes
        out = np.zeros((b, h, d, sp), np.uint8)
    else:
        ds = None
        src = np.asarray(v).view(np.uint16)
        out = np.zeros((b, h, d, sp), np.uint16)
    pos_of = (np.arange(sp) // PERM_GROUP) * PERM_GROUP + perm_pi(np.arange(sp) % PERM_GROUP)
    for bi in range(b):
        s0, s1 = int(cu_seqlens[bi]), int(cu_seqlens[bi + 1])
        n = s1 - s0
        # token i of the sequence goes to stored position pos_of[i]
        out[bi][:, :, pos_of[:n]] = np.transpose(src[s0:s1], (1, 2, 0))
    if not fp8 and dtype == "fp16":
        out = out.view(np.float16)
    return out, ds


def v_unpermute(v_out: np.ndarray, seqlens) -> list:
    """Inverse of v_permute's layout: per sequence an array [L_b, H, D]."""
    sp = v_out.shape[-1]
    pos_of = (np.arange(sp) // PERM_GROUP) * PERM_GROUP + perm_pi(np.arange(sp) % PERM_GROUP)
    res = []
    for bi, n in enumerate(seqlens):
        res.append(np.transpose(v_out[bi][:, :, pos_of[:int(n)]], (2, 0, 1)))
    return res


def channel_mean_fp16(x: np.ndarray, cu_seqlens) -> np.ndarray:
    """Per-sequence, per-channel mean of fp16 x [T, H, D] -> fp32 [B, H, D]
    (SageAttention's K smoothing; PaddleNLP "Sage Attention Support Varlen").
    Reading: the sum S over the sequence's tokens is exact (every fp16 value
    is an integer number of 2^-24 units; the units are summed as integers),
    then mean = fp32(fp64(S) / fp64(L)); 0 for an empty sequence."""
    units = (np.asarray(x, np.float16).astype(np.float64) * 2.0 ** 24).astype(np.int64)
    cu = np.asarray(cu_seqlens, np.int64)
    b = len(cu) - 1
    out = np.zeros((b,) + units.shape[1:], np.float32)
    for i in range(b):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        if s1 > s0:
            tot = units[s0:s1].sum(axis=0, dtype=np.int64)
            out[i] = (tot.astype(np.float64) / np.float64(s1 - s0)).astype(np.float32) * np.float32(2.0 ** -24)
    return out


def smooth_quant_k(k: np.ndarray, cu_seqlens, max_seqlen: int, block_tokens: int = 128):
    """K smoothing then int8 per block: codes and scales of fp32(k) - mean
    (one fp32 subtraction per element), and the means."""
    mean = channel_mean_fp16(k, cu_seqlens)
    k32 = as_f32(k, "fp16").copy()
    cu = np.asarray(cu_seqlens, np.int64)
    for i in range(len(cu) - 1):
        k32[cu[i]:cu[i + 1]] = k32[cu[i]:cu[i + 1]] - mean[i][None]
    codes, scales = quant_int8_per_block(k32, "f32", cu_seqlens, max_seqlen, block_tokens)
    return codes, scales, mean
