"""Pure-Python scalar versions of the path for tiny inputs (oracle: test
infrastructure only).

These loops restate the definitions one scalar at a time, with their own
decoders (bit fields via ``struct``) and a nearest-grid-point search for the
fp8 encoder, so that a slip in the vectorised oracle (a dropped term, a
wrong sign or index, a transposed operand) shows up as a disagreement.
Intended sizes: a few sequences of a few tokens, head dims of at most 8.
"""
from __future__ import annotations

import math
import struct

import numpy as np


# ---------------------------------------------------------------------------
# scalar formats
# ---------------------------------------------------------------------------
def e4m3fn_value(code: int) -> float:
    """Value of an e4m3fn code from its bit fields (NaN for S.1111.111)."""
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1 + m / 8) * 2.0 ** (e - 7)


def e4m3fn_encode_search(v: float) -> int:
    """Nearest finite code by exhaustive search; ties go to the even code
    (mantissa LSB 0); |v| is clamped to 448; NaN -> 0x7F; sign kept."""
    if math.isnan(v):
        return 0x7F
    neg = math.copysign(1.0, v) < 0
    a = min(abs(v), 448.0)
    best, best_err = None, None
    for c in range(0x7F):                      # non-negative finite codes
        err = abs(e4m3fn_value(c) - a)
        if best is None or err < best_err or (err == best_err and (c & 1) == 0 and (best & 1) == 1):
            best, best_err = c, err
    return best | (0x80 if neg else 0)


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def f32(x) -> np.float32:
    return np.float32(x)


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------
def quant_fp8_per_head(x32: np.ndarray):
    """x32 [T, H, D] fp32 -> (codes [T,H,D], descale [H]) by scalar loops."""
    t, h, d = x32.shape
    codes = np.zeros((t, h, d), np.uint8)
    ds = np.zeros(h, np.float32)
    for hh in range(h):
        amax = 0.0
        for i in range(t):
            for k in range(d):
                amax = max(amax, abs(float(x32[i, hh, k])))
        desc = f32(1.0) if amax == 0 else f32(amax) / f32(448.0)
        ds[hh] = desc
        for i in range(t):
            for k in range(d):
                codes[i, hh, k] = e4m3fn_encode_search(float(f32(x32[i, hh, k]) / desc))
    return codes, ds


def quant_fp8_per_channel(x32: np.ndarray, cu):
    """x32 [T, H, D] fp32 -> (codes [T,H,D], descale [B,H,D]) by scalar loops:
    one descale per (sequence, head, channel)."""
    t, h, d = x32.shape
    b = len(cu) - 1
    codes = np.zeros((t, h, d), np.uint8)
    ds = np.ones((b, h, d), np.float32)
    for bi in range(b):
        for hh in range(h):
            for k in range(d):
                amax = 0.0
                for i in range(int(cu[bi]), int(cu[bi + 1])):
                    amax = max(amax, abs(float(x32[i, hh, k])))
                desc = f32(1.0) if amax == 0 else f32(amax) / f32(448.0)
                ds[bi, hh, k] = desc
                for i in range(int(cu[bi]), int(cu[bi + 1])):
                    codes[i, hh, k] = e4m3fn_encode_search(float(f32(x32[i, hh, k]) / desc))
    return codes, ds


def quant_int8_per_block(x32: np.ndarray, cu, block: int):
    t, h, d = x32.shape
    codes = np.zeros((t, h, d), np.int8)
    scales = {}
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        j = 0
        while s0 + j * block < s1:
            r0, r1 = s0 + j * block, min(s0 + (j + 1) * block, s1)
            for hh in range(h):
                amax = 0.0
                for i in range(r0, r1):
                    for k in range(d):
                        amax = max(amax, abs(float(x32[i, hh, k])))
                sc = f32(1.0) if amax == 0 else f32(amax) / f32(127.0)
                scales[(b, hh, j)] = sc
                for i in range(r0, r1):
                    for k in range(d):
                        v = float(f32(x32[i, hh, k]) / sc)
                        r = round(v)                     # Python round: ties to even
                        codes[i, hh, k] = max(-127, min(127, r))
            j += 1
    return codes, scales


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------
def attend_one(q, keys, vals, scale):
    """One query against lists of key / value vectors, scalar math."""
    if not keys:
        return [0.0] * (len(vals[0]) if vals else 0), float("-inf")
    logits = [scale * sum(qa * ka for qa, ka in zip(q, k)) for k in keys]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    tot = sum(w)
    out = [sum(w[j] * vals[j][c] for j in range(len(vals))) / tot for c in range(len(vals[0]))]
    return out, m + math.log(tot)


def prefill(qd, kd, vd, cu_q, cu_k, scale, causal):
    """qd [Tq,Hq,D], kd/vd [Tk,Hkv,D] fp64 arrays -> (O [Tq,Hq,D], lse [Hq,Tq])."""
    tq, hq, d = qd.shape
    hkv = kd.shape[1]
    o = np.zeros((tq, hq, vd.shape[2]))
    lse = np.full((hq, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        lq = int(cu_q[b + 1] - cu_q[b])
        lk = int(cu_k[b + 1] - cu_k[b])
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(lq):
                keys, vals = [], []
                for j in range(lk):
                    if causal and j > i + lk - lq:
                        continue
                    keys.append(list(kd[cu_k[b] + j, g]))
                    vals.append(list(vd[cu_k[b] + j, g]))
                if not keys:
                    continue
                out, l = attend_one(list(qd[cu_q[b] + i, h]), keys, vals, scale)
                o[cu_q[b] + i, h] = out
                lse[h, cu_q[b] + i] = l
    return o, lse


def decode_paged(q_bits, k_cache, v_cache, k_scale, v_scale, indptr, indices, last, scale):
    b_, hq, d = q_bits.shape
    ps, hkv = k_cache.shape[1], k_cache.shape[2]
    o = np.zeros((b_, hq, d))
    lse = np.full((b_, hq), -np.inf)
    for b in range(b_):
        npg = int(indptr[b + 1] - indptr[b])
        n = 0 if npg == 0 else (npg - 1) * ps + int(last[b])
        for h in range(hq):
            g = h // (hq // hkv)
            keys, vals = [], []
            for t in range(n):
                page = int(indices[int(indptr[b]) + t // ps])
                slot = t % ps
                keys.append([e4m3fn_value(int(k_cache[page, slot, g, c])) * float(k_scale[g]) for c in range(d)])
                vals.append([e4m3fn_value(int(v_cache[page, slot, g, c])) * float(v_scale[g]) for c in range(d)])
            if not keys:
                continue
            q = [bf16_value(q_bits[b, h, c]) for c in range(d)]
            o[b, h], lse[b, h] = attend_one(q, keys, vals, scale)
    return o, lse


def prefill_paged(q_codes, q_scale, k_cache, v_cache, k_scale, v_scale, indptr, indices, last, cu_q,
                  scale, causal):
    """Scalar page walk of a prefill chunk over fp8 pages: query i of
    sequence b (of L_q) sits at position i + n - L_q of its n cached tokens."""
    tq, hq, d = q_codes.shape
    ps, hkv = k_cache.shape[1], k_cache.shape[2]
    o = np.zeros((tq, hq, d))
    lse = np.full((hq, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        npg = int(indptr[b + 1] - indptr[b])
        n = 0 if npg == 0 else (npg - 1) * ps + int(last[b])
        lq = int(cu_q[b + 1] - cu_q[b])
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(lq):
                keys, vals = [], []
                for t in range(n):
                    if causal and t > i + n - lq:
                        continue
                    page = int(indices[int(indptr[b]) + t // ps])
                    slot = t % ps
                    keys.append([e4m3fn_value(int(k_cache[page, slot, g, c])) * float(k_scale[g]) for c in range(d)])
                    vals.append([e4m3fn_value(int(v_cache[page, slot, g, c])) * float(v_scale[g]) for c in range(d)])
                if not keys:
                    continue
                r = int(cu_q[b]) + i
                q = [e4m3fn_value(int(q_codes[r, h, c])) * float(q_scale[h]) for c in range(d)]
                o[r, h], lse[h, r] = attend_one(q, keys, vals, scale)
    return o, lse


def sparse_mla(q_bits, kv_cache, block_table, kv_lens, sparse_indices, scale, kv_dtype="int8",
               sparse_block_size=1, sparse_mode=0):
    """Scalar sparse MLA decode; rows parsed with struct.  Entry e >= 0 covers
    tokens e*sbs .. e*sbs+sbs-1; a token counts if it is below kv_len and
    (sparse_mode 3) not past kv_len - s_q + s."""
    b_, sq, h, dq = q_bits.shape
    bs = kv_cache.shape[1]
    o = np.zeros((b_, sq, h, 512))
    lse = np.full((b_, sq, h), -np.inf)
    for b in range(b_):
        for s in range(sq):
            keys, vals = [], []
            toks = []
            for e in sparse_indices[b, s, 0]:
                e = int(e)
                if e < 0:
                    continue
                for j in range(sparse_block_size):
                    toks.append(e * sparse_block_size + j)
            for idx in toks:
                if idx >= int(kv_lens[b]):
                    continue
                if sparse_mode == 3 and idx > int(kv_lens[b]) - sq + s:
                    continue
                blk = int(block_table[b][idx // bs])
                raw = bytes(kv_cache[blk, idx % bs, 0])
                if kv_dtype == "fp8":
                    codes = [e4m3fn_value(c) for c in raw[:512]]
                else:
                    codes = struct.unpack("<512b", raw[:512])
                rope = [bf16_value(x) for x in struct.unpack("<64H", raw[512:640])]
                sc = struct.unpack("<4f", raw[640:656])
                nope = [codes[c] * sc[c // 128] for c in range(512)]
                keys.append(nope + rope)
                vals.append(nope)
            for hh in range(h):
                if not keys:
                    continue
                q = [bf16_value(q_bits[b, s, hh, c]) for c in range(dq)]
                o[b, s, hh], lse[b, s, hh] = attend_one(q, keys, vals, scale)
    return o, lse


def rope_token(x32_row: np.ndarray, cs_row: np.ndarray) -> np.ndarray:
    """Rotate one head vector (fp32) with the fp32 table row [D/2, 2]."""
    d = x32_row.shape[0]
    half = d // 2
    y = np.zeros(d, np.float32)
    for i in range(half):
        c, s = f32(cs_row[i, 0]), f32(cs_row[i, 1])
        a, b = f32(x32_row[i]), f32(x32_row[i + half])
        y[i] = f32(f32(a * c) - f32(b * s))
        y[i + half] = f32(f32(b * c) + f32(a * s))
    return y
