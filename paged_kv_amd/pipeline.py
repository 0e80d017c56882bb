"""Call sequences of the path over device tensors (allocation + C-ABI calls).

Each function allocates its outputs with torch (device memory plumbing) and
enqueues the library's entry points in order on the current stream; every
step of the computation runs in libattnq's HIP kernels.  Inputs are torch
tensors already on the GPU, with the dtypes named in include/attnq.h
(bf16 / fp16 data, uint8 fp8 codes, int32 indices, fp32 scales).
"""
from __future__ import annotations

import torch

from . import api as A


def _round_up(x: int, m: int) -> int:
    return (x + m - 1) // m * m


def _scale(sm_scale) -> float:
    """None selects the library's default scale 1/sqrt(d_k) (passed as NaN)."""
    return float("nan") if sm_scale is None else float(sm_scale)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return A.BF16
    if t.dtype == torch.float16:
        return A.FP16
    raise TypeError(f"unsupported dtype {t.dtype}")


class Fp8Prefill:
    """fp8 per-head quantization of Q/K/V followed by the varlen prefill
    (the aiter fp8 flash_attn_func flow over a ragged batch).  With
    wide_v (default) the permuted V holds each fp8 code's exact fp16 value,
    which the prefill stages without a widening step.  QK^T is summed
    exactly from the codes; fp8_mma8 selects the fp8 matrix instruction
    instead (faster, with its documented accumulation error)."""

    def __init__(self, q, k, v, cu_seqlens, max_seqlen, sm_scale, causal=True,
                 out_dtype=torch.bfloat16, want_lse=False, amax=None, wide_v=True, fp8_mma8=False):
        dev = q.device
        self.q, self.k, self.v, self.cu = q, k, v, cu_seqlens
        self.t, self.hq, self.d = q.shape
        self.hkv = k.shape[1]
        self.b = cu_seqlens.numel() - 1
        self.max_seqlen = int(max_seqlen)
        self.sm_scale, self.causal = _scale(sm_scale), bool(causal)
        self.amax = amax  # optional (amax_q, amax_k, amax_v) from the append step
        self.qc = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        self.kc = torch.empty(k.shape, dtype=torch.uint8, device=dev)
        self.wide_v = bool(wide_v)
        self.qk_mode = A.Q_FP8_PER_HEAD_MFMA8 if fp8_mma8 else A.Q_FP8_PER_HEAD
        self.vp = torch.empty((self.b, self.hkv, self.d, _round_up(self.max_seqlen, 128)),
                              dtype=torch.float16 if self.wide_v else torch.uint8, device=dev)
        self.qs = torch.empty(self.hq, dtype=torch.float32, device=dev)
        self.ks = torch.empty(self.hkv, dtype=torch.float32, device=dev)
        self.vs = torch.empty(self.hkv, dtype=torch.float32, device=dev)
        self.o = torch.empty((self.t, self.hq, self.d), dtype=out_dtype, device=dev)
        self.lse = torch.empty((self.hq, self.t), dtype=torch.float32, device=dev) if want_lse else None

    def quantize(self):
        dt = _dtype_code(self.q)
        aq, ak, av = self.amax if self.amax is not None else (None, None, None)
        A.attn_quant_qk(self.q, dt, self.cu, self.b, self.max_seqlen, self.t, self.hq, self.d,
                        A.Q_FP8_PER_HEAD, 128, aq, self.qc, self.qs)
        A.attn_quant_qk(self.k, dt, self.cu, self.b, self.max_seqlen, self.t, self.hkv, self.d,
                        A.Q_FP8_PER_HEAD, 128, ak, self.kc, self.ks)
        A.attn_quant_v_permute(self.v, dt, self.cu, self.b, self.max_seqlen, self.t, self.hkv,
                               self.d, A.Q_FP8_PER_HEAD_WIDE if self.wide_v else A.Q_FP8_PER_HEAD,
                               av, self.vp, self.vs)

    def attend(self):
        A.attn_prefill_varlen(self.qc, self.kc, self.vp, A.FP8E4M3,
                              A.FP16 if self.wide_v else A.FP8E4M3, self.qs, self.ks,
                              self.vs, A.Q_FP8_PER_HEAD, self.qk_mode, self.cu, self.cu, self.b, self.max_seqlen,
                              self.max_seqlen, self.t, self.t, self.hq, self.hkv, self.d,
                              self.sm_scale, self.causal, self.o, _dtype_code(self.o), self.lse)

    def run(self):
        self.quantize()
        self.attend()
        return self.o


class SagePrefill:
    """SageAttention-style flow: per-128-token-block int8 Q/K, fp16 V in the
    permuted transposed layout, int8 QK / fp16 PV prefill, fp16 output.
    With fuse_q (default) the prefill quantizes each 128-query block of the
    16-bit Q itself (same codes and scales as attn_quant_qk; the scales land
    in qs) instead of reading int8 codes written by a separate pass.  With
    smooth_k each sequence's per-channel mean of K (kept in kmean) is
    subtracted before K's int8 quantization (attn_smooth_quant_k): the same
    softmax output, with lse lower by sm_scale * q . mean.  With
    v_fp8_per_channel V is fp8 e4m3fn with one descale per (sequence, kv head,
    channel) (kept in vs), stored as the codes' fp16 values; the prefill
    scales each output column by its channel's descale."""

    def __init__(self, q, k, v, cu_seqlens, max_seqlen, sm_scale, causal=True, want_lse=False,
                 fuse_q=True, smooth_k=False, v_fp8_per_channel=False):
        dev = q.device
        self.q, self.k, self.v, self.cu = q, k, v, cu_seqlens
        self.t, self.hq, self.d = q.shape
        self.hkv = k.shape[1]
        self.b = cu_seqlens.numel() - 1
        self.max_seqlen = int(max_seqlen)
        self.sm_scale, self.causal = _scale(sm_scale), bool(causal)
        self.fuse_q = bool(fuse_q)
        self.smooth_k = bool(smooth_k)
        self.v_chan = bool(v_fp8_per_channel)
        if self.smooth_k and k.dtype != torch.float16:
            raise TypeError("K smoothing takes fp16 K")
        if v.dtype != torch.float16:
            raise TypeError("SagePrefill takes fp16 V (the PV product runs on fp16 V^T)")
        nblk = (self.max_seqlen + 127) // 128
        self.qc = None if self.fuse_q else torch.empty(q.shape, dtype=torch.int8, device=dev)
        self.kc = torch.empty(k.shape, dtype=torch.int8, device=dev)
        self.qs = torch.empty((self.b, self.hq, nblk), dtype=torch.float32, device=dev)
        self.ks = torch.empty((self.b, self.hkv, nblk), dtype=torch.float32, device=dev)
        self.kmean = torch.empty((self.b, self.hkv, self.d), dtype=torch.float32, device=dev) if self.smooth_k else None
        self.vs = torch.empty((self.b, self.hkv, self.d), dtype=torch.float32, device=dev) if self.v_chan else None
        self.vp = torch.empty((self.b, self.hkv, self.d, _round_up(self.max_seqlen, 128)),
                              dtype=torch.float16, device=dev)
        self.o = torch.empty((self.t, self.hq, self.d), dtype=torch.float16, device=dev)
        self.lse = torch.empty((self.hq, self.t), dtype=torch.float32, device=dev) if want_lse else None

    def quantize(self):
        if not self.fuse_q:
            A.attn_quant_qk(self.q, _dtype_code(self.q), self.cu, self.b, self.max_seqlen, self.t,
                            self.hq, self.d, A.Q_INT8_PER_BLOCK, 128, None, self.qc, self.qs)
        if not self.smooth_k and not self.v_chan and self.k.dtype == self.v.dtype:
            # K int8 blocks and the V permute side by side in one launch
            A.attn_quant_kv(self.k, self.v, _dtype_code(self.k), self.cu, self.b, self.max_seqlen, self.t,
                            self.hkv, self.d, 128, self.kc, self.ks, self.vp)
            return
        if self.smooth_k:
            A.attn_smooth_quant_k(self.k, self.cu, self.b, self.max_seqlen, self.t, self.hkv, self.d, 128,
                                  self.kc, self.ks, self.kmean)
        else:
            A.attn_quant_qk(self.k, _dtype_code(self.k), self.cu, self.b, self.max_seqlen, self.t,
                            self.hkv, self.d, A.Q_INT8_PER_BLOCK, 128, None, self.kc, self.ks)
        A.attn_quant_v_permute(self.v, A.FP16, self.cu, self.b, self.max_seqlen, self.t, self.hkv,
                               self.d, A.Q_FP8_PER_CHANNEL_WIDE if self.v_chan else A.Q_NONE, None,
                               self.vp, self.vs)

    def attend(self):
        if self.fuse_q:
            q, qk_dtype, mode = self.q, _dtype_code(self.q), A.Q_INT8_PER_BLOCK_RAW_Q
        else:
            q, qk_dtype, mode = self.qc, A.INT8, A.Q_INT8_PER_BLOCK
        A.attn_prefill_varlen(q, self.kc, self.vp, qk_dtype, A.FP16, self.qs, self.ks, self.vs,
                              A.Q_FP8_PER_CHANNEL if self.v_chan else A.Q_FP8_PER_HEAD, mode, self.cu, self.cu, self.b, self.max_seqlen,
                              self.max_seqlen, self.t, self.t, self.hq, self.hkv, self.d,
                              self.sm_scale, self.causal, self.o, A.FP16, self.lse)

    def run(self):
        self.quantize()
        self.attend()
        return self.o


class AppendRopeFp8Prefill:
    """RoPE + paged bf16 cache write with fused per-head amax, then the fp8
    prefill on the rotated Q/K and V (the long-context flow)."""

    def __init__(self, q, k, v, cu_seqlens, kv_len_before, max_seqlen, rope_cos_sin, k_cache,
                 v_cache, kv_indptr, kv_indices, page_size, sm_scale, causal=True, want_lse=False,
                 fp8_mma8=False):
        dev = q.device
        self.q, self.k, self.v = q, k, v
        self.cu, self.before = cu_seqlens, kv_len_before
        self.cs, self.kcache, self.vcache = rope_cos_sin, k_cache, v_cache
        self.indptr, self.indices, self.page_size = kv_indptr, kv_indices, int(page_size)
        self.t, self.hq, self.d = q.shape
        self.hkv = k.shape[1]
        self.b = cu_seqlens.numel() - 1
        self.amax = tuple(torch.empty(h, dtype=torch.float32, device=dev)
                          for h in (self.hq, self.hkv, self.hkv))
        self.prefill = Fp8Prefill(q, k, v, cu_seqlens, max_seqlen, sm_scale, causal,
                                  want_lse=want_lse, amax=self.amax, fp8_mma8=fp8_mma8)

    def append(self):
        A.attn_append_kv_rope(self.q, self.k, self.v, _dtype_code(self.q), self.cu, self.before,
                              self.b, self.t, self.hq, self.hkv, self.d, self.cs, self.cs.shape[0],
                              self.kcache, self.vcache, self.indptr, self.indices,
                              self.kcache.shape[0], self.page_size, *self.amax)

    def run(self):
        self.append()
        return self.prefill.run()


class PagedPrefill:
    """A prefill chunk against a paged 16-bit KV cache (FlashInfer's paged
    prefill run): the sequences' pages are read into the ragged layout
    (attn_gather_paged_kv), then Q (the chunk), K and V (the gathered cache)
    get fp8 per-head quantization (V permuted, each code stored as its exact
    fp16 value) and the varlen prefill runs with cu_seqlens_q != cu_seqlens_k,
    the chunk's queries aligned to the end of their sequence's keys."""

    def __init__(self, q, k_cache, v_cache, kv_indptr, kv_indices, kv_last_page_len, cu_q, cu_k,
                 max_q, max_k, sm_scale, causal=True, out_dtype=torch.bfloat16, want_lse=False):
        dev = q.device
        if k_cache.dtype not in (torch.bfloat16, torch.float16) or v_cache.dtype != k_cache.dtype:
            raise TypeError("PagedPrefill takes bf16 or fp16 caches of one dtype")
        self.q, self.kc_pages, self.vc_pages = q, k_cache, v_cache
        self.ip, self.ix, self.lpl, self.cu_q, self.cu_k = kv_indptr, kv_indices, kv_last_page_len, cu_q, cu_k
        self.tq, self.hq, self.d = q.shape
        self.num_pages, self.page_size, self.hkv, _ = k_cache.shape
        self.b = cu_q.numel() - 1
        self.max_q, self.max_k = int(max_q), int(max_k)
        self.tk = int(cu_k[-1].item())
        self.sm_scale, self.causal = _scale(sm_scale), bool(causal)
        self.kg = torch.empty((self.tk, self.hkv, self.d), dtype=k_cache.dtype, device=dev)
        self.vg = torch.empty_like(self.kg)
        self.qc = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        self.kc = torch.empty(self.kg.shape, dtype=torch.uint8, device=dev)
        self.vp = torch.empty((self.b, self.hkv, self.d, _round_up(self.max_k, 128)), dtype=torch.float16,
                              device=dev)
        self.qs = torch.empty(self.hq, dtype=torch.float32, device=dev)
        self.ks = torch.empty(self.hkv, dtype=torch.float32, device=dev)
        self.vs = torch.empty(self.hkv, dtype=torch.float32, device=dev)
        self.o = torch.empty((self.tq, self.hq, self.d), dtype=out_dtype, device=dev)
        self.lse = torch.empty((self.hq, self.tq), dtype=torch.float32, device=dev) if want_lse else None

    def gather(self):
        for pages, out in ((self.kc_pages, self.kg), (self.vc_pages, self.vg)):
            A.attn_gather_paged_kv(pages, 2, self.ip, self.ix, self.lpl, self.cu_k, self.b, self.max_k,
                                   self.num_pages, self.page_size, self.hkv, self.d, out)

    def quantize(self):
        dq, dk = _dtype_code(self.q), _dtype_code(self.kg)
        A.attn_quant_qk(self.q, dq, self.cu_q, self.b, self.max_q, self.tq, self.hq, self.d,
                        A.Q_FP8_PER_HEAD, 128, None, self.qc, self.qs)
        A.attn_quant_qk(self.kg, dk, self.cu_k, self.b, self.max_k, self.tk, self.hkv, self.d,
                        A.Q_FP8_PER_HEAD, 128, None, self.kc, self.ks)
        A.attn_quant_v_permute(self.vg, dk, self.cu_k, self.b, self.max_k, self.tk, self.hkv, self.d,
                               A.Q_FP8_PER_HEAD_WIDE, None, self.vp, self.vs)

    def attend(self):
        A.attn_prefill_varlen(self.qc, self.kc, self.vp, A.FP8E4M3, A.FP16, self.qs, self.ks, self.vs,
                              A.Q_FP8_PER_HEAD, A.Q_FP8_PER_HEAD, self.cu_q, self.cu_k, self.b, self.max_q, self.max_k,
                              self.tq, self.tk, self.hq, self.hkv, self.d, self.sm_scale, self.causal,
                              self.o, _dtype_code(self.o), self.lse)

    def run(self):
        self.gather()
        self.quantize()
        self.attend()
        return self.o


class PagedPrefillFp8:
    """A prefill chunk against a paged fp8 e4m3fn cache (the pages and
    per-head descales attn_decode_paged reads), the pages read inside the
    attention kernel (FlashInfer's paged prefill run; aiter's
    flash_attn_with_kvcache with an fp8 cache and a page table): Q gets fp8
    per-head quantization (attn_quant_qk), then attn_prefill_paged, the
    chunk's queries aligned to the end of their sequence's cached keys."""

    def __init__(self, q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices, kv_last_page_len, cu_q,
                 max_q, max_kv_len, sm_scale, causal=True, out_dtype=torch.bfloat16, want_lse=False,
                 fp8_mma8=False):
        dev = q.device
        if k_cache.dtype != torch.uint8 or v_cache.dtype != torch.uint8:
            raise TypeError("PagedPrefillFp8 takes fp8 e4m3fn caches as uint8 codes")
        self.q, self.kc, self.vc, self.ks, self.vs = q, k_cache, v_cache, k_scale, v_scale
        self.ip, self.ix, self.lpl, self.cu_q = kv_indptr, kv_indices, kv_last_page_len, cu_q
        self.tq, self.hq, self.d = q.shape
        self.num_pages, self.page_size, self.hkv, _ = k_cache.shape
        self.b = cu_q.numel() - 1
        self.max_q, self.max_kv = int(max_q), int(max_kv_len)
        self.sm_scale, self.causal = _scale(sm_scale), bool(causal)
        self.mode = A.Q_FP8_PER_HEAD_MFMA8 if fp8_mma8 else A.Q_FP8_PER_HEAD
        self.qc = torch.empty(q.shape, dtype=torch.uint8, device=dev)
        self.qs = torch.empty(self.hq, dtype=torch.float32, device=dev)
        self.o = torch.empty((self.tq, self.hq, self.d), dtype=out_dtype, device=dev)
        self.lse = torch.empty((self.hq, self.tq), dtype=torch.float32, device=dev) if want_lse else None

    def quantize(self):
        A.attn_quant_qk(self.q, _dtype_code(self.q), self.cu_q, self.b, self.max_q, self.tq, self.hq, self.d,
                        A.Q_FP8_PER_HEAD, 128, None, self.qc, self.qs)

    def attend(self):
        A.attn_prefill_paged(self.qc, self.qs, self.mode, self.kc, self.vc, self.ks, self.vs, self.ip, self.ix,
                             self.lpl, self.cu_q, self.b, self.num_pages, self.page_size, self.max_q, self.max_kv,
                             self.tq, self.hq, self.hkv, self.d, self.sm_scale, self.causal, self.o,
                             _dtype_code(self.o), self.lse)

    def run(self):
        self.quantize()
        self.attend()
        return self.o


class PagedDecode:
    """Split-KV paged fp8 decode + log-sum-exp merge."""

    def __init__(self, q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices,
                 kv_last_page_len, max_kv_len, sm_scale, want_lse=False):
        dev = q.device
        self.args = (q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices, kv_last_page_len)
        self.b, self.hq, self.d = q.shape
        self.num_pages, self.page_size, self.hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
        self.max_kv_len, self.sm_scale = int(max_kv_len), _scale(sm_scale)
        self.ws_bytes = A.attn_decode_paged_workspace_size(self.b, self.hq, self.d, self.max_kv_len,
                                                           self.page_size)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.o = torch.empty((self.b, self.hq, self.d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((self.b, self.hq), dtype=torch.float32, device=dev) if want_lse else None

    def run(self):
        A.attn_decode_paged(*self.args, self.b, self.num_pages, self.page_size, self.hq, self.hkv,
                            self.d, self.max_kv_len, self.sm_scale, self.ws, self.ws_bytes, self.o,
                            self.lse)
        return self.o


class SparseMlaDecode:
    """MLA-absorb sparse decode over int8 (or fp8 e4m3, kv_fp8) cache rows with
    tile-128 scales; an index names sparse_block_size consecutive tokens;
    sparse_mode 3 adds the right-down causal mask over the s_q query rows."""

    def __init__(self, q, kv_cache, block_table, kv_lens, sparse_indices, sm_scale=None,
                 want_lse=False, kv_fp8=False, sparse_block_size=1, sparse_mode=0):
        dev = q.device
        self.q, self.cache, self.table, self.kv_lens, self.idx = q, kv_cache, block_table, kv_lens, sparse_indices
        self.b, self.sq, self.h, dq = q.shape
        self.topk = sparse_indices.shape[-1]
        self.kv_dtype = A.FP8E4M3 if kv_fp8 else A.INT8
        self.sbs, self.mode = int(sparse_block_size), int(sparse_mode)
        self.sm_scale = _scale(sm_scale)
        self.ws_bytes = A.attn_sparse_mla_decode_workspace_size(self.b, self.sq, self.h, self.topk, self.sbs)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self.o = torch.empty((self.b, self.sq, self.h, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((self.b, self.sq, self.h), dtype=torch.float32, device=dev) if want_lse else None

    def run(self):
        A.attn_sparse_mla_decode(self.q, self.cache, self.kv_dtype, self.table, self.table.shape[1], self.kv_lens,
                                 self.idx, self.topk, self.sbs, self.mode, self.b, self.sq, self.h, self.cache.shape[0],
                                 self.cache.shape[1], self.sm_scale, self.ws, self.ws_bytes, self.o,
                                 self.lse)
        return self.o
