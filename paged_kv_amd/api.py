"""ctypes binding of libattnq (argument marshalling only).

Each function has the name, argument order and meaning of the C entry point
in include/attnq.h.  Array arguments are torch tensors on the GPU (or None
where the C argument is optional); they are passed as device pointers
without copies or checks beyond what the library itself validates.  The
stream defaults to torch's current stream on the tensors' device.  A
negative status raises RuntimeError with attnq_last_error().
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "BF16", "FP16", "FP8E4M3", "INT8", "Q_FP8_PER_HEAD", "Q_INT8_PER_BLOCK", "Q_NONE", "Q_FP8_PER_HEAD_WIDE", "Q_FP8_PER_CHANNEL", "Q_FP8_PER_CHANNEL_WIDE",
    "Q_FP8_PER_HEAD_MFMA8",
    "Q_INT8_PER_BLOCK_RAW_Q",
    "library_path", "lib", "abi_version",
    "attn_quant_qk", "attn_quant_v_permute", "attn_append_kv_rope", "attn_prefill_varlen",
    "attn_smooth_quant_k", "attn_gather_paged_kv", "attn_prefill_paged", "attn_decode_paged_workspace_size",
    "attn_decode_paged", "attn_decode_paged_noalloc",
    "attn_sparse_mla_decode_workspace_size", "attn_sparse_mla_decode", "attn_quant_kv",
    "SYMBOLS",
]

BF16, FP16, FP8E4M3, INT8 = 0, 1, 2, 3
Q_FP8_PER_HEAD, Q_INT8_PER_BLOCK, Q_NONE, Q_FP8_PER_HEAD_WIDE, Q_INT8_PER_BLOCK_RAW_Q = 0, 1, 2, 3, 4
Q_FP8_PER_CHANNEL, Q_FP8_PER_CHANNEL_WIDE, Q_FP8_PER_HEAD_MFMA8 = 5, 6, 7

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

# name -> (restype, argtypes), in the order of include/attnq.h
SYMBOLS = {
    "attnq_abi_version": (_I, []),
    "attnq_last_error": (ctypes.c_char_p, []),
    "attn_quant_qk": (_I, [_P, _I, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "attn_quant_kv": (_I, [_P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "attn_quant_v_permute": (_I, [_P, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "attn_append_kv_rope": (_I, [_P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P,
                                 _P, _P, _I, _I, _P, _P, _P, _P]),
    "attn_prefill_varlen": (_I, [_P, _P, _P, _I, _I, _P, _P, _P, _I, _I, _P, _P, _I, _I, _I, _I,
                                 _I, _I, _I, _I, _F, _I, _P, _I, _P, _P]),
    "attn_smooth_quant_k": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "attn_gather_paged_kv": (_I, [_P, _I, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "attn_prefill_paged": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I,
                                _I, _F, _I, _P, _I, _P, _P]),
    "attn_decode_paged_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "attn_decode_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                               _P, _Z, _P, _P, _P]),
    "attn_decode_paged_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                       _P, _P, _P]),
    "attn_sparse_mla_decode_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "attn_sparse_mla_decode": (_I, [_P, _P, _I, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _P, _Z,
                                    _P, _P, _P]),
}

_LIB = None


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnq.so")


def lib():
    """Load libattnq.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_amd.build`")
        h = ctypes.CDLL(path)
        for name, (res, args) in SYMBOLS.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = h
    return _LIB


def abi_version() -> int:
    return lib().attnq_abi_version()


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, name: str) -> None:
    if status != 0:
        msg = lib().attnq_last_error()
        raise RuntimeError(f"{name} failed with status {status}: {msg.decode() if msg else ''}")


def attn_quant_qk(x, x_dtype, cu_seqlens, batch, max_seqlen, total_tokens, num_heads, head_dim,
                  mode, block_tokens, amax_in, codes, scales, stream=None):
    s = _stream(stream, x, codes, scales)
    _check(lib().attn_quant_qk(_ptr(x), x_dtype, _ptr(cu_seqlens), batch, max_seqlen, total_tokens,
                               num_heads, head_dim, mode, block_tokens, _ptr(amax_in), _ptr(codes),
                               _ptr(scales), s), "attn_quant_qk")


def attn_quant_kv(k, v, dtype, cu_seqlens, batch, max_seqlen, total_tokens, num_kv_heads, head_dim,
                  block_tokens, k_codes, k_scales, v_out, stream=None):
    s = _stream(stream, k, v_out)
    _check(lib().attn_quant_kv(_ptr(k), _ptr(v), dtype, _ptr(cu_seqlens), batch, max_seqlen, total_tokens,
                               num_kv_heads, head_dim, block_tokens, _ptr(k_codes), _ptr(k_scales), _ptr(v_out),
                               s), "attn_quant_kv")


def attn_quant_v_permute(v, v_dtype, cu_seqlens, batch, max_seqlen, total_tokens, num_kv_heads,
                         head_dim, mode, amax_in, v_out, v_scales, stream=None):
    s = _stream(stream, v, v_out)
    _check(lib().attn_quant_v_permute(_ptr(v), v_dtype, _ptr(cu_seqlens), batch, max_seqlen,
                                      total_tokens, num_kv_heads, head_dim, mode, _ptr(amax_in),
                                      _ptr(v_out), _ptr(v_scales), s), "attn_quant_v_permute")


def attn_append_kv_rope(q, k, v, dtype, cu_seqlens, kv_len_before, batch, total_tokens,
                        num_q_heads, num_kv_heads, head_dim, rope_cos_sin, max_pos, k_cache,
                        v_cache, kv_indptr, kv_indices, num_pages, page_size, amax_q=None,
                        amax_k=None, amax_v=None, stream=None):
    s = _stream(stream, q, k_cache)
    _check(lib().attn_append_kv_rope(_ptr(q), _ptr(k), _ptr(v), dtype, _ptr(cu_seqlens),
                                     _ptr(kv_len_before), batch, total_tokens, num_q_heads,
                                     num_kv_heads, head_dim, _ptr(rope_cos_sin), max_pos,
                                     _ptr(k_cache), _ptr(v_cache), _ptr(kv_indptr),
                                     _ptr(kv_indices), num_pages, page_size, _ptr(amax_q),
                                     _ptr(amax_k), _ptr(amax_v), s), "attn_append_kv_rope")


def attn_prefill_varlen(q, k, v_perm, qk_dtype, v_dtype, q_scale, k_scale, v_scale, v_scale_mode, scale_mode,
                        cu_seqlens_q, cu_seqlens_k, batch, max_seqlen_q, max_seqlen_k, total_q,
                        total_k, num_q_heads, num_kv_heads, head_dim, sm_scale, causal, o,
                        o_dtype, lse=None, stream=None):
    s = _stream(stream, q, o)
    _check(lib().attn_prefill_varlen(_ptr(q), _ptr(k), _ptr(v_perm), qk_dtype, v_dtype,
                                     _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), v_scale_mode, scale_mode,
                                     _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), batch, max_seqlen_q,
                                     max_seqlen_k, total_q, total_k, num_q_heads, num_kv_heads,
                                     head_dim, float(sm_scale), int(causal), _ptr(o), o_dtype,
                                     _ptr(lse), s), "attn_prefill_varlen")


def attn_smooth_quant_k(k, cu_seqlens, batch, max_seqlen, total_tokens, num_kv_heads, head_dim,
                        block_tokens, codes, scales, mean, stream=None):
    s = _stream(stream, k, codes)
    _check(lib().attn_smooth_quant_k(_ptr(k), _ptr(cu_seqlens), batch, max_seqlen, total_tokens,
                                     num_kv_heads, head_dim, block_tokens, _ptr(codes), _ptr(scales),
                                     _ptr(mean), s), "attn_smooth_quant_k")


def attn_gather_paged_kv(cache, elem_bytes, kv_indptr, kv_indices, kv_last_page_len, cu_seqlens_k,
                         batch, max_seqlen_k, num_pages, page_size, num_kv_heads, head_dim, out,
                         stream=None):
    s = _stream(stream, cache, out)
    _check(lib().attn_gather_paged_kv(_ptr(cache), elem_bytes, _ptr(kv_indptr), _ptr(kv_indices),
                                      _ptr(kv_last_page_len), _ptr(cu_seqlens_k), batch,
                                      max_seqlen_k, num_pages, page_size, num_kv_heads, head_dim,
                                      _ptr(out), s), "attn_gather_paged_kv")


def attn_prefill_paged(q, q_scale, scale_mode, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices,
                       kv_last_page_len, cu_seqlens_q, batch, num_pages, page_size, max_seqlen_q, max_kv_len,
                       total_q, num_q_heads, num_kv_heads, head_dim, sm_scale, causal, o, o_dtype, lse=None,
                       stream=None):
    s = _stream(stream, q, o)
    _check(lib().attn_prefill_paged(_ptr(q), _ptr(q_scale), scale_mode, _ptr(k_cache), _ptr(v_cache),
                                    _ptr(k_scale), _ptr(v_scale), _ptr(kv_indptr), _ptr(kv_indices),
                                    _ptr(kv_last_page_len), _ptr(cu_seqlens_q), batch, num_pages, page_size,
                                    max_seqlen_q, max_kv_len, total_q, num_q_heads, num_kv_heads, head_dim,
                                    float(sm_scale), int(causal), _ptr(o), o_dtype, _ptr(lse), s),
           "attn_prefill_paged")


def attn_decode_paged_workspace_size(batch, num_q_heads, head_dim, max_kv_len, page_size) -> int:
    return int(lib().attn_decode_paged_workspace_size(batch, num_q_heads, head_dim, max_kv_len,
                                                      page_size))


def attn_decode_paged(q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices,
                      kv_last_page_len, batch, num_pages, page_size, num_q_heads, num_kv_heads,
                      head_dim, max_kv_len, sm_scale, workspace, workspace_bytes, o, lse=None,
                      stream=None):
    s = _stream(stream, q, o)
    _check(lib().attn_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                   _ptr(v_scale), _ptr(kv_indptr), _ptr(kv_indices),
                                   _ptr(kv_last_page_len), batch, num_pages, page_size,
                                   num_q_heads, num_kv_heads, head_dim, max_kv_len,
                                   float(sm_scale), _ptr(workspace), int(workspace_bytes), _ptr(o),
                                   _ptr(lse), s), "attn_decode_paged")


def attn_decode_paged_noalloc(q, k_cache, v_cache, k_scale, v_scale, kv_indptr, kv_indices,
                              kv_last_page_len, batch, num_pages, page_size, num_q_heads, num_kv_heads,
                              head_dim, max_kv_len, sm_scale, o, lse=None, stream=None):
    s = _stream(stream, q, o)
    _check(lib().attn_decode_paged_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                           _ptr(v_scale), _ptr(kv_indptr), _ptr(kv_indices),
                                           _ptr(kv_last_page_len), batch, num_pages, page_size,
                                           num_q_heads, num_kv_heads, head_dim, max_kv_len,
                                           float(sm_scale), _ptr(o), _ptr(lse), s),
           "attn_decode_paged_noalloc")


def attn_sparse_mla_decode_workspace_size(batch, s_q, num_heads, topk, sparse_block_size=1) -> int:
    return int(lib().attn_sparse_mla_decode_workspace_size(batch, s_q, num_heads, topk, sparse_block_size))


def attn_sparse_mla_decode(q, kv_cache, kv_dtype, block_table, max_blocks_per_seq, kv_lens, sparse_indices,
                           topk, sparse_block_size, sparse_mode, batch, s_q, num_heads, num_blocks,
                           block_size, sm_scale, workspace, workspace_bytes, o, lse=None, stream=None):
    s = _stream(stream, q, o)
    _check(lib().attn_sparse_mla_decode(_ptr(q), _ptr(kv_cache), kv_dtype, _ptr(block_table),
                                        max_blocks_per_seq, _ptr(kv_lens), _ptr(sparse_indices),
                                        topk, sparse_block_size, sparse_mode, batch, s_q, num_heads,
                                        num_blocks, block_size,
                                        float(sm_scale), _ptr(workspace), int(workspace_bytes),
                                        _ptr(o), _ptr(lse), s), "attn_sparse_mla_decode")
