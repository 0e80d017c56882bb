"""The C ABI on the CPU: the library loads, exports what include/attnq.h
declares, and rejects bad host arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import paged_kv_amd as pk

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(pk.library_path()),
                                reason="libattnq.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[\w]+\**\s+\**(\w+)\s*\(", src, flags=re.M)


def test_header_declares_the_calls():
    names = set(_declared())
    for n in ["attn_quant_qk", "attn_quant_kv", "attn_quant_v_permute", "attn_append_kv_rope", "attn_prefill_varlen",
              "attn_gather_paged_kv", "attn_decode_paged", "attn_sparse_mla_decode"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    h = ctypes.CDLL(pk.library_path())
    for name in _declared():
        assert hasattr(h, name), name
    assert set(_declared()) == set(pk.api.SYMBOLS)


def test_abi_version():
    assert pk.abi_version() == 2


def _err():
    return pk.lib().attnq_last_error().decode()


FAKE = 1 << 20          # aligned, never dereferenced: validation fails first


def test_quant_qk_validation():
    L = pk.lib()
    assert L.attn_quant_qk(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 96, 0, 128, None, FAKE, FAKE, None) == -2
    assert "head_dim" in _err()
    assert L.attn_quant_qk(FAKE, pk.FP8E4M3, FAKE, 1, 10, 10, 2, 64, 0, 128, None, FAKE, FAKE, None) == -2
    assert L.attn_quant_qk(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 64, 7, 128, None, FAKE, FAKE, None) == -1
    assert L.attn_quant_qk(FAKE + 2, pk.BF16, FAKE, 1, 10, 10, 2, 64, 0, 128, None, FAKE, FAKE, None) == -1
    assert "aligned" in _err()
    assert L.attn_quant_qk(FAKE, pk.FP16, FAKE, 1, 10, 10, 2, 64, 1, 64, None, FAKE, FAKE, None) == -2
    assert "block_tokens" in _err()
    assert L.attn_quant_qk(FAKE, pk.FP16, None, 1, 10, 10, 2, 64, 1, 128, None, FAKE, FAKE, None) == -1
    assert "cu_seqlens" in _err()


def test_v_permute_validation():
    L = pk.lib()
    assert L.attn_quant_v_permute(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 64, pk.Q_INT8_PER_BLOCK, None, FAKE, FAKE, None) == -1
    assert L.attn_quant_v_permute(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 64, pk.Q_FP8_PER_HEAD, None, FAKE, None, None) == -1
    assert "v_scales" in _err()
    assert L.attn_quant_v_permute(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 64, pk.Q_FP8_PER_HEAD_WIDE, None, FAKE, None,
                                  None) == -1
    assert "v_scales" in _err()
    assert L.attn_quant_v_permute(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 64, 7, None, FAKE, FAKE, None) != 0
    # per-channel modes: no per-head amax_in, a descale buffer is required
    assert L.attn_quant_v_permute(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 64, pk.Q_FP8_PER_CHANNEL, FAKE, FAKE, FAKE,
                                  None) == -1 and "amax_in" in _err()
    assert L.attn_quant_v_permute(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 64, pk.Q_FP8_PER_CHANNEL_WIDE, None, FAKE, None,
                                  None) == -1 and "v_scales" in _err()


def test_append_validation():
    L = pk.lib()
    args = [FAKE, FAKE, FAKE, pk.BF16, FAKE, None, 1, 4, 2, 2, 64, FAKE, 8, FAKE, FAKE, FAKE, FAKE, 4, 16,
            None, None, None, None]
    bad = list(args)
    bad[18] = 2048
    assert L.attn_append_kv_rope(*bad) == -1 and "page_size" in _err()
    bad = list(args)
    bad[12] = 0
    assert L.attn_append_kv_rope(*bad) == -1
    bad = list(args)
    bad[8], bad[9] = 1000, 1000
    assert L.attn_append_kv_rope(*bad) == -2


def _prefill(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, qk=pk.FP8E4M3, vd=pk.FP8E4M3, qs=FAKE, ks=FAKE, vs=FAKE,
             vmode=pk.Q_FP8_PER_HEAD, mode=pk.Q_FP8_PER_HEAD, cq=FAKE, ck=FAKE, b=1, mq=8, mk=8, tq=8, tk=8, hq=4, hkv=2,
             d=128, sc=0.1, causal=1, o=FAKE, od=pk.BF16, lse=None, st=None)
    a.update(kw)
    return pk.lib().attn_prefill_varlen(*a.values())


def test_prefill_validation():
    assert _prefill(vmode=pk.Q_INT8_PER_BLOCK) == -1 and "v_scale_mode" in _err()
    assert _prefill(vmode=pk.Q_FP8_PER_CHANNEL, vd=pk.FP16, vs=None) == -1 and "v_scale" in _err()
    assert _prefill(vmode=pk.Q_FP8_PER_CHANNEL, vs=FAKE + 4) == -1 and "aligned" in _err()
    assert _prefill(hq=3, hkv=2) == -1 and "multiple" in _err()
    assert _prefill(d=96) == -2
    assert _prefill(qk=pk.INT8) == -2            # int8 codes need per-block scales
    assert _prefill(vd=pk.BF16) == -2
    assert _prefill(od=pk.FP8E4M3) == -2
    assert _prefill(sc=float("inf")) == -1 and "sm_scale" in _err()
    # NaN selects the default 1/sqrt(head_dim): validation goes on to the next argument
    assert _prefill(sc=float("nan"), cq=None) == -1 and "cu_seqlens_q" in _err()
    assert _prefill(cq=None) == -1
    assert _prefill(vs=None) == -1 and "v_scale" in _err()
    assert _prefill(mk=1 << 21, hkv=8, hq=8) == -2 and "2 GiB" in _err()   # 32-bit tile offsets
    # 16-bit Q quantized inside the call: only with INT8_PER_BLOCK_RAW_Q, which takes no codes
    raw = dict(vd=pk.FP16, mode=pk.Q_INT8_PER_BLOCK_RAW_Q)
    assert _prefill(qk=pk.FP16, mode=pk.Q_INT8_PER_BLOCK) == -2
    assert _prefill(qk=pk.INT8, **raw) == -2
    assert _prefill(qk=pk.FP8E4M3, **raw) == -2
    # q_scale is an optional output there; k_scale stays required
    assert _prefill(qk=pk.BF16, qs=None, ks=None, **raw) == -1 and "k_scale" in _err()
    assert _prefill(qk=pk.FP16, qs=FAKE + 2, **raw) == -1 and "q_scale" in _err()


def _decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, ip=FAKE, ind=FAKE, last=FAKE, b=2, np_=10,
             ps=16, hq=32, hkv=8, d=128, mkv=100, sc=0.1, ws=FAKE, wsb=1 << 30, o=FAKE, lse=None, st=None)
    a.update(kw)
    return pk.lib().attn_decode_paged(*a.values())


def test_decode_noalloc_validates_before_touching_a_device():
    # argument errors come first, whatever the device state (no GPU here)
    L = pk.lib()
    assert L.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 16, 32, 8, 96, 100,
                                       0.1, FAKE, None, None) == -2 and "head_dim" in _err()
    assert L.attn_decode_paged_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 2, 10, 8, 32, 8, 128, 100,
                                       0.1, FAKE, None, None) == -1 and "page_size" in _err()
    assert L.attn_decode_paged_noalloc(None, None, None, None, None, None, None, None, 0, 10, 16, 32, 8, 128, 100,
                                       0.1, None, None, None) == 0


def test_decode_validation():
    assert _decode(ps=8) == -1 and "page_size" in _err()
    assert _decode(ps=2048) == -1
    assert _decode(d=96) == -2 and "head_dim" in _err()
    assert _decode(hq=32, hkv=1) == -2
    assert _decode(sc=float("inf")) == -1 and "sm_scale" in _err()
    assert _decode(sc=float("nan"), b=0) == 0      # default scale; nothing to do
    assert _decode(wsb=16) == -3 and "workspace" in _err()
    need = pk.attn_decode_paged_workspace_size(2, 32, 128, 100, 16)
    assert need > 0
    assert _decode(wsb=need - 1) == -3
    assert _decode(ws=FAKE + 8) == -1


def _ppaged(**kw):
    a = dict(q=FAKE, qs=FAKE, mode=pk.Q_FP8_PER_HEAD, kc=FAKE, vc=FAKE, ks=FAKE, vs=FAKE, ip=FAKE, ix=FAKE,
             lpl=FAKE, cu=FAKE, b=2, np_=64, ps=16, mq=100, mk=1000, tq=150, hq=32, hkv=8, d=128, sc=0.1,
             causal=1, o=FAKE, od=pk.BF16, lse=None, st=None)
    a.update(kw)
    return pk.lib().attn_prefill_paged(*a.values())


def test_prefill_paged_validation():
    assert _ppaged(ps=8) == -1 and "page_size" in _err()
    assert _ppaged(ps=40) == -1
    assert _ppaged(d=96) == -2 and "head_dim" in _err()
    assert _ppaged(hq=30, hkv=8) == -1
    assert _ppaged(mode=pk.Q_INT8_PER_BLOCK) == -2 and "scale_mode" in _err()
    assert _ppaged(od=pk.FP8E4M3) == -2
    assert _ppaged(np_=0) == -1 and "num_pages" in _err()
    assert _ppaged(np_=1 << 14, ps=1024) == -2 and "2 GiB" in _err()
    assert _ppaged(sc=float("inf")) == -1 and "sm_scale" in _err()
    assert _ppaged(sc=float("nan"), b=0) == 0      # default scale; nothing to do
    assert _ppaged(tq=0) == 0
    assert _ppaged(kc=FAKE + 8) == -1 and "aligned" in _err()
    assert _ppaged(ix=None) == -1


def _gather(**kw):
    a = dict(c=FAKE, eb=2, ip=FAKE, ix=FAKE, lpl=FAKE, cu=FAKE, b=2, mk=100, np_=64, ps=16, hkv=8,
             d=128, out=FAKE, st=None)
    a.update(kw)
    return pk.lib().attn_gather_paged_kv(*a.values())


def test_gather_validation():
    assert _gather(eb=4) == -1 and "elem_bytes" in _err()
    assert _gather(d=96) == -2 and "head_dim" in _err()
    assert _gather(ps=0) == -1
    assert _gather(np_=0) == -1
    assert _gather(b=-1) == -1
    assert _gather(out=FAKE + 4) == -1 and "aligned" in _err()
    assert _gather(cu=None) == -1 and "cu_seqlens_k" in _err()
    assert _gather(b=0, c=None) == 0          # nothing to do: no pointer is needed
    assert _gather(mk=0, c=None) == 0


def _smooth(**kw):
    a = dict(k=FAKE, cu=FAKE, b=1, mx=10, t=10, h=2, d=128, bt=128, codes=FAKE, sc=FAKE, mean=FAKE, st=None)
    a.update(kw)
    return pk.lib().attn_smooth_quant_k(*a.values())


def test_smooth_quant_k_validation():
    assert _smooth(d=96) == -2 and "head_dim" in _err()
    assert _smooth(bt=64) == -2 and "block_tokens" in _err()
    assert _smooth(h=0) == -1
    assert _smooth(t=-1) == -1
    assert _smooth(mean=None) == -1 and "mean" in _err()
    assert _smooth(codes=FAKE + 4) == -1 and "aligned" in _err()
    assert _smooth(b=0, k=None, cu=None, mean=None) == 0     # nothing to do: no pointer is needed


def _mla(**kw):
    a = dict(q=FAKE, c=FAKE, kvd=pk.INT8, bt=FAKE, mb=4, kl=FAKE, idx=FAKE, topk=8, sbs=1, mode=0, b=1, sq=1,
             h=16, nb=8, bs=64, sc=0.04, ws=FAKE, wsb=1 << 30, o=FAKE, lse=None, st=None)
    a.update(kw)
    return pk.lib().attn_sparse_mla_decode(*a.values())


def test_mla_validation():
    assert _mla(h=12) == -2 and "num_heads" in _err()
    assert _mla(topk=0) == -1 and "topk" in _err()
    assert _mla(bs=8) == -1 and "block_size" in _err()
    assert _mla(bs=1040) == -1
    assert _mla(wsb=8) == -3
    assert _mla(kvd=pk.BF16) == -2 and "kv_dtype" in _err()
    assert _mla(sbs=3) == -2 and "sparse_block_size" in _err()
    assert _mla(sbs=32) == -2
    assert _mla(mode=1) == -2 and "sparse_mode" in _err()
    assert _mla(sc=float("-inf")) == -1 and "sm_scale" in _err()
    assert _mla(sc=float("nan"), b=0) == 0         # default 1/sqrt(576); nothing to do
    L = pk.lib()
    assert L.attn_sparse_mla_decode_workspace_size(1, 1, 16, 8, 3) == 0
    assert L.attn_sparse_mla_decode_workspace_size(1, 1, 16, 300, 4) == L.attn_sparse_mla_decode_workspace_size(1, 1, 16, 1200, 1)


def test_python_binding_raises_with_message():
    with pytest.raises(RuntimeError, match="head_dim"):
        pk.attn_quant_qk(FAKE, pk.BF16, FAKE, 1, 10, 10, 2, 96, pk.Q_FP8_PER_HEAD, 128, None, FAKE,
                         FAKE, stream=0)


def _qkv(**kw):
    a = dict(k=FAKE, v=FAKE, dt=pk.FP16, cu=FAKE, b=2, mx=300, t=400, h=8, d=128, bt=128, kc=FAKE, ks=FAKE, vo=FAKE,
             st=None)
    a.update(kw)
    return pk.lib().attn_quant_kv(*a.values())


def test_quant_kv_validation():
    assert _qkv(dt=pk.INT8) == -2 and "dtype" in _err()
    assert _qkv(d=96) == -2 and "head_dim" in _err()
    assert _qkv(bt=64) == -2 and "block_tokens" in _err()
    assert _qkv(h=0) == -1
    assert _qkv(vo=None) == -1 and "v_out" in _err()
    assert _qkv(kc=FAKE + 8) == -1 and "aligned" in _err()
    assert _qkv(b=0, k=None, v=None, cu=None) == 0           # nothing to do


def test_grid_dimension_limits():
    L = pk.lib()
    assert _smooth(b=70000) == -2 and "batch" in _err()
    assert _mla(b=300, sq=300) == -2 and "s_q" in _err()
    assert _qkv(b=70000) == -2 and "batch" in _err()
    assert _gather(b=70000) == -2 and "batch" in _err()
    assert L.attn_quant_v_permute(FAKE, pk.BF16, FAKE, 70000, 10, 10, 2, 64, pk.Q_NONE, None, FAKE, None, None) == -2
    assert L.attn_quant_qk(FAKE, pk.BF16, FAKE, 70000, 10, 10, 2, 64, pk.Q_INT8_PER_BLOCK, 128, None, FAKE, FAKE,
                           None) == -2
