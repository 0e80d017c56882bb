"""The flows recorded into a HIP graph and replayed (the pages' decode/prefill
plans take an enable_cuda_graph flag; the Ascend operator supports graph
mode).  Every call only enqueues kernels (no allocation, memset, copy or
synchronization), so a recorded flow must reproduce the eager result bit for
bit on every replay -- with unrelated eager work and synchronizations between
replays and the outputs poisoned before each -- and must read its input
buffers live: after new inputs are copied in place, a replay equals an eager
run on the new inputs."""
import math

import numpy as np
import pytest

import gen
from tests.parity import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bits(t):
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().copy()


def _record(run):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()                                    # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    torch.cuda.synchronize()
    return g


def _check_replays(make, refresh, label):
    """make() -> (flow object, output tensors); refresh(flow) copies new
    inputs in place and returns a fresh flow object on the same new data."""
    p, outs = make()
    p.run()
    torch.cuda.synchronize()
    want = [_bits(o) for o in outs]
    g = _record(p.run)
    noise = torch.randn(1024, 1024, device="cuda")
    for i in range(3):
        for o in outs:
            o.view(torch.uint8).fill_(0xFF)      # poison (NaN patterns) outside the graph
        (noise @ noise).sum().item()             # unrelated eager work + a synchronization
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert np.array_equal(_bits(o), w), f"{label}: replay {i} differs from the eager run"
    q, q_outs = refresh(p)
    q.run()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for o, w in zip(outs, q_outs):
        assert np.array_equal(_bits(o), _bits(w)), f"{label}: replay on new inputs differs"
    assert not all(np.array_equal(_bits(o), w) for o, w in zip(outs, want)), f"{label}: inputs not read live"


def test_graph_sage_refined_flow():
    from paged_kv_amd.pipeline import SagePrefill
    x = gen.sage_inputs(101, [700, 129, 1, 300], 8, 2, 128, offset_frac=0.05, v_channel_sd=1.0)
    y = gen.sage_inputs(102, [700, 129, 1, 300], 8, 2, 128, offset_frac=0.05, v_channel_sd=1.0)
    cu, mx = to_dev(x["cu_seqlens"]), 700

    def make():
        p = SagePrefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), cu, mx, 128 ** -0.5, want_lse=True,
                        smooth_k=True, v_fp8_per_channel=True)
        return p, [p.o, p.lse]

    def refresh(p):
        for t, n in ((p.q, "q"), (p.k, "k"), (p.v, "v")):
            t.copy_(to_dev(y[n]))
        r = SagePrefill(to_dev(y["q"]), to_dev(y["k"]), to_dev(y["v"]), cu, mx, 128 ** -0.5, want_lse=True,
                        smooth_k=True, v_fp8_per_channel=True)
        return r, [r.o, r.lse]

    _check_replays(make, refresh, "sage refined")


def test_graph_fp8_prefill():
    from paged_kv_amd.pipeline import Fp8Prefill
    x = gen.prefill_fp8_inputs(103, [513, 64, 0, 200], 8, 2, 128)
    y = gen.prefill_fp8_inputs(104, [513, 64, 0, 200], 8, 2, 128)
    cu = to_dev(x["cu_seqlens"])

    def make():
        p = Fp8Prefill(to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"]), cu, 513, 1 / math.sqrt(128), want_lse=True)
        return p, [p.o, p.lse]

    def refresh(p):
        for t, n in ((p.q, "q"), (p.k, "k"), (p.v, "v")):
            t.copy_(to_dev(y[n]))
        r = Fp8Prefill(to_dev(y["q"]), to_dev(y["k"]), to_dev(y["v"]), cu, 513, 1 / math.sqrt(128), want_lse=True)
        return r, [r.o, r.lse]

    _check_replays(make, refresh, "fp8 prefill")


def test_graph_paged_decode():
    from paged_kv_amd.pipeline import PagedDecode
    x = gen.paged_decode_inputs(105, [700, 64, 2000, 1], 16, 4, 128, page_size=16)
    y = gen.paged_decode_inputs(106, [700, 64, 2000, 1], 16, 4, 128, page_size=16)

    def build(z, q=None):
        p = PagedDecode(to_dev(z["q"]) if q is None else q, to_dev(z["k_cache"]), to_dev(z["v_cache"]),
                        to_dev(z["k_scale"]), to_dev(z["v_scale"]), to_dev(z["kv_indptr"]), to_dev(z["kv_indices"]),
                        to_dev(z["kv_last_page_len"]), z["max_kv_len"], 1 / math.sqrt(128), want_lse=True)
        return p, [p.o, p.lse]

    def refresh(p):
        p.args[0].copy_(to_dev(y["q"]))          # new queries against the same cache
        return build(dict(x, q=y["q"]))

    _check_replays(lambda: build(x), refresh, "paged decode")


def test_graph_sparse_mla_variant():
    from paged_kv_amd.pipeline import SparseMlaDecode
    x = gen.sparse_mla_inputs(107, 2, 3, 16, [1200, 300], 64, 100, n_valid=90, kv_dtype="fp8",
                              sparse_block_size=4)
    q2 = gen.sparse_mla_inputs(108, 2, 3, 16, [1200, 300], 64, 100, n_valid=90, kv_dtype="fp8",
                               sparse_block_size=4)["q"]

    def build(q):
        p = SparseMlaDecode(to_dev(q), to_dev(x["kv_cache"]), to_dev(x["block_table"]), to_dev(x["kv_lens"]),
                            to_dev(x["sparse_indices"]), 1 / 24, want_lse=True, kv_fp8=True, sparse_block_size=4,
                            sparse_mode=3)
        return p, [p.o, p.lse]

    def refresh(p):
        p.q.copy_(to_dev(q2))
        return build(q2)

    _check_replays(lambda: build(x["q"]), refresh, "sparse mla fp8/block/causal")


def test_graph_paged_prefill():
    from paged_kv_amd.pipeline import PagedPrefill
    x = gen.paged_prefill_inputs(109, [1000, 300], [200, 300], 8, 2, 128, page_size=64)
    q2 = gen.paged_prefill_inputs(110, [1000, 300], [200, 300], 8, 2, 128, page_size=64)["q"]

    def build(q):
        p = PagedPrefill(to_dev(q), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["kv_indptr"]),
                         to_dev(x["kv_indices"]), to_dev(x["kv_last_page_len"]), to_dev(x["cu_q"]),
                         to_dev(x["cu_k"]), x["max_q"], x["max_k"], 1 / math.sqrt(128), want_lse=True)
        return p, [p.o, p.lse]

    def refresh(p):
        p.q.copy_(to_dev(q2))
        return build(q2)

    _check_replays(lambda: build(x["q"]), refresh, "paged prefill")
