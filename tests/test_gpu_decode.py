"""GPU parity of the split-KV paged fp8 decode through the C ABI."""
import math

import numpy as np
import pytest

import gen
from oracle.attention import decode_paged
from tests.parity import to_dev, from_dev_bits, decode_out, compare_outputs, compare_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(x, sm_scale):
    from paged_kv_amd.pipeline import PagedDecode
    p = PagedDecode(to_dev(x["q"]), to_dev(x["k_cache"]), to_dev(x["v_cache"]), to_dev(x["k_scale"]),
                    to_dev(x["v_scale"]), to_dev(x["kv_indptr"]), to_dev(x["kv_indices"]),
                    to_dev(x["kv_last_page_len"]), x["max_kv_len"], sm_scale, want_lse=True)
    p.run()
    torch.cuda.synchronize()
    return p


def _check(x, sm_scale, batches=None, label=""):
    p = _run(x, sm_scale)
    ref = decode_paged(x["q"], x["k_cache"], x["v_cache"], x["k_scale"], x["v_scale"], x["kv_indptr"],
                       x["kv_indices"], x["kv_last_page_len"], sm_scale, batches=batches)
    sel = list(range(x["q"].shape[0])) if batches is None else list(batches)
    got = decode_out(from_dev_bits(p.o), "bf16")[sel]
    st = compare_outputs(got, ref["o"][sel], ref["o_exact"][sel], "bf16", label)
    compare_lse(p.lse.cpu().numpy()[sel], ref["lse"][sel], label)
    return p, st


@pytest.mark.parametrize("ps", [16, 32, 64])
def test_decode_small(ps):
    x = gen.paged_decode_inputs(51, [5, 0, 33, 16, 600, 1, 1025], 32, 8, 128, page_size=ps)
    _check(x, 1 / math.sqrt(128), label=f"ps={ps}")


def test_decode_odd_step_tails_repeated():
    """Chunks with an odd number of 32-token steps end in a step that fetches
    nothing ahead: its V stage, loaded during the step before, must have
    landed before its transposed reads.  Tails of 1, 3, .. 15 steps, each call
    against the oracle once, then bit-identical over repeated calls (the split
    and merge are deterministic)."""
    lens = [512 + 32 * (2 * i + 1) - 7 for i in range(8)] + [32 * (2 * i + 1) for i in range(8)]
    x = gen.paged_decode_inputs(77, lens, 32, 8, 128, page_size=16)
    p, _ = _check(x, 1 / math.sqrt(128), label="odd step tails")
    first = p.o.clone()
    for _ in range(20):
        p.run()
        torch.cuda.synchronize()
        assert torch.equal(p.o, first)


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 1), (12, 4), (6, 3), (10, 5), (16, 16)])
def test_decode_group_sizes(hq, hkv):
    x = gen.paged_decode_inputs(52, [700, 64, 2000], hq, hkv, 128, page_size=16)
    _check(x, 0.09, label=f"{hq}/{hkv}")


@pytest.mark.parametrize("ps", [48, 1024])
def test_decode_page_sizes_and_chunk_edges(ps):
    # pages that do not divide the 512-token chunk (48) or hold two chunks (1024);
    # lengths on and next to chunk and page boundaries
    x = gen.paged_decode_inputs(54, [511, 512, 513, 1537, 47, 2048], 16, 4, 128, page_size=ps)
    _check(x, 1 / math.sqrt(128), label=f"ps={ps}")


def test_decode_page_permutation_bit_identical():
    x = gen.paged_decode_inputs(53, [900, 300], 32, 8, 128)
    a = from_dev_bits(_run(x, 0.1).o).copy()
    rng = np.random.default_rng(1)
    perm = rng.permutation(x["num_pages"])
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    y = dict(x)
    y["k_cache"], y["v_cache"] = x["k_cache"][perm], x["v_cache"][perm]
    y["kv_indices"] = inv[x["kv_indices"]].astype(np.int32)
    assert np.array_equal(from_dev_bits(_run(y, 0.1).o), a)


def test_config3_full_size():
    """Paged fp8 decode at full size (B=64, kv lens U{1024..32768}, page 16,
    32/8 heads): every sequence and head against the oracle."""
    x = gen.config3()
    p, st = _check(x, x["sm_scale"], label="config3")
    assert torch.isfinite(p.o.float()).all()
    print("PARITY config3 (all 64 sequences):", st)
