"""GPU parity of the sparse MLA-absorb decode through the C ABI."""
import numpy as np
import pytest

import gen
from oracle.attention import sparse_mla_decode
from tests.parity import to_dev, from_dev_bits, decode_out, compare_outputs, compare_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(x, sm_scale):
    from paged_kv_amd.pipeline import SparseMlaDecode
    p = SparseMlaDecode(to_dev(x["q"]), to_dev(x["kv_cache"]), to_dev(x["block_table"]),
                        to_dev(x["kv_lens"]), to_dev(x["sparse_indices"]), sm_scale, want_lse=True)
    p.run()
    torch.cuda.synchronize()
    return p


def _check(x, sm_scale, batches=None, label=""):
    p = _run(x, sm_scale)
    ref = sparse_mla_decode(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"], x["sparse_indices"],
                            sm_scale, batches=batches)
    sel = list(range(x["q"].shape[0])) if batches is None else list(batches)
    got = decode_out(from_dev_bits(p.o), "bf16")[sel]
    st = compare_outputs(got, ref["o"][sel], ref["o_exact"][sel], "bf16", label)
    compare_lse(p.lse.cpu().numpy()[sel], ref["lse"][sel], label)
    return p, st


@pytest.mark.parametrize("heads", [128, 16, 48, 1])
def test_mla_small(heads):
    # ragged valid counts (some -1 padding), two queries per sequence
    x = gen.sparse_mla_inputs(61, 3, 2, heads, [300, 64, 1000], 64, 100, n_valid=70, spare_blocks=3)
    _check(x, 1 / 24, label=f"H={heads}")


def test_mla_topk_not_multiple_of_step_and_invalid_entries():
    x = gen.sparse_mla_inputs(62, 2, 1, 32, [129, 40], 16, 37)
    idx = x["sparse_indices"].copy()
    idx[0, 0, 0, 3] = 129          # == kv_len: unused
    idx[1, 0, 0, 5] = -7           # negative: unused
    idx[1, 0, 0, 6] = idx[1, 0, 0, 7]  # duplicate: counted twice
    x["sparse_indices"] = idx
    _check(x, 0.05, label="ragged topk")


def test_mla_no_valid_entry():
    x = gen.sparse_mla_inputs(63, 2, 1, 16, [64, 64], 64, 40)
    x["sparse_indices"][1] = -1
    p, _ = _check(x, 1 / 24, label="empty row")
    assert not p.o[1].float().abs().sum().item()


def test_mla_index_order_invariance():
    x = gen.sparse_mla_inputs(64, 1, 1, 64, [4096], 64, 512)
    a = decode_out(from_dev_bits(_run(x, 1 / 24).o), "bf16")
    y = dict(x)
    y["sparse_indices"] = x["sparse_indices"][..., ::-1].copy()
    b = decode_out(from_dev_bits(_run(y, 1 / 24).o), "bf16")
    assert np.abs(a - b).max() <= 2e-2 and np.abs(a - b).mean() <= 2e-3


def test_config4_full_size():
    """The sparse MLA workload at full size (B=32, 128 heads, 65536-token
    caches in 64-token blocks, 2048 distinct indices, NaN in every
    unselected row): every batch and head against the oracle."""
    x = gen.config4()
    p, st = _check(x, x["sm_scale"], label="config4")
    assert torch.isfinite(p.o.float()).all()
    print("PARITY config4 (all 32 batches):", st)
