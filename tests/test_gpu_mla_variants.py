"""GPU parity of the sparse MLA variants through the C ABI: fp8 e4m3 rows,
block-wise sparse selection (sparse_block_size > 1) and the right-down causal
mask (sparse_mode 3) over several query rows, alone and together."""
import numpy as np
import pytest

import gen
from oracle.attention import sparse_mla_decode
from tests.parity import to_dev, from_dev_bits, decode_out, compare_outputs, compare_lse

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _check(x, mode, sm_scale=1 / 24, batches=None, label=""):
    from paged_kv_amd.pipeline import SparseMlaDecode
    p = SparseMlaDecode(to_dev(x["q"]), to_dev(x["kv_cache"]), to_dev(x["block_table"]),
                        to_dev(x["kv_lens"]), to_dev(x["sparse_indices"]), sm_scale, want_lse=True,
                        kv_fp8=x["kv_dtype"] == "fp8", sparse_block_size=x["sparse_block_size"],
                        sparse_mode=mode)
    p.run()
    torch.cuda.synchronize()
    ref = sparse_mla_decode(x["q"], x["kv_cache"], x["block_table"], x["kv_lens"], x["sparse_indices"],
                            sm_scale, batches=batches, kv_dtype=x["kv_dtype"],
                            sparse_block_size=x["sparse_block_size"], sparse_mode=mode)
    sel = list(range(x["q"].shape[0])) if batches is None else list(batches)
    got = decode_out(from_dev_bits(p.o), "bf16")[sel]
    compare_outputs(got, ref["o"][sel], ref["o_exact"][sel], "bf16", label)
    compare_lse(p.lse.cpu().numpy()[sel], ref["lse"][sel], label)
    return p, ref


@pytest.mark.parametrize("mode", [0, 3])
@pytest.mark.parametrize("sbs", [1, 4, 16])
@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_mla_variants(kv, sbs, mode):
    # three query rows per sequence; topk * sbs spans one or two 512-slot splits;
    # -1 padding after the valid entries; a sequence shorter than the query rows
    topk = {1: 100, 4: 60, 16: 40}[sbs]
    x = gen.sparse_mla_inputs(71, 4, 3, 32, [300, 64, 1000, 2], 64, topk, n_valid=topk - 7,
                              spare_blocks=2, kv_dtype=kv, sparse_block_size=sbs)
    idx = x["sparse_indices"]
    idx[0, 1, 0, 2] = idx[0, 1, 0, 0]            # duplicate entry: counted twice
    _check(x, mode, label=f"{kv} sbs={sbs} mode={mode}")


@pytest.mark.parametrize("heads", [128, 1])
def test_mla_right_down_causal_long_rows(heads):
    # 8 query rows against the last tokens: every row's mask cuts differently
    x = gen.sparse_mla_inputs(72, 2, 8, heads, [2048, 517], 64, 600, n_valid=590)
    kv = x["kv_lens"]
    idx = x["sparse_indices"]
    rows = x["kv_cache"].reshape(-1, 656)
    data_row = rows[x["block_table"][0][idx[0, 0, 0, 0] // 64] * 64 + idx[0, 0, 0, 0] % 64].copy()
    for b in range(2):                            # put some selections right at the diagonal
        idx[b, :, 0, :8] = (kv[b] - 8 + np.arange(8))[None, :]
        for t in kv[b] - 8 + np.arange(8):        # and give their rows data (unselected rows hold NaN)
            r = x["block_table"][b][t // 64] * 64 + t % 64
            if np.isnan(rows[r, 640:656].view(np.float32)).any():
                rows[r] = data_row
    _, ref = _check(x, 3, label=f"causal H={heads}")
    assert np.isfinite(ref["lse"]).all()


def test_mla_fp8_rows_at_scale():
    # 128 heads, 2048 selections over 16K tokens per sequence, fp8 rows
    x = gen.sparse_mla_inputs(73, 4, 1, 128, 16384, 64, 2048, kv_dtype="fp8")
    _check(x, 0, batches=[0, 3], label="fp8 at scale")
