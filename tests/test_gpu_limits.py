"""GPU parity at the limits of the paged and sparse calls: a sparse block as
long as a page (16 tokens in 16-token pages), the largest page (1024 rows)
with 2-token blocks, the odd head count 48 with the causal mode and more
query rows than some sequences have tokens, and a prefill chunk against
1024-token pages with single-token and whole-sequence chunks."""
import pytest

import gen
from tests.test_gpu_mla_variants import _check as _mla_check
from tests.test_gpu_paged_prefill import _check as _paged_check

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kv", ["int8", "fp8"])
def test_mla_sparse_block_equals_page(kv):
    x = gen.sparse_mla_inputs(131, 3, 2, 16, [512, 37, 1000], 16, 40, n_valid=33, spare_blocks=4,
                              kv_dtype=kv, sparse_block_size=16)
    _mla_check(x, 3, label=f"sbs = page = 16, {kv}")


def test_mla_largest_page_small_blocks():
    x = gen.sparse_mla_inputs(132, 2, 3, 128, [3000, 1500], 1024, 700, n_valid=650, spare_blocks=1,
                              kv_dtype="fp8", sparse_block_size=2)
    _mla_check(x, 0, label="page 1024, sbs 2")


def test_mla_48_heads_causal_short_sequences():
    # 6 query rows; sequences of 3 and 0 tokens leave some rows with nothing to see
    x = gen.sparse_mla_inputs(133, 3, 6, 48, [3, 0, 900], 64, 64, n_valid=60, sparse_block_size=8)
    _mla_check(x, 3, label="H=48 causal short")


def test_paged_prefill_largest_page():
    x = gen.paged_prefill_inputs(134, [3000, 1, 1025, 2048], [1, 1, 1025, 700], 8, 2, 128, page_size=1024)
    x["sm_scale"] = 128 ** -0.5
    _paged_check(x, True, "page 1024")
