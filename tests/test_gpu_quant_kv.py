"""GPU parity of attn_quant_kv (K int8 blocks and the V permute in one
launch): bit-identical to attn_quant_qk INT8_PER_BLOCK on K plus
attn_quant_v_permute NONE on V, and to the oracle; every output position is
written (outputs start as garbage)."""
import numpy as np
import pytest

import gen
from oracle.quant import quant_int8_per_block, v_permute, s_pad
from tests.parity import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run(k, v, cu, mx, dtype, fused):
    import paged_kv_amd as A
    t, h, d = k.shape
    b = len(cu) - 1
    nblk = (mx + 127) // 128
    kc = torch.full((t, h, d), 77, dtype=torch.int8, device="cuda")
    ks = torch.full((b, h, nblk), 3.0, dtype=torch.float32, device="cuda")
    vo = torch.full((b, h, d, s_pad(mx)), 7.0, dtype=torch.float16, device="cuda")
    dk, dv, dcu = to_dev(k), to_dev(v), to_dev(cu)
    code = A.BF16 if dtype == "bf16" else A.FP16
    if fused:
        A.attn_quant_kv(dk, dv, code, dcu, b, mx, t, h, d, 128, kc, ks, vo)
    else:
        A.attn_quant_qk(dk, code, dcu, b, mx, t, h, d, A.Q_INT8_PER_BLOCK, 128, None, kc, ks)
        A.attn_quant_v_permute(dv, code, dcu, b, mx, t, h, d, A.Q_NONE, None, vo, None)
    torch.cuda.synchronize()
    return kc.cpu().numpy(), ks.cpu().numpy(), vo.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_quant_kv_equals_separate_calls_and_oracle(dtype, d):
    lens = [300, 1, 0, 129, 64]
    x = gen.prefill_fp8_inputs(121, lens, 2, 2, d) if dtype == "bf16" else gen.sage_inputs(121, lens, 2, 2, d)
    cu, mx = x["cu_seqlens"], max(lens)
    f = _run(x["k"], x["v"], cu, mx, dtype, True)
    sep = _run(x["k"], x["v"], cu, mx, dtype, False)
    for a, b_ in zip(f, sep):
        assert np.array_equal(a, b_)
    kc, ks = quant_int8_per_block(x["k"], dtype, cu, mx)
    vref, _ = v_permute(x["v"], dtype, cu, mx, fp8=False)
    assert np.array_equal(f[0], kc)
    assert np.array_equal(f[1].view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(f[2], np.asarray(vref).view(np.uint16))


def test_quant_kv_config2():
    x = gen.config2()
    cu, mx = x["cu_seqlens"], int(x["seqlens"].max())
    f = _run(x["k"], x["v"], cu, mx, "fp16", True)
    sep = _run(x["k"], x["v"], cu, mx, "fp16", False)
    for a, b_ in zip(f, sep):
        assert np.array_equal(a, b_)
