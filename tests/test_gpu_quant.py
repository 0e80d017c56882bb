"""GPU parity of the quantizers through the C ABI: codes and scales bit-exact."""
import numpy as np
import pytest

import gen
from oracle.numerics import e4m3fn_encode
from oracle.quant import quant_fp8_per_head, quant_int8_per_block, v_permute
from tests.parity import to_dev, dev_u8

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _run_fp8(x_np, dtype, cu):
    import paged_kv_amd as pk
    x = to_dev(x_np)
    t, h, d = x.shape
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(h, dtype=torch.float32, device="cuda")
    pk.attn_quant_qk(x, pk.BF16 if dtype == "bf16" else pk.FP16, to_dev(cu), len(cu) - 1, 0, t, h, d,
                     pk.Q_FP8_PER_HEAD, 128, None, codes, scales)
    torch.cuda.synchronize()
    return dev_u8(codes), scales.cpu().numpy()


@pytest.mark.parametrize("name", ["q", "k", "v"])
def test_fp8_per_head_config1(name):
    x = gen.config1()
    codes, ds = _run_fp8(x[name], "bf16", x["cu_seqlens"])
    rc, rd = quant_fp8_per_head(x[name], "bf16")
    assert np.array_equal(ds.view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(codes, rc)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 128), ("bf16", 64)])
def test_fp8_per_head_ragged_with_outliers(dtype, d):
    x = gen.prefill_fp8_inputs(77, [1, 700, 0, 1299], 8, 8, d, outlier_p=0.001)
    q = x["q"] if dtype == "bf16" else (x["q"].astype(np.uint32) << 16).view(np.float32).astype(np.float16)
    codes, ds = _run_fp8(q, dtype, x["cu_seqlens"])
    rc, rd = quant_fp8_per_head(q, dtype)
    assert np.array_equal(ds.view(np.uint32), rd.view(np.uint32))
    assert np.array_equal(codes, rc)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fp8_encoder_on_every_16bit_value(dtype):
    # one head holds every finite 16-bit value with |x| <= 448 (and 448
    # itself), so its descale is exactly 1 and each code is the plain
    # encoding of that value; the other head is all zero (descale 1, codes 0)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if dtype == "bf16":
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        keep = np.isfinite(vals) & (np.abs(vals) <= 448)
        x16 = bits[keep]
        v32 = vals[keep]
    else:
        vals = bits.view(np.float16).astype(np.float32)
        keep = np.isfinite(vals) & (np.abs(vals) <= 448)
        x16 = bits[keep]
        v32 = vals[keep]
    n = ((x16.size + 127) // 128) * 128
    pad = np.zeros(n, np.uint16)
    pad[:x16.size] = x16
    arr = np.zeros((n // 128, 2, 128), np.uint16)
    arr[:, 0, :] = pad.reshape(-1, 128)
    if dtype == "fp16":
        arr = arr.view(np.float16)
    codes, ds = _run_fp8(arr, dtype, np.array([0, n // 128], np.int32))
    assert ds[0] == 1.0 and ds[1] == 1.0
    assert np.array_equal(codes[:, 0, :].reshape(-1)[:x16.size], e4m3fn_encode(v32))
    assert not codes[:, 1, :].any()


@pytest.mark.parametrize("lens", [[130, 257, 1, 0, 384], [4096, 512]])
def test_int8_per_block(lens):
    x = gen.sage_inputs(5, lens, 4, 2, 128)
    import paged_kv_amd as pk
    cu = x["cu_seqlens"]
    mx = max(lens)
    for name, h in (("q", 4), ("k", 2)):
        xd = to_dev(x[name])
        t = xd.shape[0]
        nblk = (mx + 127) // 128
        codes = torch.zeros(xd.shape, dtype=torch.int8, device="cuda")
        scales = torch.full((len(lens), h, nblk), -7.0, dtype=torch.float32, device="cuda")
        pk.attn_quant_qk(xd, pk.FP16, to_dev(cu), len(lens), mx, t, h, 128, pk.Q_INT8_PER_BLOCK, 128,
                         None, codes, scales)
        torch.cuda.synchronize()
        rc, rs = quant_int8_per_block(x[name], "fp16", cu, mx, 128)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32)), name
        assert np.array_equal(codes.cpu().numpy(), rc), name


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("fp8,dtype", [(True, "bf16"), (False, "fp16"), (False, "bf16"), (True, "fp16")])
def test_v_permute(fp8, dtype, d):
    import paged_kv_amd as pk
    lens = [37, 64, 1, 0, 200, 65, 131]
    if dtype == "bf16":
        v = gen.prefill_fp8_inputs(9, lens, 2, 2, d)["v"]
    else:
        v = gen.sage_inputs(9, lens, 2, 2, d)["v"]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    mx = max(lens)
    sp = (mx + 127) // 128 * 128
    vd = to_dev(v)
    out = torch.full((len(lens), 2, d, sp), 0x55 if fp8 else 0, dtype=torch.uint8 if fp8 else torch.int16,
                     device="cuda")
    vs = torch.empty(2, dtype=torch.float32, device="cuda")
    pk.attn_quant_v_permute(vd, pk.BF16 if dtype == "bf16" else pk.FP16, to_dev(cu), len(lens), mx, cu[-1],
                            2, d, pk.Q_FP8_PER_HEAD if fp8 else pk.Q_NONE, None, out, vs if fp8 else None)
    torch.cuda.synchronize()
    ref, rds = v_permute(v, dtype, cu, mx, fp8=fp8)
    got = out.cpu().numpy()
    if fp8:
        assert np.array_equal(vs.cpu().numpy().view(np.uint32), rds.view(np.uint32))
        assert np.array_equal(got, ref)
    else:
        assert np.array_equal(got.view(np.uint16), np.asarray(ref).view(np.uint16))
