"""GPU parity of the 128x128 block-scaled FP8 path (qlin_gemv_fp8_blk): the
exported activation codes and UE8M0 exponents are compared bit-exactly, the
output under the float rules of oracle/compare.py."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits, lib, need_gpu, padded
from oracle.compare import check_float
from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_fp8_blk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _gpu(ql, d, w_dev=None):
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), dev(d["w"]) if w_dev is None else w_dev, dev(d["ws"]))
    torch.cuda.synchronize()
    return host_bits(y), host(xq), host(xs)


def _check(orc, d, got):
    y, xq, xs = got
    oxq, oxs, oy, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert np.array_equal(xs, oxs), "UE8M0 activation exponents differ"
    bad = np.argwhere(xq != oxq)
    assert bad.size == 0, f"E4M3 activation codes differ at {bad[:5].tolist()}"
    return check_float(y, ye, S, d["w"].shape[1])


@pytest.mark.parametrize("M", list(range(1, 17)))
def test_blk_small_all_M(ql, orc, M):
    d = gen_fp8_blk(M, 384, 1024, seed=M)
    _check(orc, d, _gpu(ql, d))


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (2, 130, 384), (3, 257, 896), (9, 100, 640), (16, 555, 1152),
                                   # M = 1 kernel: partial step, two batches, three batches with a short last one
                                   (1, 5, 1152), (1, 67, 9216), (1, 3, 16512),
                                   # 512..1023 row tiles: eight waves split K
                                   (4, 9000, 2048), (16, 8200, 2304),
                                   # one workgroup exports every group; M = 1 past the fused path's K limit
                                   (7, 1, 2048), (16, 9, 1280), (1, 3, 33024), (2, 3, 33024)])
def test_blk_ragged(ql, orc, M, N, K):
    d = gen_fp8_blk(M, N, K, seed=N + K)
    _check(orc, d, _gpu(ql, d))


@pytest.mark.parametrize("M", [1, 8, 16])
def test_blk_full(ql, orc, M):
    d = gen_fp8_blk(M, 4096, 7168, seed=0)
    stats = _check(orc, d, _gpu(ql, d))
    assert stats["ref_bits_equal"] > 0.99


def test_blk_act_quant_edge_values(ql, orc):
    # every E4M3 midpoint and its neighbours, zero groups, tiny / huge groups, signed zeros
    rng = np.random.default_rng(40)
    K = 128 * 12
    x = rng.standard_normal((3, K)).astype(np.float32)
    e4 = orc.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mids = ((e4[:-1] + e4[1:]) / 2).astype(np.float32)  # exact midpoints (bf16 may round some)
    x[0, :126] = mids
    x[0, 126] = 448.0
    x[0, 128:254] = -mids
    x[0, 254] = -448.0
    x[1, 256:384] = 0.0
    x[1, 384:512] = -0.0
    x[1, 512:640] *= 1e-35
    x[1, 640:768] *= 3e25  # E ~ 202; the result stays inside the fp32/bf16 range
    x[2, 768:896] = np.where(np.arange(128) % 2 == 0, 1e-6, -1e-6)
    x[2, 800] = 100.0
    x[2, 1024:1152] *= 1e-38  # below every exponent byte above 0: E clamped at 1
    x[2, 1152:1280] *= 1e-40  # bf16 subnormals
    d = {"x": bf16_bits(x), "w": rng.integers(0, 0x7E, (130, K)).astype(np.uint8),
         "ws": rng.integers(110, 140, (2, K // 128)).astype(np.uint8)}
    assert np.all(np.isfinite(bf16_values(orc.fp8_blk(d["x"], d["w"], d["ws"])[2])))
    _check(orc, d, _gpu(ql, d))


def test_blk_unit_scales_match_plain_fp8(ql, orc):
    # all weight scale bytes 127 and x already on E4M3 values with group max 448:
    # the block path must equal the weight-only path with ws = 1
    rng = np.random.default_rng(41)
    K, N = 1024, 200
    fin = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    xc = fin[rng.integers(0, fin.size, (2, K))]
    xc[:, ::128] = 0x7E
    x = bf16_bits(orc.e4m3_decode(xc.astype(np.uint8)).astype(np.float32))
    w = fin[rng.integers(0, fin.size, (N, K))].astype(np.uint8)
    d = {"x": x, "w": w, "ws": np.full(((N + 127) // 128, K // 128), 127, np.uint8)}
    yb, xq, xs = _gpu(ql, d)
    assert np.all(xs == 127)
    yp = host_bits(ql.qlin_gemv_fp8(dev_bf16(x), dev(w), dev(np.ones(1, np.float32))))
    _, ye, S = orc.gemv_fp8(x, w, np.ones(1, np.float32))
    check_float(yb, ye, S, K)
    check_float(yp, ye, S, K)


def test_blk_padded_row_stride(ql, orc):
    d = gen_fp8_blk(2, 300, 1024, seed=42)
    wp = padded(d["w"], 256)
    a = _gpu(ql, d, w_dev=wp)
    b = _gpu(ql, d)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_blk_deterministic(ql):
    d = gen_fp8_blk(16, 4096, 7168, seed=43)
    x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
    ref = ql.qlin_gemv_fp8_blk(x, w, ws)[0]
    for _ in range(10):
        assert torch.equal(ql.qlin_gemv_fp8_blk(x, w, ws)[0].view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M", [1, 5, 16])
def test_blk_padded_activation_stride(ql, orc, M):
    d = gen_fp8_blk(M, 300, 1024, seed=44 + M)
    xp = padded(d["x"].view(np.int16), 40).view(torch.bfloat16)  # row pitch 1064 elements
    y, xq, xs = ql.qlin_gemv_fp8_blk(xp, dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    _check(orc, d, (host_bits(y), host(xq), host(xs)))


def test_blk_act_quant_edge_values_one_token(ql, orc):
    # the same edge rows one token at a time: the one-kernel path (quantiser
    # fused into the M = 1 GEMV) sees midpoints, signed zeros, zero / tiny /
    # huge groups
    rng = np.random.default_rng(40)
    K = 128 * 12
    x = rng.standard_normal((3, K)).astype(np.float32)
    e4 = orc.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mids = ((e4[:-1] + e4[1:]) / 2).astype(np.float32)
    x[0, :126] = mids
    x[0, 126] = 448.0
    x[0, 128:254] = -mids
    x[0, 254] = -448.0
    x[1, 256:384] = 0.0
    x[1, 384:512] = -0.0
    x[1, 512:640] *= 1e-35
    x[1, 640:768] *= 3e25
    x[2, 768:896] = np.where(np.arange(128) % 2 == 0, 1e-6, -1e-6)
    x[2, 800] = 100.0
    x[2, 1024:1152] *= 1e-38  # below every exponent byte above 0: E clamped at 1
    x[2, 1152:1280] *= 1e-40  # bf16 subnormals
    w = rng.integers(0, 0x7E, (130, K)).astype(np.uint8)
    ws = rng.integers(110, 140, (2, K // 128)).astype(np.uint8)
    for r in range(3):
        print(f"blk edge row {r} as one token", flush=True)
        d = {"x": bf16_bits(x[r:r + 1]), "w": w, "ws": ws}
        _check(orc, d, _gpu(ql, d))


@pytest.mark.parametrize("M", [1, 16])
def test_blk_extreme_weight_scale_bytes(ql, orc, M):
    # weight scale bytes 0 (2^-127, an fp32 subnormal), 1, 253 and 254 (2^127);
    # activation groups sized so every output stays finite: tiny groups where
    # the weight scale is huge, large groups where it is tiny
    rng = np.random.default_rng(45)
    K, N = 128 * 4, 256
    ws = np.array([[0, 1, 253, 254], [1, 0, 254, 253]], np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, 0:256] *= 1e10    # groups 0, 1: weight scales 2^-127 / 2^-126
    x[:, 256:512] *= 1e-30  # groups 2, 3: weight scales 2^126 / 2^127
    w = gen_fp8_blk(1, N, K, seed=46)["w"]
    d = {"x": bf16_bits(x), "w": w, "ws": ws}
    assert np.all(np.isfinite(bf16_values(orc.fp8_blk(d["x"], d["w"], d["ws"])[2])))
    print(f"blk extreme scale bytes M={M}", flush=True)
    _check(orc, d, _gpu(ql, d))


def test_blk_one_token_without_exported_codes(ql, orc):
    # one token: the codes / scales buffers are optional (NULL: not written)
    d = gen_fp8_blk(1, 4096, 7168, seed=47)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]), export=False)
    torch.cuda.synchronize()
    assert xq is None and xs is None
    y_ref = _gpu(ql, d)[0]
    assert np.array_equal(host_bits(y), y_ref)
    with pytest.raises(ql.QlinError):  # two tokens need the buffers
        ql.qlin_gemv_fp8_blk(dev_bf16(gen_fp8_blk(2, 64, 256, seed=1)["x"]), dev(d["w"][:64, :256]),
                             dev(d["ws"][:1, :2].copy()), export=False)
