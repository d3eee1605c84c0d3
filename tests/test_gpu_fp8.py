"""GPU parity of the FP8-E4M3 weight-only GEMV (qlin_gemv_fp8) against the CPU
oracle, under the float comparison rules of oracle/compare.py, plus an exhaustive
check of the hardware E4M3 decode through the product path."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host_bits, lib, need_gpu, padded
from oracle.compare import bf16_to_f64, check_float
from skinny_gemm_qlin_amd.inputs import bf16_bits, gen_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _gpu(ql, d, w_dev=None):
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), dev(d["w"]) if w_dev is None else w_dev, dev(d["ws"]))
    torch.cuda.synchronize()
    return host_bits(y)


def test_e4m3_decode_every_code(ql, orc):
    # row n holds code n at column k; x one-hot at k; ws = 1 -> y[n] = bf16(decode(code n)) exactly
    K, k = 64, 37
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    w = np.zeros((codes.size, K), np.uint8)
    w[:, k] = codes
    x = np.zeros((1, K), np.float32)
    x[0, k] = 1.0
    d = {"x": bf16_bits(x), "w": w, "ws": np.ones(codes.size, np.float32)}
    y = bf16_to_f64(_gpu(ql, d))[0]
    ref = orc.e4m3_decode(codes)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("per_tensor", [False, True])
def test_fp8_small_all_M(ql, orc, M, per_tensor):
    d = gen_fp8(M, 1024, 1024, seed=M, per_tensor=per_tensor)
    y, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(_gpu(ql, d), ye, S, 1024)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (2, 3, 48), (3, 37, 272), (4, 129, 1040),
                                   (8, 255, 4112), (11, 17, 2064), (16, 1001, 784),
                                   # 512..1023 row tiles: eight waves split K
                                   (3, 9000, 2048), (16, 9001, 2320)])
def test_fp8_ragged(ql, orc, M, N, K):
    d = gen_fp8(M, N, K, seed=N + K)
    y, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(_gpu(ql, d), ye, S, K)


# one token with 9 to 16 steps of 1 KB per row (8192 < K <= 16384): the
# LDS-staged kernel with every step in flight; a partial last step, N not a
# multiple of the 8 rows of a workgroup, a padded row stride; longer rows up
# to K = 32768 on fewer than 4096 rows: the row in LDS taken 16 steps at a
# time; the rest on the per-tile matrix-core kernel
@pytest.mark.parametrize("N,K,per_tensor,pad", [(777, 8208, False, 0), (4099, 12288, True, 0),
                                                (300, 14336, False, 256), (1001, 16384, False, 0),
                                                (65, 16368, True, 48), (130, 16400, False, 0),
                                                (1000, 20480, True, 48), (2049, 32768, False, 16),
                                                (33, 32784, False, 0), (4100, 20480, False, 0)])
def test_fp8_one_token_long_rows(ql, orc, N, K, per_tensor, pad):
    d = gen_fp8(1, N, K, seed=N + K, per_tensor=per_tensor)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("per_tensor", [False, True])
def test_fp8_decode_full(ql, orc, M, per_tensor):
    d = gen_fp8(M, 17408, 5120, seed=0, per_tensor=per_tensor)
    y, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    stats = check_float(_gpu(ql, d), ye, S, 5120)
    assert stats["ref_bits_equal"] > 0.99


def test_fp8_padded_row_stride(ql, orc):
    d = gen_fp8(3, 200, 1024, seed=5)
    wp = padded(d["w"], 256)
    assert _gpu(ql, d, w_dev=wp).tolist() == _gpu(ql, d).tolist()


def test_fp8_deterministic(ql):
    d = gen_fp8(8, 2048, 5120, seed=6)
    x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
    ref = ql.qlin_gemv_fp8(x, w, ws)
    for _ in range(20):
        assert torch.equal(ql.qlin_gemv_fp8(x, w, ws).view(torch.int16), ref.view(torch.int16))


# two tokens with both rows staged in LDS (K <= 16384): K from one chunk to
# the largest, ragged N, padded weight and activation pitches; past 16384 the
# per-tile matrix-core kernel
@pytest.mark.parametrize("M,N,K", [(2, 1001, 16), (2, 77, 1040), (2, 1001, 5120), (2, 300, 16384), (2, 2000, 10912),
                                   (2, 9, 8192), (2, 4097, 7168), (2, 1, 4096), (2, 130, 16400), (2, 1001, 24576)])
def test_fp8_two_tokens_rows_in_lds(ql, orc, M, N, K):
    d = gen_fp8(M, N, K, seed=M * 11 + N + K, per_tensor=N % 2 == 0)
    xp = np.zeros((M, K + 24), np.uint16)
    xp[:, :K] = d["x"]
    x = dev_bf16(xp)[:, :K]
    y = ql.qlin_gemv_fp8(x, padded(d["w"], 48), dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)
