"""GPU parity of the block-scaled FP8 path at block shapes other than
128 x 128 (qlin_gemv_fp8_blk_ex) against the CPU oracle: activation codes and
exponents bit-exact, outputs under the float comparison rules."""
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


def _run(ql, d, bn, bk, w_dev=None):
    y, xq, xs = ql.qlin_gemv_fp8_blk_ex(dev_bf16(d["x"]), dev(d["w"]) if w_dev is None else w_dev, dev(d["ws"]),
                                        bn, bk)
    torch.cuda.synchronize()
    return host_bits(y), host(xq), host(xs)


def _check(orc, d, bn, bk, got, K):
    y, xq, xs = got
    oxq, oxs, _, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"], bn, bk)
    assert np.array_equal(xq, oxq), "activation codes differ"
    assert np.array_equal(xs, oxs), "activation exponents differ"
    check_float(y, ye, S, K)


@pytest.mark.parametrize("bn,bk", [(1, 32), (1, 64), (16, 32), (32, 128), (64, 64), (7, 32), (128, 256),
                                   (3, 96), (128, 64), (1, 128)])
@pytest.mark.parametrize("M", [1, 5, 16])
def test_blk_shapes(ql, orc, bn, bk, M):
    N, K = 300, 768
    d = gen_fp8_blk(M, N, K, seed=bn * 100 + bk + M, scale_lo=110, scale_hi=135, block_n=bn, block_k=bk)
    _check(orc, d, bn, bk, _run(ql, d, bn, bk), K)


@pytest.mark.parametrize("M,N,K,bn,bk", [(2, 17, 32, 1, 32), (3, 1001, 1056, 1, 32), (16, 129, 2304, 16, 64),
                                         (9, 4096, 7168, 1, 32), (12, 9000, 512, 1, 32),
                                         (33, 200, 512, 1, 32), (70, 130, 1024, 32, 64)])
def test_blk_shapes_ragged_and_prefill(ql, orc, M, N, K, bn, bk):
    d = gen_fp8_blk(M, N, K, seed=M + N + K, block_n=bn, block_k=bk)
    _check(orc, d, bn, bk, _run(ql, d, bn, bk), K)


# above 16 tokens with K % 128 == 0: one tiled GEMM with the scales applied in
# the operand converts; (800, 1, 32) has K % 128 != 0 (GEMV per 16 tokens)
@pytest.mark.parametrize("bn,bk", [(1, 32), (16, 32), (32, 128), (64, 64), (7, 32), (128, 256), (3, 96),
                                   (128, 64), (1, 128)])
@pytest.mark.parametrize("M", [17, 100, 300])
def test_blk_shapes_prefill_gemm(ql, orc, bn, bk, M):
    N, K = 300, 768
    d = gen_fp8_blk(M, N, K, seed=bn * 7 + bk + M, scale_lo=110, scale_hi=135, block_n=bn, block_k=bk)
    _check(orc, d, bn, bk, _run(ql, d, bn, bk), K)


def test_blk_shapes_prefill_k_not_multiple_of_128(ql, orc):
    d = gen_fp8_blk(40, 150, 800, seed=3, block_n=1, block_k=32)
    _check(orc, d, 1, 32, _run(ql, d, 1, 32), 800)


def test_blk_shapes_prefill_full_mx_shape(ql, orc):
    # the 4096 x 7168 block-FP8 matrix with MX-style 1 x 32 scales, 128 tokens
    d = gen_fp8_blk(128, 4096, 7168, seed=4, block_n=1, block_k=32)
    _check(orc, d, 1, 32, _run(ql, d, 1, 32), 7168)


@pytest.mark.parametrize("byte,x_exp", [(10, 0), (246, -100)])
def test_blk_shapes_prefill_scale_range_ends(ql, orc, byte, x_exp):
    # the ends of the weight-scale range in which the GEMM's scaled converts are
    # exact (x scaled so that the outputs stay finite)
    M, N, K, bn, bk = 40, 64, 256, 1, 32
    d = gen_fp8_blk(M, N, K, seed=6, block_n=bn, block_k=bk)
    d["ws"][:] = byte
    d["x"] = bf16_bits(bf16_values(d["x"]) * np.float32(2.0 ** x_exp))
    _check(orc, d, bn, bk, _run(ql, d, bn, bk), K)


def test_blk_shapes_edge_scales(ql, orc):
    # scale bytes at the ends of their range (2^-127 and large) and a zero group
    M, N, K, bn, bk = 3, 64, 256, 1, 32
    d = gen_fp8_blk(M, N, K, seed=5, block_n=bn, block_k=bk)
    d["ws"][0, :] = 0
    d["ws"][1, :] = 200
    x = bf16_values(d["x"]).copy()
    x[1, 32:64] = 0.0
    d["x"] = bf16_bits(x)
    _check(orc, d, bn, bk, _run(ql, d, bn, bk), K)


def test_blk_shapes_128_is_the_tested_path(ql, orc):
    d = gen_fp8_blk(4, 256, 1024, seed=8)
    a = _run(ql, d, 128, 128)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    assert np.array_equal(a[0], host_bits(y)) and np.array_equal(a[1], host(xq))


def test_blk_shapes_padded_and_deterministic(ql, orc):
    d = gen_fp8_blk(6, 200, 1024, seed=9, block_n=1, block_k=32)
    ref = _run(ql, d, 1, 32)
    assert np.array_equal(_run(ql, d, 1, 32, w_dev=padded(d["w"], 64))[0], ref[0])
    for _ in range(5):
        assert np.array_equal(_run(ql, d, 1, 32)[0], ref[0])
