"""GPU parity of the prefill path (M > 16: the tiled matrix-core GEMM behind
the dense entry points) against the CPU oracle.  INT8 codes, scales, int32
accumulators and bf16 outputs are bit-exact; FP8 outputs follow the float
comparison rules of oracle/compare.py.  Small shapes are compared in full
(several 128 x 128 tiles, ragged M, N and K); the 17408 x 5120 decode matrix
at M = 512 is compared on sampled tokens and rows, each computed by the
oracle one by one."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits, lib, need_gpu, padded
from oracle.compare import check_float
from skinny_gemm_qlin_amd.inputs import bf16_bits, gen_fp8, gen_fp8_blk, gen_fp8_w8a8, gen_int8

pytestmark = pytest.mark.gpu

SHAPES = [(17, 128, 64), (33, 129, 272), (100, 250, 1040), (128, 128, 128), (129, 383, 528),
          (300, 77, 2064), (257, 1000, 784)]


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


# ----------------------------------------------------------------------------- INT8

@pytest.mark.parametrize("M,N,K", SHAPES)
def test_prefill_int8_bit_exact(ql, orc, M, N, K):
    d = gen_int8(M, N, K, seed=M + N + K)
    x = dev_bf16(d["x"])
    xq, xs = ql.qlin_act_quant_i8(x)
    acc = ql.qlin_gemv_i8(xq, xs, dev(d["w"]), dev(d["ws"]), out_kind=1)
    y = ql.qlin_gemv_i8(xq, xs, dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_i8(d["x"])
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(xs).view(np.uint32), oxs.view(np.uint32))
    oacc, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"])
    assert np.array_equal(host(acc), oacc)
    assert np.array_equal(host_bits(y), oy)


def test_prefill_int8_bias_per_tensor_and_padded(ql, orc):
    M, N, K = 70, 300, 1024
    d = gen_int8(M, N, K, seed=5)
    rng = np.random.default_rng(6)
    bias = bf16_bits(rng.standard_normal(N).astype(np.float32))
    oxq, oxs = orc.act_quant_i8(d["x"])
    for xs_t, ws_t in ((oxs, d["ws"]), (oxs[:1], d["ws"]), (oxs, d["ws"][:1])):
        y = ql.qlin_gemv_i8(dev(oxq), dev(xs_t), padded(d["w"], 64), dev(ws_t), bias=dev_bf16(bias))
        torch.cuda.synchronize()
        _, oy = orc.gemv_i8(oxq, xs_t, d["w"], ws_t, bias=bias)
        assert np.array_equal(host_bits(y), oy)


def test_prefill_int8_extreme_accumulators(ql, orc):
    # every product +-127*127 of one sign: the largest int32 accumulators of the shape
    M, N, K = 40, 136, 4096
    xq = np.full((M, K), 127, np.int8)
    xq[1::2] = -127
    w = np.full((N, K), -127, np.int8)
    acc = ql.qlin_gemv_i8(dev(xq), dev(np.ones(M, np.float32)), dev(w), dev(np.ones(N, np.float32)), out_kind=1)
    torch.cuda.synchronize()
    oacc, _ = orc.gemv_i8(xq, np.ones(M, np.float32), w, np.ones(N, np.float32))
    assert np.array_equal(host(acc), oacc) and oacc[0, 0] == -127 * 127 * K


# K % 128 == 0: the direct-to-LDS kernel (64 x 64 tiles up to 256 tokens,
# 64 x 128 up to 1024, 128 x 128 above); ragged M and N in every tile size
DMA_SHAPES = [(17, 64, 128), (33, 129, 256), (100, 250, 1024), (256, 64, 384), (257, 1000, 768),
              (600, 65, 640), (1024, 130, 256), (1030, 200, 384), (1100, 383, 512)]


@pytest.mark.parametrize("M,N,K", DMA_SHAPES)
def test_prefill_int8_dma_bit_exact(ql, orc, M, N, K):
    d = gen_int8(M, N, K, seed=M * 3 + N + K)
    rng = np.random.default_rng(M)
    bias = bf16_bits(rng.standard_normal(N).astype(np.float32))
    xq, xs = ql.qlin_act_quant_i8(dev_bf16(d["x"]))
    acc = ql.qlin_gemv_i8(xq, xs, dev(d["w"]), dev(d["ws"]), out_kind=1)
    y = ql.qlin_gemv_i8(xq, xs, padded(d["w"], 128), dev(d["ws"]), bias=dev_bf16(bias))
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_i8(d["x"])
    oacc, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"], bias=bias)
    assert np.array_equal(host(acc), oacc)
    assert np.array_equal(host_bits(y), oy)


@pytest.mark.parametrize("M,N,K", DMA_SHAPES)
@pytest.mark.parametrize("per_tensor", [False, True])
def test_prefill_fp8_dma(ql, orc, M, N, K, per_tensor):
    d = gen_fp8(M, N, K, seed=M * 11 + N + K, per_tensor=per_tensor)
    y = ql.qlin_gemv_fp8(padded(d["x"].view(np.int16), 64).view(torch.bfloat16), padded(d["w"], 128),
                         dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K", DMA_SHAPES)
@pytest.mark.parametrize("x_fmt,w_fmt", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_prefill_fp8_w8a8_dma(ql, orc, M, N, K, x_fmt, w_fmt):
    d = gen_fp8_w8a8(M, N, K, w_fmt=w_fmt, seed=M + 5 * N + K)
    xq, xs = ql.qlin_act_quant_fp8(dev_bf16(d["x"]), x_fmt, True)
    y = ql.qlin_gemv_fp8_w8a8(xq, xs, dev(d["w"]), dev(d["ws"]), x_fmt, w_fmt)
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_fp8(d["x"], x_fmt, True)
    assert np.array_equal(host(xq), oxq)
    _, ye, S = orc.gemv_fp8_w8a8(oxq, oxs, x_fmt, d["w"], d["ws"], w_fmt)
    check_float(host_bits(y), ye, S, K)


# ----------------------------------------------------------------------------- FP8 weight-only

@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("per_tensor", [False, True])
def test_prefill_fp8(ql, orc, M, N, K, per_tensor):
    d = gen_fp8(M, N, K, seed=M * 7 + N, per_tensor=per_tensor)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


# ----------------------------------------------------------------------------- FP8 W8A8

@pytest.mark.parametrize("M,N,K", SHAPES[:5])
@pytest.mark.parametrize("x_fmt,w_fmt", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_prefill_fp8_w8a8(ql, orc, M, N, K, x_fmt, w_fmt):
    d = gen_fp8_w8a8(M, N, K, w_fmt=w_fmt, seed=M + 3 * N)
    xq, xs = ql.qlin_act_quant_fp8(dev_bf16(d["x"]), x_fmt, True)
    y = ql.qlin_gemv_fp8_w8a8(xq, xs, dev(d["w"]), dev(d["ws"]), x_fmt, w_fmt)
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_fp8(d["x"], x_fmt, True)
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(xs), oxs)
    _, ye, S = orc.gemv_fp8_w8a8(oxq, oxs, x_fmt, d["w"], d["ws"], w_fmt)
    check_float(host_bits(y), ye, S, K)


def test_prefill_fp8_w8a8_static_per_tensor_scale(ql, orc):
    # a per-tensor activation scale supplied by the caller (e.g. calibrated)
    M, N, K = 200, 256, 512
    d = gen_fp8_w8a8(M, N, K, seed=11)
    oxq, oxs = orc.act_quant_fp8(d["x"][:16], 0, False)  # per-tensor scale of 16 rows
    xq = np.concatenate([oxq] * (M // 16 + 1))[:M]
    y = ql.qlin_gemv_fp8_w8a8(dev(xq), dev(oxs), dev(d["w"]), dev(d["ws"]), 0, 0)
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8_w8a8(xq, oxs, 0, d["w"], d["ws"], 0)
    check_float(host_bits(y), ye, S, K)


# ----------------------------------------------------------------------------- block FP8

@pytest.mark.parametrize("M,N,K", [(17, 128, 128), (33, 129, 256), (100, 250, 1024), (129, 383, 512),
                                   (300, 77, 2048), (257, 1000, 768), (1030, 200, 384), (1100, 130, 640)])
def test_prefill_fp8_blk(ql, orc, M, N, K):
    d = gen_fp8_blk(M, N, K, seed=M + N)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs, _, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(xs), oxs)
    check_float(host_bits(y), ye, S, K)


# ----------------------------------------------------------------------------- full decode matrix, M = 512

@pytest.fixture(scope="module")
def sample():
    rng = np.random.default_rng(99)
    ms = np.sort(rng.choice(512, 24, replace=False))
    ns = np.sort(np.concatenate([rng.choice(17408, 40, replace=False), [0, 127, 128, 17407]]))
    return ms, ns


def test_prefill_int8_full_sampled(ql, orc, sample):
    ms, ns = sample
    d = gen_int8(512, 17408, 5120, seed=0)
    xq, xs = ql.qlin_act_quant_i8(dev_bf16(d["x"]))
    y = ql.qlin_gemv_i8(xq, xs, dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    hxq, hxs, hy = host(xq), host(xs), host_bits(y)
    oxq, oxs = orc.act_quant_i8(d["x"][ms])
    assert np.array_equal(hxq[ms], oxq) and np.array_equal(hxs[ms], oxs)
    _, oy = orc.gemv_i8(oxq, oxs, d["w"][ns], d["ws"][ns])
    assert np.array_equal(hy[np.ix_(ms, ns)], oy)


def test_prefill_fp8_full_sampled(ql, orc, sample):
    ms, ns = sample
    d = gen_fp8(512, 17408, 5120, seed=0)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"][ms], d["w"][ns], d["ws"][ns])
    check_float(host_bits(y)[np.ix_(ms, ns)], ye, S, 5120)


def test_prefill_fp8_w8a8_full_sampled(ql, orc, sample):
    ms, ns = sample
    d = gen_fp8_w8a8(512, 17408, 5120, seed=0)
    xq, xs = ql.qlin_act_quant_fp8(dev_bf16(d["x"]), 0, True)
    y = ql.qlin_gemv_fp8_w8a8(xq, xs, dev(d["w"]), dev(d["ws"]), 0, 0)
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_fp8(d["x"][ms], 0, True)
    assert np.array_equal(host(xq)[ms], oxq)
    _, ye, S = orc.gemv_fp8_w8a8(oxq, oxs, 0, d["w"][ns], d["ws"][ns], 0)
    check_float(host_bits(y)[np.ix_(ms, ns)], ye, S, 5120)


def test_prefill_fp8_blk_full_sampled(ql, orc, sample):
    ms, _ = sample
    d = gen_fp8_blk(512, 4096, 7168, seed=0)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs, _, ye, S = orc.fp8_blk(d["x"][ms], d["w"], d["ws"])
    assert np.array_equal(host(xq)[ms], oxq) and np.array_equal(host(xs)[ms], oxs)
    check_float(host_bits(y)[ms], ye, S, 7168)


def test_prefill_deterministic(ql):
    d = gen_fp8(200, 1024, 2048, seed=3)
    x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
    ref = ql.qlin_gemv_fp8(x, w, ws)
    for _ in range(10):
        assert torch.equal(ql.qlin_gemv_fp8(x, w, ws).view(torch.int16), ref.view(torch.int16))


# ----------------------------------------------------------------------------- few rows: split-K

# Fewer than a quarter of the compute units' worth of 64 x 64 output tiles:
# the matrix-core kernels over 16-row x 16-token workgroups, K split between
# the waves of each and summed in wave order.  The shapes the Z100 record
# lists for its small-N gap (N = 48 at M = 64) and its neighbours, plus
# ragged ones.
SPLIT_SHAPES = [(64, 48, 5120), (512, 48, 5120), (64, 96, 5120), (512, 96, 5120), (64, 200, 5120),
                (512, 200, 5120), (17, 47, 1040), (100, 1, 272), (513, 33, 2064)]


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_prefill_split_int8(ql, orc, M, N, K):
    d = gen_int8(M, N, K, seed=M + 2 * N + K)
    oxq, oxs = orc.act_quant_i8(d["x"])
    rng = np.random.default_rng(N)
    bias = bf16_bits(rng.standard_normal(N).astype(np.float32))
    acc = ql.qlin_gemv_i8(dev(oxq), dev(oxs), dev(d["w"]), dev(d["ws"]), out_kind=1)
    y = ql.qlin_gemv_i8(dev(oxq), dev(oxs), dev(d["w"]), dev(d["ws"]), bias=dev_bf16(bias))
    torch.cuda.synchronize()
    oacc, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"], bias=bias)
    assert np.array_equal(host(acc), oacc)
    assert np.array_equal(host_bits(y), oy)


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_prefill_split_fp8(ql, orc, M, N, K):
    d = gen_fp8(M, N, K, seed=M + 3 * N + K)
    y = ql.qlin_gemv_fp8(padded(d["x"].view(np.int16), 64).view(torch.bfloat16), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K", SPLIT_SHAPES)
def test_prefill_split_fp8_w8a8(ql, orc, M, N, K):
    d = gen_fp8_w8a8(M, N, K, w_fmt=0, seed=M + 5 * N + K)
    oxq, oxs = orc.act_quant_fp8(d["x"], 0, True)
    y = ql.qlin_gemv_fp8_w8a8(dev(oxq), dev(oxs), dev(d["w"]), dev(d["ws"]), 0, 0)
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8_w8a8(oxq, oxs, 0, d["w"], d["ws"], 0)
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K", [(64, 48, 5120), (512, 48, 5120), (512, 200, 5120), (17, 47, 1024),
                                   (100, 130, 384)])
def test_prefill_split_fp8_blk(ql, orc, M, N, K):
    d = gen_fp8_blk(M, N, K, seed=M + 7 * N)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs, _, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(xs), oxs)
    check_float(host_bits(y), ye, S, K)


def test_prefill_split_deterministic(ql):
    d = gen_fp8(512, 48, 5120, seed=8)
    x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
    ref = ql.qlin_gemv_fp8(x, w, ws)
    for _ in range(10):
        assert torch.equal(ql.qlin_gemv_fp8(x, w, ws).view(torch.int16), ref.view(torch.int16))


# ----------------------------------------------------------------------------- enough rows for the tiled GEMM

# at least a quarter of the compute units' worth of 64 x 64 tiles, ragged M and
# N at every tile size; K % 128 != 0 (register-staged kernel) and K % 128 == 0
# (direct-to-LDS kernel)
GEMM_SHAPES = [(17, 4100, 272), (129, 2050, 528), (300, 1100, 2064), (17, 4100, 128), (100, 2050, 1024),
               (256, 1030, 384), (600, 530, 640), (1030, 520, 384)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_prefill_gemm_int8(ql, orc, M, N, K):
    d = gen_int8(M, N, K, seed=M + 11 * N + K)
    oxq, oxs = orc.act_quant_i8(d["x"])
    acc = ql.qlin_gemv_i8(dev(oxq), dev(oxs), dev(d["w"]), dev(d["ws"]), out_kind=1)
    y = ql.qlin_gemv_i8(dev(oxq), dev(oxs), padded(d["w"], 64), dev(d["ws"]))
    torch.cuda.synchronize()
    oacc, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"])
    assert np.array_equal(host(acc), oacc)
    assert np.array_equal(host_bits(y), oy)


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_prefill_gemm_fp8(ql, orc, M, N, K):
    d = gen_fp8(M, N, K, seed=M + 13 * N + K)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
@pytest.mark.parametrize("x_fmt,w_fmt", [(0, 0), (1, 0)])
def test_prefill_gemm_fp8_w8a8(ql, orc, M, N, K, x_fmt, w_fmt):
    d = gen_fp8_w8a8(M, N, K, w_fmt=w_fmt, seed=M + 17 * N + K)
    oxq, oxs = orc.act_quant_fp8(d["x"], x_fmt, True)
    y = ql.qlin_gemv_fp8_w8a8(dev(oxq), dev(oxs), dev(d["w"]), dev(d["ws"]), x_fmt, w_fmt)
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8_w8a8(oxq, oxs, x_fmt, d["w"], d["ws"], w_fmt)
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K", [(17, 4100, 128), (100, 2050, 1024), (600, 530, 640), (1030, 520, 384)])
def test_prefill_gemm_fp8_blk(ql, orc, M, N, K):
    d = gen_fp8_blk(M, N, K, seed=M + 19 * N)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs, _, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(xs), oxs)
    check_float(host_bits(y), ye, S, K)
