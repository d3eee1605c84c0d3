"""GPU parity of qlin_linear_i8 (the whole INT8 decode linear layer in one
call: per-token quantisation + W8A8 GEMV; one kernel for one token) and of
the two- and three-token INT8 GEMV kernels that stage the codes in LDS, all
against the CPU oracle bit for bit: codes, scales and bf16 outputs."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, host_bits, lib, need_gpu, padded
from skinny_gemm_qlin_amd.inputs import bf16_bits, gen_int8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _bf16(bits, pad=0):
    if pad:
        return padded(bits.view(np.int16), pad).view(torch.bfloat16)
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def _check(ql, orc, x_bits, w, ws, bias=None, x_pad=0, w_pad=0):
    M, K = x_bits.shape
    print(f"linear_i8 M={M} N={w.shape[0]} K={K} x_pad={x_pad} w_pad={w_pad}", flush=True)
    wd = dev(w) if w_pad == 0 else padded(w, w_pad)
    y, xq, xs = ql.qlin_linear_i8(_bf16(x_bits, x_pad), wd, dev(ws), bias=None if bias is None else _bf16(bias))
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_i8(x_bits)
    _, oy = orc.gemv_i8(oxq, oxs, w, ws, bias=bias)
    assert np.array_equal(host(xq), oxq), "int8 codes differ"
    assert np.array_equal(host(xs).view(np.uint32), oxs.view(np.uint32)), "scales differ"
    assert np.array_equal(host_bits(y), oy), "bf16 outputs differ"


@pytest.fixture(scope="module")
def decode():
    return gen_int8(16, 17408, 5120, seed=0)


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_linear_i8_decode_workload(ql, orc, decode, M):
    _check(ql, orc, decode["x"][:M], decode["w"], decode["ws"])


# one token: K across the fused kernel's range and past it (8208: two launches),
# N from one row to a partial last workgroup
@pytest.mark.parametrize("N,K", [(1, 16), (7, 48), (129, 272), (1001, 1040), (300, 2064), (17, 4112),
                                 (1001, 8192), (9, 8208), (9001, 2048)])
def test_linear_i8_one_token_shapes(ql, orc, N, K):
    d = gen_int8(1, N, K, seed=N + K)
    _check(ql, orc, d["x"], d["w"], d["ws"])


def test_linear_i8_one_token_edge_rows(ql, orc):
    # each row alone through the one-kernel path: zero row (s = 0), ties at
    # s = 1, a one-hot row, huge and tiny magnitudes, and the searched rows
    # where x * (1/s) would round to another code than x / s
    from test_oracle_int8 import DIV_CASES
    K = 256
    rows = np.zeros((5 + len(DIV_CASES), K), np.float32)
    rows[1, :8] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]
    rows[2, 77] = -3.0
    rows[3] = np.linspace(-3e30, 2e30, K)
    rows[4] = np.linspace(-1e-30, 3e-30, K)
    for i, (amax, xv, _) in enumerate(DIV_CASES):
        rows[5 + i, :3] = [amax, xv, -xv]
        rows[5 + i, 100:110] = xv
    x = bf16_bits(rows)
    rng = np.random.default_rng(9)
    w = rng.integers(-128, 128, size=(40, K), dtype=np.int8)
    ws = rng.uniform(1e-3, 1e-2, 40).astype(np.float32)
    for r in range(x.shape[0]):
        _check(ql, orc, x[r:r + 1], w, ws)


def test_linear_i8_bias_broadcast_and_pitches(ql, orc):
    for M in (1, 3):
        d = gen_int8(M, 513, 2048, seed=8 + M)
        bias = bf16_bits(np.random.default_rng(8).standard_normal(513).astype(np.float32))
        _check(ql, orc, d["x"], d["w"], d["ws"], bias=bias, x_pad=64, w_pad=256)
        _check(ql, orc, d["x"], d["w"], np.array([0.004], np.float32))


def test_linear_i8_repeats_are_identical(ql):
    d = gen_int8(1, 4096, 5120, seed=12)
    x, w, ws = _bf16(d["x"]), dev(d["w"]), dev(d["ws"])
    ref, _, _ = ql.qlin_linear_i8(x, w, ws)
    for _ in range(20):
        y, _, _ = ql.qlin_linear_i8(x, w, ws)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


# the two- and three-token GEMV kernels (codes in LDS, K <= 16384; for one
# token from K = 8208; longer rows 16 steps at a time while the codes fit in
# 64 KB and N < 4096) and the per-tile matrix-core kernel past that
@pytest.mark.parametrize("M,N,K", [(2, 17408, 5120), (3, 17408, 5120), (2, 1, 16), (3, 9, 8192), (2, 100, 8208),
                                   (3, 1001, 1040),
                                   # 9 to 16 steps of 1 KB per row, also for one token
                                   (2, 4096, 14336), (3, 1001, 8208), (2, 77, 16384), (3, 513, 12304),
                                   (1, 4096, 14336), (1, 77, 8208), (1, 1001, 16384),
                                   # 16 steps at a time
                                   (2, 300, 16400), (2, 1001, 20480), (2, 100, 32768), (3, 777, 21840),
                                   # past them: the per-tile matrix-core kernel
                                   (3, 64, 32768), (2, 50, 32784), (2, 4096, 20480)])
def test_gemv_i8_two_three_tokens(ql, orc, M, N, K):
    d = gen_int8(M, N, K, seed=M * 100 + N)
    oxq, oxs = orc.act_quant_i8(d["x"])
    oacc, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"])
    acc = ql.qlin_gemv_i8(dev(oxq), dev(oxs), dev(d["w"]), dev(d["ws"]), out_kind=1)
    y = ql.qlin_gemv_i8(dev(oxq), dev(oxs), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), oacc)
    assert np.array_equal(host_bits(y), oy)
