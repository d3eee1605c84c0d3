"""GPU parity of the W8A8 INT8 path (qlin_act_quant_i8 + qlin_gemv_i8) against
the CPU oracle: codes, scales, int32 accumulators and the bf16 epilogue are all
compared bit-exactly."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits, lib, need_gpu, padded
from skinny_gemm_qlin_amd.inputs import bf16_bits, gen_int8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _run_full(ql, x_bits, w, ws, bias=None, w_dev=None):
    x = dev_bf16(x_bits)
    xq, xs = ql.qlin_act_quant_i8(x)
    wd = dev(w) if w_dev is None else w_dev
    acc = ql.qlin_gemv_i8(xq, xs, wd, dev(ws), out_kind=1)
    y = ql.qlin_gemv_i8(xq, xs, wd, dev(ws), bias=None if bias is None else dev_bf16(bias))
    torch.cuda.synchronize()
    return host(xq), host(xs), host(acc), host_bits(y)


def _check(orc, x_bits, w, ws, got, bias=None):
    xq, xs, acc, y = got
    oxq, oxs = orc.act_quant_i8(x_bits)
    assert np.array_equal(xq, oxq), "int8 codes differ"
    assert np.array_equal(xs.view(np.uint32), oxs.view(np.uint32)), "scales differ"
    oacc, oy = orc.gemv_i8(oxq, oxs, w, ws, bias=bias)
    assert np.array_equal(acc, oacc), "int32 accumulators differ"
    assert np.array_equal(y, oy), "bf16 outputs differ"


# small config: M=1, N=K=1024 (seed 0) and every M on the same shape
@pytest.mark.parametrize("M", list(range(1, 17)))
def test_int8_small_all_M(ql, orc, M):
    d = gen_int8(M, 1024, 1024, seed=0)
    _check(orc, d["x"], d["w"], d["ws"], _run_full(ql, d["x"], d["w"], d["ws"]))


# ragged shapes: N not a multiple of the row tile, K not a multiple of the K step
@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (2, 3, 48), (3, 37, 272), (5, 129, 1040),
                                   (7, 255, 4112), (9, 61, 528), (13, 17, 2064), (16, 1001, 784),
                                   # 512..1023 row tiles: eight waves split K
                                   (4, 9000, 2048), (16, 9001, 2320)])
def test_int8_ragged(ql, orc, M, N, K):
    d = gen_int8(M, N, K, seed=M * 1000 + N)
    _check(orc, d["x"], d["w"], d["ws"], _run_full(ql, d["x"], d["w"], d["ws"]))


# >= 1024 row tiles (four waves split K) and M >= 12: every 256-K chunk of a
# wave in flight at once for 1..5 chunks per wave, the chunk loop above that;
# ragged K tails inside the last chunk
@pytest.mark.parametrize("M,K", [(12, 768), (12, 1040), (16, 2064), (13, 3072), (16, 4096), (16, 5008), (12, 5376)])
def test_int8_large_n_chunks_in_flight(ql, orc, M, K):
    d = gen_int8(M, 16400, K, seed=M + K)
    _check(orc, d["x"], d["w"], d["ws"], _run_full(ql, d["x"], d["w"], d["ws"]))


# decode config: N=17408, K=5120, every M of the workload, full comparison
@pytest.fixture(scope="module")
def decode_w():
    d = gen_int8(16, 17408, 5120, seed=0)
    return d


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_int8_decode_full(ql, orc, decode_w, M):
    d = gen_int8(M, 17408, 5120, seed=0)
    assert np.array_equal(d["w"], decode_w["w"])
    _check(orc, d["x"], d["w"], d["ws"], _run_full(ql, d["x"], d["w"], d["ws"]))


def test_int8_padded_row_stride_and_broadcast(ql, orc):
    # weights stored with a padded row pitch (K + 256) read the same as contiguous
    d = gen_int8(4, 300, 1024, seed=7)
    wp = padded(d["w"], 256)
    assert wp.stride(0) == 1024 + 256
    got = _run_full(ql, d["x"], d["w"], d["ws"], w_dev=wp)
    _check(orc, d["x"], d["w"], d["ws"], got)
    # broadcast scales [1]
    x = dev_bf16(d["x"])
    xq, xs = ql.qlin_act_quant_i8(x)
    ws1 = np.array([0.004], np.float32)
    y = ql.qlin_gemv_i8(xq, xs[:1].contiguous(), dev(d["w"]), dev(ws1))
    oxq, oxs = orc.act_quant_i8(d["x"])
    _, oy = orc.gemv_i8(oxq, oxs[:1], d["w"], ws1)
    assert np.array_equal(host_bits(y), oy)


def test_int8_bias(ql, orc):
    d = gen_int8(3, 513, 2048, seed=8)
    bias = bf16_bits(np.random.default_rng(8).standard_normal(513).astype(np.float32))
    _check(orc, d["x"], d["w"], d["ws"], _run_full(ql, d["x"], d["w"], d["ws"], bias=bias), bias=bias)


def test_int8_edge_rows(ql, orc):
    # zero row (s = 0), ties (amax = 127 -> s = 1), a one-hot row, huge and tiny magnitudes
    K = 256
    rows = np.zeros((5, K), np.float32)
    rows[1, :8] = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5]
    rows[2, 77] = -3.0
    rows[3] = np.linspace(-3e30, 2e30, K)
    rows[4] = np.linspace(-1e-30, 3e-30, K)
    x = bf16_bits(rows)
    w = np.random.default_rng(9).integers(-128, 128, size=(40, K), dtype=np.int8)
    ws = np.random.default_rng(9).uniform(1e-3, 1e-2, 40).astype(np.float32)
    _check(orc, x, w, ws, _run_full(ql, x, w, ws))


def test_int8_max_k_exact(ql, orc):
    # K at its limit with every product at +-127*128: int32 accumulation stays exact
    K = 131072
    x = bf16_bits(np.full((1, K), 5.0, np.float32))       # codes all 127
    w = np.full((4, K), -128, np.int8)
    w[1] = 127
    w[2, ::2] = 127
    w[3] = np.random.default_rng(10).integers(-128, 128, K, dtype=np.int8)
    ws = np.ones(4, np.float32)
    _check(orc, x, w, ws, _run_full(ql, x, w, ws))


def test_int8_errors_leave_output_untouched(ql):
    d = gen_int8(2, 64, 256, seed=11)
    xq = dev(np.zeros((2, 256), np.int8))
    xs = dev(np.ones(2, np.float32))
    y = torch.full((2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    lib_ = ql.load()
    st = lib_.qlin_gemv_i8(xq.data_ptr(), 256, xs.data_ptr(), 1, 0, 256, dev(d["w"]).data_ptr(), 256, 64,
                           dev(d["ws"]).data_ptr(), 1, None, y.data_ptr(), 64, 0, None)
    assert st == -2
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
    with pytest.raises(ql.QlinError):
        ql.qlin_gemv_i8(xq[:, :250], xs, dev(d["w"])[:, :250], dev(d["ws"]))


def test_int8_deterministic(ql):
    d = gen_int8(8, 4096, 5120, seed=12)
    x = dev_bf16(d["x"])
    w = dev(d["w"])
    ws = dev(d["ws"])
    xq, xs = ql.qlin_act_quant_i8(x)
    ref = ql.qlin_gemv_i8(xq, xs, w, ws)
    for _ in range(20):
        xq2, xs2 = ql.qlin_act_quant_i8(x)
        y = ql.qlin_gemv_i8(xq2, xs2, w, ws)
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_int8_quantiser_divides(ql, orc):
    # bf16 inputs on which x/s and x*(1/s) give different codes: the kernel's
    # codes must be those of the one correctly rounded division
    from test_oracle_int8 import DIV_CASES
    K = 16
    rows = np.zeros((len(DIV_CASES), K), np.float32)
    for i, (amax, xv, _) in enumerate(DIV_CASES):
        rows[i, :3] = [amax, xv, -xv]
    x = bf16_bits(rows)
    xq, xs = ql.qlin_act_quant_i8(dev_bf16(x))
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_i8(x)
    assert np.array_equal(host(xq), oxq) and np.array_equal(host(xs).view(np.uint32), oxs.view(np.uint32))
    for i, (_, _, code) in enumerate(DIV_CASES):
        assert list(host(xq)[i, :3]) == [127, code, -code]


# Each epilogue kernel applies (acc*xs)*ws itself: the vector kernels (1-2
# tokens), the matrix-core kernel (K not a multiple of 1024), the K-slice
# kernel (K a multiple of 1024) and the prefill GEMM (more than 16 tokens).
@pytest.mark.parametrize("K,reps", [(16, 1), (1024, 1), (16, 3)])
def test_int8_epilogue_order_constructed(ql, orc, K, reps):
    from test_oracle_int8 import epilogue_case_arrays
    xq4, w4, xs, ws = epilogue_case_arrays()
    C = len(xs)
    xq = np.zeros((C * reps, K), np.int8)
    xq[:, :4] = np.tile(xq4, (reps, 1))
    xsr = np.tile(xs, reps)
    w = np.zeros((C, K), np.int8)
    w[:, :4] = w4
    _, oy = orc.gemv_i8(xq, xsr, w, ws)
    for M in sorted({1, 2, C * reps}):
        y = ql.qlin_gemv_i8(dev(xq[:M]), dev(xsr[:M]), dev(w), dev(ws))
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(y), oy[:M]), f"M={M}"
