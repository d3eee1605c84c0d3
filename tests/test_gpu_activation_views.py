"""GPU parity of the dense decode GEMVs with activation rows stored at a padded
pitch (ldx > K) on every decode kernel family (one-token, two-token, K-slice
and matrix-core kernels), and of the one-token FP8 kernels (activations staged
once per workgroup in LDS) at ragged shapes.  INT8 is compared bit-exactly,
the float kinds under the comparison rules of oracle/compare.py."""
import numpy as np
import pytest
import torch

from gpu_util import dev, host, host_bits, lib, need_gpu, padded
from oracle.compare import check_float
from skinny_gemm_qlin_amd.inputs import gen_fp8, gen_fp8_w8a8, gen_int8

pytestmark = pytest.mark.gpu

PADS = [64, 256]
FMTS = [(0, 0), (1, 1), (0, 1), (1, 0)]  # (x_fmt, w_fmt)


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _bf16_view(bits, pad):
    """bf16 device view [R, C] of a [R, C + pad] buffer (junk in the padding)."""
    v = padded(bits.view(np.int16), pad)
    return v.view(torch.bfloat16)


# M = 1, 2 (vector kernels), M >= 3 with K a multiple of 1024 (K-slice), and
# K not a multiple of 1024 (matrix-core kernels)
SHAPES = [(1, 300, 1024), (1, 4100, 5120), (2, 300, 1040), (2, 257, 2048),
          (3, 2000, 2048), (8, 5000, 4096), (16, 3000, 5120), (5, 700, 2064), (16, 129, 784)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_int8_padded_activations(ql, orc, M, N, K):
    d = gen_int8(M, N, K, seed=M * 31 + N)
    oxq, oxs = orc.act_quant_i8(d["x"])
    oacc, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"])
    w, ws = dev(d["w"]), dev(d["ws"])
    for pad in PADS:
        print(f"int8 padded activations M={M} N={N} K={K} pad={pad}", flush=True)
        xv = _bf16_view(d["x"], pad)
        assert xv.stride(0) == K + pad
        xq, xs = ql.qlin_act_quant_i8(xv)                       # padded bf16 rows in
        xqp = padded(oxq, pad)                                  # padded code rows in
        acc = ql.qlin_gemv_i8(xqp, dev(oxs), w, ws, out_kind=1)
        y = ql.qlin_gemv_i8(xqp, dev(oxs), w, ws)
        torch.cuda.synchronize()
        assert np.array_equal(host(xq), oxq) and np.array_equal(host(xs), oxs)
        assert np.array_equal(host(acc), oacc), "int32 sums differ"
        assert np.array_equal(host_bits(y), oy), "bf16 outputs differ"


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp8_padded_activations(ql, orc, M, N, K):
    d = gen_fp8(M, N, K, seed=M * 37 + N)
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    w, ws = dev(d["w"]), dev(d["ws"])
    for pad in PADS:
        print(f"fp8 padded activations M={M} N={N} K={K} pad={pad}", flush=True)
        y = ql.qlin_gemv_fp8(_bf16_view(d["x"], pad), w, ws)
        torch.cuda.synchronize()
        check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w8a8_padded_activations(ql, orc, M, N, K):
    d = gen_fp8_w8a8(M, N, K, w_fmt=0, seed=M * 41 + N)
    xq, xs = orc.act_quant_fp8(d["x"], 0, True)
    _, ye, S = orc.gemv_fp8_w8a8(xq, xs, 0, d["w"], d["ws"], 0)
    w, ws = dev(d["w"]), dev(d["ws"])
    for pad in PADS:
        print(f"w8a8 padded activations M={M} N={N} K={K} pad={pad}", flush=True)
        xqp = padded(xq, pad)
        y = ql.qlin_gemv_fp8_w8a8(xqp, dev(xs), w, ws, 0, 0)
        torch.cuda.synchronize()
        check_float(host_bits(y), ye, S, K)


# ----------------------------------------------------------------------------- one token, FP8 weights

# K from one chunk to past the LDS-staged kernel's 8192 (which then falls
# back to the register kernel); N from one row to several workgroups with a
# partial last one (8 rows per workgroup)
ONE_TOKEN = [(1, 16), (7, 48), (129, 272), (1001, 1040), (300, 2064), (17, 4112), (1001, 8192), (9, 8208),
             (17408, 5120)]


@pytest.mark.parametrize("N,K", ONE_TOKEN)
@pytest.mark.parametrize("per_tensor", [False, True])
def test_fp8_one_token_shapes(ql, orc, N, K, per_tensor):
    d = gen_fp8(1, N, K, seed=N + K, per_tensor=per_tensor)
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    y = ql.qlin_gemv_fp8(dev(d["x"].view(np.int16)).view(torch.bfloat16), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("N,K", ONE_TOKEN[:-1])
@pytest.mark.parametrize("x_fmt,w_fmt", FMTS)
def test_w8a8_one_token_shapes(ql, orc, N, K, x_fmt, w_fmt):
    d = gen_fp8_w8a8(1, N, K, w_fmt=w_fmt, seed=N * 3 + K)
    xq, xs = orc.act_quant_fp8(d["x"], x_fmt, True)
    _, ye, S = orc.gemv_fp8_w8a8(xq, xs, x_fmt, d["w"], d["ws"], w_fmt)
    y = ql.qlin_gemv_fp8_w8a8(dev(xq), dev(xs), dev(d["w"]), dev(d["ws"]), x_fmt, w_fmt)
    torch.cuda.synchronize()
    check_float(host_bits(y), ye, S, K)


def test_fp8_one_token_padded_weights_and_repeats(ql, orc):
    # a padded weight pitch reads the same values; 10 repeated calls are bit-identical
    d = gen_fp8(1, 1000, 5120, seed=77)
    x = dev(d["x"].view(np.int16)).view(torch.bfloat16)
    ref = ql.qlin_gemv_fp8(x, dev(d["w"]), dev(d["ws"]))
    yp = ql.qlin_gemv_fp8(x, padded(d["w"], 256), dev(d["ws"]))
    assert torch.equal(ref.view(torch.int16), yp.view(torch.int16))
    for _ in range(10):
        assert torch.equal(ql.qlin_gemv_fp8(x, dev(d["w"]), dev(d["ws"])).view(torch.int16), ref.view(torch.int16))
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(ref), ye, S, 5120)
