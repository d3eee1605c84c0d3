"""GPU parity of the FP8 W8A8 path (qlin_act_quant_fp8, qlin_gemv_fp8_w8a8)
against the CPU oracle: codes and scales bit-exact, GEMV outputs under the
float comparison rules of oracle/compare.py; every E4M3 / E5M2 code decoded
through the product path on both operands."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits, lib, need_gpu, padded
from oracle.compare import bf16_to_f64, check_float
from skinny_gemm_qlin_amd.inputs import bf16_bits, gen_fp8_w8a8

pytestmark = pytest.mark.gpu

FMTS = [(0, 0), (1, 1), (0, 1), (1, 0)]  # (x_fmt, w_fmt)
ONE = {0: 0x38, 1: 0x3C}  # code of 1.0


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _quant(ql, x_bits, fmt, per_token):
    xq, xs = ql.qlin_act_quant_fp8(dev_bf16(x_bits), fmt, per_token)
    torch.cuda.synchronize()
    return host(xq), host(xs)


def _gemv(ql, xq, xs, x_fmt, w, ws, w_fmt, w_dev=None):
    y = ql.qlin_gemv_fp8_w8a8(dev(xq), dev(xs), dev(w) if w_dev is None else w_dev, dev(ws), x_fmt, w_fmt)
    torch.cuda.synchronize()
    return host_bits(y)


def _finite_codes(fmt):
    if fmt == 0:
        return np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    return np.array([c for c in range(256) if (c & 0x7C) != 0x7C], np.uint8)


# ----------------------------------------------------------------------------- quantiser

@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("per_token", [True, False])
@pytest.mark.parametrize("M,K", [(1, 16), (1, 5120), (3, 272), (5, 2064), (16, 7168), (16, 16384), (2, 40000)])
def test_act_quant_fp8_bit_exact(ql, orc, fmt, per_token, M, K):
    rng = np.random.default_rng(M * 1000 + K + fmt)
    scale = 10.0 ** rng.uniform(-3, 3, (M, 1))
    x = bf16_bits((rng.standard_normal((M, K)) * scale).astype(np.float32))
    q_ref, s_ref = orc.act_quant_fp8(x, fmt, per_token)
    q, s = _quant(ql, x, fmt, per_token)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q, q_ref)


@pytest.mark.parametrize("fmt", [0, 1])
def test_act_quant_fp8_zero_and_tiny_rows(ql, orc, fmt):
    # an all-zero row (s = 0, codes 0), a row with -0.0, a row whose amax is a
    # bf16 subnormal (s is an fp32 subnormal, quotients saturate), a row of
    # one large value
    x = np.zeros((4, 64), np.float32)
    x[1, :] = -0.0
    x[1, 5] = 3.0
    x[2, :7] = np.array([1e-39, -2e-39, 5e-40, 0, 9e-41, -1e-39, 3e-39], np.float32)
    x[3, 63] = -3.0e38
    xb = bf16_bits(x)
    for per_token in (True, False):
        q_ref, s_ref = orc.act_quant_fp8(xb, fmt, per_token)
        q, s = _quant(ql, xb, fmt, per_token)
        assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
        assert np.array_equal(q, q_ref)
    q, s = _quant(ql, xb, fmt, True)
    assert s[0] == 0.0 and np.all(q[0] == 0)


@pytest.mark.parametrize("fmt,amax,xv", [(0, 4.5299530029296875e-06, 2.0736479200422764e-10),
                                         (0, 3504693313536.0, 160432128.0),
                                         (1, 33792.0, 3.147125244140625e-05),
                                         (1, 80216064.0, 0.07470703125)])
def test_act_quant_fp8_true_division(ql, orc, fmt, amax, xv):
    # inputs where x / s and x * (1 / s) give different codes (the oracle's pin)
    x = bf16_bits(np.array([[amax, xv, -xv] + [0.0] * 13], np.float32))
    q_ref, s_ref = orc.act_quant_fp8(x, fmt, True)
    q, s = _quant(ql, x, fmt, True)
    assert s[0] == s_ref[0] and np.array_equal(q, q_ref)


def test_act_quant_fp8_padded_pitch(ql, orc):
    rng = np.random.default_rng(7)
    x = bf16_bits(rng.standard_normal((3, 1024)).astype(np.float32))
    xp = padded(x.view(np.int16), 64).view(torch.bfloat16)
    xq, xs = ql.qlin_act_quant_fp8(xp, 0, True)
    torch.cuda.synchronize()
    q_ref, s_ref = orc.act_quant_fp8(x, 0, True)
    assert np.array_equal(host(xq), q_ref) and np.array_equal(host(xs), s_ref)


# ----------------------------------------------------------------------------- decode of every code

@pytest.mark.parametrize("w_fmt", [0, 1])
def test_weight_decode_every_code(ql, orc, w_fmt):
    # row n holds code n at column k; x = code of 1.0 at k; scales 1
    K, k = 64, 21
    codes = _finite_codes(w_fmt)
    w = np.zeros((codes.size, K), np.uint8)
    w[:, k] = codes
    xq = np.zeros((1, K), np.uint8)
    xq[0, k] = ONE[0]
    y = bf16_to_f64(_gemv(ql, xq, np.ones(1, np.float32), 0, w, np.ones(codes.size, np.float32), w_fmt))[0]
    ref = orc.e5m2_decode(codes) if w_fmt == 1 else orc.e4m3_decode(codes)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("x_fmt", [0, 1])
@pytest.mark.parametrize("M", [1, 2, 16])
def test_activation_decode_every_code(ql, orc, x_fmt, M):
    # token m holds code c at column k; one weight row with 1.0 at k
    K, k = 48, 33
    codes = _finite_codes(x_fmt)
    w = np.zeros((1, K), np.uint8)
    w[0, k] = ONE[0]
    ref_all = orc.e5m2_decode(codes) if x_fmt == 1 else orc.e4m3_decode(codes)
    for c0 in range(0, codes.size, M):
        cs = codes[c0:c0 + M]
        xq = np.zeros((M, K), np.uint8)
        xq[:cs.size, k] = cs
        y = bf16_to_f64(_gemv(ql, xq, np.ones(M, np.float32), x_fmt, w, np.ones(1, np.float32), 0))[:, 0]
        assert np.array_equal(y[:cs.size], ref_all[c0:c0 + M])


# ----------------------------------------------------------------------------- GEMV parity

def _case(orc, M, N, K, x_fmt, w_fmt, seed, per_channel=True, per_token=True):
    d = gen_fp8_w8a8(M, N, K, w_fmt=w_fmt, per_channel=per_channel, seed=seed)
    xq, xs = orc.act_quant_fp8(d["x"], x_fmt, per_token)
    y, ye, S = orc.gemv_fp8_w8a8(xq, xs, x_fmt, d["w"], d["ws"], w_fmt)
    return d, xq, xs, ye, S


@pytest.mark.parametrize("x_fmt,w_fmt", FMTS)
@pytest.mark.parametrize("M", list(range(1, 17)))
def test_w8a8_small_all_M(ql, orc, x_fmt, w_fmt, M):
    d, xq, xs, ye, S = _case(orc, M, 512, 1024, x_fmt, w_fmt, seed=M)
    check_float(_gemv(ql, xq, xs, x_fmt, d["w"], d["ws"], w_fmt), ye, S, 1024)


@pytest.mark.parametrize("M", [1, 2, 5])
@pytest.mark.parametrize("per_channel,per_token", [(False, True), (True, False), (False, False)])
def test_w8a8_per_tensor_scales(ql, orc, M, per_channel, per_token):
    d, xq, xs, ye, S = _case(orc, M, 384, 2048, 0, 0, seed=40 + M, per_channel=per_channel, per_token=per_token)
    assert xs.size == (M if per_token else 1) and d["ws"].size == (384 if per_channel else 1)
    check_float(_gemv(ql, xq, xs, 0, d["w"], d["ws"], 0), ye, S, 2048)


@pytest.mark.parametrize("M,N,K", [(1, 1, 16), (2, 3, 48), (3, 37, 272), (4, 129, 1040), (1, 77, 16400),
                                   (8, 255, 4112), (11, 17, 2064), (16, 1001, 784),
                                   (3, 9000, 2048), (16, 9001, 2320),
                                   # two and three tokens above K = 8192: the per-tile matrix-core kernel
                                   (2, 1001, 8208), (3, 300, 14336), (2, 64, 20480), (3, 5, 9216)])
@pytest.mark.parametrize("x_fmt,w_fmt", [(0, 0), (1, 1)])
def test_w8a8_ragged(ql, orc, M, N, K, x_fmt, w_fmt):
    d, xq, xs, ye, S = _case(orc, M, N, K, x_fmt, w_fmt, seed=N + K)
    check_float(_gemv(ql, xq, xs, x_fmt, d["w"], d["ws"], w_fmt), ye, S, K)


@pytest.mark.parametrize("M", [1, 2, 4, 8, 16])
def test_w8a8_decode_full(ql, orc, M):
    # 17408 x 5120, E4M3 both operands, the quantiser and the GEMV on the GPU
    d = gen_fp8_w8a8(M, 17408, 5120, w_fmt=0, seed=0)
    xq_ref, xs_ref = orc.act_quant_fp8(d["x"], 0, True)
    xq, xs = ql.qlin_act_quant_fp8(dev_bf16(d["x"]), 0, True)
    y = ql.qlin_gemv_fp8_w8a8(xq, xs, dev(d["w"]), dev(d["ws"]), 0, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host(xq), xq_ref) and np.array_equal(host(xs), xs_ref)
    _, ye, S = orc.gemv_fp8_w8a8(xq_ref, xs_ref, 0, d["w"], d["ws"], 0)
    stats = check_float(host_bits(y), ye, S, 5120)
    assert stats["ref_bits_equal"] > 0.99


def test_w8a8_padded_row_stride(ql, orc):
    d, xq, xs, ye, S = _case(orc, 3, 200, 1024, 0, 0, seed=5)
    wp = padded(d["w"], 256)
    assert _gemv(ql, xq, xs, 0, d["w"], d["ws"], 0, w_dev=wp).tolist() == \
        _gemv(ql, xq, xs, 0, d["w"], d["ws"], 0).tolist()


def test_w8a8_deterministic(ql):
    d = gen_fp8_w8a8(8, 2048, 5120, seed=6)
    x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
    xq, xs = ql.qlin_act_quant_fp8(x, 0, True)
    ref = ql.qlin_gemv_fp8_w8a8(xq, xs, w, ws)
    for _ in range(20):
        assert torch.equal(ql.qlin_gemv_fp8_w8a8(xq, xs, w, ws).view(torch.int16), ref.view(torch.int16))


def test_w8a8_accepts_float8_tensors(ql, orc):
    d, xq, xs, ye, S = _case(orc, 2, 64, 256, 1, 0, seed=9)
    y = ql.qlin_gemv_fp8_w8a8(dev(xq).view(torch.float8_e5m2), dev(xs), dev(d["w"]).view(torch.float8_e4m3fn),
                              dev(d["ws"]), 1, 0)
    torch.cuda.synchronize()
    check_float(host_bits(y), ye, S, 256)
