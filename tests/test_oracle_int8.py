"""Pins of the oracle's W8A8 INT8 path (activation quantisation, int32 GEMV,
epilogue).  Checked against invariants of a symmetric round-half-even
quantiser, constructed ties, numpy's int64 matmul and torch's fp32/bf16
arithmetic (library routines the oracle does not use)."""
from fractions import Fraction

import numpy as np
import torch

from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_int8


def _row(vals):
    return bf16_bits(np.array(vals, dtype=np.float32))[None, :]


# ----------------------------------------------------------------------------- activation quant

def test_act_quant_invariants(orc):
    rng = np.random.default_rng(10)
    x = bf16_bits(rng.standard_normal((6, 333), dtype=np.float32) * np.float32([[1], [1e-3], [50], [1], [7], [1e-30]]))
    xq, xs = orc.act_quant_i8(x)
    xf = bf16_values(x)
    for m in range(x.shape[0]):
        amax = np.abs(xf[m]).max()
        s = xs[m]
        # s is the correctly rounded fp32 quotient amax / 127
        err = abs(Fraction(float(s)) - Fraction(float(amax)) / 127)
        assert err <= Fraction(float(np.spacing(s))) / 2
        q = xq[m].astype(np.int64)
        assert np.all(np.abs(q) <= 127)
        assert np.all((q == 0) | (np.sign(q) == np.sign(xf[m])))
        i = int(np.argmax(np.abs(xf[m])))
        assert abs(q[i]) == 127
        # q is within half a step of x/s (exact arithmetic, plus the fp32 rounding of x/s)
        for k in range(0, x.shape[1], 7):
            t = Fraction(float(xf[m, k])) / Fraction(float(s))
            assert abs(Fraction(int(q[k])) - t) <= Fraction(1, 2) + abs(t) * Fraction(1, 2**23)
        # monotone: larger x never gets a smaller code
        order = np.argsort(xf[m], kind="stable")
        assert np.all(np.diff(q[order]) >= 0)


def test_act_quant_ties_to_even():
    import oracle
    # amax = 127 makes s exactly 1, so x/s = x and the codes are rne(x)
    x = _row([127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 3.25, -3.75])
    xq, xs = oracle.act_quant_i8(x)
    assert xs[0] == 1.0
    assert list(xq[0]) == [127, 0, 2, 2, 0, -2, -2, 126, 3, -4]


def test_act_quant_zero_row_and_row_independence(orc):
    x = np.zeros((1, 64), dtype=np.uint16)
    xq, xs = orc.act_quant_i8(x)
    assert xs[0] == 0.0 and not xq.any()
    rng = np.random.default_rng(11)
    x = bf16_bits(rng.standard_normal((4, 96), dtype=np.float32))
    xq, xs = orc.act_quant_i8(x)
    for m in range(4):
        q1, s1 = orc.act_quant_i8(x[m:m + 1])
        assert np.array_equal(q1[0], xq[m]) and s1[0] == xs[m]


# ----------------------------------------------------------------------------- GEMV + epilogue

def test_gemv_i8_acc_matches_numpy(orc):
    rng = np.random.default_rng(12)
    for (M, N, K) in [(1, 7, 16), (3, 33, 80), (16, 5, 1024)]:
        xq = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
        w = rng.integers(-128, 128, size=(N, K), dtype=np.int8)
        acc, _ = orc.gemv_i8(xq, np.ones(M, np.float32), w, np.ones(N, np.float32))
        ref = xq.astype(np.int64) @ w.astype(np.int64).T
        assert np.array_equal(acc.astype(np.int64), ref)


def test_gemv_i8_epilogue_matches_torch(orc):
    d = gen_int8(4, 64, 256, seed=13)
    xq, xs = orc.act_quant_i8(d["x"])
    acc, y = orc.gemv_i8(xq, xs, d["w"], d["ws"])
    t = torch.from_numpy(acc.astype(np.int64)).to(torch.float32)
    t = t * torch.from_numpy(xs)[:, None]
    t = t * torch.from_numpy(d["ws"])[None, :]
    ref = t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


def test_gemv_i8_large_acc_rounds_once(orc):
    # acc = 127*127*K exceeds 2^24, so int->fp32 conversion rounds (to nearest even)
    K = 2048
    xq = np.full((1, K), 127, dtype=np.int8)
    w = np.full((3, K), 127, dtype=np.int8)
    w[1] = -127
    w[2, ::2] = -127
    acc, y = orc.gemv_i8(xq, np.array([1.0], np.float32), w, np.array([1.0], np.float32))
    assert list(acc[0]) == [127 * 127 * K, -127 * 127 * K, 0]
    ref = torch.tensor([127 * 127 * K, -127 * 127 * K, 0], dtype=torch.int64).to(torch.float32)
    ref = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y[0], ref)


def test_gemv_i8_broadcast_scales(orc):
    rng = np.random.default_rng(14)
    xq = rng.integers(-127, 128, size=(3, 48), dtype=np.int8)
    w = rng.integers(-127, 128, size=(9, 48), dtype=np.int8)
    a1, y1 = orc.gemv_i8(xq, np.array([0.02], np.float32), w, np.array([0.003], np.float32))
    a2, y2 = orc.gemv_i8(xq, np.full(3, 0.02, np.float32), w, np.full(9, 0.003, np.float32))
    assert np.array_equal(a1, a2) and np.array_equal(y1, y2)


def test_gemv_i8_bias_after_cast(orc):
    rng = np.random.default_rng(15)
    xq = rng.integers(-127, 128, size=(2, 64), dtype=np.int8)
    w = rng.integers(-127, 128, size=(11, 64), dtype=np.int8)
    xs = np.array([0.011, 0.017], np.float32)
    ws = rng.uniform(1e-3, 1e-2, 11).astype(np.float32)
    bias = bf16_bits(rng.standard_normal(11, dtype=np.float32))
    _, y0 = orc.gemv_i8(xq, xs, w, ws)
    _, yb = orc.gemv_i8(xq, xs, w, ws, bias=bias)
    tb = torch.from_numpy(y0.view(np.int16)).view(torch.bfloat16)
    bb = torch.from_numpy(bias.view(np.int16)).view(torch.bfloat16)
    ref = (tb + bb[None, :]).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb, ref)


def test_gemv_i8_one_hot_closed_form(orc):
    # x one-hot at column k -> y[n] = bf16((q_k * w[n,k] * s) * ws[n]) with q_k = 127
    K, N, k = 128, 40, 77
    x = np.zeros((1, K), dtype=np.float32)
    x[0, k] = 2.5
    xq, xs = orc.act_quant_i8(bf16_bits(x))
    assert xq[0, k] == 127 and np.count_nonzero(xq) == 1
    rng = np.random.default_rng(16)
    w = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    ws = rng.uniform(1e-3, 1e-2, N).astype(np.float32)
    acc, y = orc.gemv_i8(xq, xs, w, ws)
    assert np.array_equal(acc[0], 127 * w[:, k].astype(np.int32))
    t = (torch.from_numpy((127 * w[:, k].astype(np.int64))).float() * float(xs[0])) * torch.from_numpy(ws)
    assert np.array_equal(y[0], t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
