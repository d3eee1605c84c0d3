"""Pins of the oracle's W8A8 INT8 path (activation quantisation, int32 GEMV,
epilogue).  Checked against invariants of a symmetric round-half-even
quantiser, constructed ties, numpy's int64 matmul and torch's fp32/bf16
arithmetic (library routines the oracle does not use)."""
from fractions import Fraction

import numpy as np
import pytest
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


# ----------------------------------------------------------------------------- division and epilogue order

# bf16 pairs (amax, x) found by exhaustive search over x for random amax:
# with s = fp32(amax / 127), the fp32 quotient x / s and the product
# x * fp32(1 / s) land on opposite sides of (or on) a rounding boundary, so
# the code depends on the quantiser using one correctly rounded division
# (stated scale absmax/127, round half to even).
DIV_CASES = [(1.6875, 0.84375, 64), (0.296875, 0.1484375, 64), (0.00162506103515625, 0.000812530517578125, 64),
             (208.0, 104.0, 63), (298.0, 149.0, 63), (0.0003414154052734375, 0.00017070770263671875, 63)]


def _torch_codes(xf32):
    """Reference quantiser from torch fp32 primitives: s = amax / 127 (one
    IEEE division), q = round_half_even(x / s) clamped to +-127."""
    x = torch.from_numpy(xf32)
    amax = x.abs().amax(dim=1, keepdim=True)
    s = amax / 127.0
    q = torch.where(amax > 0, torch.round(x / s), torch.zeros_like(x)).clamp(-127, 127)
    return q.to(torch.int8).numpy(), s[:, 0].numpy()


@pytest.mark.parametrize("amax,xv,code", DIV_CASES)
def test_act_quant_i8_divides_rather_than_multiplies(orc, amax, xv, code):
    x = _row([amax, xv, -xv])
    assert np.array_equal(bf16_values(x)[0], np.float32([amax, xv, -xv]))
    xq, xs = orc.act_quant_i8(x)
    s = np.float32(np.float32(amax) / np.float32(127))
    assert xs[0] == s
    t_div = np.float32(np.float32(xv) / s)
    t_mul = np.float32(np.float32(xv) * (np.float32(1) / s))
    assert np.rint(t_div) != np.rint(t_mul)
    assert int(np.rint(t_div)) == code
    assert list(xq[0]) == [127, code, -code]


def test_act_quant_i8_equals_torch_division_and_round(orc):
    # 100,000 random rows with magnitudes spread over many binades, plus the
    # rows of the 17408 x 5120 decode workload (16 tokens of 5120 values)
    rng = np.random.default_rng(17)
    R, K = 100_000, 16
    mag = np.float32(2.0) ** rng.integers(-40, 40, size=(R, 1)).astype(np.float32)
    x = bf16_bits(rng.standard_normal((R, K), dtype=np.float32) * mag)
    xq, xs = orc.act_quant_i8(x)
    q_ref, s_ref = _torch_codes(bf16_values(x))
    assert np.array_equal(xs.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(xq, q_ref)
    d = gen_int8(16, 8, 5120, seed=0)
    xq, xs = orc.act_quant_i8(d["x"])
    q_ref, s_ref = _torch_codes(bf16_values(d["x"]))
    assert np.array_equal(xs.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(xq, q_ref)


# Int8 dot products (4 terms) with fp32 scales found by a random search over
# 2e6 triples: bf16((acc*xs)*ws) differs from bf16((acc*ws)*xs) ("swap"),
# from bf16(acc*(xs*ws)) ("combined scale") or from the once-rounded exact
# product ("fp64") on some of them.  The epilogue order is the page's:
# (acc * x_s) * w_s in fp32, then the cast to bf16.
EPI_CASES = [
    ([93, -55, 26, -114], [4, -3, -1, -24], 0.016517382115125656, 0.001961976522579789),
    ([125, 126, 92, 38], [-119, -98, 110, 76], 0.037236087024211884, 0.002826492767781019),
    ([23, -127, 90, -121], [51, 68, -110, 72], 0.024325739592313766, 0.005899771116673946),
    ([33, -98, 109, -89], [59, 117, -68, -87], 0.03755415230989456, 0.0015679452335461974),
    ([-13, 107, -58, -83], [37, 8, -44, 9], 0.030231665819883347, 0.005378833040595055),
    ([46, -107, -48, -112], [-123, 114, -125, -88], 0.03696686774492264, 0.005032483953982592),
    ([99, -92, 111, -101], [-55, 82, 6, -49], 0.017969688400626183, 0.0024983659386634827),
    ([-118, 45, -1, 90], [-96, 24, 98, -45], 0.020163405686616898, 0.005523406434804201),
    ([-24, 68, -61, -99], [42, -93, 110, -56], 0.03669118881225586, 0.0062264129519462585),
]


def epilogue_case_arrays():
    """(xq [C,4] int8, w [C,4] int8, xs [C] f32, ws [C] f32): case i is token i
    against weight row i."""
    xq = np.array([c[0] for c in EPI_CASES], np.int8)
    w = np.array([c[1] for c in EPI_CASES], np.int8)
    xs = np.array([c[2] for c in EPI_CASES], np.float32)
    ws = np.array([c[3] for c in EPI_CASES], np.float32)
    return xq, w, xs, ws


def _bf16_bits_t(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_gemv_i8_epilogue_order_constructed(orc):
    xq, w, xs, ws = epilogue_case_arrays()
    acc, y = orc.gemv_i8(xq, xs, w, ws)
    acc_ref = xq.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(acc.astype(np.int64), acc_ref)
    a = torch.from_numpy(acc_ref).to(torch.float32)
    txs, tws = torch.from_numpy(xs), torch.from_numpy(ws)
    ref = _bf16_bits_t((a * txs[:, None]) * tws[None, :])
    assert np.array_equal(y, ref)
    # each alternative order is wrong on at least one diagonal case
    diag = np.arange(len(EPI_CASES))
    swap = _bf16_bits_t((a * tws[None, :]) * txs[:, None])
    comb = _bf16_bits_t(a * (txs[:, None] * tws[None, :]))
    f64 = _bf16_bits_t(torch.from_numpy(acc_ref).double() * txs.double()[:, None] * tws.double()[None, :])
    for alt in (swap, comb, f64):
        assert np.any(alt[diag, diag] != ref[diag, diag])
