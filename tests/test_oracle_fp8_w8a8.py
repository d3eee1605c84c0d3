"""Pins of the oracle's FP8 W8A8 path: the E5M2 codec, the dynamic FP8
activation quantiser and the W8A8 GEMV.

References: torch's float8_e5m2 / float8_e4m3fn casts (decode tables and RNE
encodes), numpy fp32 division for the activation scales, exact rational
arithmetic on tiny shapes, numpy fp64 matmul over torch-decoded codes, and
composition with the separately pinned weight-only FP8 GEMV."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_fp8_w8a8

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
E5M2 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e5m2).to(torch.float64).numpy()
DT = {0: torch.float8_e4m3fn, 1: torch.float8_e5m2}
FMAX = {0: 448.0, 1: 57344.0}
TAB = {0: E4M3, 1: E5M2}


# ----------------------------------------------------------------------------- E5M2

def test_e5m2_decode_matches_torch_all_codes(orc):
    got = orc.e5m2_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(E5M2)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], E5M2[~nan])
    assert got[0x7C] == np.inf and got[0xFC] == -np.inf
    assert got[0x7B] == 57344.0 and got[0x01] == 2.0 ** -16 and got[0x04] == 2.0 ** -14 and got[0x3C] == 1.0


def test_e5m2_encode_matches_torch(orc):
    rng = np.random.default_rng(60)
    v = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-6, 4.5, 20000),
                        E5M2[np.isfinite(E5M2)]])
    # midpoints between neighbouring finite codes: ties go to the even code
    fin = np.sort(np.unique(np.abs(E5M2[np.isfinite(E5M2)])))
    mids = (fin[:-1] + fin[1:]) / 2
    v = np.concatenate([v, mids, -mids])
    v = v[np.abs(v) <= 57344.0]
    ref = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    got = orc.e5m2_encode(v)
    assert np.array_equal(got, ref)
    assert np.array_equal(orc.e5m2_decode(orc.e5m2_encode(E5M2[np.isfinite(E5M2)])), E5M2[np.isfinite(E5M2)])


def test_e5m2_encode_saturates(orc):
    got = orc.e5m2_encode(np.array([57344.0, 61439.0, 61440.0, 1e9, np.inf, -1e9, -np.inf]))
    assert list(got) == [0x7B, 0x7B, 0x7B, 0x7B, 0x7B, 0xFB, 0xFB]
    assert orc.e5m2_encode(np.array([np.nan]))[0] == 0x7F


# ----------------------------------------------------------------------------- activation quantiser

@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("per_token", [True, False])
def test_act_quant_fp8_scale_and_codes(orc, fmt, per_token):
    rng = np.random.default_rng(61 + fmt)
    x = bf16_bits((rng.standard_normal((5, 300)) * np.array([[1.0], [1e-3], [30.0], [0.5], [7.0]])).astype(np.float32))
    xq, xs = orc.act_quant_fp8(x, fmt, per_token)
    xf = bf16_values(x)
    amax = np.abs(xf).max(axis=1) if per_token else np.array([np.abs(xf).max()], np.float32)
    s_ref = (amax.astype(np.float32) / np.float32(FMAX[fmt])).astype(np.float32)
    assert np.array_equal(xs, s_ref)
    s_row = s_ref if per_token else np.repeat(s_ref, 5)
    # torch: one fp32 division, then its RNE cast to the format
    q_ref = (torch.from_numpy(xf) / torch.from_numpy(s_row)[:, None]).to(DT[fmt]).view(torch.uint8).numpy()
    assert np.array_equal(xq, q_ref)
    dec = TAB[fmt][xq]
    assert np.all(np.abs(dec) <= FMAX[fmt])
    rows = range(5) if per_token else [int(np.argmax(np.abs(xf).max(axis=1)))]
    for m in rows:
        k = int(np.argmax(np.abs(xf[m])))
        assert abs(dec[m, k]) == FMAX[fmt]


def test_act_quant_fp8_zero_row(orc):
    x = np.zeros((2, 64), np.uint16)
    x[1, 3] = bf16_bits(np.array([2.5], np.float32))[0]
    xq, xs = orc.act_quant_fp8(x, 0, True)
    assert xs[0] == 0.0 and np.all(xq[0] == 0)
    assert E4M3[xq[1, 3]] == 448.0 and np.sum(xq[1] != 0) == 1


# ----------------------------------------------------------------------------- W8A8 GEMV

@pytest.mark.parametrize("x_fmt,w_fmt", [(0, 0), (1, 1), (0, 1), (1, 0)])
def test_gemv_w8a8_exact_rational_tiny(orc, x_fmt, w_fmt):
    rng = np.random.default_rng(62)
    for (M, N, K) in [(1, 3, 16), (3, 4, 48)]:
        xq = rng.integers(0, 256, (M, K)).astype(np.uint8)
        w = rng.integers(0, 256, (N, K)).astype(np.uint8)
        xq[~np.isfinite(TAB[x_fmt][xq])] = 0x11
        w[~np.isfinite(TAB[w_fmt][w])] = 0x22
        xs = rng.uniform(0.01, 2.0, M).astype(np.float32)
        ws = rng.uniform(0.01, 2.0, N).astype(np.float32)
        y, ye, S = orc.gemv_fp8_w8a8(xq, xs, x_fmt, w, ws, w_fmt)
        for m in range(M):
            for n in range(N):
                sc = Fraction(float(xs[m])) * Fraction(float(ws[n]))
                terms = [Fraction(float(TAB[x_fmt][xq[m, k]])) * Fraction(float(TAB[w_fmt][w[n, k]])) for k in range(K)]
                ex = sc * sum(terms)
                sa = abs(sc) * sum(abs(t) for t in terms)
                assert abs(Fraction(ye[m, n]) - ex) <= sa * Fraction(1, 2 ** 44) + Fraction(1, 2 ** 300)
                assert y[m, n] == orc.f64_to_bf16(np.array([float(ex)]))[0]


def test_gemv_w8a8_matches_numpy_and_per_tensor(orc):
    d = gen_fp8_w8a8(4, 96, 512, w_fmt=0, seed=63)
    xq, xs = orc.act_quant_fp8(d["x"], 0, True)
    y, ye, S = orc.gemv_fp8_w8a8(xq, xs, 0, d["w"], d["ws"], 0)
    ref = (E4M3[xq] @ E4M3[d["w"]].T) * xs[:, None].astype(np.float64) * d["ws"][None, :].astype(np.float64)
    assert np.allclose(ye, ref, rtol=0, atol=1e-12 * S.max())
    # a per-tensor weight scale equals a per-channel one with all entries equal
    y1, ye1, _ = orc.gemv_fp8_w8a8(xq, xs, 0, d["w"], d["ws"][:1], 0)
    y2, ye2, _ = orc.gemv_fp8_w8a8(xq, xs, 0, d["w"], np.full(96, d["ws"][0], np.float32), 0)
    assert np.array_equal(y1, y2) and np.array_equal(ye1, ye2)


def test_gemv_w8a8_reduces_to_weight_only_fp8(orc):
    # E4M3 activation codes with unit scale are exactly representable in bf16:
    # the W8A8 GEMV must equal the pinned weight-only GEMV on those values
    d = gen_fp8_w8a8(3, 64, 256, w_fmt=0, seed=64)
    xq, _ = orc.act_quant_fp8(d["x"], 0, True)
    xb = bf16_bits(E4M3[xq].astype(np.float32))
    y, ye, S = orc.gemv_fp8_w8a8(xq, np.ones(3, np.float32), 0, d["w"], d["ws"], 0)
    yw, yew, Sw = orc.gemv_fp8(xb, d["w"], d["ws"])
    assert np.array_equal(y, yw)
    assert np.allclose(ye, yew, rtol=0, atol=1e-13 * Sw.max())


@pytest.mark.parametrize("fmt,amax,xv", [(0, 4.5299530029296875e-06, 2.0736479200422764e-10),
                                         (0, 3504693313536.0, 160432128.0),
                                         (1, 33792.0, 3.147125244140625e-05),
                                         (1, 80216064.0, 0.07470703125)])
def test_act_quant_fp8_divides_rather_than_multiplies(orc, fmt, amax, xv):
    # bf16 pairs found by exhaustive search: x / s and x * (1 / s) round to
    # neighbouring fp32 values on either side of an FP8 rounding boundary, so
    # the quantiser's code depends on using one correctly rounded division
    x = bf16_bits(np.array([[amax, xv, -xv]], np.float32))
    assert np.array_equal(bf16_values(x), np.array([[amax, xv, -xv]], np.float32))
    xq, xs = orc.act_quant_fp8(x, fmt, True)
    s = np.float32(np.float32(amax) / np.float32(FMAX[fmt]))
    assert xs[0] == s
    t_div = np.float32(np.float32(xv) / s)
    t_mul = np.float32(np.float32(xv) * np.float32(np.float32(1.0) / s))
    code = lambda t: int(torch.tensor([float(t)], dtype=torch.float32).to(DT[fmt]).view(torch.uint8)[0])
    assert code(t_div) != code(t_mul)
    assert xq[0, 1] == code(t_div) and xq[0, 2] == code(t_div) | 0x80
