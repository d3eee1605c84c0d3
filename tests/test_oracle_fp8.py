"""Pins of the oracle's FP8 paths: E4M3 weight-only GEMV and the 128x128
block-scaled GEMV with its UE8M0 activation quantiser.

References used: exact rational arithmetic on tiny inputs, numpy float64
matmul over torch-decoded E4M3 tables, torch's float8 cast for the activation
codes, closed forms (one-hot x, unit scales), and the scale-folding identity
of the block path (fold per K block == dequantise then GEMV)."""
from fractions import Fraction

import numpy as np
import torch

from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_fp8, gen_fp8_blk

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _frac_to_bf16(orc, v: Fraction):
    # float(Fraction) is correctly rounded to double; the oracle's f64->bf16 is pinned separately
    return orc.f64_to_bf16(np.array([float(v)]))[0]


# ----------------------------------------------------------------------------- weight-only

def test_fp8_exact_rational_tiny(orc):
    rng = np.random.default_rng(20)
    for (M, N, K) in [(1, 3, 16), (3, 5, 64), (2, 4, 48)]:
        w = rng.integers(0, 254, size=(N, K)).astype(np.uint8)
        w[(w & 0x7F) == 0x7F] = 0x7E
        x = bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
        ws = rng.uniform(1e-3, 1.0, N).astype(np.float32)
        y, ye, S = orc.gemv_fp8(x, w, ws)
        xf = bf16_values(x)
        for m in range(M):
            for n in range(N):
                ex = Fraction(float(ws[n])) * sum(Fraction(float(E4M3[w[n, k]])) * Fraction(float(xf[m, k])) for k in range(K))
                sa = abs(Fraction(float(ws[n]))) * sum(abs(Fraction(float(E4M3[w[n, k]])) * Fraction(float(xf[m, k]))) for k in range(K))
                assert abs(Fraction(ye[m, n]) - ex) <= sa * Fraction(1, 2**44) + Fraction(1, 2**200)
                assert abs(Fraction(S[m, n]) - sa) <= sa * Fraction(1, 2**44)
                assert y[m, n] == _frac_to_bf16(orc, ex)


def test_fp8_matches_numpy_dense(orc):
    d = gen_fp8(4, 96, 512, seed=21)
    y, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    ref = (bf16_values(d["x"]).astype(np.float64) @ E4M3[d["w"]].T) * d["ws"][None, :].astype(np.float64)
    assert np.all(np.abs(ye - ref) <= 1e-12 * S + 1e-300)


def test_fp8_one_hot_closed_form(orc):
    K, k = 64, 17
    w = np.arange(256, dtype=np.uint8)[:, None].repeat(K, axis=1)  # row n holds code n everywhere
    w = w[(np.arange(256) & 0x7F) != 0x7F]
    x = np.zeros((1, K), np.float32)
    x[0, k] = 1.0
    ws = np.full(w.shape[0], 0.25, np.float32)  # power of two: the product is exact
    y, _, _ = orc.gemv_fp8(bf16_bits(x), w, ws)
    ref = torch.from_numpy(E4M3[w[:, 0]] * 0.25).to(torch.float32).to(torch.bfloat16)
    ref = ref.view(torch.int16).numpy().view(np.uint16)
    # compare values: an IEEE sum of signed zeros is +0, so the -0 code's row reads +0
    assert np.array_equal(bf16_values(y[0]), bf16_values(ref))


def test_fp8_per_tensor_equals_per_channel(orc):
    d = gen_fp8(2, 40, 128, seed=22, per_tensor=True)
    y1, ye1, _ = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    y2, ye2, _ = orc.gemv_fp8(d["x"], d["w"], np.full(40, d["ws"][0], np.float32))
    assert np.array_equal(y1, y2) and np.array_equal(ye1, ye2)


# ----------------------------------------------------------------------------- block activation quant

def test_blk_act_quant_scale_rule_and_codes(orc):
    rng = np.random.default_rng(23)
    scales = np.float32([[1.0], [1e-4], [300.0], [1e-20], [2.0 ** 20]])
    x = bf16_bits(rng.standard_normal((5, 512), dtype=np.float32) * scales)
    xq, xs = orc.blk_act_quant(x)
    xf = bf16_values(x).astype(np.float64)
    for m in range(5):
        for kb in range(4):
            g = xf[m, kb * 128:(kb + 1) * 128]
            amax = np.abs(g).max()
            E = int(xs[m, kb])
            # E is the smallest exponent whose 448 * 2^(E-127) covers the group
            assert amax <= 448.0 * 2.0 ** (E - 127)
            assert E == 1 or amax > 448.0 * 2.0 ** (E - 128)
            # codes are torch's RNE float8 cast of x / 2^(E-127)
            v = (g / 2.0 ** (E - 127)).astype(np.float32)
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(xq[m, kb * 128:(kb + 1) * 128], ref)
            # dequant(quant(x)) = code * scale, within half an E4M3 step of x
            deq = E4M3[xq[m, kb * 128:(kb + 1) * 128]] * 2.0 ** (E - 127)
            step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6))) - 3), 2.0 ** -9)
            assert np.all(np.abs(deq - g) <= step / 2 * 2.0 ** (E - 127) * (1 + 1e-12))


def test_blk_act_quant_zero_group(orc):
    x = np.zeros((2, 256), np.uint16)
    x[1, 128:] = bf16_bits(np.full(128, 3.0, np.float32))
    xq, xs = orc.blk_act_quant(x)
    # 448 * 2^-8 = 1.75 < 3.0 <= 448 * 2^-7 = 3.5 -> p = -7, E = 120;
    # 3 * 2^7 = 384 = 1.5 * 2^8 -> code 0.1111.100 = 0x7C
    assert list(xs[0]) == [127, 127] and list(xs[1]) == [127, 120]
    assert not xq[0].any() and not xq[1, :128].any()
    assert np.all(xq[1, 128:] == 0x7C)


def test_blk_act_quant_exponent_clamp(orc):
    # groups too small for any exponent byte above 0: the exponent stays at
    # its lower clamp E = 1 (scale 2^-126) and the codes are x * 2^126;
    # bf16 subnormals included
    rng = np.random.default_rng(24)
    g = rng.standard_normal((3, 128)).astype(np.float32)
    g[0] *= np.float32(1e-38)
    g[1] *= np.float32(1e-40)
    g[2, :] = 0.0
    g[2, 5] = np.float32(2.0 ** -133)  # one subnormal value, the rest zero
    x = bf16_bits(g)
    xq, xs = orc.blk_act_quant(x)
    xf = bf16_values(x).astype(np.float64)
    for m in range(3):
        amax = np.abs(xf[m]).max()
        assert 0.0 < amax <= 448.0 * 2.0 ** -126
        assert xs[m, 0] == 1
        v = (xf[m] * 2.0 ** 126).astype(np.float32)
        ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(xq[m], ref)
    # just above the clamp the rule applies again: amax in (448 * 2^-126, 448 * 2^-125] gives E = 2
    x2 = bf16_bits(np.full((1, 128), 448.0 * 2.0 ** -125, np.float32))
    _, xs2 = orc.blk_act_quant(x2)
    assert xs2[0, 0] == 2


# ----------------------------------------------------------------------------- block GEMV

def test_blk_unit_scales_reduce_to_plain_gemv(orc):
    # x made of E4M3 values with a group max in (224, 448] quantises with E = 127
    # and codes that decode to x itself; unit weight scales -> plain fp8 GEMV
    rng = np.random.default_rng(24)
    M, N, K = 3, 130, 256
    fin = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    xc = fin[rng.integers(0, fin.size, (M, K))]
    xc[:, ::128] = 0x7E  # 448 in every group
    x = bf16_bits(E4M3[xc].astype(np.float32))
    w = fin[rng.integers(0, fin.size, (N, K))].astype(np.uint8)
    ws = np.full(((N + 127) // 128, K // 128), 127, np.uint8)
    xq, xs, y, ye, S = orc.fp8_blk(x, w, ws)
    assert np.all(xs == 127) and np.array_equal(xq, xc.astype(np.uint8))
    ref = E4M3[xc] @ E4M3[w].T
    assert np.all(np.abs(ye - ref) <= 1e-12 * S)


def test_blk_scale_fold_equals_dequant_then_gemv(orc):
    d = gen_fp8_blk(4, 300, 512, seed=25, scale_lo=100, scale_hi=140)
    # spread magnitudes per token and per 128-group so every (m, kb) gets its own exponent
    spread = np.float32([1.0, 37.0, 1e-3, 5e3])[:, None] * np.repeat(np.float32([1.0, 0.01, 90.0, 3.0]), 128)[None, :]
    d["x"] = bf16_bits(bf16_values(d["x"]) * spread)
    xq, xs, y, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert len(np.unique(xs)) >= 8
    N, K = d["w"].shape
    wsc = 2.0 ** (d["ws"].astype(np.float64) - 127)
    Wd = E4M3[d["w"]] * np.repeat(np.repeat(wsc, 128, axis=0)[:N], 128, axis=1)
    Xd = E4M3[xq] * np.repeat(2.0 ** (xs.astype(np.float64) - 127), 128, axis=1)
    ref = Xd @ Wd.T
    assert np.all(np.abs(ye - ref) <= 1e-12 * S)
    # and the quantised activations stay close to x
    assert np.all(np.abs(Xd - bf16_values(d["x"])) <= np.abs(bf16_values(d["x"])) * 2.0 ** -4 + 1e-30 + np.repeat(2.0 ** (xs.astype(np.float64) - 127 - 9), 128, axis=1))


def test_blk_exact_rational_tiny(orc):
    d = gen_fp8_blk(2, 3, 256, seed=26)
    xq, xs, y, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    for m in range(2):
        for n in range(3):
            ex = Fraction(0)
            for kb in range(2):
                part = sum(Fraction(float(E4M3[xq[m, k]])) * Fraction(float(E4M3[d["w"][n, k]])) for k in range(kb * 128, kb * 128 + 128))
                ex += part * Fraction(2) ** (int(xs[m, kb]) - 127) * Fraction(2) ** (int(d["ws"][n // 128, kb]) - 127)
            assert abs(Fraction(ye[m, n]) - ex) <= Fraction(S[m, n]) * Fraction(1, 2**44)
            assert y[m, n] == _frac_to_bf16(orc, ex)
