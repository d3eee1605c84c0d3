"""Pins of the oracle's block-scaled FP8 path at block shapes other than
128 x 128 (block_k a multiple of 32; block_n down to 1, the MX-style per-row
scale): the activation exponent rule per block_k group, the scale-fold
identity against numpy dequantise-then-matmul, exact rational sums."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_fp8_blk

E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
SHAPES = [(1, 32), (1, 64), (16, 32), (32, 128), (64, 64), (7, 32), (128, 256)]


def _frac_to_bf16(orc, fr):
    return orc.f64_to_bf16(np.array([float(fr)]))[0]


@pytest.mark.parametrize("bk", [32, 64, 256])
def test_act_quant_exponent_rule_per_group(orc, bk):
    rng = np.random.default_rng(bk)
    K = 512
    spread = np.repeat(10.0 ** rng.uniform(-6, 6, K // bk), bk).astype(np.float32)
    x = bf16_bits(rng.standard_normal((3, K), dtype=np.float32) * spread)
    xq, xs = orc.blk_act_quant(x, bk)
    assert xs.shape == (3, K // bk)
    xf = bf16_values(x).astype(np.float64)
    for m in range(3):
        for kb in range(K // bk):
            g = xf[m, kb * bk:(kb + 1) * bk]
            amax, E = np.abs(g).max(), int(xs[m, kb])
            assert amax <= 448.0 * 2.0 ** (E - 127)
            assert E == 1 or amax > 448.0 * 2.0 ** (E - 128)
            v = (g / 2.0 ** (E - 127)).astype(np.float32)
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(xq[m, kb * bk:(kb + 1) * bk], ref)


@pytest.mark.parametrize("bn,bk", SHAPES)
def test_scale_fold_equals_dequant_then_matmul(orc, bn, bk):
    M, N, K = 3, 150, 512
    d = gen_fp8_blk(M, N, K, seed=bn * 1000 + bk, scale_lo=100, scale_hi=140, block_n=bn, block_k=bk)
    xq, xs, y, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"], bn, bk)
    wsc = 2.0 ** (d["ws"].astype(np.float64) - 127)
    Wd = E4M3[d["w"]] * np.repeat(np.repeat(wsc, bn, axis=0)[:N], bk, axis=1)
    Xd = E4M3[xq] * np.repeat(2.0 ** (xs.astype(np.float64) - 127), bk, axis=1)
    ref = Xd @ Wd.T
    assert np.all(np.abs(ye - ref) <= 1e-12 * S)
    assert d["ws"].shape == ((N + bn - 1) // bn, K // bk) and xs.shape == (M, K // bk)


@pytest.mark.parametrize("bn,bk", [(1, 32), (3, 64)])
def test_exact_rational_tiny(orc, bn, bk):
    M, N, K = 2, 5, 128
    d = gen_fp8_blk(M, N, K, seed=7 + bn, scale_lo=90, scale_hi=160, block_n=bn, block_k=bk)
    xq, xs, y, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"], bn, bk)
    for m in range(M):
        for n in range(N):
            ex = Fraction(0)
            for kb in range(K // bk):
                part = sum(Fraction(float(E4M3[xq[m, k]])) * Fraction(float(E4M3[d["w"][n, k]]))
                           for k in range(kb * bk, (kb + 1) * bk))
                ex += part * Fraction(2) ** (int(xs[m, kb]) - 127) * Fraction(2) ** (int(d["ws"][n // bn, kb]) - 127)
            assert abs(Fraction(ye[m, n]) - ex) <= Fraction(S[m, n]) * Fraction(1, 2 ** 44)
            assert y[m, n] == _frac_to_bf16(orc, ex)


def test_per_row_scales_are_independent(orc):
    # block_n = 1: changing one row's scale byte moves only that row, by the
    # exact power of two, and only through its own K block
    M, N, K = 2, 4, 96
    d = gen_fp8_blk(M, N, K, seed=3, block_n=1, block_k=32)
    _, xs, _, ye, _ = orc.fp8_blk(d["x"], d["w"], d["ws"], 1, 32)
    ws2 = d["ws"].copy()
    ws2[2, 1] += 3
    xq, xs2, _, ye2, _ = orc.fp8_blk(d["x"], d["w"], ws2, 1, 32)
    assert np.array_equal(xs, xs2)
    assert np.array_equal(ye[:, [0, 1, 3]], ye2[:, [0, 1, 3]])
    blk = np.array([sum(E4M3[xq[m, k]] * E4M3[d["w"][2, k]] for k in range(32, 64)) for m in range(M)])
    sc = 2.0 ** (xs[:, 1].astype(np.float64) - 127) * 2.0 ** (d["ws"][2, 1].astype(np.float64) - 127)
    assert np.allclose(ye2[:, 2] - ye[:, 2], blk * sc * 7, rtol=1e-12, atol=1e-300)
