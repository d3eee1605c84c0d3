"""The float comparison rules must accept the oracle's own correctly rounded
bf16 output and reject outputs with a plausible kernel mistake."""
import numpy as np

import oracle
from oracle.compare import bf16_to_f64, bf16_ulp, check_float
import pytest

from skinny_gemm_qlin_amd.inputs import gen_fp8, gen_fp8_blk, gen_moe


def test_ulp():
    assert bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([1.99]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([-3.0]))[0] == 2.0 ** -6
    assert bf16_ulp(np.array([0.0]))[0] == 2.0 ** -133
    assert bf16_ulp(np.array([1e-45]))[0] == 2.0 ** -133


def test_rules_accept_oracle_rounding():
    # heavy-tailed E4M3 codes put |y| close to S: the rounded output must still pass
    d = gen_fp8_blk(4, 256, 1024, seed=0)
    xq, xs, y, ye, S = oracle.fp8_blk(d["x"], d["w"], d["ws"])
    check_float(y, ye, S, 1024)
    d = gen_fp8(3, 300, 1024, seed=1)
    y, ye, S = oracle.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(y, ye, S, 1024)
    d = gen_moe(4, 8, 64, 512, 2, seed=2)
    y, ye, S = oracle.moe_mxfp4(d["x"], d["w"], d["s"], d["ids"], d["gw"])
    check_float(y, ye, S, 512)


def test_rules_reject_dropped_term():
    d = gen_fp8(2, 200, 1024, seed=3)
    y, ye, S = oracle.gemv_fp8(d["x"], d["w"], d["ws"])
    w2 = d["w"].copy()
    w2[:, 500] = 0  # drop one K term in every row
    y2, _, _ = oracle.gemv_fp8(d["x"], w2, d["ws"])
    with pytest.raises(AssertionError):
        check_float(y2, ye, S, 1024)


def test_rules_reject_wrong_block_scale():
    d = gen_fp8_blk(2, 256, 1024, seed=4)
    xq, xs, y, ye, S = oracle.fp8_blk(d["x"], d["w"], d["ws"])
    ws2 = d["ws"].copy()
    ws2[1, 3] += 1  # one block of one row-block off by a factor 2
    y2, _, _ = oracle.gemv_fp8_blk(xq, xs, d["w"], ws2)
    with pytest.raises(AssertionError):
        check_float(y2, ye, S, 1024)
