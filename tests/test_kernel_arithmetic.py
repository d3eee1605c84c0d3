"""Arithmetic identities the HIP kernels rely on, checked exhaustively on the
CPU with numpy (no GPU, no oracle): they justify replacing an operation of
the method by a cheaper one that gives the same bits."""
import numpy as np


def test_division_by_fp64_reciprocal_equals_fp32_division():
    # The INT8 quantisers form x / s as fl32(fl64(x) * fl64(1 / s)).  For every
    # positive finite bf16 x and a spread of fp32 scales
    # (amax / 127 for bf16 amax, and raw fp32 bit patterns from subnormal to
    # huge) this must equal the IEEE fp32 quotient bit for bit.
    rng = np.random.default_rng(0)
    xb = (np.arange(1, 0x7F80, dtype=np.uint32) << 16).view(np.float32)
    xd = xb.astype(np.float64)
    amax = (rng.integers(1, 0x7F80, 600).astype(np.uint32) << 16).view(np.float32)
    scales = np.concatenate([(amax / np.float32(127)).astype(np.float32),
                             rng.integers(1, 0x7F800000, 600).astype(np.uint32).view(np.float32)])
    with np.errstate(over="ignore"):
        for s in scales:
            s = np.float32(s)
            ref = xb / s
            alt = (xd * (np.float64(1.0) / np.float64(s))).astype(np.float32)
            assert np.array_equal(ref.view(np.uint32), alt.view(np.uint32)), float(s)


def test_fp32_reciprocal_is_not_enough():
    # the same identity with an fp32 reciprocal and product fails (the
    # mutation the oracle's pins reject), so the check above is not vacuous;
    # random fp32 x pass the fp64 form as well (a quotient of two floats is
    # never an exact rounding midpoint)
    rng = np.random.default_rng(1)
    x = rng.standard_normal(200_000).astype(np.float32)
    for s in (np.float32(0.0123456789), np.float32(3.0), np.float32(1.6875 / 127)):
        ref = x / s
        alt64 = (x.astype(np.float64) * (1.0 / np.float64(s))).astype(np.float32)
        alt32 = x * (np.float32(1.0) / s)
        assert np.array_equal(ref, alt64)
        assert np.any(ref != alt32)
