"""Comparison rules of the parity checks (HIP path vs CPU oracle).

Test infrastructure, like the rest of this package.

Integer, code and index outputs: bit-exact.

Float outputs y (bf16) are compared with the oracle's fp64 value y_exact and
S = sum_k |w_k x_k| (times the |scales|, and |g| for the MoE), element by
element, with BOTH rules:

  (i)  |y - y_exact| <= 1e-3 * S + 1e-6 + ulp(y_exact) / 2  (the stated tolerance on
       the fp32-accumulated value, plus the half-ulp rounding of the bf16 output:
       when |y| is close to S -- heavy-tailed E4M3 codes -- the correctly rounded
       bf16 value alone can sit more than 1e-3 * S from y_exact)
  (ii) bf16(y_exact - eps) <= y <= bf16(y_exact + eps)       (bf16 rounding of the
       oracle, allowing for the kernel's fp32 accumulation), with
       eps = (K/8 + 32) * 2^-24 * S, a bound on the fp32 rounding error of the
       kernels' summation order (at most K/16 sequential fp32 additions per
       lane, a 4-level lane tree, the scale multiplications; factor 2 margin).

When eps is below half a bf16 ulp, (ii) means y is bf16(y_exact) or one of
its two neighbours, i.e. "within 1 ulp of the oracle's rounding".  Rule (ii)
is much tighter than (i): a dropped K-term, a wrong scale or a wrong index
fails it.
"""
import numpy as np


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_ulp(v):
    """Spacing of bf16 values at |v| (8 significant bits; 2^-133 below 2^-126)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, -126.0), -126.0)
    return np.exp2(e - 7)


def f64_to_bf16_val(v):
    """fp64 -> bf16 value with ONE round-to-nearest-even (the oracle's routine;
    going through float32 first would round twice)."""
    from . import f64_to_bf16
    return bf16_to_f64(f64_to_bf16(v))


def check_float(y_bits, y_exact, S, K, what="y"):
    y = bf16_to_f64(y_bits)
    y_exact = np.asarray(y_exact, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    assert y.shape == y_exact.shape == S.shape, (y.shape, y_exact.shape, S.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite outputs"
    err = np.abs(y - y_exact)
    tol = 1e-3 * S + 1e-6 + bf16_ulp(y_exact) / 2
    bad = err > tol
    assert not bad.any(), (f"{what}: rule (i) fails at {np.argwhere(bad)[:5].tolist()}; "
                           f"max err/tol {np.max(err / tol):.3g}")
    eps = (K / 8 + 32) * 2.0 ** -24 * S
    lo = f64_to_bf16_val(y_exact - eps)
    hi = f64_to_bf16_val(y_exact + eps)
    bad = (y < lo) | (y > hi)
    assert not bad.any(), (f"{what}: rule (ii) fails at {np.argwhere(bad)[:5].tolist()}: "
                           f"y={y[bad][:5]} ref={y_exact[bad][:5]}")
    return {"max_err_over_S": float(np.max(err / np.maximum(S, 1e-300))),
            "ref_bits_equal": float(np.mean(f64_to_bf16_val(y_exact) == y))}
