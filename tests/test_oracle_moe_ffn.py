"""Pins of the oracle's routed MXFP4 expert FFN (router -> top-k -> softmax ->
gate/up -> clamped SwiGLU -> down -> weighted sum).

References, none of them a re-typing of the oracle's own loops:
  * torch.nn.functional.silu and closed forms for the clamped SwiGLU
    ([DSV4] sections 6.6 and 9.4: gate clamped above at the limit, up clamped
    to [-limit, limit], alpha 1.0, limit 10.0);
  * numpy matmul for the router logits, numpy's stable argsort for the top-k
    order (ties to the lower expert id), scipy's softmax for the weights;
  * composition with the separately pinned MXFP4 expert GEMV (oracle
    moe_mxfp4): gate/up rows through it give the SwiGLU inputs, the bf16
    activation through the down experts gives the output;
  * degenerate cases (alpha 0 or limit 0 give zero outputs) and the rule that
    an out-of-range expert id contributes nothing."""
import numpy as np
import pytest
import scipy.special
import torch

from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_moe_ffn

ALPHA, LIMIT = 1.0, 10.0


# ----------------------------------------------------------------------------- SwiGLU

def test_swiglu_inside_the_limits_is_silu_times_up(orc):
    rng = np.random.default_rng(40)
    g = rng.uniform(-9.99, 9.99, 2000)
    u = rng.uniform(-9.99, 9.99, 2000)
    ref = (torch.nn.functional.silu(torch.tensor(g, dtype=torch.float64)) * torch.tensor(u)).numpy()
    assert np.allclose(orc.swiglu(g, u), ref, rtol=1e-14, atol=1e-300)
    # alpha scales the gate inside the silu
    ref2 = (torch.nn.functional.silu(torch.tensor(2.0 * g)) * torch.tensor(u)).numpy()
    assert np.allclose(orc.swiglu(g, u, alpha=2.0), ref2, rtol=1e-14, atol=1e-300)


def test_swiglu_clamps(orc):
    L = LIMIT
    silu_L = L / (1.0 + np.exp(-L))
    g = np.array([10.0, 11.0, 1e6, 50.0, 3.0, 3.0, 3.0, -1e6, 0.0])
    u = np.array([2.0, 2.0, -3.0, 100.0, 12.0, -12.0, 10.0, 5.0, 7.0])
    got = orc.swiglu(g, u)
    silu3 = 3.0 / (1.0 + np.exp(-3.0))
    want = np.array([silu_L * 2, silu_L * 2, silu_L * -3, silu_L * L, silu3 * L, silu3 * -L, silu3 * L,
                     0.0, 0.0])
    assert np.allclose(got, want, rtol=1e-15, atol=0.0)
    # gate is clamped from above only: a very negative gate drives silu to 0
    assert abs(orc.swiglu(np.array([-50.0]), np.array([1.0]))[0]) < 1e-19


# ----------------------------------------------------------------------------- routing

def test_router_logits_match_numpy(orc):
    d = gen_moe_ffn(3, 16, 512, 64, 4, seed=41)
    lg = orc.router_logits(d["x"], d["wr"])
    ref = bf16_values(d["x"]).astype(np.float64) @ bf16_values(d["wr"]).astype(np.float64).T
    assert np.allclose(lg, ref, rtol=1e-13, atol=1e-13)


def test_topk_order_and_ties(orc):
    rng = np.random.default_rng(42)
    lg = rng.standard_normal((5, 37))
    lg[1, [3, 9, 20]] = 5.0          # a three-way tie at the top: lower ids first
    lg[2, :] = 0.25                   # all equal: ids 0..k-1
    lg[3, [0, 36]] = lg[3].max() + 1  # tie between the first and the last expert
    for k in (1, 4, 8):
        ids = orc.topk(lg, k)
        ref = np.argsort(-lg, axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref.astype(np.int32))
    assert list(orc.topk(lg, 3)[1]) == [3, 9, 20]


def test_topk_softmax_matches_scipy(orc):
    rng = np.random.default_rng(43)
    lg = rng.standard_normal((4, 64)) * 3
    ids = orc.topk(lg, 6)
    g = orc.topk_softmax(lg, ids)
    ref = scipy.special.softmax(np.take_along_axis(lg, ids.astype(np.int64), axis=1), axis=1)
    assert np.allclose(g, ref, rtol=1e-14, atol=0)
    assert np.allclose(g.sum(axis=1), 1.0, rtol=1e-15)
    assert np.all(np.diff(g, axis=1) <= 0)  # largest logit first -> largest weight first


# ----------------------------------------------------------------------------- expert FFN

def _one_expert(orc, d, e, t):
    """SwiGLU activation of expert e for token t from the pinned MXFP4 GEMV."""
    H = d["x"].shape[1]
    I = d["w13"].shape[1] // 2
    ids = np.array([[e]], np.int32)
    one = np.ones((1, 1), np.float32)
    _, gu, _ = orc.moe_mxfp4(d["x"][t:t + 1], d["w13"], d["s13"], ids, one)
    return orc.f64_to_bf16(orc.swiglu(gu[0, :I], gu[0, I:]))


def test_ffn_gate_up_and_down_compose_from_the_plain_gemv(orc):
    d = gen_moe_ffn(2, 4, 256, 96, 1, seed=44)
    ids = np.array([[2], [0]], np.int32)
    g = np.ones((2, 1))
    act, y, ye, S = orc.moe_ffn_mxfp4(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], ids, g)
    for t in range(2):
        e = int(ids[t, 0])
        a = _one_expert(orc, d, e, t)
        assert np.array_equal(act[t], a)
        # down projection of that bf16 activation through the plain expert GEMV
        yd, yde, Sd = orc.moe_mxfp4(a[None, :], d["w2"], d["s2"], np.array([[e]], np.int32),
                                    np.ones((1, 1), np.float32))
        assert np.array_equal(y[t], yd[0])
        assert np.allclose(ye[t], yde[0], rtol=0, atol=1e-12 * Sd[0].max())


def test_ffn_weighted_sum_over_slots(orc):
    d = gen_moe_ffn(2, 6, 256, 64, 3, seed=45)
    ids = np.array([[5, 1, 3], [0, 2, 4]], np.int32)
    g = np.array([[0.5, 0.3, 0.2], [0.7, 0.2, 0.1]])
    act, y, ye, S = orc.moe_ffn_mxfp4(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], ids, g)
    for t in range(2):
        tot = np.zeros(256)
        for j in range(3):
            e = int(ids[t, j])
            a = _one_expert(orc, d, e, t)
            assert np.array_equal(act[t * 3 + j], a)
            _, yde, _ = orc.moe_mxfp4(a[None, :], d["w2"], d["s2"], np.array([[e]], np.int32),
                                      np.ones((1, 1), np.float32))
            tot += g[t, j] * yde[0]
        assert np.allclose(ye[t], tot, rtol=1e-13, atol=1e-13 * S[t].max())


def test_ffn_degenerate_alpha_and_limit(orc):
    d = gen_moe_ffn(2, 4, 128, 64, 2, seed=46)
    ids = np.array([[0, 3], [1, 2]], np.int32)
    g = np.array([[0.6, 0.4], [0.5, 0.5]])
    for kw in ({"alpha": 0.0}, {"limit": 0.0}):
        act, y, ye, S = orc.moe_ffn_mxfp4(d["x"], d["w13"], d["s13"], d["w2"], d["s2"], ids, g, **kw)
        assert np.all(bf16_values(act) == 0) and np.all(ye == 0) and np.all(bf16_values(y) == 0)


def test_ffn_out_of_range_ids_contribute_nothing(orc):
    d = gen_moe_ffn(2, 4, 128, 64, 2, seed=47)
    g = np.array([[0.6, 0.4], [0.5, 0.5]])
    a1, y1, ye1, _ = orc.moe_ffn_mxfp4(d["x"], d["w13"], d["s13"], d["w2"], d["s2"],
                                       np.array([[0, 7], [-1, 2]], np.int32), g)
    # the same tokens with the invalid slot's weight moved to zero and a valid id
    a2, y2, ye2, _ = orc.moe_ffn_mxfp4(d["x"], d["w13"], d["s13"], d["w2"], d["s2"],
                                       np.array([[0, 1], [3, 2]], np.int32), np.array([[0.6, 0.0], [0.0, 0.5]]))
    assert np.array_equal(ye1, ye2)
    assert np.all(a1[1] == 0) and np.all(a1[2] == 0)


def test_routed_ffn_end_to_end_is_the_composition(orc):
    d = gen_moe_ffn(3, 8, 256, 64, 3, seed=48)
    ids, g, lg, act, y, ye, S = orc.moe_ffn_route_mxfp4(d["x"], d["wr"], 3, d["w13"], d["s13"], d["w2"], d["s2"])
    ref_lg = bf16_values(d["x"]).astype(np.float64) @ bf16_values(d["wr"]).astype(np.float64).T
    assert np.array_equal(ids, np.argsort(-ref_lg, axis=1, kind="stable")[:, :3].astype(np.int32))
    assert np.allclose(g, scipy.special.softmax(np.take_along_axis(ref_lg, ids.astype(np.int64), 1), 1),
                       rtol=1e-12)


# ----------------------------------------------------------------------------- activation rounding

# (gate, up) bf16 pairs found by a random search: the fp64 SwiGLU value lies a
# fraction of an fp32 ulp from a bf16 rounding midpoint, so rounding it once
# to bf16 differs from rounding it to fp32 first and then to bf16 (ties to
# even).  The activation is the input of the bf16 down projection and is
# rounded once.
ROUNDING_PAIRS = [(-0.1923828125, 4.03125), (-0.7578125, -1.5546875), (-0.1923828125, 8.0625),
                  (-0.7578125, 6.21875)]


def _bf16_nearest_exact(v: float) -> int:
    """bf16 bits of the value nearest to v, by exact rational comparison of
    the two bf16 neighbours (v is never a tie here)."""
    from fractions import Fraction
    f = np.float32(v)
    hi = int(f.view(np.uint32)) >> 16
    cands = [hi - 1, hi, hi + 1]
    vals = [Fraction(float(np.uint32(c << 16).view(np.float32))) for c in cands]
    d = [abs(c - Fraction(v)) for c in vals]
    assert sorted(d)[0] != sorted(d)[1]
    return cands[d.index(min(d))]


def test_ffn_activation_is_rounded_once(orc):
    import math
    I, H = 32, 64
    w13 = np.zeros((1, 2 * I, H // 2), np.uint8)
    s13 = np.full((1, 2 * I, H // 32), 127, np.uint8)  # scale 2^0
    x = np.zeros((1, H), np.float32)
    expect = {}
    for i, (a, b) in enumerate(ROUNDING_PAIRS):
        # gate row i reads x[i], up row i reads x[I + i], each through code 1.0 (nibble 0b0010)
        w13[0, i, i // 2] |= 0x2 << (4 * (i % 2))
        w13[0, I + i, (I + i) // 2] |= 0x2 << (4 * ((I + i) % 2))
        x[0, i], x[0, I + i] = a, b
        v = a / (1.0 + math.exp(-a)) * b
        single = _bf16_nearest_exact(v)
        f = np.float32(v)
        double = int(torch.tensor([float(f)], dtype=torch.float32).to(torch.bfloat16).view(torch.int16)[0]) & 0xFFFF
        assert single != double
        expect[i] = single
    w2 = np.zeros((1, H, I // 2), np.uint8)
    s2 = np.full((1, H, I // 32), 127, np.uint8)
    xb = bf16_bits(x)
    assert np.array_equal(bf16_values(xb), x)
    act, _, _, _ = orc.moe_ffn_mxfp4(xb, w13, s13, w2, s2, np.zeros((1, 1), np.int32), np.ones((1, 1)))
    for i, bits in expect.items():
        assert int(act[0, i]) == bits, (i, hex(int(act[0, i])), hex(bits))
    assert not act[0, len(ROUNDING_PAIRS):].any()
