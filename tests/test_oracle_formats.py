"""Pins of the oracle's number formats (bf16, E4M3, E2M1, UE8M0).

Each oracle routine is checked against something other than itself: values the
pages print (tests/golden), torch's own float8_e4m3fn / bfloat16 casts
(library rounding), the OCP E2M1 value table, and constructed special cases.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from conftest import read_golden


def _torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ----------------------------------------------------------------------------- bf16

def test_bf16_round_matches_torch(orc):
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 2**32, size=4000, dtype=np.uint64).astype(np.uint32)
    # force exact ties (dropped half == 0x8000) on both parities, and near-ties
    bits[:500] = (bits[:500] & 0xFFFF0000) | 0x8000
    bits[500:600] = (bits[500:600] & 0xFFFF0000) | 0x7FFF
    bits[600:700] = (bits[600:700] & 0xFFFF0000) | 0x8001
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    extra = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, 3.3895314e38, 3.4e38,
                      1e-40, -1e-40, 1.401298e-45], dtype=np.float32)
    f = np.concatenate([f, extra])
    got = orc.f32_to_bf16(f)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_nan_is_canonical(orc):
    assert orc.f32_to_bf16(np.array([np.nan], dtype=np.float32))[0] == 0x7FC0
    assert orc.f64_to_bf16(np.array([np.nan]))[0] == 0x7FC0


def test_bf16_widen_is_exact(orc):
    h = np.arange(0, 65536, 97, dtype=np.uint16)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).to(torch.float32).numpy()
    got = orc.bf16_to_f32(h)
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all()


def test_f64_to_bf16_single_rounding(orc):
    # float32-representable doubles must round like the (torch-pinned) f32 path
    rng = np.random.default_rng(2)
    f = (rng.standard_normal(2000) * 10.0 ** rng.integers(-30, 30, 2000)).astype(np.float32)
    assert np.array_equal(orc.f64_to_bf16(f.astype(np.float64)), orc.f32_to_bf16(f))
    # a value a hair above a bf16 midpoint must round up, although rounding it to
    # float32 first would land exactly on the midpoint and tie to the even side
    lo = 1.0  # bf16 1.0 = 0x3F80 (even); next bf16 is 1 + 2^-7
    mid = lo + 2.0 ** -8
    assert orc.f64_to_bf16(np.array([mid]))[0] == 0x3F80                 # exact tie -> even
    assert orc.f64_to_bf16(np.array([mid + 2.0 ** -40]))[0] == 0x3F81    # above tie -> up
    assert orc.f64_to_bf16(np.array([-(mid + 2.0 ** -40)]))[0] == 0xBF81
    assert orc.f64_to_bf16(np.array([mid - 2.0 ** -40]))[0] == 0x3F80
    # overflow to infinity, subnormal spacing 2^-133
    assert orc.f64_to_bf16(np.array([3.4e38]))[0] == 0x7F80
    assert orc.f64_to_bf16(np.array([2.0 ** -133]))[0] == 0x0001
    assert orc.f64_to_bf16(np.array([2.0 ** -134]))[0] == 0x0000        # tie -> even (0)
    assert orc.f64_to_bf16(np.array([1.5 * 2.0 ** -133]))[0] == 0x0002  # tie -> even (2)


# ----------------------------------------------------------------------------- E4M3

def test_e4m3_decode_matches_torch_all_codes(orc):
    got = orc.e4m3_decode(np.arange(256))
    ref = _torch_e4m3_table()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    # signs: code 0x80 is -0
    assert math.copysign(1.0, got[0x80]) == -1.0


def test_e4m3_anchor_values(orc):
    d = orc.e4m3_decode(np.arange(256))
    assert d[0x38] == 1.0
    assert d[0x7E] == 448.0 and np.nanmax(d) == 448.0
    assert d[0x01] == 2.0 ** -9
    # page fact: magnitudes below 2^-6 are subnormal (exponent field 0)
    facts = {k: int(v) for k, v in read_golden("e4m3_facts.txt")}
    bound = 2.0 ** facts["subnormal_below_log2"]
    assert d[0x08] == bound  # smallest normal
    assert all(abs(d[c]) < bound for c in range(0x00, 0x08))
    assert all(abs(d[c]) >= bound for c in range(0x08, 0x7F))


def test_e4m3_fp16_lossless(orc):
    # page fact: a 256-entry fp16 table decodes every finite code exactly
    d = orc.e4m3_decode(np.arange(256))
    fin = d[~np.isnan(d)]
    assert fin.size == 254
    assert np.array_equal(fin.astype(np.float16).astype(np.float64), fin)


def test_e4m3_encode_roundtrip_and_ties(orc):
    tab = _torch_e4m3_table()
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    # every finite value encodes back to its code (incl. -0 -> 0x80)
    assert np.array_equal(orc.e4m3_encode(tab[codes]), codes.astype(np.uint8))
    # midpoints between consecutive positive codes, and a hair either side,
    # against torch's float8 cast (RNE)
    pos = tab[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2.0
    vals = np.concatenate([mids, mids * (1 + 2.0 ** -20), mids * (1 - 2.0 ** -20)])
    vals = np.concatenate([vals, -vals]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(vals.astype(np.float64)), ref)


def test_e4m3_encode_random_matches_torch(orc):
    rng = np.random.default_rng(3)
    v = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2.6, 20000)).astype(np.float32)
    v = v[np.abs(v) <= 448.0]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(orc.e4m3_encode(v.astype(np.float64)), ref)


def test_e4m3_encode_saturates(orc):
    v = np.array([448.0, 449.0, 464.0, 500.0, 1e6, -449.0, -1e30])
    assert list(orc.e4m3_encode(v)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE]
    assert orc.e4m3_encode(np.array([np.nan]))[0] == 0x7F


# ----------------------------------------------------------------------------- E2M1

OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # OCP MX spec, E2M1 magnitudes by code 0..7


def test_e2m1_decode_table(orc):
    d = orc.e2m1_decode(np.arange(16))
    assert list(d[:8]) == OCP_E2M1
    assert list(-d[8:]) == OCP_E2M1
    assert math.copysign(1.0, d[8]) == -1.0


# ----------------------------------------------------------------------------- UE8M0

def test_ue8m0_worked_bytes(orc):
    rows = read_golden("ue8m0_worked_bytes.txt")
    assert rows, "fixture empty"
    for b, lg in rows:
        assert orc.ue8m0_decode(np.array([int(b)]))[0] == 2.0 ** int(lg)


def test_ue8m0_special_bytes(orc):
    d = orc.ue8m0_decode(np.arange(256))
    assert d[127] == 1.0
    assert d[0] == 2.0 ** -127 and d[254] == 2.0 ** 127
    assert np.isnan(d[255])
    # strictly doubling byte to byte
    assert np.all(d[1:255] / d[0:254] == 2.0)


def test_block_config_fixture():
    import oracle
    cfg = {r[0]: r[1:] for r in read_golden("block_quant_config.txt")}
    assert cfg["fmt"] == ["e4m3"] and cfg["scale_fmt"] == ["ue8m0"]
    assert cfg["activation_scheme"] == ["dynamic"]
    assert [int(v) for v in cfg["weight_block_size"]] == [oracle.BLK, oracle.BLK]
