"""GPU parity of the 128x128 block-scaled FP8 call (qlin_gemv_fp8_blk) at 2..16
tokens on decode-sized matrices: K multiples of 1024 up to 8192, N from one
row to 4096 with partial row runs and 128-row blocks, padded pitches, edge
values, extreme weight scale bytes, a scale buffer at an odd address, and
repeat determinism.  Exported E4M3 codes and UE8M0 exponents are compared
bit-exactly with the CPU oracle, outputs under the float rules of
oracle/compare.py."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits, lib, need_gpu, padded
from oracle.compare import check_float
from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_fp8_blk

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _run(ql, x, w, ws):
    y, xq, xs = ql.qlin_gemv_fp8_blk(x, w, ws)
    torch.cuda.synchronize()
    return host_bits(y), host(xq), host(xs)


def _check(orc, d, got):
    y, xq, xs = got
    oxq, oxs, oy, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert np.array_equal(xs, oxs), "UE8M0 activation exponents differ"
    bad = np.argwhere(xq != oxq)
    assert bad.size == 0, f"E4M3 activation codes differ at {bad[:5].tolist()}"
    return check_float(y, ye, S, d["w"].shape[1])


# K = 1024 L for L = 2..8; N from one row to 16 rows per compute unit, with
# partial row runs and row blocks; token counts across 2..16
SHAPES = [(2, 4096, 7168), (3, 4096, 7168), (8, 4096, 7168), (16, 4096, 7168), (5, 4096, 8192),
          (13, 4000, 2048), (16, 300, 2048), (7, 1, 3072), (9, 129, 5120), (16, 4095, 6144), (11, 17, 4096),
          (4, 2049, 7168)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_blk_decode_shapes(ql, orc, M, N, K):
    print(f"blk decode M={M} N={N} K={K}", flush=True)
    d = gen_fp8_blk(M, N, K, seed=M * 1000 + N + K)
    stats = _check(orc, d, _run(ql, dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])))
    if M * N >= 4096:  # enough outputs for the fraction to mean something
        assert stats["ref_bits_equal"] > 0.98


def test_blk_decode_pitches(ql, orc):
    # padded activation and weight rows (row pitches 2048 + 40 and 2048 + 256)
    d = gen_fp8_blk(6, 1000, 2048, seed=51)
    xp = padded(d["x"].view(np.int16), 40).view(torch.bfloat16)
    wp = padded(d["w"], 256)
    print("blk decode padded pitches", flush=True)
    _check(orc, d, _run(ql, xp, wp, dev(d["ws"])))


def test_blk_decode_misaligned_scales(ql, orc):
    # the weight scale buffer at an odd address: the same codes, exponents
    # and outputs as from an aligned copy
    d = gen_fp8_blk(16, 4096, 7168, seed=52)
    x, w = dev_bf16(d["x"]), dev(d["w"])
    ws = dev(d["ws"])
    raw = torch.empty(ws.numel() + 1, dtype=torch.uint8, device=ws.device)
    wsu = raw[1:].view(ws.shape)
    wsu.copy_(ws)
    assert wsu.data_ptr() % 4 != 0
    print("blk decode misaligned scales", flush=True)
    a = _run(ql, x, w, ws)
    b = _run(ql, x, w, wsu)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    _check(orc, d, a)


def test_blk_decode_edge_values(ql, orc):
    # E4M3 midpoints and their negatives, a zero and a signed-zero group, tiny
    # and huge groups, one outlier per group: three tokens, K = 2048
    rng = np.random.default_rng(53)
    K = 2048
    x = rng.standard_normal((3, K)).astype(np.float32)
    e4 = orc.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mids = ((e4[:-1] + e4[1:]) / 2).astype(np.float32)
    x[0, :126] = mids
    x[0, 126] = 448.0
    x[0, 128:254] = -mids
    x[0, 254] = -448.0
    x[1, 256:384] = 0.0
    x[1, 384:512] = -0.0
    x[1, 512:640] *= 1e-35
    x[1, 640:768] *= 3e25
    x[2, 768:896] = np.where(np.arange(128) % 2 == 0, 1e-6, -1e-6)
    x[2, 800] = 100.0
    x[2, 1920:2048] = 0.0
    d = {"x": bf16_bits(x), "w": rng.integers(0, 0x7E, (130, K)).astype(np.uint8),
         "ws": rng.integers(110, 140, (2, K // 128)).astype(np.uint8)}
    assert np.all(np.isfinite(bf16_values(orc.fp8_blk(d["x"], d["w"], d["ws"])[2])))
    print("blk decode edge values", flush=True)
    _check(orc, d, _run(ql, dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])))


@pytest.mark.parametrize("M", [2, 16])
def test_blk_decode_extreme_weight_scale_bytes(ql, orc, M):
    # weight scale bytes 0, 1, 253, 254 in every row block; activation groups
    # sized so that every output stays finite
    rng = np.random.default_rng(54)
    K, N = 2048, 256
    pat = np.array([[0, 1, 253, 254], [1, 0, 254, 253]], np.uint8)
    ws = np.tile(pat, (1, K // 512))
    x = rng.standard_normal((M, K)).astype(np.float32)
    for kb in range(K // 128):
        x[:, kb * 128:(kb + 1) * 128] *= 1e10 if kb % 4 < 2 else 1e-30
    w = gen_fp8_blk(1, N, K, seed=55)["w"]
    d = {"x": bf16_bits(x), "w": w, "ws": ws}
    assert np.all(np.isfinite(bf16_values(orc.fp8_blk(d["x"], d["w"], d["ws"])[2])))
    print(f"blk decode extreme scale bytes M={M}", flush=True)
    _check(orc, d, _run(ql, dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])))


def test_blk_decode_repeats_are_identical(ql):
    d = gen_fp8_blk(8, 4096, 7168, seed=56)
    x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
    ref = ql.qlin_gemv_fp8_blk(x, w, ws)[0]
    for _ in range(10):
        assert torch.equal(ql.qlin_gemv_fp8_blk(x, w, ws)[0].view(torch.int16), ref.view(torch.int16))
