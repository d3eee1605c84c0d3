"""GPU parity of the K-slice decode kernels (K a multiple of 1024, M <= 16:
INT8 from M = 3, E4M3 weight-only from M = 2, FP8 W8A8 from M = 3)
against the CPU oracle, over every slice length L = K/1024 and every tile
count T per workgroup they are built for.  The (L, T) noted per case is what
a 256-compute-unit device runs: one workgroup per compute unit, or one per 16
rows when N < 4096; a workgroup with more than six tiles runs them in passes
of T tiles; parity does not depend on it.  INT8 is compared bit-exactly
(codes, int32 sums, bf16 outputs), the float kinds under the comparison rules
of oracle/compare.py."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits, lib, need_gpu, padded
from oracle.compare import check_float
from skinny_gemm_qlin_amd.inputs import bf16_bits, gen_fp8, gen_fp8_w8a8, gen_int8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


# ----------------------------------------------------------------------------- INT8

def _i8(ql, orc, M, N, K, seed, w_pad=0, bias=False):
    d = gen_int8(M, N, K, seed=seed)
    b = bf16_bits(np.random.default_rng(seed).standard_normal(N).astype(np.float32)) if bias else None
    xq, xs = orc.act_quant_i8(d["x"])
    wd = dev(d["w"]) if w_pad == 0 else padded(d["w"], w_pad)
    acc = ql.qlin_gemv_i8(dev(xq), dev(xs), wd, dev(d["ws"]), out_kind=1)
    y = ql.qlin_gemv_i8(dev(xq), dev(xs), wd, dev(d["ws"]), bias=None if b is None else dev_bf16(b))
    torch.cuda.synchronize()
    oacc, oy = orc.gemv_i8(xq, xs, d["w"], d["ws"], bias=b)
    assert np.array_equal(host(acc), oacc), "int32 sums differ"
    assert np.array_equal(host_bits(y), oy), "bf16 outputs differ"


@pytest.mark.parametrize("M,N,K", [
    (3, 100, 2048),     # L=2, T=1, 7 workgroups
    (16, 4096, 3072),   # L=3, T=1
    (5, 5000, 4096),    # L=4, T=2
    (8, 9001, 5120),    # L=5, T=3
    (12, 13000, 6144),  # L=6, T=4
    (16, 17000, 7168),  # L=7, T=5
    (4, 21000, 8192),   # L=8, T=6
    (7, 3000, 9216),    # L=9 (one tile in flight from here, up to 8 tokens), T=1
    (8, 1001, 12288),   # L=12
    (4, 8192, 12288),   # L=12 with two tiles per unit: the per-tile matrix-core kernel
    (6, 6000, 13312),   # L=13, two tiles: the same
    (4, 4096, 14336),   # L=14, T=1
    (5, 28672, 10240),  # L=10, seven tiles: two passes of four
    (12, 1001, 12288),  # above 8 lines and 8 tokens: the per-tile matrix-core kernel
    (16, 9000, 14336),
    (6, 700, 15360),    # L=15: past the K-slice kernels, the per-tile matrix-core kernel
    (7, 30000, 2048),   # eight tiles per unit: two passes of four
    (4, 28672, 4096),   # L=4, seven tiles: two passes of four, the last tile empty
    (9, 50001, 2048),   # 13 tiles: three passes of five
    (16, 1, 2048),      # one row
    (3, 17, 2048),      # two workgroups, 9 and 8 rows
    # from 12 tokens the rows are split into contiguous blocks
    (16, 30000, 2048),  # 256 blocks of 29 runs, the first 76 with one more: two passes
    (12, 17, 2048),     # two blocks, 3 runs and 2 runs (the last one row)
    (13, 17412, 5120),  # 4353 runs: one block of 18, the rest 17
    (16, 28675, 4096),  # 7169 runs: blocks of 28 or 29 runs, two passes of four tiles
    (12, 50001, 3072),  # three passes of five tiles
])
def test_ks_int8_tiles_and_slices(ql, orc, M, N, K):
    _i8(ql, orc, M, N, K, seed=M * 7 + N)


@pytest.mark.parametrize("M", list(range(3, 17)))
def test_ks_int8_every_m(ql, orc, M):
    _i8(ql, orc, M, 2000, 2048, seed=M)


def test_ks_int8_padded_pitch_and_bias(ql, orc):
    _i8(ql, orc, 6, 3000, 2048, seed=3, w_pad=256, bias=True)


def test_ks_int8_decode_shape_is_deterministic(ql):
    d = gen_int8(16, 17408, 5120, seed=21)
    xq, xs = ql.qlin_act_quant_i8(dev_bf16(d["x"]))
    w, ws = dev(d["w"]), dev(d["ws"])
    ref = ql.qlin_gemv_i8(xq, xs, w, ws, out_kind=1)
    for _ in range(10):
        assert torch.equal(ql.qlin_gemv_i8(xq, xs, w, ws, out_kind=1), ref)


# ----------------------------------------------------------------------------- E4M3 weight-only

@pytest.mark.parametrize("M,N,K", [
    (3, 100, 2048),     # L=2, T=1
    (16, 4096, 3072),   # L=3, T=1
    (5, 5000, 4096),    # L=4, T=2
    (8, 9001, 5120),    # L=5, T=3
    (11, 13000, 2048),  # L=2, T=4
    (16, 16500, 2048),  # L=2, T=5
    (4, 21000, 2048),   # L=2, T=6
    (7, 30000, 2048),   # eight tiles per unit: two passes of four
    (2, 28672, 4096),   # two passes of four, the last tile empty
    (9, 1, 5120),
    # from 12 tokens whole 16-row tiles are dealt out in turn, then the runs left
    (12, 30000, 2048),  # 7 whole tiles each, then 1 or 2 of the 332 runs left: two passes
    (16, 17, 2048),     # two workgroups, no whole tiles
    (13, 17412, 5120),  # 4 whole tiles each, then 257 runs
    (16, 50001, 2048),  # 12 whole tiles each, then 0 or 1 of the 213 runs left: three passes of five
    (2, 3000, 6144),    # L=6, two tiles in flight
    (5, 14336, 7168),   # L=7, one tile in flight, T=4
    (16, 6001, 8192),   # L=8, T=2
    (4, 28672, 8192),   # L=8, two passes of four
])
def test_ks_fp8_tiles_and_slices(ql, orc, M, N, K):
    d = gen_fp8(M, N, K, seed=M + N)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M", list(range(2, 17)))
def test_ks_fp8_every_m(ql, orc, M):
    d = gen_fp8(M, 1500, 3072, seed=M, per_tensor=M % 2 == 0)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), padded(d["w"], 128), dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, 3072)


# ----------------------------------------------------------------------------- W8A8 E4M3 x E4M3

def _w8a8(ql, orc, M, N, K, seed, per_channel=True, per_token=True, w_pad=0, x_fmt=0, w_fmt=0):
    d = gen_fp8_w8a8(M, N, K, w_fmt=w_fmt, per_channel=per_channel, seed=seed)
    xq, xs = orc.act_quant_fp8(d["x"], x_fmt, per_token)
    wd = dev(d["w"]) if w_pad == 0 else padded(d["w"], w_pad)
    y = ql.qlin_gemv_fp8_w8a8(dev(xq), dev(xs), wd, dev(d["ws"]), x_fmt, w_fmt)
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8_w8a8(xq, xs, x_fmt, d["w"], d["ws"], w_fmt)
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K", [
    (4, 100, 2048),     # L=2, T=1
    (16, 4096, 3072),   # L=3, T=1
    (5, 5000, 4096),    # L=4, T=2
    (8, 9001, 5120),    # L=5, T=3
    (11, 13000, 2048),  # L=2, T=4
    (16, 16500, 2048),  # L=2, T=5
    (4, 21000, 2048),   # L=2, T=6
    (7, 30000, 2048),   # eight tiles per unit: two passes of four
    (3, 28672, 4096),   # two passes of four, the last tile empty
    # from 8 tokens whole 16-row tiles are dealt out in turn, then the runs left
    (8, 30000, 2048),   # 7 whole tiles each, then 1 or 2 of the 332 runs left: two passes
    (9, 17, 2048),      # two workgroups, no whole tiles
    (16, 17412, 5120),  # 4 whole tiles each, then 257 runs (one workgroup takes two)
    (12, 50001, 3072),  # three passes of five
    (3, 5000, 6144),    # L=6 at three tokens
    (8, 14336, 7168),   # L=7, T=4
    (16, 20000, 8192),  # L=8, T=5
    (6, 6144, 8192),    # two tiles per unit: the per-tile matrix-core kernel
])
def test_ks_w8a8_tiles_and_slices(ql, orc, M, N, K):
    _w8a8(ql, orc, M, N, K, seed=M + N)


@pytest.mark.parametrize("M", list(range(3, 17)))
def test_ks_w8a8_every_m(ql, orc, M):
    _w8a8(ql, orc, M, 1500, 3072, seed=M, per_channel=M % 2 == 0, per_token=M % 3 != 0, w_pad=256)


# ----------------------------------------------------------------------------- output rows

def test_ks_unaligned_output_rows(ql, orc):
    # output views with an odd row pitch and a 2- or 4-byte base offset: every
    # output lands in place and nothing outside the [M, N] view is written
    M, N, K = 5, 1001, 2048
    d = gen_int8(M, N, K, seed=31)
    xq, xs = orc.act_quant_i8(d["x"])
    oacc, oy = orc.gemv_i8(xq, xs, d["w"], d["ws"])
    buf = torch.full((M, N + 3), -1.0, dtype=torch.bfloat16, device="cuda")
    y = ql.qlin_gemv_i8(dev(xq), dev(xs), dev(d["w"]), dev(d["ws"]), y=buf[:, 1:N + 1])
    buf32 = torch.full((M, N + 2), 7, dtype=torch.int32, device="cuda")
    acc = ql.qlin_gemv_i8(dev(xq), dev(xs), dev(d["w"]), dev(d["ws"]), y=buf32[:, 1:N + 1], out_kind=1)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), oy)
    assert np.array_equal(host(acc), oacc)
    assert torch.all(buf[:, 0] == -1.0) and torch.all(buf[:, N + 1:] == -1.0)
    assert torch.all(buf32[:, 0] == 7) and torch.all(buf32[:, N + 1:] == 7)

    f = gen_fp8(M, N, K, seed=32)
    _, ye, S = orc.gemv_fp8(f["x"], f["w"], f["ws"])
    buf = torch.full((M, N + 3), -1.0, dtype=torch.bfloat16, device="cuda")
    y = ql.qlin_gemv_fp8(dev_bf16(f["x"]), dev(f["w"]), dev(f["ws"]), y=buf[:, 1:N + 1])
    torch.cuda.synchronize()
    check_float(host_bits(y), ye, S, K)
    assert torch.all(buf[:, 0] == -1.0) and torch.all(buf[:, N + 1:] == -1.0)


@pytest.mark.parametrize("x_fmt,w_fmt", [(0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("M,N,K", [(3, 700, 2048), (16, 5000, 5120), (9, 17408, 4096)])
def test_ks_w8a8_other_formats(ql, orc, M, N, K, x_fmt, w_fmt):
    # E5M2 activations and / or weights: the same kernels with the other widening
    _w8a8(ql, orc, M, N, K, seed=M + N + 10 * x_fmt + w_fmt, x_fmt=x_fmt, w_fmt=w_fmt)
