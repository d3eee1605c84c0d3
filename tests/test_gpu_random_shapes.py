"""Seeded random shapes through the dense entry points and the MXFP4 expert
GEMV, against the CPU oracle.  Decode (M = 1..16: INT8 GEMV and whole linear
layer, E4M3 weight-only, FP8 W8A8, 128x128 block-scaled FP8): N from one row to tens of thousands, K on and off the
multiples of 1024 that pick the K-slice kernels (up to 14 lines for INT8, 8
for the float kinds), padded weight pitches.  The per-M / per-shape kernel
choice (VALU kernels, codes or rows in LDS, K-slice with 1-3 tiles in flight
and in one or more passes, per-tile matrix-core kernels) is crossed many
times over.  Prefill (M = 17..1100: the tiled matrix-core GEMMs, split-K
over token blocks for few rows) and the expert GEMV at any M (one to 128
experts, top-1 to top-8, the decode kernel and the sorted grouped GEMM).
INT8 is compared bit-exactly, the float kinds under the comparison rules of
oracle/compare.py."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host, host_bits, lib, need_gpu, padded
from oracle.compare import check_float
from skinny_gemm_qlin_amd.inputs import gen_fp8, gen_fp8_blk, gen_fp8_w8a8, gen_int8, gen_moe

pytestmark = pytest.mark.gpu

MAX_MACS = 4e8  # M * N * K per case: the oracle's share stays within a second or so


def _shapes(seed, n, kmax_lines, kstep=16):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(1, 17))
        if rng.random() < 0.6:
            K = 1024 * int(rng.integers(2, kmax_lines + 1))
        else:
            K = kstep * int(rng.integers(1, 16384 // kstep + 1))
        N = int(np.exp(rng.uniform(0, np.log(60000))))
        N = max(1, min(N, int(MAX_MACS / (M * K))))
        pad = int(rng.choice([0, 0, 0, 16, 48, 256]))
        out.append((M, N, K, pad))
    return out


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


@pytest.mark.parametrize("M,N,K,pad", _shapes(501, 24, 14))
def test_random_int8(ql, orc, M, N, K, pad):
    print(f"int8 M={M} N={N} K={K} pad={pad}", flush=True)
    d = gen_int8(M, N, K, seed=M * 131 + N + K)
    xq, xs = orc.act_quant_i8(d["x"])
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    acc = ql.qlin_gemv_i8(dev(xq), dev(xs), wd, dev(d["ws"]), out_kind=1)
    y = ql.qlin_gemv_i8(dev(xq), dev(xs), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    oacc, oy = orc.gemv_i8(xq, xs, d["w"], d["ws"])
    assert np.array_equal(host(acc), oacc), "int32 sums differ"
    assert np.array_equal(host_bits(y), oy), "bf16 outputs differ"


@pytest.mark.parametrize("M,N,K,pad", _shapes(502, 20, 8))
def test_random_fp8(ql, orc, M, N, K, pad):
    print(f"fp8 M={M} N={N} K={K} pad={pad}", flush=True)
    d = gen_fp8(M, N, K, seed=M * 137 + N + K, per_tensor=(N + K) % 3 == 0)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K,pad", _shapes(503, 20, 8))
def test_random_fp8_w8a8(ql, orc, M, N, K, pad):
    print(f"w8a8 M={M} N={N} K={K} pad={pad}", flush=True)
    x_fmt, w_fmt = (M + N) % 2, (N + K // 16) % 2
    d = gen_fp8_w8a8(M, N, K, w_fmt=w_fmt, per_channel=N % 2 == 0, seed=M * 139 + N + K)
    xq, xs = orc.act_quant_fp8(d["x"], x_fmt, K % 3 != 0)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y = ql.qlin_gemv_fp8_w8a8(dev(xq), dev(xs), wd, dev(d["ws"]), x_fmt, w_fmt)
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8_w8a8(xq, xs, x_fmt, d["w"], d["ws"], w_fmt)
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K,pad", _shapes(504, 16, 14))
def test_random_linear_i8(ql, orc, M, N, K, pad):
    print(f"linear_i8 M={M} N={N} K={K} pad={pad}", flush=True)
    d = gen_int8(M, N, K, seed=M * 149 + N + K)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y, xq, xs = ql.qlin_linear_i8(dev_bf16(d["x"]), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_i8(d["x"])
    _, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"])
    assert np.array_equal(host(xq), oxq), "int8 codes differ"
    assert np.array_equal(host(xs).view(np.uint32), oxs.view(np.uint32)), "scales differ"
    assert np.array_equal(host_bits(y), oy), "bf16 outputs differ"


@pytest.mark.parametrize("M,N,K,pad", _shapes(505, 16, 8, kstep=128))
def test_random_fp8_blk(ql, orc, M, N, K, pad):
    print(f"fp8_blk M={M} N={N} K={K} pad={pad}", flush=True)
    d = gen_fp8_blk(M, N, K, seed=M * 151 + N + K)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs, _, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert np.array_equal(host(xs), oxs), "UE8M0 activation exponents differ"
    assert np.array_equal(host(xq), oxq), "E4M3 activation codes differ"
    check_float(host_bits(y), ye, S, K)


# ----------------------------------------------------------------------------- prefill

def _prefill_shapes(seed, n, kstep=16):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(np.exp(rng.uniform(np.log(17), np.log(1100))))
        K = kstep * int(rng.integers(1, 8192 // kstep + 1))
        N = int(np.exp(rng.uniform(0, np.log(4000))))
        N = max(1, min(N, int(MAX_MACS / (M * K))))
        out.append((M, N, K, int(rng.choice([0, 0, 16, 48]))))
    return out


@pytest.mark.parametrize("M,N,K,pad", _prefill_shapes(511, 12))
def test_random_prefill_int8(ql, orc, M, N, K, pad):
    print(f"prefill int8 M={M} N={N} K={K} pad={pad}", flush=True)
    d = gen_int8(M, N, K, seed=M * 157 + N + K)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y, xq, xs = ql.qlin_linear_i8(dev_bf16(d["x"]), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs = orc.act_quant_i8(d["x"])
    _, oy = orc.gemv_i8(oxq, oxs, d["w"], d["ws"])
    assert np.array_equal(host(xq), oxq), "int8 codes differ"
    assert np.array_equal(host(xs).view(np.uint32), oxs.view(np.uint32)), "scales differ"
    assert np.array_equal(host_bits(y), oy), "bf16 outputs differ"


@pytest.mark.parametrize("M,N,K,pad", _prefill_shapes(512, 10))
def test_random_prefill_fp8(ql, orc, M, N, K, pad):
    print(f"prefill fp8 M={M} N={N} K={K} pad={pad}", flush=True)
    d = gen_fp8(M, N, K, seed=M * 163 + N + K, per_tensor=N % 2 == 1)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y = ql.qlin_gemv_fp8(dev_bf16(d["x"]), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8(d["x"], d["w"], d["ws"])
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K,pad", _prefill_shapes(513, 10))
def test_random_prefill_fp8_w8a8(ql, orc, M, N, K, pad):
    print(f"prefill w8a8 M={M} N={N} K={K} pad={pad}", flush=True)
    x_fmt, w_fmt = M % 2, (N + 1) % 2
    d = gen_fp8_w8a8(M, N, K, w_fmt=w_fmt, per_channel=K % 32 == 0, seed=M * 167 + N + K)
    xq, xs = orc.act_quant_fp8(d["x"], x_fmt, True)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y = ql.qlin_gemv_fp8_w8a8(dev(xq), dev(xs), wd, dev(d["ws"]), x_fmt, w_fmt)
    torch.cuda.synchronize()
    _, ye, S = orc.gemv_fp8_w8a8(xq, xs, x_fmt, d["w"], d["ws"], w_fmt)
    check_float(host_bits(y), ye, S, K)


@pytest.mark.parametrize("M,N,K,pad", _prefill_shapes(514, 10, kstep=128))
def test_random_prefill_fp8_blk(ql, orc, M, N, K, pad):
    print(f"prefill fp8_blk M={M} N={N} K={K} pad={pad}", flush=True)
    d = gen_fp8_blk(M, N, K, seed=M * 173 + N + K)
    wd = dev(d["w"]) if pad == 0 else padded(d["w"], pad)
    y, xq, xs = ql.qlin_gemv_fp8_blk(dev_bf16(d["x"]), wd, dev(d["ws"]))
    torch.cuda.synchronize()
    oxq, oxs, _, ye, S = orc.fp8_blk(d["x"], d["w"], d["ws"])
    assert np.array_equal(host(xs), oxs), "UE8M0 activation exponents differ"
    assert np.array_equal(host(xq), oxq), "E4M3 activation codes differ"
    check_float(host_bits(y), ye, S, K)


# ----------------------------------------------------------------------------- MXFP4 expert GEMV

def _moe_shapes(seed, n):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(1, 17)) if rng.random() < 0.6 else int(np.exp(rng.uniform(np.log(17), np.log(600))))
        E = int(np.exp(rng.uniform(0, np.log(128))))
        topk = int(rng.integers(1, min(E, 8) + 1))
        K = 32 * int(rng.integers(1, 8192 // 32 + 1))
        N = int(np.exp(rng.uniform(0, np.log(3000))))
        N = max(1, min(N, int(MAX_MACS / 4 / (M * topk * K)), int(2e8 / (E * K / 2))))
        out.append((M, E, N, K, topk))
    return out


@pytest.mark.parametrize("M,E,N,K,topk", _moe_shapes(521, 16))
def test_random_moe(ql, orc, M, E, N, K, topk):
    print(f"moe M={M} E={E} N={N} K={K} topk={topk}", flush=True)
    d = gen_moe(M, E, N, K, topk, seed=M * 179 + E + N + K)
    y = ql.qlin_moe_mxfp4(dev_bf16(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["ids"]), dev(d["gw"]))
    torch.cuda.synchronize()
    _, ye, S = orc.moe_mxfp4(d["x"], d["w"], d["s"], d["ids"], d["gw"])
    check_float(host_bits(y), ye, S, K)
