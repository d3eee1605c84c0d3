"""GPU parity of the top-k MXFP4 expert GEMV (qlin_moe_mxfp4) against the CPU
oracle, under the float rules of oracle/compare.py; includes an exhaustive
E2M1 decode / nibble-order check through the product path."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host_bits, lib, need_gpu
from oracle.compare import bf16_to_f64, check_float
from skinny_gemm_qlin_amd.inputs import gen_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _gpu(ql, d, ids=None, gw=None):
    y = ql.qlin_moe_mxfp4(dev_bf16(d["x"]), dev(d["w"]), dev(d["s"]),
                          dev(d["ids"] if ids is None else ids), dev(d["gw"] if gw is None else gw))
    torch.cuda.synchronize()
    return host_bits(y)


def _check(orc, ql, d, ids=None, gw=None):
    ids = d["ids"] if ids is None else ids
    gw = d["gw"] if gw is None else gw
    y, ye, S = orc.moe_mxfp4(d["x"], d["w"], d["s"], ids, gw)
    return check_float(_gpu(ql, d, ids, gw), ye, S, d["x"].shape[1])


def test_e2m1_decode_and_nibble_order(ql, orc):
    # expert row n = 16*a + b holds byte (b << 4) | a at byte 3 (elements 6 and 7)
    K = 64
    w = np.zeros((1, 256, K // 2), np.uint8)
    w[0, :, 3] = [((n % 16) << 4) | (n // 16) for n in range(256)]
    s = np.full((1, 256, K // 32), 127, np.uint8)
    ids = np.zeros((2, 1), np.int32)
    gw = np.ones((2, 1), np.float32)
    x = np.zeros((2, K), np.uint16)
    x[0, 6] = 0x3F80  # token 0 reads element 6 (low nibble), token 1 element 7 (high nibble)
    x[1, 7] = 0x3F80
    d = {"x": x, "w": w, "s": s, "ids": ids, "gw": gw}
    y = bf16_to_f64(_gpu(ql, d))
    n = np.arange(256)
    assert np.array_equal(y[0], orc.e2m1_decode((n // 16).astype(np.uint8)))
    assert np.array_equal(y[1], orc.e2m1_decode((n % 16).astype(np.uint8)))


def test_moe_full_config(ql, orc):
    d = gen_moe(8, 64, 2048, 7168, 6, seed=0)
    stats = _check(orc, ql, d)
    assert stats["ref_bits_equal"] > 0.99


@pytest.mark.parametrize("M,E,N,K,topk", [(1, 4, 64, 256, 1), (2, 8, 100, 512, 2), (3, 16, 37, 1024, 4),
                                          (5, 6, 130, 96, 3), (8, 64, 256, 7168, 6), (16, 32, 64, 2048, 8),
                                          (16, 3, 40, 512, 16),
                                          # 2 and 1 tokens per LDS pass, then the largest K accepted
                                          (6, 8, 70, 8192, 3), (5, 4, 33, 16384, 2), (3, 2, 16, 30720, 2),
                                          # expert ids up to the first-occurrence table's size, then past it
                                          (16, 1024, 24, 128, 16), (4, 1100, 16, 64, 8), (16, 1500, 8, 96, 16)])
def test_moe_shapes(ql, orc, M, E, N, K, topk):
    if topk > E:
        d = gen_moe(M, E, N, K, 1, seed=M + N)
        rng = np.random.default_rng(M)
        d["ids"] = rng.integers(0, E, (M, topk)).astype(np.int32)  # repeated experts within a token
        d["gw"] = rng.uniform(-1, 1, (M, topk)).astype(np.float32)
    else:
        d = gen_moe(M, E, N, K, topk, seed=M + N)
    _check(orc, ql, d)


def test_moe_all_tokens_one_expert(ql, orc):
    # 16 tokens routed to the same experts: more pairs than one pass holds
    d = gen_moe(16, 4, 96, 512, 2, seed=50)
    ids = np.tile(np.array([[1, 3]], np.int32), (16, 1))
    _check(orc, ql, d, ids=ids)


def test_moe_invalid_ids_contribute_nothing(ql, orc):
    d = gen_moe(4, 8, 64, 256, 3, seed=51)
    ids = d["ids"].copy()
    ids[0, 0] = -1
    ids[1, 2] = 8
    ids[3, :] = [100, -7, 9]  # a token with no valid expert -> y = 0
    stats = _check(orc, ql, d, ids=ids)
    y = _gpu(ql, d, ids=ids)
    assert np.all(bf16_to_f64(y[3]) == 0.0)


def test_moe_deterministic(ql):
    d = gen_moe(8, 64, 2048, 7168, 6, seed=52)
    args = [dev_bf16(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["ids"]), dev(d["gw"])]
    ref = ql.qlin_moe_mxfp4(*args)
    for _ in range(10):
        assert torch.equal(ql.qlin_moe_mxfp4(*args).view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("M", [1, 8, 16])
def test_moe_extreme_scale_bytes(ql, orc, M):
    # UE8M0 bytes 0 (2^-127, an fp32 subnormal), 1, 253 and 254 (2^127) on the
    # decode path; 32-blocks with a huge scale see tiny activations, blocks with
    # a tiny scale ordinary ones, so every output stays finite
    from skinny_gemm_qlin_amd.inputs import bf16_bits
    E, N, K, topk = 8, 96, 512, 3
    d = gen_moe(M, E, N, K, topk, seed=60 + M)
    rng = np.random.default_rng(61)
    nkb = K // 32
    huge = (np.arange(nkb) % 2 == 0)
    s = np.where(huge[None, None, :], rng.choice([253, 254], (E, N, nkb)), rng.choice([0, 1], (E, N, nkb)))
    d["s"] = s.astype(np.uint8)
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, np.repeat(huge, 32)] *= 1e-30
    d["x"] = bf16_bits(x)
    _, ye, _ = orc.moe_mxfp4(d["x"], d["w"], d["s"], d["ids"], d["gw"])
    assert np.all(np.isfinite(ye))
    print(f"moe extreme scale bytes M={M}", flush=True)
    _check(orc, ql, d)
