"""GPU parity of the MXFP4 top-k expert GEMV at prefill-sized M (> 16: the
pair sort and grouped matrix-core GEMM) against the CPU oracle, under the
float comparison rules."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host_bits, lib, need_gpu
from oracle.compare import bf16_to_f64, check_float
from skinny_gemm_qlin_amd.inputs import bf16_bits, bf16_values, gen_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _run(ql, d, ids=None, gw=None):
    y = ql.qlin_moe_mxfp4(dev_bf16(d["x"]), dev(d["w"]), dev(d["s"]),
                          dev(d["ids"] if ids is None else ids), dev(d["gw"] if gw is None else gw))
    torch.cuda.synchronize()
    return host_bits(y)


def _check(orc, ql, d, ids=None, gw=None):
    ids = d["ids"] if ids is None else ids
    gw = d["gw"] if gw is None else gw
    y, ye, S = orc.moe_mxfp4(d["x"], d["w"], d["s"], ids, gw)
    return check_float(_run(ql, d, ids, gw), ye, S, d["x"].shape[1])


@pytest.mark.parametrize("M,E,N,K,topk", [(17, 8, 128, 256, 2), (33, 4, 200, 512, 2), (64, 16, 130, 1056, 4),
                                          (100, 64, 256, 512, 6), (257, 8, 64, 320, 8), (40, 1, 96, 128, 1),
                                          (300, 32, 1000, 256, 3),
                                          # many pair tiles per expert
                                          (512, 16, 300, 512, 4), (260, 4, 129, 768, 2)])
def test_moe_prefill_shapes(ql, orc, M, E, N, K, topk):
    d = gen_moe(M, E, N, K, topk, seed=M + E + N)
    _check(orc, ql, d)


@pytest.mark.parametrize("K", [256, 320])
def test_moe_prefill_skewed_routing_and_bad_ids(ql, orc, K):
    # every token routes slot 0 to expert 3 (one expert holds > 64 pairs: several
    # pair tiles), slot 1 spread, slot 2 out of range (-1 and E): contributes nothing
    M, E, N, topk = 150, 12, 192, 3
    d = gen_moe(M, E, N, K, topk, seed=5)
    ids = d["ids"].copy()
    ids[:, 0] = 3
    ids[:, 1] = np.arange(M) % E
    ids[::2, 2] = -1
    ids[1::2, 2] = E
    _check(orc, ql, d, ids=ids)


@pytest.mark.parametrize("K", [128, 256])  # register-staged and direct-to-LDS kernels
@pytest.mark.parametrize("byte,x_exp", [(2, 0), (252, -40)])
def test_moe_prefill_edge_scale_bytes(ql, orc, byte, x_exp, K):
    # the grouped GEMM applies the block scale in the E2M1 -> bf16 convert:
    # exact for scale bytes 2..252 (x scaled so that y stays finite in bf16)
    M, E, N, topk = 20, 2, 64, 2
    d = gen_moe(M, E, N, K, topk, seed=6)
    d["s"][:] = byte
    d["x"] = bf16_bits(bf16_values(d["x"]) * np.float32(2.0 ** x_exp))
    _check(orc, ql, d)


def test_moe_prefill_unaligned_scales_fall_back(ql, orc):
    # scale rows that do not start on a 4-byte boundary cannot use the 4-byte
    # direct loads: the register-staged kernel runs instead, same results
    M, E, N, K, topk = 70, 8, 160, 512, 2
    d = gen_moe(M, E, N, K, topk, seed=9)
    flat = torch.empty(d["s"].size + 1, dtype=torch.uint8, device="cuda")
    flat[1:] = dev(d["s"].reshape(-1))
    s_off = flat[1:].view(E, N, K // 32)
    assert s_off.data_ptr() % 4 == 1
    y = ql.qlin_moe_mxfp4(dev_bf16(d["x"]), dev(d["w"]), s_off, dev(d["ids"]), dev(d["gw"]))
    torch.cuda.synchronize()
    _, ye, S = orc.moe_mxfp4(d["x"], d["w"], d["s"], d["ids"], d["gw"])
    check_float(host_bits(y), ye, S, K)
    check_float(_run(ql, d), ye, S, K)  # the aligned call (direct-to-LDS kernel)


def test_moe_prefill_full_expert_shape(ql, orc):
    # 64 experts of 2048 x 7168, 64 tokens, top-6, compared on every output
    d = gen_moe(64, 64, 2048, 7168, 6, seed=0)
    stats = _check(orc, ql, d)
    assert stats["ref_bits_equal"] > 0.95


def test_moe_prefill_matches_decode_path_per_token(ql):
    # the same tokens through the M <= 16 path (16 at a time) agree to the
    # float rule with the grouped GEMM (both against exact sums)
    d = gen_moe(48, 16, 256, 512, 4, seed=7)
    y_big = bf16_to_f64(_run(ql, d))
    parts = []
    for m0 in range(0, 48, 16):
        sub = {k: (v[m0:m0 + 16] if k in ("x", "ids", "gw") else v) for k, v in d.items()}
        parts.append(bf16_to_f64(_run(ql, sub)))
    y_small = np.concatenate(parts)
    assert np.allclose(y_big, y_small, rtol=2 ** -7, atol=1e-3 * np.abs(y_small).max())


def test_moe_prefill_deterministic(ql):
    d = gen_moe(200, 16, 256, 512, 4, seed=8)
    ref = _run(ql, d)
    for _ in range(10):
        assert np.array_equal(_run(ql, d), ref)
