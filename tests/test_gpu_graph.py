"""HIP graph capture and replay of every entry point.  Each call is captured
once on preallocated buffers, then the graph is replayed several times with
new inputs copied into the captured input buffers, with eager work and
synchronisations between the replays; every replay must equal an eager call
on the same inputs bit for bit (the kernels are deterministic and the
captured launches are the eager ones).  No entry point records a memset or
allocates, so nothing but kernels is captured."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, lib, need_gpu
from skinny_gemm_qlin_amd.inputs import (gen_fp8, gen_fp8_blk, gen_fp8_w8a8, gen_int8, gen_moe, gen_moe_ffn)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _bits(t):
    return t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def _check_replays(step, inputs, feeds):
    """step() launches the call(s) on the tensors in `inputs` and returns the
    (preallocated) output tensors; feeds: dicts of new values for `inputs`."""
    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for feed in feeds:
        for k, v in feed.items():
            inputs[k].copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        eager = [o.clone() for o in step()]
        torch.cuda.synchronize()
        for a, b in zip(got, eager):
            assert torch.equal(_bits(a), _bits(b))


def _xfeeds(gen, n=3):
    return [{"x": dev_bf16(gen(seed)["x"])} for seed in range(100, 100 + n)]


@pytest.mark.parametrize("M", [1, 16, 100])
def test_graph_int8(ql, M):
    N, K = 512, 1024
    d = gen_int8(M, N, K, seed=1)
    inp = {"x": dev_bf16(d["x"])}
    w, ws = dev(d["w"]), dev(d["ws"])
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ql.qlin_act_quant_i8(inp["x"], xq=xq, xs=xs)
        ql.qlin_gemv_i8(xq, xs, w, ws, y=y)
        return [xq, xs, y]
    _check_replays(step, inp, _xfeeds(lambda s: gen_int8(M, N, K, seed=s)))


@pytest.mark.parametrize("M", [1, 8, 300])
def test_graph_fp8(ql, M):
    N, K = 512, 1024
    d = gen_fp8(M, N, K, seed=2)
    inp = {"x": dev_bf16(d["x"])}
    w, ws = dev(d["w"]), dev(d["ws"])
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ql.qlin_gemv_fp8(inp["x"], w, ws, y=y)
        return [y]
    _check_replays(step, inp, _xfeeds(lambda s: gen_fp8(M, N, K, seed=s)))


@pytest.mark.parametrize("M", [2, 40])
def test_graph_fp8_w8a8(ql, M):
    N, K = 384, 1024
    d = gen_fp8_w8a8(M, N, K, seed=3)
    inp = {"x": dev_bf16(d["x"])}
    w, ws = dev(d["w"]), dev(d["ws"])
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ql.qlin_act_quant_fp8(inp["x"], 0, True, xq=xq, xs=xs)
        ql.qlin_gemv_fp8_w8a8(xq, xs, w, ws, 0, 0, y=y)
        return [xq, xs, y]
    _check_replays(step, inp, _xfeeds(lambda s: gen_fp8_w8a8(M, N, K, seed=s)))


@pytest.mark.parametrize("M,bn,bk", [(1, 128, 128), (8, 128, 128), (64, 128, 128), (3, 1, 32), (40, 1, 32)])
def test_graph_fp8_blk(ql, M, bn, bk):
    N, K = 256, 1024
    d = gen_fp8_blk(M, N, K, seed=4, block_n=bn, block_k=bk)
    inp = {"x": dev_bf16(d["x"])}
    w, ws = dev(d["w"]), dev(d["ws"])
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // bk), dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ql.qlin_gemv_fp8_blk_ex(inp["x"], w, ws, bn, bk, xq=xq, xs=xs, y=y)
        return [xq, xs, y]
    _check_replays(step, inp, _xfeeds(lambda s: gen_fp8_blk(M, N, K, seed=s, block_n=bn, block_k=bk)))


@pytest.mark.parametrize("M", [8, 64])
def test_graph_moe(ql, M):
    E, N, K, topk = 16, 256, 512, 4
    d = gen_moe(M, E, N, K, topk, seed=5)
    inp = {"x": dev_bf16(d["x"]), "ids": dev(d["ids"]), "gw": dev(d["gw"])}
    w, s = dev(d["w"]), dev(d["s"])
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((ql.qlin_moe_mxfp4_workspace_bytes(M, N, topk, E),), dtype=torch.uint8, device="cuda")

    def step():
        ql.qlin_moe_mxfp4(inp["x"], w, s, inp["ids"], inp["gw"], y=y, workspace=ws)
        return [y]
    feeds = []
    for seed in (200, 201, 202):  # new tokens and a new routing each replay
        e = gen_moe(M, E, N, K, topk, seed=seed)
        feeds.append({"x": dev_bf16(e["x"]), "ids": dev(e["ids"]), "gw": dev(e["gw"])})
    _check_replays(step, inp, feeds)


def test_graph_moe_ffn(ql):
    M, E, H, I, topk = 4, 8, 256, 128, 2
    d = gen_moe_ffn(M, E, H, I, topk, seed=6)
    inp = {"x": dev_bf16(d["x"])}
    t = {k: dev(d[k]) for k in ("w13", "s13", "w2", "s2")}
    wr = dev_bf16(d["wr"])
    y = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((M, topk), dtype=torch.int32, device="cuda")
    gw = torch.empty((M, topk), dtype=torch.float32, device="cuda")
    ws = torch.empty((ql.qlin_moe_ffn_mxfp4_workspace_bytes(M, H, I, topk, E),), dtype=torch.uint8, device="cuda")

    def step():
        ql.qlin_moe_ffn_mxfp4(inp["x"], wr, t["w13"], t["s13"], t["w2"], t["s2"], topk, y=y, workspace=ws,
                              ids=ids, gw=gw)
        return [y, ids, gw]
    _check_replays(step, inp, _xfeeds(lambda s: gen_moe_ffn(M, E, H, I, topk, seed=s)))


@pytest.mark.parametrize("M", [1, 4])
def test_graph_linear_i8(ql, M):
    # the one-call INT8 layer: one fused kernel at M = 1, quantiser + GEMV above
    N, K = 512, 1024
    d = gen_int8(M, N, K, seed=7)
    inp = {"x": dev_bf16(d["x"])}
    w, ws = dev(d["w"]), dev(d["ws"])
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ql.qlin_linear_i8(inp["x"], w, ws, xq=xq, xs=xs, y=y)
        return [xq, xs, y]
    _check_replays(step, inp, _xfeeds(lambda s: gen_int8(M, N, K, seed=s)))


def test_graph_fp8_blk_one_token_without_export(ql):
    # one token, no code / scale buffers (NULL): the fused kernel alone
    N, K = 512, 2048
    d = gen_fp8_blk(1, N, K, seed=8)
    inp = {"x": dev_bf16(d["x"])}
    w, ws = dev(d["w"]), dev(d["ws"])
    y = torch.empty((1, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ql.qlin_gemv_fp8_blk(inp["x"], w, ws, y=y, export=False)
        return [y]
    _check_replays(step, inp, _xfeeds(lambda s: gen_fp8_blk(1, N, K, seed=s)))


def test_graph_moe_noalloc(ql):
    # the entry point that allocates nothing (its workspace is the library's
    # static per-GPU array): captured like the others
    M, E, N, K, topk = 8, 16, 256, 512, 4
    d = gen_moe(M, E, N, K, topk, seed=9)
    inp = {"x": dev_bf16(d["x"]), "ids": dev(d["ids"]), "gw": dev(d["gw"])}
    w, s = dev(d["w"]), dev(d["s"])
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def step():
        ql.qlin_moe_mxfp4_noalloc(inp["x"], w, s, inp["ids"], inp["gw"], y)
        return [y]
    feeds = []
    for seed in (210, 211, 212):
        e = gen_moe(M, E, N, K, topk, seed=seed)
        feeds.append({"x": dev_bf16(e["x"]), "ids": dev(e["ids"]), "gw": dev(e["gw"])})
    _check_replays(step, inp, feeds)
