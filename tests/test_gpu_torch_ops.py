"""PyTorch integration on the GPU: every qlin custom operator passes
torch.library.opcheck (schema, fake-vs-real, dispatch), and a layer built
from them gives bit-identical results eagerly, through torch.compile
(dynamo + AOT dispatch, fullgraph) and through the plain binding, with the
hit counters showing that the compiled graph ran each HIP kernel."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, lib, need_gpu
from skinny_gemm_qlin_amd.inputs import gen_fp8, gen_fp8_blk, gen_fp8_w8a8, gen_int8, gen_moe, gen_moe_ffn

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


@pytest.fixture(scope="module")
def args(ql):
    d8 = gen_int8(4, 256, 1024, seed=1)
    df = gen_fp8(3, 256, 1024, seed=2)
    db = gen_fp8_blk(5, 256, 1024, seed=3)
    dm = gen_moe(4, 8, 128, 512, 2, seed=4)
    dn = gen_moe_ffn(4, 8, 256, 64, 2, seed=5)
    dw = gen_fp8_w8a8(6, 256, 1024, w_fmt=1, seed=6)
    dx = gen_fp8_blk(3, 256, 1024, seed=7, block_n=1, block_k=32)
    return {
        "gemv_fp8_blk_ex": (dev_bf16(dx["x"]), dev(dx["w"]), dev(dx["ws"]), 1, 32),
        "linear_fp8_w8a8": (dev_bf16(dw["x"]), dev(dw["w"]), dev(dw["ws"]), 0, 1, True),
        "linear_i8": (dev_bf16(d8["x"]), dev(d8["w"]), dev(d8["ws"])),
        "gemv_fp8": (dev_bf16(df["x"]), dev(df["w"]), dev(df["ws"])),
        "gemv_fp8_blk": (dev_bf16(db["x"]), dev(db["w"]), dev(db["ws"])),
        "moe_mxfp4": (dev_bf16(dm["x"]), dev(dm["w"]), dev(dm["s"]), dev(dm["ids"]), dev(dm["gw"])),
        "moe_ffn_mxfp4": (dev_bf16(dn["x"]), dev_bf16(dn["wr"]), dev(dn["w13"]), dev(dn["s13"]), dev(dn["w2"]),
                          dev(dn["s2"]), 2),
    }


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_opcheck_every_operator(ql, args):
    import skinny_gemm_qlin_amd.torch_ops  # noqa: F401
    x8, w8, ws8 = args["linear_i8"]
    xq, xs = torch.ops.qlin.act_quant_i8(x8)
    xw, ww, wsw = args["linear_fp8_w8a8"][:3]
    xq8, xs8 = torch.ops.qlin.act_quant_fp8(xw, 0, True)
    cases = [(torch.ops.qlin.act_quant_i8.default, (x8,)),
             (torch.ops.qlin.act_quant_fp8.default, (xw, 1, False)),
             (torch.ops.qlin.gemv_fp8_w8a8.default, (xq8, xs8, ww, wsw, 0, 1)),
             (torch.ops.qlin.linear_fp8_w8a8.default, args["linear_fp8_w8a8"]),
             (torch.ops.qlin.gemv_i8.default, (xq, xs, w8, ws8)),
             (torch.ops.qlin.linear_i8.default, args["linear_i8"]),
             (torch.ops.qlin.gemv_fp8.default, args["gemv_fp8"]),
             (torch.ops.qlin.gemv_fp8_blk.default, args["gemv_fp8_blk"]),
             (torch.ops.qlin.gemv_fp8_blk_ex.default, args["gemv_fp8_blk_ex"]),
             (torch.ops.qlin.moe_mxfp4.default, args["moe_mxfp4"]),
             (torch.ops.qlin.moe_ffn_mxfp4.default, args["moe_ffn_mxfp4"])]
    for op, a in cases:
        torch.library.opcheck(op, a)


def test_compiled_layer_equals_eager_and_reaches_every_kernel(ql, args):
    import skinny_gemm_qlin_amd.torch_ops as tops

    def layer(a8, af, ab, am, an, aw):
        r0 = torch.ops.qlin.linear_i8(*a8)
        r1 = torch.ops.qlin.gemv_fp8(*af)
        r2 = torch.ops.qlin.gemv_fp8_blk(*ab)
        r3 = torch.ops.qlin.moe_mxfp4(*am)
        y, ids, gw = torch.ops.qlin.moe_ffn_mxfp4(*an)
        r4 = torch.ops.qlin.linear_fp8_w8a8(*aw)
        return r0, r1, r2, r3, y, ids, gw, r4

    a = (args["linear_i8"], args["gemv_fp8"], args["gemv_fp8_blk"], args["moe_mxfp4"], args["moe_ffn_mxfp4"],
         args["linear_fp8_w8a8"])
    eager = layer(*a)
    torch.cuda.synchronize()

    # the plain binding gives the same bits
    x8, w8, ws8 = args["linear_i8"]
    xq, xs = ql.qlin_act_quant_i8(x8)
    ref = [ql.qlin_gemv_i8(xq, xs, w8, ws8), ql.qlin_gemv_fp8(*args["gemv_fp8"]),
           ql.qlin_gemv_fp8_blk(*args["gemv_fp8_blk"])[0], ql.qlin_moe_mxfp4(*args["moe_mxfp4"]),
           *ql.qlin_moe_ffn_mxfp4(*args["moe_ffn_mxfp4"])]
    xw, ww, wsw, xf, wf, pt = args["linear_fp8_w8a8"]
    ref.append(ql.qlin_gemv_fp8_w8a8(*ql.qlin_act_quant_fp8(xw, xf, pt), ww, wsw, xf, wf))
    torch.cuda.synchronize()
    for e, r in zip(eager, ref):
        assert torch.equal(_bits(e), _bits(r))

    compiled = torch.compile(layer, backend="aot_eager", fullgraph=True)
    compiled(*a)  # compile
    torch.cuda.synchronize()
    tops.reset_hits()
    for _ in range(3):
        out = compiled(*a)
        torch.cuda.synchronize()
        for e, c in zip(eager, out):
            assert torch.equal(_bits(e), _bits(c))
    assert dict(tops.hits) == {"linear_i8": 3, "gemv_fp8": 3, "gemv_fp8_blk": 3, "moe_mxfp4": 3,
                               "moe_ffn_mxfp4": 3, "linear_fp8_w8a8": 3}


def test_one_dynamic_graph_serves_every_M(ql):
    # compiled once with M as an unbacked (fully dynamic) size, the graph is
    # reused down to M = 1 and up to M = 16: the operator dispatches on M
    # inside its opaque body.  (A merely dynamic size would still be
    # specialised at 1 by the compiler's own rule.)
    import torch._dynamo
    import skinny_gemm_qlin_amd.torch_ops as tops
    d = gen_int8(16, 256, 1024, seed=11)
    x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])

    def f(xm):
        return torch.ops.qlin.linear_i8(xm, w, ws)

    torch._dynamo.reset()
    compiled = torch.compile(f, backend="aot_eager", dynamic=True, fullgraph=True)
    frames = torch._dynamo.utils.counters["stats"]["unique_graphs"]
    tops.reset_hits()
    for M in (3, 1, 16, 8, 2):
        xm = x[:M]
        torch._dynamo.decorators.mark_unbacked(xm, 0)
        got = compiled(xm)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), f(x[:M]).view(torch.int16))
    assert torch._dynamo.utils.counters["stats"]["unique_graphs"] - frames == 1
    assert tops.hits["linear_i8"] == 10
