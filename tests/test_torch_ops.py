"""PyTorch integration without a GPU: the qlin custom operators register,
their fake (meta) implementations give the right output shapes and dtypes,
and a traced graph keeps every operator as one opaque node (the compiler
cannot replace the kernel by a decomposition)."""
import pytest
import torch
from torch._subclasses.fake_tensor import FakeTensorMode
from torch.fx.experimental.proxy_tensor import make_fx

import skinny_gemm_qlin_amd.torch_ops  # noqa: F401  (registers torch.ops.qlin.*)


def _inputs(M=3, N=256, K=512, E=8, H=256, I=64):
    return {
        "x": torch.empty((M, K), dtype=torch.bfloat16),
        "xq": torch.empty((M, K), dtype=torch.int8),
        "xs": torch.empty((M,), dtype=torch.float32),
        "w8": torch.empty((N, K), dtype=torch.int8),
        "wf8": torch.empty((N, K), dtype=torch.uint8),
        "ws": torch.empty((N,), dtype=torch.float32),
        "wsb": torch.empty(((N + 127) // 128, K // 128), dtype=torch.uint8),
        "wsmx": torch.empty((N, K // 32), dtype=torch.uint8),
        "wm": torch.empty((E, N, K // 2), dtype=torch.uint8),
        "sm": torch.empty((E, N, K // 32), dtype=torch.uint8),
        "ids": torch.empty((M, 2), dtype=torch.int32),
        "gw": torch.empty((M, 2), dtype=torch.float32),
        "xh": torch.empty((M, H), dtype=torch.bfloat16),
        "wr": torch.empty((E, H), dtype=torch.bfloat16),
        "w13": torch.empty((E, 2 * I, H // 2), dtype=torch.uint8),
        "s13": torch.empty((E, 2 * I, H // 32), dtype=torch.uint8),
        "w2": torch.empty((E, H, I // 2), dtype=torch.uint8),
        "s2": torch.empty((E, H, I // 32), dtype=torch.uint8),
    }


def test_fake_shapes_and_dtypes():
    with FakeTensorMode() as mode:
        d = {k: mode.from_tensor(v) for k, v in _inputs().items()}
        xq, xs = torch.ops.qlin.act_quant_i8(d["x"])
        assert xq.shape == (3, 512) and xq.dtype == torch.int8 and xs.shape == (3,) and xs.dtype == torch.float32
        for y in (torch.ops.qlin.gemv_i8(d["xq"], d["xs"], d["w8"], d["ws"]),
                  torch.ops.qlin.linear_i8(d["x"], d["w8"], d["ws"]),
                  torch.ops.qlin.gemv_fp8(d["x"], d["wf8"], d["ws"]),
                  torch.ops.qlin.gemv_fp8_blk(d["x"], d["wf8"], d["wsb"]),
                  torch.ops.qlin.gemv_fp8_blk_ex(d["x"], d["wf8"], d["wsmx"], 1, 32),
                  torch.ops.qlin.moe_mxfp4(d["x"], d["wm"], d["sm"], d["ids"], d["gw"])):
            assert y.shape == (3, 256) and y.dtype == torch.bfloat16
        for fmt in (0, 1):
            for per_token, ns in ((True, 3), (False, 1)):
                xq8, xs8 = torch.ops.qlin.act_quant_fp8(d["x"], fmt, per_token)
                assert xq8.shape == (3, 512) and xq8.dtype == torch.uint8
                assert xs8.shape == (ns,) and xs8.dtype == torch.float32
        for y in (torch.ops.qlin.gemv_fp8_w8a8(d["wf8"][:3], d["xs"], d["wf8"], d["ws"], 1, 0),
                  torch.ops.qlin.linear_fp8_w8a8(d["x"], d["wf8"], d["ws"], 0, 1, False)):
            assert y.shape == (3, 256) and y.dtype == torch.bfloat16
        y, ids, gw = torch.ops.qlin.moe_ffn_mxfp4(d["xh"], d["wr"], d["w13"], d["s13"], d["w2"], d["s2"], 2)
        assert y.shape == (3, 256) and y.dtype == torch.bfloat16
        assert ids.shape == (3, 2) and ids.dtype == torch.int32 and gw.shape == (3, 2) and gw.dtype == torch.float32


def test_traced_graph_keeps_the_operators_opaque():
    d = _inputs()

    def layer(x, w8, ws, wf8, wsb):
        return torch.ops.qlin.linear_i8(x, w8, ws) + torch.ops.qlin.gemv_fp8(x, wf8, ws) \
            + torch.ops.qlin.gemv_fp8_blk(x, wf8, wsb) + torch.ops.qlin.linear_fp8_w8a8(x, wf8, ws)

    g = make_fx(layer, tracing_mode="fake")(d["x"], d["w8"], d["ws"], d["wf8"], d["wsb"])
    targets = [str(n.target) for n in g.graph.nodes if n.op == "call_function"]
    assert "qlin.linear_i8.default" in targets
    assert "qlin.gemv_fp8.default" in targets
    assert "qlin.gemv_fp8_blk.default" in targets
    assert "qlin.linear_fp8_w8a8.default" in targets
    # nothing else computes the products: only the three adds remain
    assert sorted(t for t in targets if not t.startswith("qlin.")) == ["aten.add.Tensor"] * 3
