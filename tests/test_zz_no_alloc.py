"""GPU test of qlin_moe_mxfp4_noalloc, the MXFP4 expert GEMV entry point that
takes its workspace from the library's per-GPU scratch array instead of a
caller buffer.  Its outputs must equal qlin_moe_mxfp4's (same kernels) bit for
bit, on consecutive calls whose sizes shrink (the scratch keeps the previous
call's contents), and match the CPU oracle under the float rules."""
import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, host_bits, lib, need_gpu
from oracle.compare import check_float
from skinny_gemm_qlin_amd.inputs import gen_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _both(ql, d):
    args = (dev_bf16(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["ids"]), dev(d["gw"]))
    M, N = d["x"].shape[0], d["w"].shape[1]
    y_ref = ql.qlin_moe_mxfp4(*args)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = ql.qlin_moe_mxfp4_noalloc(*args, y)
    torch.cuda.synchronize()
    assert out is y
    return host_bits(y), host_bits(y_ref)


@pytest.mark.parametrize("sizes", [
    # (M, E, N, K, topk, seed): the MXFP4 expert workload, then a smaller call
    [(8, 64, 2048, 7168, 6, 0), (3, 16, 512, 1024, 4, 1)],
    # more than 16 tokens (the grouped prefill path keeps its pair sort in the
    # scratch too), then the decode path
    [(40, 32, 1024, 2048, 6, 2), (5, 8, 256, 512, 2, 3)],
])
def test_noalloc_equals_workspace_entry_point(ql, orc, sizes):
    for (M, E, N, K, topk, seed) in sizes:
        print(f"noalloc: M={M} E={E} N={N} K={K} topk={topk} seed={seed}", flush=True)
        d = gen_moe(M, E, N, K, topk, seed=seed)
        y, y_ref = _both(ql, d)
        assert np.array_equal(y, y_ref), f"M={M}: differs from qlin_moe_mxfp4"
        _, ye, S = orc.moe_mxfp4(d["x"], d["w"], d["s"], d["ids"], d["gw"])
        check_float(y, ye, S, K, f"noalloc M={M}")


def test_noalloc_rejects_oversized_workspace(ql):
    # M * topk * N * 4 = 8 MiB > the 4 MiB scratch: host-side error, output untouched
    M, E, N, K, topk = 16, 4, 8192, 64, 16
    assert ql.qlin_moe_mxfp4_workspace_bytes(M, N, topk, E) > ql.QLIN_NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((E, N, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.full((E, N, K // 32), 127, dtype=torch.uint8, device="cuda")
    ids = torch.zeros((M, topk), dtype=torch.int32, device="cuda")
    gw = torch.ones((M, topk), dtype=torch.float32, device="cuda")
    y = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ql.QlinError) as ei:
        ql.qlin_moe_mxfp4_noalloc(x, w, s, ids, gw, y)
    assert ei.value.status == -5
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
