"""The entry points keep no state between calls (qlin.h: stateless and
thread-safe; qlin_moe_mxfp4_noalloc excepted): calls running at the same time
on different streams, issued from different host threads, give the same bits
as the same calls run one at a time."""
import threading

import numpy as np
import pytest
import torch

from gpu_util import dev, dev_bf16, lib, need_gpu
from skinny_gemm_qlin_amd.inputs import gen_fp8, gen_fp8_blk, gen_int8, gen_moe

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ql():
    need_gpu()
    return lib()


def _jobs(ql):
    """(name, fn(stream) -> tuple of output tensors); every job its own inputs."""
    jobs = []
    for i, M in enumerate((1, 2, 5, 16)):
        d = gen_int8(M, 3000 + 16 * i, 4096, seed=300 + i)
        x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
        jobs.append((f"linear_i8 M={M}", lambda s, x=x, w=w, ws=ws: ql.qlin_linear_i8(x, w, ws, stream=s)))
    for i, M in enumerate((1, 8)):
        d = gen_fp8(M, 2048, 5120, seed=310 + i)
        x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
        jobs.append((f"gemv_fp8 M={M}", lambda s, x=x, w=w, ws=ws: (ql.qlin_gemv_fp8(x, w, ws, stream=s),)))
    for i, M in enumerate((1, 16)):
        d = gen_fp8_blk(M, 1024, 7168, seed=320 + i)
        x, w, ws = dev_bf16(d["x"]), dev(d["w"]), dev(d["ws"])
        jobs.append((f"gemv_fp8_blk M={M}", lambda s, x=x, w=w, ws=ws: ql.qlin_gemv_fp8_blk(x, w, ws, stream=s)))
    d = gen_moe(8, 16, 512, 2048, 6, seed=330)
    x, w, sc, ids, gw = dev_bf16(d["x"]), dev(d["w"]), dev(d["s"]), dev(d["ids"]), dev(d["gw"])
    jobs.append(("moe_mxfp4 M=8", lambda s: (ql.qlin_moe_mxfp4(x, w, sc, ids, gw, stream=s),)))
    return jobs


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def test_concurrent_streams_and_threads(ql):
    jobs = _jobs(ql)
    ref = []
    for name, fn in jobs:
        out = fn(None)
        torch.cuda.synchronize()
        ref.append([_bits(t).clone() for t in out])
    streams = [torch.cuda.Stream() for _ in jobs]
    got = [None] * len(jobs)

    def run(i):
        name, fn = jobs[i]
        with torch.cuda.stream(streams[i]):
            outs = []
            for _ in range(8):  # several calls in flight per stream
                outs.append(fn(streams[i]))
            got[i] = outs

    for rnd in range(3):
        print(f"concurrent round {rnd}", flush=True)
        threads = [threading.Thread(target=run, args=(i,)) for i in range(len(jobs))]
        for th in threads:
            th.start()
        for th in threads:
            th.join()
        torch.cuda.synchronize()
        for i, (name, _) in enumerate(jobs):
            for out in got[i]:
                for a, b in zip(out, ref[i]):
                    assert torch.equal(_bits(a), b), f"{name}: differs when run concurrently"
