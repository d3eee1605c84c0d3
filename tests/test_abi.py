"""C-ABI contract tests that need no GPU.

The library must load, export every function include/qlin.h declares, and
reject every invalid argument with the documented status BEFORE anything is
enqueued.  Pointer arguments here are fake, never-dereferenced addresses (a
valid call would reach HIP and is not made on the CPU)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "qlin.h")

A = 0x10000  # 16-byte aligned fake device address, never dereferenced


@pytest.fixture(scope="module")
def q():
    from skinny_gemm_qlin_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from skinny_gemm_qlin_amd import _build
        _build.build()
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z_0-9]*\s*\*?\s*(qlin_[a-z0-9_]+)\s*\(", text, re.M)
    return sorted(set(names))


def test_exports_match_header(q):
    from skinny_gemm_qlin_amd import _lib
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(q, name), f"libqlin.so does not export {name}"


def test_status_strings(q):
    from skinny_gemm_qlin_amd import _lib
    for code in range(0, -8, -1):
        s = _lib.status_str(code)
        assert s.startswith("QLIN_")
    assert _lib.status_str(-99) == "QLIN_ERR_UNKNOWN"
    assert q.qlin_version() >= 100


def test_act_quant_errors(q):
    f = q.qlin_act_quant_i8
    assert f(None, 1024, 1, 1024, A, 1024, A, None) == -1
    assert f(A, 1024, 1, 1024, None, 1024, A, None) == -1
    assert f(A, 1024, 0, 1024, A, 1024, A, None) == -2          # M = 0
    assert f(A, 1024, 16385, 1024, A, 1024, A, None) == -2      # M > QLIN_MAX_M_PREFILL
    assert f(A, 1024, 1, 1000, A, 1024, A, None) == -2          # K % 16
    assert f(A, 1 << 20, 1, 131088, A, 1 << 20, A, None) == -2  # K too large for exact int32
    assert f(A, 512, 1, 1024, A, 1024, A, None) == -3           # ldx < K
    assert f(A, 1024, 1, 1024, A, 1000, A, None) == -3          # ldxq < K
    assert f(A + 2, 1024, 1, 1024, A, 1024, A, None) == -4      # x misaligned
    assert f(A, 1028, 1, 1024, A, 1024, A, None) == -4          # ldx % 8
    assert f(A, 1024, 1, 1024, A + 8, 1024, A, None) == -4
    assert f(A, 1024, 1, 1024, A, 1040 + 8, A, None) == -4      # ldxq % 16
    assert f(A, 1024, 1, 1024, A, 1024, A + 2, None) == -4      # xs misaligned


def test_gemv_i8_errors(q):
    def call(xq=A, ldxq=1024, xs=A, xpt=1, M=1, K=1024, w=A, ldw=1024, N=64, ws=A, wpr=1, bias=None,
             y=A, ldy=64, ok=0):
        return q.qlin_gemv_i8(xq, ldxq, xs, xpt, M, K, w, ldw, N, ws, wpr, bias, y, ldy, ok, None)
    assert call(ok=2) == -6
    assert call(xpt=2) == -6
    assert call(wpr=-1) == -6
    assert call(xq=None) == -1
    assert call(w=None) == -1
    assert call(y=None) == -1
    assert call(xs=None) == -1
    assert call(ws=None) == -1
    assert call(M=0) == -2
    assert call(M=16385) == -2
    assert call(N=0) == -2
    assert call(K=0) == -2
    assert call(K=1032, ldxq=1040, ldw=1040) == -2
    assert call(ldw=1000) == -3
    assert call(ldy=63) == -3
    assert call(ldxq=1008) == -3
    assert call(w=A + 8) == -4
    assert call(ldw=1024 + 8) == -4
    assert call(y=A + 1) == -4
    assert call(bias=A + 1) == -4
    assert call(ok=1, y=A + 2) == -4        # int32 output needs 4-byte alignment


def test_linear_i8_errors(q):
    def call(x=A, ldx=1024, M=1, K=1024, w=A, ldw=1024, N=64, ws=A, wpr=1, bias=None, xq=A, ldxq=1024, xs=A,
             y=A, ldy=64):
        return q.qlin_linear_i8(x, ldx, M, K, w, ldw, N, ws, wpr, bias, xq, ldxq, xs, y, ldy, None)
    assert call(wpr=2) == -6
    for name in ("x", "w", "ws", "xq", "xs", "y"):
        assert call(**{name: None}) == -1
    assert call(M=0) == -2
    assert call(M=16385) == -2
    assert call(N=0) == -2
    assert call(K=1000, ldx=1008, ldxq=1008, ldw=1008) == -2
    assert call(K=131088, ldx=131088, ldxq=131088, ldw=131088) == -2
    assert call(ldx=512) == -3
    assert call(ldxq=1008) == -3
    assert call(ldw=1008) == -3
    assert call(ldy=63) == -3
    assert call(x=A + 2) == -4
    assert call(ldx=1028) == -4
    assert call(xq=A + 8) == -4
    assert call(ldxq=1032) == -4
    assert call(xs=A + 2) == -4
    assert call(w=A + 8) == -4
    assert call(ws=A + 2) == -4
    assert call(y=A + 1) == -4
    assert call(bias=A + 1) == -4


def test_moe_noalloc_errors(q):
    # checked on the host before the library's scratch array is looked up
    def call(x=A, ldx=7168, M=8, K=7168, w=A, s=A, E=64, N=2048, ids=A, gw=A, topk=6, y=A, ldy=2048):
        return q.qlin_moe_mxfp4_noalloc(x, ldx, M, K, w, s, E, N, ids, gw, topk, y, ldy, None)
    for name in ("x", "w", "s", "ids", "gw", "y"):
        assert call(**{name: None}) == -1
    assert call(topk=0) == -2
    assert call(K=7168 + 16, ldx=7184) == -2
    assert call(ldy=100) == -3
    assert call(w=A + 8) == -4
    assert q.qlin_moe_mxfp4_workspace_bytes(16, 8192, 16, 4) > 4 << 20
    assert call(M=16, N=8192, ldy=8192, topk=16, E=4) == -5   # more than the 4 MiB scratch


def test_gemv_fp8_errors(q):
    def call(x=A, ldx=5120, M=1, K=5120, w=A, ldw=5120, N=128, ws=A, wpr=1, y=A, ldy=128):
        return q.qlin_gemv_fp8(x, ldx, M, K, w, ldw, N, ws, wpr, y, ldy, None)
    assert call(wpr=3) == -6
    assert call(ws=None) == -1
    assert call(M=0) == -2
    assert call(M=16385) == -2
    assert call(K=5128, ldx=5136, ldw=5136) == -2
    assert call(ldx=5000) == -3
    assert call(ldx=5124) == -4
    assert call(w=A + 4) == -4
    assert call(ldw=5120 + 4) == -4


def test_act_quant_fp8_errors(q):
    def call(x=A, ldx=1024, M=1, K=1024, fmt=0, pt=1, xq=A, ldxq=1024, xs=A):
        return q.qlin_act_quant_fp8(x, ldx, M, K, fmt, pt, xq, ldxq, xs, None)
    assert call(fmt=2) == -6
    assert call(fmt=-1) == -6
    assert call(pt=2) == -6
    assert call(x=None) == -1
    assert call(xq=None) == -1
    assert call(xs=None) == -1
    assert call(M=0) == -2
    assert call(M=16385) == -2
    assert call(M=17, pt=0) == -2  # the per-tensor scale: one workgroup, M <= 16
    assert call(K=1000) == -2
    assert call(K=(1 << 24) + 16, ldx=(1 << 24) + 16, ldxq=(1 << 24) + 16) == -2
    assert call(ldx=512) == -3
    assert call(ldxq=1000) == -3
    assert call(x=A + 2) == -4
    assert call(ldx=1028) == -4
    assert call(xq=A + 8) == -4
    assert call(ldxq=1032) == -4
    assert call(xs=A + 2) == -4


def test_gemv_fp8_w8a8_errors(q):
    def call(xq=A, ldxq=1024, xs=A, xpt=1, xf=0, M=1, K=1024, w=A, ldw=1024, N=64, ws=A, wpr=1, wf=0,
             y=A, ldy=64):
        return q.qlin_gemv_fp8_w8a8(xq, ldxq, xs, xpt, xf, M, K, w, ldw, N, ws, wpr, wf, y, ldy, None)
    assert call(xf=2) == -6
    assert call(wf=7) == -6
    assert call(xpt=-1) == -6
    assert call(wpr=2) == -6
    for name in ("xq", "xs", "w", "ws", "y"):
        assert call(**{name: None}) == -1
    assert call(M=0) == -2
    assert call(M=16385) == -2
    assert call(N=0) == -2
    assert call(K=8, ldxq=16, ldw=16) == -2
    assert call(K=1032, ldxq=1040, ldw=1040) == -2
    assert call(ldxq=1008) == -3
    assert call(ldw=1008) == -3
    assert call(ldy=63) == -3
    assert call(xq=A + 8) == -4
    assert call(ldxq=1032) == -4
    assert call(w=A + 4) == -4
    assert call(ldw=1024 + 4) == -4
    assert call(xs=A + 1) == -4
    assert call(ws=A + 2) == -4
    assert call(y=A + 1) == -4


def test_gemv_fp8_blk_errors(q):
    def call(x=A, ldx=7168, M=1, K=7168, w=A, ldw=7168, N=256, ws=A, xq=A, xs=A, y=A, ldy=256):
        return q.qlin_gemv_fp8_blk(x, ldx, M, K, w, ldw, N, ws, xq, xs, y, ldy, None)
    assert call(M=2, ldy=256, xq=None) == -1     # more than one token: the codes are needed
    assert call(M=2, xs=None) == -1
    assert call(K=32896, ldx=32896, ldw=32896, xq=None) == -1   # one token past the fused kernel's K
    assert call(ws=None) == -1
    assert call(y=None) == -1
    assert call(K=7168 + 16, ldx=7184, ldw=7184) == -2   # K % 128
    assert call(M=16385) == -2
    assert call(ldw=7000) == -3
    assert call(xq=A + 8) == -4


def test_gemv_fp8_blk_ex_errors(q):
    def call(x=A, ldx=1024, M=1, K=1024, w=A, ldw=1024, N=64, ws=A, bn=1, bk=32, xq=A, xs=A, y=A, ldy=64):
        return q.qlin_gemv_fp8_blk_ex(x, ldx, M, K, w, ldw, N, ws, bn, bk, xq, xs, y, ldy, None)
    for name in ("x", "w", "ws", "xq", "xs", "y"):
        assert call(**{name: None}) == -1
    assert call(bn=0) == -2
    assert call(bk=48) == -2            # block_k % 32
    assert call(bk=16) == -2
    assert call(K=1056, ldx=1056, ldw=1056, bk=64) == -2  # K % block_k
    assert call(M=0) == -2
    assert call(M=16385) == -2
    assert call(K=32800, ldx=32800, ldw=32800) == -2  # K > 32768 for the general shapes
    assert call(ldx=512) == -3
    assert call(ldy=63) == -3
    assert call(x=A + 2) == -4
    assert call(ldw=1024 + 8) == -4
    assert call(bn=128, bk=128, K=1000, ldx=1000, ldw=1000) == -2  # forwarded to qlin_gemv_fp8_blk


def test_moe_errors(q):
    assert q.qlin_moe_mxfp4_workspace_bytes(8, 2048, 6, 64) == 8 * 6 * 2048 * 4
    assert q.qlin_moe_mxfp4_workspace_bytes(1, 3, 1, 1) == 256
    assert q.qlin_moe_mxfp4_workspace_bytes(0, 3, 1, 1) == 0
    need = q.qlin_moe_mxfp4_workspace_bytes(8, 2048, 6, 64)

    def call(x=A, ldx=7168, M=8, K=7168, w=A, s=A, E=64, N=2048, ids=A, gw=A, topk=6, y=A, ldy=2048,
             ws=A, wsb=need):
        return q.qlin_moe_mxfp4(x, ldx, M, K, w, s, E, N, ids, gw, topk, y, ldy, ws, wsb, None)
    assert call(ids=None) == -1
    assert call(gw=None) == -1
    assert call(topk=0) == -2
    assert call(topk=17) == -2
    assert call(E=0) == -2
    assert call(K=7168 + 16, ldx=7184) == -2
    assert call(K=30720 + 32, ldx=30752) == -2   # one staged activation row must fit 64 KiB of LDS
    assert call(ldy=100) == -3
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5
    assert call(ws=A + 4) == -4
    assert call(w=A + 8) == -4
    # prefill (M > 16): the workspace also holds the pair sort (offsets and order)
    big = q.qlin_moe_mxfp4_workspace_bytes(512, 2048, 6, 64)
    part = 512 * 6 * 2048 * 4
    assert big == part + (((2 * 65 + 512 * 6) * 4 + 255) // 256) * 256
    assert call(M=512, wsb=part) == -5
    assert call(M=16385, wsb=big) == -2
    assert call(M=17, E=1025, wsb=q.qlin_moe_mxfp4_workspace_bytes(17, 2048, 6, 1025)) == -2


def test_moe_ffn_errors(q):
    need = q.qlin_moe_ffn_mxfp4_workspace_bytes(8, 7168, 2048, 6, 64)
    assert need == 8 * 64 * 4 + 8 * 6 * 2048 * 2 + 8 * 6 * 7168 * 4  # every region a multiple of 256 here
    assert q.qlin_moe_ffn_mxfp4_workspace_bytes(1, 32, 32, 1, 1) == 256 + 256 + 256
    assert q.qlin_moe_ffn_mxfp4_workspace_bytes(0, 32, 32, 1, 1) == 0

    def call(x=A, ldx=7168, M=8, H=7168, wr=A, E=64, topk=6, w13=A, s13=A, I=2048, w2=A, s2=A,
             alpha=1.0, limit=10.0, ids=A, gw=A, y=A, ldy=7168, ws=A, wsb=need):
        return q.qlin_moe_ffn_mxfp4(x, ldx, M, H, wr, E, topk, w13, s13, I, w2, s2, alpha, limit, ids, gw,
                                    y, ldy, ws, wsb, None)
    assert call(wr=None) == -1
    assert call(s2=None) == -1
    assert call(ids=None) == -1
    assert call(M=0) == -2
    assert call(M=17) == -2
    assert call(E=1025) == -2
    assert call(topk=17) == -2
    assert call(E=4, topk=5) == -2           # more slots than experts
    assert call(H=7168 + 16, ldx=7184, ldy=7184) == -2
    assert call(I=30720 + 32) == -2
    assert call(ldx=7000) == -3
    assert call(ldy=100) == -3
    assert call(x=A + 8) == -4
    assert call(wr=A + 2) == -4
    assert call(ws=None) == -5
    assert call(wsb=need - 1) == -5
