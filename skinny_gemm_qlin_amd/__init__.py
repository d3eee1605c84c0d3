"""skinny_gemm_qlin_amd -- weight-quantized decode GEMV for MI355X (gfx950).

Thin torch-facing binding of the C ABI in include/qlin.h (libqlin.so).  The
functions carry the C names and only marshal arguments: they check dtype,
device and that the innermost dimension is contiguous, pass data pointers,
row pitches and torch's current HIP stream, and raise QlinError on a non-zero
status.  Outputs that are not supplied are allocated with torch (device
memory plumbing only).  Every arithmetic step runs in the HIP kernels.

Storage conventions: bf16 tensors are torch.bfloat16; int8 codes are
torch.int8; E4M3 codes, UE8M0 scale bytes and packed E2M1 nibbles are
torch.uint8 (a torch.float8_e4m3fn tensor may be passed for E4M3 codes).
"""
from __future__ import annotations

import torch

from ._lib import QLIN_FMT_E4M3, QLIN_FMT_E5M2, QlinError, check, load, status_str  # noqa: F401

__all__ = [
    "QlinError", "qlin_act_quant_i8", "qlin_gemv_i8", "qlin_linear_i8", "qlin_gemv_fp8", "qlin_gemv_fp8_blk",
    "qlin_act_quant_fp8", "qlin_gemv_fp8_w8a8", "QLIN_FMT_E4M3", "QLIN_FMT_E5M2", "qlin_gemv_fp8_blk_ex",
    "qlin_moe_mxfp4", "qlin_moe_mxfp4_workspace_bytes", "qlin_moe_mxfp4_noalloc", "status_str",
]


def _stream(t: torch.Tensor, stream):
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _need(t: torch.Tensor, name: str, dtypes, dims: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor, got {t.device}")
    if t.dim() != dims:
        raise ValueError(f"{name}: expected {dims} dims, got shape {tuple(t.shape)}")
    if dims >= 1 and t.numel() > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name}: innermost dimension must be contiguous (stride {t.stride(-1)})")
    return t


_U8 = (torch.uint8, torch.float8_e4m3fn)


def qlin_act_quant_i8(x, xq=None, xs=None, stream=None):
    """Per-token INT8 quantisation of bf16 x [M, K] -> (xq int8 [M, K], xs fp32 [M])."""
    _need(x, "x", (torch.bfloat16,), 2)
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    _need(xq, "xq", (torch.int8,), 2)
    _need(xs, "xs", (torch.float32,), 1)
    check(load().qlin_act_quant_i8(x.data_ptr(), x.stride(0), M, K, xq.data_ptr(), xq.stride(0),
                                   xs.data_ptr(), _stream(x, stream)), "qlin_act_quant_i8")
    return xq, xs


def qlin_gemv_i8(xq, xs, w, ws, bias=None, y=None, out_kind=0, stream=None):
    """W8A8 GEMV: xq int8 [M, K], xs fp32 [M] or [1], w int8 [N, K] (row pitch
    w.stride(0)), ws fp32 [N] or [1], bias bf16 [N] or None.  out_kind 0 ->
    y bf16 [M, N]; out_kind 1 -> y int32 [M, N] holding the raw accumulators."""
    _need(xq, "xq", (torch.int8,), 2)
    _need(w, "w", (torch.int8,), 2)
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w has K={w.shape[1]}, xq has K={K}")
    _need(xs, "xs", (torch.float32,), 1)
    _need(ws, "ws", (torch.float32,), 1)
    if bias is not None:
        _need(bias, "bias", (torch.bfloat16,), 1)
    if y is None:
        y = torch.empty((M, N), dtype=torch.int32 if out_kind == 1 else torch.bfloat16, device=xq.device)
    _need(y, "y", (torch.int32,) if out_kind == 1 else (torch.bfloat16,), 2)
    check(load().qlin_gemv_i8(xq.data_ptr(), xq.stride(0), xs.data_ptr(), int(xs.numel() > 1), M, K,
                              w.data_ptr(), w.stride(0), N, ws.data_ptr(), int(ws.numel() > 1),
                              None if bias is None else bias.data_ptr(), y.data_ptr(), y.stride(0),
                              int(out_kind), _stream(xq, stream)), "qlin_gemv_i8")
    return y


def qlin_linear_i8(x, w, ws, bias=None, xq=None, xs=None, y=None, stream=None):
    """The whole INT8 decode linear layer in one call: per-token quantisation of
    bf16 x [M, K] (codes and scales into xq int8 [M, K] / xs fp32 [M]) and the
    W8A8 GEMV with its bf16 epilogue.  One kernel for one token.
    Returns (y bf16 [M, N], xq, xs)."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.int8,), 2)
    _need(ws, "ws", (torch.float32,), 1)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w has K={w.shape[1]}, x has K={K}")
    if bias is not None:
        _need(bias, "bias", (torch.bfloat16,), 1)
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if xs is None:
        xs = torch.empty((M,), dtype=torch.float32, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(xq, "xq", (torch.int8,), 2)
    _need(xs, "xs", (torch.float32,), 1)
    _need(y, "y", (torch.bfloat16,), 2)
    check(load().qlin_linear_i8(x.data_ptr(), x.stride(0), M, K, w.data_ptr(), w.stride(0), N, ws.data_ptr(),
                                int(ws.numel() > 1), None if bias is None else bias.data_ptr(), xq.data_ptr(),
                                xq.stride(0), xs.data_ptr(), y.data_ptr(), y.stride(0), _stream(x, stream)),
          "qlin_linear_i8")
    return y, xq, xs


def qlin_gemv_fp8(x, w, ws, y=None, stream=None):
    """E4M3 weight-only GEMV: x bf16 [M, K], w E4M3 codes [N, K], ws fp32 [N] or [1]."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", _U8, 2)
    _need(ws, "ws", (torch.float32,), 1)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w has K={w.shape[1]}, x has K={K}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", (torch.bfloat16,), 2)
    check(load().qlin_gemv_fp8(x.data_ptr(), x.stride(0), M, K, w.data_ptr(), w.stride(0), N,
                               ws.data_ptr(), int(ws.numel() > 1), y.data_ptr(), y.stride(0),
                               _stream(x, stream)), "qlin_gemv_fp8")
    return y


_FP8_DT = {QLIN_FMT_E4M3: torch.float8_e4m3fn, QLIN_FMT_E5M2: torch.float8_e5m2}


def _codes(t: torch.Tensor, name: str, fmt: int) -> torch.Tensor:
    """FP8 codes as stored: torch.uint8, or the float8 dtype of the format."""
    if fmt not in _FP8_DT:
        raise ValueError(f"{name}: unknown FP8 format {fmt}")
    _need(t, name, (torch.uint8, _FP8_DT[fmt]), 2)
    return t


def qlin_act_quant_fp8(x, fmt=QLIN_FMT_E4M3, per_token=True, xq=None, xs=None, stream=None):
    """Dynamic FP8 quantisation of bf16 x [M, K] -> (xq uint8 codes [M, K] of
    format fmt, xs fp32 [M] (per_token) or [1])."""
    _need(x, "x", (torch.bfloat16,), 2)
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((M if per_token else 1,), dtype=torch.float32, device=x.device)
    _codes(xq, "xq", fmt)
    _need(xs, "xs", (torch.float32,), 1)
    if xs.numel() < (M if per_token else 1):
        raise ValueError(f"xs holds {xs.numel()} scales, needs {M if per_token else 1}")
    check(load().qlin_act_quant_fp8(x.data_ptr(), x.stride(0), M, K, int(fmt), int(bool(per_token)),
                                    xq.data_ptr(), xq.stride(0), xs.data_ptr(), _stream(x, stream)),
          "qlin_act_quant_fp8")
    return xq, xs


def qlin_gemv_fp8_w8a8(xq, xs, w, ws, x_fmt=QLIN_FMT_E4M3, w_fmt=QLIN_FMT_E4M3, y=None, stream=None):
    """FP8 W8A8 GEMV: xq codes [M, K] (format x_fmt), xs fp32 [M] or [1], w codes
    [N, K] (format w_fmt, row pitch w.stride(0)), ws fp32 [N] or [1] -> y bf16 [M, N]."""
    _codes(xq, "xq", x_fmt)
    _codes(w, "w", w_fmt)
    _need(xs, "xs", (torch.float32,), 1)
    _need(ws, "ws", (torch.float32,), 1)
    M, K = xq.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w has K={w.shape[1]}, xq has K={K}")
    if xs.numel() not in (1, M) or ws.numel() not in (1, N):
        raise ValueError(f"xs must hold 1 or M={M} scales, ws 1 or N={N}")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _need(y, "y", (torch.bfloat16,), 2)
    check(load().qlin_gemv_fp8_w8a8(xq.data_ptr(), xq.stride(0), xs.data_ptr(), int(xs.numel() > 1),
                                    int(x_fmt), M, K, w.data_ptr(), w.stride(0), N, ws.data_ptr(),
                                    int(ws.numel() > 1), int(w_fmt), y.data_ptr(), y.stride(0),
                                    _stream(xq, stream)), "qlin_gemv_fp8_w8a8")
    return y


def qlin_gemv_fp8_blk(x, w, ws, xq=None, xs=None, y=None, stream=None, export=True):
    """Block-scaled FP8: x bf16 [M, K], w E4M3 [N, K], ws UE8M0 [ceil(N/128), K/128].
    Returns (y bf16 [M, N], xq E4M3 [M, K], xs UE8M0 [M, K/128]).  export=False
    passes NULL code / scale buffers (accepted for one token, K <= 32768) and
    returns (y, None, None)."""
    if not export:
        _need(x, "x", (torch.bfloat16,), 2)
        if y is None:
            y = torch.empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16, device=x.device)
        check(load().qlin_gemv_fp8_blk(x.data_ptr(), x.stride(0), x.shape[0], x.shape[1], w.data_ptr(),
                                       w.stride(0), w.shape[0], ws.data_ptr(), None, None, y.data_ptr(),
                                       y.stride(0), _stream(x, stream)), "qlin_gemv_fp8_blk")
        return y, None, None
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", _U8, 2)
    _need(ws, "ws", (torch.uint8,), 2)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K:
        raise ValueError(f"w has K={w.shape[1]}, x has K={K}")
    if tuple(ws.shape) != ((N + 127) // 128, K // 128) or not ws.is_contiguous():
        raise ValueError(f"ws must be contiguous [{(N + 127) // 128}, {K // 128}], got {tuple(ws.shape)}")
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((M, K // 128), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if not xq.is_contiguous() or not xs.is_contiguous():
        raise ValueError("xq / xs must be contiguous")
    _need(y, "y", (torch.bfloat16,), 2)
    check(load().qlin_gemv_fp8_blk(x.data_ptr(), x.stride(0), M, K, w.data_ptr(), w.stride(0), N,
                                   ws.data_ptr(), xq.data_ptr(), xs.data_ptr(), y.data_ptr(),
                                   y.stride(0), _stream(x, stream)), "qlin_gemv_fp8_blk")
    return y, xq, xs


def qlin_gemv_fp8_blk_ex(x, w, ws, block_n, block_k, xq=None, xs=None, y=None, stream=None):
    """Block-scaled FP8 at any block shape: x bf16 [M, K], w E4M3 [N, K], ws UE8M0
    [ceil(N/block_n), K/block_k].  Returns (y bf16 [M, N], xq E4M3 [M, K], xs UE8M0 [M, K/block_k])."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", _U8, 2)
    _need(ws, "ws", (torch.uint8,), 2)
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or K % block_k:
        raise ValueError(f"w has K={w.shape[1]}, x has K={K}, block_k={block_k}")
    if tuple(ws.shape) != ((N + block_n - 1) // block_n, K // block_k) or not ws.is_contiguous():
        raise ValueError(f"ws must be contiguous [{(N + block_n - 1) // block_n}, {K // block_k}], got {tuple(ws.shape)}")
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if xs is None:
        xs = torch.empty((M, K // block_k), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    if not xq.is_contiguous() or not xs.is_contiguous():
        raise ValueError("xq / xs must be contiguous")
    _need(y, "y", (torch.bfloat16,), 2)
    check(load().qlin_gemv_fp8_blk_ex(x.data_ptr(), x.stride(0), M, K, w.data_ptr(), w.stride(0), N,
                                      ws.data_ptr(), int(block_n), int(block_k), xq.data_ptr(), xs.data_ptr(),
                                      y.data_ptr(), y.stride(0), _stream(x, stream)), "qlin_gemv_fp8_blk_ex")
    return y, xq, xs


def qlin_moe_mxfp4_workspace_bytes(M: int, N: int, topk: int, E: int) -> int:
    return int(load().qlin_moe_mxfp4_workspace_bytes(M, N, topk, E))


def qlin_moe_mxfp4(x, w, s, topk_ids, topk_w, y=None, workspace=None, stream=None):
    """Top-k MXFP4 expert GEMV: x bf16 [M, K]; w uint8 [E, N, K/2] (element 2i in
    the low nibble); s UE8M0 [E, N, K/32]; topk_ids int32 [M, topk]; topk_w fp32
    [M, topk].  Returns y bf16 [M, N]."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 3)
    _need(s, "s", (torch.uint8,), 3)
    _need(topk_ids, "topk_ids", (torch.int32,), 2)
    _need(topk_w, "topk_w", (torch.float32,), 2)
    M, K = x.shape
    E, N, Kh = w.shape
    topk = topk_ids.shape[1]
    if Kh * 2 != K or tuple(s.shape) != (E, N, K // 32):
        raise ValueError(f"w {tuple(w.shape)} / s {tuple(s.shape)} do not match K={K}")
    if not (w.is_contiguous() and s.is_contiguous() and topk_ids.is_contiguous() and topk_w.is_contiguous()):
        raise ValueError("w, s, topk_ids, topk_w must be contiguous")
    if tuple(topk_ids.shape) != (M, topk) or tuple(topk_w.shape) != (M, topk):
        raise ValueError("topk_ids / topk_w must be [M, topk]")
    need = qlin_moe_mxfp4_workspace_bytes(M, N, topk, E)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", (torch.bfloat16,), 2)
    check(load().qlin_moe_mxfp4(x.data_ptr(), x.stride(0), M, K, w.data_ptr(), s.data_ptr(), E, N,
                                topk_ids.data_ptr(), topk_w.data_ptr(), topk, y.data_ptr(), y.stride(0),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                _stream(x, stream)), "qlin_moe_mxfp4")
    return y


QLIN_NOALLOC_SCRATCH_BYTES = 4 << 20  # the library's per-GPU scratch array behind qlin_moe_mxfp4_noalloc


def qlin_moe_mxfp4_noalloc(x, w, s, topk_ids, topk_w, y, stream=None):
    """qlin_moe_mxfp4 with the library's own per-GPU scratch array as its
    workspace: the call allocates nothing (y, the output, is the caller's).
    Calls that can overlap on one GPU share that array and must be serialised."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(w, "w", (torch.uint8,), 3)
    _need(s, "s", (torch.uint8,), 3)
    _need(topk_ids, "topk_ids", (torch.int32,), 2)
    _need(topk_w, "topk_w", (torch.float32,), 2)
    _need(y, "y", (torch.bfloat16,), 2)
    M, K = x.shape
    E, N, Kh = w.shape
    topk = topk_ids.shape[1]
    if Kh * 2 != K or tuple(s.shape) != (E, N, K // 32):
        raise ValueError(f"w {tuple(w.shape)} / s {tuple(s.shape)} do not match K={K}")
    if not (w.is_contiguous() and s.is_contiguous() and topk_ids.is_contiguous() and topk_w.is_contiguous()):
        raise ValueError("w, s, topk_ids, topk_w must be contiguous")
    if tuple(topk_ids.shape) != (M, topk) or tuple(topk_w.shape) != (M, topk) or tuple(y.shape) != (M, N):
        raise ValueError("topk_ids / topk_w must be [M, topk] and y [M, N]")
    check(load().qlin_moe_mxfp4_noalloc(x.data_ptr(), x.stride(0), M, K, w.data_ptr(), s.data_ptr(), E, N,
                                        topk_ids.data_ptr(), topk_w.data_ptr(), topk, y.data_ptr(), y.stride(0),
                                        _stream(x, stream)), "qlin_moe_mxfp4_noalloc")
    return y


def qlin_moe_ffn_mxfp4_workspace_bytes(M: int, H: int, I: int, topk: int, E: int) -> int:
    return int(load().qlin_moe_ffn_mxfp4_workspace_bytes(M, H, I, topk, E))


def _round256(b: int) -> int:
    return (b + 255) // 256 * 256


def qlin_moe_ffn_mxfp4(x, wr, w13, s13, w2, s2, topk, alpha=1.0, limit=10.0, y=None, workspace=None,
                       stream=None, return_internals=False, ids=None, gw=None):
    """Routed MXFP4 expert FFN with on-device routing.  x bf16 [M, H]; wr bf16
    [E, H]; w13 uint8 [E, 2I, H/2] (gate rows then up rows); s13 [E, 2I, H/32];
    w2 uint8 [E, H, I/2]; s2 [E, H, I/32].  Returns (y bf16 [M, H], topk_ids
    int32 [M, topk], topk_w fp32 [M, topk]); with return_internals also the
    router logits fp32 [M, E] and the activations bf16 [M*topk, I] read back
    from the workspace (valid once the stream has run the call)."""
    _need(x, "x", (torch.bfloat16,), 2)
    _need(wr, "wr", (torch.bfloat16,), 2)
    for name, t in (("w13", w13), ("s13", s13), ("w2", w2), ("s2", s2)):
        _need(t, name, (torch.uint8,), 3)
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not wr.is_contiguous():
        raise ValueError("wr must be contiguous")
    M, H = x.shape
    E = wr.shape[0]
    I = w13.shape[1] // 2
    if (tuple(wr.shape) != (E, H) or tuple(w13.shape) != (E, 2 * I, H // 2) or tuple(s13.shape) != (E, 2 * I, H // 32)
            or tuple(w2.shape) != (E, H, I // 2) or tuple(s2.shape) != (E, H, I // 32)):
        raise ValueError("router / expert tensor shapes do not match x")
    need = qlin_moe_ffn_mxfp4_workspace_bytes(M, H, I, topk, E)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", (torch.bfloat16,), 2)
    if ids is None:
        ids = torch.empty((M, topk), dtype=torch.int32, device=x.device)
    if gw is None:
        gw = torch.empty((M, topk), dtype=torch.float32, device=x.device)
    _need(ids, "ids", (torch.int32,), 2)
    _need(gw, "gw", (torch.float32,), 2)
    if tuple(ids.shape) != (M, topk) or tuple(gw.shape) != (M, topk) or not (ids.is_contiguous() and gw.is_contiguous()):
        raise ValueError("ids / gw must be contiguous [M, topk]")
    check(load().qlin_moe_ffn_mxfp4(x.data_ptr(), x.stride(0), M, H, wr.data_ptr(), E, topk,
                                    w13.data_ptr(), s13.data_ptr(), I, w2.data_ptr(), s2.data_ptr(),
                                    float(alpha), float(limit), ids.data_ptr(), gw.data_ptr(),
                                    y.data_ptr(), y.stride(0), workspace.data_ptr(),
                                    workspace.numel() * workspace.element_size(), _stream(x, stream)),
          "qlin_moe_ffn_mxfp4")
    if not return_internals:
        return y, ids, gw
    o_act = _round256(M * E * 4)
    logits = workspace[:M * E * 4].view(torch.float32).view(M, E)
    act = workspace[o_act:o_act + M * topk * I * 2].view(torch.bfloat16).view(M * topk, I)
    return y, ids, gw, logits, act
