"""The qlin entry points as PyTorch custom operators (namespace ``qlin``).

Each operator is opaque to the compiler: ``torch.compile`` and graph capture
keep the call instead of tracing into it, so the HIP kernel cannot be
silently replaced by a decomposition, and all M dispatch happens inside the
body.  Every operator has a fake (meta) implementation that only computes
output shapes and dtypes, so graphs can be traced without a GPU.

``hits`` counts how many times each operator's real body ran; a test (or a
caller) can read it to confirm that a compiled graph still reaches the
kernel.  The bodies call the ctypes binding of ``libqlin.so``; there is no
fallback.

    import skinny_gemm_qlin_amd.torch_ops  # registers torch.ops.qlin.*
    y = torch.ops.qlin.gemv_fp8(x, w, ws)
"""
from __future__ import annotations

import collections
from typing import Optional, Tuple

import torch

from . import (qlin_act_quant_fp8, qlin_act_quant_i8, qlin_gemv_fp8, qlin_gemv_fp8_blk, qlin_gemv_fp8_blk_ex,
               qlin_gemv_fp8_w8a8, qlin_gemv_i8, qlin_linear_i8, qlin_moe_ffn_mxfp4, qlin_moe_mxfp4)

hits = collections.Counter()


def reset_hits() -> None:
    hits.clear()


# ----------------------------------------------------------------------------- W8A8 INT8

@torch.library.custom_op("qlin::act_quant_i8", mutates_args=())
def act_quant_i8(x: torch.Tensor) -> Tuple[torch.Tensor, torch.Tensor]:
    hits["act_quant_i8"] += 1
    return qlin_act_quant_i8(x)


@act_quant_i8.register_fake
def _(x):
    M, K = x.shape
    return x.new_empty((M, K), dtype=torch.int8), x.new_empty((M,), dtype=torch.float32)


@torch.library.custom_op("qlin::gemv_i8", mutates_args=())
def gemv_i8(xq: torch.Tensor, xs: torch.Tensor, w: torch.Tensor, ws: torch.Tensor,
            bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    hits["gemv_i8"] += 1
    return qlin_gemv_i8(xq, xs, w, ws, bias=bias)


@gemv_i8.register_fake
def _(xq, xs, w, ws, bias=None):
    return xq.new_empty((xq.shape[0], w.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("qlin::linear_i8", mutates_args=())
def linear_i8(x: torch.Tensor, w: torch.Tensor, ws: torch.Tensor,
              bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Dynamic per-token quantisation and the INT8 GEMV through qlin_linear_i8
    (one kernel for one token, quantiser + GEMV otherwise)."""
    hits["linear_i8"] += 1
    return qlin_linear_i8(x, w, ws, bias=bias)[0]


@linear_i8.register_fake
def _(x, w, ws, bias=None):
    return x.new_empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16)


# ----------------------------------------------------------------------------- FP8

@torch.library.custom_op("qlin::gemv_fp8", mutates_args=())
def gemv_fp8(x: torch.Tensor, w: torch.Tensor, ws: torch.Tensor) -> torch.Tensor:
    hits["gemv_fp8"] += 1
    return qlin_gemv_fp8(x, w, ws)


@gemv_fp8.register_fake
def _(x, w, ws):
    return x.new_empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16)


# ----------------------------------------------------------------------------- FP8 W8A8 (fmt 0 = E4M3, 1 = E5M2)

@torch.library.custom_op("qlin::act_quant_fp8", mutates_args=())
def act_quant_fp8(x: torch.Tensor, fmt: int = 0, per_token: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    hits["act_quant_fp8"] += 1
    return qlin_act_quant_fp8(x, fmt, per_token)


@act_quant_fp8.register_fake
def _(x, fmt=0, per_token=True):
    M, K = x.shape
    return x.new_empty((M, K), dtype=torch.uint8), x.new_empty((M if per_token else 1,), dtype=torch.float32)


@torch.library.custom_op("qlin::gemv_fp8_w8a8", mutates_args=())
def gemv_fp8_w8a8(xq: torch.Tensor, xs: torch.Tensor, w: torch.Tensor, ws: torch.Tensor, x_fmt: int = 0,
                  w_fmt: int = 0) -> torch.Tensor:
    hits["gemv_fp8_w8a8"] += 1
    return qlin_gemv_fp8_w8a8(xq, xs, w, ws, x_fmt, w_fmt)


@gemv_fp8_w8a8.register_fake
def _(xq, xs, w, ws, x_fmt=0, w_fmt=0):
    return xq.new_empty((xq.shape[0], w.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("qlin::linear_fp8_w8a8", mutates_args=())
def linear_fp8_w8a8(x: torch.Tensor, w: torch.Tensor, ws: torch.Tensor, x_fmt: int = 0, w_fmt: int = 0,
                    per_token: bool = True) -> torch.Tensor:
    """Dynamic FP8 activation quantisation followed by the W8A8 GEMV (two kernels)."""
    hits["linear_fp8_w8a8"] += 1
    xq, xs = qlin_act_quant_fp8(x, x_fmt, per_token)
    return qlin_gemv_fp8_w8a8(xq, xs, w, ws, x_fmt, w_fmt)


@linear_fp8_w8a8.register_fake
def _(x, w, ws, x_fmt=0, w_fmt=0, per_token=True):
    return x.new_empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("qlin::gemv_fp8_blk", mutates_args=())
def gemv_fp8_blk(x: torch.Tensor, w: torch.Tensor, ws: torch.Tensor) -> torch.Tensor:
    hits["gemv_fp8_blk"] += 1
    # one token: the fused kernel needs no code / scale buffers
    return qlin_gemv_fp8_blk(x, w, ws, export=not (x.shape[0] == 1 and x.shape[1] <= 32768))[0]


@gemv_fp8_blk.register_fake
def _(x, w, ws):
    return x.new_empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16)


@torch.library.custom_op("qlin::gemv_fp8_blk_ex", mutates_args=())
def gemv_fp8_blk_ex(x: torch.Tensor, w: torch.Tensor, ws: torch.Tensor, block_n: int, block_k: int) -> torch.Tensor:
    hits["gemv_fp8_blk_ex"] += 1
    return qlin_gemv_fp8_blk_ex(x, w, ws, block_n, block_k)[0]


@gemv_fp8_blk_ex.register_fake
def _(x, w, ws, block_n, block_k):
    return x.new_empty((x.shape[0], w.shape[0]), dtype=torch.bfloat16)


# ----------------------------------------------------------------------------- MXFP4 MoE

@torch.library.custom_op("qlin::moe_mxfp4", mutates_args=())
def moe_mxfp4(x: torch.Tensor, w: torch.Tensor, s: torch.Tensor, topk_ids: torch.Tensor,
              topk_w: torch.Tensor) -> torch.Tensor:
    hits["moe_mxfp4"] += 1
    return qlin_moe_mxfp4(x, w, s, topk_ids, topk_w)


@moe_mxfp4.register_fake
def _(x, w, s, topk_ids, topk_w):
    return x.new_empty((x.shape[0], w.shape[1]), dtype=torch.bfloat16)


@torch.library.custom_op("qlin::moe_ffn_mxfp4", mutates_args=())
def moe_ffn_mxfp4(x: torch.Tensor, wr: torch.Tensor, w13: torch.Tensor, s13: torch.Tensor, w2: torch.Tensor,
                  s2: torch.Tensor, topk: int, alpha: float = 1.0,
                  limit: float = 10.0) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    hits["moe_ffn_mxfp4"] += 1
    return qlin_moe_ffn_mxfp4(x, wr, w13, s13, w2, s2, topk, alpha, limit)


@moe_ffn_mxfp4.register_fake
def _(x, wr, w13, s13, w2, s2, topk, alpha=1.0, limit=10.0):
    M, H = x.shape
    return (x.new_empty((M, H), dtype=torch.bfloat16), x.new_empty((M, topk), dtype=torch.int32),
            x.new_empty((M, topk), dtype=torch.float32))
