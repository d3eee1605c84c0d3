"""CPU oracle for the weight-quantized decode GEMV (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.

The arithmetic lives in ``qlin_oracle.c`` (plain loops, fp64/int64
accumulation, one final round to bf16); this module only marshals numpy
arrays through ctypes.  bf16 arrays are carried as ``uint16`` bit patterns.
Each wrapper names the page section its C function follows (see the header of
``qlin_oracle.c`` for the page titles).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qlin_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BLK = 128  # weight block edge and activation group width of the block-scaled path


def build(verbose: bool = False) -> str:
    """Compile ``qlin_oracle.c`` into ``liboracle.so`` (gcc -O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", _LIB_PATH + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.orc_set_threads.argtypes = [I]
    lib.orc_max_threads.restype = I
    lib.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f32.restype = ctypes.c_float
    lib.orc_f32_to_bf16.argtypes = [ctypes.c_float]
    lib.orc_f32_to_bf16.restype = ctypes.c_uint16
    lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_encode.argtypes = [ctypes.c_double]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e2m1_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e2m1_decode.restype = ctypes.c_double
    lib.orc_ue8m0_decode.argtypes = [ctypes.c_uint8]
    lib.orc_ue8m0_decode.restype = ctypes.c_double
    lib.orc_f64_to_bf16_n.argtypes = [P, I64, P]
    lib.orc_f32_to_bf16_n.argtypes = [P, I64, P]
    lib.orc_e4m3_decode_n.argtypes = [P, I64, P]
    lib.orc_e4m3_encode_n.argtypes = [P, I64, P]
    lib.orc_e5m2_decode_n.argtypes = [P, I64, P]
    lib.orc_e5m2_encode_n.argtypes = [P, I64, P]
    lib.orc_act_quant_fp8.argtypes = [P, I64, I64, I64, I, I, P, I64, P]
    lib.orc_gemv_fp8_w8a8.argtypes = [P, I64, P, I, I, I64, I64, P, I64, I64, P, I, I, P, I64, P, P]
    lib.orc_act_quant_i8.argtypes = [P, I64, I64, I64, P, I64, P]
    lib.orc_gemv_i8.argtypes = [P, I64, P, I, I64, I64, P, I64, I64, P, I, P, P, P, I64]
    lib.orc_gemv_fp8.argtypes = [P, I64, I64, I64, P, I64, I64, P, I, P, I64, P, P]
    lib.orc_blk_act_quant.argtypes = [P, I64, I64, I64, P, P]
    lib.orc_gemv_fp8_blk.argtypes = [P, P, I64, I64, P, I64, I64, P, P, I64, P, P]
    lib.orc_blk_act_quant_g.argtypes = [P, I64, I64, I64, I64, P, P]
    lib.orc_gemv_fp8_blk_g.argtypes = [P, P, I64, I64, P, I64, I64, P, I64, I64, P, I64, P, P]
    lib.orc_moe_mxfp4.argtypes = [P, I64, I64, I64, P, P, I64, I64, P, P, I64, P, I64, P, P]
    lib.orc_router_logits.argtypes = [P, I64, I64, I64, P, I64, P]
    lib.orc_topk.argtypes = [P, I64, I64, I64, P]
    lib.orc_topk_softmax.argtypes = [P, I64, I64, P, I64, P]
    lib.orc_swiglu.argtypes = [ctypes.c_double] * 4
    lib.orc_swiglu.restype = ctypes.c_double
    lib.orc_swiglu_n.argtypes = [P, P, I64, ctypes.c_double, ctypes.c_double, P]
    D = ctypes.c_double
    lib.orc_moe_ffn_mxfp4.argtypes = [P, I64, I64, I64, P, P, P, P, I64, I64, P, P, I64, D, D, P, P, I64, P, P]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def set_threads(n: int) -> None:
    _load().orc_set_threads(int(n))


def max_threads() -> int:
    return int(_load().orc_max_threads())


# --------------------------------------------------------------------------- formats

def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    lib = _load()
    h = np.asarray(h, dtype=np.uint16)
    return np.array([lib.orc_bf16_to_f32(int(v)) for v in h.ravel()], dtype=np.float32).reshape(h.shape)


def _map(fn, a, in_dtype, out_dtype):
    a = np.ascontiguousarray(a, dtype=in_dtype)
    out = np.empty(a.shape, dtype=out_dtype)
    getattr(_load(), fn)(a.ctypes.data, a.size, out.ctypes.data)
    return out


def f32_to_bf16(f: np.ndarray) -> np.ndarray:
    return _map("orc_f32_to_bf16_n", f, np.float32, np.uint16)


def f64_to_bf16(d: np.ndarray) -> np.ndarray:
    return _map("orc_f64_to_bf16_n", d, np.float64, np.uint16)


def e4m3_decode(codes) -> np.ndarray:
    return _map("orc_e4m3_decode_n", codes, np.uint8, np.float64)


def e4m3_encode(values) -> np.ndarray:
    return _map("orc_e4m3_encode_n", values, np.float64, np.uint8)


def e5m2_decode(codes) -> np.ndarray:
    return _map("orc_e5m2_decode_n", codes, np.uint8, np.float64)


def e5m2_encode(values) -> np.ndarray:
    return _map("orc_e5m2_encode_n", values, np.float64, np.uint8)


def e2m1_decode(nibbles) -> np.ndarray:
    lib = _load()
    c = np.asarray(nibbles, dtype=np.uint8)
    return np.array([lib.orc_e2m1_decode(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


def ue8m0_decode(b) -> np.ndarray:
    lib = _load()
    c = np.asarray(b, dtype=np.uint8)
    return np.array([lib.orc_ue8m0_decode(int(v)) for v in c.ravel()], dtype=np.float64).reshape(c.shape)


# --------------------------------------------------------------------------- (a) INT8

def act_quant_i8(x_bf16: np.ndarray):
    """Per-token dynamic symmetric INT8 quantisation ([Z100] section 2.1).

    x_bf16: uint16 [M, K].  Returns (xq int8 [M, K], xs float32 [M])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    xq = np.zeros((M, K), dtype=np.int8)
    xs = np.zeros((M,), dtype=np.float32)
    _load().orc_act_quant_i8(_p(x), K, M, K, _p(xq), K, _p(xs))
    return xq, xs


def gemv_i8(xq, xs, w, ws, bias=None):
    """W8A8 GEMV with int32 accumulation and the (acc*x_s)*w_s -> bf16 -> +bias
    epilogue ([Z100] section 2 table, INT8 row).

    xs is [M] or [1]; ws is [N] or [1].  Returns (acc int32 [M, N], y uint16 [M, N])."""
    xq = _c(xq, np.int8)
    w = _c(w, np.int8)
    xs = _c(np.atleast_1d(xs), np.float32)
    ws = _c(np.atleast_1d(ws), np.float32)
    M, K = xq.shape
    N, Kw = w.shape
    assert Kw == K
    b = None if bias is None else _c(bias, np.uint16)
    acc = np.zeros((M, N), dtype=np.int32)
    y = np.zeros((M, N), dtype=np.uint16)
    _load().orc_gemv_i8(_p(xq), K, _p(xs), int(xs.size > 1), M, K, _p(w), K, N,
                        _p(ws), int(ws.size > 1), _p(b), _p(acc), _p(y), N)
    return acc, y


# --------------------------------------------------------------------------- (b) FP8 weight-only

def gemv_fp8(x_bf16, w_e4m3, ws):
    """FP8-E4M3 weight-only GEMV, scale applied once ([Z100] section 2.2).

    Returns (y uint16 [M, N], y_exact float64 [M, N], S float64 [M, N])."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_e4m3, np.uint8)
    ws = _c(np.atleast_1d(ws), np.float32)
    M, K = x.shape
    N = w.shape[0]
    y = np.zeros((M, N), dtype=np.uint16)
    ye = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    _load().orc_gemv_fp8(_p(x), K, M, K, _p(w), K, N, _p(ws), int(ws.size > 1), _p(y), N, _p(ye), _p(S))
    return y, ye, S


# --------------------------------------------------------------------------- (c) block-scaled FP8

def blk_act_quant(x_bf16, block_k=BLK):
    """Per-token, per-block_k-group E4M3 quantisation with a UE8M0 scale
    ([DSV4] section 3.3; block_k 128 there).  Returns (xq uint8 [M, K], xs uint8 [M, K/block_k])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    assert K % block_k == 0
    xq = np.zeros((M, K), dtype=np.uint8)
    xs = np.zeros((M, K // block_k), dtype=np.uint8)
    _load().orc_blk_act_quant_g(_p(x), K, M, K, int(block_k), _p(xq), _p(xs))
    return xq, xs


def gemv_fp8_blk(xq, xs, w_e4m3, ws_blk, block_n=BLK, block_k=BLK):
    """Block-scaled GEMV core ([Z100] section 2.4).  ws_blk is [ceil(N/block_n), K/block_k].

    Returns (y uint16 [M, N], y_exact float64, S float64)."""
    xq = _c(xq, np.uint8)
    xs = _c(xs, np.uint8)
    w = _c(w_e4m3, np.uint8)
    wsb = _c(ws_blk, np.uint8)
    M, K = xq.shape
    N = w.shape[0]
    assert wsb.shape == ((N + block_n - 1) // block_n, K // block_k) and xs.shape == (M, K // block_k)
    y = np.zeros((M, N), dtype=np.uint16)
    ye = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    _load().orc_gemv_fp8_blk_g(_p(xq), _p(xs), M, K, _p(w), K, N, _p(wsb), int(block_n), int(block_k),
                               _p(y), N, _p(ye), _p(S))
    return y, ye, S


def fp8_blk(x_bf16, w_e4m3, ws_blk, block_n=BLK, block_k=BLK):
    """Whole block-scaled path: activation quantisation then GEMV.

    Returns (xq, xs, y, y_exact, S)."""
    xq, xs = blk_act_quant(x_bf16, block_k)
    y, ye, S = gemv_fp8_blk(xq, xs, w_e4m3, ws_blk, block_n, block_k)
    return xq, xs, y, ye, S


# --------------------------------------------------------------------------- (d) MXFP4 MoE

def moe_mxfp4(x_bf16, w_fp4, s_ue8m0, topk_ids, topk_w):
    """Top-k routed MXFP4 expert GEMV with weighted sum ([DSV4] section 9.3).

    w_fp4: uint8 [E, N, K/2] (element 2i in the low nibble); s_ue8m0: uint8
    [E, N, K/32]; topk_ids int32 [M, topk]; topk_w float32 [M, topk].
    Returns (y uint16 [M, N], y_exact float64, S float64)."""
    x = _c(x_bf16, np.uint16)
    w = _c(w_fp4, np.uint8)
    s = _c(s_ue8m0, np.uint8)
    ids = _c(topk_ids, np.int32)
    gw = _c(topk_w, np.float32)
    M, K = x.shape
    E, N, Kh = w.shape
    assert Kh * 2 == K and s.shape == (E, N, K // 32)
    topk = ids.shape[1]
    y = np.zeros((M, N), dtype=np.uint16)
    ye = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    _load().orc_moe_mxfp4(_p(x), K, M, K, _p(w), _p(s), E, N, _p(ids), _p(gw), topk, _p(y), N, _p(ye), _p(S))
    return y, ye, S


# --------------------------------------------------------------------------- MoE expert FFN

SWIGLU_ALPHA = 1.0   # [DSV4] sections 6.6 (J09) and 9.4
SWIGLU_LIMIT = 10.0


def router_logits(x_bf16, wr_bf16):
    """logit[m, e] = sum_k x[m, k] * wr[e, k] in fp64 (bf16 inputs); router read as a plain bf16 linear."""
    x = _c(x_bf16, np.uint16)
    wr = _c(wr_bf16, np.uint16)
    M, H = x.shape
    E = wr.shape[0]
    assert wr.shape == (E, H)
    out = np.zeros((M, E), dtype=np.float64)
    _load().orc_router_logits(_p(x), H, M, H, _p(wr), E, _p(out))
    return out


def topk(logits, k):
    """The k largest logits per token, largest first; equal logits -> lower expert id."""
    lg = _c(logits, np.float64)
    M, E = lg.shape
    ids = np.zeros((M, k), dtype=np.int32)
    _load().orc_topk(_p(lg), M, E, k, _p(ids))
    return ids


def topk_softmax(logits, ids):
    """Softmax over each token's selected logits (fp64)."""
    lg = _c(logits, np.float64)
    ids = _c(ids, np.int32)
    M, E = lg.shape
    k = ids.shape[1]
    g = np.zeros((M, k), dtype=np.float64)
    _load().orc_topk_softmax(_p(lg), M, E, _p(ids), k, _p(g))
    return g


def swiglu(gate, up, alpha=SWIGLU_ALPHA, limit=SWIGLU_LIMIT):
    """silu(alpha * min(gate, limit)) * clamp(up, -limit, limit) elementwise, fp64."""
    gt = _c(np.asarray(gate, dtype=np.float64), np.float64)
    u = _c(np.asarray(up, dtype=np.float64), np.float64)
    assert gt.shape == u.shape
    out = np.zeros(gt.shape, dtype=np.float64)
    _load().orc_swiglu_n(_p(gt), _p(u), gt.size, float(alpha), float(limit), _p(out))
    return out


def moe_ffn_mxfp4(x_bf16, w13, s13, w2, s2, ids, g, alpha=SWIGLU_ALPHA, limit=SWIGLU_LIMIT):
    """Routed MXFP4 expert FFN for a given routing ([DSV4] sections 9.3, 6.6, 9.4).

    w13 uint8 [E, 2I, H/2] (gate rows then up rows), s13 uint8 [E, 2I, H/32],
    w2 uint8 [E, H, I/2], s2 uint8 [E, H, I/32]; ids int32 [M, k]; g float64 [M, k].
    Returns (act uint16 [M*k, I], y uint16 [M, H], y_exact float64, S float64)."""
    x = _c(x_bf16, np.uint16)
    w13 = _c(w13, np.uint8)
    s13 = _c(s13, np.uint8)
    w2 = _c(w2, np.uint8)
    s2 = _c(s2, np.uint8)
    ids = _c(ids, np.int32)
    g = _c(np.asarray(g, dtype=np.float64), np.float64)
    M, H = x.shape
    E, I2, Hh = w13.shape
    I = I2 // 2
    assert Hh * 2 == H and s13.shape == (E, 2 * I, H // 32)
    assert w2.shape == (E, H, I // 2) and s2.shape == (E, H, I // 32)
    k = ids.shape[1]
    act = np.zeros((M * k, I), dtype=np.uint16)
    y = np.zeros((M, H), dtype=np.uint16)
    ye = np.zeros((M, H), dtype=np.float64)
    S = np.zeros((M, H), dtype=np.float64)
    _load().orc_moe_ffn_mxfp4(_p(x), H, M, H, _p(w13), _p(s13), _p(w2), _p(s2), E, I, _p(ids), _p(g), k,
                              float(alpha), float(limit), _p(act), _p(y), H, _p(ye), _p(S))
    return act, y, ye, S


def moe_ffn_route_mxfp4(x_bf16, wr_bf16, k, w13, s13, w2, s2, alpha=SWIGLU_ALPHA, limit=SWIGLU_LIMIT):
    """Whole routed FFN: router logits -> top-k -> softmax -> expert FFN.
    Returns (ids, g, logits, act, y, y_exact, S)."""
    lg = router_logits(x_bf16, wr_bf16)
    ids = topk(lg, k)
    g = topk_softmax(lg, ids)
    act, y, ye, S = moe_ffn_mxfp4(x_bf16, w13, s13, w2, s2, ids, g, alpha, limit)
    return ids, g, lg, act, y, ye, S


# --------------------------------------------------------------------------- FP8 W8A8

FMT_E4M3 = 0
FMT_E5M2 = 1


def act_quant_fp8(x_bf16, fmt=FMT_E4M3, per_token=True):
    """Dynamic FP8 activation quantisation ([Z100] FP8 row): s = amax/fmax, q = enc(fl32(x/s)).
    Returns (xq uint8 [M, K], xs float32 [M] or [1])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    xq = np.zeros((M, K), dtype=np.uint8)
    xs = np.zeros((M if per_token else 1,), dtype=np.float32)
    _load().orc_act_quant_fp8(_p(x), K, M, K, int(fmt), int(bool(per_token)), _p(xq), K, _p(xs))
    return xq, xs


def gemv_fp8_w8a8(xq, xs, x_fmt, w, ws, w_fmt):
    """y = bf16(xs * ws * sum_k dec(xq) * dec(w)); xs [M] or [1], ws [N] or [1].
    Returns (y uint16 [M, N], y_exact float64, S float64)."""
    xq = _c(xq, np.uint8)
    w = _c(w, np.uint8)
    xs = _c(np.atleast_1d(xs).astype(np.float32), np.float32)
    ws = _c(np.atleast_1d(ws).astype(np.float32), np.float32)
    M, K = xq.shape
    N = w.shape[0]
    assert w.shape == (N, K) and xs.size in (1, M) and ws.size in (1, N)
    y = np.zeros((M, N), dtype=np.uint16)
    ye = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    _load().orc_gemv_fp8_w8a8(_p(xq), K, _p(xs), int(xs.size == M), int(x_fmt), M, K,
                              _p(w), K, N, _p(ws), int(ws.size == N), int(w_fmt), _p(y), N, _p(ye), _p(S))
    return y, ye, S
