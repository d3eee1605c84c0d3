"""Seeded synthetic inputs for the quantized decode GEMV workloads.

This module is shared by the tests, the benchmark and the smoke check, and is
the ONLY code the HIP path and the CPU oracle have in common.  It holds none
of the method's arithmetic: values are drawn with ``numpy.random.default_rng``
(PCG64) and rounded to bf16 / E4M3 storage with torch's own CPU casts (library
rounding, nearest-even).  Draw order inside one generator is always:
weights, then weight scales, then activations, then routing.

Workload shapes and distributions (all "seed 0" unless a test says otherwise):

* ``int8_small``  W8A8 GEMV, M=1, N=K=1024.
* ``int8_decode`` W8A8 GEMV, N=17408, K=5120, M in {1,2,4,8,16}.
  W int8 uniform in [-127, 127]; per-row fp32 scale uniform in [1e-3, 1e-2];
  x bf16 ~ N(0, 1).
* ``fp8_decode``  E4M3 weight-only GEMV, N=17408, K=5120, M in {1,4,8}.
  Weights drawn bf16 ~ N(0, 0.02) and stored as E4M3 codes with a per-row
  (or per-tensor) fp32 scale absmax/448; x bf16 ~ N(0, 1).
* ``fp8_blk``     block-scaled FP8, N=4096, K=7168, M in {1,8,16}.  Weight
  codes uniform over the 254 finite E4M3 codes; one UE8M0 byte uniform in
  [115, 125] per 128x128 block; x bf16 ~ N(0, 1).
* ``moe_mxfp4``   64 experts of [N=2048, K=7168] E2M1 nibbles uniform over
  all 16 codes, one UE8M0 byte uniform in [118, 126] per (expert, row,
  32-wide K group); M=8 tokens, x bf16 ~ N(0, 1); per token 6 distinct
  experts drawn uniformly, weights = softmax of 6 iid N(0, 1) logits.
"""
from __future__ import annotations

import numpy as np
import torch

# 254 finite OCP E4M3 codes (every byte except S.1111.111)
_E4M3_FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _e4m3_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> OCP E4M3 codes via torch's float8_e4m3fn cast (inputs are in range)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def gen_int8(M: int, N: int, K: int, seed: int = 0) -> dict:
    rng = np.random.default_rng(seed)
    w = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    ws = rng.uniform(1e-3, 1e-2, size=(N,)).astype(np.float32)
    x = bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    return {"w": w, "ws": ws, "x": x}


def gen_fp8(M: int, N: int, K: int, seed: int = 0, per_tensor: bool = False) -> dict:
    rng = np.random.default_rng(seed)
    wf = bf16_values(bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)))
    if per_tensor:
        ws = np.array([np.abs(wf).max() / np.float32(448.0)], dtype=np.float32)
        codes = _e4m3_bits(wf / ws[0])
    else:
        ws = (np.abs(wf).max(axis=1) / np.float32(448.0)).astype(np.float32)
        ws = np.where(ws == 0, np.float32(1.0), ws).astype(np.float32)
        codes = _e4m3_bits(wf / ws[:, None])
    x = bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    return {"w": codes, "ws": ws, "x": x}


def gen_fp8_blk(M: int, N: int, K: int, seed: int = 0, scale_lo: int = 115, scale_hi: int = 125,
                block_n: int = 128, block_k: int = 128) -> dict:
    """Block-scaled FP8 inputs: W codes uniform over the finite E4M3 codes, one
    UE8M0 byte U{scale_lo..scale_hi} per block_n x block_k weight block
    ([ceil(N/block_n)][K/block_k]), x bf16 N(0, 1)."""
    rng = np.random.default_rng(seed)
    w = _E4M3_FINITE[rng.integers(0, _E4M3_FINITE.size, size=(N, K))]
    nb = (N + block_n - 1) // block_n
    ws = rng.integers(scale_lo, scale_hi + 1, size=(nb, K // block_k)).astype(np.uint8)
    x = bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    return {"w": w, "ws": ws, "x": x}


def gen_moe(M: int, E: int, N: int, K: int, topk: int, seed: int = 0,
            scale_lo: int = 118, scale_hi: int = 126) -> dict:
    rng = np.random.default_rng(seed)
    w = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)  # two uniform nibbles per byte
    s = rng.integers(scale_lo, scale_hi + 1, size=(E, N, K // 32)).astype(np.uint8)
    x = bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    ids = np.stack([rng.choice(E, size=topk, replace=False) for _ in range(M)]).astype(np.int32)
    logits = rng.standard_normal((M, topk))
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    gw = (e / e.sum(axis=1, keepdims=True)).astype(np.float32)
    return {"x": x, "w": w, "s": s, "ids": ids, "gw": gw}


def gen_fp8_w8a8(M: int, N: int, K: int, w_fmt: int = 0, per_channel: bool = True, seed: int = 0) -> dict:
    """FP8 W8A8 inputs: W bf16 N(0, 0.02) -> per-row (or one) fp32 scale absmax/fmax
    -> E4M3 (w_fmt 0) or E5M2 (w_fmt 1) codes by torch's cast; x bf16 N(0, 1)
    (the activation codes are made by the quantiser under test)."""
    rng = np.random.default_rng(seed)
    w = bf16_values(bf16_bits(rng.normal(0.0, 0.02, size=(N, K)).astype(np.float32)))
    fmax = 448.0 if w_fmt == 0 else 57344.0
    amax = np.abs(w).max(axis=1) if per_channel else np.full(N, np.abs(w).max())
    ws = (amax / np.float32(fmax)).astype(np.float32)
    ws[ws == 0] = 1.0
    dt = torch.float8_e4m3fn if w_fmt == 0 else torch.float8_e5m2
    codes = (torch.from_numpy(w) / torch.from_numpy(ws)[:, None]).to(dt).view(torch.uint8).numpy()
    x = bf16_bits(rng.standard_normal((M, K), dtype=np.float32))
    return {"x": x, "w": codes, "ws": ws if per_channel else ws[:1].copy(), "w_fmt": w_fmt}


def gen_moe_ffn(M: int, E: int, H: int, I: int, topk: int, seed: int = 0,
                s13_lo: int = 116, s13_hi: int = 122, s2_lo: int = 118, s2_hi: int = 124) -> dict:
    """Routed MXFP4 expert FFN inputs.  Draw order: router weights, gate/up
    codes and scales, down codes and scales, x.  Router weights are bf16
    N(0, 1/H) so the logits are about N(0, 1); the gate/up scale range puts a
    few gate/up values past the SwiGLU limit of 10."""
    rng = np.random.default_rng(seed)
    wr = bf16_bits((rng.standard_normal((E, H), dtype=np.float32) / np.float32(np.sqrt(H))).astype(np.float32))
    w13 = rng.integers(0, 256, size=(E, 2 * I, H // 2), dtype=np.uint8)
    s13 = rng.integers(s13_lo, s13_hi + 1, size=(E, 2 * I, H // 32)).astype(np.uint8)
    w2 = rng.integers(0, 256, size=(E, H, I // 2), dtype=np.uint8)
    s2 = rng.integers(s2_lo, s2_hi + 1, size=(E, H, I // 32)).astype(np.uint8)
    x = bf16_bits(rng.standard_normal((M, H), dtype=np.float32))
    return {"x": x, "wr": wr, "w13": w13, "s13": s13, "w2": w2, "s2": s2, "topk": topk}


# Named workloads (shapes fixed by the published decode configurations).
WORKLOADS = {
    "int8_small": {"kind": "int8", "N": 1024, "K": 1024, "Ms": [1]},
    "int8_decode": {"kind": "int8", "N": 17408, "K": 5120, "Ms": [1, 2, 4, 8, 16]},
    "fp8_decode": {"kind": "fp8", "N": 17408, "K": 5120, "Ms": [1, 4, 8]},
    "fp8_w8a8": {"kind": "fp8_w8a8", "N": 17408, "K": 5120, "Ms": [1, 2, 4, 8, 16]},
    "int8_prefill": {"kind": "int8", "N": 17408, "K": 5120, "Ms": [128, 512, 2048]},
    "fp8_prefill": {"kind": "fp8", "N": 17408, "K": 5120, "Ms": [128, 512, 2048]},
    "int8_prefill_smalln": {"kind": "int8", "N": 48, "K": 5120, "Ms": [64, 512]},
    "fp8_blk": {"kind": "fp8_blk", "N": 4096, "K": 7168, "Ms": [1, 8, 16]},
    "moe_mxfp4": {"kind": "moe", "E": 64, "N": 2048, "K": 7168, "Ms": [8], "topk": 6},
    "moe_prefill": {"kind": "moe", "E": 64, "N": 2048, "K": 7168, "Ms": [64, 512], "topk": 6},
    "moe_ffn_mxfp4": {"kind": "moe_ffn", "E": 64, "H": 7168, "I": 2048, "Ms": [8], "topk": 6},
}
