"""Helpers for the GPU tests: numpy <-> device tensors and the library handle."""
import numpy as np
import pytest
import torch


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def lib():
    """The product binding; raises (never falls back) if libqlin.so is missing."""
    import skinny_gemm_qlin_amd as ql
    ql.load()
    return ql


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def host_bits(t):
    """bf16 device tensor -> uint16 numpy bit patterns."""
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def host(t):
    return t.contiguous().cpu().numpy()


def padded(a, pad, fill=0x5A):
    """Copy a [R, C] array into a [R, C+pad] buffer (filled with junk) and return
    the device view of its first C columns: a non-contiguous row pitch."""
    R, C = a.shape
    buf = np.full((R, C + pad), fill, dtype=a.dtype)
    buf[:, :C] = a
    return dev(buf)[:, :C]
