"""Device-side twin of the seeded generator (synth/libmla_synth.so).

Fills torch bf16 tensors in GPU memory with exactly the values
``synth.normal_bf16_bits`` gives on the host for the same (seed, tensor,
layer, index).  Input generation only.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import TOKMAX, QMAX, T_LATENT, T_KPE, T_QNOPE, T_QPE, T_WKVB, W_STD

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_synth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_fill_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64,
                                               ctypes.c_double, ctypes.c_void_p]
        lib.synth_fill_normal_bf16.restype = ctypes.c_int
        lib.synth_stream_key.argtypes = [ctypes.c_uint64] * 3
        lib.synth_stream_key.restype = ctypes.c_uint64
        _LIB = lib
    return _LIB


def fill(out: torch.Tensor, seed: int, tensor: int, layer: int, base_row: int, std: float = 1.0):
    """out viewed as rows x width (last dim = width, any row stride) <- normals
    at flat indices (base_row + r) * width + d."""
    assert out.dtype == torch.bfloat16 and out.device.type == "cuda"
    o2 = out.reshape(-1, out.shape[-1]) if out.is_contiguous() else out
    assert o2.dim() == 2 and o2.stride(1) == 1
    rows, width = o2.shape
    rc = _lib().synth_fill_normal_bf16(ctypes.c_void_p(o2.data_ptr()), rows, width, o2.stride(0), seed,
                                       tensor, layer, base_row, std,
                                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_bf16 launch failed ({rc})")
    return out


def latent(out, seed, layer, b, t0):
    """out[i, :] = c_kv[t0 + i, :] of sequence b (width 512)."""
    return fill(out, seed, T_LATENT, layer, b * TOKMAX + t0)


def kpe(out, seed, layer, b, t0):
    """out[i, :] = k_pe[t0 + i, :] of sequence b before RoPE (width 64)."""
    return fill(out, seed, T_KPE, layer, b * TOKMAX + t0)


def qnope(out, seed, layer, b):
    """out [Sq, 32, 128] of sequence b."""
    return fill(out.view(-1, 128), seed, T_QNOPE, layer, b * QMAX * 32)


def qpe(out, seed, layer, b):
    """out [Sq, 32, 64] of sequence b before RoPE."""
    return fill(out.view(-1, 64), seed, T_QPE, layer, b * QMAX * 32)


def wkvb(out, seed, layer):
    """out [8192, 512], N(0, 1/512)."""
    return fill(out, seed, T_WKVB, layer, 0, W_STD)
