"""Seeded synthetic inputs for MLA decode: the one module both sides draw from.

This module generates random numbers and workload shapes only.  It holds none
of the attention arithmetic: no RoPE, no projection, no softmax.  The CPU
oracle (``oracle/``) and the HIP path each take its outputs as inputs.

Generator (counter based, so any slice can be regenerated without the rest):

* SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; the 64-bit finaliser as published by Vigna).
  The n-th output from state ``k`` is ``mix64(k + (n + 1) * GAMMA)``.
* A stream key per (seed, tensor id, layer):
  ``k0 = mix64((seed+1)*GAMMA)``, ``k1 = mix64(k0 ^ (tensor+1)*GAMMA)``,
  ``k2 = mix64(k1 ^ (layer+1)*GAMMA)`` (all mod 2**64).
* Normal draws by the Box-Muller transform (Box and Muller, 1958) in fp64
  from one 64-bit word: ``u1 = (hi32 + 0.5) / 2**32``, ``u2 = lo32 / 2**32``,
  ``z = sqrt(-2 ln u1) * cos(2 pi u2)``; the value ``z * std`` is rounded
  straight from fp64 to bfloat16, round-to-nearest-even.

The GPU twin (``synth/gpu_gen.hip``) implements the same definition so that
multi-gigabyte caches can be generated in device memory; a GPU test checks
the two agree.

Logical element indices (``TOKMAX = 2**20`` tokens per sequence, ``QMAX = 16``
query tokens per sequence; a single-sequence prefill chunk, b = 0, may take any
number of query tokens, its indices running on past QMAX):

====================  =========================================
tensor (id)           flat index of element
====================  =========================================
latent c_kv (1)       ``(b*TOKMAX + t)*512 + d``
rope key k_pe (2)     ``(b*TOKMAX + t)*64 + d``   (before RoPE)
q_nope (3)            ``((b*QMAX + j)*32 + h)*128 + d``
q_pe (4)              ``((b*QMAX + j)*32 + h)*64 + d``  (before RoPE)
kv_b_proj weight (5)  ``row*512 + col`` (row in [0, 8192))
page permutation (6)  draw ``n`` for Fisher-Yates step ``n``
context lengths (7)   draw ``b`` for sequence ``b``
====================  =========================================
"""
from __future__ import annotations

import math

import numpy as np

GAMMA = 0x9E3779B97F4A7C15
MASK64 = (1 << 64) - 1
TOKMAX = 1 << 20
QMAX = 16

T_LATENT, T_KPE, T_QNOPE, T_QPE, T_WKVB, T_PAGES, T_LENS = 1, 2, 3, 4, 5, 6, 7

_U64 = np.uint64


def _mix64_int(z: int) -> int:
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _U64(30))) * _U64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> _U64(27))) * _U64(0x94D049BB133111EB)
        return z ^ (z >> _U64(31))


def stream_key(seed: int, tensor: int, layer: int) -> int:
    """64-bit key of the stream for (seed, tensor id, layer)."""
    k0 = _mix64_int(((seed + 1) * GAMMA) & MASK64)
    k1 = _mix64_int(k0 ^ (((tensor + 1) * GAMMA) & MASK64))
    return _mix64_int(k1 ^ (((layer + 1) * GAMMA) & MASK64))


def draw_u64(key: int, index: np.ndarray) -> np.ndarray:
    """SplitMix64 outputs ``mix64(key + (index+1)*GAMMA)`` for uint64 ``index``."""
    idx = np.asarray(index, dtype=_U64)
    with np.errstate(over="ignore"):
        z = _U64(key) + (idx + _U64(1)) * _U64(GAMMA)
    return _mix64_np(z)


def normal_f64(key: int, index: np.ndarray) -> np.ndarray:
    """Box-Muller standard normals, one per 64-bit draw, in fp64."""
    u = draw_u64(key, index)
    hi = (u >> _U64(32)).astype(np.float64)
    lo = (u & _U64(0xFFFFFFFF)).astype(np.float64)
    u1 = (hi + 0.5) * (2.0 ** -32)
    u2 = lo * (2.0 ** -32)
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * math.pi * u2)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 straight to bfloat16 (nearest, ties to even); uint16 bits.

    Valid for finite values in bfloat16's normal range, which is all this
    generator produces.
    """
    b = np.ascontiguousarray(x, dtype=np.float64).view(_U64)
    lsb = (b >> _U64(45)) & _U64(1)
    with np.errstate(over="ignore"):
        b = (b + _U64((1 << 44) - 1) + lsb) & _U64(~((1 << 45) - 1) & MASK64)
    f32 = b.view(np.float64).astype(np.float32)  # exact: 8 significant bits
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def normal_bf16_bits(seed: int, tensor: int, layer: int, index: np.ndarray, std: float = 1.0) -> np.ndarray:
    """bfloat16 bits of ``std * N(0,1)`` for the given flat indices."""
    z = normal_f64(stream_key(seed, tensor, layer), index)
    return f64_to_bf16_bits(z * std)


W_STD = 1.0 / math.sqrt(512.0)  # N(0, 1/512): variance 1/512


# ---------------------------------------------------------------------------
# Logical tensors (bf16 bits, uint16 arrays)
# ---------------------------------------------------------------------------

def latent_bits(seed, layer, b, t0, t1):
    """c_kv[t0:t1, 0:512] of sequence b, layer ``layer``."""
    t = np.arange(t0, t1, dtype=np.uint64)[:, None]
    d = np.arange(512, dtype=np.uint64)[None, :]
    idx = (_U64(b) * _U64(TOKMAX) + t) * _U64(512) + d
    return normal_bf16_bits(seed, T_LATENT, layer, idx)


def kpe_bits(seed, layer, b, t0, t1):
    """k_pe[t0:t1, 0:64] of sequence b before RoPE."""
    t = np.arange(t0, t1, dtype=np.uint64)[:, None]
    d = np.arange(64, dtype=np.uint64)[None, :]
    idx = (_U64(b) * _U64(TOKMAX) + t) * _U64(64) + d
    return normal_bf16_bits(seed, T_KPE, layer, idx)


def qnope_bits(seed, layer, b, sq):
    """q_nope[0:sq, 0:32, 0:128] of sequence b."""
    j = np.arange(sq, dtype=np.uint64)[:, None, None]
    h = np.arange(32, dtype=np.uint64)[None, :, None]
    d = np.arange(128, dtype=np.uint64)[None, None, :]
    idx = ((_U64(b) * _U64(QMAX) + j) * _U64(32) + h) * _U64(128) + d
    return normal_bf16_bits(seed, T_QNOPE, layer, idx)


def qpe_bits(seed, layer, b, sq):
    """q_pe[0:sq, 0:32, 0:64] of sequence b before RoPE."""
    j = np.arange(sq, dtype=np.uint64)[:, None, None]
    h = np.arange(32, dtype=np.uint64)[None, :, None]
    d = np.arange(64, dtype=np.uint64)[None, None, :]
    idx = ((_U64(b) * _U64(QMAX) + j) * _U64(32) + h) * _U64(64) + d
    return normal_bf16_bits(seed, T_QPE, layer, idx)


def wkvb_bits(seed, layer):
    """kv_b_proj weight [8192, 512] (nn.Linear storage: out x in), N(0, 1/512)."""
    idx = np.arange(8192 * 512, dtype=np.uint64).reshape(8192, 512)
    return normal_bf16_bits(seed, T_WKVB, layer, idx, W_STD)


# ---------------------------------------------------------------------------
# Workload structure: context lengths and page assignment
# ---------------------------------------------------------------------------

def loguniform_lengths(seed: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """L_b = floor(exp(u)), u ~ U[ln lo, ln hi), clamped to [lo, hi]."""
    u = draw_u64(stream_key(seed, T_LENS, 0), np.arange(batch, dtype=np.uint64))
    frac = (u >> _U64(11)).astype(np.float64) * (2.0 ** -53)
    x = np.floor(np.exp(math.log(lo) + frac * (math.log(hi) - math.log(lo))))
    return np.clip(x, lo, hi).astype(np.int64)


def page_permutation(seed: int, num_pages: int) -> np.ndarray:
    """Seeded Fisher-Yates shuffle of ``range(num_pages)``."""
    perm = np.arange(num_pages, dtype=np.int64)
    if num_pages < 2:
        return perm
    draws = draw_u64(stream_key(seed, T_PAGES, 0), np.arange(num_pages - 1, dtype=np.uint64))
    for n, i in enumerate(range(num_pages - 1, 0, -1)):
        j = int(draws[n] % _U64(i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


def block_tables(seed: int, lens, page_size: int = 64, permute: bool = True):
    """Pages of a shared pool assigned to sequences.

    Sequence b owns ``ceil(L_b / page_size)`` pages taken, in order, from a
    seeded permutation of the pool (identity when ``permute`` is False).
    Returns (block_table int32 [B, max_pages], num_pages).  Unused entries
    are -1.
    """
    lens = [int(x) for x in lens]
    need = [(x + page_size - 1) // page_size for x in lens]
    pool = sum(need)
    perm = page_permutation(seed, pool) if permute else np.arange(pool, dtype=np.int64)
    width = max(need) if need else 0
    bt = np.full((len(lens), max(width, 1)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[off:off + n]
        off += n
    return bt, pool
