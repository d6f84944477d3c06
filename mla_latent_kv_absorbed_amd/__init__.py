"""Python binding of the MLA latent-KV decode library (lib/libmla.so).

Argument marshalling only: every step runs in the HIP library.  Tensors are
torch tensors on the GPU (torch provides device memory and the stream); the
functions pass their pointers, sizes and the current HIP stream to the C ABI
declared in include/mla.h and raise ``MlaError`` on any non-zero status.
There is no CPU path: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import lib_path

__all__ = [
    "MlaError", "MlaShape", "MlaRopeParams", "default_shape", "default_rope", "library",
    "CACHE_BF16", "CACHE_FP8_E4M3", "cache_row_width",
    "mla_rope_yarn", "mla_cache_append", "mla_decode", "mla_decode_paged", "mla_decode_step",
    "mla_decode_workspace_size", "mla_decode_auto_chunk", "mla_status_string",
    "mla_prefill", "mla_prefill_workspace_size",
    "mla_timing_enable", "mla_timing_collect", "mla_timing_disable", "mla_read_probe", "READ_PROBE_SINK_INTS",
    "mla_decode_step_paged_noalloc", "STATIC_SCRATCH_BYTES", "mla_device_faults", "mla_check_decode_inputs",
    "mla_check_slot_mapping", "FAULT_SLOT", "FAULT_PAGE", "FAULT_CTX_LEN", "FAULT_FP16_RANGE",
]


class MlaError(RuntimeError):
    pass


class MlaShape(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("kv_lora_rank", ctypes.c_int32),
                ("qk_nope_head_dim", ctypes.c_int32), ("qk_rope_head_dim", ctypes.c_int32),
                ("v_head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("kv_cache_dtype", ctypes.c_int32)]


CACHE_BF16 = 0          # rows of 576 bf16: [latent | rope key]
FAULT_SLOT = 1          # MLA_FAULT_* bits of the device fault word
FAULT_PAGE = 2
FAULT_CTX_LEN = 4
FAULT_FP16_RANGE = 8
STATIC_SCRATCH_BYTES = 64 << 20   # MLA_STATIC_SCRATCH_BYTES
CACHE_FP8_E4M3 = 1      # rows of 656 bytes: [512 E4M3 codes | 4 fp32 scales | 64 bf16 rope key]


class MlaRopeParams(ctypes.Structure):
    _fields_ = [("base", ctypes.c_double), ("factor", ctypes.c_double),
                ("original_max_position", ctypes.c_double), ("beta_fast", ctypes.c_double),
                ("beta_slow", ctypes.c_double), ("rope_dim", ctypes.c_int32)]


_LIB = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def library() -> ctypes.CDLL:
    """The loaded libmla.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise MlaError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(hipcc, gfx950); there is no fallback")
        lib = ctypes.CDLL(path)
        sig = {
            "mla_default_shape": [ctypes.POINTER(MlaShape)],
            "mla_default_rope": [ctypes.POINTER(MlaRopeParams)],
            "mla_rope_yarn": [ctypes.POINTER(MlaRopeParams), _P, _I64, _P, _I64, _P, _I64, _P],
            "mla_cache_append": [ctypes.POINTER(MlaShape), _P, _I64, _P, _I64, _P, _I64, _P, _I64, _P],
            "mla_decode": [ctypes.POINTER(MlaShape), _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32, _I32,
                           _P, _P, _P, ctypes.c_size_t, _P],
            "mla_decode_paged": [ctypes.POINTER(MlaShape), _P, _P, _P, _P, _I64, _P, _I32, _P, _I32,
                                 _I32, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P],
            "mla_decode_step": [ctypes.POINTER(MlaShape), ctypes.POINTER(MlaRopeParams), _P, _P, _P, _I64, _P,
                                _I64, _P, _P, _I64, _P, _I32, _I32, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P],
            "mla_decode_step_paged": [ctypes.POINTER(MlaShape), ctypes.POINTER(MlaRopeParams), _P, _P, _P, _I64,
                                      _P, _I64, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32, _P, _P, _P,
                                      ctypes.c_size_t, _P],
            "mla_decode_workspace_size": [ctypes.POINTER(MlaShape), _I32, _I32, _I32, _I32,
                                          ctypes.POINTER(ctypes.c_size_t)],
            "mla_decode_auto_chunk": [_I32, _I32, _I32, ctypes.POINTER(_I32)],
            "mla_prefill_workspace_size": [ctypes.POINTER(MlaShape), _I32, ctypes.POINTER(ctypes.c_size_t)],
            "mla_prefill": [ctypes.POINTER(MlaShape), _P, _P, _P, _P, _I32, _I32, _P, _P, _P, ctypes.c_size_t, _P],
            "mla_timing_enable": [_I32],
            "mla_timing_collect": [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(_I32)],
            "mla_timing_disable": [],
            "mla_read_probe": [_P, ctypes.c_size_t, _P, _P],
            "mla_decode_step_paged_noalloc": [ctypes.POINTER(MlaShape), ctypes.POINTER(MlaRopeParams), _P, _P, _P,
                                              _I64, _P, _I64, _P, _P, _I64, _P, _I32, _P, _I32, _I32, _I32, _I32,
                                              _P, _P, _P],
            "mla_device_faults": [ctypes.POINTER(ctypes.c_uint32), _I32],
            "mla_check_decode_inputs": [_I32, _I32, _I32, _P, _P, _I32, _I64, ctypes.POINTER(ctypes.c_uint32)],
            "mla_check_slot_mapping": [_P, _I64, _I64, ctypes.POINTER(ctypes.c_uint32)],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int32
        lib.mla_status_string.argtypes = [ctypes.c_int32]
        lib.mla_status_string.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def mla_status_string(code: int) -> str:
    return library().mla_status_string(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise MlaError(f"{what}: {mla_status_string(code)} ({code})")


def default_shape(kv_cache_dtype: int = CACHE_BF16) -> MlaShape:
    s = MlaShape()
    _check(library().mla_default_shape(ctypes.byref(s)), "mla_default_shape")
    s.kv_cache_dtype = kv_cache_dtype
    return s


def cache_row_width(shape: MlaShape) -> tuple:
    """(torch dtype, elements per cache row) of the shape's cache format."""
    if shape.kv_cache_dtype == CACHE_FP8_E4M3:
        return torch.uint8, 656
    return torch.bfloat16, 576


def _check_cache(cache, shape, name="cache", gpu=True):
    dtype, width = cache_row_width(shape)
    _need(cache, dtype, name, gpu=gpu)
    if cache.shape[-1] != width:
        raise MlaError(f"{name} rows must hold {width} {dtype} values for this cache format")
    return width


def default_rope() -> MlaRopeParams:
    p = MlaRopeParams()
    _check(library().mla_default_rope(ctypes.byref(p)), "mla_default_rope")
    return p


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, dtype, name, last_contig=True, shape=None, device=None, gpu=True):
    """Type, contiguity, (optionally) exact shape and device of a tensor argument; ``gpu=False``
    leaves the GPU check to the caller (which then checks the common device once)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise MlaError(f"{name} must be {dtype} (got {t.dtype})")
    if last_contig and not t.is_contiguous():
        raise MlaError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MlaError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if device is not None and t.device != device:
        raise MlaError(f"{name} is on {t.device}, the other arguments on {device}")
    if gpu and t.device.type != "cuda":
        raise MlaError(f"{name} must be on the GPU (got {t.device})")


def _rows2d(x, name):
    if x.dtype != torch.bfloat16 or x.device.type != "cuda":
        raise MlaError(f"{name} must be a bf16 GPU tensor")
    if x.dim() == 1:
        return x.view(1, -1)
    if x.is_contiguous():
        return x.reshape(-1, x.shape[-1])
    if x.dim() == 2 and x.stride(1) == 1:
        return x
    raise MlaError(f"{name} must be contiguous or a 2-D row-strided view")


def mla_rope_yarn(src: torch.Tensor, positions: torch.Tensor, dst: torch.Tensor | None = None,
                  params: MlaRopeParams | None = None, stream=None) -> torch.Tensor:
    """dst rows = YaRN RoPE of src rows (first 64 elements) at ``positions``.

    Rows run along the last dimension; ``dst`` defaults to ``src`` (in place).
    """
    _need(positions, torch.int32, "positions")
    s2 = _rows2d(src, "src")
    d2 = s2 if dst is None else _rows2d(dst, "dst")
    n = s2.shape[0]
    if d2.shape[0] != n or positions.numel() != n:
        raise MlaError(f"src has {n} rows, dst {d2.shape[0]}, positions {positions.numel()}")
    p = params if params is not None else default_rope()
    _check(library().mla_rope_yarn(ctypes.byref(p), _ptr(s2), s2.stride(0), _ptr(d2), d2.stride(0),
                                   _ptr(positions), n, _stream(stream)), "mla_rope_yarn")
    return src if dst is None else dst


def mla_cache_append(cache: torch.Tensor, c_kv: torch.Tensor, k_pe: torch.Tensor,
                     slot_mapping: torch.Tensor, shape: MlaShape | None = None, stream=None):
    """cache row[slot] = [c_kv row | k_pe row] (a bit copy for bf16 rows, quantised latent for
    fp8 rows); slot < 0 skips."""
    s = shape if shape is not None else default_shape()
    width = _check_cache(cache, s)
    _need(slot_mapping, torch.int64, "slot_mapping", device=cache.device)
    for t, name in ((c_kv, "c_kv"), (k_pe, "k_pe")):
        if t.dtype != torch.bfloat16 or t.device.type != "cuda" or t.dim() != 2 or t.stride(1) != 1:
            raise MlaError(f"{name} must be a 2-D bf16 GPU tensor with unit column stride")
        if t.device != cache.device:
            raise MlaError(f"{name} is on {t.device}, the cache on {cache.device}")
    n = c_kv.shape[0]
    if k_pe.shape[0] != n or slot_mapping.numel() != n:
        raise MlaError("c_kv, k_pe and slot_mapping need the same number of rows")
    num_slots = cache.numel() // width
    _check(library().mla_cache_append(ctypes.byref(s), _ptr(cache), num_slots, _ptr(c_kv), c_kv.stride(0),
                                      _ptr(k_pe), k_pe.stride(0), _ptr(slot_mapping), n, _stream(stream)),
           "mla_cache_append")


def mla_decode_workspace_size(B: int, Sq: int, max_ctx_len: int, kv_chunk: int = 0,
                              shape: MlaShape | None = None) -> int:
    s = shape if shape is not None else default_shape()
    out = ctypes.c_size_t()
    _check(library().mla_decode_workspace_size(ctypes.byref(s), B, Sq, max_ctx_len, kv_chunk,
                                               ctypes.byref(out)), "mla_decode_workspace_size")
    return out.value


def mla_decode_auto_chunk(B: int, Sq: int, max_ctx_len: int) -> int:
    out = _I32()
    _check(library().mla_decode_auto_chunk(B, Sq, max_ctx_len, ctypes.byref(out)), "mla_decode_auto_chunk")
    return out.value


def _decode_io(q_nope, q_pe, w_kv_b, ctx_lens, out, lse, workspace, B, Sq, max_ctx_len, kv_chunk, shape,
               cache=None, block_table=None, need_workspace=True):
    _need(q_nope, torch.bfloat16, "q_nope", shape=(B, Sq, 32, 128), gpu=False)
    dev = q_nope.device
    _need(q_pe, torch.bfloat16, "q_pe", shape=(B, Sq, 32, 64), device=dev, gpu=False)
    _need(w_kv_b, torch.bfloat16, "w_kv_b", shape=(8192, 512), device=dev, gpu=False)
    _need(ctx_lens, torch.int32, "ctx_lens", shape=(B,), device=dev, gpu=False)
    for t, name in ((cache, "cache"), (block_table, "block_table")):
        if t is not None and t.device != dev:
            raise MlaError(f"{name} is on {t.device}, q_nope on {dev}")
    if out is not None:
        _need(out, torch.bfloat16, "out", shape=(B, Sq, 32, 128), device=dev, gpu=False)
    if lse is not None:
        _need(lse, torch.float32, "lse", shape=(B, Sq, 32), device=dev, gpu=False)
    if dev.type != "cuda":
        raise MlaError(f"the arguments must be on the GPU (got {dev})")
    if out is None:
        out = torch.empty((B, Sq, 32, 128), dtype=torch.bfloat16, device=dev)
    s = shape if shape is not None else default_shape()
    if need_workspace:
        need = mla_decode_workspace_size(B, Sq, max_ctx_len, kv_chunk, s)
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        _need(workspace, torch.uint8, "workspace", device=dev)
    return out, lse, workspace, s


def mla_decode(q_nope, q_pe, w_kv_b, cache, ctx_lens, max_ctx_len: int, kv_chunk: int = 0,
               out=None, lse=None, workspace=None, shape: MlaShape | None = None, stream=None):
    """Decode against a contiguous cache [B, stride, row]; returns (out, lse)."""
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    width = _check_cache(cache, shape if shape is not None else default_shape(), gpu=False)
    if cache.dim() != 3 or cache.shape[0] != B:
        raise MlaError(f"cache must be [B, stride, {width}]")
    out, lse, workspace, s = _decode_io(q_nope, q_pe, w_kv_b, ctx_lens, out, lse, workspace, B, Sq,
                                        max_ctx_len, kv_chunk, shape, cache=cache)
    _check(library().mla_decode(ctypes.byref(s), _ptr(q_nope), _ptr(q_pe), _ptr(w_kv_b), _ptr(cache),
                                cache.shape[1], _ptr(ctx_lens), max_ctx_len, B, Sq, kv_chunk, _ptr(out),
                                _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)),
           "mla_decode")
    return out, lse


def mla_decode_paged(q_nope, q_pe, w_kv_b, cache, block_table, ctx_lens, max_ctx_len: int,
                     kv_chunk: int = 0, out=None, lse=None, workspace=None,
                     shape: MlaShape | None = None, stream=None):
    """Decode against a paged cache [num_pages, 64, row]; returns (out, lse)."""
    width = _check_cache(cache, shape if shape is not None else default_shape(), gpu=False)
    _need(block_table, torch.int32, "block_table", gpu=False)
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    if cache.dim() != 3 or cache.shape[1] != 64:
        raise MlaError(f"cache must be [num_pages, 64, {width}]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise MlaError("block_table must be [B, max_pages_per_seq]")
    out, lse, workspace, s = _decode_io(q_nope, q_pe, w_kv_b, ctx_lens, out, lse, workspace, B, Sq,
                                        max_ctx_len, kv_chunk, shape, cache=cache, block_table=block_table)
    _check(library().mla_decode_paged(ctypes.byref(s), _ptr(q_nope), _ptr(q_pe), _ptr(w_kv_b), _ptr(cache),
                                      cache.shape[0], _ptr(block_table), block_table.shape[1],
                                      _ptr(ctx_lens), max_ctx_len, B, Sq, kv_chunk, _ptr(out), _ptr(lse),
                                      _ptr(workspace), workspace.numel(), _stream(stream)),
           "mla_decode_paged")
    return out, lse


def mla_decode_step(q_nope, q_pe, c_kv_new, k_pe_new, w_kv_b, cache, ctx_lens, max_ctx_len: int,
                    kv_chunk: int = 0, block_table=None, out=None, lse=None, workspace=None,
                    rope: MlaRopeParams | None = None, shape: MlaShape | None = None, stream=None):
    """One fused decode step: rotate q_pe and the new rope rows at p = L_b - Sq + j, write the new
    tokens' rows [c_kv_new | rot(k_pe_new)] into the cache, then decode.  q_pe and k_pe_new are
    NOT rotated.  ``block_table`` selects the paged layout [num_pages, 64, 576]; otherwise the
    cache is contiguous [B, stride, row].  Returns (out, lse)."""
    width = _check_cache(cache, shape if shape is not None else default_shape(), gpu=False)
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    for t, name, width in ((c_kv_new, "c_kv_new", 512), (k_pe_new, "k_pe_new", 64)):
        if t.dtype != torch.bfloat16 or t.device.type != "cuda" or t.dim() != 2 or t.stride(1) != 1:
            raise MlaError(f"{name} must be a 2-D bf16 GPU tensor with unit column stride")
        if t.shape[0] != B * Sq or t.shape[1] < width:
            raise MlaError(f"{name} must have B*Sq rows of at least {width} values")
    for t, name in ((c_kv_new, "c_kv_new"), (k_pe_new, "k_pe_new")):
        if t.device != q_nope.device:
            raise MlaError(f"{name} is on {t.device}, q_nope on {q_nope.device}")
    out, lse, workspace, s = _decode_io(q_nope, q_pe, w_kv_b, ctx_lens, out, lse, workspace, B, Sq,
                                        max_ctx_len, kv_chunk, shape, cache=cache, block_table=block_table)
    r = rope if rope is not None else default_rope()
    lib = library()
    if block_table is None:
        if cache.dim() != 3 or cache.shape[0] != B:
            raise MlaError(f"cache must be [B, stride, {width}]")
        code = lib.mla_decode_step(ctypes.byref(s), ctypes.byref(r), _ptr(q_nope), _ptr(q_pe), _ptr(c_kv_new),
                                   c_kv_new.stride(0), _ptr(k_pe_new), k_pe_new.stride(0), _ptr(w_kv_b),
                                   _ptr(cache), cache.shape[1], _ptr(ctx_lens), max_ctx_len, B, Sq, kv_chunk,
                                   _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream))
        _check(code, "mla_decode_step")
    else:
        _need(block_table, torch.int32, "block_table")
        if cache.dim() != 3 or cache.shape[1] != 64:
            raise MlaError(f"cache must be [num_pages, 64, {width}]")
        if block_table.dim() != 2 or block_table.shape[0] != B:
            raise MlaError("block_table must be [B, max_pages_per_seq]")
        code = lib.mla_decode_step_paged(ctypes.byref(s), ctypes.byref(r), _ptr(q_nope), _ptr(q_pe),
                                         _ptr(c_kv_new), c_kv_new.stride(0), _ptr(k_pe_new), k_pe_new.stride(0),
                                         _ptr(w_kv_b), _ptr(cache), cache.shape[0], _ptr(block_table),
                                         block_table.shape[1], _ptr(ctx_lens), max_ctx_len, B, Sq, kv_chunk,
                                         _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
                                         _stream(stream))
        _check(code, "mla_decode_step_paged")
    return out, lse


def mla_prefill_workspace_size(ctx_len: int, shape: MlaShape | None = None) -> int:
    s = shape if shape is not None else default_shape()
    out = ctypes.c_size_t()
    _check(library().mla_prefill_workspace_size(ctypes.byref(s), ctx_len, ctypes.byref(out)),
           "mla_prefill_workspace_size")
    return out.value


def mla_prefill(q_nope, q_pe, w_kv_b, cache, ctx_len: int, out=None, lse=None, workspace=None,
                shape: MlaShape | None = None, stream=None):
    """Chunked prefill of one sequence: q_nope [Tq, 32, 128], q_pe [Tq, 32, 64] (rotated) at
    positions ctx_len - Tq + j, cache [>= ctx_len, 576] bf16 rows; returns (out, lse)."""
    Tq = q_nope.shape[0] if isinstance(q_nope, torch.Tensor) and q_nope.dim() > 0 else 0
    _need(q_nope, torch.bfloat16, "q_nope", shape=(Tq, 32, 128), gpu=False)
    dev = q_nope.device
    _need(q_pe, torch.bfloat16, "q_pe", shape=(Tq, 32, 64), device=dev, gpu=False)
    _need(w_kv_b, torch.bfloat16, "w_kv_b", shape=(8192, 512), device=dev, gpu=False)
    s = shape if shape is not None else default_shape()
    width = _check_cache(cache, s, gpu=False)
    if cache.device != dev:
        raise MlaError(f"cache is on {cache.device}, q_nope on {dev}")
    if cache.dim() != 2 or cache.shape[0] < ctx_len:
        raise MlaError(f"cache must be [>= ctx_len, {width}]")
    if out is not None:
        _need(out, torch.bfloat16, "out", shape=(Tq, 32, 128), device=dev, gpu=False)
    if lse is not None:
        _need(lse, torch.float32, "lse", shape=(Tq, 32), device=dev, gpu=False)
    if dev.type != "cuda":
        raise MlaError(f"the arguments must be on the GPU (got {dev})")
    if out is None:
        out = torch.empty((Tq, 32, 128), dtype=torch.bfloat16, device=dev)
    need = mla_prefill_workspace_size(ctx_len, s)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    _need(workspace, torch.uint8, "workspace", device=dev)
    _check(library().mla_prefill(ctypes.byref(s), _ptr(q_nope), _ptr(q_pe), _ptr(w_kv_b), _ptr(cache), ctx_len,
                                 Tq, _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)),
           "mla_prefill")
    return out, lse


def mla_timing_enable(max_calls: int):
    """Record HIP events around the split-KV kernel of the next max_calls decode calls."""
    _check(library().mla_timing_enable(max_calls), "mla_timing_enable")


def mla_timing_collect():
    """(summed split-KV kernel milliseconds, timed decode calls); waits for the events."""
    ms, n = ctypes.c_double(), _I32()
    _check(library().mla_timing_collect(ctypes.byref(ms), ctypes.byref(n)), "mla_timing_collect")
    return ms.value, n.value


def mla_timing_disable():
    _check(library().mla_timing_disable(), "mla_timing_disable")


READ_PROBE_SINK_INTS = 8192   # MLA_READ_PROBE_SINK_INTS


def mla_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """One streaming read of all of `buf` (a contiguous device tensor, a multiple of 16 bytes);
    `sink` is a device int32 tensor of READ_PROBE_SINK_INTS elements that receives the digests."""
    if not (buf.is_cuda and buf.is_contiguous()):
        raise MlaError("buf: contiguous device tensor required")
    _need(sink, torch.int32, "sink")
    if sink.numel() < READ_PROBE_SINK_INTS:
        raise MlaError(f"sink: {READ_PROBE_SINK_INTS} int32 elements required")
    _check(library().mla_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), _stream(stream)),
           "mla_read_probe")


def mla_decode_step_paged_noalloc(q_nope, q_pe, c_kv_new, k_pe_new, w_kv_b, cache, block_table, ctx_lens,
                                  max_ctx_len: int, out, lse=None, kv_chunk: int = 0,
                                  rope: MlaRopeParams | None = None, shape: MlaShape | None = None, stream=None):
    """mla_decode_step on a paged cache with no workspace argument and no allocation: the library
    takes the workspace from its static device scratch (STATIC_SCRATCH_BYTES); ``out`` (and
    ``lse`` if wanted) must be given.  Calls that overlap on one device race on that scratch."""
    if out is None:
        raise MlaError("out must be given: the no-allocation entry point allocates nothing")
    width = _check_cache(cache, shape if shape is not None else default_shape())
    B, Sq = q_nope.shape[0], q_nope.shape[1]
    for t, name, w in ((c_kv_new, "c_kv_new", 512), (k_pe_new, "k_pe_new", 64)):
        if t.dtype != torch.bfloat16 or t.device.type != "cuda" or t.dim() != 2 or t.stride(1) != 1:
            raise MlaError(f"{name} must be a 2-D bf16 GPU tensor with unit column stride")
        if t.shape[0] != B * Sq or t.shape[1] < w:
            raise MlaError(f"{name} must have B*Sq rows of at least {w} values")
        if t.device != q_nope.device:
            raise MlaError(f"{name} is on {t.device}, q_nope on {q_nope.device}")
    _need(block_table, torch.int32, "block_table")
    if cache.dim() != 3 or cache.shape[1] != 64:
        raise MlaError(f"cache must be [num_pages, 64, {width}]")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise MlaError("block_table must be [B, max_pages_per_seq]")
    out, lse, _, s = _decode_io(q_nope, q_pe, w_kv_b, ctx_lens, out, lse, None, B, Sq, max_ctx_len, kv_chunk,
                                shape, cache=cache, block_table=block_table, need_workspace=False)
    r = rope if rope is not None else default_rope()
    _check(library().mla_decode_step_paged_noalloc(
        ctypes.byref(s), ctypes.byref(r), _ptr(q_nope), _ptr(q_pe), _ptr(c_kv_new), c_kv_new.stride(0),
        _ptr(k_pe_new), k_pe_new.stride(0), _ptr(w_kv_b), _ptr(cache), cache.shape[0], _ptr(block_table),
        block_table.shape[1], _ptr(ctx_lens), max_ctx_len, B, Sq, kv_chunk, _ptr(out), _ptr(lse), _stream(stream)),
        "mla_decode_step_paged_noalloc")
    return out, lse


def mla_device_faults(clear: bool = False) -> int:
    """The current device's fault word (FAULT_* bits raised by the kernels since it was last
    cleared), read after all work on the device has finished; ``clear`` resets it."""
    v = ctypes.c_uint32()
    _check(library().mla_device_faults(ctypes.byref(v), 1 if clear else 0), "mla_device_faults")
    return v.value


def mla_check_decode_inputs(ctx_lens, Sq: int, max_ctx_len: int, block_table=None, num_pages: int = 0) -> int:
    """FAULT_* bits the decode kernels would raise for these host arrays (numpy or CPU tensors):
    ctx_lens int32 [B], block_table int32 [B, max_pages] or None (contiguous layout)."""
    import numpy as np
    lens = np.ascontiguousarray(np.asarray(ctx_lens, dtype=np.int32))
    B = lens.shape[0]
    bt, mp = None, 0
    if block_table is not None:
        bt = np.ascontiguousarray(np.asarray(block_table, dtype=np.int32))
        if bt.ndim != 2 or bt.shape[0] != B:
            raise MlaError("block_table must be [B, max_pages_per_seq]")
        mp = bt.shape[1]
    v = ctypes.c_uint32()
    _check(library().mla_check_decode_inputs(B, Sq, max_ctx_len, lens.ctypes.data_as(_P),
                                             None if bt is None else bt.ctypes.data_as(_P), mp, num_pages,
                                             ctypes.byref(v)), "mla_check_decode_inputs")
    return v.value


def mla_check_slot_mapping(slot_mapping, num_slots: int) -> int:
    """FAULT_SLOT if a slot of this host array (int64) is at or beyond num_slots, else 0."""
    import numpy as np
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64))
    v = ctypes.c_uint32()
    _check(library().mla_check_slot_mapping(sm.ctypes.data_as(_P), sm.size, num_slots, ctypes.byref(v)),
           "mla_check_slot_mapping")
    return v.value
