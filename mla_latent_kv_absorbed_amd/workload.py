"""Device-resident decode (and chunked-prefill) inputs, built with the library itself.

For each layer: the seeded raw values (``synth.gpu``) are drawn straight into
device memory, the rope keys of all cached tokens are rotated by
``mla_rope_yarn`` at their positions and every row is written into the cache
(contiguous [B, stride, 576] or paged [pages, 64, 576]) by
``mla_cache_append``.  A decode step of one layer then runs the whole path on
the Sq new tokens of every sequence: RoPE of their query and key rope parts,
append of their cache rows and the decode, either fused in one
``mla_decode_step`` call (``step``) or as ``mla_rope_yarn``,
``mla_cache_append`` and ``mla_decode`` / ``mla_decode_paged`` (``step_unfused``).
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

import synth
import synth.gpu as sgpu
from synth.configs import Workload

from . import (CACHE_BF16, CACHE_FP8_E4M3, cache_row_width, default_shape, mla_cache_append, mla_decode,
               mla_decode_paged, mla_decode_step, mla_decode_workspace_size, mla_decode_auto_chunk, mla_prefill,
               mla_prefill_workspace_size, mla_rope_yarn)

BF16_NAN = 0x7FC1   # bit pattern written into unused cache slots when poisoning
FP8_NAN = 0x7F      # E4M3 NaN byte, the same for 8-bit cache rows


@dataclass
class LayerInputs:
    layer: int
    cache: torch.Tensor
    w_kv_b: torch.Tensor
    q_nope: torch.Tensor        # [B, Sq, 32, 128]
    q_pe_raw: torch.Tensor      # [B, Sq, 32, 64] before RoPE
    q_pe: torch.Tensor          # rotated (written by the step)
    new_c: torch.Tensor         # [B*Sq, 512] latent rows of the new tokens
    new_kpe_raw: torch.Tensor   # [B*Sq, 64] before RoPE
    new_kpe: torch.Tensor       # rotated (written by the step)


class DeviceWorkload:
    def __init__(self, wl: Workload, device: str = "cuda:0", paged: bool | None = None,
                 kv_chunk: int | None = None, poison: bool = False, permute_pages: bool | None = None,
                 cache_dtype: str = "bf16"):
        self.wl = wl
        self.fp8 = cache_dtype == "fp8"
        self.shape = default_shape(CACHE_FP8_E4M3 if self.fp8 else CACHE_BF16)
        self.cache_torch_dtype, self.row_width = cache_row_width(self.shape)
        self.dev = torch.device(device)
        self.B, self.Sq = wl.batch, wl.sq
        self.lens = [int(x) for x in wl.lens]
        self.max_ctx = max(self.lens)
        self.paged = wl.paged if paged is None else paged
        self.kv_chunk = wl.kv_chunk if kv_chunk is None else kv_chunk
        self.poison = poison
        self.seed = wl.seed
        B, Sq = self.B, self.Sq
        self.ctx_lens = torch.tensor(self.lens, dtype=torch.int32, device=self.dev)
        if self.paged:
            permute = wl.permute_pages if permute_pages is None else permute_pages
            bt, pool = synth.block_tables(self.seed, self.lens, 64, permute)
            self.block_table_host = bt
            self.block_table = torch.from_numpy(bt).to(self.dev)
            self.block_table64 = torch.from_numpy(bt.astype("int64")).to(self.dev)   # for slot arithmetic
            self.num_pages = pool
            self.cache_shape = (pool, 64, self.row_width)
        else:
            self.block_table_host = None
            self.block_table = None
            self.stride = self.max_ctx
            self.cache_shape = (B, self.stride, self.row_width)
        # positions of the queries (rows b, j, h) and of the new tokens (b, j)
        qpos, npos = [], []
        for b in range(B):
            for j in range(Sq):
                p = self.lens[b] - Sq + j
                npos.append(p)
                qpos.extend([p] * 32)
        self.q_pos = torch.tensor(qpos, dtype=torch.int32, device=self.dev)
        self.new_pos = torch.tensor(npos, dtype=torch.int32, device=self.dev)
        self.new_slots = self.slots_of(torch.arange(B, device=self.dev).repeat_interleave(Sq),
                                       torch.tensor(npos, dtype=torch.int64, device=self.dev))
        self.workspace_bytes = mla_decode_workspace_size(B, Sq, self.max_ctx, self.kv_chunk, self.shape)
        self.workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.dev)
        self.chunk_used = self.kv_chunk or mla_decode_auto_chunk(B, Sq, self.max_ctx)

    # ---- addressing
    def slots_of(self, b, t: torch.Tensor) -> torch.Tensor:
        """Cache slot of token t of sequence b (t an int64 tensor, b an int or an int64 tensor)."""
        if self.paged:
            pages = self.block_table64[b, t // 64]
            return pages * 64 + t % 64
        return b * self.stride + t

    # ---- construction
    def build_layer(self, layer: int) -> LayerInputs:
        B, Sq, dev, seed = self.B, self.Sq, self.dev, self.seed
        if self.poison and self.fp8:
            cache = torch.full(self.cache_shape, FP8_NAN, dtype=torch.uint8, device=dev)
        elif self.poison:
            cache = torch.full(self.cache_shape, 0, dtype=torch.int16, device=dev)
            cache.fill_(BF16_NAN)
            cache = cache.view(torch.bfloat16)
        else:
            cache = torch.empty(self.cache_shape, dtype=self.cache_torch_dtype, device=dev)
        for b, L in enumerate(self.lens):
            step = 1 << 20
            for t0 in range(0, L, step):
                n = min(step, L - t0)
                c = torch.empty((n, 512), dtype=torch.bfloat16, device=dev)
                k = torch.empty((n, 64), dtype=torch.bfloat16, device=dev)
                sgpu.latent(c, seed, layer, b, t0)
                sgpu.kpe(k, seed, layer, b, t0)
                pos = torch.arange(t0, t0 + n, dtype=torch.int32, device=dev)
                mla_rope_yarn(k, pos)
                slots = self.slots_of(b, torch.arange(t0, t0 + n, dtype=torch.int64, device=dev))
                mla_cache_append(cache, c, k, slots, shape=self.shape)
                del c, k
        w = torch.empty((8192, 512), dtype=torch.bfloat16, device=dev)
        sgpu.wkvb(w, seed, layer)
        q_nope = torch.empty((B, Sq, 32, 128), dtype=torch.bfloat16, device=dev)
        q_pe_raw = torch.empty((B, Sq, 32, 64), dtype=torch.bfloat16, device=dev)
        new_c = torch.empty((B * Sq, 512), dtype=torch.bfloat16, device=dev)
        new_kpe_raw = torch.empty((B * Sq, 64), dtype=torch.bfloat16, device=dev)
        for b, L in enumerate(self.lens):
            sgpu.qnope(q_nope[b], seed, layer, b)
            sgpu.qpe(q_pe_raw[b], seed, layer, b)
            sgpu.latent(new_c[b * Sq:(b + 1) * Sq], seed, layer, b, L - Sq)
            sgpu.kpe(new_kpe_raw[b * Sq:(b + 1) * Sq], seed, layer, b, L - Sq)
        return LayerInputs(layer, cache, w, q_nope, q_pe_raw, torch.empty_like(q_pe_raw), new_c,
                           new_kpe_raw, torch.empty_like(new_kpe_raw))

    # ---- one decode step of one layer (the whole hot path)
    def step(self, li: LayerInputs, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
             kv_chunk: int | None = None):
        """The fused step: one library call rotates, appends and decodes."""
        chunk = self.kv_chunk if kv_chunk is None else kv_chunk
        ws = self._workspace(chunk)
        return mla_decode_step(li.q_nope, li.q_pe_raw, li.new_c, li.new_kpe_raw, li.w_kv_b, li.cache,
                               self.ctx_lens, self.max_ctx, chunk, block_table=self.block_table,
                               out=out, lse=lse, workspace=ws, shape=self.shape)

    def step_unfused(self, li: LayerInputs, out: torch.Tensor | None = None, lse: torch.Tensor | None = None,
                     kv_chunk: int | None = None):
        """The same step as separate calls: RoPE of q and of the new keys, append, decode."""
        mla_rope_yarn(li.q_pe_raw, self.q_pos, dst=li.q_pe)
        mla_rope_yarn(li.new_kpe_raw, self.new_pos, dst=li.new_kpe)
        mla_cache_append(li.cache, li.new_c, li.new_kpe, self.new_slots, shape=self.shape)
        return self.decode(li, out, lse, kv_chunk)

    def _workspace(self, chunk: int) -> torch.Tensor:
        need = mla_decode_workspace_size(self.B, self.Sq, self.max_ctx, chunk, self.shape)
        if need > self.workspace.numel():
            self.workspace = torch.empty(need, dtype=torch.uint8, device=self.dev)
        return self.workspace

    def decode(self, li: LayerInputs, out=None, lse=None, kv_chunk: int | None = None):
        chunk = self.kv_chunk if kv_chunk is None else kv_chunk
        ws = self._workspace(chunk)
        if self.paged:
            return mla_decode_paged(li.q_nope, li.q_pe, li.w_kv_b, li.cache, self.block_table, self.ctx_lens,
                                    self.max_ctx, chunk, out=out, lse=lse, workspace=ws, shape=self.shape)
        return mla_decode(li.q_nope, li.q_pe, li.w_kv_b, li.cache, self.ctx_lens, self.max_ctx, chunk,
                          out=out, lse=lse, workspace=ws, shape=self.shape)


@dataclass
class PrefillInputs:
    layer: int
    cache: torch.Tensor        # bf16 [L, 576]: the sequence's rows, the chunk's own included
    w_kv_b: torch.Tensor       # bf16 [8192, 512]
    q_nope: torch.Tensor       # [Tq, 32, 128]
    q_pe: torch.Tensor         # [Tq, 32, 64], rotated at L - Tq + j


class DevicePrefill:
    """Device inputs of a chunked prefill: one sequence of L cached tokens whose last
    Tq are the chunk (synthetic, seeded as the decode workloads: sequence 0 of seed)."""

    def __init__(self, seed: int, L: int, Tq: int, device: str = "cuda:0"):
        self.seed, self.L, self.Tq = seed, L, Tq
        self.dev = torch.device(device)
        self.workspace = torch.empty(mla_prefill_workspace_size(L), dtype=torch.uint8, device=self.dev)
        self.q_pos = (torch.arange(Tq, dtype=torch.int32, device=self.dev) + (L - Tq)).repeat_interleave(32)

    def build_layer(self, layer: int) -> PrefillInputs:
        dev, L, Tq, seed = self.dev, self.L, self.Tq, self.seed
        cache = torch.empty((L, 576), dtype=torch.bfloat16, device=dev)
        step = 1 << 18
        for t0 in range(0, L, step):
            n = min(step, L - t0)
            c = torch.empty((n, 512), dtype=torch.bfloat16, device=dev)
            k = torch.empty((n, 64), dtype=torch.bfloat16, device=dev)
            sgpu.latent(c, seed, layer, 0, t0)
            sgpu.kpe(k, seed, layer, 0, t0)
            pos = torch.arange(t0, t0 + n, dtype=torch.int32, device=dev)
            mla_rope_yarn(k, pos)
            mla_cache_append(cache, c, k, torch.arange(t0, t0 + n, dtype=torch.int64, device=dev))
            del c, k
        w = torch.empty((8192, 512), dtype=torch.bfloat16, device=dev)
        sgpu.wkvb(w, seed, layer)
        q_nope = torch.empty((Tq, 32, 128), dtype=torch.bfloat16, device=dev)
        q_pe = torch.empty((Tq, 32, 64), dtype=torch.bfloat16, device=dev)
        sgpu.qnope(q_nope, seed, layer, 0)
        sgpu.qpe(q_pe, seed, layer, 0)
        mla_rope_yarn(q_pe.view(-1, 64), self.q_pos)
        return PrefillInputs(layer, cache, w, q_nope, q_pe)

    def run(self, li: PrefillInputs, out=None, lse=None):
        return mla_prefill(li.q_nope, li.q_pe, li.w_kv_b, li.cache, self.L, out=out, lse=lse,
                           workspace=self.workspace)

