"""The five MLA decode workloads (shapes only; values come from ``synth``).

Shape of every layer (Xing4.0-29B-A4B attention, from the model's config.json
as printed in "256K 长上下文真能本地用？Xing4.0 原生长上下文的工程代价拆解", §一,
and the Xing4_0Attention fields in "mHC+MLA+MTP 是什么？拆开给 Agent 用的百亿
MoE", section "MLA：256K 上下文的内存革命"): 32 heads, kv_lora_rank 512,
qk_nope 128, qk_rope 64, v_head 128, 40 layers.

The seed of workload k is k.  Query token j of sequence b sits at position
L_b - Sq + j and its latent row is already in the cache.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import loguniform_lengths


@dataclass(frozen=True)
class Workload:
    index: int
    name: str
    batch: int
    sq: int
    layers: int
    lens: tuple
    paged: bool
    kv_chunk: int = 0          # 0: let the library choose
    permute_pages: bool = True
    note: str = ""

    @property
    def seed(self) -> int:
        return self.index

    @property
    def latent_bytes_per_layer(self) -> int:
        return sum(self.lens) * 576 * 2


def workload(k: int) -> Workload:
    if k == 0:
        return Workload(0, "mla-1layer-b1-ctx1k", 1, 1, 1, (1024,), False, 0,
                        note="single layer, batch 1, 1 query token, context 1024")
    if k == 1:
        return Workload(1, "mla-decode-b1-ctx32k", 1, 1, 40, (32768,), False, 0,
                        note="40-layer decode step, batch 1, context 32768, contiguous cache")
    if k == 2:
        return Workload(2, "mla-paged-b16-ctx64k", 16, 1, 40, (65536,) * 16, True, 0,
                        note="batch 16 x 65536, 64-token pages from a permuted shared pool")
    if k == 3:
        return Workload(3, "mla-long-b1-ctx256k", 1, 1, 40, (262144,), False, 4096,
                        note="batch 1, context 262144, KV chunks of 4096 with LSE combine")
    if k == 4:
        lens = tuple(int(x) for x in loguniform_lengths(4, 32, 4096, 131072))
        return Workload(4, "mla-mtp-verify-b32-sq2", 32, 2, 40, lens, True, 0,
                        note="batch 32, 2 causal query tokens, log-uniform contexts in [4096, 131072]")
    # Beyond the five workloads above: deeper speculative verify (drafts of up
    # to 3 tokens, the --spec-draft-n-max 3 server setting of the
    # Swift-Qwen3.8-27B-GGUF page; the Xing4.0 pages' MTP drafting) and the
    # 512,000-token extension that "China Telecom's Xing4.0 Runs a 29B Coding
    # Agent on 19GB Locally" mentions, taken as 2^19 tokens with the same
    # YaRN parameters.
    if k in (5, 7):
        sq = 4 if k == 5 else 3
        lens = tuple(int(x) for x in loguniform_lengths(k, 32, 4096, 131072))
        return Workload(k, f"mla-mtp-verify-b32-sq{sq}", 32, sq, 40, lens, True, 0,
                        note=f"batch 32, {sq} causal query tokens, log-uniform contexts in [4096, 131072]")
    if k == 6:
        return Workload(6, "mla-long-b1-ctx512k", 1, 1, 40, (524288,), False, 0,
                        note="batch 1, context 524288 (positions past the 262144 of the YaRN table)")
    raise ValueError(f"no workload {k}")


ALL = (0, 1, 2, 3, 4)
EXTENDED = (5, 6, 7)
