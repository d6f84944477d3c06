"""Chunked prefill (mla_prefill) against the oracle's un-absorbed definition.

Inputs come from ``synth`` on both sides: sequence 0 of the seed, Tq query
tokens at positions L - Tq .. L - 1, the chunk's own cache rows included.
Small cases compare every output with the fp64 un-absorbed oracle; the
full-size chunks (4096 new tokens on 32768- and 131072-token contexts, the
shapes the benchmark times) compare sampled rows, each against the oracle run
on that row's visible prefix.  The tolerances are those of the decode path.
"""
import numpy as np
import pytest
import torch

import oracle as O
from mla_latent_kv_absorbed_amd.workload import DevicePrefill

import mla_latent_kv_absorbed_amd as M

from oracle_inputs import compare, expected, sequence_inputs, weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def gpu_run(seed, L, Tq, layer=0, reps=1):
    dp = DevicePrefill(seed, L, Tq, device=DEV)
    li = dp.build_layer(layer)
    outs = []
    for _ in range(reps):
        lse = torch.empty((Tq, 32), dtype=torch.float32, device=DEV)
        out, lse = dp.run(li, lse=lse)
        torch.cuda.synchronize()
        outs.append((out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy(), out.clone()))
    del li, dp
    torch.cuda.empty_cache()
    return outs


# one token; exactly one and one-plus 256-token expansion tile; query tiles of
# 256 rows with a ragged last tile; a context that is all query tokens
@pytest.mark.parametrize("L,Tq", [(1024, 256), (333, 100), (200, 200), (777, 1), (130, 129), (1, 1), (256, 256),
                                  (257, 2), (2100, 600), (600, 600)])
def test_prefill_matches_the_unabsorbed_oracle(L, Tq):
    go, gl, _ = gpu_run(81, L, Tq, layer=1)[0]
    ref_o, ref_l = expected(81, 1, L, Tq, 0)
    s = compare(go, gl, ref_o, ref_l)
    print(f"prefill L={L} Tq={Tq}: max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}", flush=True)


def test_prefill_is_deterministic():
    runs = gpu_run(82, 700, 300, reps=2)
    assert torch.equal(runs[0][2], runs[1][2])
    assert np.array_equal(runs[0][1], runs[1][1])


def check_sampled_rows(seed, L, Tq, rows):
    go, gl, _ = gpu_run(seed, L, Tq)[0]
    qn, qp, c, k = sequence_inputs(seed, 0, L, Tq, 0)
    w = weights(seed, 0)
    for j in rows:
        Lj = L - Tq + j + 1
        ref_o, ref_l = O.mla_attention_absorbed(qn[j:j + 1], qp[j:j + 1], c[:Lj], k[:Lj], w, O.softmax_scale())
        s = compare(go[j:j + 1], gl[j:j + 1], ref_o, ref_l)
        print(f"prefill {Tq}/{L} row {j}: max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}", flush=True)


def test_prefill_fullsize_chunk4k_ctx32k_sampled_rows():
    check_sampled_rows(8, 32768, 4096, (0, 1, 255, 256, 2047, 4095))


def test_prefill_fullsize_chunk4k_ctx128k_sampled_rows():
    check_sampled_rows(8, 131072, 4096, (0, 1000, 4095))


def test_prefill_rows_seeing_one_to_three_tokens_over_many_seeds():
    # rows that see one, two or three tokens: no averaging of the expanded
    # keys' rounding in their LSE, the case that decides the fp16 expansion
    worst = 0.0
    for seed in range(90, 98):
        go, gl, _ = gpu_run(seed, 3, 3)[0]
        ref_o, ref_l = expected(seed, 0, 3, 3, 0)
        s = compare(go, gl, ref_o, ref_l)
        worst = max(worst, s[2])
    print(f"prefill rows of 1-3 tokens, 8 seeds: worst lse error {worst:.2e}", flush=True)


def test_prefill_raises_the_fp16_range_fault_and_stays_clear_otherwise():
    M.mla_device_faults(clear=True)
    gpu_run(85, 300, 100)
    assert M.mla_device_faults() == 0
    dp = DevicePrefill(85, 300, 100, device=DEV)
    li = dp.build_layer(0)
    li.q_nope[7, 3, 5] = 1.0e5          # beyond the largest fp16 (65504)
    dp.run(li)
    torch.cuda.synchronize()
    assert M.mla_device_faults(clear=True) & M.FAULT_FP16_RANGE
    del li, dp
    torch.cuda.empty_cache()


def test_prefill_long_chunk_from_scratch_sampled_rows():
    # a long chunk from an empty context: ragged last tiles, first rows seeing few tokens
    check_sampled_rows(83, 2100, 2100, (0, 1, 2, 63, 64, 255, 256, 1000, 2047, 2048, 2099))


def test_prefill_longest_context_sampled_rows():
    # the largest context the call accepts (2^20 tokens) with a 64-token chunk
    print("prefill 64 / 2^20: building", flush=True)
    check_sampled_rows(84, 1 << 20, 64, (0, 63))
