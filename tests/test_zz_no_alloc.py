"""The no-allocation decode entry point (mla_decode_step_paged_noalloc) gives
bitwise the results of mla_decode_step_paged with a caller's workspace: on two
calls in a row, the second with a smaller input (fewer sequences, shorter
contexts, fewer query tokens), so that the static scratch still holds the
first call's contents when the second runs."""
import pytest
import torch

from synth.configs import Workload

import mla_latent_kv_absorbed_amd as M
from mla_latent_kv_absorbed_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _both(wl, cache_dtype="bf16"):
    dw = DeviceWorkload(wl, device=DEV, paged=True, cache_dtype=cache_dtype)
    li = dw.build_layer(0)
    B, Sq = dw.B, dw.Sq
    res = []
    for noalloc in (False, True):
        cache = li.cache.clone()
        out = torch.full((B, Sq, 32, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, Sq, 32), float("nan"), dtype=torch.float32, device=DEV)
        if noalloc:
            M.mla_decode_step_paged_noalloc(li.q_nope, li.q_pe_raw, li.new_c, li.new_kpe_raw, li.w_kv_b, cache,
                                            dw.block_table, dw.ctx_lens, dw.max_ctx, out, lse=lse, shape=dw.shape)
        else:
            M.mla_decode_step(li.q_nope, li.q_pe_raw, li.new_c, li.new_kpe_raw, li.w_kv_b, cache, dw.ctx_lens,
                              dw.max_ctx, 0, block_table=dw.block_table, out=out, lse=lse, shape=dw.shape)
        torch.cuda.synchronize()
        res.append((out, lse, cache))
    (o1, l1, c1), (o2, l2, c2) = res
    assert torch.isfinite(o1.float()).all()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
    assert torch.equal(c1.view(torch.uint8), c2.view(torch.uint8))
    del li, dw


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_noalloc_step_equals_the_workspace_step_on_two_calls(cache_dtype):
    M.mla_device_faults(clear=True)
    # first call: 6 sequences x 3 query tokens, contexts up to 9,000 tokens
    _both(Workload(101, "noalloc-a", 6, 3, 1, (9000, 4100, 64, 700, 3, 2500), True), cache_dtype)
    # second, smaller: 2 sequences x 1 query token, short contexts
    _both(Workload(102, "noalloc-b", 2, 1, 1, (130, 1), True), cache_dtype)
    assert M.mla_device_faults() == 0


def test_noalloc_rejects_a_request_beyond_its_scratch():
    B, Sq, L = 4095, 16, 64
    assert M.mla_decode_workspace_size(B, Sq, L) > M.STATIC_SCRATCH_BYTES
    q = torch.zeros((B, Sq, 32, 128), dtype=torch.bfloat16, device=DEV)
    qp = torch.zeros((B, Sq, 32, 64), dtype=torch.bfloat16, device=DEV)
    new = torch.zeros((B * Sq, 576), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((8192, 512), dtype=torch.bfloat16, device=DEV)
    cache = torch.zeros((B, 64, 576), dtype=torch.bfloat16, device=DEV)
    bt = torch.arange(B, dtype=torch.int32, device=DEV).view(B, 1)
    lens = torch.full((B,), L, dtype=torch.int32, device=DEV)
    out = torch.empty((B, Sq, 32, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(M.MlaError, match="MLA_ERR_SCRATCH"):
        M.mla_decode_step_paged_noalloc(q, qp, new[:, :512], new[:, 512:], w, cache, bt, lens, L, out)
