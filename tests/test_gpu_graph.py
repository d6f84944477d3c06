"""HIP-graph capture of the decode step, the way a serving loop replays a whole
step: a graph of several layers' fused steps (RoPE, append, decode) is replayed
again and again with other work between the replays (an eager step of another
batch on the same workspace or static scratch, the workspace overwritten, the
outputs overwritten with NaN), and every replay gives bitwise the eager step's
outputs, LSE values and cache rows."""
import pytest
import torch

from synth.configs import Workload

import mla_latent_kv_absorbed_amd as M
from mla_latent_kv_absorbed_amd.workload import DeviceWorkload

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LAYERS = 3
REPLAYS = 4


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("entry", ["workspace", "noalloc"])
def test_graph_replays_equal_the_eager_step(entry, cache_dtype):
    M.mla_device_faults(clear=True)
    dw = DeviceWorkload(Workload(111, "graph-a", 5, 2, LAYERS, (5000, 70, 1500, 2, 900), True), device=DEV,
                        cache_dtype=cache_dtype)
    dwo = DeviceWorkload(Workload(112, "graph-b", 3, 3, 1, (2600, 9, 400), True), device=DEV,
                         cache_dtype=cache_dtype)
    layers = [dw.build_layer(layer) for layer in range(LAYERS)]
    lo = dwo.build_layer(0)
    B, Sq = dw.B, dw.Sq
    outs = [torch.empty((B, Sq, 32, 128), dtype=torch.bfloat16, device=DEV) for _ in layers]
    lses = [torch.empty((B, Sq, 32), dtype=torch.float32, device=DEV) for _ in layers]
    out_o = torch.empty((dwo.B, dwo.Sq, 32, 128), dtype=torch.bfloat16, device=DEV)

    def run(w, li, out, lse):
        if entry == "noalloc":
            M.mla_decode_step_paged_noalloc(li.q_nope, li.q_pe_raw, li.new_c, li.new_kpe_raw, li.w_kv_b, li.cache,
                                            w.block_table, w.ctx_lens, w.max_ctx, out, lse=lse, shape=w.shape)
        else:
            w.step(li, out=out, lse=lse)

    def step():
        for li, o, l in zip(layers, outs, lses):
            run(dw, li, o, l)

    step()
    torch.cuda.synchronize()
    ref_o = [o.clone() for o in outs]
    ref_l = [l.clone() for l in lses]
    ref_c = [li.cache.clone() for li in layers]
    assert all(torch.isfinite(o.float()).all() for o in ref_o)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    for rep in range(REPLAYS):
        # other work on the same scratch (or workspace), then stale outputs
        run(dwo, lo, out_o, None)
        dw.workspace.fill_(0xFF)
        for o, l in zip(outs, lses):
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in range(LAYERS):
            assert torch.equal(outs[k].view(torch.int16), ref_o[k].view(torch.int16)), (rep, k)
            assert torch.equal(lses[k], ref_l[k]), (rep, k)
            assert torch.equal(layers[k].cache.view(torch.uint8), ref_c[k].view(torch.uint8)), (rep, k)
    del g
    assert M.mla_device_faults() == 0
