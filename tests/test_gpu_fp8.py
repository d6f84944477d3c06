"""GPU parity of the 8-bit latent cache path (E4M3 codes, per-128 fp32 scales).

The cache writer must produce the oracle's bytes exactly; the decode must
match the oracle's attention over the dequantised latent within the same
tolerance as the bf16 path.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import synth.gpu as sgpu
from synth.configs import Workload, workload

import mla_latent_kv_absorbed_amd as M
from mla_latent_kv_absorbed_amd.workload import DeviceWorkload

from oracle_inputs import compare, expected_fp8, sequence_inputs_fp8, weights

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def fp8_shape():
    return M.default_shape(M.CACHE_FP8_E4M3)


def gpu_out(out):
    return out.float().cpu().numpy().astype(np.float64)


def test_fp8_append_bytes_match_the_oracle():
    n, num_slots = 700, 900
    c = torch.empty((n, 512), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((n, 64), dtype=torch.bfloat16, device=DEV)
    sgpu.latent(c, 11, 0, 0, 0)
    sgpu.kpe(k, 11, 0, 0, 0)
    # exponent range and special rows (all exact bf16 operations)
    c[1] *= 2.0 ** 20
    c[2] *= 2.0 ** -20
    c[3, 128:256] = 0.0          # an all-zero group
    c[4, :7] = -0.0
    c[5, 300] = 1e4              # one large value squeezes the group's others
    cache = torch.full((num_slots, 656), 0x7F, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(2)
    slots = rng.permutation(num_slots)[:n].astype(np.int64)
    slots[::9] = -1
    M.mla_cache_append(cache, c, k, torch.from_numpy(slots).to(DEV), shape=fp8_shape())
    got = cache.cpu().numpy()
    cb = c.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    kb = k.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    codes, scales = O.quantize_latent_fp8(O.bf16_bits_to_float(cb).astype(np.float32))
    want = O.fp8_cache_row_bytes(codes, scales, kb)
    live = slots >= 0
    np.testing.assert_array_equal(got[slots[live]], want[live])
    untouched = np.setdiff1d(np.arange(num_slots), slots[live])
    assert np.all(got[untouched] == 0x7F)


RAGGED = [
    (1, (1, 2, 63, 64, 65, 700)),
    (2, (2, 3, 64, 65, 129, 333)),
    (3, (3, 70, 200)),
    (4, (4, 100, 500)),
    (16, (16, 40, 300)),
    (2, (2500, 9)),   # chunk 0: 20 splits of 2 tiles dealt out tile by tile, the last tile partial
]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("sq,lens", RAGGED)
@pytest.mark.parametrize("chunk", [64, 0])
def test_fp8_ragged_batches(paged, sq, lens, chunk):
    wl = Workload(98, "fp8-ragged", len(lens), sq, 1, lens, True)
    dw = DeviceWorkload(wl, paged=paged, kv_chunk=chunk, poison=True, cache_dtype="fp8")
    li = dw.build_layer(2)
    lse = torch.empty((len(lens), sq, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    go, gl = gpu_out(out), lse.cpu().numpy()
    for b, L in enumerate(lens):
        ref_o, ref_l = expected_fp8(wl.seed, 2, L, sq, b)
        compare(go[b], gl[b], ref_o, ref_l)


@pytest.mark.parametrize("chunk", [0, 256])
def test_fp8_config0_all_heads(chunk):
    wl = workload(0)
    dw = DeviceWorkload(wl, kv_chunk=chunk, cache_dtype="fp8")
    li = dw.build_layer(0)
    lse = torch.empty((1, 1, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = expected_fp8(wl.seed, 0, 1024, 1, 0)
    s = compare(gpu_out(out[0]), lse[0].cpu().numpy(), ref_o, ref_l)
    print(f"fp8 config0 chunk={chunk}: max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}")


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_fused_step_equals_separate_calls_and_is_deterministic(paged):
    lens = (2, 65, 700, 130)      # the shortest context the contract allows: Sq tokens
    wl = Workload(99, "fp8-fused", len(lens), 2, 1, lens, True)
    res = []
    for fused in (True, False, True):
        dw = DeviceWorkload(wl, paged=paged, kv_chunk=64, cache_dtype="fp8")
        li = dw.build_layer(0)
        li.cache.view(-1, 656)[dw.new_slots] = 0x7F      # only the step's append fills these
        lse = torch.empty((len(lens), 2, 32), dtype=torch.float32, device=DEV)
        out, lse = (dw.step if fused else dw.step_unfused)(li, lse=lse)
        torch.cuda.synchronize()
        valid = torch.cat([dw.slots_of(torch.full((L,), b, dtype=torch.int64, device=DEV),
                                       torch.arange(L, dtype=torch.int64, device=DEV))
                           for b, L in enumerate(lens)])
        res.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy().copy(),
                    li.cache.view(-1, 656)[valid].cpu().numpy()))
    for r in res[1:]:
        np.testing.assert_array_equal(r[2], res[0][2])
        np.testing.assert_array_equal(r[0], res[0][0])
        np.testing.assert_array_equal(r[1], res[0][1])


@pytest.mark.parametrize("sq", [1, 3])   # one token per workgroup; two, with an odd last group
def test_fp8_paged_equals_contiguous_bitwise(sq):
    lens = (1000, 64, 130)
    wl = Workload(100, "fp8-same", len(lens), sq, 1, lens, True, permute_pages=True)
    outs = []
    for paged in (False, True):
        dw = DeviceWorkload(wl, paged=paged, kv_chunk=128, cache_dtype="fp8")
        li = dw.build_layer(0)
        lse = torch.empty((len(lens), sq, 32), dtype=torch.float32, device=DEV)
        o, l = dw.step(li, lse=lse)
        outs.append((o.view(torch.int16).cpu().numpy(), l.cpu().numpy().copy()))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("sq", [1, 2])
def test_fp8_score_jump_takes_the_second_pass(sq):
    L = 1500
    wl = Workload(101, "fp8-jump", 1, sq, 1, (L,), False, kv_chunk=1024)
    dw = DeviceWorkload(wl, kv_chunk=1024, cache_dtype="fp8")
    li = dw.build_layer(0)
    # the rope key of token 700 (bytes 528..656 of its row) set to bf16 256.0
    li.cache[0, 700, 528:].view(torch.bfloat16).fill_(256.0)
    lse = torch.empty((1, sq, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    qn, qp, c, k = sequence_inputs_fp8(wl.seed, 0, L, sq, 0)
    k[700] = 256.0
    ref_o, ref_l = O.mla_attention_unabsorbed(qn, qp, c, k, weights(wl.seed, 0), O.softmax_scale())
    assert (ref_l.max() - np.median(ref_l)) * 1.4427 > 64
    compare(gpu_out(out[0]), lse[0].cpu().numpy(), ref_o, ref_l)


def test_fp8_fullsize_ctx32k():
    wl = workload(1)
    dw = DeviceWorkload(wl, cache_dtype="fp8")
    li = dw.build_layer(0)
    lse = torch.empty((1, 1, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = expected_fp8(wl.seed, 0, 32768, 1, 0, absorbed=True)
    s = compare(gpu_out(out[0]), lse[0].cpu().numpy(), ref_o, ref_l)
    print(f"fp8 32K: max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}")


def _fp8_step(k):
    wl = workload(k)
    dw = DeviceWorkload(wl, kv_chunk=0, cache_dtype="fp8")   # the benchmark's launch configuration
    li = dw.build_layer(0)
    lse = torch.empty((dw.B, dw.Sq, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    go, gl = gpu_out(out), lse.cpu().numpy()
    del li, dw
    torch.cuda.empty_cache()
    return wl, go, gl


def test_fp8_fullsize_ctx256k_balanced():
    wl, go, gl = _fp8_step(3)
    ref_o, ref_l = expected_fp8(wl.seed, 0, wl.lens[0], 1, 0, absorbed=True)
    s = compare(go[0], gl[0], ref_o, ref_l)
    print(f"fp8 256K: max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}", flush=True)


def test_fp8_fullsize_verify_b32_sq2():
    wl, go, gl = _fp8_step(4)
    lens = np.array(wl.lens)
    for b in sorted({int(lens.argmin()), int(lens.argmax()), 5, 17}):
        ref_o, ref_l = expected_fp8(wl.seed, 0, wl.lens[b], wl.sq, b, absorbed=True)
        s = compare(go[b], gl[b], ref_o, ref_l)
        print(f"fp8 verify 32x2 seq {b} (L={wl.lens[b]}): max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}",
              flush=True)


def test_fp8_query_pieces_over_extreme_block_scales():
    # The 8-bit kernel takes the absorbed query as two E4M3 pieces with a
    # power-of-two scale per 32 columns.  Heads whose query is zero, below the
    # pieces' range (2^-120: taken as zero), small (2^-30) or large (2^3), and
    # one 32-column block of head 4's W_UK scaled by 2^-60 (a block far below
    # its row's others), against the oracle on the same inputs.
    lens = (70, 300)
    sq = 2
    wl = Workload(102, "fp8-qscale", len(lens), sq, 1, lens, True)
    dw = DeviceWorkload(wl, kv_chunk=64, cache_dtype="fp8")
    li = dw.build_layer(0)
    qscale = {0: 0.0, 1: 2.0 ** -120, 2: 2.0 ** -30, 3: 2.0 ** 3}
    qn_host = li.q_nope.double().cpu()
    for h, f in qscale.items():
        qn_host[:, :, h] *= f
    li.q_nope.copy_(qn_host.to(torch.bfloat16))
    li.w_kv_b.view(32, 256, 512)[4, :128, 64:96] *= 2.0 ** -60
    lse = torch.empty((len(lens), sq, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    go, gl = gpu_out(out), lse.cpu().numpy()
    w = weights(wl.seed, 0).copy()
    w.reshape(32, 256, 512)[4, :128, 64:96] *= 2.0 ** -60
    for b, L in enumerate(lens):
        qn, qp, c, k = sequence_inputs_fp8(wl.seed, 0, L, sq, b)
        for h, f in qscale.items():
            qn[:, h] *= f
        ref_o, ref_l = O.mla_attention_unabsorbed(qn, qp, c, k, w, O.softmax_scale())
        s = compare(go[b], gl[b], ref_o, ref_l)
        print(f"fp8 query scales seq {b}: max_abs={s[0]:.3e} rel_l2={s[1]:.3e} lse={s[2]:.3e}", flush=True)
