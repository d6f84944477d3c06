"""GPU parity of the HIP path against the CPU oracle (small and medium sizes).

Every device call goes through the C ABI via the ctypes binding.  Inputs are
seeded: the GPU side draws them with the device generator and prepares the
cache with its own RoPE and append kernels; the oracle draws the same values
on the host and prepares them with its own fp64 RoPE.
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

from oracle_inputs import compare, expected, expected_fp8

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def gpu_out(out):
    return out.float().cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------------------
# generator twin, RoPE, append
# ---------------------------------------------------------------------------

def test_device_generator_matches_host_generator():
    c = torch.empty((300, 512), dtype=torch.bfloat16, device=DEV)
    sgpu.latent(c, 3, 5, 2, 1000)
    np.testing.assert_array_equal(bits(c), synth.latent_bits(3, 5, 2, 1000, 1300))
    q = torch.empty((2, 32, 64), dtype=torch.bfloat16, device=DEV)
    sgpu.qpe(q, 4, 7, 9)
    np.testing.assert_array_equal(bits(q), synth.qpe_bits(4, 7, 9, 2))
    w = torch.empty((8192, 512), dtype=torch.bfloat16, device=DEV)
    sgpu.wkvb(w, 1, 39)
    np.testing.assert_array_equal(bits(w), synth.wkvb_bits(1, 39))


def test_rope_matches_oracle_bit_exact():
    n = 4096
    raw = torch.empty((n, 64), dtype=torch.bfloat16, device=DEV)
    sgpu.kpe(raw, 0, 0, 0, 0)
    rng = np.random.default_rng(0)
    pos = np.concatenate([[0, 1, 4095, 4096, 131071, 262143], rng.integers(0, 262144, n - 6)]).astype(np.int32)
    dst = torch.empty_like(raw)
    M.mla_rope_yarn(raw, torch.from_numpy(pos).to(DEV), dst=dst)
    want = O.round_to_bf16(O.rope_rotate(O.bf16_bits_to_float(synth.kpe_bits(0, 0, 0, 0, n)), pos, O.yarn_inv_freq()))
    got = O.bf16_bits_to_float(bits(dst))
    mism = int((got != want).sum())
    # fp64 on both sides, one rounding to bf16: equal unless a value lies within
    # a few fp64 ulps of a bf16 rounding boundary
    assert mism <= 2, f"{mism} mismatches"
    assert np.abs(got - want).max() <= 2.0 ** -7 * np.abs(want).max()
    # in place gives the same bits
    M.mla_rope_yarn(raw, torch.from_numpy(pos).to(DEV))
    np.testing.assert_array_equal(bits(raw), bits(dst))


def test_rope_strided_rows_touch_only_the_rope_part():
    x = torch.zeros((10, 576), dtype=torch.bfloat16, device=DEV)
    sgpu.fill(x, 9, 2, 0, 0)
    before = bits(x).copy()
    view = x[:, 512:]
    M.mla_rope_yarn(view, torch.arange(10, dtype=torch.int32, device=DEV) * 1000)
    after = bits(x)
    np.testing.assert_array_equal(after[:, :512], before[:, :512])
    want = O.round_to_bf16(O.rope_rotate(O.bf16_bits_to_float(before[:, 512:]), np.arange(10) * 1000, O.yarn_inv_freq()))
    assert int((O.bf16_bits_to_float(after[:, 512:]) != want).sum()) <= 1


def test_cache_append_bit_exact_and_skips():
    num_slots = 500
    cache = torch.full((num_slots, 576), 0, dtype=torch.int16, device=DEV)
    cache.fill_(0x7FC1)
    cache = cache.view(torch.bfloat16)
    n = 300
    src = torch.randint(-32768, 32767, (n, 640), dtype=torch.int16, device=DEV).view(torch.bfloat16)
    c_kv = src[:, :512]            # row stride 640
    k_pe = src[:, 576:]            # offset rows, stride 640
    rng = np.random.default_rng(1)
    slots = rng.permutation(num_slots)[:n].astype(np.int64)
    slots[::7] = -1
    M.mla_cache_append(cache, c_kv, k_pe, torch.from_numpy(slots).to(DEV))
    got = bits(cache)
    s_host = bits(src)
    for i in range(n):
        if slots[i] >= 0:
            np.testing.assert_array_equal(got[slots[i], :512], s_host[i, :512])
            np.testing.assert_array_equal(got[slots[i], 512:], s_host[i, 576:640])
    untouched = np.setdiff1d(np.arange(num_slots), slots[slots >= 0])
    assert np.all(got[untouched] == 0x7FC1)


def test_paged_cache_rows_follow_the_block_table():
    wl = Workload(90, "paging", 3, 1, 1, (65, 200, 1), True)
    dw = DeviceWorkload(wl, poison=True)
    li = dw.build_layer(0)
    cache = bits(li.cache).reshape(-1, 576)
    inv = O.yarn_inv_freq()
    for b, L in enumerate(wl.lens):
        lat = synth.latent_bits(wl.seed, 0, b, 0, L)
        kr = O.round_to_bf16(O.rope_rotate(O.bf16_bits_to_float(synth.kpe_bits(wl.seed, 0, b, 0, L)), np.arange(L), inv))
        slots = O.paged_slot(dw.block_table_host[b], np.arange(L))
        np.testing.assert_array_equal(cache[slots, :512], lat)
        assert int((O.bf16_bits_to_float(cache[slots, 512:]) != kr).sum()) <= 1
    used = np.concatenate([O.paged_slot(dw.block_table_host[b], np.arange(L)) for b, L in enumerate(wl.lens)])
    unused = np.setdiff1d(np.arange(cache.shape[0]), used)
    assert len(unused) == 64 * dw.num_pages - sum(wl.lens) and np.all(cache[unused] == 0x7FC1)


# ---------------------------------------------------------------------------
# decode parity
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [0, 1024, 256, 64])
def test_config0_parity_all_heads(chunk):
    wl = workload(0)
    dw = DeviceWorkload(wl, kv_chunk=chunk)
    li = dw.build_layer(0)
    lse = torch.empty((1, 1, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    ref_o, ref_l = expected(wl.seed, 0, 1024, 1, 0)
    stats = compare(gpu_out(out[0]), lse[0].cpu().numpy(), ref_o, ref_l)
    print(f"config0 chunk={chunk}: max_abs={stats[0]:.3e} rel_l2={stats[1]:.3e} lse={stats[2]:.3e}")


RAGGED = [
    (1, (1, 2, 63, 64, 65, 700)),
    (2, (2, 3, 64, 65, 129, 333)),
    (3, (3, 70, 200)),
    (4, (4, 64, 1000)),
    (5, (5, 130)),
    (16, (16, 17, 300)),
    # with the balanced schedule (chunk 0) the 4,000- and 2,500-token sequences
    # get 32 and 20 splits of 2 tiles, dealt out tile by tile (every 32nd /
    # 20th tile from tile k), their last tiles partial; the 1,300-token one
    # gets 11 contiguous splits
    (1, (4000, 7)),
    (3, (3, 2500, 1300, 90)),
]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("sq,lens", RAGGED)
@pytest.mark.parametrize("chunk", [64, 128, 0])
def test_ragged_batches(paged, sq, lens, chunk):
    wl = Workload(91, "ragged", len(lens), sq, 1, lens, True)
    dw = DeviceWorkload(wl, paged=paged, kv_chunk=chunk, poison=True)
    li = dw.build_layer(2)
    lse = torch.empty((len(lens), sq, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    go, gl = gpu_out(out), lse.cpu().numpy()
    for b, L in enumerate(lens):
        ref_o, ref_l = expected(wl.seed, 2, L, sq, b)
        compare(go[b], gl[b], ref_o, ref_l)


def test_paged_equals_contiguous_bitwise_and_runs_are_deterministic():
    lens = (1000, 64, 130, 777)
    wl = Workload(92, "same", len(lens), 2, 1, lens, True, permute_pages=True)
    outs = []
    for paged in (False, True):
        dw = DeviceWorkload(wl, paged=paged, kv_chunk=128)
        li = dw.build_layer(0)
        lse = torch.empty((len(lens), 2, 32), dtype=torch.float32, device=DEV)
        o1, l1 = dw.step(li, lse=lse)
        o1, l1 = bits(o1), l1.cpu().numpy().copy()
        o2, l2 = dw.step(li, lse=lse)
        np.testing.assert_array_equal(bits(o2), o1)
        np.testing.assert_array_equal(l2.cpu().numpy(), l1)
        outs.append((o1, l1))
    np.testing.assert_array_equal(outs[0][0], outs[1][0])
    np.testing.assert_array_equal(outs[0][1], outs[1][1])


def test_chunk_size_changes_only_rounding():
    wl = Workload(93, "chunks", 2, 1, 1, (3000, 1200), False)
    dw = DeviceWorkload(wl)
    li = dw.build_layer(0)
    res = []
    for chunk in (64, 512, 4096):
        out, _ = dw.step(li, kv_chunk=chunk)
        res.append(gpu_out(out))
    for r in res[1:]:
        assert np.abs(r - res[0]).max() < 1e-2


def test_empty_batch_is_a_no_op():
    out = torch.full((0, 1, 32, 128), 1.0, dtype=torch.bfloat16, device=DEV)
    z = torch.empty((0, 1, 32, 128), dtype=torch.bfloat16, device=DEV)
    M.mla_decode(z, torch.empty((0, 1, 32, 64), dtype=torch.bfloat16, device=DEV),
                 torch.zeros((8192, 512), dtype=torch.bfloat16, device=DEV),
                 torch.zeros((0, 64, 576), dtype=torch.bfloat16, device=DEV),
                 torch.zeros((0,), dtype=torch.int32, device=DEV), 64, out=out)
    torch.cuda.synchronize()


def test_every_query_row_gets_its_rope_part_with_a_dirty_workspace():
    # Query rows r = 1, 2, 3 (mod 4) once kept stale workspace bytes in the
    # rope part of the absorbed query; a NaN-filled workspace exposes that.
    lens = (5, 9, 17, 33, 65, 100, 7)
    wl = Workload(94, "rows", len(lens), 2, 1, lens, True)
    dw = DeviceWorkload(wl, paged=True, kv_chunk=64)
    dw.workspace.view(torch.int16)[: dw.workspace.numel() // 2].fill_(0x7FC1)
    li = dw.build_layer(0)
    lse = torch.empty((len(lens), 2, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    go, gl = gpu_out(out), lse.cpu().numpy()
    for b, L in enumerate(lens):
        ref_o, ref_l = expected(wl.seed, 0, L, 2, b)
        compare(go[b], gl[b], ref_o, ref_l)


@pytest.mark.parametrize("sq", [1, 2])
def test_score_jump_beyond_headroom_takes_the_second_pass(sq):
    # Token 700's rope key is set to 256 in every dimension: for heads whose
    # q_pe sums positive its score is hundreds of log2 units above the first
    # tile's maximum, beyond the kernel's headroom, so the split is streamed a
    # second time with the true maxima as references.
    import oracle as O
    from oracle_inputs import sequence_inputs, weights
    L = 1500
    wl = Workload(95, "jump", 1, sq, 1, (L,), False, kv_chunk=1024)
    dw = DeviceWorkload(wl, kv_chunk=1024)
    li = dw.build_layer(0)
    li.cache[0, 700, 512:] = 256.0
    lse = torch.empty((1, sq, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    qn, qp, c, k = sequence_inputs(wl.seed, 0, L, sq, 0)
    k[700] = 256.0
    ref_o, ref_l = O.mla_attention_unabsorbed(qn, qp, c, k, weights(wl.seed, 0), O.softmax_scale())
    assert (ref_l.max() - np.median(ref_l)) * 1.4427 > 64     # the jump really exceeds the headroom
    compare(gpu_out(out[0]), lse[0].cpu().numpy(), ref_o, ref_l)


FUSED = [
    (1, (1, 65, 700)),
    (2, (2, 130, 64)),
    (3, (3, 200)),
    # 35 query rows: three 16-row blocks of the preparation kernel, whose four
    # rope columns take 4 rows each (the last block's partly empty)
    (5, (5, 70, 300, 64, 129, 200, 1000)),
]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("sq,lens", FUSED)
def test_fused_step_equals_separate_calls_bitwise(paged, sq, lens):
    # mla_decode_step (RoPE + append + decode in one call) against
    # mla_rope_yarn + mla_cache_append + mla_decode.  The new tokens' cache
    # rows are poisoned first, so only the step's own append can fill them.
    wl = Workload(96, "fused", len(lens), sq, 1, lens, True)
    res = []
    for fused in (True, False):
        dw = DeviceWorkload(wl, paged=paged, kv_chunk=64)
        li = dw.build_layer(1)
        li.cache.view(torch.int16).view(-1, 576)[dw.new_slots] = 0x7FC1
        lse = torch.empty((len(lens), sq, 32), dtype=torch.float32, device=DEV)
        out, lse = (dw.step if fused else dw.step_unfused)(li, lse=lse)
        torch.cuda.synchronize()
        valid = torch.cat([dw.slots_of(torch.full((L,), b, dtype=torch.int64, device=DEV),
                                       torch.arange(L, dtype=torch.int64, device=DEV))
                           for b, L in enumerate(lens)])
        res.append((bits(out), lse.cpu().numpy().copy(), bits(li.cache.view(-1, 576)[valid])))
    np.testing.assert_array_equal(res[0][2], res[1][2])   # every cached row of every sequence
    np.testing.assert_array_equal(res[0][0], res[1][0])
    np.testing.assert_array_equal(res[0][1], res[1][1])
    go = O.bf16_bits_to_float(res[0][0]).reshape(len(lens), sq, 32, 128)
    for b, L in enumerate(lens):
        ref_o, ref_l = expected(wl.seed, 1, L, sq, b)
        compare(go[b], res[0][1][b], ref_o, ref_l)


def test_balanced_schedule_over_many_short_sequences():
    # 300 sequences: the device-side schedule scans the lengths in two
    # 256-wide passes; every tenth sequence is checked against the oracle.
    rng = np.random.default_rng(7)
    lens = tuple(int(x) for x in rng.integers(1, 200, 300))
    wl = Workload(97, "many", len(lens), 1, 1, lens, True)
    dw = DeviceWorkload(wl, paged=True, kv_chunk=0)
    li = dw.build_layer(0)
    lse = torch.empty((len(lens), 1, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    go, gl = gpu_out(out), lse.cpu().numpy()
    for b in range(0, len(lens), 10):
        ref_o, ref_l = expected(wl.seed, 0, lens[b], 1, b)
        compare(go[b], gl[b], ref_o, ref_l)


def test_widest_batch_takes_the_schedules_serial_path():
    # B * Sq = 4095 * 16 = 65,520 rows (calls accept up to 65,535) and
    # B > 2,048 sequences, so the device schedule takes its serial path;
    # short ragged contexts, the balanced and a fixed split; a sample of
    # sequences (both sides of 2,048 among them) against the oracle.
    rng = np.random.default_rng(11)
    lens = tuple(int(x) for x in rng.integers(16, 200, 4095))
    wl = Workload(98, "widest", len(lens), 16, 1, lens, True)
    dw = DeviceWorkload(wl, paged=True, kv_chunk=0)
    li = dw.build_layer(0)
    print(f"built {len(lens)} sequences", flush=True)
    picks = sorted({0, 1, 2047, 2048, 2049, 4094} | {int(x) for x in rng.integers(0, 4095, 6)})
    idx = torch.tensor(picks, device=DEV)
    for chunk, run in ((0, dw.step), (64, dw.step_unfused)):
        lse = torch.empty((len(lens), 16, 32), dtype=torch.float32, device=DEV)
        out, lse = run(li, lse=lse, kv_chunk=chunk)
        torch.cuda.synchronize()
        go, gl = gpu_out(out[idx]), lse[idx].cpu().numpy()
        for i, b in enumerate(picks):
            ref_o, ref_l = expected(wl.seed, 0, lens[b], 16, b)
            compare(go[i], gl[i], ref_o, ref_l)
        print(f"chunk {chunk}: {len(picks)} sequences match", flush=True)
        del out, lse


@pytest.mark.parametrize("chunk", [0, 128])
def test_host_length_bound_above_the_lengths_changes_nothing(chunk):
    # max_ctx_len only sizes the workspace and the grid: a bound 8x the longest
    # context, with the cache rows at 8x the stride, gives bitwise the same
    # result (the schedule follows the actual lengths on the device)
    wl = Workload(99, "bound", 3, 2, 1, (700, 130, 1500), False)
    dw = DeviceWorkload(wl, paged=False, kv_chunk=chunk)
    li = dw.build_layer(0)
    ref, ref_lse = dw.step_unfused(li, lse=torch.empty((3, 2, 32), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    wide = torch.zeros((3, 8 * dw.stride, 576), dtype=torch.bfloat16, device=DEV)
    wide[:, :dw.stride] = li.cache
    out, lse = M.mla_decode(li.q_nope, li.q_pe, li.w_kv_b, wide, dw.ctx_lens, 8 * dw.max_ctx, chunk,
                            lse=torch.empty((3, 2, 32), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and torch.equal(lse, ref_lse)


def test_fp8_batch_above_the_schedules_lds_capacity():
    # 2,100 sequences (> 2,048: the serial schedule path) over the 8-bit cache
    rng = np.random.default_rng(12)
    lens = tuple(int(x) for x in rng.integers(1, 150, 2100))
    wl = Workload(96, "wide8", len(lens), 1, 1, lens, True)
    dw = DeviceWorkload(wl, paged=True, kv_chunk=0, cache_dtype="fp8")
    li = dw.build_layer(0)
    lse = torch.empty((len(lens), 1, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    picks = [0, 2047, 2048, 2099] + [int(x) for x in rng.integers(0, 2100, 4)]
    idx = torch.tensor(picks, device=DEV)
    go, gl = gpu_out(out[idx]), lse[idx].cpu().numpy()
    for i, b in enumerate(picks):
        ref_o, ref_l = expected_fp8(wl.seed, 0, lens[b], 1, b)
        compare(go[i], gl[i], ref_o, ref_l)


# ---------------------------------------------------------------------------
# streaming-read probe (a measurement aid): every word is read exactly once
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 3 << 20])
def test_read_probe_digests_xor_to_the_buffer_xor(nbytes):
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.to(DEV)
    sink = torch.full((M.READ_PROBE_SINK_INTS,), -1, dtype=torch.int32, device=DEV)
    M.mla_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(sink.cpu().numpy()) == np.bitwise_xor.reduce(host.numpy())
