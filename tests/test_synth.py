"""Checks of the seeded input generator (host side): determinism, slicing,
distribution, rounding and page assignment."""
import numpy as np
import torch

import synth
from synth import configs


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 1234567: first outputs of the published generator
    # (state += GAMMA, then the finaliser).
    state = 1234567
    want = []
    for _ in range(3):
        state = (state + synth.GAMMA) & synth.MASK64
        want.append(synth._mix64_int(state))
    got = synth.draw_u64(1234567, np.arange(3, dtype=np.uint64))
    assert [int(x) for x in got] == want
    assert want[0] == 6457827717110365317   # published first output for seed 1234567


def test_slices_regenerate_identically():
    full = synth.latent_bits(3, 7, 2, 0, 50)
    part = synth.latent_bits(3, 7, 2, 20, 30)
    np.testing.assert_array_equal(full[20:30], part)
    assert not np.array_equal(synth.latent_bits(3, 8, 2, 0, 50), full)   # other layer
    assert not np.array_equal(synth.latent_bits(4, 7, 2, 0, 50), full)   # other seed


def test_normal_moments_and_weight_scale():
    z = synth.bf16_bits_to_f64(synth.latent_bits(0, 0, 0, 0, 400))
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    w = synth.bf16_bits_to_f64(synth.wkvb_bits(0, 0))
    assert abs(w.var() * 512 - 1.0) < 0.01


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(200000).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(synth.f64_to_bf16_bits(x.astype(np.float64)), want)


def test_block_tables_partition_the_pool():
    lens = [1, 63, 64, 65, 1000]
    bt, pool = synth.block_tables(5, lens)
    need = [(x + 63) // 64 for x in lens]
    assert pool == sum(need)
    used = np.concatenate([bt[b, :n] for b, n in enumerate(need)])
    assert sorted(used.tolist()) == list(range(pool))
    assert np.all(bt[0, 1:] == -1)
    bt2, _ = synth.block_tables(5, lens)
    np.testing.assert_array_equal(bt, bt2)


def test_workloads():
    w4 = configs.workload(4)
    assert len(w4.lens) == 32 and min(w4.lens) >= 4096 and max(w4.lens) <= 131072
    assert w4.lens == configs.workload(4).lens
    assert configs.workload(1).latent_bytes_per_layer == 37748736
    assert configs.workload(2).latent_bytes_per_layer == 1207959552
    assert configs.workload(3).latent_bytes_per_layer == 301989888
