"""Parity at the full workload sizes, in the launch configuration the
benchmark times (the fused decode step, kv_chunk as the benchmark passes it).

The oracle computes sampled outputs one sequence at a time: every head of
the sampled sequences through the absorbed fp64 reference (equal to the
un-absorbed definition up to rounding, which the CPU tests pin), and two
heads of the 32K workload through the un-absorbed definition itself.
Host inputs come from ``synth`` only.
"""
import numpy as np
import pytest
import torch

from synth.configs import workload
from mla_latent_kv_absorbed_amd.workload import DeviceWorkload

from oracle_inputs import compare, expected

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ALL_HEADS = list(range(32))
_REF = {}


def reference(wl, layer, b, heads, absorbed=True):
    key = (wl.index, layer, b, tuple(heads), absorbed)
    if key not in _REF:
        _REF[key] = expected(wl.seed, layer, wl.lens[b], wl.sq, b, heads=heads, absorbed=absorbed)
    return _REF[key]


def run_step(k, layer, kv_chunk=None):
    wl = workload(k)
    dw = DeviceWorkload(wl, device=DEV, kv_chunk=kv_chunk)
    li = dw.build_layer(layer)
    lse = torch.empty((dw.B, dw.Sq, 32), dtype=torch.float32, device=DEV)
    out, lse = dw.step(li, lse=lse)
    torch.cuda.synchronize()
    go = out.float().cpu().numpy().astype(np.float64)
    gl = lse.cpu().numpy()
    del li, dw
    torch.cuda.empty_cache()
    return wl, go, gl


def check(wl, layer, go, gl, seqs, heads=ALL_HEADS, absorbed=True):
    for b in seqs:
        ref_o, ref_l = reference(wl, layer, b, heads, absorbed)
        stats = compare(go[b][:, heads], gl[b][:, heads], ref_o, ref_l)
        print(f"{wl.name} layer {layer} seq {b} (L={wl.lens[b]}): max_abs={stats[0]:.2e} "
              f"rel_l2={stats[1]:.2e} lse={stats[2]:.2e}", flush=True)


@pytest.mark.parametrize("layer", [0, 39])
def test_ctx32k_b1(layer):
    wl, go, gl = run_step(1, layer)
    check(wl, layer, go, gl, [0])
    if layer == 0:
        check(wl, layer, go, gl, [0], heads=[0, 31], absorbed=False)


def test_paged_b16_ctx64k():
    wl, go, gl = run_step(2, 0)
    check(wl, 0, go, gl, [0, 7, 15])


@pytest.mark.parametrize("kv_chunk", [4096, 0])
def test_ctx256k_b1(kv_chunk):
    wl, go, gl = run_step(3, 0, kv_chunk=kv_chunk)
    check(wl, 0, go, gl, [0])


def test_mtp_verify_b32_sq2():
    wl, go, gl = run_step(4, 0)
    lens = np.array(wl.lens)
    seqs = sorted({int(lens.argmin()), int(lens.argmax()), 5, 17})
    check(wl, 0, go, gl, seqs)


@pytest.mark.parametrize("k", [5, 7])
def test_mtp_verify_b32_deeper(k):
    # 4 and 3 query tokens per sequence: every query group of a split in one launch
    wl, go, gl = run_step(k, 0)
    lens = np.array(wl.lens)
    seqs = sorted({int(lens.argmin()), int(lens.argmax()), 9})
    check(wl, 0, go, gl, seqs)


def test_ctx512k_b1():
    wl, go, gl = run_step(6, 0)
    check(wl, 0, go, gl, [0])
