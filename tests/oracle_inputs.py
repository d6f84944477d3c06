"""Oracle-side view of a workload: host-generated inputs and expected outputs.

Everything here comes from ``synth`` (host generator) and ``oracle``; nothing
is read back from the GPU.
"""
import numpy as np

import oracle as O
import synth


def f(bits):
    return O.bf16_bits_to_float(bits)


def sequence_inputs(seed, layer, length, sq, b):
    """(q_nope, q_pe rotated, c_kv, k_pe rotated, w) of sequence b, fp64 arrays."""
    inv = O.yarn_inv_freq()
    c = f(synth.latent_bits(seed, layer, b, 0, length))
    k = O.round_to_bf16(O.rope_rotate(f(synth.kpe_bits(seed, layer, b, 0, length)), np.arange(length), inv))
    qn = f(synth.qnope_bits(seed, layer, b, sq))
    qpos = (length - sq + np.arange(sq))[:, None]
    qp = O.round_to_bf16(O.rope_rotate(f(synth.qpe_bits(seed, layer, b, sq)), qpos, inv))
    return qn, qp, c, k


_W_CACHE = {}


def weights(seed, layer):
    key = (seed, layer)
    if key not in _W_CACHE:
        _W_CACHE.clear()
        _W_CACHE[key] = f(synth.wkvb_bits(seed, layer))
    return _W_CACHE[key]


def expected(seed, layer, length, sq, b, heads=None, absorbed=False):
    """Oracle (out [Sq, H', 128], lse [Sq, H']) for sequence b."""
    qn, qp, c, k = sequence_inputs(seed, layer, length, sq, b)
    fn = O.mla_attention_absorbed if absorbed else O.mla_attention_unabsorbed
    return fn(qn, qp, c, k, weights(seed, layer), O.softmax_scale(), heads)


# Tolerances: outputs as stated for the path (bf16 outputs, fp32 accumulation).
# LSE: rounding the absorbed query q_lat (std ~0.5) to bf16 moves a score by
# rms ~0.145 * 0.5 * 1.1e-3 * sqrt(512) ~ 1.8e-3; the library corrects the LSE to
# first order with the fp32 residual, leaving second-order terms (< 1e-5) and
# fp32 rounding, so 5e-3 bounds the LSE with a wide margin.
OUT_MAX_ABS = 2e-2
OUT_REL_L2 = 5e-3
LSE_MAX_ABS = 5e-3


def compare(out_gpu, lse_gpu, out_ref, lse_ref, lse_tol=LSE_MAX_ABS, abs_tol=OUT_MAX_ABS):
    """Returns (max_abs, rel_l2, lse_max_abs); asserts the tolerances."""
    og = np.asarray(out_gpu, dtype=np.float64)
    d = og - out_ref
    max_abs = float(np.abs(d).max())
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(out_ref), 1e-30))
    lmax = float(np.abs(np.asarray(lse_gpu, dtype=np.float64) - lse_ref).max()) if lse_gpu is not None else 0.0
    assert np.isfinite(og).all(), "non-finite GPU output"
    assert max_abs <= abs_tol, f"max abs {max_abs}"
    assert rel <= OUT_REL_L2, f"rel L2 {rel}"
    assert lmax <= lse_tol, f"lse max abs {lmax}"
    return max_abs, rel, lmax


def sequence_inputs_fp8(seed, layer, length, sq, b):
    """As sequence_inputs, with the latent replaced by its 8-bit cache value
    (quantised by the oracle, dequantised exactly)."""
    qn, qp, c, k = sequence_inputs(seed, layer, length, sq, b)
    codes, scales = O.quantize_latent_fp8(c.astype(np.float32))
    return qn, qp, O.dequantize_latent_fp8(codes, scales), k


def expected_fp8(seed, layer, length, sq, b, heads=None, absorbed=False):
    """Oracle (out, lse) for sequence b over the 8-bit cache."""
    qn, qp, c, k = sequence_inputs_fp8(seed, layer, length, sq, b)
    fn = O.mla_attention_absorbed if absorbed else O.mla_attention_unabsorbed
    return fn(qn, qp, c, k, weights(seed, layer), O.softmax_scale(), heads)
