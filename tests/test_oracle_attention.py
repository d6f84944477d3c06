"""Pins of the oracle's attention, split combine and paging.

Pins: brute force in pure Python on tiny shapes, special cases with a
closed-form answer (one token, equal scores, a dominant score), scipy's
softmax / logsumexp on a rope-only case, zeroed halves of kv_b_proj (which fix
the [k_nope | v] head order), causality of two query tokens, token
permutation and score-shift invariance, and the algebraic identity between
the absorbed and un-absorbed forms.  A last group plants mistakes into the
oracle and checks that the pins catch every one.
"""
import math

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle as O
from oracle import mla_oracle as M

FORMS = [O.mla_attention_unabsorbed, O.mla_attention_absorbed]


def _tiny(rng, sq, length, h=2, r=3, n=2, p=2, v=2):
    return (rng.standard_normal((sq, h, n)), rng.standard_normal((sq, h, p)),
            rng.standard_normal((length, r)), rng.standard_normal((length, p)),
            rng.standard_normal((h * (n + v), r)))


def _brute(qn, qp, c, kp, w, scale):
    """Pure-Python loops: expand K and V entry by entry, then softmax."""
    sq, nh, nope = len(qn), len(qn[0]), len(qn[0][0])
    length, rank, pdim = len(c), len(c[0]), len(kp[0])
    vdim = len(w) // nh - nope
    out = [[[0.0] * vdim for _ in range(nh)] for _ in range(sq)]
    lse = [[0.0] * nh for _ in range(sq)]
    for j in range(sq):
        vis = length - sq + j + 1
        for h in range(nh):
            base = h * (nope + vdim)
            scores = []
            for t in range(vis):
                s = 0.0
                for a in range(nope):
                    k = sum(float(w[base + a][r]) * float(c[t][r]) for r in range(rank))
                    s += float(qn[j][h][a]) * k
                for a in range(pdim):
                    s += float(qp[j][h][a]) * float(kp[t][a])
                scores.append(scale * s)
            mx = max(scores)
            es = [math.exp(s - mx) for s in scores]
            tot = sum(es)
            for a in range(vdim):
                acc = 0.0
                for t in range(vis):
                    val = sum(float(w[base + nope + a][r]) * float(c[t][r]) for r in range(rank))
                    acc += es[t] * val
                out[j][h][a] = acc / tot
            lse[j][h] = mx + math.log(tot)
    return np.array(out), np.array(lse)


# ---------------------------------------------------------------------------
# Pin checks, written against a generic attention function so that the
# mutation tests below can run them on planted mistakes.
# ---------------------------------------------------------------------------

def check_brute_force(fn):
    rng = np.random.default_rng(10)
    for sq in (1, 2):
        for length in (1, 2, 3, 7):
            if sq > length:
                continue
            args = _tiny(rng, sq, length)
            out, lse = fn(*args, 0.7)
            bo, bl = _brute(*args, 0.7)
            np.testing.assert_allclose(out, bo, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(lse, bl, rtol=1e-12, atol=1e-12)


def check_single_token(fn):
    rng = np.random.default_rng(11)
    qn, qp, c, kp, w = _tiny(rng, 1, 1, h=3, r=5, n=4, p=2, v=3)
    out, lse = fn(qn, qp, c, kp, w, 0.3)
    for h in range(3):
        wv = w[h * 7 + 4:h * 7 + 7]
        np.testing.assert_allclose(out[0, h], wv @ c[0], rtol=1e-14)
        s0 = 0.3 * (qn[0, h] @ (w[h * 7:h * 7 + 4] @ c[0]) + qp[0, h] @ kp[0])
        assert lse[0, h] == pytest.approx(s0, rel=1e-13)


def check_equal_scores(fn):
    rng = np.random.default_rng(12)
    qn, qp, c, kp, w = _tiny(rng, 1, 9, h=2, r=6, n=3, p=4, v=3)
    out, lse = fn(np.zeros_like(qn), np.zeros_like(qp), c, kp, w, 0.5)
    for h in range(2):
        v = c @ w[h * 6 + 3:h * 6 + 6].T
        np.testing.assert_allclose(out[0, h], v.mean(axis=0), rtol=1e-13)
        assert lse[0, h] == pytest.approx(math.log(9), rel=1e-14)


def check_dominant_score(fn):
    rng = np.random.default_rng(13)
    qn, qp, c, kp, w = _tiny(rng, 1, 6, h=1, r=4, n=2, p=2, v=2)
    w[:2] = 0.0                       # no nope contribution
    kp[:] = 0.0
    kp[3] = [1.0, 0.0]
    qp[0, 0] = [120.0, 0.0]           # score of token 3 is 60 above the rest at scale 0.5
    out, lse = fn(qn, qp, c, kp, w, 0.5)
    np.testing.assert_allclose(out[0, 0], w[2:4] @ c[3], rtol=1e-20, atol=1e-20 + 1e-24)
    assert lse[0, 0] == pytest.approx(60.0 + math.log1p(5 * math.exp(-60.0)), rel=1e-15)


def check_rope_only_against_scipy(fn):
    # W_UK half zero: scores come from the rope key alone; compare softmax and
    # logsumexp with scipy's routines.  This also fixes W_UK as the first half.
    rng = np.random.default_rng(14)
    qn, qp, c, kp, w = _tiny(rng, 1, 40, h=2, r=8, n=4, p=6, v=4)
    for h in range(2):
        w[h * 8:h * 8 + 4] = 0.0
    out, lse = fn(qn, qp, c, kp, w, 0.25)
    for h in range(2):
        s = 0.25 * kp @ qp[0, h]
        v = c @ w[h * 8 + 4:h * 8 + 8].T
        np.testing.assert_allclose(out[0, h], softmax(s) @ v, rtol=1e-12)
        assert lse[0, h] == pytest.approx(logsumexp(s), rel=1e-13)


def check_zero_value_half(fn):
    rng = np.random.default_rng(15)
    qn, qp, c, kp, w = _tiny(rng, 2, 11, h=2, r=5, n=3, p=2, v=3)
    for h in range(2):
        w[h * 6 + 3:h * 6 + 6] = 0.0
    out, _ = fn(qn, qp, c, kp, w, 0.4)
    assert np.all(out == 0.0)


def check_causality(fn):
    rng = np.random.default_rng(16)
    qn, qp, c, kp, w = _tiny(rng, 2, 12, h=2, r=5, n=3, p=4, v=3)
    out, lse = fn(qn, qp, c, kp, w, 0.6)
    o0, l0 = fn(qn[:1], qp[:1], c[:-1], kp[:-1], w, 0.6)     # query 0 alone at position L-2
    np.testing.assert_allclose(out[0], o0[0], rtol=1e-13)
    np.testing.assert_allclose(lse[0], l0[0], rtol=1e-13)
    c2, kp2 = c.copy(), kp.copy()
    c2[-1] += 5.0
    kp2[-1] -= 3.0
    out2, _ = fn(qn, qp, c2, kp2, w, 0.6)
    np.testing.assert_array_equal(out2[0], out[0])            # query 0 never sees token L-1
    assert np.abs(out2[1] - out[1]).max() > 1e-3               # query 1 does


def check_invariances(fn):
    rng = np.random.default_rng(17)
    qn, qp, c, kp, w = _tiny(rng, 1, 15, h=2, r=6, n=3, p=4, v=3)
    out, lse = fn(qn, qp, c, kp, w, 0.35)
    perm = rng.permutation(15)
    o_p, l_p = fn(qn, qp, c[perm], kp[perm], w, 0.35)
    np.testing.assert_allclose(o_p, out, rtol=1e-12)
    np.testing.assert_allclose(l_p, lse, rtol=1e-13)
    u = rng.standard_normal(4)                                  # same shift for every token
    o_s, l_s = fn(qn, qp, c, kp + u, w, 0.35)
    np.testing.assert_allclose(o_s, out, rtol=1e-11, atol=1e-13)
    for h in range(2):
        assert l_s[0, h] == pytest.approx(lse[0, h] + 0.35 * qp[0, h] @ u, rel=1e-12)


PIN_CHECKS = [check_brute_force, check_single_token, check_equal_scores, check_dominant_score,
              check_rope_only_against_scipy, check_zero_value_half, check_causality, check_invariances]


@pytest.mark.parametrize("fn", FORMS, ids=["unabsorbed", "absorbed"])
@pytest.mark.parametrize("check", PIN_CHECKS, ids=lambda c: c.__name__)
def test_pin(fn, check):
    check(fn)


def test_absorbed_equals_unabsorbed_at_model_shape():
    rng = np.random.default_rng(20)
    scale = O.softmax_scale()
    for sq, length in [(1, 1024), (2, 333)]:
        qn = rng.standard_normal((sq, 32, 128))
        qp = rng.standard_normal((sq, 32, 64))
        c = rng.standard_normal((length, 512))
        kp = rng.standard_normal((length, 64))
        w = rng.standard_normal((8192, 512)) / math.sqrt(512)
        ou, lu = O.mla_attention_unabsorbed(qn, qp, c, kp, w, scale)
        oa, la = O.mla_attention_absorbed(qn, qp, c, kp, w, scale)
        assert np.linalg.norm(oa - ou) / np.linalg.norm(ou) < 1e-12
        np.testing.assert_allclose(la, lu, rtol=1e-13)


def test_chunked_combine_equals_single_pass():
    rng = np.random.default_rng(21)
    s = rng.standard_normal(5000) * 3
    v = rng.standard_normal((5000, 7))
    ref = softmax(s) @ v
    for chunk in (64, 512, 4096, 5000, 9000):
        o, l = O.lse_combine(O.attention_chunk_partials(s, v, chunk))
        np.testing.assert_allclose(o, ref, rtol=1e-12)
        assert l == pytest.approx(logsumexp(s), rel=1e-14)
    masked = s.copy()
    masked[512:1024] = -np.inf                                # chunk 1 of 512 fully masked
    masked[1600:1700] = -np.inf                               # and part of chunk 3
    parts = O.attention_chunk_partials(masked, v, 512)
    assert parts[1][1] == -math.inf and np.all(parts[1][0] == 0)
    keep = np.isfinite(masked)
    o, l = O.lse_combine(parts)
    np.testing.assert_allclose(o, softmax(s[keep]) @ v[keep], rtol=1e-12)
    assert l == pytest.approx(logsumexp(s[keep]), rel=1e-14)
    with pytest.raises(ValueError):
        O.lse_combine([(np.zeros(3), -math.inf)])


def test_paged_slots_are_a_bijection_and_reconstruct_the_sequence():
    rng = np.random.default_rng(22)
    lens = [1, 64, 65, 200, 1000]
    need = [(x + 63) // 64 for x in lens]
    perm = rng.permutation(sum(need))
    pool = np.full((sum(need) * 64, 3), -1.0)
    rows = [rng.standard_normal((x, 3)) for x in lens]
    seen = set()
    off = 0
    for b, x in enumerate(lens):
        bt = perm[off:off + need[b]]
        off += need[b]
        slots = O.paged_slot(bt, np.arange(x))
        assert len(set(slots.tolist()) & seen) == 0
        seen.update(slots.tolist())
        pool[slots] = rows[b]
        np.testing.assert_array_equal(pool[O.paged_slot(bt, np.arange(x))], rows[b])
    assert len(seen) == sum(lens)


# ---------------------------------------------------------------------------
# Planted mistakes: every mutant must fail at least one pin.
# ---------------------------------------------------------------------------

def _run_pins(fn):
    failures = 0
    for check in PIN_CHECKS:
        try:
            check(fn)
        except (AssertionError, ValueError, IndexError):
            failures += 1
    return failures


def _swapped_halves(w, h, nope, vdim):
    rows = w[h * (nope + vdim):(h + 1) * (nope + vdim)]
    return rows[vdim:], rows[:vdim]


def test_planted_mistakes_are_caught(monkeypatch):
    base = O.mla_attention_unabsorbed
    mutants = {
        "rope term dropped": lambda qn, qp, c, kp, w, s, heads=None: base(qn, 0 * qp, c, kp, w, s, heads),
        "rope sign flipped": lambda qn, qp, c, kp, w, s, heads=None: base(qn, -qp, c, kp, w, s, heads),
        "nope term dropped": lambda qn, qp, c, kp, w, s, heads=None: base(0 * qn, qp, c, kp, w, s, heads),
        "one token short": lambda qn, qp, c, kp, w, s, heads=None: base(qn, qp, c[:-1], kp[:-1], w, s, heads),
        "scale applied twice": lambda qn, qp, c, kp, w, s, heads=None: base(qn, qp, c, kp, w, s * s, heads),
        "latent rows reversed": lambda qn, qp, c, kp, w, s, heads=None: base(qn, qp, c[::-1], kp, w, s, heads),
    }
    for name, fn in mutants.items():
        assert _run_pins(fn) > 0, name
    monkeypatch.setattr(M, "_head_weights", _swapped_halves)
    assert _run_pins(O.mla_attention_unabsorbed) > 0, "kv_b_proj halves swapped"
    assert _run_pins(O.mla_attention_absorbed) > 0, "kv_b_proj halves swapped (absorbed)"


def test_planted_rope_and_scale_mistakes_are_caught():
    f = O.yarn_inv_freq()
    x = np.random.default_rng(5).standard_normal(64)

    def wrong_sign(x, pos, inv):
        k = x.shape[-1] // 2
        a = pos * inv
        return np.concatenate([x[:k] * np.cos(a) + x[k:] * np.sin(a), x[k:] * np.cos(a) - x[:k] * np.sin(a)])

    z = (x[:32] + 1j * x[32:]) * np.exp(1j * 77 * f)
    assert not np.allclose(wrong_sign(x, 77, f), np.concatenate([z.real, z.imag]))
    assert not np.allclose(1 / math.sqrt(192), 0.14467962580268925)
