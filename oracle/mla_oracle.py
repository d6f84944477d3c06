"""CPU oracle for MLA decode over a latent KV cache: plain numpy, fp64.

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg import this module.  The HIP library never calls
it; the two share no code, headers, tables or helpers.  Inputs come from the
seeded generator in ``synth`` (random numbers only) or from the caller.

Pages cited (titles as printed):

* [KV-ledger] "256K 长上下文真能本地用？Xing4.0 原生长上下文的工程代价拆解"
  (lpnh.cn): §一 "256K 的规格真相" (config.json, parameter table), §二 "KV Cache
  显存账本" (per-token cache arithmetic and the MLA / MHA table).
* [MLA-arch] "mHC+MLA+MTP 是什么？拆开给 Agent 用的百亿 MoE" (hotelren.com),
  section "MLA：256K 上下文的内存革命" (Xing4_0Attention fields, kv_a_proj_with_mqa,
  kv_b_proj, YaRN with yarn_get_mscale).

What the oracle computes is the un-absorbed form that [MLA-arch] describes:
the cache holds, per token, a 512-wide latent plus a 64-wide rope key; at
attention time kv_b_proj expands full per-head keys and values from the latent
and ordinary softmax attention follows.  Every floating-point step runs in
fp64 on the bf16 input values (which fp64 holds exactly).

Readings of points the pages leave open:

* kv_b_proj output rows of head h are [k_nope (128) | v (128)], heads in order
  (the declared out width num_heads * (qk_nope_head_dim + v_head_dim)).
* no bias (config ``attention_bias: false`` in [KV-ledger §一]).
* softmax scale = (qk_nope + qk_rope) ** -0.5 * mscale ** 2 with
  mscale = 0.1 * mscale_all_dim * ln(factor) + 1 (YaRN's attention temperature;
  [MLA-arch] names yarn_get_mscale without printing it).
* rope base 10000 and half-split pairing (i, i + 32): not printed for this
  model; they shape the prepared inputs only.
* YaRN frequencies: NTK-by-parts (Peng et al., 2023) in the form of the
  authors' public implementation, which the MLA model code that defines
  yarn_get_mscale follows: a blend weight linear in the PAIR INDEX between
  floor(d(beta_fast)) = 10 and ceil(d(beta_slow)) = 23.  (The paper's
  equation writes the ramp as linear in the rotation count r instead; the
  pages print only the parameters, and the two forms differ inside the ramp.)
* query j of Sq new tokens sits at position L - Sq + j and sees cache tokens
  0 .. L - Sq + j (its own latent is already cached).
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Model constants: [KV-ledger §一] config.json and parameter table;
# [MLA-arch] Xing4_0Attention fields.
# ---------------------------------------------------------------------------
NUM_HEADS = 32              # num_attention_heads / num_key_value_heads 32 / 32
KV_LORA_RANK = 512          # kv_lora_rank
QK_NOPE_HEAD_DIM = 128      # qk_nope_head_dim
QK_ROPE_HEAD_DIM = 64       # qk_rope_head_dim
V_HEAD_DIM = 128            # v_head_dim
NUM_LAYERS = 40             # num_hidden_layers
MAX_POSITIONS = 262144      # max_position_embeddings
ROPE_SCALING = dict(type="yarn", factor=64.0, original_max_position_embeddings=4096,
                    beta_fast=32.0, beta_slow=1.0, mscale=1.0, mscale_all_dim=1.0)
ROPE_THETA = 10000.0        # reading: not printed for this model
PAGE_SIZE = 64              # tokens per cache page (paged layout of the workloads)


# ---------------------------------------------------------------------------
# YaRN: attention temperature and rotary frequencies
# ---------------------------------------------------------------------------

def yarn_get_mscale(scale: float, mscale: float = 1.0) -> float:
    """YaRN attention-temperature factor, 0.1 * mscale * ln(scale) + 1.

    [MLA-arch] says the rope uses YaRN with a yarn_get_mscale correction of
    the attention scaling; YaRN (Peng et al., 2023) sets sqrt(1/t) to
    0.1 ln(s) + 1.  A scale of at most 1 means no correction.
    """
    if scale <= 1.0:
        return 1.0
    return 0.1 * mscale * math.log(scale) + 1.0


def softmax_scale(qk_nope: int = QK_NOPE_HEAD_DIM, qk_rope: int = QK_ROPE_HEAD_DIM,
                  rope_scaling: dict = ROPE_SCALING) -> float:
    """1/sqrt(qk_nope + qk_rope) times mscale**2 (mscale from mscale_all_dim)."""
    m = yarn_get_mscale(rope_scaling["factor"], rope_scaling["mscale_all_dim"])
    return (qk_nope + qk_rope) ** -0.5 * m * m


def yarn_inv_freq(dim: int = QK_ROPE_HEAD_DIM, base: float = ROPE_THETA,
                  rope_scaling: dict = ROPE_SCALING) -> np.ndarray:
    """Per-pair rotary frequencies after YaRN's NTK-by-parts blend (fp64).

    Pair i has base frequency f_i = base ** (-2i/dim) and wavelength 2 pi / f_i.
    Pairs that turn more than beta_fast times over the original context keep
    f_i; pairs that turn fewer than beta_slow times take f_i / factor; a linear
    ramp over the pair index joins them.  d(r) below is the (fractional) pair
    index whose wavelength fits r times into the original context.
    """
    factor = float(rope_scaling["factor"])
    orig = float(rope_scaling["original_max_position_embeddings"])
    i = np.arange(dim // 2, dtype=np.float64)
    f = base ** (-2.0 * i / dim)
    if factor <= 1.0:
        return f

    def d(r):
        return dim * math.log(orig / (2.0 * math.pi * r)) / (2.0 * math.log(base))

    low = max(math.floor(d(rope_scaling["beta_fast"])), 0)
    high = min(math.ceil(d(rope_scaling["beta_slow"])), dim - 1)
    if high == low:
        high = low + 1e-3
    ramp = np.clip((i - low) / (high - low), 0.0, 1.0)
    return f * (1.0 - ramp) + (f / factor) * ramp


def yarn_correction_range(dim: int = QK_ROPE_HEAD_DIM, base: float = ROPE_THETA,
                          rope_scaling: dict = ROPE_SCALING):
    """(low, high) pair indices of the ramp used by :func:`yarn_inv_freq`."""
    orig = float(rope_scaling["original_max_position_embeddings"])

    def d(r):
        return dim * math.log(orig / (2.0 * math.pi * r)) / (2.0 * math.log(base))

    return (max(math.floor(d(rope_scaling["beta_fast"])), 0),
            min(math.ceil(d(rope_scaling["beta_slow"])), dim - 1))


def rope_rotate(x: np.ndarray, positions: np.ndarray, inv_freq: np.ndarray) -> np.ndarray:
    """Rotate the last axis of ``x`` (width 2K) by position * inv_freq (fp64).

    Half-split pairing: element i pairs with i + K.  ``positions`` broadcasts
    against ``x.shape[:-1]``.  Angles are formed in fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    k = x.shape[-1] // 2
    ang = np.asarray(positions, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = x[..., :k], x[..., k:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each fp64 entry, as fp64.

    bfloat16 keeps 8 significant bits; normal range only (all values here).
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # rint: half to even


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Decode uint16 bfloat16 bit patterns to fp64."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Bit patterns of values that are already exact bfloat16 numbers."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# Cache rows and paging
# ---------------------------------------------------------------------------

def paged_slot(block_table_row: np.ndarray, t: np.ndarray, page_size: int = PAGE_SIZE) -> np.ndarray:
    """Physical slot of logical token t: page block_table[t // P] * P + t % P."""
    t = np.asarray(t, dtype=np.int64)
    return np.asarray(block_table_row, dtype=np.int64)[t // page_size] * page_size + t % page_size


# ---------------------------------------------------------------------------
# 8-bit latent cache.  [KV-ledger §三] (plan A) keeps the KV cache in 8 bits
# (llama.cpp's q8_0), which halves its bytes against bf16 at a small cost in
# long-context accuracy.  The pages fix neither the number format nor the
# scale granularity; readings: OCP FP8 E4M3 codes (sign, 4 exponent bits with
# bias 7, 3 mantissa bits, no infinities, code 0x7F / 0xFF = NaN, largest
# finite value 448), one fp32 scale per group of 128 latent values of a token
# (scale = group max |x| / 448, computed in fp32), and the rope key kept in
# bf16.  A token's fp8 row is [512 codes | 4 fp32 scales | 64 bf16 rope key]
# = 656 bytes.
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0
FP8_GROUP = 128
FP8_ROW_BYTES = KV_LORA_RANK + 4 * (KV_LORA_RANK // FP8_GROUP) + 2 * QK_ROPE_HEAD_DIM   # 656


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """fp64 value of E4M3 codes: (-1)^s * 2^(e-7) * (1 + m/8) for e > 0,
    (-1)^s * 2^-6 * m/8 for e = 0; NaN for exponent and mantissa all ones."""
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def round_to_e4m3(x: np.ndarray) -> np.ndarray:
    """E4M3 code of the representable value nearest to each x (|x| <= 448),
    ties to the code with an even mantissa; the sign bit follows x's sign."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("round_to_e4m3 takes |x| <= 448")
    grid = e4m3_value(np.arange(0, 0x7F))            # codes 0x00..0x7E, increasing
    a = np.abs(x)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    return (code | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def quantize_latent_fp8(c_kv: np.ndarray):
    """codes uint8 [..., 512] and fp32 scales [..., 4] of latent rows.

    Per group of 128 values, in fp32 as the cache writer does it: amax = max |x|,
    scale = amax / 448, code = e4m3(clamp(x / scale, -448, 448)); a group of
    zeros gets scale 0 and codes 0.
    """
    x = np.asarray(c_kv, dtype=np.float32)
    g = x.reshape(x.shape[:-1] + (-1, FP8_GROUP))
    amax = np.abs(g).max(axis=-1)
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0))
    y = (g / safe[..., None]).astype(np.float32)
    y = np.clip(y, -np.float32(E4M3_MAX), np.float32(E4M3_MAX))
    y = np.where(scale[..., None] > 0, y, np.float32(0.0))
    codes = round_to_e4m3(y.astype(np.float64)).reshape(x.shape)
    return codes, scale


def dequantize_latent_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp64 latent values code * scale (exact in fp64)."""
    v = e4m3_value(codes).reshape(np.shape(codes)[:-1] + (-1, FP8_GROUP))
    return (v * np.asarray(scales, dtype=np.float64)[..., None]).reshape(np.shape(codes))


def fp8_cache_row_bytes(codes: np.ndarray, scales: np.ndarray, k_pe_bits: np.ndarray) -> np.ndarray:
    """Bytes of fp8 cache rows [512 codes | 4 fp32 scales | 64 bf16 rope key] (656 per token)."""
    n = np.shape(codes)[0]
    out = np.empty((n, FP8_ROW_BYTES), dtype=np.uint8)
    out[:, :KV_LORA_RANK] = codes
    out[:, KV_LORA_RANK:KV_LORA_RANK + 16] = np.asarray(scales, dtype="<f4").view(np.uint8).reshape(n, 16)
    out[:, KV_LORA_RANK + 16:] = np.asarray(k_pe_bits, dtype="<u2").view(np.uint8).reshape(n, 128)
    return out


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _head_weights(w_kv_b: np.ndarray, h: int, nope: int, vdim: int):
    rows = w_kv_b[h * (nope + vdim):(h + 1) * (nope + vdim)]
    return rows[:nope], rows[nope:]          # W_UK[h] (nope x R), W_UV[h] (vdim x R)


def mla_attention_unabsorbed(q_nope, q_pe, c_kv, k_pe, w_kv_b, scale, heads=None):
    """Decode attention of one sequence, expanding keys and values per head.

    q_nope [Sq, H, N], q_pe [Sq, H, P] (rotated), c_kv [L, R], k_pe [L, P]
    (rotated), w_kv_b [H*(N+V), R] in nn.Linear storage.  For each head the
    latent of every visible token is expanded by kv_b_proj into
    k_nope = W_UK c and v = W_UV c ([MLA-arch]); the key is [k_nope ; k_pe]
    with the rope key shared by all heads (kv_a_proj_with_mqa).  Scores
    scale * q.k, softmax with max subtraction, output sum_t p_t v_t.

    Returns (out [Sq, len(heads), V], lse [Sq, len(heads)]) in fp64, where
    lse is the natural log of sum_t exp(score_t).
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    w = np.asarray(w_kv_b, dtype=np.float64)
    sq, nh, nope = q_nope.shape
    length = c_kv.shape[0]
    vdim = w.shape[0] // nh - nope
    heads = list(range(nh)) if heads is None else list(heads)
    if not 1 <= sq <= length:
        raise ValueError("need 1 <= Sq <= L")
    out = np.zeros((sq, len(heads), vdim))
    lse = np.zeros((sq, len(heads)))
    for hi, h in enumerate(heads):
        w_uk, w_uv = _head_weights(w, h, nope, vdim)
        k_nope = c_kv @ w_uk.T               # [L, N]
        v = c_kv @ w_uv.T                    # [L, V]
        for j in range(sq):
            visible = length - sq + j + 1    # tokens 0 .. L - Sq + j
            s = scale * (k_nope[:visible] @ q_nope[j, h] + k_pe[:visible] @ q_pe[j, h])
            m = s.max()
            e = np.exp(s - m)
            tot = e.sum()
            out[j, hi] = (e @ v[:visible]) / tot
            lse[j, hi] = m + math.log(tot)
    return out, lse


def mla_attention_absorbed(q_nope, q_pe, c_kv, k_pe, w_kv_b, scale, heads=None):
    """Same result as :func:`mla_attention_unabsorbed`, with W_UK folded into q.

    q_lat = W_UK[h]^T q_nope, score = scale (q_lat . c_t + q_pe . k_pe_t),
    o_lat = sum_t p_t c_t, out = W_UV[h] o_lat.  Exact algebra for the
    bias-free linear kv_b_proj; the companion reference for large sizes.
    """
    q_nope = np.asarray(q_nope, dtype=np.float64)
    q_pe = np.asarray(q_pe, dtype=np.float64)
    c_kv = np.asarray(c_kv, dtype=np.float64)
    k_pe = np.asarray(k_pe, dtype=np.float64)
    w = np.asarray(w_kv_b, dtype=np.float64)
    sq, nh, nope = q_nope.shape
    length = c_kv.shape[0]
    vdim = w.shape[0] // nh - nope
    heads = list(range(nh)) if heads is None else list(heads)
    out = np.zeros((sq, len(heads), vdim))
    lse = np.zeros((sq, len(heads)))
    for hi, h in enumerate(heads):
        w_uk, w_uv = _head_weights(w, h, nope, vdim)
        for j in range(sq):
            visible = length - sq + j + 1
            q_lat = w_uk.T @ q_nope[j, h]
            s = scale * (c_kv[:visible] @ q_lat + k_pe[:visible] @ q_pe[j, h])
            m = s.max()
            e = np.exp(s - m)
            tot = e.sum()
            o_lat = (e @ c_kv[:visible]) / tot
            out[j, hi] = w_uv @ o_lat
            lse[j, hi] = m + math.log(tot)
    return out, lse


def attention_chunk_partials(scores: np.ndarray, values: np.ndarray, chunk: int):
    """Split-KV partials of one softmax row: per chunk (normalised o_i, lse_i).

    Chunk i covers tokens [i*chunk, (i+1)*chunk).  Scores of -inf are masked;
    a chunk with no visible token has lse_i = -inf and o_i = 0.
    """
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    parts = []
    for a in range(0, scores.shape[0], chunk):
        s = scores[a:a + chunk]
        if not np.isfinite(s).any():
            parts.append((np.zeros(values.shape[1:]), -math.inf))
            continue
        m = s[np.isfinite(s)].max()
        e = np.where(np.isfinite(s), np.exp(s - m), 0.0)
        tot = e.sum()
        parts.append(((e @ values[a:a + chunk]) / tot, m + math.log(tot)))
    return parts


def lse_combine(parts):
    """Merge split partials: LSE = log sum_i exp(lse_i); o = sum_i exp(lse_i - LSE) o_i."""
    lses = np.array([p[1] for p in parts], dtype=np.float64)
    big = lses.max()
    if not np.isfinite(big):
        raise ValueError("every chunk is empty")
    wts = np.exp(lses - big)                 # exp(-inf) = 0 for empty chunks
    tot = wts.sum()
    o = sum(wt * p[0] for wt, p in zip(wts, parts)) / tot
    return o, big + math.log(tot)


# ---------------------------------------------------------------------------
# Cache-size accounting ([KV-ledger §二]; [MLA-arch] MLA section)
# ---------------------------------------------------------------------------

def cache_elems_per_token(convention: str = "latent+rope") -> int:
    """Cached bf16 elements per token per layer under each convention.

    * "latent+rope": 512 latent + 64 rope key ([MLA-arch]): 576.
    * "latent+v": 512 latent + v_head_dim 128 ([KV-ledger §二]): 640.
    * "latent+per-head-rope": 512 + 32 x 64 ([MLA-arch]'s "about" figure): 2560.
    """
    if convention == "latent+rope":
        return KV_LORA_RANK + QK_ROPE_HEAD_DIM
    if convention == "latent+v":
        return KV_LORA_RANK + V_HEAD_DIM
    if convention == "latent+per-head-rope":
        return KV_LORA_RANK + NUM_HEADS * QK_ROPE_HEAD_DIM
    raise ValueError(convention)


def mla_cache_bytes(tokens: int, convention: str = "latent+rope", layers: int = NUM_LAYERS,
                    bytes_per_elem: int = 2) -> int:
    """Whole-model MLA cache bytes for ``tokens`` tokens."""
    return tokens * cache_elems_per_token(convention) * layers * bytes_per_elem


def mha_cache_bytes(tokens: int, heads: int = NUM_HEADS,
                    qk_dim: int = QK_NOPE_HEAD_DIM + QK_ROPE_HEAD_DIM,
                    layers: int = NUM_LAYERS, bytes_per_elem: int = 2) -> int:
    """MHA baseline of [KV-ledger §二]: heads x 192 dims x 2 (K and V) x layers x 2 B."""
    return tokens * heads * qk_dim * 2 * layers * bytes_per_elem
