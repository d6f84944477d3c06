"""C-ABI boundary on the host: the library loads, exports every declared entry
point, and rejects bad arguments before enqueuing anything (no GPU needed)."""
import ctypes
import os
import re

import pytest

import mla_latent_kv_absorbed_amd as M
import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")

OK, ERR_NULL, ERR_SHAPE, ERR_RANGE, ERR_ALIGN, ERR_WORKSPACE = 0, 1, 2, 3, 4, 5
FAKE = 1 << 20   # an aligned non-null address; validation fails before any use


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:mla_status|const char\*)\s+(mla_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(M.build.lib_path())
    for n in names:
        assert hasattr(lib, n), n


def test_default_shape_and_scale():
    s = M.default_shape()
    assert (s.num_heads, s.kv_lora_rank, s.qk_nope_head_dim, s.qk_rope_head_dim, s.v_head_dim,
            s.page_size) == (32, 512, 128, 64, 128, 64)
    assert s.softmax_scale == pytest.approx(O.softmax_scale(), rel=1e-7)
    r = M.default_rope()
    assert (r.base, r.factor, r.original_max_position, r.beta_fast, r.beta_slow, r.rope_dim) == \
        (10000.0, 64.0, 4096.0, 32.0, 1.0, 64)


def test_status_strings():
    for code in range(9):
        assert M.mla_status_string(code).startswith("MLA_")
    assert "scratch" in M.mla_status_string(8)


def _decode(lib, shape, **kw):
    a = dict(q=FAKE, qp=FAKE, w=FAKE, cache=FAKE, stride=1024, lens=FAKE, maxctx=1024, B=1, Sq=1,
             chunk=0, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.mla_decode(ctypes.byref(shape), a["q"], a["qp"], a["w"], a["cache"], a["stride"], a["lens"],
                          a["maxctx"], a["B"], a["Sq"], a["chunk"], a["out"], a["lse"], a["ws"], a["wsb"], None)


def test_decode_argument_errors():
    lib = M.library()
    s = M.default_shape()
    assert _decode(lib, s, q=None) == ERR_NULL
    assert _decode(lib, s, ws=None) == ERR_NULL
    assert _decode(lib, s, chunk=100) == ERR_RANGE          # not a multiple of 64
    assert _decode(lib, s, Sq=0) == ERR_RANGE
    assert _decode(lib, s, Sq=17) == ERR_RANGE
    assert _decode(lib, s, maxctx=1, Sq=2) == ERR_RANGE
    assert _decode(lib, s, stride=512) == ERR_RANGE          # stride < max_ctx_len
    assert _decode(lib, s, q=FAKE + 2) == ERR_ALIGN
    assert _decode(lib, s, ws=FAKE + 16) == ERR_ALIGN
    assert _decode(lib, s, wsb=10) == ERR_WORKSPACE
    assert _decode(lib, s, B=0, q=None) == OK                # empty batch: no-op
    bad = M.default_shape()
    bad.num_heads = 16
    assert _decode(lib, bad) == ERR_SHAPE
    bad = M.default_shape()
    bad.softmax_scale = float("nan")
    assert _decode(lib, bad) == ERR_RANGE


def test_paged_argument_errors():
    lib = M.library()
    s = M.default_shape()

    def call(**kw):
        a = dict(bt=FAKE, maxpages=16, pages=100, maxctx=1024)
        a.update(kw)
        return lib.mla_decode_paged(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, a["pages"], a["bt"], a["maxpages"],
                                    FAKE, a["maxctx"], 1, 1, 0, FAKE, None, FAKE, 1 << 40, None)
    assert call(bt=None) == ERR_NULL
    assert call(maxpages=15) == ERR_RANGE                    # 1024 tokens need 16 pages
    assert call(pages=0) == ERR_RANGE


def test_append_and_rope_argument_errors():
    lib = M.library()
    s = M.default_shape()
    assert lib.mla_cache_append(ctypes.byref(s), FAKE, 10, FAKE, 512, FAKE, 64, FAKE, 0, None) == OK
    assert lib.mla_cache_append(ctypes.byref(s), None, 10, FAKE, 512, FAKE, 64, FAKE, 1, None) == ERR_NULL
    assert lib.mla_cache_append(ctypes.byref(s), FAKE, 10, FAKE, 500, FAKE, 64, FAKE, 1, None) == ERR_RANGE
    assert lib.mla_cache_append(ctypes.byref(s), FAKE, 10, FAKE, 516, FAKE, 64, FAKE, 1, None) == ERR_ALIGN
    p = M.default_rope()
    assert lib.mla_rope_yarn(ctypes.byref(p), FAKE, 64, FAKE, 64, FAKE, 0, None) == OK
    assert lib.mla_rope_yarn(ctypes.byref(p), None, 64, FAKE, 64, FAKE, 3, None) == ERR_NULL
    assert lib.mla_rope_yarn(ctypes.byref(p), FAKE, 60, FAKE, 64, FAKE, 3, None) == ERR_RANGE
    p.rope_dim = 32
    assert lib.mla_rope_yarn(ctypes.byref(p), FAKE, 64, FAKE, 64, FAKE, 3, None) == ERR_SHAPE


def test_workspace_size_and_auto_chunk():
    # Without a GPU the library assumes 256 compute units: the balanced
    # schedule aims at one split per unit and never below 2 tiles (128 tokens).
    assert M.mla_decode_auto_chunk(1, 1, 32768) == 128
    assert M.mla_decode_auto_chunk(1, 1, 262144) == 1024
    assert M.mla_decode_auto_chunk(16, 1, 65536) == 4096
    for B, Sq, L in [(1, 1, 1024), (1, 1, 32768), (16, 1, 65536), (1, 1, 262144), (32, 2, 131072), (3, 5, 100)]:
        chunk = M.mla_decode_auto_chunk(B, Sq, L)
        assert chunk % 64 == 0 and chunk >= 128
        assert B * -(-L // chunk) <= 256 or chunk == 128
        # partials (512 bf16 + one fp32 LSE per row) for up to 256 + B
        # segments, plus the query rows
        need = M.mla_decode_workspace_size(B, Sq, L)
        assert need >= B * Sq * 32 * (576 * 2 + 512 * 4) + (256 + B) * Sq * 32 * (512 * 2 + 4)
        fixed = M.mla_decode_workspace_size(B, Sq, L, kv_chunk=128)
        assert fixed >= B * Sq * 32 * (576 * 2 + 512 * 4) + B * -(-L // 128) * Sq * 32 * (512 * 2 + 4)
    with pytest.raises(M.MlaError):
        M.mla_decode_workspace_size(1, 1, 100, kv_chunk=65)
    # more sequences than compute units: every sequence is one split, so the
    # split never grows past the longest sequence (it used to grow without bound)
    assert M.mla_decode_auto_chunk(65535, 1, 100) == 128
    assert M.mla_decode_auto_chunk(4095, 16, 200) == 256
    assert M.mla_decode_auto_chunk(65535, 1, 1 << 20) == 1 << 20
    assert M.mla_decode_auto_chunk(300, 1, 64) == 128
    # an empty batch needs no workspace and must not trip the split heuristic
    assert M.mla_decode_workspace_size(0, 1, 1024) == 0
    assert M.mla_decode_auto_chunk(0, 1, 1024) % 64 == 0


def _prefill(lib, shape, **kw):
    a = dict(q=FAKE, qp=FAKE, w=FAKE, cache=FAKE, L=1024, Tq=256, out=FAKE, lse=None, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.mla_prefill(ctypes.byref(shape), a["q"], a["qp"], a["w"], a["cache"], a["L"], a["Tq"], a["out"],
                           a["lse"], a["ws"], a["wsb"], None)


def test_prefill_argument_errors_and_workspace():
    lib = M.library()
    s = M.default_shape()
    assert _prefill(lib, s, q=None) == ERR_NULL
    assert _prefill(lib, s, ws=None) == ERR_NULL
    assert _prefill(lib, s, Tq=0) == ERR_RANGE
    assert _prefill(lib, s, Tq=1025) == ERR_RANGE                 # more query tokens than context
    assert _prefill(lib, s, L=(1 << 20) + 1, Tq=1) == ERR_RANGE
    assert _prefill(lib, s, out=FAKE + 8) == ERR_ALIGN
    assert _prefill(lib, s, wsb=1000) == ERR_WORKSPACE
    f8 = M.default_shape(M.CACHE_FP8_E4M3)
    assert _prefill(lib, f8) == 7                                 # MLA_ERR_UNSUPPORTED
    # expanded rows [8192 | 64 rope] bf16 per token, context rounded up to 256
    assert M.mla_prefill_workspace_size(1024) == 1024 * 8256 * 2
    assert M.mla_prefill_workspace_size(1000) == 1024 * 8256 * 2
    assert M.mla_prefill_workspace_size(129) == 256 * 8256 * 2
    assert M.mla_prefill_workspace_size(300) == 512 * 8256 * 2
    with pytest.raises(M.MlaError):
        M.mla_prefill_workspace_size(0)


def test_read_probe_argument_errors():
    lib = M.library()
    assert lib.mla_read_probe(None, 1024, FAKE, None) == ERR_NULL
    assert lib.mla_read_probe(FAKE, 1024, None, None) == ERR_NULL
    assert lib.mla_read_probe(FAKE, 0, FAKE, None) == ERR_RANGE
    assert lib.mla_read_probe(FAKE, 1000, FAKE, None) == ERR_RANGE      # not a multiple of 16
    assert lib.mla_read_probe(FAKE + 8, 1024, FAKE, None) == ERR_ALIGN


def test_read_probe_sink_size_matches_the_header():
    m = re.search(r"#define MLA_READ_PROBE_SINK_INTS (\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == M.READ_PROBE_SINK_INTS


def _header_define(name):
    m = re.search(r"#define %s\s+\(?(\d+)u?(?:\s*<<\s*(\d+))?\)?" % name, open(HEADER).read())
    assert m, name
    return int(m.group(1)) << int(m.group(2) or 0)


def test_fault_bits_and_static_scratch_size_match_the_header():
    assert _header_define("MLA_FAULT_SLOT") == M.FAULT_SLOT
    assert _header_define("MLA_FAULT_PAGE") == M.FAULT_PAGE
    assert _header_define("MLA_FAULT_CTX_LEN") == M.FAULT_CTX_LEN
    assert _header_define("MLA_FAULT_FP16_RANGE") == M.FAULT_FP16_RANGE
    assert _header_define("MLA_STATIC_SCRATCH_BYTES") == M.STATIC_SCRATCH_BYTES == 64 << 20


def test_host_checks_of_lengths_and_pages():
    # the range rules the kernels apply, run on host copies of the arrays
    assert M.mla_check_decode_inputs([5, 64, 100], 1, 100) == 0
    assert M.mla_check_decode_inputs([5, 101], 1, 100) == M.FAULT_CTX_LEN        # above max_ctx_len
    assert M.mla_check_decode_inputs([1, 100], 2, 100) == M.FAULT_CTX_LEN        # below Sq
    assert M.mla_check_decode_inputs([0], 1, 100) == M.FAULT_CTX_LEN
    bt = [[3, 0], [1, 2]]
    assert M.mla_check_decode_inputs([128, 65], 1, 128, bt, num_pages=4) == 0
    assert M.mla_check_decode_inputs([128, 65], 1, 128, bt, num_pages=3) == M.FAULT_PAGE   # page 3 of 3
    assert M.mla_check_decode_inputs([128, 64], 1, 128, [[0, 1], [2, -1]], num_pages=4) == 0  # entry unused
    assert M.mla_check_decode_inputs([128, 65], 1, 128, [[0, 1], [2, -1]], num_pages=4) == M.FAULT_PAGE
    # a clamped length decides which entries count: 200 tokens clamp to 128 (two pages)
    assert M.mla_check_decode_inputs([200], 1, 128, [[0, 1]], num_pages=2) == M.FAULT_CTX_LEN
    assert M.mla_check_decode_inputs([200], 1, 128, [[0, 9]], num_pages=2) == M.FAULT_CTX_LEN | M.FAULT_PAGE
    with pytest.raises(M.MlaError):
        M.mla_check_decode_inputs([10], 1, 128, [[0]], num_pages=2)               # table narrower than 128 tokens
    assert M.mla_check_slot_mapping([0, 5, -1, 9], 10) == 0
    assert M.mla_check_slot_mapping([0, 10], 10) == M.FAULT_SLOT
    assert M.mla_check_slot_mapping([], 0) == 0


def test_noalloc_entry_point_argument_errors():
    lib = M.library()
    s = M.default_shape()
    r = M.default_rope()

    def call(**kw):
        a = dict(pages=100, bt=FAKE, maxpages=16, maxctx=1024, B=1, Sq=1, chunk=0, out=FAKE)
        a.update(kw)
        return lib.mla_decode_step_paged_noalloc(ctypes.byref(s), ctypes.byref(r), FAKE, FAKE, FAKE, 512, FAKE, 64,
                                                 FAKE, FAKE, a["pages"], a["bt"], a["maxpages"], FAKE, a["maxctx"],
                                                 a["B"], a["Sq"], a["chunk"], a["out"], None, None)
    assert call(out=None) == ERR_NULL
    assert call(bt=None) == ERR_NULL
    assert call(maxpages=15) == ERR_RANGE
    assert call(B=0) == OK
    # a workspace beyond the static scratch: 4096 sequences x 16 query tokens
    # need more than 64 MiB of query rows alone
    assert call(B=4095, Sq=16, maxctx=1024) == 8                  # MLA_ERR_SCRATCH
    assert M.mla_decode_workspace_size(4095, 16, 1024) > M.STATIC_SCRATCH_BYTES
    # fixed 64-token splits over long contexts: many segments
    assert call(B=16, maxctx=65536, maxpages=1024, chunk=64) == 8
    assert M.mla_decode_workspace_size(16, 1, 65536, kv_chunk=64) > M.STATIC_SCRATCH_BYTES


def test_binding_checks_shapes_and_devices_before_the_gpu():
    # shape, dtype and same-device checks of the Python binding come before
    # the GPU check, so they run here on CPU tensors
    import torch
    B, Sq = 2, 1
    q = torch.zeros(B, Sq, 32, 128, dtype=torch.bfloat16)
    qp = torch.zeros(B, Sq, 32, 64, dtype=torch.bfloat16)
    w = torch.zeros(8192, 512, dtype=torch.bfloat16)
    lens = torch.full((B,), 64, dtype=torch.int32)
    cache = torch.zeros(B, 64, 576, dtype=torch.bfloat16)
    with pytest.raises(M.MlaError, match="out must have shape"):
        M.mla_decode(q, qp, w, cache, lens, 64, out=torch.zeros(B, Sq, 32, 64, dtype=torch.bfloat16))
    with pytest.raises(M.MlaError, match="lse must have shape"):
        M.mla_decode(q, qp, w, cache, lens, 64, out=torch.zeros(B, Sq, 32, 128, dtype=torch.bfloat16),
                     lse=torch.zeros(B, Sq, 16, dtype=torch.float32))
    with pytest.raises(M.MlaError, match="ctx_lens must have shape"):
        M.mla_decode(q, qp, w, cache, lens[:1], 64)
    with pytest.raises(M.MlaError, match="q_pe must have shape"):
        M.mla_decode(q, qp[:, :, :16].contiguous(), w, cache, lens, 64)
    with pytest.raises(M.MlaError, match="is on meta"):
        M.mla_decode(q, qp.to("meta"), w, cache, lens, 64)
    with pytest.raises(M.MlaError, match="must be on the GPU"):
        M.mla_decode(q, qp, w, cache, lens, 64, out=torch.zeros(B, Sq, 32, 128, dtype=torch.bfloat16))
    Tq = 4
    with pytest.raises(M.MlaError, match="out must have shape"):
        M.mla_prefill(torch.zeros(Tq, 32, 128, dtype=torch.bfloat16), torch.zeros(Tq, 32, 64, dtype=torch.bfloat16),
                      w, torch.zeros(64, 576, dtype=torch.bfloat16), 64,
                      out=torch.zeros(Tq - 1, 32, 128, dtype=torch.bfloat16))
    with pytest.raises(M.MlaError, match="lse must have shape"):
        M.mla_prefill(torch.zeros(Tq, 32, 128, dtype=torch.bfloat16), torch.zeros(Tq, 32, 64, dtype=torch.bfloat16),
                      w, torch.zeros(64, 576, dtype=torch.bfloat16), 64,
                      out=torch.zeros(Tq, 32, 128, dtype=torch.bfloat16), lse=torch.zeros(Tq, dtype=torch.float32))
