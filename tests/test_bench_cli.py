"""Host behaviour of bench.py that needs no GPU: more than one GPU is refused with a
message, the counters summary keeps its calibration arithmetic, and the counter
record's source hash ignores comments but not code."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_committed_counters_record_is_consistent():
    # the record bench.py reads for "traffic": bytes = KiB per dispatch x 1024 x scale, summed
    with open(os.path.join(ROOT, "profiles", "splitkv_decode_counters.json")) as fh:
        c = json.load(fh)
    k = c["kernels"]["splitkv_decode"]
    f, w = k["fetch"], k["write"]
    assert abs(f["bytes_scaled"] - f["kib_per_dispatch"] * 1024 * c["FETCH_SIZE_scale"]) < 1e-3 * f["bytes_scaled"]
    assert abs(w["bytes_scaled"] - w["kib_per_dispatch"] * 1024 * c["WRITE_SIZE_scale"]) < 1e-3 * w["bytes_scaled"]
    assert abs(k["hbm_bytes_per_launch"] - f["bytes_scaled"] - w["bytes_scaled"]) < 1.0
    # the calibration copy of copy_bytes reads and writes exactly that many bytes
    assert abs(c["FETCH_SIZE_copy_kib"] * c["FETCH_SIZE_scale"] * 1024 - c["copy_bytes"]) < 1e-6 * c["copy_bytes"]
    assert abs(c["WRITE_SIZE_copy_kib"] * c["WRITE_SIZE_scale"] * 1024 - c["copy_bytes"]) < 1e-6 * c["copy_bytes"]
    # at least the cache itself is read (37,748,736 B at 32K)
    assert f["bytes_scaled"] >= 37748736


def test_counter_record_hash_ignores_comments_but_not_code(tmp_path, monkeypatch):
    # the record stays valid across a comment edit of the kernel sources and not
    # across a code edit
    sys.path.insert(0, ROOT)
    import bench

    src = tmp_path / "k.hip"
    hdr = tmp_path / "k.h"
    src.write_text("// kernel\nint f(int x) { return x + 1; }  /* one */\n")
    hdr.write_text("#define N 4\n")
    monkeypatch.setattr(bench, "DECODE_SRC", [str(src), str(hdr)])
    h0 = bench.source_hash()
    src.write_text("// the kernel, reworded\nint f(int x) {\n  return x + 1;   /* one,\n two */\n}\n")
    assert bench.source_hash() == h0
    src.write_text("// kernel\nint f(int x) { return x + 2; }  /* one */\n")
    assert bench.source_hash() != h0
