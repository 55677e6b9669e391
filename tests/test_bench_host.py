"""Host-side checks of bench.py (no GPU): the one-GPU rule, the algorithmic byte count the
GB/s figure rests on, and the HBM traffic figure derived from a counter record."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def test_algorithmic_bytes():
    b = _bench()
    # 2 B of BF16 read once, and per layout 0.5 B of codes + 1/16 B of scales per element
    # and one 4-byte tensor scale
    assert b.alg_bytes(16384, 8192) == 419_430_408
    assert b.alg_bytes(16384, 8192, layouts=1) == 2 * 16384 * 8192 + 16384 * 8192 // 2 + \
        16384 * 8192 // 16 + 4
    assert b.mx_alg_bytes(16384, 8192) == 2 * 16384 * 8192 + 2 * (16384 * 8192 // 2 +
                                                                   16384 * 8192 // 32)


def test_traffic_scales_each_counter_by_the_copy():
    b = _bench()
    rec = {"fetch_kib": 100.0, "write_kib": 30.0, "copy_bytes": 1000,
           "copy_fetch_kib": 50.0, "copy_write_kib": 100.0}
    # FETCH_SIZE reads half the copy's bytes (factor 2), WRITE_SIZE all of them (factor 1)
    assert b.measured_traffic(rec) == 100 * 1000 // 50 + 30 * 1000 // 100
    assert b.measured_traffic(None) is None


def test_source_hash_ignores_comments(tmp_path, monkeypatch):
    b = _bench()
    src = tmp_path / "k.hip"
    src.write_text("int f() { return 1; }  // one\n/* block */\n")
    monkeypatch.setattr(b, "KERNEL_SOURCES", [str(src)])
    h0 = b.kernel_source_hash()
    src.write_text("int f() {\n  return 1;  // another comment\n}\n")
    assert b.kernel_source_hash() == h0
    src.write_text("int f() { return 2; }\n")
    assert b.kernel_source_hash() != h0
