"""bench.py's host logic, without a GPU: the algorithmic byte and flop counts
behind its rooflines, the hash-keyed reading of committed counter summaries,
and the single-GPU refusal."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_counts():
    # decode B=8, Hq=32, Hkv=8, d=128, 8000 cells: K and V once per KV group
    # (262,144,000 B) plus Q read and O written (131,072 B)
    assert bench.decode_bytes(8, 32, 8, 128, 8000) == 262_275_072
    # the endpoint sweep: K/V bytes scale with Hkv, Q/O stay
    assert [bench.decode_bytes(16, 8, h, 128, 8000) for h in (8, 2, 1)] == \
        [524_353_536, 131_137_536, 65_601_536]
    # causal prefill T=4096, Hq=32, d=128: 4*d flops per permitted pair
    assert bench.prefill_flops(32, 128, 4096) == 137_472_507_904
    assert bench.prefill_flops(1, 1, 1) == 4


def test_counter_summaries_follow_the_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_text("// a kernel\n")
    h = bench.source_hash(str(src))
    traffic = tmp_path / "traffic.txt"
    traffic.write_text(f"# comment = ignored\nhbm_bytes_per_call = 123456\n"
                       f"decode_source_sha256_16 = {h}\n")
    mfma = tmp_path / "mfma.txt"
    mfma.write_text(f"mfma_busy_frac = 0.5\nsustained_clock_ghz = 2.1\n"
                    f"mfma_gflop_executed = 140.0\nprefill_source_sha256_16 = {h}\n")
    monkeypatch.setattr(bench, "DECODE_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    monkeypatch.setattr(bench, "PREFILL_SRC", str(src))
    monkeypatch.setattr(bench, "MFMA_FILE", str(mfma))
    assert bench.measured_traffic() == 123456
    assert bench.measured_mfma()["mfma_busy_frac"] == 0.5
    # a changed kernel source invalidates both
    src.write_text("// the kernel, changed\n")
    assert bench.measured_traffic() is None
    assert bench.measured_mfma() is None
    # so does a missing summary
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "none.txt"))
    monkeypatch.setattr(bench, "MFMA_FILE", str(tmp_path / "none.txt"))
    assert bench.measured_traffic() is None and bench.measured_mfma() is None


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
