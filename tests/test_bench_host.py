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
    traffic.write_text(f"# comment = ignored\ndecode.hbm_bytes_per_call = 123456\n"
                       f"prefill.hbm_bytes_per_call = 654321\n"
                       f"decode_source_sha256_16 = {h}\nprefill_source_sha256_16 = {h}\n")
    mfma = tmp_path / "mfma.txt"
    mfma.write_text(f"mfma_busy_frac = 0.5\nsustained_clock_ghz = 2.1\n"
                    f"mfma_gflop_executed = 140.0\nprefill_source_sha256_16 = {h}\n")
    monkeypatch.setattr(bench, "DECODE_SRC", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic))
    monkeypatch.setattr(bench, "PREFILL_SRC", str(src))
    monkeypatch.setattr(bench, "MFMA_FILE", str(mfma))
    monkeypatch.setattr(bench, "LEG_SOURCE", {"decode": str(src), "prefill": str(src)})
    assert bench.measured_traffic() == 123456
    assert bench.measured_traffic("prefill") == 654321
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


def _write_counter_csv(path, rows):
    """rows: (dispatch id, kernel name, value) in rocprofv3's counter CSV layout."""
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id",
            "Grid_Size", "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size",
            "Scratch_Size", "VGPR_Count", "Accum_VGPR_Count", "SGPR_Count", "Counter_Name",
            "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=cols)
        w.writeheader()
        for did, name, val in rows:
            r = {c: 0 for c in cols}
            r.update(Dispatch_Id=did, Kernel_Name=name, Counter_Name="X", Counter_Value=val)
            w.writerow(r)


def test_traffic_summary_per_leg(tmp_path):
    # two legs, each from its own runs: the calibration copy (1 GiB) reads
    # 524288 KiB on FETCH_SIZE (scale 2) and writes 1048576 KiB (scale 1); a
    # call is the split kernel plus the merge; input fills are ignored
    cal = "void __amd_rocclr_copyBuffer(...)"
    fill = "void at::native::vectorized_elementwise_kernel<FillFunctor>(...)"
    dk = "void gqa::decode_kernel<128, false, false>(gqa::DecodeArgs)"
    dm = "void gqa::decode_merge_kernel<128, false>(gqa::MergeArgs)"
    pk = "void gqa::prefill_mfma_kernel<128, false>(gqa::PrefillArgs)"
    for leg, main, merge, fk, wk in (("decode", dk, dm, 1000.0, 10.0),
                                     ("prefill", pk, None, 500.0, 300.0)):
        for ctr, per, calv in (("fetch", fk, 524288.0), ("write", wk, 1048576.0)):
            rows = [(1, fill, 99999.0)]
            for i in range(3):  # three calls
                rows.append((2 + 2 * i, main, per))
                if merge:
                    rows.append((3 + 2 * i, merge, 1.0))
            rows.append((20, cal, calv))
            _write_counter_csv(tmp_path / leg / ctr / "run" / "ctr_counter_collection.csv", rows)
    text = bench.summarize_counters(str(tmp_path))
    vals = {ln.split("=")[0].strip(): ln.split("=")[1].strip()
            for ln in text.splitlines() if "=" in ln and not ln.startswith("#")}
    # decode: (1000 + 1) KiB read x 2 + (10 + 1) KiB written x 1, per call
    assert int(vals["decode.hbm_bytes_per_call"]) == (1001 * 2 + 11) * 1024
    assert int(vals["prefill.hbm_bytes_per_call"]) == (500 * 2 + 300) * 1024
    assert "sweep8.hbm_bytes_per_call" not in vals  # no runs for that leg
    assert vals["decode_source_sha256_16"] == bench.source_hash(bench.DECODE_SRC)
    assert vals["prefill_source_sha256_16"] == bench.source_hash(bench.PREFILL_SRC)


def test_packed_pairs():
    # segments of 3 and 2 cells: 1 + 2 + 3 and 1 + 2 permitted pairs
    assert bench.packed_pairs([0, 0, 0, 3, 3]) == (9, [3, 2])
    assert bench.packed_pairs([0] * 7) == (28, [7])
    from gqa_kv_cache_02_amd import synth
    c = synth.CONFIGS["packed_b1_t4096_hq32_hkv8_d128"]
    segs = synth.packed_segment_starts(1, c["T"], *c["seg_len"], c["seed"])[0].tolist()
    pairs, lens = bench.packed_pairs(segs)
    assert sum(lens) == c["T"] and all(64 <= n <= 1024 for n in lens[:-1])
    assert pairs == sum(n * (n + 1) // 2 for n in lens)
    # Q and O of 32 heads, K and V of 8, 4096 cells of 128 bf16 features
    assert bench.algorithmic_bytes("packed") == 2 * 4096 * 128 * (2 * 32 + 2 * 8) == 83_886_080


def test_algorithmic_bytes_of_the_legs():
    assert bench.algorithmic_bytes("decode") == 262_275_072
    assert bench.algorithmic_bytes("sweep1") == 65_601_536
    assert bench.algorithmic_bytes("prefill") is None
    # the two ragged legs draw the same kind of lengths with different seeds;
    # the rolling cache adds the candidate's read and commit
    assert 50e6 < bench.algorithmic_bytes("ragged") < 70e6
    assert 50e6 < bench.algorithmic_bytes("ring") < 70e6
