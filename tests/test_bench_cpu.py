"""CPU checks of the benchmark's host logic: the one-GPU guard and the rule
that a stored HBM-traffic figure is reported only while the kernel sources
still hash to the ones it was measured with."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _fake_tree(tmp_path, source):
    csrc = tmp_path / "moe_decode_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "decode.hip").write_text(source)
    (csrc / "common.hpp").write_text("// header\n")
    (csrc / "prefill.hip").write_text("// another kernel file\n")
    (tmp_path / "profiles").mkdir()


def test_traffic_follows_the_source_hash(tmp_path, monkeypatch):
    _fake_tree(tmp_path, "// kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h = bench.kernel_source_hash("k_gateup_t1")
    prof = tmp_path / "profiles" / "k_gateup_t1_c4_i4_T1_pmc.md"
    prof.write_text(f"summary\n\ntraffic_bytes_per_launch: 12345\nsource_sha256: {h}\n")
    assert bench.traffic_record("k_gateup_t1", "c4_i4_T1") == 12345.0
    # a file outside the kernel's own source and the headers does not matter
    (tmp_path / "moe_decode_amd" / "csrc" / "prefill.hip").write_text("// changed\n")
    assert bench.traffic_record("k_gateup_t1", "c4_i4_T1") == 12345.0
    # the kernel's source or a header changing voids the figure
    (tmp_path / "moe_decode_amd" / "csrc" / "common.hpp").write_text("// header, edited\n")
    assert bench.traffic_record("k_gateup_t1", "c4_i4_T1") is None
    # no summary for the workload: no figure
    assert bench.traffic_record("k_gateup_t1", "c4_i4_T4") is None


def test_committed_summary_names_a_hash_and_a_figure():
    text = open(os.path.join(ROOT, "profiles", "k_gateup_t1_c4_i4_T1_pmc.md")).read()
    assert "traffic_bytes_per_launch:" in text and "source_sha256:" in text


def test_mfma_stats_by_hand():
    """Every token of a 128-token chunk chooses experts 0..7: 8 experts of
    128 tokens = 64 tiles of 16; useful ops 2 * (2F * H) per (token, slot)
    pair; issued = 16 positions * 64 tiles * 4 digit passes = 4x useful."""
    import numpy as np
    from synth import workloads as W
    sp = W.spec("c4_i4")
    idx = np.tile(np.arange(8, dtype=np.int32), (128, 1))[None]
    st = bench.mfma_stats(sp, idx, 1.0, "int8")
    useful = 2.0 * 2 * 2048 * 6144 * 1024
    assert st["tiles_per_call"] == 64
    assert abs(st["useful_TOPS"] - useful / 1e-3 / 1e12) < 1e-9
    assert abs(st["issued_TOPS"] / st["useful_TOPS"] - 4.0) < 1e-12
    assert st["peak_TOPS"] == 5000.0
    b = bench.mfma_stats(sp, idx, 1.0, "bf16")
    assert abs(b["issued_TOPS"] / b["useful_TOPS"] - 2.0) < 1e-12 and b["peak_TOPS"] == 2500.0
    # one token per expert: a tile of 16 for each pair, 16x the useful work per pass
    idx1 = np.arange(128 * 8, dtype=np.int32).reshape(1, 128, 8) % 256
    s1 = bench.mfma_stats(sp, idx1, 1.0, "int8")
    assert s1["tiles_per_call"] == 256


def test_records_are_plain():
    h = bench.host_record()
    assert h["logical_cpus"] == os.cpu_count()
    assert bench.source_hash() == bench.source_hash() and len(bench.source_hash()) == 64
