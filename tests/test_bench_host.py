"""Host logic of bench.py (CPU only): the one-GPU refusal and the readers of
the committed counter summaries, which must report a figure only for the
kernel source and the workload the counters were taken on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""   # no benchmark line


def _summary(path, lines):
    with open(path, "w") as f:
        f.write("# counter summary written by the test\n")
        for k, v in lines.items():
            f.write(f"{k}: {v}\n")


def test_traffic_only_for_its_source_and_workload(tmp_path, monkeypatch):
    p = tmp_path / "pmc.txt"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(p))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    assert bench.read_traffic(1000) is None          # no summary
    _summary(p, {"hbm_bytes_per_launch": 1050, "algorithmic_bytes_per_launch": 1000,
                 "kernel_source_sha256": "abc123"})
    assert bench.read_traffic(1000) == 1050.0
    assert bench.read_traffic(999) is None           # another workload
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "def456")
    assert bench.read_traffic(1000) is None          # another kernel source


def test_mfma_busy_only_for_its_source_and_workload(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    name = bench.MFMA_SUMMARIES["v32f"]
    assert bench.read_mfma_busy("v32f", 8.365e10) is None      # no summary
    _summary(tmp_path / "profiles" / name,
             {"mfma_busy_fraction": "0.243   (busy cycles / (1024 SIMDs x cycles))",
              "mfma_flop_per_dispatch": "9.413e+10   (counted x 512; algorithmic 8.365e+10)",
              "kernel_source_sha256": "abc123"})
    got = bench.read_mfma_busy("v32f", 83647168512)
    assert got == {"fraction": 0.243, "from": "profiles/" + name}
    assert bench.read_mfma_busy("v32f", 4.2e10) is None        # another workload's FLOPs
    assert bench.read_mfma_busy("v16f", 83647168512) is None   # no summary for it
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "def456")
    assert bench.read_mfma_busy("v32f", 83647168512) is None   # another kernel source
    # the decode summary states its algorithmic FLOPs on a line of their own
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "abc123")
    _summary(tmp_path / "profiles" / bench.MFMA_SUMMARIES["2"],
             {"mfma_busy_fraction": "0.136", "algorithmic_flop_per_dispatch": "1.075e+10",
              "kernel_source_sha256": "abc123"})
    assert bench.read_mfma_busy("2", 10749935616)["fraction"] == 0.136


def test_committed_summaries_match_their_workloads():
    """Every committed MFMA summary that was taken on the current kernel
    source names its own workload's algorithmic FLOPs."""
    import paged_fp8_kv_amd.workloads as W
    for cid, name in bench.MFMA_SUMMARIES.items():
        assert os.path.exists(os.path.join(ROOT, "profiles", name)), name
        with open(os.path.join(ROOT, "profiles", name)) as f:
            text = f.read()
        if f"kernel_source_sha256: {bench.kernel_source_hash()}" not in text:
            continue   # taken on an earlier source: the bench reports null
        got = bench.read_mfma_busy(cid, W.config(cid).attn_flops)
        assert got is not None and 0.0 < got["fraction"] < 1.0, (cid, name)
