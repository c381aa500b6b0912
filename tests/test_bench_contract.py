"""Host-side parts of bench.py's report (no GPU): the counter-profile guard
behind `roofline.traffic`, and the refusal of multi-GPU runs."""

import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _profile(path, sha, nbytes):
    with open(path, "w") as f:
        f.write(f"# counters\n\nsource sha256: {sha}\n(note)\n\nhbm bytes per launch: {nbytes}\n")


def test_traffic_reported_only_for_the_profiled_source(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "counters.md"
    _profile(prof, sha, 123456789)
    assert bench.traffic_from_profile(str(src), str(prof)) == 123456789.0
    # any edit of the source invalidates the counters
    src.write_text("// kernel source, changed\n")
    assert bench.traffic_from_profile(str(src), str(prof)) is None
    # a missing or malformed summary gives no figure
    assert bench.traffic_from_profile(str(src), str(tmp_path / "absent.md")) is None
    (tmp_path / "bad.md").write_text("no figures here\n")
    assert bench.traffic_from_profile(str(src), str(tmp_path / "bad.md")) is None


def test_first_recorded_hash_is_the_one_checked(tmp_path):
    # a summary may mention an older source by a shortened hash; only a full
    # 64-digit hash counts
    src = tmp_path / "kernel.hip"
    src.write_text("// v2\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "counters.md"
    prof.write_text(f"source sha256: {sha}\n(taken at source 8f308c58754d...)\n\n"
                    "hbm bytes per launch: 42\n")
    assert bench.traffic_from_profile(str(src), str(prof)) == 42.0


def test_multi_gpu_run_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_run_metadata_and_cpu_baseline_protocol():
    """The record names its sources and seeds; the CPU baseline states its
    workers, CPU model and the tokens it covered (a tiny workload here)."""
    from fine_grained_mixture_amd import synth
    wl = synth.TINY
    meta = bench.run_metadata(wl)
    assert len(meta["source_sha256"]) == 64 and meta["input_seed"] == wl.seed
    inp = synth.make_inputs(wl)
    r = bench.cpu_baseline(wl, inp, 0)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0
    assert 1 <= r["cores"] <= min(len(os.sched_getaffinity(0)), bench.MAX_CPU_WORKERS)
    assert r["cpu_model"] and f"{wl.T} of the {wl.T} tokens" in r["sample"]
