"""CPU checks of the benchmark script's contract that need no GPU: it refuses
more than one GPU before touching the device, and the HBM traffic it reports
comes from a committed rocprofv3 counter summary only while that summary's
kernel-source hash matches the current attention-kernel source."""

import glob
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def _summary(root, workload, sha, hbm):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "profiles", f"attn_fwd_{workload}_traffic.txt"), "w") as f:
        f.write("# rocprofv3 counter summary (test)\n")
        f.write(f"kernel_source_sha {sha}\n")
        f.write(f"hbm_bytes_per_launch {hbm}\n")


def test_traffic_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    assert len(sha) == 16
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # kernel_source_sha reads the sources under ROOT: keep it on the real tree
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    assert bench.load_traffic("absent") is None
    _summary(str(tmp_path), "current", sha, 123456789)
    assert bench.load_traffic("current") == 123456789.0
    _summary(str(tmp_path), "stale", "0" * 16, 123456789)
    assert bench.load_traffic("stale") is None


def test_committed_summaries_name_their_commands_and_bytes():
    paths = sorted(glob.glob(os.path.join(ROOT, "profiles", "attn_fwd_*_traffic.txt")))
    assert {os.path.basename(p) for p in paths} >= {
        "attn_fwd_hunyuan_traffic.txt", "attn_fwd_wan720p_traffic.txt", "attn_fwd_medium_traffic.txt"}
    for p in paths:
        text = open(p).read()
        kv = dict(ln.split(None, 1) for ln in text.splitlines() if ln and not ln.startswith("#"))
        assert len(kv["kernel_source_sha"].strip()) == 16, p
        assert float(kv["hbm_bytes_per_launch"]) > 0, p
        # the commands that produced the figures run committed files only
        cmds = [ln for ln in text.splitlines() if "rocprofv3" in ln and "-- python3" in ln]
        assert len(cmds) >= 5, p
        assert all(" bench.py " in c + " " for c in cmds), p
