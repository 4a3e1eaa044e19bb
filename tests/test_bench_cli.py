"""bench.py's contract, checked on the CPU: one GPU only, the algorithmic byte counts the
throughput is quoted on, and the HBM traffic records staying attached to the pack source
they were measured on."""
from __future__ import annotations

import glob
import json
import os
import subprocess
import sys

import bench
from precision_attention_input_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line for an unsupported configuration


# Pack and unpack bytes per workload from the byte formulas (Q, K, V read at 2 bytes and
# written at 1 byte per element, amax / scale / mean traffic, the V tail): the table the
# throughput figures are quoted on.
EXPECTED = {
    W.TINY.name: (591_104, 393_472),
    W.UNALIGNED_PADDED.name: (147_523_584, 98_464_768),
    W.VIDEO_DIT_ALIGNED.name: (1_208_287_232, 805_568_512),
    W.LONG_UNALIGNED.name: (3_451_310_080, 2_301_062_400),
    W.BATCHED_SMALL_HEAD.name: (226_615_296, 151_079_424),
}


def test_algorithmic_bytes_per_workload():
    for name, (pack, unpack) in EXPECTED.items():
        nb = bench.algorithmic_bytes(W.BY_NAME[name])
        assert (nb["pack"], nb["unpack"]) == (pack, unpack), name


def test_algorithmic_bytes_count_each_byte_once():
    """Independent of the formulas above: pack moves 9 bytes per element triple plus small
    terms, unpack 6 plus the V tail, on every workload."""
    for w in W.WORKLOADS:
        nb = bench.algorithmic_bytes(w)
        n = nb["N"]
        assert 9 * n <= nb["pack"] < 9 * n * 1.01, w.name
        assert 6 * n <= nb["unpack"] < 6 * n * 1.02, w.name


def test_kernel_hash_ignores_comments_and_whitespace(tmp_path, monkeypatch):
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    a.write_text("// header\nint f(int x) {\n    return x + 1;  /* one */\n}\n")
    b.write_text("int f(int x) { return x + 1; }  // reformatted, other comments\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["a.hip"])
    ha = bench.kernel_hash()
    monkeypatch.setattr(bench, "KERNEL_SOURCES", ["b.hip"])
    assert bench.kernel_hash() == ha
    b.write_text("int f(int x) { return x + 2; }\n")
    assert bench.kernel_hash() != ha


def test_recorded_traffic_belongs_to_the_current_pack_source():
    """The committed rocprofv3 traffic records were taken on the pack as it is now (the
    benchmark reports no traffic otherwise), one per large workload, and show no wasted
    re-reads by either counter measure."""
    recs = sorted(glob.glob(os.path.join(ROOT, "profiles", "pack_kernel_*_traffic.json")))
    assert len(recs) == 4
    for path in recs:
        with open(path) as f:
            rec = json.load(f)
        assert rec["kernel_hash"] == bench.kernel_hash(), os.path.basename(path)
        ratio = rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
        assert 0.99 < ratio < 1.01, (os.path.basename(path), ratio)
        # the uncalibrated measure (DRAM requests in 32-byte units) agrees, and read the
        # calibration copy's bytes exactly
        ratio = rec["dram_request_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
        assert 0.99 < ratio < 1.01, (os.path.basename(path), ratio)
        assert abs(rec["copy_dram_request_bytes"] / rec["copy_bytes"] - 1) < 1e-4
        # the unpack's bytes, recorded beside the pack's for the counter-based pair figure
        assert rec["unpack_kernel_hash"] == bench.kernel_hash(bench.UNPACK_SOURCES)
        ratio = (rec["unpack_dram_request_bytes_per_launch"] /
                 rec["unpack_algorithmic_bytes_per_launch"])
        assert 0.99 < ratio < 1.01, (os.path.basename(path), ratio)
