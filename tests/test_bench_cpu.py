"""Host-side pieces of bench.py: the counter digest and the traffic file.

The HBM traffic that bench.py reports comes from counters taken on earlier
runs; it is reported only while the digest of the kernel's code still
matches the one stored with the counters (else it is null until the
counters are taken again).  Editing a comment must not count as a change
of the kernel; editing code must.
"""

import os
import re

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_code_only_ignores_comments_and_spacing():
    a = "int f(int x) {\n  // doubles x\n  return 2 * x; /* fast */\n}\n"
    b = "int f(int x) {\n  // returns twice x\n\n  return 2 *   x;   /* multi\n line */ }"
    assert bench._code_only(a) == bench._code_only(b)


def test_code_only_sees_code_changes():
    a = "int f(int x) { return 2 * x; } // note"
    b = "int f(int x) { return 3 * x; } // note"
    assert bench._code_only(a) != bench._code_only(b)


def test_traffic_file_lines_are_well_formed():
    path = os.path.join(ROOT, "profiles", "hbm_traffic_headline.txt")
    with open(path) as fh:
        lines = [l for l in fh if l.startswith("kernel=")]
    assert lines
    for line in lines:
        key = re.search(r"kernel=(\S+)", line).group(1)
        assert key in bench.KERNEL_SOURCES
        assert re.search(r"hbm_bytes_per_launch=\d+ ", line)
        assert re.search(r"source_digest=[0-9a-f]{16}$", line.strip())


def test_stale_counters_are_not_reported(tmp_path, monkeypatch):
    # a line whose digest does not match the current code gives None; a
    # matching one gives its bytes
    key = "dispatch_bf16"
    good = bench.source_digest(key)
    f = tmp_path / "traffic.txt"
    f.write_text(f"kernel={key} fetch_kib=1.0 write_kib=1.0 hbm_bytes_per_launch=123 "
                 f"source_digest={'0' * 16}\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic(key) is None
    f.write_text(f"kernel={key} fetch_kib=1.0 write_kib=1.0 hbm_bytes_per_launch=123 "
                 f"source_digest={good}\n")
    assert bench.read_traffic(key) == 123


def test_more_than_one_gpu_is_refused():
    # one GPU's share is what bench.py measures: --gpus N > 1, or a launch
    # with WORLD_SIZE > 1, exits with status 2 and says why, before touching
    # torch or a device
    import subprocess
    import sys
    for extra, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "8"})):
        res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *extra],
                             capture_output=True, text=True, timeout=60,
                             env={**os.environ, **env}, cwd=ROOT)
        assert res.returncode == 2
        assert "more than one GPU" in res.stderr
        assert res.stdout == ""
