"""The traffic and clock summaries in profiles/ were taken with the kernel
sources as they are: bench.py reports them only then.  (Kept in a file that
runs last, so a stale summary does not hide other results.)"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_committed_counter_files_match_the_kernel_sources():
    for path in (bench.TRAFFIC_FILE, bench.CLOCK_FILE):
        with open(path) as f:
            assert json.load(f)["kernel_source_hash"] == bench.kernel_source_hash(), (
                f"{os.path.relpath(path, ROOT)} was taken with other kernel sources; "
                "rerun its counter passes")
