"""Host-side pieces of bench.py (CPU): the kernel-source hash that decides
whether committed counter runs still describe the current kernels."""

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_code_only_drops_comments_and_layout():
    a = "int x = 1;  // one\n/* block\n comment */ int y = x +\n  2;\n"
    b = "int x = 1;\nint y = x + 2;  // two\n"
    assert bench._code_only(a) == bench._code_only(b) == "int x = 1; int y = x + 2;"
    assert bench._code_only("int x = 1;") != bench._code_only("int x = 2;")


def test_traffic_files_name_known_kernels_and_hashes():
    # every committed counter summary names a kernel the hash covers; a file
    # whose hash no longer matches is reported as null traffic, never used
    prof = os.path.join(ROOT, "profiles")
    for f in os.listdir(prof):
        if f.endswith("_traffic.json"):
            d = json.load(open(os.path.join(prof, f)))
            assert d["kernel"] in bench.KERNEL_SOURCES, f
            assert len(d["kernel_source_hash"]) == 16
            workload = f[len(d["kernel"]) + 1:-len("_traffic.json")]
            ok = d["kernel_source_hash"] == bench.kernel_source_hash(d["kernel"])
            assert (bench.measured_traffic(workload, d["kernel"]) is not None) == ok
