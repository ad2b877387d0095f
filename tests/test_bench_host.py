"""Host logic of bench.py that needs no GPU: the HBM traffic of the dominant
kernel is reported from the committed counter summary only while the kernel
sources still hash to the value recorded with the counters."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _summary(tmp_path, sha, traffic=123456789):
    p = tmp_path / "traffic.md"
    p.write_text(f"# counters\n\ntraffic_bytes_per_launch: {traffic}\nsource_sha256: {sha}\n")
    return str(p)


def test_traffic_reported_while_sources_match(tmp_path):
    committed = bench.measured_traffic()
    if committed is None:
        pytest.skip("the kernel sources changed since the committed counters were taken")
    assert committed > 0
    # the committed summary's hash, reused in a copy, gives back its value
    text = open(bench.TRAFFIC_PROFILE).read()
    sha = [l.split(": ", 1)[1].strip() for l in text.splitlines() if l.startswith("source_sha256: ")][0]
    assert bench.measured_traffic(_summary(tmp_path, sha, 987654321)) == 987654321


def test_traffic_null_when_sources_changed(tmp_path):
    assert bench.measured_traffic(_summary(tmp_path, "0" * 64)) is None


def test_traffic_null_without_summary(tmp_path):
    assert bench.measured_traffic(str(tmp_path / "missing.md")) is None
