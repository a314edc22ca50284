"""Host-side pieces of bench.py: the algorithmic byte counts and the lookup of
measured HBM traffic (no GPU needed)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from workloads import config_by_name  # noqa: E402


def test_algorithmic_bytes_2p7b():
    cfg = config_by_name("mamba2-2.7b")
    cost = bench.algorithmic_cost(cfg)
    x = 4 * 8192 * 80 * 64 * 2
    st = 4 * 80 * 32 * 64 * 128 * 4
    bc = 4 * 8192 * 128 * 2
    gq = 4 * 80 * 8192 * 4
    assert cost["ssd_chunk_scan"][0] == 2 * x + 2 * bc + 2 * gq + st + 80 * 4
    assert cost["ssd_chunk_state"][0] == x + bc + 2 * gq + st


def test_traffic_lookup_follows_source_hash(tmp_path, monkeypatch):
    # Every kernel named in the summary has a well-formed entry.
    for k in bench.KERNELS:
        v = bench.measured_traffic("mamba2-2.7b", k)
        assert v is None or v > 0
    # A summary whose recorded hash differs from the sources yields None.
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "t.md").write_text(
        "traffic ssd_chunk_scan 123 aa\n"
        "traffic ssd_chunk_state 456 0000000000000000\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", {"w": "t.md"})
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_hash", lambda k: {"ssd_chunk_scan": "aa", "ssd_chunk_state": "bb"}[k])
    assert bench.measured_traffic("w", "ssd_chunk_scan") == 123
    assert bench.measured_traffic("w", "ssd_chunk_state") is None
    assert bench.measured_traffic("nope", "ssd_chunk_scan") is None
