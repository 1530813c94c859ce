"""Host-side logic of bench.py: the HBM-traffic figure read from a committed
counter summary, reported only while the kernel's sources are unchanged."""

import hashlib
import os

import bench


def _tree(tmp_path, sources, traffic, sha=None):
    csrc = tmp_path / "fp4_kv_cache_index_amd" / "csrc"
    csrc.mkdir(parents=True)
    h = hashlib.sha256()
    for name, text in sources.items():
        (csrc / name).write_bytes(text)
        h.update(text)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "index_score_decode64k_hbm_counters.md").write_text(
        "# HBM traffic counters\n\n"
        "| kernel | FETCH_SIZE KiB/dispatch |\n|---|---:|\n| `x` | 1.0 |\n\n"
        "Machine-read values (prose with: a colon):\n\n"
        f"kernel: index_score\n"
        f"kernel_source_files: {' '.join(sources)}\n"
        f"kernel_source_sha256: {sha or h.hexdigest()}\n"
        f"traffic_bytes_per_launch: {traffic}\n")
    return csrc


def test_counter_traffic_reported_while_sources_match(tmp_path, monkeypatch):
    csrc = _tree(tmp_path, {"a.hip": b"kernel one\n", "b.h": b"header\n"}, 12345)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("index_score") == 12345
    # any change to a listed source withdraws the figure
    (csrc / "b.h").write_bytes(b"header, edited\n")
    assert bench.counter_traffic("index_score") is None


def test_counter_traffic_missing_or_stale_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("index_score") is None          # no summary at all
    _tree(tmp_path, {"a.hip": b"k\n"}, 7, sha="0" * 64)
    assert bench.counter_traffic("index_score") is None          # recorded hash differs
    assert bench.counter_traffic("other_kernel") is None         # no summary for that kernel


def test_committed_summary_is_readable():
    """The committed summary parses; its figure is either withheld (sources
    edited since the counters were taken) or a plausible byte count."""
    t = bench.counter_traffic("index_score")
    assert t is None or 5e8 < t < 1e9
    assert os.path.exists(os.path.join(bench.ROOT, "profiles", "index_score_decode64k_hbm_counters.md"))
