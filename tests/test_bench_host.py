"""Host logic of bench.py that needs no GPU: the counted-traffic figure is
taken from a counter summary only while that summary's kernel-source hash is
the current one, and every committed summary parses."""
import glob
import os

import pytest

import bench

TRAFFIC_LINE = ("traffic: source_hash={h} bytes_per_launch=423637438 fetch_bytes=249508286 write_bytes=174129152 "
                "fetch_scale=1.9999 write_scale=1.0000\n")


def _profile_dir(tmp_path, name, h):
    d = tmp_path / "profiles"
    d.mkdir()
    (d / name).write_text("# summary\n\nsome text\n\n" + TRAFFIC_LINE.format(h=h))
    return tmp_path


def test_read_traffic_current_hash(tmp_path, monkeypatch):
    root = _profile_dir(tmp_path, "prefill_kernel_chunked_prefill_traffic.md", "0123456789abcdef")
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "source_hash", lambda: "0123456789abcdef")
    assert bench.read_traffic("prefill_kernel", "chunked_prefill") == 423637438.0
    # another kernel or workload has no summary
    assert bench.read_traffic("prefill_kernel", "mixed_serving") is None
    assert bench.read_traffic("decode_split_kernel", "chunked_prefill") is None


def test_read_traffic_stale_hash_is_null(tmp_path, monkeypatch):
    root = _profile_dir(tmp_path, "decode_split_kernel_long_decode_traffic.md", "0123456789abcdef")
    monkeypatch.setattr(bench, "ROOT", str(root))
    monkeypatch.setattr(bench, "source_hash", lambda: "fedcba9876543210")
    assert bench.read_traffic("decode_split_kernel", "long_decode") is None


SUMMARIES = sorted(glob.glob(os.path.join(os.path.dirname(os.path.abspath(bench.__file__)), "profiles", "*_traffic.md")))


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_committed_traffic_summaries_parse(path):
    lines = [ln for ln in open(path) if ln.startswith("traffic:")]
    assert len(lines) == 1, path
    rec = dict(kv.split("=") for kv in lines[0][len("traffic:"):].split())
    assert len(rec["source_hash"]) == 16
    fetch, write, total = int(rec["fetch_bytes"]), int(rec["write_bytes"]), int(rec["bytes_per_launch"])
    assert fetch > 0 and write > 0 and total == fetch + write
    assert 1.5 < float(rec["fetch_scale"]) < 2.5 and 0.5 < float(rec["write_scale"]) < 1.5
