"""Host-side logic of bench.py (no GPU): the kernel-source hash that keys the
committed counter runs, and the lookup that reports their traffic only while
the kernels are unchanged."""
import json
import os
import shutil

import bench


def _copy_sources(tmp_path):
    csrc = tmp_path / "memory_efficient_attention_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(bench.ROOT, "memory_efficient_attention_amd", "csrc", f), csrc / f)
    return csrc


def test_source_hash_ignores_comments_and_blank_space(tmp_path, monkeypatch):
    csrc = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    f = csrc / bench.KERNEL_SOURCES[0]
    text = f.read_text()
    f.write_text("// a new line comment\n/* and a\n   block comment */\n\n" + text.replace("\n", "\n\n", 3))
    assert bench.kernel_source_hash() == h0
    f.write_text(text + "\nnamespace mea { constexpr int kAnotherConstant = 1; }\n")
    assert bench.kernel_source_hash() != h0


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec = {"source_hash": bench.kernel_source_hash(), "kernels": {"fwd_decode": 4553691582}}
    tf = tmp_path / "traffic.json"
    tf.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tf))
    assert bench.measured_traffic("fwd_decode") == 4553691582
    assert bench.measured_traffic("no_such_kernel") is None
    rec["source_hash"] = "0" * 16
    tf.write_text(json.dumps(rec))
    assert bench.measured_traffic("fwd_decode") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic("fwd_decode") is None
