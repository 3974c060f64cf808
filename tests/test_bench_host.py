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


def test_trace_summary_groups_dispatches_by_workload(tmp_path, monkeypatch):
    """A miniature kernel trace in the default run's call order: each dispatch
    lands in its workload's group, pre-passes with the call they precede and
    second launches / combines with the call they follow."""
    import csv
    t = [0]

    def row(name, us, grid=1024):
        t[0] += 10_000
        r = {"Kernel_Name": f"void mea::{name}(mea::FwdArgs)", "Start_Timestamp": t[0],
             "End_Timestamp": t[0] + int(us * 1000), "Grid_Size_X": grid}
        t[0] += int(us * 1000)
        return r

    pf = "fwd_prefill_kernel<128, true, true, {a}, false, {f}, {v}, {p}>"
    rows = []
    for _ in range(5):  # the step: prefill (pre-pass, main, second launch), then decode
        rows += [row("vt_images_kernel<128, true, false, false>", 100),
                 row(pf.format(a="false", f="false", v="false", p="true"), 3000),
                 row(pf.format(a="false", f="false", v="true", p="false"), 4),
                 row("fwd_decode_partial_kernel<128, true, false, false, false>", 700),
                 row("fwd_decode_combine_kernel<128, true>", 5)]
    rows += [row("vt_images_kernel<128, true, false, false>", 8),
             row(pf.format(a="true", f="false", v="false", p="false"), 160),
             row(pf.format(a="true", f="false", v="true", p="false"), 4)]
    rows += [row("bwd_prep_kernel<128, true>", 400), row("bwd_dkdv_kernel<128, true, true, false>", 7000),
             row("bwd_dq_kernel<128, true, true, false>", 5000)]
    rows += [row("vt_images_kernel<128, true, false, false>", 15),
             row(pf.format(a="false", f="false", v="false", p="false"), 250),
             row(pf.format(a="false", f="false", v="true", p="false"), 4),
             row("fwd_decode_partial_kernel<128, true, false, false, false>", 620),
             row("fwd_decode_combine_kernel<128, true>", 4)]
    rows += [row("vt_images_kernel<128, true, false, true>", 88),
             row(pf.format(a="false", f="true", v="false", p="true"), 2700),
             row("ffn_gemm_kernel<true, true>", 21000)]
    d = tmp_path / "trace"
    d.mkdir()
    with open(d / "kt_kernel_trace.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=list(rows[0].keys()))
        w.writeheader()
        w.writerows(rows)
    out = tmp_path / "stats.md"
    monkeypatch.setattr(bench, "TRACE_SUMMARY_FILE", str(out))
    bench.trace_summary(str(d))
    table = {}
    for line in out.read_text().splitlines():
        cells = [c.strip() for c in line.strip("|").split("|")]
        if len(cells) == 6 and cells[1].startswith("`"):
            table[(cells[0], cells[1].strip("`"))] = (int(cells[2]), float(cells[3]))
    assert table[("prefill (64 sequences)", "vt_images_kernel<128, true, false, false>")] == (5, 100.0)
    assert table[("prefill (64 sequences)", pf.format(a="false", f="false", v="false", p="true"))] == (5, 3000.0)
    assert table[("prefill (64 sequences)", pf.format(a="false", f="false", v="true", p="false"))] == (5, 4.0)
    assert table[("decode", "fwd_decode_combine_kernel<128, true>")] == (5, 5.0)
    assert table[("4 x 2048 prefill + ALiBi", "vt_images_kernel<128, true, false, false>")] == (1, 8.0)
    assert table[("backward", "bwd_dq_kernel<128, true, true, false>")] == (1, 5000.0)
    assert table[("mixed batch: prefill part", pf.format(a="false", f="false", v="false", p="false"))] == (1, 250.0)
    assert table[("mixed batch: decode part", "fwd_decode_combine_kernel<128, true>")] == (1, 4.0)
    assert table[("fp8 prefill", "vt_images_kernel<128, true, false, true>")] == (1, 88.0)
    assert table[("SwiGLU feed-forward", "ffn_gemm_kernel<true, true>")] == (1, 21000.0)
    assert len(table) == 19   # 3 + 2 + 3 + 3 + 3 + 2 + 2 + 1 (workload, kernel) pairs
