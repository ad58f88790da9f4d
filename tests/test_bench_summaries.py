"""bench.py's reading of the committed rocprofv3 summaries (host logic only)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _write(path, workload, digest, extra):
    lines = ["# summary", "", "- workload: `%s`" % workload]
    lines += ["- %s: `%s`" % kv for kv in extra.items()]
    lines.append("- kernel_source_sha256: `%s`" % digest)
    path.write_text("\n".join(lines) + "\n")


COUNTERS = {"mfma_busy_frac": "0.5", "clock_ghz": "1.9", "valu_coexec_frac": "0.4",
            "valu_insts_per_score_element": "5.0", "trans_insts_per_score_element": "1.0",
            "lds_insts_per_wave_tile": "48.0", "lds_bank_conflict_cycles": "0"}


def test_summaries_read_only_when_current(tmp_path, monkeypatch):
    wl = "B2_H32_L4096_d128_bf16_causal"
    t, c = tmp_path / "traffic.md", tmp_path / "counters.md"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(t))
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(c))
    assert bench.stored_traffic(wl) is None and bench.stored_counters(wl) is None   # missing files
    digest = bench.kernel_source_digest()
    _write(t, wl, digest, {"hbm_bytes_per_launch": "123456"})
    _write(c, wl, digest, COUNTERS)
    assert bench.stored_traffic(wl) == 123456.0
    got = bench.stored_counters(wl)
    assert got["mfma_busy_frac"] == 0.5 and got["lds_insts_per_wave_tile"] == 48.0
    assert bench.stored_traffic("B1_H16_L16384_d128_bf16_causal") is None        # other workload
    _write(t, wl, "0" * 16, {"hbm_bytes_per_launch": "123456"})                   # stale kernel
    _write(c, wl, "0" * 16, COUNTERS)
    assert bench.stored_traffic(wl) is None and bench.stored_counters(wl) is None
    bad = dict(COUNTERS)
    del bad["clock_ghz"]
    _write(c, wl, digest, bad)                                                     # incomplete
    assert bench.stored_counters(wl) is None


def test_digest_ignores_comments(tmp_path, monkeypatch):
    """Editing a comment in the kernel sources does not make stored counters stale."""
    src = os.path.join(ROOT, "flashattention_forward_fwd_amd", "csrc")
    copy = tmp_path / "flashattention_forward_fwd_amd" / "csrc"
    copy.mkdir(parents=True)
    for name in os.listdir(src):
        if name.endswith((".h", ".hip")):
            (copy / name).write_text(open(os.path.join(src, name)).read())
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    d0 = bench.kernel_source_digest()
    k = copy / "fa2_fwd_bf16.hip"
    k.write_text("// a new comment line\n" + k.read_text().replace("// ", "//  ", 3))
    assert bench.kernel_source_digest() == d0
    k.write_text(k.read_text() + "\nstatic int changed_code = 1;\n")
    assert bench.kernel_source_digest() != d0
