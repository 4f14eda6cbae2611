"""Host logic of bench.py that needs no GPU: the lookup of calibrated HBM
traffic in the profile summaries, which must match the kernel name (names
carry spaces, as rocprofv3 prints them) and the fingerprint of the current
library sources, and nothing else."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _tree(tmp_path, source_text):
    csrc = tmp_path / "hierarchical_sparse_attention_build_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text(source_text)
    (tmp_path / "include").mkdir()
    (tmp_path / "include" / "hga.h").write_text("/* header */\n")
    (tmp_path / "profiles").mkdir()
    return tmp_path


def test_traffic_lookup_matches_spaced_names_and_current_sources(tmp_path, monkeypatch):
    root = _tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    fp = bench.source_fingerprint()
    (root / "profiles" / "p.md").write_text(
        "| table | row |\n"
        f"`traffic decode_step_kernel<bf16, 128, 4> 49820462 sources {fp}`  \n"
        f"`traffic hga_attend_prefill 1699086511 sources {fp}`  \n"
        "`traffic old_kernel<1, 2> 5 sources 0000`  \n")
    assert bench.measured_traffic("decode_step_kernel<bf16,128,4>") == 49820462
    assert bench.measured_traffic("decode_step_kernel<bf16, 128, 4>") == 49820462
    assert bench.measured_traffic("hga_attend_prefill") == 1699086511
    assert bench.measured_traffic("decode_step_kernel<bf16,128,2>") is None
    assert bench.measured_traffic("old_kernel<1,2>") is None  # taken on other sources


def test_traffic_lookup_ignores_counters_of_changed_sources(tmp_path, monkeypatch):
    root = _tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    fp_old = bench.source_fingerprint()
    (root / "profiles" / "p.md").write_text(f"`traffic k<128, 4> 77 sources {fp_old}`\n")
    assert bench.measured_traffic("k<128,4>") == 77
    (root / "hierarchical_sparse_attention_build_amd" / "csrc" / "k.hip").write_text("kernel v2\n")
    assert bench.source_fingerprint() != fp_old
    assert bench.measured_traffic("k<128,4>") is None
