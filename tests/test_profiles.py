"""The committed rocprofv3 summaries: each gives the command that made it and
the traffic figures bench.py reports still belong to the current sources."""
import glob
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

PROFILES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md")))


def test_every_summary_names_its_command():
    assert PROFILES
    for p in PROFILES:
        text = open(p).read()
        assert "rocprofv3" in text or "calibration" in os.path.basename(p), p
        assert "/root/repo/" in text, p          # the command runs committed files of the repository


def test_traffic_summaries_are_well_formed():
    """Each traffic summary carries the figure bench.py reads, the kernel's
    sources (files of the repository) and their hash; bench.py reports the
    figure only while the sources still hash to it (else null)."""
    traffic = [p for p in PROFILES if p.endswith("_hbm_traffic.md")]
    assert traffic
    for p in traffic:
        fields = dict(l.split(": ", 1) for l in open(p).read().splitlines()
                      if l.startswith(("traffic_bytes_per_launch:", "kernel_sources:", "kernel_source_sha256:")))
        assert int(fields["traffic_bytes_per_launch"]) > 0, p
        assert len(fields["kernel_source_sha256"]) == 64, p
        for f in fields["kernel_sources"].split():
            assert os.path.exists(os.path.join(ROOT, f)), (p, f)


def test_stale_hash_is_not_reported(tmp_path, monkeypatch):
    src = os.path.join(ROOT, "profiles", "k_matmul_q4_0_2048x12288x4096_hbm_traffic.md")
    text = open(src).read()
    lines = [l if not l.startswith("kernel_source_sha256:") else "kernel_source_sha256: " + "0" * 64
             for l in text.splitlines()]
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / os.path.basename(src)).write_text("\n".join(lines))
    for f in ("matmul_quantize_q8_amd",):
        os.symlink(os.path.join(ROOT, f), tmp_path / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.committed_traffic("k_matmul_q4_0", "2048x12288x4096") is None
