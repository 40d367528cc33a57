"""bench.py's memory-traffic figure: read from the committed counter summaries, null once the
kernel source they were measured on has changed (CPU only)."""
import os
import shutil

import bench


def test_every_traffic_summary_is_machine_readable():
    for wl, (prof, src) in bench.TRAFFIC_PROFILES.items():
        text = open(os.path.join(bench.ROOT, "profiles", prof)).read()
        assert "\ntraffic_gb_per_launch: " in text, prof
        assert f"\nsource_sha256: {src} " in text, prof
        assert os.path.exists(os.path.join(bench.ROOT, "deepseek_gate_expert_amd", "csrc", src))


def test_traffic_is_null_when_the_kernel_source_changed(tmp_path, monkeypatch):
    prof, src = bench.TRAFFIC_PROFILES["c3"]
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "deepseek_gate_expert_amd" / "csrc"
    csrc.mkdir(parents=True)
    shutil.copy(os.path.join(bench.ROOT, "profiles", prof), tmp_path / "profiles" / prof)
    text = (tmp_path / "profiles" / prof).read_text()
    sha = [ln.split()[2] for ln in text.splitlines() if ln.startswith("source_sha256:")][0]
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # a source whose digest is the recorded one cannot be forged here; any other content must give null
    (csrc / src).write_text("// not the measured kernel\n")
    gb, why = bench.traffic_gb("c3")
    assert gb is None and "changed" in why
    # a summary without the machine-readable lines gives null too
    (tmp_path / "profiles" / prof).write_text(text.replace("traffic_gb_per_launch:", "traffic:"))
    gb, why = bench.traffic_gb("c3")
    assert gb is None and sha  # the recorded digest was present; the figure was not


def test_workloads_without_a_summary_report_null():
    gb, why = bench.traffic_gb("c5")
    assert gb is None
