"""bench.py's memory-traffic figure: read from the committed counter summaries, null once the
code of the kernel source they were measured on has changed (CPU only)."""
import os
import shutil

import bench


def test_every_traffic_summary_is_machine_readable():
    for wl, (prof, src) in bench.TRAFFIC_PROFILES.items():
        text = open(os.path.join(bench.ROOT, "profiles", prof)).read()
        assert "\ntraffic_gb_per_launch: " in text, prof
        assert f"\ncode_sha256: {src} " in text, prof
        assert os.path.exists(os.path.join(bench.ROOT, "deepseek_gate_expert_amd", "csrc", src))


def test_code_hash_ignores_comments_and_layout_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text('int f(int x) {\n  return x + 1;  // one more\n}\nconst char* s = "a // b";\n')
    b = tmp_path / "b.hip"
    b.write_text('/* doc */ int f(int x)\n{ return x + 1; }\n\n// trailing\nconst char* s = "a // b";\n')
    c = tmp_path / "c.hip"
    c.write_text('int f(int x) {\n  return x + 2;  // one more\n}\nconst char* s = "a // b";\n')
    d = tmp_path / "d.hip"
    d.write_text('int f(int x) {\n  return x + 1;  // one more\n}\nconst char* s = "a /* b";\n')
    h = bench.code_sha256
    assert h(str(a)) == h(str(b))
    assert h(str(a)) != h(str(c))      # a changed token
    assert h(str(a)) != h(str(d))      # comment markers inside a string literal are code


def _sandbox(tmp_path, monkeypatch, workload):
    prof, src = bench.TRAFFIC_PROFILES[workload]
    (tmp_path / "profiles").mkdir()
    csrc = tmp_path / "deepseek_gate_expert_amd" / "csrc"
    csrc.mkdir(parents=True)
    shutil.copy(os.path.join(bench.ROOT, "profiles", prof), tmp_path / "profiles" / prof)
    code = open(os.path.join(bench.ROOT, "deepseek_gate_expert_amd", "csrc", src)).read()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path / "profiles" / prof, csrc / src, code


def test_traffic_kept_across_comment_edits_and_null_after_code_edits(tmp_path, monkeypatch):
    prof_path, src_path, code = _sandbox(tmp_path, monkeypatch, "c3")
    src_path.write_text(code)
    measured, _ = bench.traffic_gb("c3")
    if measured is None:
        return  # the committed summary is stale for the current source; nothing to compare
    src_path.write_text("// a new comment line\n" + code.replace("\n", "  \n", 3))
    assert bench.traffic_gb("c3")[0] == measured
    src_path.write_text(code + "\nstatic int extra_symbol_for_the_test;\n")
    gb, why = bench.traffic_gb("c3")
    assert gb is None and "changed" in why


def test_traffic_is_null_without_the_machine_readable_lines(tmp_path, monkeypatch):
    prof_path, src_path, code = _sandbox(tmp_path, monkeypatch, "c3")
    src_path.write_text(code)
    prof_path.write_text(prof_path.read_text().replace("traffic_gb_per_launch:", "traffic:"))
    gb, why = bench.traffic_gb("c3")
    assert gb is None


def test_workloads_without_a_summary_report_null():
    gb, why = bench.traffic_gb("c5")
    assert gb is None
