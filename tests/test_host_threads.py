"""Thread safety of the library's process-wide host state (CPU only).

The measurement hook (moe_set_stage_events) is the one piece of mutable state that every
moe_forward call reads; its registry (``csrc/stage_hook.hpp``, host code with no HIP header) is
driven here from eight threads under ThreadSanitizer: two re-set the hook while six take event
pairs as concurrent layer calls do.  The program checks that every pair comes from one
consistent setting; ThreadSanitizer checks for data races.  (The other per-device state, the
tiled kernels' configuration, is initialised through std::call_once.)
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build(tmp_path, extra):
    exe = str(tmp_path / "hook_threads")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-pthread", "-I", os.path.join(ROOT, "deepseek_gate_expert_amd", "csrc"),
           os.path.join(ROOT, "tests", "csrc", "hook_threads.cpp"), "-o", exe] + extra
    subprocess.check_call(cmd)
    return exe


def test_hook_registry_under_thread_sanitizer(tmp_path):
    try:
        exe = _build(tmp_path, ["-fsanitize=thread"])
    except subprocess.CalledProcessError:
        pytest.skip("g++ cannot build with ThreadSanitizer here")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, TSAN_OPTIONS="halt_on_error=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ThreadSanitizer" not in r.stderr, r.stderr[-3000:]
    assert "inconsistent 0" in r.stdout


def test_hook_registry_plain_build(tmp_path):
    r = subprocess.run([_build(tmp_path, ["-O2"])], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "inconsistent 0" in r.stdout, r.stdout + r.stderr
