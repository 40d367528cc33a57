"""The oracle and the input generator under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The gate page's test plan and its author's reply hold the GPU suites to ASan/UBSan cleanliness
("feat(engine): E1 DeepSeek-style MoE gate (sigmoid, group top-k, bias) (#108)", "Test plan").
Here the host C of this repository -- ``oracle/oracle.c`` and ``synth/synth.c`` -- is rebuilt
with ``-fsanitize=address,undefined`` (errors fatal) and every oracle pin runs against those
builds in a child process that preloads the ASan runtime.  A canary first shows that the same
flags do catch an out-of-bounds read and a signed overflow.
"""
import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
LIB_FLAGS = ["-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off"]
PINS = ["test_oracle_dispatch.py", "test_oracle_gate.py", "test_oracle_router.py", "test_oracle_exp.py",
        "test_oracle_layer.py", "test_oracle_dense.py", "test_oracle_fp8.py", "test_oracle_softmax.py"]


def _runtime():
    p = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


ASAN_RT = _runtime()
pytestmark = pytest.mark.skipif(ASAN_RT is None, reason="gcc has no AddressSanitizer runtime here")


def _env(extra=None):
    env = dict(os.environ)
    env.update({"LD_PRELOAD": ASAN_RT, "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
                "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"})
    env.update(extra or {})
    return env


@pytest.fixture(scope="module")
def san_libs(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    out = {}
    for name, src in (("oracle", "oracle/oracle.c"), ("synth", "synth/synth.c")):
        so = str(d / f"lib{name}_san.so")
        subprocess.check_call(["gcc"] + SAN + LIB_FLAGS + [os.path.join(ROOT, src), "-o", so, "-lm"])
        out[name] = so
    return out


@pytest.mark.parametrize("kind,body", [
    ("heap-buffer-overflow", "int *a = malloc(4 * sizeof(int)); volatile int i = 4; int v = a[i]; free(a); return v;"),
    ("signed-integer-overflow", "volatile int x = 2147483647; x = x + 1; return x & 1;"),
])
def test_canary_flags_catch_errors(tmp_path, kind, body):
    src = tmp_path / "canary.c"
    src.write_text(textwrap.dedent(f"""
        #include <stdlib.h>
        int main(void) {{ {body} }}
    """))
    exe = str(tmp_path / "canary")
    subprocess.check_call(["gcc"] + SAN + [str(src), "-o", exe])
    r = subprocess.run([exe], capture_output=True, text=True, env=_env({"LD_PRELOAD": ""}))
    assert r.returncode != 0 and ("AddressSanitizer" in r.stderr or "runtime error" in r.stderr), r.stderr


def test_oracle_pins_clean_under_sanitizers(san_libs):
    script = textwrap.dedent(f"""
        import sys
        sys.path.insert(0, {ROOT!r})
        import oracle, synth
        oracle._L(); synth._L()
        maps = open("/proc/self/maps").read()
        assert "liboracle_san.so" in maps and "libsynth_san.so" in maps, "sanitized builds not loaded"
        assert "liboracle.so" not in maps and "libsynth.so" not in maps
        import pytest
        sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu"] +
                             [{os.path.join(ROOT, "tests")!r} + "/" + f for f in {PINS!r}]))
    """)
    env = _env({"DSMOE_ORACLE_LIB": san_libs["oracle"], "DSMOE_SYNTH_LIB": san_libs["synth"]})
    r = subprocess.run([sys.executable, "-c", script], capture_output=True, text=True, env=env, cwd=ROOT,
                       timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "failed" not in r.stdout, tail
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, tail
