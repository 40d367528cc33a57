"""Pins of the oracle's fp32 exponential and sigmoid (CPU only).

The sigmoid of the gate (page "feat(engine): E1 DeepSeek-style MoE gate ...", section
"Algorithm": sigmoid of the fp32 gate logits) is 1/(1+exp(-x)).  The oracle's exp is the
Cody-Waite + Taylor construction documented in oracle/oracle.c.  Pins: an exhaustive sweep of
every fp32 input against the fp64 libm exp (closed-form accuracy bound), and exact special
values.
"""
import math
import os
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_exp_special_values():
    assert oracle.exp(0.0) == 1.0
    assert oracle.exp(-0.0) == 1.0
    assert math.isinf(oracle.exp(89.0)) and oracle.exp(89.0) > 0
    assert oracle.exp(float.fromhex("0x1.62e430p+6")) == math.inf
    assert oracle.exp(-88.0) == 0.0  # below ln(FLT_MIN): flushed
    assert oracle.exp(-1000.0) == 0.0
    assert math.isnan(oracle.exp(float("nan")))
    assert oracle.exp(math.inf) == math.inf and oracle.exp(-math.inf) == 0.0
    # exp(1) within 1 ulp of e
    e32 = np.float32(math.e)
    assert abs(oracle.exp(1.0) - float(e32)) <= float(np.spacing(e32))


def test_sigmoid_special_values():
    s = oracle.sigmoid(np.array([0.0, -0.0, 100.0, -100.0, 1e30, -1e30], np.float32))
    assert s[0] == 0.5 and s[1] == 0.5
    assert s[2] == 1.0 and s[4] == 1.0
    assert s[3] < 1e-40 + 1e-43 and s[5] == 0.0
    # symmetry sigma(-x) = 1 - sigma(x) holds to rounding
    x = np.linspace(-10, 10, 2001, dtype=np.float32)
    sp, sm = oracle.sigmoid(x), oracle.sigmoid(-x)
    assert np.max(np.abs((sp.astype(np.float64) + sm) - 1.0)) < 2e-7
    # monotone non-decreasing
    assert np.all(np.diff(sp.astype(np.float64)) >= 0)


def test_sigmoid_matches_fp64_within_2ulp():
    x = np.linspace(-20, 20, 40001, dtype=np.float32)
    s = oracle.sigmoid(x).astype(np.float64)
    ref = 1.0 / (1.0 + np.exp(-x.astype(np.float64)))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(s - ref) / ulp) <= 2.0


def test_exp_exhaustive_sweep(tmp_path):
    """Every fp32 input: max error <= 2 ulp in the normal-result range; +inf above
    ln(FLT_MAX); 0 below ln(FLT_MIN); NaN propagates."""
    exe = str(tmp_path / "exp_sweep")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", os.path.join(HERE, "csrc", "exp_sweep.c"),
                           oracle.lib_path(), "-o", exe, "-lm", f"-Wl,-rpath,{os.path.dirname(oracle.lib_path())}"])
    out = subprocess.check_output([exe], text=True, timeout=600)
    parts = out.split()
    maxulp, checked, special_fail = float(parts[1]), int(parts[5]), int(parts[7])
    assert special_fail == 0, out
    assert checked > 2_000_000_000, out
    assert maxulp <= 2.0, out
