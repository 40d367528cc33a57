"""Pins of the oracle's router (CPU only).

The router is the linear layer whose fp32 output the gate consumes (gate page, merge
recommendation: router linear, then route; "Algorithm": the gate casts the logits to f32).
Reading: fp32 accumulation by one fused multiply-add per input element, in ascending order,
from +0.  Pins: exact integer dot products (closed form), a cancellation case whose result
is fixed by that order, the forward-error bound of recursive summation against fp64, bf16
inputs widened exactly, and the additive logit offset.
"""
import numpy as np

import oracle
import synth


def test_exact_integer_dot_products():
    rng = np.random.default_rng(0)
    x = rng.integers(-8, 9, (5, 37)).astype(np.float32)
    w = rng.integers(-8, 9, (11, 37)).astype(np.float32)
    got = oracle.router(x, w, "f32")
    assert np.array_equal(got, (x.astype(np.int64) @ w.astype(np.int64).T).astype(np.float32))


def test_summation_order_is_sequential_fp32():
    # 2^25 + 1 - 2^25: ascending-order fp32 accumulation loses the 1 (ulp at 2^25 is 4).
    x = np.array([[2.0 ** 25, 1.0, -(2.0 ** 25)]], np.float32)
    w = np.ones((1, 3), np.float32)
    assert oracle.router(x, w, "f32")[0, 0] == 0.0
    # reversed order keeps it only after the cancellation: -2^25 + 1 + 2^25 = 0 as well; 1 last -> 1
    x2 = np.array([[2.0 ** 25, -(2.0 ** 25), 1.0]], np.float32)
    assert oracle.router(x2, w, "f32")[0, 0] == 1.0


def test_error_bound_against_fp64():
    rng = np.random.default_rng(1)
    H = 1024
    x = rng.normal(0, 1, (16, H)).astype(np.float32)
    w = rng.normal(0, 1 / 32, (24, H)).astype(np.float32)
    got = oracle.router(x, w, "f32").astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    mag = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    gamma = H * 2.0 ** -24 / (1 - H * 2.0 ** -24)
    assert np.all(np.abs(got - ref) <= gamma * mag)


def test_bf16_inputs_are_widened_exactly():
    rng = np.random.default_rng(2)
    xf = rng.normal(0, 1, (8, 64)).astype(np.float32)
    wf = rng.normal(0, 0.1, (4, 64)).astype(np.float32)
    xb, wb = synth.f32_to_bf16(xf), synth.f32_to_bf16(wf)
    a = oracle.router(xb, wb, "bf16")
    b = oracle.router(synth.bf16_to_f32(xb).reshape(8, 64), synth.bf16_to_f32(wb).reshape(4, 64), "f32")
    assert np.array_equal(a, b)


def test_offset_is_one_fp32_add():
    rng = np.random.default_rng(3)
    x = rng.normal(0, 1, (8, 32)).astype(np.float32)
    w = rng.normal(0, 0.2, (6, 32)).astype(np.float32)
    off = rng.normal(0, 2, 6).astype(np.float32)
    assert np.array_equal(oracle.router(x, w, "f32", off), (oracle.router(x, w, "f32") + off).astype(np.float32))
