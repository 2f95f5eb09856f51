"""Pins for oracle.bits: the Cassandra bf16 worked example and library cross-checks."""
import json
import os

import numpy as np

from oracle import bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_fields_and_value():
    g = _golden("cassandra_bf16_worked_example.json")
    s, e, m = g["fields"].split()
    b = int(s + e + m, 2)
    assert b == 0x3E20
    S, E, M = bits.bf16_fields(np.array([b], np.uint16))
    assert (int(S[0]), int(E[0])) == (g["sign"], g["exponent_biased"])
    assert int(E[0]) - 127 == g["exponent_unbiased"]
    assert int(M[0]) / 128 == g["mantissa_fraction"]
    assert bits.bf16_value(np.array([b], np.uint16))[0] == g["value"]


def test_worked_example_long_mantissa_value():
    g = _golden("cassandra_bf16_worked_example.json")
    b = int("0" + "01111100" + g["long_mantissa_field"], 2)
    assert b == 0x3E27
    # 1.0100111b * 2^-3 = (128 + 39) / 128 / 8
    assert bits.bf16_value(np.array([b], np.uint16))[0] == (128 + 39) / 1024


def test_bf16_value_matches_float32_view():
    rng = np.random.default_rng(1)
    b = rng.integers(0, 1 << 16, 200000, dtype=np.uint32).astype(np.uint16)
    b = b[((b >> 7) & 0xFF) != 255]
    ref = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(bits.bf16_value(b), ref)


def test_bf16_rejects_inf_nan():
    import pytest
    with pytest.raises(ValueError):
        bits.bf16_value(np.array([0x7F80], np.uint16))


def _fp16_midpoints(rng, n):
    h = rng.integers(0, 0x7BFF, n).astype(np.uint16)
    lo = np.array(h, np.uint16).view(np.float16).astype(np.float64)
    hi = np.array(h + 1, np.uint16).view(np.float16).astype(np.float64)
    return (lo + hi) / 2          # exact in float64


def test_fp16_rne_matches_numpy_half():
    rng = np.random.default_rng(2)
    v = np.concatenate([
        rng.standard_normal(100000) * 10.0 ** rng.integers(-9, 5, 100000),
        _fp16_midpoints(rng, 50000),
        -_fp16_midpoints(rng, 50000),
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e6, 2.0 ** -24, 2.0 ** -25,
                  2.0 ** -25 * 1.0000001, 3 * 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25]),
    ])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(bits.fp16_rne(v), ref)


def test_fp16_value_matches_numpy_half():
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    h = np.concatenate([h, h | 0x8000])
    np.testing.assert_array_equal(bits.fp16_value(h), h.view(np.float16).astype(np.float64))
