"""Pins for oracle.gemv: exact Fraction dot products, one-hot columns, library
agreement at size, and the MoE routing definition."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bits, gemv, ternary
from tests._exact import bf16_frac


def test_gemv_exact_fraction_tiny():
    rng = np.random.default_rng(0)
    M, K, B = 3, 256, 2
    w = synth.f32_to_bf16_bits((rng.standard_normal((M, K)) * 0.02).astype(np.float32))
    x = synth.f32_to_bf16_bits(rng.standard_normal((B, K)).astype(np.float32))
    q, s = ternary.quantize(w)
    deq = ternary.dequant(q, s)
    y = gemv.gemv(deq, x)
    for b in range(B):
        for m in range(M):
            exact = sum(Fraction(float(deq[m, k])) * bf16_frac(x[b, k]) for k in range(K))
            assert abs(Fraction(float(y[b, m])) - exact) <= abs(exact) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 80)


def test_gemv_one_hot_column():
    rng = np.random.default_rng(1)
    w = rng.standard_normal((16, 128))
    x = np.zeros((1, 128), np.uint16)
    x[0, 37] = 0x3F80                                  # 1.0
    np.testing.assert_array_equal(gemv.gemv(w, x)[0], w[:, 37])


def test_gemv_matches_float_sum_at_size():
    wl = synth.WORKLOADS["ternary_1k"]
    w = synth.gen_weights(wl)
    q, s = ternary.quantize(w)
    deq = ternary.dequant(q, s)
    x = synth.gen_x(wl, 1)
    y = gemv.gemv(deq, x)[0]
    xv = bits.bf16_value(x)[0]
    ref = np.array([np.sum(deq[m] * xv) for m in range(deq.shape[0])])
    assert gemv.rel_l2(y, ref) < 1e-12


def test_moe_definition_small():
    rng = np.random.default_rng(2)
    ups = {e: rng.standard_normal((4, 8)) for e in range(3)}
    downs = {e: rng.standard_normal((8, 4)) for e in range(3)}
    routes = np.array([[2, 0], [1, 2]], np.int32)
    x = synth.f32_to_bf16_bits(rng.standard_normal((2, 8)).astype(np.float32))
    a = synth.f32_to_bf16_bits(rng.standard_normal((2, 2, 4)).astype(np.float32))
    yu, yd = gemv.moe(ups, downs, routes, x, a)
    np.testing.assert_allclose(yu[1, 0], ups[1] @ bits.bf16_value(x[1]))
    np.testing.assert_allclose(yd[0, 0], downs[2] @ bits.bf16_value(a[0, 0]))


def test_rel_l2():
    assert gemv.rel_l2([1.0, 0.0], [1.0, 0.0]) == 0.0
    assert abs(gemv.rel_l2([1.0, 1.0], [1.0, 0.0]) - 1.0) < 1e-15


def test_worst_row():
    ref = np.array([[3.0, 4.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0]])   # row RMS 2.5 and 1
    assert gemv.worst_row(ref, ref) == 0.0
    y = ref.copy()
    y[0, 2] += 0.5                                                  # 0.5 / 2.5
    assert gemv.worst_row(y, ref) == pytest.approx(0.2, abs=1e-15)
    y[1, 3] -= 0.3                                                  # 0.3 / 1 dominates
    assert gemv.worst_row(y, ref) == pytest.approx(0.3, abs=1e-15)
    assert gemv.worst_row([[0.0, 0.25]], [[0.0, 0.0]]) == 0.25    # all-zero row: absolute
    # one wrong element among many: rel_l2 dilutes it by sqrt(M), worst_row does not
    M = 8192
    ref = np.ones((1, M))
    y = ref.copy()
    y[0, 17] += 0.05
    assert gemv.rel_l2(y, ref) == pytest.approx(0.05 / np.sqrt(M), rel=1e-12)
    assert gemv.worst_row(y, ref) == pytest.approx(0.05, rel=1e-12)
