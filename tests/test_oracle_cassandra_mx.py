"""Pins for the Cassandra-2 (MX-32 exponent code) speculation oracle: the printed
bf16 worked example, the pruning and tile table shared with Cassandra-1, exact
agreement with Cassandra-1's draft where a value sits at its group's exponent,
truncation to the shared-exponent grid checked with exact fractions, and the
error bound of one grid step."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bits, cassandra, cassandra_mx
from tests._exact import bf16_frac

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def rows():
    wl = synth.WORKLOADS["cassandra_spec"]
    w = synth.gen_weights(wl, 0, 24)
    norms = synth.gen_act_norms(wl)
    return w, norms, cassandra.pack(w, norms), cassandra_mx.pack_spec(w, norms)


def test_worked_example_at_the_shared_exponent():
    # [Cassandra] §3.1 prints 0.15625 = 0 01111100 0100000; with its 3 kept mantissa
    # bits 010 it is exact, and it stays exact at the group's largest exponent
    g = json.load(open(os.path.join(GOLDEN, "cassandra_bf16_worked_example.json")))
    E, H = g["exponent_biased"], int(g["kept_mantissa_field"], 2)
    mag, X, _ = cassandra_mx.mx_encode(np.array([0, 0]), np.array([E, E - 3]), np.array([H, 7]))
    assert X[0] == E and mag[0] == 8 + H
    assert np.ldexp(float(mag[0]), int(X[0]) - 130) == g["value"]
    # the smaller value, 3 binades down, keeps only its leading bit: 15 >> 3 = 1
    assert mag[1] == 1


def test_pruning_and_tiles_as_cassandra1(rows):
    w, norms, c1, c2 = rows
    np.testing.assert_array_equal(c2["bitmap"], c1["bitmap"])
    np.testing.assert_array_equal(c2["kprefix"], c1["kprefix"])
    assert c2["n_kept"] == c1["n_kept"]
    n = c2["n_kept"]
    assert c2["mx_nib"].size == (n + 7) // 8 and c2["mx_sign"].size == c2["mx_exp"].size == (n + 31) // 32


def test_truncation_to_the_shared_grid(rows):
    """Each draft value is the Cassandra-1 draft value truncated toward zero to a
    multiple of 2^(X - 130), X the largest effective exponent of its group of 32
    kept values (exact fractions)."""
    w, norms, c1, c2 = rows
    M, K = w.shape
    n = c2["n_kept"]
    d1 = cassandra.spec_decode(c1, M, K).reshape(-1)
    keep = cassandra.unpack_bits_lsb(c1["bitmap"], M * K)
    v1 = d1[keep]
    v2 = cassandra_mx.draft_values(c2, n)
    _, E, _ = bits.bf16_fields(v1)
    for g in range(0, (n + 31) // 32, 7):
        sl = slice(32 * g, min(n, 32 * g + 32))
        X = int(np.maximum(E[sl], 1).max())
        assert int(c2["mx_exp"][g]) == X
        step = Fraction(2) ** (X - 130)
        for a, b in zip(v1[sl], v2[sl]):
            exact = bf16_frac(int(a))
            q = abs(exact) // step                          # truncation toward zero
            want = q * step * (1 if exact >= 0 else -1)
            assert Fraction(float(b)) == want


def test_exact_at_group_exponent_and_error_bound(rows):
    w, norms, c1, c2 = rows
    M, K = w.shape
    n = c2["n_kept"]
    keep = cassandra.unpack_bits_lsb(c1["bitmap"], M * K)
    v1 = bits.bf16_value(cassandra.spec_decode(c1, M, K).reshape(-1)[keep])
    v2 = cassandra_mx.draft_values(c2, n)
    _, E, _ = bits.bf16_fields(cassandra.spec_decode(c1, M, K).reshape(-1)[keep])
    X = np.asarray(c2["mx_exp"], np.int64)[np.arange(n) // 32]
    top = np.maximum(E, 1) == X
    np.testing.assert_array_equal(v2[top], v1[top])             # no shift: exact
    assert np.all(np.abs(v2) <= np.abs(v1))
    assert np.all(np.abs(v1 - v2) < np.ldexp(1.0, X - 130))     # below one grid step
    assert np.all(np.sign(v2[v2 != 0]) == np.sign(v1[v2 != 0]))


def test_equal_exponents_reduce_to_cassandra1():
    # all kept values in one binade: MX-32 loses nothing against the unary code
    rng = np.random.default_rng(3)
    M, K = 4, 256
    w = ((rng.integers(0, 2, (M, K)) << 15) | (125 << 7) | rng.integers(0, 128, (M, K))).astype(np.uint16)
    norms = np.ones(K, np.float32)
    c1, c2 = cassandra.pack(w, norms), cassandra_mx.pack_spec(w, norms)
    np.testing.assert_array_equal(cassandra_mx.spec_decode(c2, M, K), cassandra.spec_decode(c1, M, K))


def test_decode_bits_and_pruned_zero(rows):
    w, norms, c1, c2 = rows
    M, K = w.shape
    d = cassandra_mx.spec_decode(c2, M, K)
    keep = cassandra.unpack_bits_lsb(c2["bitmap"], M * K).reshape(M, K)
    assert np.all(d[~keep] == 0)
    vals = bits.bf16_value(d[keep])
    np.testing.assert_array_equal(np.abs(vals), np.abs(cassandra_mx.draft_values(c2, int(keep.sum()))))


def test_subnormal_and_zero_kept_values():
    # a kept zero and a kept subnormal (E = 0): effective exponent 1, no implicit one
    mag, X, _ = cassandra_mx.mx_encode(np.array([0, 1, 0]), np.array([0, 0, 3]), np.array([0, 5, 2]))
    assert X[0] == 3
    assert list(mag) == [0, 5 >> 2, 10]
    assert np.ldexp(10.0, 3 - 130) == bits.bf16_value(np.array([(3 << 7) | (2 << 4)], np.uint16))[0]


def test_spec_bits_below_unary(rows):
    w, norms, c1, c2 = rows
    M, K = w.shape
    n = c2["n_kept"]
    unary_spec = 8 * sum(np.asarray(c1[k]).nbytes for k in ("bitmap", "spec_nib", "unary", "codebook", "bitoff", "kprefix"))
    assert cassandra_mx.spec_bits(c2) < unary_spec
    # 4-bit magnitude, a sign bit and an eighth of a bit of shared exponent per kept value
    assert cassandra_mx.spec_bits(c2) - 8 * c2["bitmap"].nbytes - 8 * c2["kprefix"].nbytes == \
        32 * ((n + 7) // 8) + 32 * ((n + 31) // 32) + 8 * ((n + 31) // 32)
