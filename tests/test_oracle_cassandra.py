"""Pins for the Cassandra and MX-32 oracles: printed example and codewords,
spec + verification = original, Wanda top-k invariants, unary/tile-table
invariants, entropy bound, brute force and MX invariants."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bits, cassandra, mx
from tests._exact import bf16_frac

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _stream_bits(words, n):
    return "".join("1" if b else "0" for b in cassandra.unpack_bits_lsb(words, n))


@pytest.fixture(scope="module")
def spec_rows():
    wl = synth.WORKLOADS["cassandra_spec"]
    w = synth.gen_weights(wl, 0, 96)
    norms = synth.gen_act_norms(wl)
    return w, norms, cassandra.pack(w, norms)


def test_unary_printed_codewords():
    g = _golden("cassandra_unary_codewords.json")["codewords"]
    for r, cw in g.items():
        words, lengths = cassandra.unary_encode(np.array([int(r)]))
        assert _stream_bits(words, int(lengths[0])) == cw
    words, lengths = cassandra.unary_encode(np.array([0, 1, 2]))
    assert _stream_bits(words, int(lengths.sum())) == g["0"] + g["1"] + g["2"]
    assert int(words[0]) == 0b100101


def test_unary_decode_inverts_encode():
    r = np.random.default_rng(0).geometric(0.45, 5000) - 1
    words, _ = cassandra.unary_encode(r)
    np.testing.assert_array_equal(cassandra.unary_decode(words, r.size), r)


def test_worked_example_truncation_and_restore():
    g = _golden("cassandra_bf16_worked_example.json")
    K = 128
    w = np.full((1, K), 0x3C00, np.uint16)          # 1.0 everywhere
    w[0, 7] = int("0" + "01111100" + g["long_mantissa_field"], 2)   # 0x3E27
    norms = np.ones(K, np.float32)
    norms[7] = 1000.0                                  # make sure element 7 is kept
    sec = cassandra.pack(w, norms)
    keep = cassandra.unpack_bits_lsb(sec["bitmap"], K)
    assert keep[7]
    spec = cassandra.spec_decode(sec, 1, K)
    expect = int("0" + "01111100" + g["long_mantissa_truncated_restored"], 2)
    assert spec[0, 7] == expect == 0x3E20
    assert bits.bf16_value(np.array([expect], np.uint16))[0] == g["value"]
    nib = cassandra.unpack_nibbles(sec["spec_nib"], sec["n_kept"])
    j = int(keep[:7].sum())
    assert format(int(nib[j]) & 7, "03b") == g["kept_mantissa_field"]
    np.testing.assert_array_equal(cassandra.restore(sec, 1, K), w)


def test_speculation_plus_verification_is_original(spec_rows):
    w, norms, sec = spec_rows
    M, K = w.shape
    np.testing.assert_array_equal(cassandra.restore(sec, M, K), w)
    keep = cassandra.unpack_bits_lsb(sec["bitmap"], M * K).reshape(M, K)
    spec = cassandra.spec_decode(sec, M, K)
    np.testing.assert_array_equal(spec, np.where(keep, w & 0xFFF0, 0))


def test_wanda_topk_invariants(spec_rows):
    w, norms, sec = spec_rows
    M, K = w.shape
    keep = cassandra.unpack_bits_lsb(sec["bitmap"], M * K).reshape(M, K)
    assert np.all(keep.sum(axis=1) == (3 * K) // 10)
    score = np.abs(bits.bf16_value(w)) * norms.astype(np.float64)
    for m in range(M):
        assert score[m][keep[m]].min() >= score[m][~keep[m]].max()


def test_wanda_bruteforce_and_ties():
    rng = np.random.default_rng(21)
    for M, K in [(2, 40), (3, 64)]:
        w = synth.f32_to_bf16_bits((rng.standard_t(4, (M, K)) * 0.02).astype(np.float32))
        w[0, 3] = w[0, 9] = w[0, 1]                      # exact ties in |w|
        norms = rng.lognormal(0, 1, K).astype(np.float32)
        norms[3] = norms[9] = norms[1]
        keep = cassandra.keep_mask(w, norms)
        nk = (3 * K) // 10
        for m in range(M):
            sc = [(-(abs(bf16_frac(w[m, k])) * Fraction(float(norms[k]))), k) for k in range(K)]
            chosen = {k for _, k in sorted(sc)[:nk]}
            assert set(np.flatnonzero(keep[m]).tolist()) == chosen


def test_codebook_ranking_and_ties():
    e = np.array([120] * 5 + [121] * 7 + [119] * 5 + [125] * 1)
    cb = cassandra.build_codebook(e)
    assert list(cb) == [121, 119, 120, 125]


def test_tile_table_invariants(spec_rows):
    w, _, sec = spec_rows
    M, K = w.shape
    n = M * K
    T = -(-n // cassandra.TILE)
    bo, kp = sec["bitoff"].astype(np.int64), sec["kprefix"].astype(np.int64)
    assert bo.size == kp.size == T + 1
    keep = cassandra.unpack_bits_lsb(sec["bitmap"], n)
    sbits = cassandra.unpack_bits_lsb(sec["unary"], sec["unary"].size * 32)
    assert int(sbits.sum()) == sec["n_kept"] == kp[-1]
    assert bo[-1] == sec["unary_bits"]
    for t in range(T):
        a, b = t * cassandra.TILE, min(n, (t + 1) * cassandra.TILE)
        assert kp[t + 1] - kp[t] == keep[a:b].sum()
        assert sbits[bo[t]:bo[t + 1]].sum() == kp[t + 1] - kp[t]
        if bo[t] > 0:
            assert sbits[bo[t] - 1]                      # a tile starts right after a codeword end


def test_section_sizes_closed_form(spec_rows):
    w, _, sec = spec_rows
    M, K = w.shape
    nk = sec["n_kept"]
    assert sec["bitmap"].nbytes == M * K // 8
    assert sec["spec_nib"].nbytes == sec["lo_nib"].nbytes == -(-nk // 8) * 4
    assert sec["pruned"].nbytes == 2 * (M * K - nk)


def test_entropy_bound_and_ranges(spec_rows):
    w, _, sec = spec_rows
    st = cassandra.stats(sec, *w.shape)
    assert st["unary_avg_bits"] >= st["entropy_bits"] - 1e-12
    assert 1.0 < st["entropy_bits"] < 4.0


def test_partial_last_tile_and_straddling_rows():
    rng = np.random.default_rng(5)
    M, K = 5, 1000                                       # 5000 elements: one full and one partial tile
    w = synth.f32_to_bf16_bits((rng.standard_t(4, (M, K)) * 0.02).astype(np.float32))
    norms = rng.lognormal(0, 1, K).astype(np.float32)
    sec = cassandra.pack(w, norms)
    assert sec["bitoff"].size == 3
    np.testing.assert_array_equal(cassandra.restore(sec, M, K), w)


# ---------------------------------------------------------------- MX-32

def test_mx_invariants():
    wl = synth.WORKLOADS["cassandra_verify"]
    w = synth.gen_weights(wl, 0, 8)[:, :4096]
    w[0, :32] = 0                                        # all-zero group
    w[1, 32:64] = 0x0005                                 # subnormals only
    M, K = w.shape
    sec = mx.encode(w)
    v = mx.value(sec, M, K)
    ref = bits.bf16_value(w)
    S, E, _ = bits.bf16_fields(w)
    ep = np.maximum(E, 1).reshape(M, K // 32, 32)
    X = sec["mx_exp"].astype(np.int64)
    at_max = (ep == X[..., None]).reshape(M, K)
    np.testing.assert_array_equal(v[at_max], ref[at_max])
    assert np.all(np.abs(v) <= np.abs(ref))
    ulp = np.ldexp(1.0, X - 134)
    assert np.all(np.abs(ref - v).reshape(M, K // 32, 32) < ulp[..., None])
    assert np.all(sec["mx_mag"][0, :32] == 0)
    np.testing.assert_array_equal(v[1, 32:64], ref[1, 32:64])
    # every MX value is exactly a bf16 value
    vb = synth.f32_to_bf16_bits(v.astype(np.float32))
    np.testing.assert_array_equal(bits.bf16_value(vb), v)


# ---------------------------------------------------------------- statistics (closed form)

def _stats_matrix(counts, rng):
    """bf16 [4][1280] whose kept values (the top 384 of each row, norms all 1) have
    exponent 130 + i exactly counts[i] times per row; the pruned values have exponent
    100, far below every kept one, so the keep rule cannot pick them."""
    M, K = 4, 1280
    assert sum(counts) == cassandra.keep_count(K)
    w = np.empty((M, K), np.uint16)
    for r in range(M):
        exps = np.concatenate([np.full(c, 130 + i) for i, c in enumerate(counts)]
                              + [np.full(K - sum(counts), 100)])
        sign = rng.integers(0, 2, K) << 15
        mant = rng.integers(0, 128, K)
        w[r] = rng.permutation((sign | (exps << 7) | mant).astype(np.uint16))
    return w


@pytest.mark.parametrize("counts,H,unary", [
    # four equiprobable exponents: H = 2 bits, codewords 1, 01, 001, 0001 -> 2.5 bits
    ((96, 96, 96, 96), Fraction(2), Fraction(5, 2)),
    # p = 1/2, 1/4, 1/8, 1/8: H = 1.75 bits; average codeword 1/2 + 2/4 + 3/8 + 4/8
    ((192, 96, 48, 48), Fraction(7, 4), Fraction(15, 8)),
])
def test_stats_closed_form(counts, H, unary):
    """Cassandra review 3.3: the exponent entropy and the average unary code length of
    a histogram known in closed form; bits per weight as exact fractions of M*K.  A
    natural-log entropy (2 ln 2 = 1.386 for the first case) or probabilities taken
    over all M*K values instead of the kept ones fails here."""
    w = _stats_matrix(counts, np.random.default_rng(11))
    M, K = w.shape
    norms = np.ones(K, np.float32)
    sec = cassandra.pack(w, norms)
    st = cassandra.stats(sec, M, K)
    n, nk = M * K, M * cassandra.keep_count(K)
    assert st["kept"] == nk
    assert st["entropy_bits"] == pytest.approx(float(H), abs=1e-12)
    assert Fraction(sec["unary_bits"], nk) == unary
    assert st["unary_avg_bits"] == pytest.approx(float(unary), abs=1e-12)
    assert Fraction(st["spec_bpw"]).limit_denominator(n) == Fraction(n + 4 * nk, n) + unary * Fraction(nk, n)
    assert Fraction(st["verify_bpw"]).limit_denominator(n) == Fraction(4 * nk + 16 * (n - nk), n)
    # the codebook ranks the exponents by count, ties to the smaller exponent
    order = sorted(range(4), key=lambda i: (-counts[i], i))
    np.testing.assert_array_equal(sec["codebook"], [130 + i for i in order])
