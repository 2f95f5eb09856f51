"""Pins for the ternary and INT4 oracles: closed forms, crafted blocks, invariants,
round trips and exact Fraction brute force on tiny matrices."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import bits, ternary, int4
from tests._exact import bf16_frac, fp16_frac, fp16_bits_value, round_half_even


def _bf16(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def _tiny(seed, M, K, outliers=True):
    rng = np.random.default_rng(seed)
    w = rng.standard_t(4, (M, K)) * 0.02
    if outliers:
        idx = rng.choice(M * K, max(1, M * K // 100), replace=False)
        w.reshape(-1)[idx] *= 10
    return _bf16(w)


# ---------------------------------------------------------------- ternary

def test_ternary_closed_form_threshold():
    w = synth.gen_weights(synth.WORKLOADS["ternary_1k"], 0, 256)
    q, s = ternary.quantize(w)
    wv = bits.bf16_value(w).reshape(256, -1, 128)
    sv = bits.fp16_value(s)[..., None]
    closed = np.sign(wv) * (2 * np.abs(wv) > sv)
    np.testing.assert_array_equal(q.reshape(closed.shape), closed)


def test_ternary_crafted_blocks():
    K = 4 * 128
    w = np.zeros((1, K), np.float32)
    w[0, 0:128] = 0.03                       # constant block -> all +1
    w[0, 128 + 5] = -0.5                     # single non-zero -> -1 there, 0 elsewhere
    # block 3: half the values exactly at s/2 -> code 0, the rest at 3s/2 -> +-1
    w[0, 384:448] = 0.25
    w[0, 448:512] = -0.75                    # mean = 0.5 -> s = 0.5, s/2 = 0.25
    wb = _bf16(w)
    q, s = ternary.quantize(wb)
    sv = bits.fp16_value(s)[0]
    assert np.all(q[0, 0:128] == 1)
    assert q[0, 128 + 5] == -1 and np.count_nonzero(q[0, 128:256]) == 1
    assert sv[1] == bits.fp16_value(bits.fp16_rne(np.array([0.5 / 128])))[0]
    # block 2 is all zero: scale 1.0, all codes 0 (code word value 1)
    assert s[0, 2] == 0x3C00 and np.all(q[0, 256:384] == 0)
    assert sv[3] == 0.5
    assert np.all(q[0, 384:448] == 0) and np.all(q[0, 448:512] == -1)
    codes = ternary.pack_codes(q[:, 256:384])
    assert np.all(codes == 0x55555555)


def test_ternary_idempotent_codes():
    # one block per row, so that rows whose q*s is exact in bf16 can be re-quantized
    w = _tiny(3, 2000, 128)
    q, s = ternary.quantize(w)
    deq = ternary.dequant(q, s)
    w2 = _bf16(deq)                          # q*s is exact in bf16 when s has <= 8 significant bits
    exact = bits.bf16_value(w2) == deq
    q2, _ = ternary.quantize(w2)
    rows = np.all(exact, axis=1)
    assert rows.any()
    np.testing.assert_array_equal(q2[rows], q[rows])


def test_ternary_bruteforce_fraction():
    for seed, (M, K) in [(10, (2, 256)), (11, (3, 384))]:
        w = _tiny(seed, M, K)
        q, s = ternary.quantize(w)
        for m in range(M):
            for g in range(K // 128):
                blk = [bf16_frac(b) for b in w[m, g * 128:(g + 1) * 128]]
                mean = sum(abs(v) for v in blk) / 128
                sf = fp16_frac(mean)
                if mean == 0 or sf == 0:
                    sf = Fraction(1)
                assert fp16_bits_value(int(s[m, g])) == sf
                for i, v in enumerate(blk):
                    r = max(-1, min(1, round_half_even(v / sf)))
                    assert q[m, g * 128 + i] == r


def _tile_of(m, M):
    """(first row, rows) of the 16-row tile that holds row m."""
    t0 = (m // 16) * 16
    return t0, min(16, M - t0)


def ternary_word_index(m, k, M, K):
    """Word holding element (m, k) in the tile-interleaved ternary layout."""
    t0, R = _tile_of(m, M)
    g, kq, j = k // 128, (k % 128) // 32, (k % 32) // 16
    P = (K // 128) // 2
    base = t0 * (K // 16)
    if g < 2 * P:
        return base + (g // 2) * 16 * R + (kq * R + (m - t0)) * 4 + (g % 2) * 2 + j
    return base + P * 16 * R + (kq * R + (m - t0)) * 2 + j


def test_ternary_pack_layout_and_sizes():
    M, K = 19, 384                                     # a partial second tile, an odd block count
    q = np.random.default_rng(4).integers(-1, 2, (M, K)).astype(np.int8)
    words = ternary.pack_codes(q)
    assert words.shape == (M * K // 16,) and words.nbytes == M * K // 4
    # element t of a word (t = k % 16) at bit 2*(t//2) (t even) or 16 + 2*(t//2) (t odd)
    for m in range(M):
        for k in range(K):
            t = k % 16
            bit = 2 * (t // 2) + (16 if t % 2 else 0)
            assert (int(words[ternary_word_index(m, k, M, K)]) >> bit) & 3 == q[m, k] + 1
    one = np.zeros((1, 128), np.int8)
    one[0, 1] = 1                                      # element 1: code 2 at bit 16
    assert ternary.pack_codes(one)[0] == 0x55555555 + (1 << 16)
    np.testing.assert_array_equal(ternary.unpack_codes(words, K), q)
    with pytest.raises(ValueError):
        ternary.unpack_codes(np.full((1, 8), 0xFFFFFFFF, np.uint32), 128)
    # a stack is tiled matrix by matrix
    q2 = np.random.default_rng(5).integers(-1, 2, (2 * 21, 256)).astype(np.int8)
    np.testing.assert_array_equal(ternary.pack_codes(q2, 2),
                                  np.concatenate([ternary.pack_codes(q2[:21]), ternary.pack_codes(q2[21:])]))
    np.testing.assert_array_equal(ternary.unpack_codes(ternary.pack_codes(q2, 2), 256, 2), q2)


def test_ternary_scale_overflow_rejected():
    w = _bf16(np.full((1, 128), 1e6, np.float32))
    with pytest.raises(ValueError):
        ternary.quantize(w)


# ---------------------------------------------------------------- int4

def test_int4_clamp_and_max_code():
    w = synth.gen_weights(synth.WORKLOADS["int4_8k"], 0, 64)
    q, s = int4.quantize(w)
    assert q.min() >= -7 and q.max() <= 7
    g = np.abs(q.reshape(64, -1, 128)).max(axis=-1)
    assert np.all(g == 7)
    c = (int4.pack_codes(q)[..., None] >> int4.SHIFTS.astype(np.uint32)) & 15
    assert c.min() >= 1


def test_int4_round_trip():
    w = _tiny(5, 2000, 128)
    q, s = int4.quantize(w)
    deq = int4.dequant(q, s)
    w2 = _bf16(deq)
    rows = np.all(bits.bf16_value(w2) == deq, axis=1)
    assert rows.any()
    q2, s2 = int4.quantize(w2[rows])
    np.testing.assert_array_equal(q2, q[rows])
    np.testing.assert_array_equal(s2, s[rows])


def test_int4_zero_group_and_ties():
    s = 0.5
    w = np.zeros((1, 256), np.float32)
    w[0, 128] = 7 * s                     # group 1: scale exactly 0.5
    w[0, 129] = 2.5 * s                   # tie 2.5 -> 2 (half to even)
    w[0, 130] = -3.5 * s                  # tie -3.5 -> -4
    w[0, 131] = 0.5 * s                   # tie 0.5 -> 0
    q, sb = int4.quantize(_bf16(w))
    assert sb[0, 0] == 0x3C00 and np.all(q[0, :128] == 0)
    assert bits.fp16_value(sb)[0, 1] == s
    assert list(q[0, 128:132]) == [7, 2, -4, 0]


def test_int4_bruteforce_fraction():
    for seed, (M, K) in [(12, (2, 256)), (13, (3, 384))]:
        w = _tiny(seed, M, K)
        q, s = int4.quantize(w)
        for m in range(M):
            for g in range(K // 128):
                blk = [bf16_frac(b) for b in w[m, g * 128:(g + 1) * 128]]
                amax = max(abs(v) for v in blk)
                sf = fp16_frac(amax / 7)
                if amax == 0 or sf == 0:
                    sf = Fraction(1)
                assert fp16_bits_value(int(s[m, g])) == sf
                for i, v in enumerate(blk):
                    assert q[m, g * 128 + i] == max(-7, min(7, round_half_even(v / sf)))


def int4_word_index(m, k, M, K):
    """Word holding element (m, k) in the tile-interleaved INT4 layout."""
    t0, R = _tile_of(m, M)
    g, kq, i = k // 128, (k % 128) // 32, (k % 32) // 8
    return t0 * (K // 8) + g * 16 * R + (kq * R + (m - t0)) * 4 + i


def test_int4_pack_layout_and_sizes():
    M, K = 19, 384
    q = np.random.default_rng(6).integers(-7, 8, (M, K)).astype(np.int8)
    words = int4.pack_codes(q)
    assert words.nbytes == M * K // 2
    for m in range(M):
        for k in range(K):
            t = k % 8
            bit = 4 * (t // 2) + (16 if t % 2 else 0)
            assert (int(words[int4_word_index(m, k, M, K)]) >> bit) & 15 == q[m, k] + 8
    one = np.zeros((1, 128), np.int8)
    one[0, 3] = 7                                      # element 3: code 15 at bit 20
    assert int4.pack_codes(one)[0] == 0x88888888 + (7 << 20)
    np.testing.assert_array_equal(int4.unpack_codes(words, K), q)
    scales = int4.quantize(_tiny(7, M, K))[1]
    assert scales.nbytes == 2 * M * K // 128
    q2 = np.random.default_rng(8).integers(-7, 8, (2 * 33, 128)).astype(np.int8)
    np.testing.assert_array_equal(int4.pack_codes(q2, 2),
                                  np.concatenate([int4.pack_codes(q2[:33]), int4.pack_codes(q2[33:])]))
