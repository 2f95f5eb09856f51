"""Pins for the block-skipping ternary oracle (all-zero blocks flagged and not
stored, [Bonsai2] §3.4 / §5.5): round trip against the dense quantizer (itself
pinned by brute force), the flag rule, byte counts, and the layout against the
dense format's lone-block and pair layouts."""
import numpy as np
import pytest

import synth
from oracle import ternary, ternary_skip


def _sparse(seed, M, K, frac=0.3):
    w = synth.f32_to_bf16_bits((synth.gen_weight_rows(seed, M, K, "t4", 0.02)).astype(np.float32))
    zero = synth.gen_zero_blocks(seed, M, K, frac)
    return synth.zero_out_blocks(w, zero), zero


@pytest.mark.parametrize("M,K", [(37, 384), (16, 128), (5, 1024), (48, 256)])
def test_skip_round_trip_and_flags(M, K):
    w, zero = _sparse(11 + M, M, K)
    q, s = ternary.quantize(w)
    sec = ternary_skip.pack(w)
    # the flagged blocks are exactly the zeroed ones (absmean keeps a +-1 in every
    # block with a non-zero weight)
    np.testing.assert_array_equal(ternary_skip.zero_blocks(q), zero)
    np.testing.assert_array_equal(ternary_skip.unpack_codes(sec, M, K), q)
    np.testing.assert_array_equal(sec["scales"], s)
    assert np.all(s[zero] == 0x3C00)                     # scale 1 for an all-zero block
    stored = int((~zero).sum())
    assert int(sec["tile_base"][-1]) == stored
    assert sec["codes"].size == 8 * stored               # 32 bytes a stored block, none for a zero one
    tiles = (M + 15) // 16
    G = K // 128
    assert ternary_skip.stored_bytes(sec) == 32 * stored + 2 * M * G + 4 * tiles * G + 4 * (tiles + 1)
    np.testing.assert_array_equal(ternary_skip.unpack_dequant(sec, M, K), ternary.dequant(q, s))


def test_skip_slab_words():
    M, K = 21, 384                                       # tiles of 16 and 5 rows
    w, zero = _sparse(5, M, K, 0.4)
    sec = ternary_skip.pack(w)
    slabs = sec["slabs"]
    for t, (r0, R) in enumerate([(0, 16), (16, 5)]):
        before = 0
        for g in range(K // 128):
            mask = int(slabs[t, g]) & 0xFFFF
            want = sum(1 << m for m in range(R) if not zero[r0 + m, g])
            assert mask == want and int(slabs[t, g]) >> 16 == before
            before += bin(want).count("1")
        assert int(sec["tile_base"][t + 1]) - int(sec["tile_base"][t]) == before


def test_skip_layout_matches_dense_lone_block():
    # no flagged block, one block column: the dense format stores a lone block as
    # 8-byte units at kq * R + m, which must be the skip layout with nz = R
    for M in (16, 7, 35):
        w = synth.f32_to_bf16_bits(synth.gen_weight_rows(3, M, 128, "normal", 0.02).astype(np.float32))
        q, _ = ternary.quantize(w)
        sec = ternary_skip.pack(w)
        np.testing.assert_array_equal(sec["codes"], ternary.pack_codes(q))


def test_skip_layout_matches_dense_pair():
    # no flagged block, two block columns: a dense 16-byte unit (m, kq) holds 8
    # bytes of block 0 then 8 of block 1; the skip layout keeps each block column
    # on its own
    M = 16
    w = synth.f32_to_bf16_bits(synth.gen_weight_rows(4, M, 256, "normal", 0.02).astype(np.float32))
    q, _ = ternary.quantize(w)
    dense = ternary.pack_codes(q).reshape(4, M, 2, 2)    # [quarter][row][half][word]
    want = np.concatenate([dense[:, :, 0].reshape(-1), dense[:, :, 1].reshape(-1)])
    np.testing.assert_array_equal(ternary_skip.pack(w)["codes"], want)


def test_skip_layout_ranks_stored_rows():
    # a slab with rows 1 and 3 stored: unit (rank, kq) at kq * 2 + rank
    M, K = 4, 128
    rng = np.random.default_rng(9)
    w = np.zeros((M, K), np.float32)
    w[1] = rng.standard_normal(K)
    w[3] = rng.standard_normal(K)
    wb = synth.f32_to_bf16_bits(w)
    q, _ = ternary.quantize(wb)
    sec = ternary_skip.pack(wb)
    assert int(sec["slabs"][0, 0]) == 0b1010
    words = ternary.pack_codes(q[[1]]), ternary.pack_codes(q[[3]])   # one row: [quarter][word]
    got = sec["codes"].reshape(4, 2, 2)                  # [quarter][rank][word]
    for r in range(2):
        np.testing.assert_array_equal(got[:, r].reshape(-1), words[r])


def test_skip_all_zero_and_no_zero():
    M, K = 20, 256
    sec = ternary_skip.pack(np.zeros((M, K), np.uint16))
    assert sec["codes"].size == 0 and np.all(sec["slabs"] == 0) and np.all(sec["tile_base"] == 0)
    assert np.all(sec["scales"] == 0x3C00)
    np.testing.assert_array_equal(ternary_skip.unpack_codes(sec, M, K), np.zeros((M, K), np.int8))
    w = synth.f32_to_bf16_bits(synth.gen_weight_rows(8, M, K, "t4", 0.02).astype(np.float32))
    sec = ternary_skip.pack(w)
    assert sec["codes"].size == M * K // 16


def test_skip_rejects_bad_tables():
    M, K = 16, 256
    w, _ = _sparse(2, M, K, 0.3)
    sec = ternary_skip.pack(w)
    bad = dict(sec, slabs=sec["slabs"].copy())
    bad["slabs"][0, 1] += 1 << 16                       # wrong in-tile offset
    with pytest.raises(ValueError):
        ternary_skip.unpack_codes(bad, M, K)
    bad = dict(sec, tile_base=sec["tile_base"].copy())
    bad["tile_base"][-1] += 1
    with pytest.raises(ValueError):
        ternary_skip.unpack_codes(bad, M, K)
