"""Pins of the oracle's weight unpacker and of the reading of the page's layout.

The page ("BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核",
§5.1 and §5.2) prints the interleave pattern, part of the shift table, the
decode constants and the 16x32 permutation; tests/golden holds them.  Checks:
  * the page's own chain (+2, permute, compress, interleave) round-trips through
    the page's decode, and its printed pattern/shift table agree with each other;
  * hand-worked bytes of the 16x256-tiled layout decode to the right (n, k);
  * every 32-bit word of the tiled layout, decoded the page's way (shift, mask,
    subtract 2), gives the same 16 weights as the oracle's bit-by-bit unpack;
  * code 0 at a real position and non-zero padding are reported.
"""
import numpy as np
import pytest

import oracle
from oracle import pages_layout as pl
from conftest import read_golden


def _golden_kv(name):
    out = {}
    for line in read_golden(name):
        k, v = line.split(":", 1)
        out[k.strip()] = v.split()
    return out


def test_printed_pattern_and_shift_table_agree():
    g = _golden_kv("w2a8_5_2_interleave.txt")
    pattern = [int(v) for v in g["pattern"]]
    shifts = [int(v) for v in g["shift_prefix"]]
    assert tuple(pattern) == pl.PATTERN
    assert sorted(pattern) == list(range(16))
    # element e is moved to field f where pattern[f] == e; its bit offset is 2f
    for e, sh in enumerate(shifts):
        assert 2 * pattern.index(e) == sh
    assert int(g["decode_mask"][0], 16) == 0x03030303
    assert int(g["decode_sub"][0], 16) == 0x02020202
    assert int(g["code_offset"][0]) == 2


def test_block_map_matches_hand_worked_entries_and_is_a_bijection():
    for line in read_golden("w2a8_5_1_block_map.txt"):
        i, j, r, c = (int(v) for v in line.split())
        assert pl.block_map(i, j) == (r, c)
    seen = {pl.block_map(i, j) for i in range(16) for j in range(32)}
    assert seen == {(r, c) for r in range(16) for c in range(32)}
    # each "thread" word (16 consecutive j of one i-pair) reads one row, 16 consecutive columns
    for t in range(32):
        cells = [pl.block_map(t // 2, 16 * (t % 2) + jj) for jj in range(16)]
        assert len({r for r, _ in cells}) == 1
        cols = [c for _, c in cells]
        assert cols == list(range(cols[0], cols[0] + 16))


def test_page_layout_round_trips_through_page_decode():
    g = np.random.Generator(np.random.PCG64(41))
    w = g.integers(-1, 2, size=(32, 64), dtype=np.int8)
    packed = pl.pack(w)
    assert packed.size == w.size // 4
    np.testing.assert_array_equal(pl.unpack(packed, 32, 64), w)


def test_page_decode_of_a_word_yields_consecutive_elements():
    # one word holding codes c_e = e % 3 + 1 for elements e = 0..15, interleaved per the page
    word = 0
    for e in range(16):
        code = e % 3 + 1
        word |= code << (2 * pl.PATTERN.index(e))
    vals = pl.decode_word(word)
    assert vals == [e % 3 + 1 - 2 for e in range(16)]


def _all_zero_tile():
    return np.full(1024, 0xAA, dtype=np.uint8)     # every code 2 (weight 0)


def test_hand_worked_tiled_bytes():
    for line in read_golden("tile_examples.txt"):
        n, k, v, off, byte = line.split()
        n, k, v, off, byte = int(n), int(k), int(v), int(off), int(byte, 16)
        p = _all_zero_tile()
        p[off] = byte
        w = oracle.unpack_tiles(p, 16, 256)
        expect = np.zeros((16, 256), dtype=np.int8)
        expect[n, k] = v
        np.testing.assert_array_equal(w, expect)


def test_tiled_words_decode_the_page_way():
    # random codes in {1,2,3} in every field of a 2x2-tile matrix (no padding)
    g = np.random.Generator(np.random.PCG64(42))
    N, K = 32, 512
    codes = g.integers(1, 4, size=(oracle.packed_bytes(N, K), 4)).astype(np.uint8)
    packed = (codes[:, 0] | codes[:, 1] << 2 | codes[:, 2] << 4 | codes[:, 3] << 6).astype(np.uint8)
    w = oracle.unpack_tiles(packed, N, K)
    words = packed.view("<u4")
    steps = K // 256
    for n in (0, 1, 5, 15, 16, 22, 31):
        for k0 in range(0, K, 16):
            tile = (n // 16) * steps + k0 // 256
            slot = 16 * ((n % 16) // 4) + (k0 % 256) // 16
            word_index = (tile * 1024 + 16 * slot + 4 * (n % 4)) // 4
            assert pl.decode_word(int(words[word_index])) == w[n, k0:k0 + 16].tolist()


def test_padding_layout_and_errors():
    N, K = 70, 300                     # five bands, two steps, ragged in both
    assert oracle.packed_bytes(N, K) == 5 * 2 * 1024
    assert oracle.packed_bytes(16, 256) == 1024
    assert oracle.packed_bytes(13824, 2560) == 13824 * 2560 // 4
    p = np.zeros(oracle.packed_bytes(N, K), dtype=np.uint8)
    # fill real positions with code 2 (weight 0) byte-by-byte through the stated formula
    for n in range(N):
        for k in range(K):
            t = (n // 16) * 2 + k // 256
            e = k % 16
            slot = 16 * ((n % 16) // 4) + (k % 256) // 16
            off = t * 1024 + 16 * slot + 4 * (n % 4) + e % 4
            p[off] |= 2 << (2 * (e // 4))
    assert (oracle.unpack_tiles(p, N, K) == 0).all()
    bad = p.copy()
    bad[0] &= 0xFC                      # w[0][0] becomes code 0
    with pytest.raises(oracle.OracleError, match="code 0"):
        oracle.unpack_tiles(bad, N, K)
    bad = p.copy()
    bad[-1] = 0x01                      # a padding row of the last tile gets a code
    with pytest.raises(oracle.OracleError, match="padding"):
        oracle.unpack_tiles(bad, N, K)
