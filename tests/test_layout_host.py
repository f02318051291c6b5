"""The host-side views of the value-code tile layout (include/qjl.h, "codes"), pinned against the
documented layout written out bit by bit in plain Python."""
import numpy as np
import pytest

qjl = pytest.importorskip("bit_kv_cache_qjl_amd")
layout = qjl.layout


def tile_words_by_hand(codes, nbits, tile, ch):
    """The nbits words of (tile, channel): position 32*tile + j in bits [nbits*j, nbits*j + nbits)
    of an LSB-first stream; positions past the end count as code 0."""
    stream = 0
    for j in range(32):
        p = 32 * tile + j
        c = int(codes[p, ch]) if p < codes.shape[0] else 0
        for k in range(nbits):
            if (c >> k) & 1:
                stream |= 1 << (nbits * j + k)
    return [(stream >> (32 * w)) & 0xFFFFFFFF for w in range(nbits)]


@pytest.mark.parametrize("nbits", [2, 3, 4])
def test_tiles_match_the_documented_layout(nbits):
    rng = np.random.default_rng(nbits)
    n, d = 75, 128
    codes = rng.integers(0, 2 ** nbits, size=(n, d))
    tiles = layout.tiles_from_codes(codes, nbits, ncap=80)
    assert tiles.shape == (3, d, nbits) and tiles.dtype == np.uint32
    for tile in range(3):
        for ch in (0, 1, 17, 64, 127):
            assert [int(x) for x in tiles[tile, ch]] == tile_words_by_hand(codes, nbits, tile, ch)
    np.testing.assert_array_equal(layout.codes_from_tiles(tiles, nbits, n), codes)


def test_two_bit_tile_by_example():
    """Channel 0 of a 2-bit tile: position j's code in bits 2j, 2j+1 of word j // 16."""
    codes = np.zeros((32, 128), dtype=np.int64)
    codes[0, 0] = 3          # bits 0, 1 of word 0
    codes[15, 0] = 2         # bit 31 of word 0
    codes[16, 0] = 1         # bit 0 of word 1
    codes[5, 1] = 1          # channel 1: bit 10 of its word 0
    t = layout.tiles_from_codes(codes, 2)
    assert t.shape == (1, 128, 2)
    assert int(t[0, 0, 0]) == 0x80000003 and int(t[0, 0, 1]) == 0x1
    assert int(t[0, 1, 0]) == 1 << 10 and int(t[0, 1, 1]) == 0
    assert not t[0, 2:].any()


def test_round_trip_with_leading_dims_and_int32_views():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 4, size=(2, 3, 40, 128))
    t = layout.tiles_from_codes(codes, 2)
    back = layout.codes_from_tiles(t.view(np.int32), 2, 40)
    np.testing.assert_array_equal(back, codes)
    with pytest.raises(ValueError):
        layout.codes_from_tiles(t, 2, 65)
