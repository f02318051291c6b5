"""The host-side views of the value-code tile layout (include/qjl.h, "codes"), pinned against the
documented layout written out bit by bit in plain Python."""
import numpy as np
import pytest

qjl = pytest.importorskip("bit_kv_cache_qjl_amd")
layout = qjl.layout


def tile_words_by_hand(codes, nbits, tile, ch):
    """The nbits words of (tile, channel).  2 bits: position 32*tile + j in bits [2j, 2j + 2) of an
    LSB-first stream.  4 bits: word w, nibble e holds position 32*tile + 16*(w // 2) + 2*e + (w % 2).
    3 bits: words 0 and 1 hold the low two bits of each code as the 2-bit stream does, word 2 the high
    bit of position 32*tile + j at bit 4*((j % 16) // 2) + 2*(j // 16) + j % 2.  Positions past the end
    count as code 0."""
    def code(j):
        p = 32 * tile + j
        return int(codes[p, ch]) if p < codes.shape[0] else 0
    if nbits == 4:
        return [sum(code(16 * (w // 2) + 2 * e + (w % 2)) << (4 * e) for e in range(8)) for w in range(4)]
    if nbits == 3:
        low = sum((code(j) & 3) << (2 * j) for j in range(32))
        high = sum((code(j) >> 2) << (4 * ((j % 16) // 2) + 2 * (j // 16) + j % 2) for j in range(32))
        return [low & 0xFFFFFFFF, low >> 32, high]
    stream = 0
    for j in range(32):
        c = code(j)
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
            slot = 8 * (ch % 16) + ch // 16
            assert [int(x) for x in tiles[tile, slot]] == tile_words_by_hand(codes, nbits, tile, ch)
    np.testing.assert_array_equal(layout.codes_from_tiles(tiles, nbits, n), codes)
    # device copies take the bytes as they lie: every helper returns C-contiguous arrays
    assert tiles.flags.c_contiguous and layout.codes_from_tiles(tiles, nbits, n).flags.c_contiguous


def test_two_bit_tile_by_example():
    """Channel 0 of a 2-bit tile: position j's code in bits 2j, 2j+1 of word j // 16."""
    codes = np.zeros((32, 128), dtype=np.int64)
    codes[0, 0] = 3          # bits 0, 1 of word 0
    codes[15, 0] = 2         # bit 31 of word 0
    codes[16, 0] = 1         # bit 0 of word 1
    codes[5, 1] = 1          # channel 1 (stream slot 8): bit 10 of its word 0
    codes[31, 16] = 3        # channel 16 (stream slot 1): bits 30, 31 of its word 1
    t = layout.tiles_from_codes(codes, 2)
    assert t.shape == (1, 128, 2)
    assert int(t[0, 0, 0]) == 0x80000003 and int(t[0, 0, 1]) == 0x1
    assert int(t[0, 8, 0]) == 1 << 10 and int(t[0, 8, 1]) == 0
    assert int(t[0, 1, 0]) == 0 and int(t[0, 1, 1]) == 0xC0000000
    assert not t[0, 2:8].any() and not t[0, 9:].any()


def test_four_bit_tile_by_example():
    """Channel 0 of a 4-bit tile: word 0 holds positions 0, 2, .., 14, word 1 positions 1, 3, .., 15,
    words 2 and 3 the same for 16..31; position 2e + (w % 2) + 16 (w // 2) in nibble e of word w."""
    codes = np.zeros((32, 128), dtype=np.int64)
    codes[0, 0] = 0xF        # word 0, nibble 0
    codes[14, 0] = 0x9       # word 0, nibble 7
    codes[1, 0] = 0x3        # word 1, nibble 0
    codes[31, 0] = 0x5       # word 3, nibble 7
    codes[18, 0] = 0x2       # word 2, nibble 1
    t = layout.tiles_from_codes(codes, 4)
    assert [int(x) for x in t[0, 0]] == [0x9000000F, 0x3, 0x20, 0x50000000]


def test_three_bit_tile_by_example():
    """Channel 0 of a 3-bit tile, and the planes the decode reads: nibble n of (word 2 >> k) & 0x11111111
    is the high bit of the position whose low bits nibble n of the k-th 2-bit plane holds."""
    codes = np.zeros((32, 128), dtype=np.int64)
    codes[5, 0] = 7          # low bits 10, 11 of word 0; high bit 4*2 + 0 + 1 = 9 of word 2
    codes[20, 0] = 4         # low bits 0 (bits 8, 9 of word 1); high bit 4*2 + 2 + 0 = 10
    codes[31, 0] = 6         # low 2 at bits 30, 31 of word 1; high bit 4*7 + 2 + 1 = 31
    t = layout.tiles_from_codes(codes, 3)
    assert [int(x) for x in t[0, 0]] == [0xC00, 0x80000000, (1 << 9) | (1 << 10) | (1 << 31)]
    rng = np.random.default_rng(9)
    c = rng.integers(0, 8, size=(32, 128))
    w = layout.tiles_from_codes(c, 3)[0, 0].astype(np.int64)
    planes = [w[0] & 0x33333333, (w[0] >> 2) & 0x33333333, w[1] & 0x33333333, (w[1] >> 2) & 0x33333333]
    tokens = [[2 * n, 2 * n + 1, 16 + 2 * n, 17 + 2 * n] for n in range(8)]
    for k in range(4):
        hi = (w[2] >> k) & 0x11111111
        for n in range(8):
            j = tokens[n][k]
            assert (planes[k] >> (4 * n)) & 3 == c[j, 0] & 3
            assert (hi >> (4 * n)) & 1 == c[j, 0] >> 2


def test_round_trip_with_leading_dims_and_int32_views():
    rng = np.random.default_rng(5)
    codes = rng.integers(0, 4, size=(2, 3, 40, 128))
    t = layout.tiles_from_codes(codes, 2)
    back = layout.codes_from_tiles(t.view(np.int32), 2, 40)
    np.testing.assert_array_equal(back, codes)
    with pytest.raises(ValueError):
        layout.codes_from_tiles(t, 2, 65)


def test_sign_word_row_order():
    """m = m_out = 256 (8 + 8 words): row = 4 groups of (2 inlier, 2 outlier) words."""
    slots = layout.bits_slots(256, 256)
    # natural words 0..7 inlier, 8..15 outlier; group j holds inlier 2j, 2j+1 and outlier 8+2j, 9+2j
    expect_row = [0, 1, 8, 9, 2, 3, 10, 11, 4, 5, 12, 13, 6, 7, 14, 15]
    for slot, word in enumerate(expect_row):
        assert slots[word] == slot
    assert list(layout.bits_slots(128, 0)) == [0, 1, 2, 3]          # no outlier sketch: natural order
    assert list(layout.bits_slots(512, 0)) == list(range(16))
    # m = m_out = 128: row = inlier 0, outlier 0, inlier 1, outlier 1, ...
    assert list(layout.bits_slots(128, 128)) == [0, 2, 4, 6, 1, 3, 5, 7]
    rng = np.random.default_rng(3)
    words = rng.integers(0, 2 ** 32, size=(2, 5, 32), dtype=np.uint64).astype(np.uint32)
    for m, m_out in [(512, 512), (1024, 0), (256, 128 * 2)]:
        w = words[..., : (m + m_out) // 32]
        st = layout.bits_to_stored(w, m, m_out)
        np.testing.assert_array_equal(layout.bits_from_stored(st, m, m_out), w)
        assert st.flags.c_contiguous and layout.bits_from_stored(st, m, m_out).flags.c_contiguous
    with pytest.raises(ValueError):
        layout.bits_slots(96, 0)
