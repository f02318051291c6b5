"""Host-side views of the cache layout documented in include/qjl.h (numpy only, no device work).

Sign words: natural word w of a token holds projections 32 w .. 32 w + 31 (inlier words first); a
row stores them as 4 groups of W/4 words, group j = inlier words j Win/4 .. then outlier words
Win + j Wout/4 ...  Value codes are stored channel-major in tiles of 32 positions: for each channel,
the codes of a tile's 32 positions in nbits 32-bit words (an LSB-first stream for 2- and 4-bit codes,
a 2-bit plane plus a high-bit word for 3-bit codes), channel c in stream slot 8 (c % 16) + c // 16.  These helpers convert between the stored layout and the natural
one (sign words in projection order, integer codes [..., position, channel]), e.g. to inspect a
cache or to build one on the host.
"""
from __future__ import annotations

import numpy as np

TILE = 32


def bits_slots(m: int, m_out: int) -> np.ndarray:
    """Stored row slot of each natural sign word (index = natural word)."""
    win, wout = m // 32, m_out // 32
    if m % 128 or m_out % 128:
        raise ValueError("m and m_out must be multiples of 128")
    q = (win + wout) // 4
    slots = np.empty(win + wout, dtype=np.int64)
    for w in range(win):
        slots[w] = (w // (win // 4)) * q + w % (win // 4)
    for j in range(wout):
        slots[win + j] = (j // (wout // 4)) * q + win // 4 + j % (wout // 4)
    return slots


def bits_to_stored(words: np.ndarray, m: int, m_out: int) -> np.ndarray:
    """Sign words in natural order [..., W] -> the stored row order."""
    w = np.asarray(words)
    out = np.empty(w.shape, dtype=w.dtype)                   # C order
    out[..., bits_slots(m, m_out)] = w
    return out


def bits_from_stored(stored: np.ndarray, m: int, m_out: int) -> np.ndarray:
    """Stored rows [..., W] -> sign words in natural order (word w = projections 32 w .. 32 w + 31)."""
    return np.ascontiguousarray(np.asarray(stored)[..., bits_slots(m, m_out)])


def code_slot_of_channel(d: int = 128) -> np.ndarray:
    c = np.arange(d)
    return 8 * (c % 16) + c // 16


def code_channel_of_slot(d: int = 128) -> np.ndarray:
    p = np.arange(d)
    return 16 * (p % 8) + p // 8


def code_field_tokens(nbits: int) -> np.ndarray:
    """Token (0..31 within its tile) of each code field of a 2- or 4-bit channel stream: field f
    occupies bits [nbits*f, nbits*f + nbits).  2-bit streams are in token order; 4-bit streams hold in
    word w the tokens 16 (w // 2) + 2 e + (w % 2), e = 0..7 (so the 2-bit planes of a word follow the
    same token order as a 2-bit stream).  3-bit streams are two planes (hi3_bit)."""
    f = np.arange(TILE)
    if nbits != 4:
        return f
    w, e = f // 8, f % 8
    return 16 * (w // 2) + 2 * e + (w % 2)


def hi3_bit(j):
    """Bit of word 2 that holds the high bit of token j (0..31) in a 3-bit stream."""
    j = np.asarray(j)
    return 4 * ((j % 16) // 2) + 2 * (j // 16) + (j % 2)


def codes_from_tiles(tiles: np.ndarray, nbits: int, n: int) -> np.ndarray:
    """uint32 (or int32) code tiles [..., ntiles, d, nbits] -> int64 codes [..., n, d]."""
    t = np.ascontiguousarray(tiles).view(np.uint32)
    *lead, nt, d, nb = t.shape
    if nb != nbits or n > nt * TILE:
        raise ValueError(f"tiles of shape {t.shape} do not hold {n} positions of {nbits}-bit codes")
    bits = (t[..., None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)       # [..., nt, d, nbits, 32]
    if nbits == 3:
        # low plane: words 0, 1 as a 2-bit stream (token order); high plane: word 2 at hi3_bit(token)
        low = bits[..., :2, :].reshape(*lead, nt, d, TILE, 2).astype(np.int64)
        codes = low[..., 0] + 2 * low[..., 1] + 4 * bits[..., 2, :][..., hi3_bit(np.arange(TILE))].astype(np.int64)
    else:
        fields = bits.reshape(*lead, nt, d, TILE, nbits).astype(np.int64)        # stream bit nbits*j + k
        codes = (fields << np.arange(nbits, dtype=np.int64)).sum(axis=-1)          # [..., nt, slot, field]
        codes = codes[..., np.argsort(code_field_tokens(nbits))]                    # [..., nt, slot, token]
    codes = codes[..., code_slot_of_channel(d), :]                                  # [..., nt, channel, 32]
    codes = np.swapaxes(codes, -1, -2).reshape(*lead, nt * TILE, d)
    return np.ascontiguousarray(codes[..., :n, :])


def tiles_from_codes(codes: np.ndarray, nbits: int, ncap: int | None = None) -> np.ndarray:
    """Integer codes [..., n, d] (each < 2^nbits) -> uint32 tiles [..., ceil(ncap/32), d, nbits];
    positions from n up to the tile boundary are zero."""
    c = np.asarray(codes, dtype=np.int64)
    *lead, n, d = c.shape
    ncap = n if ncap is None else ncap
    if ncap < n:
        raise ValueError("ncap is smaller than the number of positions")
    nt = (ncap + TILE - 1) // TILE
    full = np.zeros((*lead, nt * TILE, d), dtype=np.int64)
    full[..., :n, :] = c
    per = np.swapaxes(full.reshape(*lead, nt, TILE, d), -1, -2)                    # [..., nt, channel, 32]
    per = per[..., code_channel_of_slot(d), :]                                      # [..., nt, slot, token]
    if nbits == 3:
        low = (per[..., None] >> np.arange(2, dtype=np.int64)) & 1                  # [..., nt, d, 32, 2]
        stream = low.reshape(*lead, nt, d, 2, 32).astype(np.uint64)
        hi = np.zeros((*lead, nt, d, 32), dtype=np.uint64)
        hi[..., hi3_bit(np.arange(TILE))] = (per >> 2) & 1
        stream = np.concatenate([stream, hi[..., None, :]], axis=-2)                # [..., nt, d, 3, 32]
    else:
        per = per[..., code_field_tokens(nbits)]                                    # [..., nt, slot, field]
        bits = (per[..., None] >> np.arange(nbits, dtype=np.int64)) & 1             # [..., nt, d, 32, nbits]
        stream = bits.reshape(*lead, nt, d, nbits, 32).astype(np.uint64)             # stream bit 32*w + i
    words = (stream << np.arange(32, dtype=np.uint64)).sum(axis=-1)
    return np.ascontiguousarray(words, dtype=np.uint32)     # row-major bytes, as a device copy expects
