"""Host-side views of the cache layout documented in include/qjl.h (numpy only, no device work).

Value codes are stored channel-major in tiles of 32 positions: for each channel, the codes of a
tile's 32 positions form an LSB-first bit stream of nbits 32-bit words.  These helpers convert
between that layout and plain integer codes [..., position, channel], e.g. to inspect a cache or to
build one on the host.
"""
from __future__ import annotations

import numpy as np

TILE = 32


def codes_from_tiles(tiles: np.ndarray, nbits: int, n: int) -> np.ndarray:
    """uint32 (or int32) code tiles [..., ntiles, d, nbits] -> int64 codes [..., n, d]."""
    t = np.ascontiguousarray(tiles).view(np.uint32)
    *lead, nt, d, nb = t.shape
    if nb != nbits or n > nt * TILE:
        raise ValueError(f"tiles of shape {t.shape} do not hold {n} positions of {nbits}-bit codes")
    bits = (t[..., None] >> np.arange(32, dtype=np.uint32)) & np.uint32(1)       # [..., nt, d, nbits, 32]
    fields = bits.reshape(*lead, nt, d, TILE, nbits).astype(np.int64)            # stream bit nbits*j + k
    codes = (fields << np.arange(nbits, dtype=np.int64)).sum(axis=-1)              # [..., nt, d, 32]
    codes = np.swapaxes(codes, -1, -2).reshape(*lead, nt * TILE, d)
    return codes[..., :n, :]


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
    per = np.swapaxes(full.reshape(*lead, nt, TILE, d), -1, -2)                    # [..., nt, d, 32]
    bits = (per[..., None] >> np.arange(nbits, dtype=np.int64)) & 1                 # [..., nt, d, 32, nbits]
    stream = bits.reshape(*lead, nt, d, nbits, 32).astype(np.uint64)                 # stream bit 32*w + i
    words = (stream << np.arange(32, dtype=np.uint64)).sum(axis=-1)
    return words.astype(np.uint32)
