"""Packed bytes that no encoder writes, for the tests of the decode of every
byte pattern: random tiles with the extremes of each scale type planted in
their first blocks, and E8M0 streams that pair every code pattern with every
scale byte.  Layout only (through tests/brute.py); no arithmetic of the
method."""
import numpy as np

import oracle
from tests import brute

SPECIAL_SCALES = {
    1: np.array([0x7C00, 0xFC00, 0x7E00, 0xFE00, 0x0001, 0x8001, 0x8000, 0x0000, 0x7BFF, 0xFBFF],
                dtype=np.uint16).view(np.uint8),
    2: np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0x00000001, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF,
                 0x00800000], dtype=np.uint32).view(np.uint8),
    3: np.array([0, 1, 126, 127, 128, 239, 240, 246, 247, 252, 253, 254, 255], dtype=np.uint8),
}


def arbitrary_tile(c, seed: int) -> np.ndarray:
    """One tile of random bytes for codec c, its first block scales set to
    the extremes of the scale type: infinite, NaN, subnormal and largest
    FP16/FP32 scales, and for E8M0 the bytes around each format's overflow
    threshold, 2^127 and NaN."""
    fmt, sc, _ = c
    b = np.random.default_rng(seed).integers(0, 256, brute.codec_tile_bytes(c), dtype=np.uint8)
    sp = SPECIAL_SCALES[sc]
    b[brute.CODE_BYTES[fmt]:brute.CODE_BYTES[fmt] + sp.size] = sp
    return b


CODE_BITS = {1: 4, 2: 3, 3: 8, 4: 4, 5: 8}          # INT4, INT3, E4M3, E2M1, E5M2
E8M0_CODECS = [n for n in sorted(oracle.ALL_CODECS) if oracle.ALL_CODECS[n][1] == 3]


def e8m0_every_pair_stream(c, rot: int = 0):
    """Packed tiles of an E8M0 codec in which every code pattern meets every
    scale byte: block B has scale byte B mod 256, and its element e the code
    (block * (B div 256) + e + rot) mod 2^width, so the blocks sharing a
    scale byte run through all codes.  Returns (bytes, element count)."""
    fmt, _, bl = c
    ncode = 1 << CODE_BITS[fmt]
    reps = max(1, ncode // bl)
    per_tile = brute.TILE // bl
    tiles = 256 * reps // per_tile
    out = bytearray()
    for t in range(tiles):
        codes, scales = [], bytearray()
        for b in range(per_tile):
            blk = t * per_tile + b
            scales.append(blk % 256)
            for e in range(bl):
                code = (bl * (blk // 256) + e + rot) % ncode
                codes.append(((code >> 2) << 3) | (code & 3) if fmt == 2 else code)
        out += brute.code_region(fmt, codes) + bytes(scales)
    return np.frombuffer(bytes(out), dtype=np.uint8).copy(), tiles * brute.TILE
