"""Test-side block encoders, written independently of the oracle's decoders.

They build q4_K / q6_K blocks from chosen field values by placing bits where the block
formats put them, so a test can construct weights with a known dequantised value and
check that the oracle (and the kernels) read them back. The scale packing is written as
a table of bit destinations rather than as the decode formula.
"""
import numpy as np


def f16_bits(v: float) -> int:
    return int(np.array(v, np.float16).view(np.uint16))


# q4_K: where each bit of the eight 6-bit scales and mins lives in the 12 bytes at +4.
# Entry (field, s, bit) -> (byte, bit). Sub-blocks 0..3 keep all six bits in one byte
# (scales in bytes 0..3, mins in bytes 4..7). Sub-blocks 4..7 keep their low four bits
# in bytes 8..11 (scale in the low nibble, min in the high nibble) and their top two
# bits in the top two bits of bytes 0..3 (scale) and 4..7 (min) of sub-block s-4.
def _q4k_scale_bit_map():
    mp = {}
    for s in range(8):
        for bit in range(6):
            if s < 4:
                mp[("sc", s, bit)] = (s, bit)
                mp[("m", s, bit)] = (s + 4, bit)
            else:
                if bit < 4:
                    mp[("sc", s, bit)] = (s + 4, bit)
                    mp[("m", s, bit)] = (s + 4, bit + 4)
                else:
                    mp[("sc", s, bit)] = (s - 4, bit + 2)
                    mp[("m", s, bit)] = (s, bit + 2)
    assert len(set(mp.values())) == 96      # every bit of the 12 bytes used exactly once
    return mp


_Q4K_MAP = _q4k_scale_bit_map()


def encode_q4K(d: float, dmin: float, sc, m, nib) -> np.ndarray:
    """One 144-byte block. sc, m: 8 ints in 0..63; nib: 256 ints in 0..15 (element order)."""
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([f16_bits(d)], np.uint16).view(np.uint8)
    blk[2:4] = np.array([f16_bits(dmin)], np.uint16).view(np.uint8)
    packed = [0] * 12
    for (field, s, bit), (byte, dst) in _Q4K_MAP.items():
        val = (sc if field == "sc" else m)[s]
        if (val >> bit) & 1:
            packed[byte] |= 1 << dst
    blk[4:16] = packed
    # element e = 32*s + l of sub-block s sits in byte 32*(s>>1) + l of qs,
    # low nibble for even s, high nibble for odd s.
    qs = [0] * 128
    for e in range(256):
        s, l = divmod(e, 32)
        byte = 32 * (s >> 1) + l
        qs[byte] |= (int(nib[e]) & 15) << (4 * (s & 1))
    blk[16:144] = qs
    return blk


def encode_q6K(d: float, sc, v) -> np.ndarray:
    """One 210-byte block. sc: 16 ints in -128..127; v: 256 ints in -32..31 (element order)."""
    blk = np.zeros(210, np.uint8)
    ql = [0] * 128
    qh = [0] * 64
    for e in range(256):
        u = int(v[e]) + 32                  # stored 6-bit value
        half, r = divmod(e, 128)
        quarter, l = divmod(r, 32)
        # low nibble: quarters 0/1 in the low half of ql bytes 0..31 / 32..63 of the
        # half, quarters 2/3 in the high half of the same bytes
        ql[64 * half + 32 * (quarter % 2) + l] |= (u & 15) << (4 * (quarter // 2))
        # high two bits: qh byte l of the half, bit pair number = quarter
        qh[32 * half + l] |= ((u >> 4) & 3) << (2 * quarter)
    blk[0:128] = ql
    blk[128:192] = qh
    blk[192:208] = np.array(sc, np.int64).astype(np.int8).view(np.uint8)
    blk[208:210] = np.array([f16_bits(d)], np.uint16).view(np.uint8)
    return blk


def tolerance_ok(g: np.ndarray, r: np.ndarray, rel=1e-4, abs_unit=1e-3):
    """|g - r| <= rel*|r| + abs_unit*s with s = RMS(r): the output bar of the method.
    Returns (ok, worst ratio err/bound, max relative error over |r| >= s)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    s = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    bound = rel * np.abs(r) + abs_unit * s
    ratio = float(np.max(err / np.maximum(bound, 1e-300))) if r.size else 0.0
    big = np.abs(r) >= s
    relmax = float(np.max(err[big] / np.abs(r[big]))) if np.any(big) else 0.0
    return ratio <= 1.0, ratio, relmax


def near_tie_blocks(amax: float) -> np.ndarray:
    """32-value blocks whose first value is amax = 127 * 2^-t (so d = 2^-t and 1/d = 2^t are
    exact and x * (1/d) is exact too) and whose other 31 values put x * (1/d) at n + 1/2 and
    up to three f32 steps either side of it, for n = 0..126 and both signs: every rounding
    decision of the int8 conversion next to a tie."""
    s = amax / 127.0
    v = []
    for n in range(127):
        t = np.float32(n + 0.5)
        for k in range(-3, 4):
            c = t
            for _ in range(abs(k)):
                c = np.nextafter(c, np.float32(np.inf if k > 0 else -np.inf), dtype=np.float32)
            if c <= 127.0:
                v += [c, -c]
    v = np.array(v, np.float32) * np.float32(s)
    v = np.concatenate([v, np.zeros((-len(v)) % 31, np.float32)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((len(v), 1), amax, np.float32), v], axis=1)
    blocks = np.concatenate([blocks, np.zeros(((-len(blocks)) % 8, 32), np.float32)])
    return blocks.reshape(-1, 256)
