"""Test-side encoder: integer codes -> exchange-format block bytes.

Written from the block layout independently of the oracle's decoder, so a
round trip (encode here, decode in the oracle) checks the decoder against the
layout, and hand-built special blocks (unit scales, zero mins) can be made.
Layouts (little-endian):
  Q4_K 144 B: f16 d, f16 dmin, 12 B bit stream (eight 6-bit scales, then eight
              6-bit mins), 128 B quants: byte 32g+i = element 64g+i | element 64g+32+i << 4
  Q2_K  84 B: f16 d, f16 dmin, 16 B (sc | m << 4), 64 B quants:
              byte 32h+i bits 2s..2s+1 = element 128h+32s+i
  Q6_K 210 B: f16 d, 16 x int8 scales, 128 B low nibbles
              (byte 64h+i = lo(128h+i) | lo(128h+64+i) << 4), 64 B high pairs
              (byte 32h+i bits 2s..2s+1 = hi(128h+32s+i))
  Q8_0  34 B: f16 d, 32 x int8
  Q3_K 110 B: f16 d, 12 B bit stream (sixteen 6-bit values sc + 32), 64 B low
              pairs (byte 32h+i bits 2s..2s+1 = low2(128h+32s+i)), 32 B high
              bits (byte i bit b = bit 2 of element 32b+i); w = d*sc*(q-4)
  Q5_K 176 B: the Q4_K bytes of the low nibbles, then 32 B high bits (byte i
              bit b = bit 4 of element 32b+i)
  Q4_0  18 B: f16 d, 16 B (byte i = element i | element 16+i << 4); w = d*(q-8)
  Q5_1  24 B: f16 d, f16 m, 4 B (bit i = bit 4 of element i), 16 B as Q4_0;
              w = d*q + m
"""
import numpy as np

Q4_K, Q6_K, Q2_K, Q8_0, Q3_K, Q5_K, Q4_0, Q5_1 = 1, 2, 3, 4, 5, 6, 7, 8


def f16_bytes(v: float) -> bytes:
    return np.array([v], dtype=np.float16).tobytes()


def pack_q4k(d, dmin, sc, m, q) -> bytes:
    assert len(sc) == 8 and len(m) == 8 and len(q) == 256
    bits = 0
    for j in range(8):
        bits |= (int(sc[j]) & 63) << (6 * j)
        bits |= (int(m[j]) & 63) << (48 + 6 * j)
    sm = bits.to_bytes(12, "little")
    qs = bytearray(128)
    for g in range(4):
        for i in range(32):
            qs[32 * g + i] = (int(q[64 * g + i]) & 15) | ((int(q[64 * g + 32 + i]) & 15) << 4)
    return f16_bytes(d) + f16_bytes(dmin) + sm + bytes(qs)


def pack_q2k(d, dmin, sc, m, q) -> bytes:
    assert len(sc) == 16 and len(m) == 16 and len(q) == 256
    sm = bytes(((int(sc[j]) & 15) | ((int(m[j]) & 15) << 4)) for j in range(16))
    qs = bytearray(64)
    for h in range(2):
        for s in range(4):
            for i in range(32):
                qs[32 * h + i] |= (int(q[128 * h + 32 * s + i]) & 3) << (2 * s)
    return f16_bytes(d) + f16_bytes(dmin) + sm + bytes(qs)


def pack_q6k(d, sc, q) -> bytes:
    assert len(sc) == 16 and len(q) == 256
    scb = np.array(sc, dtype=np.int8).tobytes()
    ql = bytearray(128)
    qh = bytearray(64)
    for h in range(2):
        for i in range(64):
            ql[64 * h + i] = (int(q[128 * h + i]) & 15) | ((int(q[128 * h + 64 + i]) & 15) << 4)
        for s in range(4):
            for i in range(32):
                qh[32 * h + i] |= ((int(q[128 * h + 32 * s + i]) >> 4) & 3) << (2 * s)
    return f16_bytes(d) + scb + bytes(ql) + bytes(qh)


def pack_q80(d, q) -> bytes:
    assert len(q) == 32
    return f16_bytes(d) + np.array(q, dtype=np.int8).tobytes()


def _high_bits(q, bit) -> bytes:
    qh = bytearray(32)
    for e in range(256):
        qh[e % 32] |= ((int(q[e]) >> bit) & 1) << (e // 32)
    return bytes(qh)


def pack_q3k(d, sc, q) -> bytes:
    """sc: sixteen signed scales in [-32, 31]; q: 256 codes in [0, 7]."""
    assert len(sc) == 16 and len(q) == 256
    bits = 0
    for j in range(16):
        assert -32 <= int(sc[j]) <= 31
        bits |= (int(sc[j]) + 32) << (6 * j)
    ql = bytearray(64)
    for h in range(2):
        for s in range(4):
            for i in range(32):
                ql[32 * h + i] |= (int(q[128 * h + 32 * s + i]) & 3) << (2 * s)
    return f16_bytes(d) + bits.to_bytes(12, "little") + bytes(ql) + _high_bits(q, 2)


def pack_q5k(d, dmin, sc, m, q) -> bytes:
    """q: 256 codes in [0, 31]; the rest as Q4_K."""
    assert all(0 <= int(v) < 32 for v in q)
    return pack_q4k(d, dmin, sc, m, [int(v) & 15 for v in q]) + _high_bits(q, 4)


def _nibbles32(q) -> bytes:
    return bytes((int(q[i]) & 15) | ((int(q[16 + i]) & 15) << 4) for i in range(16))


def pack_q40(d, q) -> bytes:
    """q: 32 codes in [0, 15]."""
    assert len(q) == 32 and all(0 <= int(v) < 16 for v in q)
    return f16_bytes(d) + _nibbles32(q)


def pack_q51(d, m, q) -> bytes:
    """q: 32 codes in [0, 31]; m: the block's min (added)."""
    assert len(q) == 32 and all(0 <= int(v) < 32 for v in q)
    qh = sum(((int(q[i]) >> 4) & 1) << i for i in range(32)).to_bytes(4, "little")
    return f16_bytes(d) + f16_bytes(m) + qh + _nibbles32(q)


def pack_row(fmt, blocks) -> np.ndarray:
    """blocks: list of per-block argument tuples for the format's packer."""
    fn = {Q4_K: pack_q4k, Q2_K: pack_q2k, Q6_K: pack_q6k, Q8_0: pack_q80, Q3_K: pack_q3k, Q5_K: pack_q5k,
          Q4_0: pack_q40, Q5_1: pack_q51}[fmt]
    return np.frombuffer(b"".join(fn(*b) for b in blocks), dtype=np.uint8).copy()
