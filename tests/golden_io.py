"""Reads the hand-worked fixtures in tests/golden/."""
import json
import math
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name="hand_worked.json"):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def real(s):
    """Decimal, C99 hex-float, 'nan' / '-nan' / 'inf' strings -> float."""
    s = s.strip()
    if s in ("nan", "-nan"):
        return math.copysign(math.nan, -1.0 if s.startswith("-") else 1.0)
    if "0x" in s and "p" in s:
        return float.fromhex(s)
    return float(s)


def bf16_bits(s):
    """An exact bf16 value ('3.0', '0x1p-8') or a raw pattern ('0x0001')."""
    s = s.strip()
    if s.startswith("0x") and "p" not in s and len(s) == 6:
        return int(s, 16)
    v = real(s)
    w = struct.unpack("<I", struct.pack("<f", v))[0]
    if w & 0xFFFF:
        raise ValueError("%s is not exactly representable in bf16" % s)
    return w >> 16


def f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def dense_bits(rows):
    return np.array([[bf16_bits(str(v)) for v in r] for r in rows], dtype=np.uint16)


def sparse_bits(spec):
    x = np.zeros(spec["shape"], dtype=np.uint16)
    for r, c, v in spec["entries"]:
        x[r, c] = bf16_bits(v)
    return x


def sparse_q(shape, entries, default):
    q = np.full(shape, int(default, 16), dtype=np.uint8)
    for r, c, v in entries:
        q[r, c] = int(v, 16)
    return q


def hex_matrix_u32(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.uint32)


def hex_matrix_u8(rows):
    return np.array([[int(v, 16) for v in r] for r in rows], dtype=np.uint8)
