"""Pins for the oracle's E4M3 cast (step: saturating RNE cast of fl32(x * s)).

Independent checks, none of which re-uses the oracle's own arithmetic:
* hand-worked edge codes (tests/golden/hand_worked.json, cast_edges);
* every one of the 65536 bf16 patterns, times a set of scales, against a
  nearest-neighbour search on the E4M3 grid enumerated here from the OFP8
  definition (ties to the even code);
* the same inputs against torch's CPU clamp + float8_e4m3fn conversion.
"""
import math

import numpy as np
import pytest

import golden_io


def e4m3_grid():
    """Non-negative finite E4M3 values with their codes, from the OFP8 layout:
    subnormals m * 2^-9 (exponent field 0), normals (1 + m/8) * 2^(e - 7),
    exponent field 15 with mantissa 7 reserved for NaN."""
    vals, codes = [], []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            v = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
            vals.append(v)
            codes.append((e << 3) | m)
    order = np.argsort(vals)
    return np.array(vals)[order], np.array(codes, dtype=np.uint8)[order]


def nearest_even_codes(v):
    """Reference codes for float64 values v by searching the grid."""
    vals, codes = e4m3_grid()
    v = np.asarray(v, dtype=np.float64)
    out = np.empty(v.shape, dtype=np.uint8)
    nan = np.isnan(v)
    sign = np.signbit(v).astype(np.uint8) << 7
    mag = np.minimum(np.abs(np.where(nan, 0.0, v)), 448.0)
    hi = np.searchsorted(vals, mag, side="left")          # vals[hi] >= mag
    hi = np.minimum(hi, len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = vals[hi] == mag
    d_lo = mag - vals[lo]                                  # exact (Sterbenz)
    d_hi = vals[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    idx = np.where(exact | pick_hi, hi, lo)
    out[:] = codes[idx] | sign
    out[nan] = 0x7F | sign[nan]
    return out


def all_bf16_as_f32():
    b = np.arange(65536, dtype=np.uint32)
    return (b << np.uint32(16)).view(np.float32)


SCALES = [
    1.0, float(np.float32(448.0) / np.float32(3.0)), 2.0 ** 48, 2.0 ** -120,
    float(np.float32(3e5)), float(np.float32(448.0) / np.float32(7.5)),
    float(np.float32(448.0) / np.float32(1e-12)), 0.5, 2.0 ** 10, 2.0 ** 20,
    2.0 ** -10, float(np.float32(448.0) / np.float32(0.02)),
]


def test_grid_shape():
    vals, codes = e4m3_grid()
    assert len(vals) == 127 and vals[-1] == 448.0 and codes[-1] == 0x7E
    assert vals[1] == 2.0 ** -9 and codes[1] == 0x01
    assert np.all(np.diff(vals) > 0)


def test_cast_edges_golden(oracle_mod):
    g = golden_io.load()["cast_edges"]
    for value, code in g["cases"]:
        assert oracle_mod.e4m3_encode(golden_io.real(value)) == int(code, 16), value


@pytest.mark.parametrize("scale", SCALES)
def test_cast_all_bf16_times_scale(oracle_mod, scale):
    x = all_bf16_as_f32()
    with np.errstate(over="ignore", invalid="ignore"):
        v = (x * np.float32(scale)).astype(np.float32)      # fl32(x * s)
    got = oracle_mod.e4m3_encode_array(v.astype(np.float64))
    want = nearest_even_codes(v.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(x.view(np.uint32)[i])), float(v[i]), hex(got[i]), hex(want[i]))
                           for i in bad[:8]]


def test_cast_matches_torch_cpu(oracle_mod):
    torch = pytest.importorskip("torch")
    x = all_bf16_as_f32()
    vs = []
    for s in SCALES:
        with np.errstate(over="ignore", invalid="ignore"):
            vs.append((x * np.float32(s)).astype(np.float32))
    v = np.concatenate(vs)
    v = v[np.isfinite(v)]
    ref = torch.from_numpy(v).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle_mod.e4m3_encode_array(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_decode_roundtrip(oracle_mod):
    vals, codes = e4m3_grid()
    for v, c in zip(vals, codes):
        assert oracle_mod.e4m3_decode(int(c)) == v
        assert oracle_mod.e4m3_decode(int(c) | 0x80) == -v
        assert oracle_mod.e4m3_encode(v) == c
    assert math.isnan(oracle_mod.e4m3_decode(0x7F)) and math.isnan(oracle_mod.e4m3_decode(0xFF))
