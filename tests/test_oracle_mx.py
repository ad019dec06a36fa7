"""Pins for the oracle's MX block-32 cast (amax, E8M0 exponent, cast).

* Hand-worked blocks (tests/golden/hand_worked.json, mx_blocks) covering
  both scaling types, saturation, zero and subnormal blocks.
* The exponent rule against exact integer arithmetic for every
  non-negative finite bf16 amax: FLOOR is floor(log2 amax) - 8, RCEIL is
  the smallest e with amax <= 448 * 2^e, both clamped to [-127, 127].
* Invariants on seeded blocks: RCEIL never saturates and puts the block
  maximum above 224; FLOOR puts it in [256, 448] (saturating); every code
  is within half an E4M3 step of x * 2^-e.
"""
from fractions import Fraction

import numpy as np
import pytest

import golden_io
from group_scaling_fp8_amd import workloads as wl
from test_oracle_groups import DEC, half_step


def exact_log2_floor(fr):
    """Largest integer E with 2^E <= fr, for a positive dyadic rational."""
    n, d = fr.numerator, fr.denominator
    E = n.bit_length() - d.bit_length()
    while Fraction(2) ** E > fr:
        E -= 1
    while Fraction(2) ** (E + 1) <= fr:
        E += 1
    return E


def exact_rceil(fr):
    e = exact_log2_floor(fr) - 10
    while fr > 448 * Fraction(2) ** e:
        e += 1
    return e


@pytest.mark.parametrize("mode", ["FLOOR", "RCEIL"])
def test_mx_golden(oracle_mod, mode):
    g = golden_io.load()["mx_blocks"]
    x = golden_io.sparse_bits(g["x_sparse"])
    q, s = oracle_mod.mx_quant_dim0(x, 0 if mode == "FLOOR" else 1)
    assert [hex(v) for v in s[0]] == [hex(int(v, 16)) for v in g[mode]["scales"]]
    assert np.array_equal(q, golden_io.sparse_q(x.shape, g[mode]["q_sparse"], g["q_default"]))


def test_mx_exponent_all_bf16(oracle_mod):
    for b in range(0, 0x7F80):
        a = float(np.array([b << 16], np.uint32).view(np.float32)[0])
        ef = oracle_mod.mx_exponent(a, 0)
        er = oracle_mod.mx_exponent(a, 1)
        if a == 0.0:
            assert ef == er == -127
            continue
        fr = Fraction(a)
        want_f = max(-127, min(127, exact_log2_floor(fr) - 8))
        want_r = max(-127, min(127, exact_rceil(fr)))
        assert ef == want_f, hex(b)
        assert er == want_r, hex(b)
        assert er in (ef, ef + 1)


@pytest.mark.parametrize("mode", [0, 1])
def test_mx_invariants(oracle_mod, mode):
    rng = np.random.default_rng(51 + mode)
    x = wl.randn_bf16(rng, (24, 512), 1.0, 0.01, 100.0)
    # a few blocks spanning extreme magnitudes and a zero block
    x[0, :32] = 0
    x[1, :32] = wl.f32_to_bf16_bits(rng.standard_normal(32).astype(np.float32) * np.float32(1e-38))
    x[2, :32] = wl.f32_to_bf16_bits(rng.standard_normal(32).astype(np.float32) * np.float32(1e30))
    q, s = oracle_mod.mx_quant_dim0(x, mode)
    xf = wl.bf16_bits_to_f32(x).astype(np.float64).reshape(24, 16, 32)
    e = s.astype(np.int64) - 127
    v = xf * np.exp2(-e)[..., None]
    d = DEC[q].reshape(24, 16, 32)
    vc = np.clip(v, -448, 448)
    assert np.all(np.abs(d - vc) <= half_step(vc))
    amax = np.abs(xf).max(-1)
    top = np.abs(d).max(-1)
    live = amax * np.exp2(-e) >= 2.0 ** -6
    if mode == 1:
        assert np.all(np.abs(v) <= 448.0)
        assert np.all(top[live & (e > -127)] > 224.0 - 16.0)
    else:
        assert np.all(top[live & (e > -127)] >= 256.0)
    assert np.all(s[0, 0] == 0)
