"""Pins of the oracle's MX dequantisation (the receiving side of the
quantise -> all-to-all -> dequantise pipeline of "[mxfp8 moe training] fix
mxfp8 a2a bench script; set mxfp8 a2a scaling type to RCEIL", Summary):

* every (E4M3 code, E8M0 byte) pair against torch on the CPU as a library
  routine: float8_e4m3fn decoding, an exact binary64 product with
  2^(byte - 127), and torch's bf16 rounding (the product is exact in binary32,
  so torch's rounding through binary32 rounds once);
* E8M0 byte 0xFF and E4M3 NaN codes give the quiet NaN 0x7FC0;
* blocks made of E4M3 values times 2^e come back exactly after the oracle's
  own MX quantisation (FLOOR), a round trip with no rounding on either side.
"""
import numpy as np
import pytest
import torch

import oracle


@pytest.fixture(scope="module")
def every_pair():
    # row s holds the 256 codes (8 blocks of 32) with all 8 scale bytes = s
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    return q, s, oracle.mx_dequant_dim0(q, s)


def test_every_code_and_scale_against_torch(every_pair):
    q, s, y = every_pair
    dec = torch.from_numpy(np.arange(256, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64)
    for byte in range(255):
        want = (dec * (2.0 ** (byte - 127))).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        got = y[byte]
        finite = ~np.isnan(dec.numpy())
        assert np.array_equal(got[finite], want[finite]), byte
        assert np.all(got[~finite] == 0x7FC0)


def test_nan_scale_byte(every_pair):
    _, _, y = every_pair
    assert np.all(y[255] == 0x7FC0)


def test_signed_zero_and_extremes():
    q = np.zeros((1, 32), np.uint8)
    q[0, :4] = [0x00, 0x80, 0x7E, 0xFE]        # +0, -0, 448, -448
    s = np.array([[127]], np.uint8)              # 2^0
    y = oracle.mx_dequant_dim0(q, s)
    assert list(y[0, :4]) == [0x0000, 0x8000, 0x43E0, 0xC3E0]
    s = np.array([[254]], np.uint8)              # 2^127: 448 * 2^127 overflows bf16
    assert list(oracle.mx_dequant_dim0(q, s)[0, :4]) == [0x0000, 0x8000, 0x7F80, 0xFF80]
    s = np.array([[0]], np.uint8)                # 2^-127
    q[0, 0] = 0x01                               # 2^-9 * 2^-127 = 2^-136 -> 0
    q[0, 1] = 0x08                               # 2^-6 * 2^-127 = 2^-133, the least bf16
    y = oracle.mx_dequant_dim0(q, s)
    assert list(y[0, :2]) == [0x0000, 0x0001]


def test_round_trip_of_representable_blocks():
    rng = np.random.default_rng(17)
    M, K = 64, 256
    codes = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x7E               # no NaN codes
    codes[:, ::32] = 0x7E                              # every block holds 448 ...
    codes[:, 1::32] = 0x70                             # ... and 256, so FLOOR gives e = E(448) - 8
    e = rng.integers(-100, 100, size=(M, K // 32))
    dec = oracle.e4m3_decode_table()[codes]
    x = dec * np.repeat(2.0 ** e, 32, axis=1)
    xb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    q, s = oracle.mx_quant_dim0(xb, oracle.FLOOR)
    assert np.array_equal(s.astype(np.int64) - 127, e)
    assert np.array_equal(q, codes)
    assert np.array_equal(oracle.mx_dequant_dim0(q, s), xb)


def test_shape_checks():
    with pytest.raises(ValueError):
        oracle.mx_dequant_dim0(np.zeros((2, 48), np.uint8), np.zeros((2, 1), np.uint8))


@pytest.mark.parametrize("mode", [oracle.FLOOR, oracle.RCEIL])
def test_mx_dim1_by_brute_force(mode):
    """mx_quant_dim1 against a direct per-(column, 32-row block) computation:
    the block amax by numpy, the exponent from the pinned mx_exponent, and
    each element through the pinned E4M3 encoder at an exact power of two."""
    from group_scaling_fp8_amd import workloads as wl
    rng = np.random.default_rng(53 + mode)
    x = wl.randn_bf16(rng, (64, 24), 1.0, 0.01, 100.0)
    q, s = oracle.mx_quant_dim1(x, mode)
    assert q.shape == (24, 64) and s.shape == (24, 2)
    xf = wl.bf16_bits_to_f32(x)
    for k in range(24):
        for b in range(2):
            blk = xf[32 * b:32 * b + 32, k]
            e = oracle.mx_exponent(float(np.max(np.abs(blk))), mode)
            assert s[k, b] == e + 127
            for i in range(32):
                assert q[k, 32 * b + i] == oracle.e4m3_encode(float(blk[i]) * 2.0 ** (-e))
