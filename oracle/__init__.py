"""CPU oracle for per-group fp8 scaling and the MX block-32 cast.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package. The HIP
product path never imports, links or calls it, and it shares no code with
that path: the arithmetic lives in ``mgs_oracle.c`` (plain single-threaded
C), and this module only marshals numpy arrays into it.

Every function here is pinned by ``tests/test_oracle_*.py`` against the
worked examples in ``tests/golden/``, an exhaustive nearest-even search over
all bf16 inputs, closed forms checked with exact rational arithmetic, and
invariants (see those tests for which pin covers which step).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mgs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmgs_oracle.so")

FLOOR = 0
RCEIL = 1

_lib = None


def build(force: bool = False) -> str:
    """Compiles the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)
    ):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-std=c11", "-fPIC", "-shared",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            "-o", tmp, _SRC, "-lm",
        ]
        subprocess.run(cmd, check=True, cwd=_HERE)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # MGS_ORACLE_LIB points the test suite at a deliberately broken copy of
    # the oracle (tests/test_oracle_mutants.py), to show its pins catch it.
    path = os.environ.get("MGS_ORACLE_LIB")
    if not path:
        path = build()
    lib = ctypes.CDLL(path)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    i32p = ctypes.POINTER(ctypes.c_int32)
    f32p = ctypes.POINTER(ctypes.c_float)
    i64 = ctypes.c_int64
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode_array.argtypes = [ctypes.POINTER(ctypes.c_double), i64, u8p]
    lib.oracle_e4m3_encode_array.restype = None
    lib.oracle_e4m3_encode_f32_bits.argtypes = [ctypes.c_uint32, i64, u8p]
    lib.oracle_e4m3_encode_f32_bits.restype = None
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_group_scale.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.oracle_group_scale.restype = ctypes.c_float
    lib.oracle_mx_exponent.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.oracle_mx_exponent.restype = ctypes.c_int
    for name in ("oracle_quant_groups_dim0", "oracle_quant_groups_dim1"):
        fn = getattr(lib, name)
        fn.argtypes = [u16p, i64, i64, i32p, ctypes.c_int32, ctypes.c_int, u8p, f32p]
        fn.restype = ctypes.c_int
    lib.oracle_mx_quant_dim0.argtypes = [u16p, i64, i64, ctypes.c_int, u8p, u8p]
    lib.oracle_mx_quant_dim0.restype = ctypes.c_int
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_mx_dequant_dim0.argtypes = [u8p, u8p, i64, i64, u16p]
    lib.oracle_mx_dequant_dim0.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _bf16_bits(x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns, got %s" % a.dtype)
    return a


def e4m3_encode(v: float) -> int:
    """Saturating RNE E4M3 code of the exact real value ``v``."""
    return int(_load().oracle_e4m3_encode(float(v)))


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    """Vector form of :func:`e4m3_encode`."""
    flat = np.ascontiguousarray(np.asarray(v, dtype=np.float64).ravel())
    out = np.empty(flat.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(flat, ctypes.c_double), flat.size,
                                     _ptr(out, ctypes.c_uint8))
    return out.reshape(np.shape(v))


def e4m3_encode_f32_bits(first: int, n: int) -> np.ndarray:
    """Codes of the binary32 values with bit patterns first .. first+n-1.
    The C call releases the GIL, so threads can split a large range."""
    out = np.empty(int(n), dtype=np.uint8)
    _load().oracle_e4m3_encode_f32_bits(int(first) & 0xFFFFFFFF, int(n), _ptr(out, ctypes.c_uint8))
    return out


def e4m3_decode(code: int) -> float:
    return float(_load().oracle_e4m3_decode(int(code) & 0xFF))


def e4m3_decode_table() -> np.ndarray:
    """Real value of each of the 256 E4M3 codes (NaN for the two NaN codes)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def group_scale(amax: float, pow2: bool = False) -> float:
    return float(_load().oracle_group_scale(float(amax), int(bool(pow2))))


def mx_exponent(amax: float, mode: int) -> int:
    return int(_load().oracle_mx_exponent(float(amax), int(mode)))


def quant_groups_dim0(x_bits: np.ndarray, offsets: np.ndarray, pow2: bool = False):
    """x (M, K) bf16 bits, int32 end offsets along M -> (q (M, K) u8, scales (G, K) f32)."""
    x = _bf16_bits(x_bits)
    M, K = x.shape
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    G = off.shape[0]
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((G, K), dtype=np.float32)
    rc = _load().oracle_quant_groups_dim0(
        _ptr(x, ctypes.c_uint16), M, K, _ptr(off, ctypes.c_int32), G,
        int(bool(pow2)), _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle dim0: offsets must be a non-decreasing cover of [0, M]")
    return q, s


def quant_groups_dim0_t(x_bits: np.ndarray, offsets: np.ndarray, pow2: bool = False):
    """dim0 with transposed outputs: x (M, K) bf16 bits, int32 end offsets
    along M -> (q_t (K, M) u8, scales_t (K, G) f32), the transposes of
    quant_groups_dim0's results ("test and bench new faster method for per
    group rowwise scaling", Summary: colwise per-group scales of one layout,
    transposed, are the rowwise per-group scales of its transpose). The
    values are dim0's; only the layout changes."""
    q, s = quant_groups_dim0(x_bits, offsets, pow2)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def quant_experts_dim1(w_bits: np.ndarray, pow2: bool = False):
    """w (E, D1, D2) bf16 bits -> (q (E, D1, D2) u8, scales (E, D2) f32): one
    scale per (expert, column) from the amax over the expert's D1 rows (the
    fused dim1 reduction for 3D expert weights named in the stacked changes
    of "[moe fp8 training] test and bench new faster method for per group
    rowwise scaling"). By definition this is per-group scaling along dim0 of
    the (E * D1, D2) view with E equal groups of D1 rows."""
    E, D1, D2 = w_bits.shape
    off = (np.arange(1, E + 1, dtype=np.int64) * D1).astype(np.int32)
    q, s = quant_groups_dim0(np.ascontiguousarray(w_bits).reshape(E * D1, D2), off, pow2)
    return q.reshape(E, D1, D2), s


def quant_groups_dim1(x_bits: np.ndarray, offsets: np.ndarray, pow2: bool = False):
    """x (M, K) bf16 bits, int32 end offsets along K -> (q (M, K) u8, scales (M, G) f32)."""
    x = _bf16_bits(x_bits)
    M, K = x.shape
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    G = off.shape[0]
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, G), dtype=np.float32)
    rc = _load().oracle_quant_groups_dim1(
        _ptr(x, ctypes.c_uint16), M, K, _ptr(off, ctypes.c_int32), G,
        int(bool(pow2)), _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float))
    if rc != 0:
        raise ValueError("oracle dim1: offsets must be a non-decreasing cover of [0, K]")
    return q, s


def mx_quant_dim0(x_bits: np.ndarray, mode: int):
    """x (M, K) bf16 bits, K % 32 == 0 -> (q (M, K) u8, scales (M, K/32) u8 E8M0)."""
    x = _bf16_bits(x_bits)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 32 if K % 32 == 0 else 0), dtype=np.uint8)
    rc = _load().oracle_mx_quant_dim0(
        _ptr(x, ctypes.c_uint16), M, K, int(mode), _ptr(q, ctypes.c_uint8),
        _ptr(s, ctypes.c_uint8))
    if rc != 0:
        raise ValueError("oracle mx: K must be a multiple of 32 and mode 0 or 1")
    return q, s


def f64_to_bf16(v: float) -> int:
    """bf16 bits of v rounded once, to nearest even (overflow to infinity;
    NaN gives 0x7FC0)."""
    return int(_load().oracle_f64_to_bf16(float(v)))


def mx_dequant_dim0(q: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """q (M, K) E4M3 bytes, scales (M, K/32) E8M0 bytes -> y (M, K) bf16 bits,
    y = bf16(E4M3(q) * 2^(byte - 127)) ("[mxfp8 moe training] fix mxfp8 a2a
    bench script; ...", Summary: the dequantise step of the mxfp8 all-to-all
    pipeline; E8M0 per the OCP MX spec). Byte 0xFF or an E4M3 NaN code gives
    the quiet NaN 0x7FC0."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    M, K = q.shape
    if K % 32 != 0 or s.shape != (M, K // 32):
        raise ValueError("oracle mx dequant: K % 32 == 0 and scales (M, K/32) required")
    y = np.empty((M, K), dtype=np.uint16)
    rc = _load().oracle_mx_dequant_dim0(_ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_uint8), M, K,
                                        _ptr(y, ctypes.c_uint16))
    if rc != 0:
        raise ValueError("oracle mx dequant: bad shape")
    return y


def mx_quant_dim1(x_bits: np.ndarray, mode: int):
    """x (M, K) bf16 bits, M % 32 == 0 -> (q_t (K, M) u8, scales_t (K, M/32)
    u8 E8M0): blocks of 32 consecutive rows of one column, the outputs in
    the transposed layout -- by definition mx_quant_dim0 of x^T ("[mxfp8 moe
    training] fix mxfp8 a2a bench script; ...", investigation comment: the
    cast benchmark's modes)."""
    return mx_quant_dim0(np.ascontiguousarray(np.asarray(x_bits).T), mode)
