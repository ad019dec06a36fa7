"""The CPU oracle on whole full-size tensors, in slices on a thread pool.

Test infrastructure. The oracle itself stays plain and single-threaded; this
module only cuts the input into slices whose results are independent by the
definition of each operation, calls the oracle on each slice from a pool of
threads (ctypes releases the GIL during the C call), and compares every
slice's bytes with the same slice of the GPU result:
  * per-group dim0 and its transposed form: each column's outputs depend on
    that column only (slices of columns);
  * per-group dim1, the MX cast and the MX dequantisation: each row's outputs
    depend on that row only (slices of rows);
  * the MX cast along dim0 (transposed outputs): each column of x is one row
    of x^T (slices of columns).
"""
from __future__ import annotations

import concurrent.futures as cf
import os

import numpy as np

import oracle
from gpu_util import assert_same_bytes

WORKERS = max(1, min(16, os.cpu_count() or 1))


def _slices(n, parts, align):
    """[lo, hi) ranges covering 0..n, every boundary a multiple of align."""
    step = max(align, -(-n // parts) // align * align)
    return [(lo, min(n, lo + step)) for lo in range(0, n, step)]


def _run(fn, ranges):
    with cf.ThreadPoolExecutor(WORKERS) as pool:
        for _ in pool.map(fn, ranges):
            pass


def check_dim0_whole(x, off, pow2, q, s, what):
    """q (M, K), s (G, K) from the GPU against the oracle on column slices."""
    K = x.shape[1]

    def one(r):
        lo, hi = r
        rq, rs = oracle.quant_groups_dim0(np.ascontiguousarray(x[:, lo:hi]), off, pow2)
        assert_same_bytes(s[:, lo:hi], rs, "%s scales, columns %d..%d" % (what, lo, hi))
        assert_same_bytes(q[:, lo:hi], rq, "%s q, columns %d..%d" % (what, lo, hi))

    _run(one, _slices(K, 4 * WORKERS, 8))


def check_dim0_t_whole(x, off, pow2, q_t, s_t, what):
    """q_t (K, M), s_t (K, G): the oracle's dim0_t on column slices of x."""
    K = x.shape[1]

    def one(r):
        lo, hi = r
        rq, rs = oracle.quant_groups_dim0_t(np.ascontiguousarray(x[:, lo:hi]), off, pow2)
        assert_same_bytes(s_t[lo:hi], rs, "%s scales_t, rows %d..%d" % (what, lo, hi))
        assert_same_bytes(q_t[lo:hi], rq, "%s q_t, rows %d..%d" % (what, lo, hi))

    _run(one, _slices(K, 4 * WORKERS, 8))


def check_experts_whole(w, pow2, q, s, what):
    """q (E, D1, D2), s (E, D2) against the oracle's per-expert scaling on
    slices of the D2 columns."""
    D2 = w.shape[2]

    def one(r):
        lo, hi = r
        rq, rs = oracle.quant_experts_dim1(np.ascontiguousarray(w[:, :, lo:hi]), pow2)
        assert_same_bytes(s[:, lo:hi], rs, "%s scales, columns %d..%d" % (what, lo, hi))
        assert_same_bytes(q[:, :, lo:hi], rq, "%s q, columns %d..%d" % (what, lo, hi))

    _run(one, _slices(D2, 4 * WORKERS, 8))


def check_dim1_whole(x, off, pow2, q, s, what):
    """q (M, K), s (M, G) from the GPU against the oracle on row slices."""
    M = x.shape[0]

    def one(r):
        lo, hi = r
        rq, rs = oracle.quant_groups_dim1(x[lo:hi], off, pow2)
        assert_same_bytes(s[lo:hi], rs, "%s scales, rows %d..%d" % (what, lo, hi))
        assert_same_bytes(q[lo:hi], rq, "%s q, rows %d..%d" % (what, lo, hi))

    _run(one, _slices(M, 4 * WORKERS, 1))


def check_mx_whole(x, mode, q, s, what):
    """q (M, K) and E8M0 scales (M, K/32) against the oracle on row slices."""
    M = x.shape[0]

    def one(r):
        lo, hi = r
        rq, rs = oracle.mx_quant_dim0(x[lo:hi], mode)
        assert_same_bytes(s[lo:hi], rs, "%s scales, rows %d..%d" % (what, lo, hi))
        assert_same_bytes(q[lo:hi], rq, "%s q, rows %d..%d" % (what, lo, hi))

    _run(one, _slices(M, 4 * WORKERS, 1))


def check_mx_dim1_whole(x, mode, q_t, s_t, what):
    """q_t (K, M) and scales_t (K, M/32): the oracle's MX cast of x^T, one
    slice of x's columns (rows of x^T) at a time."""
    K = x.shape[1]

    def one(r):
        lo, hi = r
        rq, rs = oracle.mx_quant_dim1(np.ascontiguousarray(x[:, lo:hi]), mode)
        assert_same_bytes(s_t[lo:hi], rs, "%s scales_t, rows %d..%d" % (what, lo, hi))
        assert_same_bytes(q_t[lo:hi], rq, "%s q_t, rows %d..%d" % (what, lo, hi))

    _run(one, _slices(K, 4 * WORKERS, 8))


def check_mx_dequant_whole(q, scales, y, what):
    """y (M, K) bf16 bits against the oracle's dequantisation on row slices."""
    M = q.shape[0]

    def one(r):
        lo, hi = r
        ry = oracle.mx_dequant_dim0(q[lo:hi], scales[lo:hi])
        assert_same_bytes(y[lo:hi], ry, "%s y, rows %d..%d" % (what, lo, hi))

    _run(one, _slices(M, 4 * WORKERS, 1))
