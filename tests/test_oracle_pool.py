"""CPU check of the slicing used by the whole-tensor GPU parity tests: the
slices cover every column or row exactly once, and a single changed byte
or scale bit anywhere is caught."""
import numpy as np
import pytest

import oracle
from group_scaling_fp8_amd import workloads as wl
import oracle_pool as op


def test_slices_cover_everything_once():
    for n, parts, align in ((4096, 64, 8), (8, 64, 8), (131072, 64, 1), (13, 5, 1), (1000, 7, 8)):
        r = op._slices(n, parts, align)
        assert r[0][0] == 0 and r[-1][1] == n
        assert all(a[1] == b[0] for a, b in zip(r, r[1:]))
        assert all(lo % align == 0 for lo, _ in r)


@pytest.mark.parametrize("which", ["dim0", "dim0_t", "dim1", "mx", "mx_dim1"])
def test_one_flipped_byte_is_caught(which):
    rng = np.random.default_rng(3)
    x = wl.randn_bf16(rng, (96, 264), 0.02, 0.01, 8.0)
    off = np.array([0, 40, 96], np.int32)
    off1 = np.array([16, 16, 264], np.int32)
    if which == "dim0":
        q, s = oracle.quant_groups_dim0(x, off)
        run = lambda q, s: op.check_dim0_whole(x, off, False, q, s, which)
    elif which == "dim0_t":
        q, s = oracle.quant_groups_dim0_t(x, off)
        run = lambda q, s: op.check_dim0_t_whole(x, off, False, q, s, which)
    elif which == "dim1":
        q, s = oracle.quant_groups_dim1(x, off1)
        run = lambda q, s: op.check_dim1_whole(x, off1, False, q, s, which)
    elif which == "mx":
        xm = np.ascontiguousarray(x[:, :256])            # K % 32 == 0
        q, s = oracle.mx_quant_dim0(xm, 1)
        run = lambda q, s: op.check_mx_whole(xm, 1, q, s, which)
    else:
        q, s = oracle.mx_quant_dim1(x, 0)
        run = lambda q, s: op.check_mx_dim1_whole(x, 0, q, s, which)
    run(q, s)                      # identical: passes
    for arr, is_q in ((q, True), (s, False)):
        bad = arr.copy()
        flat = bad.reshape(-1)
        i = int(rng.integers(0, flat.size))
        if flat.dtype == np.float32:
            flat.view(np.uint32)[i] ^= 1
        else:
            flat[i] ^= 1
        with pytest.raises(AssertionError):
            run(bad, s) if is_q else run(q, bad)


def test_dequant_and_experts_catch_a_flip():
    rng = np.random.default_rng(4)
    qq = rng.integers(0, 256, (40, 96), dtype=np.uint8)
    ss = rng.integers(100, 140, (40, 3), dtype=np.uint8)
    y = oracle.mx_dequant_dim0(qq, ss)
    op.check_mx_dequant_whole(qq, ss, y, "dequant")
    y2 = y.copy()
    y2[17, 50] ^= 1
    with pytest.raises(AssertionError):
        op.check_mx_dequant_whole(qq, ss, y2, "dequant")
    w = wl.randn_bf16(rng, (3, 20, 136), 0.02).reshape(3, 20, 136)
    q, s = oracle.quant_experts_dim1(w)
    op.check_experts_whole(w, False, q, s, "experts")
    q2 = q.copy()
    q2[2, 19, 135] ^= 1
    with pytest.raises(AssertionError):
        op.check_experts_whole(w, False, q2, s, "experts")
