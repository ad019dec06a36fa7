"""The C ABI from a plain C program (tests/c_consumer/mgs_c_consumer.c,
built with gcc against include/mgs.h and linked to libmgs.so): device
memory and a stream from the HIP runtime, the library's entry points for
the work, no Python and no torch in the process. Its outputs are compared
with the oracle byte for byte: dim0 with no workspace needed, dim0 with
chunk teams in the library's own workspace and in one the program sizes
with mgs_dim0_workspace_bytes, dim1, and the MX cast in both modes."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import __graft_entry__
from group_scaling_fp8_amd import workloads as wl
from gpu_util import assert_same_bytes

pytestmark = pytest.mark.gpu


def cases():
    rng = np.random.default_rng(930)
    w1 = wl.c1_dim0_small()
    tall = wl.randn_bf16(rng, (3000, 264), 0.02, 0.001, 8.0)
    tall_off = np.array([1400, 1400, 3000], np.int32)
    x1 = wl.randn_bf16(rng, (64, 1040), 0.02, 0.001, 8.0)
    off1 = np.array([0, 160, 480, 1040], np.int32)
    x5 = wl.randn_bf16(rng, (256, 1024), 1.0, 0.001, 100.0)
    return [("dim0", w1.x, w1.offsets, 0), ("dim0", tall, tall_off, 0), ("dim0_ws", tall, tall_off, 1),
            ("dim1", x1, off1, 0), ("mx", x5, None, 0), ("mx", x5, None, 1)]


def test_c_program_through_the_c_abi(tmp_path):
    exe = __graft_entry__.C_CONSUMER
    if not os.path.exists(exe):
        __graft_entry__.build_c_consumer()
    cs = cases()
    lines = []
    for i, (kind, x, off, arg) in enumerate(cs):
        M, K = x.shape
        G = 0 if off is None else len(off)
        lines.append("%s %d %d %d %d" % (kind, M, K, G, arg))
        x.tofile(tmp_path / ("%d.x" % i))
        if off is not None:
            off.tofile(tmp_path / ("%d.off" % i))
    (tmp_path / "cases.txt").write_text("\n".join(lines) + "\n")
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    for i, (kind, x, off, arg) in enumerate(cs):
        M, K = x.shape
        q = np.fromfile(tmp_path / ("%d.q" % i), np.uint8).reshape(M, K)
        if kind == "mx":
            rq, rs = oracle.mx_quant_dim0(x, arg)
            s = np.fromfile(tmp_path / ("%d.s" % i), np.uint8).reshape(rs.shape)
        elif kind == "dim1":
            rq, rs = oracle.quant_groups_dim1(x, off, bool(arg & 1))
            s = np.fromfile(tmp_path / ("%d.s" % i), np.float32).reshape(rs.shape)
        else:
            rq, rs = oracle.quant_groups_dim0(x, off, bool(arg & 1))
            s = np.fromfile(tmp_path / ("%d.s" % i), np.float32).reshape(rs.shape)
        assert_same_bytes(s, rs, "C case %d (%s) scales" % (i, kind))
        assert_same_bytes(q, rq, "C case %d (%s) q" % (i, kind))
