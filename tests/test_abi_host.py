"""CPU-only checks of the C ABI: the library loads, exports every entry point
declared in include/mgs.h, and rejects bad arguments on the host before any
GPU work (these calls never reach HIP, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import group_scaling_fp8_amd as mgs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mgs.h")

INVALID, UNSUPPORTED = mgs.MGS_ERR_INVALID_ARG, mgs.MGS_ERR_UNSUPPORTED
A = 1 << 20          # a fake, well-aligned "device" address; never dereferenced


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mgs_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mgs.library_path()):
        from group_scaling_fp8_amd import build
        build.build()
    return mgs.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert set(names) >= {"mgs_quant_groups_dim0", "mgs_quant_groups_dim1", "mgs_mx_quant_dim0"}
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mgs._lib.EXPORTS)


def test_status_strings(L):
    for code in range(4):
        assert L.mgs_status_string(code)
    assert L.mgs_status_string(99) == b"unknown status"


@pytest.mark.parametrize("fn", ["mgs_quant_groups_dim0", "mgs_quant_groups_dim0_t",
                                "mgs_quant_groups_dim1"])
def test_grouped_argument_errors(L, fn):
    f = getattr(L, fn)
    ok = dict(x=A, M=64, K=128, off=A, G=4, flags=0, q=A, s=A, stream=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["M"], a["K"], a["off"], a["G"], a["flags"], a["q"], a["s"], a["stream"])

    assert call(M=-1) == INVALID
    assert call(K=-8) == INVALID
    assert call(G=0) == INVALID
    assert call(G=-3) == INVALID
    assert call(G=mgs.MGS_MAX_GROUPS + 1) == UNSUPPORTED
    assert call(flags=4) == INVALID
    assert call(flags=0x80000000) == INVALID
    assert call(off=None) == INVALID
    assert call(off=A + 2) == INVALID
    assert call(x=None) == INVALID
    assert call(q=None) == INVALID
    assert call(x=A + 8) == INVALID
    assert call(q=A + 4) == INVALID
    assert call(s=None) == INVALID
    assert call(M=1 << 31) == UNSUPPORTED
    if fn.endswith("dim0"):
        assert call(K=12) == INVALID
        assert call(s=A + 4) == INVALID
        # 1024 groups of 1024-column strips over K = 2^31 - 8: the tile bound reaches 2^31
        assert call(K=(1 << 31) - 8, G=1024) == UNSUPPORTED
    elif fn.endswith("dim0_t"):
        assert call(K=12) == INVALID
        assert call(M=24) == INVALID            # M % 16
        assert call(q=A + 8) == INVALID         # q_t takes 16-byte stores
        assert call(s=A + 2) == INVALID
        assert call(K=(1 << 31) - 8, G=1024) == UNSUPPORTED
    else:
        assert call(K=24) == INVALID
        assert call(s=A + 2) == INVALID
        assert call(K=mgs._lib.MGS_DIM1_MAX_K + 16) == UNSUPPORTED


def test_experts_argument_errors(L):
    f = L.mgs_quant_experts_dim1
    assert f(A, 0, 64, 128, 0, A, A, None) == INVALID        # E >= 1
    assert f(A, 2, -1, 128, 0, A, A, None) == INVALID
    assert f(A, 1025, 16, 128, 0, A, A, None) == UNSUPPORTED
    assert f(A, 4, 1 << 30, 128, 0, A, A, None) == UNSUPPORTED   # E * D1 >= 2^31
    assert f(A, 2, 64, 12, 0, A, A, None) == INVALID         # D2 % 8
    assert f(A, 2, 64, 128, 4, A, A, None) == INVALID        # unknown flag
    assert f(A + 8, 2, 64, 128, 0, A, A, None) == INVALID
    assert f(A, 2, 64, 128, 0, A + 4, A, None) == INVALID
    assert f(A, 2, 64, 128, 0, A, A + 4, None) == INVALID
    assert f(None, 2, 64, 128, 0, A, A, None) == INVALID


def test_mx_dim1_argument_errors(L):
    f = L.mgs_mx_quant_dim1
    assert f(A, 48, 64, 0, A, A, None) == INVALID           # M % 32
    assert f(A, 64, 12, 0, A, A, None) == INVALID           # K % 8
    assert f(A, 64, 64, 2, A, A, None) == INVALID           # mode
    assert f(A + 8, 64, 64, 0, A, A, None) == INVALID
    assert f(A, 64, 64, 0, A + 4, A, None) == INVALID
    assert f(A, 64, 64, 0, A, None, None) == INVALID
    assert f(A, 0, 64, 0, A, A, None) == mgs.MGS_OK


def test_mx_dequant_argument_errors(L):
    f = L.mgs_mx_dequant_dim0
    assert f(A, A, 4, 48, A, None) == INVALID            # K % 32
    assert f(A, A, -1, 64, A, None) == INVALID
    assert f(None, A, 4, 64, A, None) == INVALID
    assert f(A, None, 4, 64, A, None) == INVALID
    assert f(A, A, 4, 64, None, None) == INVALID
    assert f(A + 8, A, 4, 64, A, None) == INVALID         # q 16-byte aligned
    assert f(A, A, 4, 64, A + 8, None) == INVALID         # y 16-byte aligned
    assert f(A, A, 0, 64, A, None) == mgs.MGS_OK
    assert f(A, A, 1 << 40, 1 << 30, A, None) == UNSUPPORTED


def test_mx_argument_errors(L):
    f = L.mgs_mx_quant_dim0
    assert f(A, 4, 48, None, 0, 0, A, A, None) == INVALID           # K % 32
    assert f(A, 4, 64, None, 0, 2, A, A, None) == INVALID           # mode
    assert f(A, -1, 64, None, 0, 0, A, A, None) == INVALID
    assert f(None, 4, 64, None, 0, 0, A, A, None) == INVALID
    assert f(A, 4, 64, None, 0, 0, None, A, None) == INVALID
    assert f(A, 4, 64, None, 0, 0, A, None, None) == INVALID
    assert f(A + 8, 4, 64, None, 0, 1, A, A, None) == INVALID


def test_noop_shapes_return_ok_without_gpu(L):
    # zero-sized work launches nothing, so these succeed even without a GPU
    assert L.mgs_quant_groups_dim1(None, 0, 128, A, 2, 0, None, None, None) == mgs.MGS_OK
    assert L.mgs_quant_groups_dim1(None, 8, 0, A, 2, 0, None, None, None) == mgs.MGS_OK
    assert L.mgs_quant_groups_dim0(None, 8, 0, A, 2, 0, None, None, None) == mgs.MGS_OK
    assert L.mgs_mx_quant_dim0(None, 0, 64, None, 0, 0, None, None, None) == mgs.MGS_OK
    assert L.mgs_cast_e4m3(None, 0, None, None) == mgs.MGS_OK
    assert L.mgs_copy(None, None, 0, None) == mgs.MGS_OK


def test_cast_and_copy_argument_errors(L):
    assert L.mgs_cast_e4m3(A, 6, A, None) == INVALID
    assert L.mgs_cast_e4m3(A + 4, 8, A, None) == INVALID
    assert L.mgs_copy(A, A, 24, None) == INVALID
    assert L.mgs_copy(A + 8, A, 32, None) == INVALID


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(16, 32, dtype=torch.bfloat16)
    off = torch.tensor([16], dtype=torch.int32)
    with pytest.raises(ValueError):
        mgs.mgs_quant_groups_dim0(x, off)
