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


def test_trace_build_exports(L):
    """libmgs_trace.so (the tile-timeline diagnostic build) exports every
    entry point of mgs.h plus the calls of mgs_trace.h; libmgs.so exports
    none of the latter."""
    from group_scaling_fp8_amd import build
    if not os.path.exists(build.LIB_TRACE):
        build.build(trace=True)
    T = ctypes.CDLL(build.LIB_TRACE)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mgs_trace.h")).read(), flags=re.S)
    trace_names = set(re.findall(r"^\s*\w+\s*\*?\s*(mgs_\w+)\s*\(", text, flags=re.M))
    assert trace_names == {"mgs_tile_trace_capacity", "mgs_tile_trace_clear", "mgs_tile_trace_read",
                           "mgs_tile_trace_stamp"}
    for n in header_functions() + sorted(trace_names):
        assert hasattr(T, n), n
    for n in trace_names:
        assert not hasattr(L, n), n
    T.mgs_tile_trace_capacity.restype = ctypes.c_int
    assert T.mgs_tile_trace_capacity() == 16384
    # argument checks come before any HIP call
    T.mgs_tile_trace_stamp.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    T.mgs_tile_trace_stamp.restype = ctypes.c_int
    assert T.mgs_tile_trace_stamp(None, None) != 0
    assert T.mgs_tile_trace_stamp(A + 4, None) != 0


def test_status_strings(L):
    for code in range(4):
        assert L.mgs_status_string(code)
    assert L.mgs_status_string(99) == b"unknown status"


@pytest.mark.parametrize("fn", ["mgs_quant_groups_dim0", "mgs_quant_groups_dim0_ws",
                                "mgs_quant_groups_dim0_noalloc", "mgs_quant_groups_dim0_t",
                                "mgs_quant_groups_dim1"])
def test_grouped_argument_errors(L, fn):
    f = getattr(L, fn)
    ok = dict(x=A, M=64, K=128, off=A, G=4, flags=0, q=A, s=A, ws=None, wsb=0, stream=None)
    takes_ws = fn.endswith("_ws") or fn.endswith("_t")

    def call(**kw):
        a = dict(ok, **kw)
        if takes_ws:
            return f(a["x"], a["M"], a["K"], a["off"], a["G"], a["flags"], a["q"], a["s"], a["ws"],
                     a["wsb"], a["stream"])
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
    if takes_ws:
        assert call(ws=None, wsb=256) == INVALID          # a size without a buffer
        assert call(ws=A + 128, wsb=1 << 20) == INVALID   # 256-byte alignment
        assert call(ws=A, wsb=-1) == INVALID
        # M = 2000 rows can make chunked groups: the workspace must be big enough
        need = ctypes.c_int64(0)
        assert L.mgs_dim0_workspace_bytes(2000, 128, ctypes.byref(need)) == mgs.MGS_OK
        assert need.value > 0
        assert call(M=2000, ws=A, wsb=need.value - 8) == INVALID
    if fn.endswith("_noalloc"):
        # inputs whose workspace would exceed the fixed scratch array
        assert call(M=300000, K=8192) == UNSUPPORTED
    if fn.endswith("dim0") or fn.endswith("dim0_ws") or fn.endswith("_noalloc"):
        assert call(K=12) == INVALID
        assert call(s=A + 4) == INVALID
        # 1024 groups over 65536 rows of K = 2^31 - 8 columns (taller groups
        # cut into chunk teams on 128-column strips): the tile bound passes 2^31
        assert call(M=65536, K=(1 << 31) - 8, G=1024) == UNSUPPORTED
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
    def f(*a):
        return L.mgs_quant_experts_dim1(*a[:7], None, 0, None)
    assert f(A, 0, 64, 128, 0, A, A) == INVALID        # E >= 1
    assert f(A, 2, -1, 128, 0, A, A) == INVALID
    assert f(A, 1025, 16, 128, 0, A, A) == UNSUPPORTED
    assert f(A, 4, 1 << 30, 128, 0, A, A) == UNSUPPORTED   # E * D1 >= 2^31
    assert f(A, 2, 64, 12, 0, A, A) == INVALID         # D2 % 8
    assert f(A, 2, 64, 128, 4, A, A) == INVALID        # unknown flag
    assert f(A + 8, 2, 64, 128, 0, A, A) == INVALID
    assert f(A, 2, 64, 128, 0, A + 4, A) == INVALID
    assert f(A, 2, 64, 128, 0, A, A + 4) == INVALID
    assert f(None, 2, 64, 128, 0, A, A) == INVALID
    # 2 experts of 1000 rows need a workspace; a short one is refused
    assert L.mgs_quant_experts_dim1(A, 2, 1000, 128, 0, A, A, A, 256, None) == INVALID


def test_workspace_size_query(L):
    n = ctypes.c_int64(-1)
    assert L.mgs_dim0_workspace_bytes(896, 4096, ctypes.byref(n)) == mgs.MGS_OK and n.value == 0
    def expect(M, K):
        c = M // 896 + M // 897
        return -(-4 * c * -(-K // 128) // 256) * 256 + 8 * c * (K // 2)
    assert L.mgs_dim0_workspace_bytes(897, 8, ctypes.byref(n)) == mgs.MGS_OK
    assert n.value == expect(897, 8) == 256 + 8 * 2 * 4
    assert L.mgs_dim0_workspace_bytes(16640, 8192, ctypes.byref(n)) == mgs.MGS_OK
    assert n.value == expect(16640, 8192)
    assert L.mgs_dim0_workspace_bytes(-1, 8, ctypes.byref(n)) == INVALID
    assert L.mgs_dim0_workspace_bytes(8, 8, None) == INVALID
    assert L.mgs_dim0_workspace_bytes(1 << 31, 8, ctypes.byref(n)) == UNSUPPORTED


def test_test_entry_argument_errors(L):
    f = L.mgs_test_quant_dim0
    # equal groups: M must be n_groups * uniform_rows, and no transposed form
    assert f(A, 300, 64, None, 3, 100, 0, 1, A, A, None, 0, -2, 0, None) == INVALID
    assert f(A, 301, 64, None, 3, 100, 0, 0, A, A, None, 0, -2, 0, None) == INVALID
    assert f(A, 64, 128, A, 4, -1, 8, 0, A, A, None, 0, -2, 0, None) == INVALID


def _undefined_symbols(path):
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", path], capture_output=True, text=True,
                         check=True).stdout
    return {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}


def test_library_reads_no_environment(L):
    """The library takes every setting as an argument: it imports no
    environment reader."""
    und = _undefined_symbols(mgs.library_path())
    assert not und & {"getenv", "secure_getenv", "__secure_getenv", "environ"}, und
    # the only allocation and the only stream wait it may make: the own
    # workspace of calls given none, and MGS_FLAG_VALIDATE's offsets copy
    assert "hipFree" not in und and "hipDeviceSynchronize" not in und


def test_mx_dim1_argument_errors(L):
    f = L.mgs_mx_quant_dim1
    assert f(A, 48, 64, 0, A, A, None) == INVALID           # M % 32
    assert f(A, 64, 12, 0, A, A, None) == INVALID           # K % 8
    assert f(A, 64, 64, 2, A, A, None) == INVALID           # mode
    assert f(A + 8, 64, 64, 0, A, A, None) == INVALID
    assert f(A, 64, 64, 0, A + 4, A, None) == INVALID
    assert f(A, 64, 64, 0, A + 8, A, None) == INVALID       # q_t takes 16-byte stores
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
    assert L.mgs_quant_groups_dim1(None, 0, 0, A, 2, 0, None, None, None) == mgs.MGS_OK
    # no columns but rows: the scales of the empty groups are still written
    assert L.mgs_quant_groups_dim1(None, 8, 0, A, 2, 0, None, None, None) == INVALID
    assert L.mgs_quant_groups_dim1(None, 8, 0, A, 2, 0, None, A + 2, None) == INVALID
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


def test_missing_library_fails_loudly():
    """Without libmgs.so the binding raises on first use: there is no CPU
    fallback to route the work through."""
    import subprocess
    import sys
    code = ("import group_scaling_fp8_amd._lib as L\n"
            "L._LIB_PATH = '/nonexistent/libmgs.so'\n"
            "try:\n    L.lib()\nexcept RuntimeError as e:\n    print('raised:', e)\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert "raised: libmgs.so not found" in r.stdout, r.stdout + r.stderr


def test_product_path_never_imports_the_oracle():
    """The package (the binding and its helpers) imports nothing from
    oracle/: the oracle is test infrastructure only."""
    import ast
    pkg = os.path.join(ROOT, "group_scaling_fp8_amd")
    for name in sorted(os.listdir(pkg)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(pkg, name)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            else:
                continue
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)


def test_counter_provenance_hash_ignores_comments():
    """bench.py reports counter traffic only while the kernel sources' code
    hash matches the one the counters were taken on: comment and blank-line
    edits keep the hash, code edits change it."""
    import bench
    code = "int f(int a) {  // one\n    return a + 1;\n}\n"
    assert bench._code_only(code) == bench._code_only("// header\n\n" + code.replace("// one", "// two"))
    assert bench._code_only(code) != bench._code_only(code.replace("a + 1", "a + 2"))
    assert len(bench.kernel_source_hash()) == 16


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with status 2 and says
    why, before touching a GPU."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""

