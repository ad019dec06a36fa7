"""The entry point that allocates nothing, mgs_quant_groups_dim0_noalloc,
called through the C ABI and compared with mgs_quant_groups_dim0_ws (the
same computation on a caller-owned workspace): calls in a row on the one
per-device scratch array, each later one on a smaller input, every E4M3
byte and every scale bit equal, and equal to the oracle. Inputs too large
for the array are refused before any GPU work."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import assert_same_bytes, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def _c_call(fn, x, off, flags, q, s, *ws):
    M, K = x.shape
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return fn(x.data_ptr(), M, K, off.data_ptr(), off.shape[0], flags, q.data_ptr(), s.data_ptr(),
              *ws, stream)


@pytest.mark.parametrize("pow2", [False, True])
def test_noalloc_matches_the_workspace_entry_point(pow2):
    L = mgs.lib()
    flags = mgs.MGS_FLAG_POW2_SCALE if pow2 else 0
    # tall groups (teams that exchange column maxima through the scratch),
    # then smaller inputs: fewer chunk rows, narrower rows, and one small
    # enough to need no workspace at all
    cases = [(16640, 2056, [200, 15000, 16640]), (9000, 520, [0, 8000, 9000]),
             (2000, 264, [641, 1300, 2000]), (600, 136, [100, 600])]
    for i, (M, K, ends) in enumerate(cases):
        rng = np.random.default_rng(1000 + i)
        xh = wl.randn_bf16(rng, (M, K), 0.02, 0.003, 8.0)
        off_h = np.array(ends, np.int32)
        x, off = to_dev(xh), to_dev(off_h)
        G = len(ends)
        q_a = torch.full((M, K), 0xA5, dtype=torch.uint8, device="cuda")
        s_a = torch.full((G, K), -1.0, dtype=torch.float32, device="cuda")
        q_b = torch.full_like(q_a, 0x5A)
        s_b = torch.full_like(s_a, -2.0)
        assert _c_call(L.mgs_quant_groups_dim0_noalloc, x, off, flags, q_a, s_a) == mgs.MGS_OK
        ws = mgs.dim0_workspace(M, K)
        assert _c_call(L.mgs_quant_groups_dim0_ws, x, off, flags, q_b, s_b,
                       ctypes.c_void_p(ws.data_ptr()), ws.numel()) == mgs.MGS_OK
        torch.cuda.synchronize()
        what = "call %d (%d, %d)" % (i, M, K)
        assert torch.equal(q_a, q_b), what + ": q differs from the workspace entry point's"
        assert torch.equal(s_a.view(torch.int32), s_b.view(torch.int32)), what + ": scales differ"
        rq, rs = oracle.quant_groups_dim0(xh, off_h, pow2)
        assert_same_bytes(s_a.cpu().numpy(), rs, what + " scales vs oracle")
        assert_same_bytes(q_a.cpu().numpy(), rq, what + " q vs oracle")


def test_noalloc_refuses_inputs_beyond_its_array():
    L = mgs.lib()
    need = ctypes.c_int64(0)
    M, K = 300000, 8192
    assert L.mgs_dim0_workspace_bytes(M, K, ctypes.byref(need)) == mgs.MGS_OK
    assert need.value > mgs._lib.MGS_NOALLOC_SCRATCH_BYTES
    A = 1 << 20     # never dereferenced: the size check comes first
    assert L.mgs_quant_groups_dim0_noalloc(A, M, K, A, 4, 0, A, A, None) == mgs.MGS_ERR_UNSUPPORTED
