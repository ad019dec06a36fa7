"""GPU parity of the per-expert scaling of 3D weights along dim 1
(mgs_quant_experts_dim1) against the oracle byte for byte: short experts on
wide strips, experts cut into chunk teams, experts with no rows, the
column-maximum tiles, pow2 scales, and a Llama4-sized weight (16 experts of
5120 x 8192) where every byte must equal dim0 with explicit offsets and
the oracle. Guard bands on every output."""
import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import Guarded, assert_same_bytes, to_dev
from oracle_pool import check_experts_whole

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def run(w, pow2=False):
    E, D1, D2 = w.shape
    gq, gs = Guarded((E, D1, D2), torch.uint8), Guarded((E, D2), torch.float32)
    mgs.mgs_quant_experts_dim1(to_dev(w), pow2, q=gq.view, scales=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


def check(w, what, pow2=False):
    q, s = run(w, pow2)
    rq, rs = oracle.quant_experts_dim1(w, pow2)
    assert_same_bytes(s, rs, what + " scales")
    assert_same_bytes(q, rq, what + " q")


def weights(seed, E, D1, D2):
    rng = np.random.default_rng(seed)
    return wl.randn_bf16(rng, (E * D1, D2), 0.02, 0.002, 8.0).reshape(E, D1, D2)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("E,D1,D2", [
    (3, 100, 264), (2, 1300, 136), (1, 640, 8), (5, 700, 72), (16, 48, 1032), (4, 0, 64),
])
def test_experts(E, D1, D2, pow2):
    check(weights(E * 131 + D1, E, D1, D2), "(%d, %d, %d)" % (E, D1, D2), pow2)


def test_experts_through_column_maximum_tiles():
    # team limit 1 through the test-only entry point (equal groups, no offsets)
    w = weights(3, 3, 1300, 136)
    E, D1, D2 = w.shape
    gq, gs = Guarded((E * D1, D2), torch.uint8), Guarded((E, D2), torch.float32)
    mgs.api._test_quant_dim0(to_dev(w.reshape(E * D1, D2)), None, gq.view, gs.view,
                             uniform_rows=D1, n_groups=E, team_max=1,
                             workspace=mgs.dim0_workspace(E * D1, D2))
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    rq, rs = oracle.quant_experts_dim1(w)
    assert_same_bytes(gs.numpy(), rs, "team limit 1 scales")
    assert_same_bytes(gq.numpy().reshape(E, D1, D2), rq, "team limit 1 q")


def test_experts_with_a_caller_workspace():
    w = weights(4, 4, 2000, 264)
    E, D1, D2 = w.shape
    ws = mgs.dim0_workspace(E * D1, D2)
    for _ in range(2):
        q, s = mgs.mgs_quant_experts_dim1(to_dev(w), workspace=ws)
        torch.cuda.synchronize()
        rq, rs = oracle.quant_experts_dim1(w)
        assert_same_bytes(s.cpu().numpy(), rs, "caller workspace scales")
        assert_same_bytes(q.cpu().numpy(), rq, "caller workspace q")


def test_llama4_sized_weight():
    """16 experts of (5120, 8192): every byte against dim0 with explicit
    offsets, and every byte and scale against the oracle."""
    E, D1, D2 = 16, 5120, 8192
    g = torch.Generator(device="cuda").manual_seed(6)
    w = (torch.randn((E, D1, D2), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    q, s = mgs.mgs_quant_experts_dim1(w)
    off = torch.arange(1, E + 1, dtype=torch.int32, device="cuda") * D1
    q0, s0 = mgs.mgs_quant_groups_dim0(w.view(E * D1, D2), off)
    torch.cuda.synchronize()
    assert torch.equal(q.view(E * D1, D2), q0)
    assert torch.equal(s.view(torch.int32), s0.view(torch.int32))
    wh = w.view(torch.int16).cpu().numpy().view(np.uint16)
    check_experts_whole(wh, False, q.cpu().numpy(), s.cpu().numpy(), "(16, 5120, 8192)")
