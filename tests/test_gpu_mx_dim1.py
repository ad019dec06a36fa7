"""GPU parity of the MX cast along dim0 with transposed outputs
(mgs_mx_quant_dim1) against the oracle, bit for bit: ragged tiles in both
dims, FLOOR and RCEIL, subnormal and zero blocks, and the MX configuration's
shape compared whole. Guard bands on both outputs."""
import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import Guarded, assert_same_bytes, to_dev
from oracle_pool import check_mx_dim1_whole

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def run(x, mode):
    M, K = x.shape
    gq, gs = Guarded((K, M), torch.uint8), Guarded((K, M // 32), torch.uint8)
    mgs.mgs_mx_quant_dim1(to_dev(x), mode, q_t=gq.view, scales_t=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


@pytest.mark.parametrize("mode", [mgs.MGS_MX_FLOOR, mgs.MGS_MX_RCEIL])
@pytest.mark.parametrize("M,K", [(32, 8), (160, 136), (256, 264), (96, 520), (4096, 128)])
def test_mx_dim1(M, K, mode):
    rng = np.random.default_rng(M * 7 + K + mode)
    x = wl.randn_bf16(rng, (M, K), 1.0, 0.001, 100.0)
    x[:32, :8] = 0                                       # an all-zero block
    if M >= 64 and K >= 16:
        x[32:64, 8:16] = 0x0001                          # a block of the least subnormal
    q, s = run(x, mode)
    rq, rs = oracle.mx_quant_dim1(x, mode)
    assert_same_bytes(s, rs, "scales_t (%d, %d)" % (M, K))
    assert_same_bytes(q, rq, "q_t (%d, %d)" % (M, K))


@pytest.mark.parametrize("mode", [mgs.MGS_MX_FLOOR, mgs.MGS_MX_RCEIL])
def test_mx_dim1_at_the_mx_shape_whole(c5, mode):
    q, s = mgs.mgs_mx_quant_dim1(to_dev(c5.x), mode)
    torch.cuda.synchronize()
    check_mx_dim1_whole(c5.x, mode, q.cpu().numpy(), s.cpu().numpy(), "mx dim1 mode %d" % mode)
