"""GPU parity of the MX dequantisation (mgs_mx_dequant_dim0) against the
oracle, bit for bit: every (E4M3 code, E8M0 byte) pair, the round trip of
the MX configuration's shape (the library's own quantisation, then its
dequantisation, every value against the oracle's dequantisation of the
same bytes), a ragged flat tail, and guard bands on the output."""
import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import Guarded, assert_same_bytes, to_dev
from oracle_pool import check_mx_dequant_whole

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def run(q, s):
    M, K = q.shape
    gy = Guarded((M, K), torch.bfloat16)
    mgs.mgs_mx_dequant_dim0(to_dev(q), to_dev(s), y=gy.view)
    torch.cuda.synchronize()
    gy.check()
    return gy.view.view(torch.int16).cpu().numpy().view(np.uint16)


def test_every_code_and_scale_byte():
    q = np.tile(np.arange(256, dtype=np.uint8), (256, 1))
    s = np.repeat(np.arange(256, dtype=np.uint8)[:, None], 8, axis=1)
    assert_same_bytes(run(q, s), oracle.mx_dequant_dim0(q, s), "all 65536 pairs")


@pytest.mark.parametrize("M,K", [(1, 32), (3, 96), (7, 160), (129, 2080)])
def test_random_bytes_ragged(M, K):
    rng = np.random.default_rng(M * 1000 + K)
    q = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    s = rng.integers(0, 256, size=(M, K // 32), dtype=np.uint8)
    assert_same_bytes(run(q, s), oracle.mx_dequant_dim0(q, s), "random bytes (%d, %d)" % (M, K))


@pytest.mark.parametrize("mode", [mgs.MGS_MX_FLOOR, mgs.MGS_MX_RCEIL])
def test_round_trip_at_the_mx_shape(c5, mode):
    """The library's quantisation of the MX configuration, then its
    dequantisation: every bf16 of y against the oracle's dequantisation of
    the same bytes (the quantisation itself is compared whole in
    test_gpu_parity.py)."""
    x = to_dev(c5.x)
    q, s = mgs.mgs_mx_quant_dim0(x, mode)
    y = mgs.mgs_mx_dequant_dim0(q, s)
    torch.cuda.synchronize()
    check_mx_dequant_whole(q.cpu().numpy(), s.cpu().numpy(),
                           y.view(torch.int16).cpu().numpy().view(np.uint16), "mx round trip")
