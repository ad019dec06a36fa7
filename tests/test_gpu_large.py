"""GPU parity past 2^31 elements: every entry point on an input of more than
2^31 bf16 values (over 4 GiB), compared whole with the oracle, byte for
byte. Element offsets there no longer fit in 32 bits, so a 32-bit product
anywhere in the index arithmetic would read or write the wrong rows.

The inputs repeat a generated block of P = 4099 rows, each repetition with
its own low-mantissa pattern: rows 2^31 elements apart (2^31 / K rows) sit
at different rows of the block, so a wrapped index reads different values
and the comparison fails."""
import numpy as np
import pytest
import torch

import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import to_dev
from oracle_pool import (check_dim0_t_whole, check_dim0_whole, check_dim1_whole, check_mx_dequant_whole,
                         check_mx_dim1_whole, check_mx_whole)

pytestmark = pytest.mark.gpu

TWO_G = 1 << 31
BLOCK_ROWS = 4099


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def big_input(M, K, seed, sigma, outlier_mag):
    assert M * K > TWO_G and (TWO_G // K) % BLOCK_ROWS != 0
    rng = np.random.default_rng(seed)
    block = wl.randn_bf16(rng, (BLOCK_ROWS, K), sigma, 0.001, outlier_mag)
    x = np.empty((M, K), np.uint16)
    for i, lo in enumerate(range(0, M, BLOCK_ROWS)):
        hi = min(M, lo + BLOCK_ROWS)
        # flips of the three low mantissa bits keep every value finite
        np.bitwise_xor(block[:hi - lo], np.uint16(i % 7 + 1), out=x[lo:hi])
    return x


@pytest.fixture(scope="module")
def tall():
    """(262400, 8192): 2,149,580,800 elements, groups along dim0."""
    return big_input(262400, 8192, 900, 0.02, 8.0)


@pytest.fixture(scope="module")
def wide_mx():
    """(419456, 5120): 2,147,614,720 elements, the MX configuration's values."""
    return big_input(419456, 5120, 901, 1.0, 100.0)


def test_dim0_past_2g_elements(tall):
    M, K = tall.shape
    off = wl.uniform_group_offsets(np.random.default_rng(910), M, 8)
    q, s = mgs.mgs_quant_groups_dim0(to_dev(tall), to_dev(off))
    torch.cuda.synchronize()
    check_dim0_whole(tall, off, False, q.cpu().numpy(), s.cpu().numpy(), "dim0 (%d, %d)" % (M, K))


def test_dim0_t_past_2g_elements(tall):
    M, K = tall.shape
    off = wl.uniform_group_offsets(np.random.default_rng(911), M, 8)
    q_t, s_t = mgs.mgs_quant_groups_dim0_t(to_dev(tall), to_dev(off), True)
    torch.cuda.synchronize()
    check_dim0_t_whole(tall, off, True, q_t.cpu().numpy(), s_t.cpu().numpy(), "dim0_t (%d, %d)" % (M, K))


def test_dim1_past_2g_elements():
    M, K = 129200, 16640          # 2,149,888,000 elements
    x = big_input(M, K, 902, 0.02, 8.0)
    off = wl.uniform_group_offsets(np.random.default_rng(912), K, 16)
    q, s = mgs.mgs_quant_groups_dim1(to_dev(x), to_dev(off))
    torch.cuda.synchronize()
    check_dim1_whole(x, off, False, q.cpu().numpy(), s.cpu().numpy(), "dim1 (%d, %d)" % (M, K))


def test_mx_and_dequant_past_2g_elements(wide_mx):
    xd = to_dev(wide_mx)
    q, s = mgs.mgs_mx_quant_dim0(xd, mgs.MGS_MX_FLOOR)
    y = mgs.mgs_mx_dequant_dim0(q, s)
    torch.cuda.synchronize()
    del xd
    qh, sh = q.cpu().numpy(), s.cpu().numpy()
    del q, s
    check_mx_whole(wide_mx, mgs.MGS_MX_FLOOR, qh, sh, "mx FLOOR %s" % (wide_mx.shape,))
    check_mx_dequant_whole(qh, sh, y.view(torch.int16).cpu().numpy().view(np.uint16),
                           "mx dequant %s" % (wide_mx.shape,))


def test_mx_dim1_past_2g_elements(wide_mx):
    q_t, s_t = mgs.mgs_mx_quant_dim1(to_dev(wide_mx), mgs.MGS_MX_RCEIL)
    torch.cuda.synchronize()
    check_mx_dim1_whole(wide_mx, mgs.MGS_MX_RCEIL, q_t.cpu().numpy(), s_t.cpu().numpy(),
                        "mx dim1 RCEIL %s" % (wide_mx.shape,))
