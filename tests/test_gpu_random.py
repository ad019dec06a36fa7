"""Seeded random shapes and group layouts for every entry point, each
compared with the oracle byte for byte: arbitrary dim0 group boundaries
(empty groups, groups of one row, groups cut into chunk teams, and with a
team limit of 1 the column-maximum tiles; up to 1024 groups), ragged K, both scale modes and
both MX modes, the transposed forms, the expert weights and the MX
dequantisation of arbitrary code and scale bytes. Values mix normal draws
with zeros of both signs, subnormals, the largest bf16 magnitudes and
outliers. Sizes stay small so the oracle answers every case in
milliseconds; each case prints its parameters."""
import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import api
from group_scaling_fp8_amd import workloads as wl
from gpu_util import assert_same_bytes, to_dev

pytestmark = pytest.mark.gpu

SPECIALS = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
                     0x0400, 0x4300, 0xC380], np.uint16)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def values(rng, shape):
    sigma = float(rng.choice([0.02, 1.0, 300.0]))
    x = wl.randn_bf16(rng, shape, sigma, 0.002, sigma * 400.0)
    flat = x.reshape(-1)
    if flat.size:
        pick = rng.choice(flat.size, size=max(1, flat.size // 50), replace=False)
        flat[pick] = SPECIALS[rng.integers(0, len(SPECIALS), len(pick))]
    return x


def end_offsets(rng, extent, G, align):
    """G non-decreasing end offsets, multiples of align, the last = extent;
    some groups empty, one often much taller than the rest."""
    units = extent // align
    cuts = np.sort(rng.integers(0, units + 1, size=G - 1))
    if G > 2 and rng.random() < 0.5:
        cuts[rng.integers(0, G - 1):] = cuts[-1]          # a run of empty groups
    return (np.concatenate([cuts, [units]]) * align).astype(np.int32)


@pytest.mark.parametrize("i", range(24))
def test_dim0_random(i):
    rng = np.random.default_rng(5000 + i)
    M = int(rng.choice([int(rng.integers(1, 300)), int(rng.integers(300, 3000)), int(rng.integers(3000, 9000))]))
    K = 8 * int(rng.integers(1, 300))
    G = int(rng.integers(1, 40))
    pow2 = bool(rng.random() < 0.5)
    team_max = int(rng.choice([0, 0, 1, 2]))
    print("dim0 M=%d K=%d G=%d pow2=%d team_max=%d" % (M, K, G, pow2, team_max), flush=True)
    x = values(rng, (M, K))
    off = end_offsets(rng, M, G, 1)
    xd, od = to_dev(x), to_dev(off)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((G, K), dtype=torch.float32, device="cuda")
    if team_max:
        api._test_quant_dim0(xd, od, q, s, pow2=pow2, team_max=team_max)
    else:
        mgs.mgs_quant_groups_dim0(xd, od, pow2, q=q, scales=s)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_groups_dim0(x, off, pow2)
    assert_same_bytes(s.cpu().numpy(), rs, "dim0 random %d scales" % i)
    assert_same_bytes(q.cpu().numpy(), rq, "dim0 random %d q" % i)


@pytest.mark.parametrize("i", range(16))
def test_dim0_many_groups_random(i):
    """More than 64 groups: the tile search splits the groups over the
    workgroup's waves. Up to the 1024-group limit, with runs of empty groups,
    one-row groups, tall groups cut into teams and, with a team limit of 1
    or 2, column-maximum tiles."""
    rng = np.random.default_rng(12000 + i)
    G = int(rng.choice([65, int(rng.integers(66, 512)), 512, 513, int(rng.integers(514, 1024)), 1024]))
    M = int(rng.choice([int(rng.integers(1, 2000)), int(rng.integers(2000, 24000))]))
    K = 8 * int(rng.integers(1, 200))
    pow2 = bool(rng.random() < 0.5)
    team_max = int(rng.choice([0, 0, 1, 2]))
    print("dim0 many groups M=%d K=%d G=%d pow2=%d team_max=%d" % (M, K, G, pow2, team_max), flush=True)
    x = values(rng, (M, K))
    off = end_offsets(rng, M, G, 1)
    if rng.random() < 0.3:
        off[rng.integers(0, G):] = M            # the tail of the groups empty
        off[-1] = M
    xd, od = to_dev(x), to_dev(off)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((G, K), dtype=torch.float32, device="cuda")
    if team_max:
        api._test_quant_dim0(xd, od, q, s, pow2=pow2, team_max=team_max)
    else:
        mgs.mgs_quant_groups_dim0(xd, od, pow2, q=q, scales=s)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_groups_dim0(x, off, pow2)
    assert_same_bytes(s.cpu().numpy(), rs, "dim0 many groups %d scales" % i)
    assert_same_bytes(q.cpu().numpy(), rq, "dim0 many groups %d q" % i)


@pytest.mark.parametrize("i", range(6))
def test_dim0_t_many_groups_random(i):
    rng = np.random.default_rng(13000 + i)
    G = int(rng.choice([65, int(rng.integers(66, 1024)), 1024]))
    M = 16 * int(rng.integers(1, 1200))
    K = 8 * int(rng.integers(1, 120))
    pow2 = bool(rng.random() < 0.5)
    print("dim0_t many groups M=%d K=%d G=%d pow2=%d" % (M, K, G, pow2), flush=True)
    x = values(rng, (M, K))
    off = end_offsets(rng, M, G, 16)
    q_t, s_t = mgs.mgs_quant_groups_dim0_t(to_dev(x), to_dev(off), pow2)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_groups_dim0_t(x, off, pow2)
    assert_same_bytes(s_t.cpu().numpy(), rs, "dim0_t many groups %d scales" % i)
    assert_same_bytes(q_t.cpu().numpy(), rq, "dim0_t many groups %d q" % i)


@pytest.mark.parametrize("i", range(12))
def test_dim0_t_random(i):
    rng = np.random.default_rng(6000 + i)
    M = 16 * int(rng.integers(1, 500))
    K = 8 * int(rng.integers(1, 200))
    G = int(rng.integers(1, 30))
    pow2 = bool(rng.random() < 0.5)
    print("dim0_t M=%d K=%d G=%d pow2=%d" % (M, K, G, pow2), flush=True)
    x = values(rng, (M, K))
    off = end_offsets(rng, M, G, 16)
    q_t, s_t = mgs.mgs_quant_groups_dim0_t(to_dev(x), to_dev(off), pow2)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_groups_dim0_t(x, off, pow2)
    assert_same_bytes(s_t.cpu().numpy(), rs, "dim0_t random %d scales" % i)
    assert_same_bytes(q_t.cpu().numpy(), rq, "dim0_t random %d q" % i)


@pytest.mark.parametrize("i", range(16))
def test_dim1_random(i):
    rng = np.random.default_rng(7000 + i)
    M = int(rng.integers(1, 200))
    K = 16 * int(rng.integers(1, 700))
    G = int(rng.integers(1, 80))
    pow2 = bool(rng.random() < 0.5)
    print("dim1 M=%d K=%d G=%d pow2=%d" % (M, K, G, pow2), flush=True)
    x = values(rng, (M, K))
    off = end_offsets(rng, K, G, 16)
    q, s = mgs.mgs_quant_groups_dim1(to_dev(x), to_dev(off), pow2)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_groups_dim1(x, off, pow2)
    assert_same_bytes(s.cpu().numpy(), rs, "dim1 random %d scales" % i)
    assert_same_bytes(q.cpu().numpy(), rq, "dim1 random %d q" % i)


@pytest.mark.parametrize("i", range(8))
def test_experts_random(i):
    rng = np.random.default_rng(8000 + i)
    E = int(rng.integers(1, 9))
    D1 = int(rng.choice([int(rng.integers(0, 100)), int(rng.integers(100, 2500))]))
    D2 = 8 * int(rng.integers(1, 100))
    pow2 = bool(rng.random() < 0.5)
    print("experts E=%d D1=%d D2=%d pow2=%d" % (E, D1, D2, pow2), flush=True)
    w = values(rng, (E, D1, D2))
    q, s = mgs.mgs_quant_experts_dim1(to_dev(w), pow2)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_experts_dim1(w, pow2)
    assert_same_bytes(s.cpu().numpy(), rs, "experts random %d scales" % i)
    assert_same_bytes(q.cpu().numpy(), rq, "experts random %d q" % i)


@pytest.mark.parametrize("i", range(12))
def test_mx_random(i):
    rng = np.random.default_rng(9000 + i)
    M = int(rng.integers(1, 700))
    K = 32 * int(rng.integers(1, 80))
    mode = int(rng.integers(0, 2))
    print("mx M=%d K=%d mode=%d" % (M, K, mode), flush=True)
    x = values(rng, (M, K))
    q, s = mgs.mgs_mx_quant_dim0(to_dev(x), mode)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quant_dim0(x, mode)
    assert_same_bytes(s.cpu().numpy(), rs, "mx random %d scales" % i)
    assert_same_bytes(q.cpu().numpy(), rq, "mx random %d q" % i)


@pytest.mark.parametrize("i", range(12))
def test_mx_dim1_random(i):
    rng = np.random.default_rng(10000 + i)
    M = 32 * int(rng.integers(1, 40))
    K = 8 * int(rng.integers(1, 100))
    mode = int(rng.integers(0, 2))
    print("mx_dim1 M=%d K=%d mode=%d" % (M, K, mode), flush=True)
    x = values(rng, (M, K))
    q_t, s_t = mgs.mgs_mx_quant_dim1(to_dev(x), mode)
    torch.cuda.synchronize()
    rq, rs = oracle.mx_quant_dim1(x, mode)
    assert_same_bytes(s_t.cpu().numpy(), rs, "mx_dim1 random %d scales" % i)
    assert_same_bytes(q_t.cpu().numpy(), rq, "mx_dim1 random %d q" % i)


@pytest.mark.parametrize("i", range(8))
def test_mx_dequant_random(i):
    rng = np.random.default_rng(11000 + i)
    M = int(rng.integers(1, 400))
    K = 32 * int(rng.integers(1, 60))
    print("mx dequant M=%d K=%d" % (M, K), flush=True)
    q = rng.integers(0, 256, size=(M, K), dtype=np.uint8)
    sc = rng.integers(0, 256, size=(M, K // 32), dtype=np.uint8)
    y = mgs.mgs_mx_dequant_dim0(to_dev(q), to_dev(sc))
    torch.cuda.synchronize()
    ry = oracle.mx_dequant_dim0(q, sc)
    assert_same_bytes(y.view(torch.int16).cpu().numpy().view(np.uint16), ry, "mx dequant random %d" % i)
