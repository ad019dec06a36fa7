"""GPU parity of dim0 where the launch shape matters: the group sizes that
give the most tiles per row (the grid is an upper bound computed from M, K
and G alone), tiles whose last rows sit in LDS instead of registers, groups
taller than a chunk (896 rows) whose column maxima pass between
workgroups of one launch (as a team of chunk tiles, or through
column-maximum tiles when a group has more chunks than the team limit,
forced low here through MGS_DIM0_TEAM_MAX), the path that computes those
maxima from x in the waiting tile itself (forced from the host by a
negative wait bound), back-to-back calls on one stream and on two, and
replays of a captured graph."""
import os

import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import Guarded, assert_same_bytes, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def run_dim0(x, off, pow2=False):
    M, K = x.shape
    gq, gs = Guarded((M, K), torch.uint8), Guarded((len(off), K), torch.float32)
    mgs.mgs_quant_groups_dim0(to_dev(x), to_dev(off), pow2, q=gq.view, scales=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


def check(x, off, what, pow2=False):
    q, s = run_dim0(x, off, pow2)
    rq, rs = oracle.quant_groups_dim0(x, off, pow2)
    assert_same_bytes(s, rs, what + " scales")
    assert_same_bytes(q, rq, what + " q")


def data(seed, M, K):
    return wl.randn_bf16(np.random.default_rng(seed), (M, K), 0.02, 0.003, 8.0)


TEAM_MAX = [None, "1"]      # the library's limit, then every tall group through maxima tiles


def team_env(monkeypatch, team_max):
    if team_max is None:
        monkeypatch.delenv("MGS_DIM0_TEAM_MAX", raising=False)
    else:
        monkeypatch.setenv("MGS_DIM0_TEAM_MAX", team_max)


# The first row count of each tiling step has the most tiles per row: 113 rows
# (512-column strips), 225 (256), 449 (128), then 896 * (c - 1) + 1 rows for a
# group cut into c chunks (897: two); the transposed kernel's steps (81, 161,
# 321, 641, ...) are covered too. K values leave a ragged last strip.
@pytest.mark.parametrize("team_max", TEAM_MAX)
@pytest.mark.parametrize("size,n,K", [
    (113, 12, 2056), (225, 12, 1032), (449, 8, 520), (897, 6, 264), (1793, 3, 264),
    (2689, 2, 136), (896, 4, 264), (1792, 3, 136), (112, 10, 1032),
    (81, 12, 2056), (161, 12, 1032), (321, 10, 520), (641, 8, 264), (1281, 4, 264),
    (1921, 3, 136), (5121, 2, 264), (5121, 3, 72), (37, 16, 4104), (577, 4, 264),
    (865, 3, 136), (640, 5, 264), (1280, 3, 136),
])
def test_most_tiles_per_row(size, n, K, team_max, monkeypatch):
    team_env(monkeypatch, team_max)
    off = (np.arange(1, n + 1) * size).astype(np.int32)
    x = data(size + n, size * n, K)
    check(x, off, "groups of %d rows" % size)


# Tiles whose rows run past the 20 register slabs into the LDS slabs, for
# every strip width: rows 20 * rps .. 28 * rps - 1 (rps = 4, 8, 16, 32 rows
# per slab), with ragged last slabs, ragged K and empty groups beside them.
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("K,sizes", [
    (2056, [81, 100, 0, 112, 7]),          # 1024-column strips, rps = 4
    (1032, [161, 200, 224, 3]),            # 512, rps = 8
    (520, [321, 400, 448, 16]),            # 256, rps = 16
    (264, [641, 700, 896, 5, 0]),          # 128, rps = 32
    (8, [700, 896, 1]),                    # one 8-column strip
])
def test_rows_held_in_lds(K, sizes, pow2):
    off = np.cumsum(sizes).astype(np.int32)
    x = data(sum(sizes) + K, int(off[-1]), K)
    check(x, off, "LDS rows %s" % (sizes,), pow2)


def test_group_past_the_team_limit():
    # 134 chunks of 896 rows, more than any team (at most 128): column-maximum
    # tiles, then casting tiles
    M, K = 120000, 64
    check(data(9, M, K), np.array([5, M - 7, M], np.int32), "120000-row group")


def test_many_groups_at_the_group_limit():
    # 1024 groups: 1000 of 81 rows then empty ones, 8 columns (one strip each)
    sizes = [81] * 1000 + [0] * 24
    off = np.cumsum(sizes).astype(np.int32)
    check(data(7, int(off[-1]), 8), off, "1024 groups")


@pytest.mark.parametrize("team_max", TEAM_MAX)
@pytest.mark.parametrize("M,K,sizes", [
    (12000, 136, [0, 11000, 1000]),
    (16640, 256, [16640]),
    (11000, 64, [5500, 5500]),
    (3000, 520, [1281, 1719]),
    (2000, 264, [641, 700, 659]),
    (2700, 264, [897, 1000, 803]),
])
def test_tall_groups_without_the_wait(M, K, sizes, team_max, monkeypatch):
    team_env(monkeypatch, team_max)
    off = np.cumsum(sizes).astype(np.int32)
    x = data(M + K, M, K)
    monkeypatch.setenv("MGS_DIM0_SPIN_TICKS", "-1")
    check(x, off, "no wait %s" % (sizes,))
    monkeypatch.setenv("MGS_DIM0_SPIN_TICKS", "0")
    check(x, off, "zero wait %s" % (sizes,))


@pytest.mark.parametrize("team_max", TEAM_MAX)
def test_back_to_back_tall_calls_on_one_stream_and_two(team_max, monkeypatch):
    team_env(monkeypatch, team_max)
    M, K = 13000, 264
    off = np.array([300, 12000, 13000], np.int32)
    xs = [data(20 + i, M, K) for i in range(3)]
    o = to_dev(off)
    outs = []
    # three calls queued without a host sync between them: each must use its
    # own column maxima, not the previous call's
    for x in xs:
        outs.append(mgs.mgs_quant_groups_dim0(to_dev(x), o))
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        xo = to_dev(xs[0][:, ::-1].copy())
        other = mgs.mgs_quant_groups_dim0(xo, to_dev(off))
    torch.cuda.synchronize()
    for i, x in enumerate(xs):
        rq, rs = oracle.quant_groups_dim0(x, off)
        assert_same_bytes(outs[i][1].cpu().numpy(), rs, "call %d scales" % i)
        assert_same_bytes(outs[i][0].cpu().numpy(), rq, "call %d q" % i)
    rq, rs = oracle.quant_groups_dim0(xs[0][:, ::-1].copy(), off)
    assert_same_bytes(other[0].cpu().numpy(), rq, "side stream q")
    assert_same_bytes(other[1].cpu().numpy(), rs, "side stream scales")


@pytest.mark.parametrize("team_max", TEAM_MAX)
def test_graph_replays_of_a_tall_group(team_max, monkeypatch):
    team_env(monkeypatch, team_max)
    M, K = 11000, 136
    off = np.array([200, 10600, 11000], np.int32)
    xs = [data(40 + i, M, K) for i in range(3)]
    s = torch.cuda.Stream()
    xd, od = to_dev(xs[0]), to_dev(off)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty((len(off), K), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        # an eager call first: it allocates this stream's workspace
        mgs.mgs_quant_groups_dim0(xd, od, q=q, scales=sc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mgs.mgs_quant_groups_dim0(xd, od, q=q, scales=sc)
    torch.cuda.synchronize()
    for i in (0, 1, 2, 1):
        xd.copy_(to_dev(xs[i]))
        q.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rq, rs = oracle.quant_groups_dim0(xs[i], off)
        assert_same_bytes(sc.cpu().numpy(), rs, "replay %d scales" % i)
        assert_same_bytes(q.cpu().numpy(), rq, "replay %d q" % i)
        # an eager call on the capturing stream between replays
        with torch.cuda.stream(s):
            qe, se = mgs.mgs_quant_groups_dim0(xd, od)
        torch.cuda.synchronize()
        assert torch.equal(qe, q) and torch.equal(se, sc)
