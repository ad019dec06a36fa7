"""GPU parity of dim0 where the launch shape matters: the group sizes that
give the most tiles per row (the grid is an upper bound computed from M, K
and G alone), tiles whose last rows sit in LDS instead of registers, groups
taller than a chunk (896 rows) whose column maxima pass between
workgroups of one launch (as a team of chunk tiles, or through
column-maximum tiles when a group has more chunks than the team limit,
forced low here through the test-only entry point's team limit), the path
that computes those maxima from x in the waiting tile itself (forced from
the host by a negative wait bound), back-to-back calls on one stream and on
two, the library's own workspace and caller-owned ones (which every call
leaves zero-filled), replays of captured graphs, teams beside other
kernels, and one-group launches of a few rounds of tiles, which run as one
resident round of workgroups."""
import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import Guarded, assert_same_bytes, to_dev
import lds_row_cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def run_dim0(x, off, pow2=False, team_max=None, spin=None, workspace=None):
    """dim0 through the public call, or through the test-only entry point
    when a team limit or a wait bound is forced."""
    M, K = x.shape
    gq, gs = Guarded((M, K), torch.uint8), Guarded((len(off), K), torch.float32)
    if team_max is None and spin is None:
        mgs.mgs_quant_groups_dim0(to_dev(x), to_dev(off), pow2, q=gq.view, scales=gs.view,
                                  workspace=workspace)
    else:
        if workspace is None:
            workspace = mgs.dim0_workspace(M, K)
        mgs.api._test_quant_dim0(to_dev(x), to_dev(off), gq.view, gs.view, pow2=pow2,
                                 spin_ticks=mgs.api.TEST_DEFAULT_SPIN if spin is None else spin,
                                 team_max=mgs.api.TEST_DEFAULT_TEAM if team_max is None else team_max,
                                 workspace=workspace)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


def check(x, off, what, pow2=False, team_max=None, spin=None, workspace=None):
    q, s = run_dim0(x, off, pow2, team_max, spin, workspace)
    rq, rs = oracle.quant_groups_dim0(x, off, pow2)
    assert_same_bytes(s, rs, what + " scales")
    assert_same_bytes(q, rq, what + " q")


def data(seed, M, K):
    return wl.randn_bf16(np.random.default_rng(seed), (M, K), 0.02, 0.003, 8.0)


TEAM_MAX = [None, 1]      # the library's limit, then every tall group through maxima tiles


# The first row count of each tiling step has the most tiles per row: 29 rows
# (2048-column strips), 57 (1024), 113 (512), 225 (256), 449 (128), then
# 896 * (c - 1) + 1 rows for a group cut into c chunks (897: two); 81, 161,
# 321 and 641 are the first rows held in LDS on 1024- to 128-column strips.
# K values leave a ragged last strip. Launches with fewer tiles than compute
# units get narrower strips, which the grid bound covers as well.
@pytest.mark.parametrize("team_max", TEAM_MAX)
@pytest.mark.parametrize("size,n,K", [
    (113, 12, 2056), (225, 12, 1032), (449, 8, 520), (897, 6, 264), (1793, 3, 264),
    (2689, 2, 136), (896, 4, 264), (1792, 3, 136), (112, 10, 1032),
    (81, 12, 2056), (161, 12, 1032), (321, 10, 520), (641, 8, 264), (1281, 4, 264),
    (1921, 3, 136), (5121, 2, 264), (5121, 3, 72), (37, 16, 4104), (577, 4, 264),
    (865, 3, 136), (640, 5, 264), (1280, 3, 136),
    (29, 100, 8200), (57, 60, 4104), (28, 90, 8200), (1, 300, 8200),
])
def test_most_tiles_per_row(size, n, K, team_max):
    off = (np.arange(1, n + 1) * size).astype(np.int32)
    x = data(size + n, size * n, K)
    check(x, off, "groups of %d rows" % size, team_max=team_max)


# Tiles whose rows run past the 20 register slabs into the LDS slabs, for
# every strip width (tests/lds_row_cases.py, whose strips a CPU test checks),
# and on one 8-column strip.
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("K,sizes", [(K, sizes) for K, sizes, _ in lds_row_cases.DIM0] +
                         [(8, [700, 896, 1])])
def test_rows_held_in_lds(K, sizes, pow2):
    off = np.cumsum(sizes).astype(np.int32)
    x = data(sum(sizes) + K, int(off[-1]), K)
    check(x, off, "LDS rows K=%d %s" % (K, sizes[-6:]), pow2)


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
def test_tall_groups_without_the_wait(M, K, sizes, team_max):
    off = np.cumsum(sizes).astype(np.int32)
    x = data(M + K, M, K)
    check(x, off, "no wait %s" % (sizes,), team_max=team_max, spin=-1)
    check(x, off, "zero wait %s" % (sizes,), team_max=team_max, spin=0)


# One group in one to three rounds of tiles (by the grid bound) runs as one
# resident round of workgroups, each walking its tiles: (16640, 4096) gives
# 608 tiles (1216 with a team limit of 4), and (30000, 2048) 544. A 19-chunk
# team straddles the first round (tiles 494-512); with a team limit of 4
# the column-maximum tiles come first and the casting tiles wait for maxima
# written in the same or an earlier pass of the resident workgroups. Two
# and three groups take the usual one workgroup per tile.
@pytest.mark.parametrize("team_max", [None, 4])
@pytest.mark.parametrize("M,K,sizes", [(16640, 4096, [16640]), (30000, 2048, [30000]),
                                       (16640, 4096, [6000, 10640]), (16640, 4096, [0, 9000, 7640])])
def test_resident_grid_launches(M, K, sizes, team_max):
    off = np.cumsum(sizes).astype(np.int32)
    x = data(len(sizes) + M // 1000, M, K)
    check(x, off, "resident grid %s" % (sizes,), team_max=team_max)


@pytest.mark.parametrize("team_max", TEAM_MAX)
def test_back_to_back_tall_calls_on_one_stream_and_two(team_max):
    M, K = 13000, 264
    off = np.array([300, 12000, 13000], np.int32)
    xs = [data(20 + i, M, K) for i in range(3)]
    o = to_dev(off)
    ws = mgs.dim0_workspace(M, K)
    outs = []
    # three calls queued without a host sync between them: each must use its
    # own column maxima, not the previous call's
    for x in xs:
        q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
        s = torch.empty((len(off), K), dtype=torch.float32, device="cuda")
        if team_max is None:
            mgs.mgs_quant_groups_dim0(to_dev(x), o, q=q, scales=s)
        else:
            mgs.api._test_quant_dim0(to_dev(x), o, q, s, team_max=team_max, workspace=ws)
        outs.append((q, s))
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


def _replays_match_oracle(g, xd, q, sc, xs, off, order, between=None):
    for i in order:
        xd.copy_(to_dev(xs[i]))
        q.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rq, rs = oracle.quant_groups_dim0(xs[i], off)
        assert_same_bytes(sc.cpu().numpy(), rs, "replay %d scales" % i)
        assert_same_bytes(q.cpu().numpy(), rq, "replay %d q" % i)
        if between is not None:
            between()


def test_graph_replays_with_the_library_workspace():
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

    def eager_between():
        # an eager call on the capturing stream between replays
        with torch.cuda.stream(s):
            qe, se = mgs.mgs_quant_groups_dim0(xd, od)
        torch.cuda.synchronize()
        assert torch.equal(qe, q) and torch.equal(se, sc)

    _replays_match_oracle(g, xd, q, sc, xs, off, (0, 1, 2, 1), eager_between)


def test_graph_keeps_its_workspace_when_the_stream_grows_its_own():
    """A graph captured on a stream keeps working after a later, larger eager
    call on that stream replaces the stream's workspace: the old buffer stays
    alive, and the workspace protocol needs nothing from the host."""
    M, K = 11000, 136
    off = np.array([200, 10600, 11000], np.int32)
    xs = [data(50 + i, M, K) for i in range(2)]
    s = torch.cuda.Stream()
    xd, od = to_dev(xs[0]), to_dev(off)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty((len(off), K), dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        mgs.mgs_quant_groups_dim0(xd, od, q=q, scales=sc)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        mgs.mgs_quant_groups_dim0(xd, od, q=q, scales=sc)
    torch.cuda.synchronize()
    big = data(59, 3 * M, K)
    big_off = np.array([300, 3 * M - 500, 3 * M], np.int32)

    def bigger_eager_call():
        with torch.cuda.stream(s):
            qb, sb = mgs.mgs_quant_groups_dim0(to_dev(big), to_dev(big_off))
        torch.cuda.synchronize()
        rq, rs = oracle.quant_groups_dim0(big, big_off)
        assert_same_bytes(sb.cpu().numpy(), rs, "larger eager call scales")
        assert_same_bytes(qb.cpu().numpy(), rq, "larger eager call q")

    _replays_match_oracle(g, xd, q, sc, xs, off, (0,), bigger_eager_call)
    _replays_match_oracle(g, xd, q, sc, xs, off, (1, 0, 1))


@pytest.mark.parametrize("team_max", TEAM_MAX)
def test_graph_capture_with_a_caller_workspace_needs_no_eager_call(team_max):
    """With a caller-owned workspace the call allocates nothing, so it can be
    captured on a stream that never ran it; replays interleave with eager
    calls on the same workspace."""
    M, K = 9000, 264
    off = np.array([0, 8000, 9000], np.int32)
    xs = [data(60 + i, M, K) for i in range(3)]
    ws = mgs.dim0_workspace(M, K)
    s = torch.cuda.Stream()
    xd, od = to_dev(xs[0]), to_dev(off)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    sc = torch.empty((len(off), K), dtype=torch.float32, device="cuda")

    def call(x, qq, ss):
        if team_max is None:
            mgs.mgs_quant_groups_dim0(x, od, q=qq, scales=ss, workspace=ws)
        else:
            mgs.api._test_quant_dim0(x, od, qq, ss, team_max=team_max, workspace=ws)

    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(xd, q, sc)
    torch.cuda.synchronize()

    def eager_between():
        with torch.cuda.stream(s):
            qe = torch.empty_like(q)
            se = torch.empty_like(sc)
            call(xd, qe, se)
        torch.cuda.synchronize()
        assert torch.equal(qe, q) and torch.equal(se, sc)

    _replays_match_oracle(g, xd, q, sc, xs, off, (0, 1, 2, 0), eager_between)


@pytest.mark.parametrize("team_max,spin", [(None, None), (1, None), (None, -1), (1, -1), (None, 0)])
def test_every_call_leaves_the_workspace_zero(team_max, spin):
    """The invariant the exchange of column maxima rests on: a zero-filled
    workspace is zero again after every call (each team's last tile clears
    its counter and words), on the team path, the column-maximum path and
    the paths where tiles stop waiting, for calls of different shapes sharing
    one workspace, dim0 and dim0_t alike."""
    ws = mgs.dim0_workspace(13000, 520)
    cases = [(13000, 520, [300, 12000, 13000]), (5000, 136, [100, 4000, 5000]),
             (2000, 264, [641, 1300, 2000]), (12800, 520, [6400, 6400, 12800]),
             (1504, 512, [1504])]       # a launch small enough to narrow strips to 64 columns
    for M, K, off in cases:
        off = np.array(off, np.int32)
        x = data(M + K, M, K)
        check(x, off, "(%d, %d)" % (M, K), team_max=team_max, spin=spin, workspace=ws)
        assert int(torch.count_nonzero(ws).item()) == 0, "workspace left dirty after (%d, %d)" % (M, K)
        if M % 16 == 0:
            off = (off // 16 * 16).astype(np.int32)      # dim0_t: group ends on the 16-row grid
            q_t = torch.empty((K, M), dtype=torch.uint8, device="cuda")
            s_t = torch.empty((K, len(off)), dtype=torch.float32, device="cuda")
            mgs.api._test_quant_dim0(to_dev(x), to_dev(off), q_t, s_t, transposed=True,
                                     spin_ticks=mgs.api.TEST_DEFAULT_SPIN if spin is None else spin,
                                     team_max=mgs.api.TEST_DEFAULT_TEAM if team_max is None else team_max,
                                     workspace=ws)
            torch.cuda.synchronize()
            rq, rs = oracle.quant_groups_dim0_t(x, off)
            assert_same_bytes(s_t.cpu().numpy(), rs, "dim0_t (%d, %d) scales_t" % (M, K))
            assert_same_bytes(q_t.cpu().numpy(), rq, "dim0_t (%d, %d) q_t" % (M, K))
            assert int(torch.count_nonzero(ws).item()) == 0, "dim0_t left the workspace dirty"


def test_teams_while_another_kernel_holds_the_cus():
    """A call whose one group is cut into 19-chunk teams, queued while copy
    kernels run on a second stream and hold CUs: teams are only guaranteed
    to be resident when whole teams fit in what the other work leaves free.
    The output must be exact, and the call must end far below the 20 ms
    bound on a tile's wait."""
    from oracle_pool import check_dim0_whole
    M, K = 16640, 8192
    off = np.array([M], np.int32)
    x = data(80, M, K)
    xd, od = to_dev(x), to_dev(off)
    q = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    s = torch.empty((1, K), dtype=torch.float32, device="cuda")
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    mgs.mgs_quant_groups_dim0(xd, od, q=q, scales=s)       # the stream's workspace exists
    side = torch.cuda.Stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    worst = 0.0
    for _ in range(3):
        q.fill_(0)
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            for _ in range(4):
                mgs.mgs_copy(src, dst)
        t0.record()
        mgs.mgs_quant_groups_dim0(xd, od, q=q, scales=s)
        t1.record()
        torch.cuda.synchronize()
        worst = max(worst, t0.elapsed_time(t1))
    check_dim0_whole(x, off, False, q.cpu().numpy(), s.cpu().numpy(), "teams beside copies")
    assert worst < 5.0, "dim0 beside copy kernels took %.2f ms" % worst
