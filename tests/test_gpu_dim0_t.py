"""GPU parity of the transposed dim0 entry point (mgs_quant_groups_dim0_t):
q_t (K, M) and scales_t (K, G) against the oracle byte for byte, over every
strip class (1024- down to 128-column strips, K narrower than a strip,
ragged last strips), tiles with rows held in LDS on every strip width,
empty groups, chunk teams and column-maximum tiles,
the path that computes the maxima in the waiting tile itself, pow2 scales,
the benchmark shape compared whole, and offsets that are not multiples
of 16 (values unspecified, writes in bounds). Every output carries guard
bands."""
import numpy as np
import pytest
import torch

import oracle
import group_scaling_fp8_amd as mgs
from group_scaling_fp8_amd import workloads as wl
from gpu_util import Guarded, assert_same_bytes, to_dev
from oracle_pool import check_dim0_t_whole
import lds_row_cases

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mgs.lib()


def run_dim0_t(x, off, pow2=False):
    M, K = x.shape
    gq, gs = Guarded((K, M), torch.uint8), Guarded((K, len(off)), torch.float32)
    mgs.mgs_quant_groups_dim0_t(to_dev(x), to_dev(off), pow2, q_t=gq.view, scales_t=gs.view)
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    return gq.numpy(), gs.numpy()


def check(x, off, what, pow2=False):
    q, s = run_dim0_t(x, off, pow2)
    rq, rs = oracle.quant_groups_dim0_t(x, off, pow2)
    assert_same_bytes(s, rs, what + " scales_t")
    assert_same_bytes(q, rq, what + " q_t")


def data(seed, M, K):
    return wl.randn_bf16(np.random.default_rng(seed), (M, K), 0.02, 0.003, 8.0)


@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("K,sizes", [
    (264, [16, 48, 0, 80, 160, 256, 320, 336, 640, 656, 896]),   # every strip width up to K, ragged K
    (520, [912, 16, 1808]),                            # two- and three-chunk teams
    (8, [32, 0, 704, 16]),                             # one 8-column strip
    (72, [320, 336, 16]),                              # K narrower than a strip
    (1032, [208, 400, 96]),
    (2056, [16, 64, 80, 0, 144, 32, 112, 224, 448]),   # 1024- and 512-column strips
])
def test_dim0_t_classes(K, sizes, pow2):
    off = np.cumsum(sizes).astype(np.int32)
    M = int(off[-1])
    check(data(M + K, M, K), off, "sizes %s K=%d" % (sizes, K), pow2)


# Tiles whose rows run past the registers into LDS (cast there, then staged
# before the register rows), on every strip width of the transposed kernel
# (tests/lds_row_cases.py, whose strips a CPU test checks).
@pytest.mark.parametrize("pow2", [False, True])
@pytest.mark.parametrize("K,sizes", [(K, sizes) for K, sizes, _ in lds_row_cases.DIM0_T])
def test_dim0_t_rows_held_in_lds(K, sizes, pow2):
    off = np.cumsum(sizes).astype(np.int32)
    M = int(off[-1])
    check(data(M + K, M, K), off, "LDS rows K=%d %s" % (K, sizes[-5:]), pow2)


# Tall groups whose chunk boundaries move onto 128-row lines (the last chunk
# still fits a tile) or stay at multiples of the chunk size from the group
# start (it would not), for group starts off the 128-row grid; as teams and,
# with a team limit of 1, as column-maximum tiles.
@pytest.mark.parametrize("team_max", [None, 1])
@pytest.mark.parametrize("sizes", [
    [16, 1808, 16],          # three chunks on lines: 624, 640, 544 rows
    [80, 4000, 48],          # five chunks on lines, the first 816 rows
    [16, 1792, 16],          # two full chunks from an unaligned start
    [48, 2688, 16],          # three full chunks from an unaligned start
    [128, 1008, 16],         # an aligned start: 512 + 496
])
def test_dim0_t_chunk_boundaries(sizes, team_max):
    off = np.cumsum(sizes).astype(np.int32)
    M, K = int(off[-1]), 264
    x = data(M + len(sizes), M, K)
    if team_max is None:
        check(x, off, "chunks %s" % (sizes,))
        return
    gq, gs = Guarded((K, M), torch.uint8), Guarded((K, len(off)), torch.float32)
    mgs.api._test_quant_dim0(to_dev(x), to_dev(off), gq.view, gs.view, transposed=True,
                             spin_ticks=mgs.api.TEST_DEFAULT_SPIN, team_max=team_max,
                             workspace=mgs.dim0_workspace(M, K))
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    rq, rs = oracle.quant_groups_dim0_t(x, off)
    assert_same_bytes(gs.numpy(), rs, "chunks %s team_max=1 scales_t" % (sizes,))
    assert_same_bytes(gq.numpy(), rq, "chunks %s team_max=1 q_t" % (sizes,))


def test_dim0_t_no_rows_writes_scales():
    x = np.zeros((0, 64), np.uint16)
    off = np.zeros(3, np.int32)
    q, s = run_dim0_t(x, off)
    rq, rs = oracle.quant_groups_dim0_t(x, off)
    assert q.shape == (64, 0)
    assert_same_bytes(s, rs, "scales_t of empty groups")


@pytest.mark.parametrize("team_max,spin", [(1, mgs.api.TEST_DEFAULT_SPIN),
                                           (mgs.api.TEST_DEFAULT_TEAM, -1)])
def test_dim0_t_tall_groups_other_paths(team_max, spin):
    # column-maximum tiles (team limit 1), then the in-tile fallback (no wait),
    # through the test-only entry point
    sizes = [1296, 16, 2000]
    off = np.cumsum(sizes).astype(np.int32)
    x = data(5, int(off[-1]), 136)
    M, K = x.shape
    gq, gs = Guarded((K, M), torch.uint8), Guarded((K, len(off)), torch.float32)
    mgs.api._test_quant_dim0(to_dev(x), to_dev(off), gq.view, gs.view, transposed=True,
                             spin_ticks=spin, team_max=team_max, workspace=mgs.dim0_workspace(M, K))
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    rq, rs = oracle.quant_groups_dim0_t(x, off)
    what = "tall groups team_max=%s spin=%s" % (team_max, spin)
    assert_same_bytes(gs.numpy(), rs, what + " scales_t")
    assert_same_bytes(gq.numpy(), rq, what + " q_t")


def test_dim0_t_at_the_benchmark_shape_whole(token_major):
    """(16640, 8192) G=64, the benchmark's offsets: every byte of q_t and
    every scale against the oracle, and against dim0's outputs transposed."""
    T = token_major
    off = wl.target_offsets(64)
    xt, ot = to_dev(T), to_dev(off)
    q0, s0 = mgs.mgs_quant_groups_dim0(xt, ot)
    qt, st = mgs.mgs_quant_groups_dim0_t(xt, ot)
    torch.cuda.synchronize()
    assert torch.equal(qt, q0.t().contiguous()), "q_t differs from dim0's q transposed"
    assert torch.equal(st.view(torch.int32), s0.t().contiguous().view(torch.int32))
    check_dim0_t_whole(T, off, False, qt.cpu().numpy(), st.cpu().numpy(), "dim0_t (16640, 8192) G=64")


def test_dim0_t_unaligned_offsets_stay_in_bounds():
    """Offsets off the 16-row grid (and unsorted ones) give unspecified values
    but no write outside the outputs."""
    x = data(7, 320, 136)
    for off in ([100, 37, 320], [5, 320], [-3, 400, 320], [320]):
        run_dim0_t(x, np.array(off, np.int32))


# K a multiple of 8 times the widest strip: the tiles are dealt to the XCDs
# by column range (each XCD the tiling of K / 8 columns), teams included
@pytest.mark.parametrize("team_max", [None, 1])
@pytest.mark.parametrize("K,sizes", [
    (8192, [0, 1600, 48, 1552, 16]),          # 3-chunk teams, an empty group, short groups
    (16384, [96, 704, 0, 320]),               # 2-chunk team, 1024- to 128-column strips
    (8192, [2048]),                           # one group, one 4-chunk team per strip
])
def test_dim0_t_tiles_by_column_range(K, sizes, team_max):
    off = np.cumsum(sizes).astype(np.int32)
    M = int(off[-1])
    x = data(M + K, M, K)
    if team_max is None:
        check(x, off, "column ranges %s K=%d" % (sizes, K))
        return
    gq, gs = Guarded((K, M), torch.uint8), Guarded((K, len(off)), torch.float32)
    mgs.api._test_quant_dim0(to_dev(x), to_dev(off), gq.view, gs.view, transposed=True,
                             team_max=team_max, workspace=mgs.dim0_workspace(M, K))
    torch.cuda.synchronize()
    gq.check()
    gs.check()
    rq, rs = oracle.quant_groups_dim0_t(x, off)
    assert_same_bytes(gs.numpy(), rs, "column ranges, team limit 1, scales_t")
    assert_same_bytes(gq.numpy(), rq, "column ranges, team limit 1, q_t")
