"""CPU check of the dim0 grid bound (mgs_dim0_layout.hpp).

The dim0 launch has one workgroup per tile and sizes its grid from (M, K, G)
alone, so the bound must hold for every way of splitting M rows into G
groups. The tile count of a group depends only on its row count, as a step
function, so the worst split is found exactly by a knapsack over the first
row count of each step (0, L/32 + 1, L/16 + 1, L/8 + 1, L/4 + 1, L/2 + 1,
then C * (c - 1) + 1 for the groups cut into c >= 2 chunks, with C = 896
the chunk rows of both kernels and L the rows at which strip widths step:
896 in the dim0 kernel, 640 in the transposed one, whose strips are also at
most 1024 columns wide against 4096). The C++ bound, compiled with g++ from
the header the library uses, must be at least that worst case, for several
team limits (the most chunks a group may have to be cast as a team)."""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "group_scaling_fp8_amd", "csrc")

BOUND_PROGRAM = r"""
#include <stdio.h>
#include "mgs_dim0_layout.hpp"
int main() {
    long long M, K, G, T, L, C, LR, X;
    while (scanf("%lld %lld %lld %lld %lld %lld %lld %lld", &M, &K, &G, &T, &L, &C, &LR, &X) == 8) {
        if (L < 0) {   // the strip-width cap for a device of -L compute units, widest 8 << X
            printf("%d\n", mgs::dim0_lt_cap(M, K, G, T, -L, C, LR, (int)X));
            continue;
        }
        printf("%lld %lld %lld\n", (long long)mgs::dim0_tile_bound(M, K, G, T, (int)L, C, LR),
               (long long)mgs::dim0_chunk_bound(M, C),
               (long long)mgs::dim0_group_tiles(M, K, T, (int)L, C, LR));
    }
    return 0;
}
"""


C896 = 896
# (chunk rows, rows at which strip widths step, widest strips) of the dim0
# and dim0_t kernels: strips of at most 4096 and 1024 columns
KERNELS = [(896, 896, 9), (896, 640, 7)]


def group_lt(R, C=896, LR=None):
    """Strip width of a group of R rows before any cap (the rule of the
    kernel's tile search): strips of 8 << lt columns."""
    LR = C if LR is None else LR
    if R > LR // 2:
        return 4
    return (9 if R <= LR // 32 else 8 if R <= LR // 16 else 7 if R <= LR // 8 else
            6 if R <= LR // 4 else 5)


def tiles(R, K, team_max, max_lt=7, C=896, LR=None):
    """Tiles of one group of R rows (the rule of the kernel's tile search),
    with strips at most 8 << max_lt columns wide, chunks of C rows and strip
    widths stepping at LR / 2^k rows."""
    chunks = -(-R // C) if R > C else 0
    lt = min(group_lt(R, C, LR), max_lt)
    while lt > 3 and (8 << (lt - 1)) >= K:
        lt -= 1
    ns = -(-K // (8 << lt))
    if chunks == 0:
        return ns
    return (1 if chunks <= team_max else 2) * chunks * ns


def worst_splits(Mmax, K, Gmax, team_max, max_lt=7, C=896, LR=None):
    """best[G][M] = the most tiles over all splits of at most M rows into
    exactly G groups."""
    LR = C if LR is None else LR
    sizes = [0, LR // 32 + 1, LR // 16 + 1, LR // 8 + 1, LR // 4 + 1, LR // 2 + 1] + \
        [C * (c - 1) + 1 for c in range(2, Mmax // C + 3)]
    sizes = [r for r in sizes if r <= Mmax]
    NEG = -(1 << 40)
    dp = np.full(Mmax + 1, NEG, np.int64)
    dp[0] = 0
    best = [np.maximum.accumulate(dp)]
    for _ in range(Gmax):
        nxt = np.full(Mmax + 1, NEG, np.int64)
        for r in sizes:
            t = tiles(r, K, team_max, max_lt, C, LR)
            np.maximum(nxt[r:], dp[:Mmax + 1 - r] + t, out=nxt[r:])
        dp = nxt
        best.append(np.maximum.accumulate(dp))
    return best


@pytest.fixture(scope="module")
def bound_tool():
    d = tempfile.mkdtemp(prefix="mgs_bound_")
    src = os.path.join(d, "bound.cpp")
    exe = os.path.join(d, "bound")
    with open(src, "w") as f:
        f.write(BOUND_PROGRAM)
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", CSRC, "-o", exe, src], check=True)

    def run(triples):
        inp = "".join("%d %d %d %d %d %d %d %d\n" % (tuple(t) + (7, 896, 896, 9)[len(t) - 4:])
                      for t in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in line.split()) for line in out.splitlines()]
    return run


@pytest.mark.parametrize("C,LR,lt", KERNELS)
@pytest.mark.parametrize("team_max", [1, 3, 26, 128])
@pytest.mark.parametrize("K", [8, 64, 72, 136, 1032, 2056, 4104, 8192])
def test_bound_covers_the_worst_split(bound_tool, K, team_max, C, LR, lt):
    Mmax, Gmax = 17000, 64
    best = worst_splits(Mmax, K, Gmax, team_max, lt, C, LR)
    Ms = [0, 1, 20, 21, 28, 29, 40, 41, 56, 57, 80, 81, 113, 400, 449, 640, 641, 896, 897, 1280, 1281,
          1793, 1921, 5120, 5121, 6000, 10242, 12000, 16640, 17000]
    Gs = [1, 2, 3, 7, 16, 64]
    triples = [(M, K, G, team_max, lt, C, LR) for M in Ms for G in Gs]
    got = bound_tool(triples)
    for (M, _, G, _, _, _, _), (b, _, one) in zip(triples, got):
        exact = int(best[G][M])
        assert b >= exact, (M, K, G, team_max, C, LR, b, exact)
        # and it is no wild over-estimate (the grid's extra workgroups exit at once)
        assert 2 * b <= 3 * exact + 32, (M, K, G, team_max, C, LR, b, exact)
        assert one == tiles(M, K, team_max, lt, C, LR)


@pytest.mark.parametrize("LR", [896, 640])
@pytest.mark.parametrize("max_lt", [3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("K", [64, 1032, 4096, 8200])
def test_bound_with_narrowed_strips(bound_tool, K, max_lt, LR):
    C = C896
    team_max = 128
    Mmax, Gmax = 17000, 64
    best = worst_splits(Mmax, K, Gmax, team_max, max_lt, C, LR)
    Ms = [0, 1, 20, 21, 29, 41, 57, 80, 81, 113, 161, 225, 321, 449, 640, 641, 897, 1281, 4096, 6000,
          16640, 17000]
    Gs = [1, 2, 4, 16, 64]
    triples = [(M, K, G, team_max, max_lt, C, LR) for M in Ms for G in Gs]
    got = bound_tool(triples)
    for (M, _, G, _, _, _, _), (b, _, one) in zip(triples, got):
        exact = int(best[G][M])
        assert exact <= b and 2 * b <= 3 * exact + 32, (M, K, G, max_lt, C, LR, b, exact)
        assert one == tiles(M, K, team_max, max_lt, C, LR)


def test_strip_cap_policy(bound_tool):
    """Tiny problems get strips narrow enough for one tile per CU (256 CUs);
    every other shape keeps the widest strips the group sizes call for (up
    to 4096 columns in the dim0 kernel, 1024 in the transposed one), and K
    alone still caps the width. Expected caps: (dim0, dim0_t)."""
    cases = [((4096, 4096, 16), (9, 7)), ((256, 4096, 4), (3, 3)), ((1024, 2048, 4), (3, 3)),
             ((16640, 8192, 64), (9, 7)), ((65536, 4096, 8), (9, 7)), ((16640, 8192, 1), (9, 7)),
             ((81920, 8192, 16), (9, 7)), ((4096, 64, 16), (3, 3)), ((2048, 8192, 64), (9, 7)),
             ((512, 4096, 8), (4, 4)), ((16384, 2048, 512), (8, 7)), ((1024, 1024, 4), (3, 3))]
    for ci, (C, LR, widest) in enumerate(KERNELS):
        got = bound_tool([(M, K, G, 128, -256, C, LR, widest) for (M, K, G), _ in cases])
        for ((M, K, G), want), (lt,) in zip(cases, got):
            assert lt == want[ci], (M, K, G, C, lt, want)
            # what the rule promises: a tile per CU for equal groups, unless the
            # narrowest strips are reached
            assert lt == 3 or G * tiles(M // G, K, 128, lt, C, LR) >= 256


@pytest.mark.parametrize("C,LR,lt", KERNELS)
def test_bound_of_the_benchmark_shape(bound_tool, C, LR, lt):
    (b, chunks, _), = bound_tool([(16640, 8192, 64, 128, lt, C, LR)])
    exact = int(worst_splits(16640, 8192, 64, 128, lt, C, LR)[64][16640])
    assert exact <= b
    assert chunks == 16640 // C + 16640 // (C + 1)


def test_chunk_bound_covers_every_chunked_split(bound_tool):
    C = C896
    # the chunked groups of any split have at most dim0_chunk_bound(M, C) chunks
    for M in (C + 1, 2 * C + 1, 2 * C + 2, 3 * C, 3 * C + 1, 4 * C + 2, 8 * C + 1, 16 * C + 2, 16640,
              40000):
        (_, chunks, _), = bound_tool([(M, 8, 1, 128, 7, C)])
        worst = 0
        for n in range(1, M // (C + 1) + 1):        # n groups of just over C rows
            rows = M // n
            worst = max(worst, n * math.ceil(rows / C))
        assert chunks >= worst, (M, C, chunks, worst)


@pytest.mark.parametrize("K,max_lt", [(8192, 7), (16384, 7), (4096, 6), (512, 3), (1024, 4)])
def test_xcd_split_tiles_are_eight_copies(bound_tool, K, max_lt):
    """When the transposed kernel deals tiles to the 8 XCDs by column range
    (K / 8 a multiple of the widest strip), every group's tiles are 8 copies
    of the tiles of a K / 8-column problem, so 8 x the bound for K / 8 covers
    the launch."""
    assert K % (64 << max_lt) == 0
    C, LR = C896, 640
    for team_max in (1, 32):
        Rs = [0, 1, 16, 80, 81, 161, 321, 640, 641, 896, 897, 1793, 5121, 20481]
        got = bound_tool([(R, K, 1, team_max, max_lt, C, LR) for R in Rs])
        part = bound_tool([(R, K // 8, 1, team_max, max_lt, C, LR) for R in Rs])
        for R, (_, _, full), (_, _, eighth) in zip(Rs, got, part):
            assert full == 8 * eighth, (R, K, max_lt, team_max, full, eighth)
        for M, G in ((16640, 64), (3200, 3), (20480, 1)):
            (b8, _, _), = bound_tool([(M, K // 8, G, team_max, max_lt, C, LR)])
            exact = int(worst_splits(M, K, G, team_max, max_lt, C, LR)[G][M])
            assert 8 * b8 >= exact, (M, K, G, team_max, b8, exact)


@pytest.mark.parametrize("LR,widest,cases", [(896, 9, "DIM0"), (640, 7, "DIM0_T")])
def test_lds_row_cases_reach_their_strips(bound_tool, LR, widest, cases):
    """The GPU tests of rows held in LDS run on the strips they name: the
    launch's strip cap lets its repeated group keep strips of 8 << lt
    columns, and that group (and at least one other) lies in the LDS range
    of those strips."""
    import lds_row_cases
    for K, sizes, lt in getattr(lds_row_cases, cases):
        M, G = sum(sizes), len(sizes)
        (cap,), = bound_tool([(M, K, G, 128, -256, C896, LR, widest)])
        assert cap >= lt and min(group_lt(sizes[0], C896, LR), cap) == lt, (K, lt, cap)
        rps = 512 >> lt
        in_lds = [R for R in sizes if min(group_lt(R, C896, LR), cap) == lt and 20 * rps < R <= 28 * rps]
        assert sizes[0] in in_lds and len(set(in_lds)) >= 2, (K, lt, sorted(set(in_lds)))
        if cases == "DIM0_T":
            assert all(R % 16 == 0 for R in sizes)


def chunk_rows(start, R, C, row_align, line):
    """The chunks [r0, r1) of a group of R > C rows starting at row start, as
    the kernels' tile search cuts them: nc = ceil(R / C) chunks of R / nc rows
    rounded up to max(row_align, line); with line > 1 (the transposed kernel,
    128) the boundaries move down to multiples of line when the last chunk
    still fits."""
    nc = -(-R // C)
    align = max(line, row_align)
    cs = -(-(-(-R // nc)) // align) * align
    s0 = start
    if line > 1:
        lead = start % line
        if R + lead - (nc - 1) * cs <= C:
            s0 = start - lead
    g1 = start + R
    out = []
    for c in range(nc):
        r0 = start if c == 0 else min(s0 + c * cs, g1)
        r1 = g1 if c == nc - 1 else min(s0 + (c + 1) * cs, g1)
        out.append((r0, r1))
    return out


@pytest.mark.parametrize("line,row_align", [(1, 1), (128, 16)])
def test_chunks_cover_the_group(line, row_align):
    """Chunks partition the group's rows, none is empty or holds more than a
    tile's C = 896 rows; with 128-row lines every inner boundary of a group
    whose start is on the 16-row grid lies on a multiple of 128 whenever
    that keeps the last chunk within C rows, and always on one for groups
    starting on a line."""
    C = 896
    rng = np.random.default_rng(5)
    Rs = list(range(C + 1, 4 * C + 200, 7)) + [16640, 16640 - 16, 120000, 2080, 8320]
    for R in Rs:
        R = R // row_align * row_align
        if R <= C:
            continue
        for start in [0, 16, 112, 128, 4096 + 48] + [int(v) * row_align for v in rng.integers(0, 1000, 4)]:
            ch = chunk_rows(start, R, C, row_align, line)
            assert ch[0][0] == start and ch[-1][1] == start + R
            for (a, b), (c2, _) in zip(ch, ch[1:]):
                assert b == c2
            assert all(0 < b - a <= C for a, b in ch), (start, R, ch)
            assert all(a % row_align == 0 for a, _ in ch)
            if line > 1 and start % line == 0:
                assert all(a % line == 0 for a, _ in ch), (start, R, ch)
