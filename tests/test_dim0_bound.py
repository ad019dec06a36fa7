"""CPU check of the dim0 grid bound (mgs_dim0_layout.hpp).

The dim0 launch has one workgroup per tile and sizes its grid from (M, K, G)
alone, so the bound must hold for every way of splitting M rows into G
groups. The tile count of a group depends only on its row count, as a step
function, so the worst split is found exactly by a knapsack over the first
row count of each step (0, 81, 161, 321, then 640 * (c - 1) + 1 for the
groups cut into c >= 2 chunks). The C++ bound, compiled with g++ from the
header the library uses, must be at least that worst case, for several team
limits (the most chunks a group may have to be cast as a team)."""
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "group_scaling_fp8_amd", "csrc")

DRIVER = r"""
#include <stdio.h>
#include "mgs_dim0_layout.hpp"
int main() {
    long long M, K, G, T, L;
    while (scanf("%lld %lld %lld %lld %lld", &M, &K, &G, &T, &L) == 5) {
        if (L < 0) {   // the strip-width cap for a device of -L compute units
            printf("%d\n", mgs::dim0_lt_cap(M, K, G, T, -L));
            continue;
        }
        printf("%lld %lld %lld\n", (long long)mgs::dim0_tile_bound(M, K, G, T, (int)L),
               (long long)mgs::dim0_chunk_bound(M), (long long)mgs::dim0_group_tiles(M, K, T, (int)L));
    }
    return 0;
}
"""


def tiles(R, K, team_max, max_lt=7):
    """Tiles of one group of R rows (the rule of the kernel's tile search),
    with strips at most 8 << max_lt columns wide."""
    if R > 640:
        lt, chunks = 4, -(-R // 640)
    else:
        lt = 7 if R <= 80 else 6 if R <= 160 else 5 if R <= 320 else 4
        chunks = 0
    lt = min(lt, max_lt)
    while lt > 3 and (8 << (lt - 1)) >= K:
        lt -= 1
    ns = -(-K // (8 << lt))
    if chunks == 0:
        return ns
    return (1 if chunks <= team_max else 2) * chunks * ns


def worst_splits(Mmax, K, Gmax, team_max, max_lt=7):
    """best[G][M] = the most tiles over all splits of at most M rows into
    exactly G groups."""
    sizes = [0, 81, 161, 321] + [640 * (c - 1) + 1 for c in range(2, Mmax // 640 + 3)]
    sizes = [r for r in sizes if r <= Mmax]
    NEG = -(1 << 40)
    dp = np.full(Mmax + 1, NEG, np.int64)
    dp[0] = 0
    best = [np.maximum.accumulate(dp)]
    for _ in range(Gmax):
        nxt = np.full(Mmax + 1, NEG, np.int64)
        for r in sizes:
            t = tiles(r, K, team_max, max_lt)
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
        f.write(DRIVER)
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", CSRC, "-o", exe, src], check=True)

    def run(triples):
        inp = "".join("%d %d %d %d %d\n" % (t + (7,) if len(t) == 4 else t) for t in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(v) for v in line.split()) for line in out.splitlines()]
    return run


@pytest.mark.parametrize("team_max", [1, 3, 26, 128])
@pytest.mark.parametrize("K", [8, 64, 72, 136, 1032, 8192])
def test_bound_covers_the_worst_split(bound_tool, K, team_max):
    Mmax, Gmax = 17000, 64
    best = worst_splits(Mmax, K, Gmax, team_max)
    Ms = [0, 1, 80, 81, 400, 640, 641, 1280, 1281, 1921, 5120, 5121, 6000, 10242, 12000, 16640, 17000]
    Gs = [1, 2, 3, 7, 16, 64]
    triples = [(M, K, G, team_max) for M in Ms for G in Gs]
    got = bound_tool(triples)
    for (M, _, G, _), (b, _, one) in zip(triples, got):
        exact = int(best[G][M])
        assert b >= exact, (M, K, G, team_max, b, exact)
        # and it is no wild over-estimate (the grid's extra workgroups exit at once)
        assert b <= 2 * exact + 16, (M, K, G, team_max, b, exact)
        assert one == tiles(M, K, team_max)


@pytest.mark.parametrize("max_lt", [3, 4, 5, 6])
@pytest.mark.parametrize("K", [64, 1032, 4096])
def test_bound_with_narrowed_strips(bound_tool, K, max_lt):
    team_max = 128
    Mmax, Gmax = 17000, 64
    best = worst_splits(Mmax, K, Gmax, team_max, max_lt)
    Ms = [0, 1, 80, 81, 161, 321, 640, 641, 1281, 4096, 6000, 16640, 17000]
    Gs = [1, 2, 4, 16, 64]
    triples = [(M, K, G, team_max, max_lt) for M in Ms for G in Gs]
    got = bound_tool(triples)
    for (M, _, G, _, _), (b, _, one) in zip(triples, got):
        exact = int(best[G][M])
        assert exact <= b <= 2 * exact + 16, (M, K, G, max_lt, b, exact)
        assert one == tiles(M, K, team_max, max_lt)


def test_strip_cap_policy(bound_tool):
    """Tiny problems get strips narrow enough for one tile per CU (256 CUs);
    every other shape keeps the widest strips the group sizes call for, and
    K alone still caps the width."""
    cases = [((4096, 4096, 16), 7), ((256, 4096, 4), 3), ((1024, 2048, 4), 3), ((16640, 8192, 64), 7),
             ((65536, 4096, 8), 7), ((16640, 8192, 1), 7), ((81920, 8192, 16), 7),
             ((4096, 64, 16), 3), ((2048, 8192, 64), 7), ((512, 4096, 8), 4)]
    got = bound_tool([(M, K, G, 128, -256) for (M, K, G), _ in cases])
    for ((M, K, G), want), (lt,) in zip(cases, got):
        assert lt == want, (M, K, G, lt, want)
        # what the rule promises: a tile per CU for equal groups, unless the
        # narrowest strips are reached
        assert lt == 3 or G * tiles(M // G, K, 128, lt) >= 256


def test_bound_of_the_benchmark_shape(bound_tool):
    (b, chunks, _), = bound_tool([(16640, 8192, 64, 128)])
    exact = int(worst_splits(16640, 8192, 64, 128)[64][16640])
    assert exact <= b
    assert chunks == 16640 // 640 + 16640 // 641


def test_chunk_bound_covers_every_chunked_split(bound_tool):
    # the chunked groups of any split have at most dim0_chunk_bound(M) chunks
    for M in (641, 1281, 1282, 1920, 1921, 2562, 5121, 10242, 10243, 16640, 40000):
        (_, chunks, _), = bound_tool([(M, 8, 1, 128)])
        worst = 0
        for n in range(1, M // 641 + 1):            # n groups of just over 640 rows
            rows = M // n
            worst = max(worst, n * math.ceil(rows / 640))
        assert chunks >= worst, (M, chunks, worst)
