// mgs_dim0_layout.hpp — dim0 tiling constants, the grid bound and the
// workspace layout (host code with no HIP dependency).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mgs {

// dim0 tiling: 512-thread workgroups holding kDim0Slabs 16-byte vectors per
// thread; groups taller than kDim0HugeRows are cut into chunks of at most
// kDim0HugeChunkRows rows whose column maxima go through a workspace.
constexpr int kDim0Slabs = 20;
constexpr int kDim0HugeRows = 5120;
constexpr int kDim0HugeChunkRows = 640;
// Largest dim0 grid launched at once; past it the workgroups loop.
constexpr int64_t kDim0MaxGrid = int64_t(1) << 22;

// Upper bound on the chunks of groups taller than kDim0HugeRows: a group of
// s rows has ceil(s / 640) <= floor(s / 640) + 1 chunks, and there are at
// most M / 5121 such groups.
inline int64_t dim0_huge_chunk_bound(int64_t M) {
    if (M <= kDim0HugeRows) return 0;
    return M / kDim0HugeChunkRows + M / (kDim0HugeRows + 1);
}

// Upper bound on the dim0 tiles for any offsets, from (M, K, G) alone.
//
// A group of R rows gets n(w) = ceil(K / w) tiles, w being its strip width:
// 1024 columns for R <= 80, 512 up to 160, 256 up to 320, 128 up to 640 and
// 64 up to 5120. A taller group gets 2 * n(128) * ceil(R / 640) tiles (one
// column-maximum tile and one casting tile per chunk and strip). So every
// group has n(1024) tiles plus at most rho * R more, where rho is the largest
// (tiles - n(1024)) / R over the first row count of each step (for the tall
// groups the ratio falls as R grows, so 5121 rows is the worst). The rows of
// all groups add up to at most M, hence
//     tiles <= G * n(1024) + floor(rho * M).
// No group has more tiles than one group of all M rows at its widest step
// would have, so tiles <= G * that as well; the bound is the smaller of the
// two.
inline int64_t dim0_tile_bound(int64_t M, int64_t K, int64_t G) {
    auto n = [K](int64_t w) { return (K + w - 1) / w; };
    const int64_t base = n(1024);
    const int64_t num[5] = {n(512) - base, n(256) - base, n(128) - base, n(64) - base,
                            18 * n(128) - base};
    const int64_t den[5] = {81, 161, 321, 641, kDim0HugeRows + 1};
    const int steps = M > kDim0HugeRows ? 5 : 4;
    int64_t extra = 0;
    for (int i = 0; i < steps; ++i) {
        const int64_t e = M * num[i] / den[i];
        if (e > extra) extra = e;
    }
    // most tiles of a single group of at most M rows
    int64_t one = base;
    const int64_t first_rows[4] = {81, 161, 321, 641};
    const int64_t step_tiles[4] = {n(512), n(256), n(128), n(64)};
    for (int i = 0; i < 4; ++i)
        if (M >= first_rows[i] && step_tiles[i] > one) one = step_tiles[i];
    if (M > kDim0HugeRows) {
        const int64_t tall = 2 * n(128) * ((M + kDim0HugeChunkRows - 1) / kDim0HugeChunkRows);
        if (tall > one) one = tall;
    }
    const int64_t spread = G * base + extra;
    return spread < G * one ? spread : G * one;
}

// dim0 workspace (needed only when M > kDim0HugeRows), 256-byte aligned
// regions: an epoch word, then the column maxima of every chunk, one 64-bit
// word per column pair (generation << 32 | two 16-bit magnitude patterns).
struct Dim0Workspace {
    int64_t chunks;
    size_t epoch_off, max_off, bytes;
};

inline Dim0Workspace dim0_workspace(int64_t M, int64_t K) {
    Dim0Workspace w;
    w.chunks = dim0_huge_chunk_bound(M);
    w.epoch_off = 0;
    w.max_off = 256;
    w.bytes = w.max_off + (size_t)(w.chunks * (K / 2)) * sizeof(uint64_t);
    return w;
}

}  // namespace mgs
