// mgs_dim0_layout.hpp — dim0 tiling constants, the grid bound and the
// workspace layout (host code with no HIP dependency).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mgs {

// dim0 tiling: 512-thread workgroups holding 16-byte vectors of the tile,
// per thread: in the plain dim0 kernel kDim0Slabs in registers (10240
// vectors, 160 KiB of bf16) and kDim0LdsSlabs more in LDS (4096 vectors,
// 64 KiB); in the transposed kernel kDim0SlabsT in registers and none in
// LDS (its LDS holds the output stage). A group of at most chunk_rows rows
// (the rows of a full 128-column tile: 896 for dim0, 640 for dim0_t) is one
// tile per column strip. A taller group is cut into chunks of at most
// chunk_rows rows on 128-column strips: a team of chunk tiles per strip when
// the chunk count is at most the team limit, else a column-maximum tile and
// a casting tile per chunk and strip.
constexpr int kDim0Slabs = 20;
constexpr int kDim0LdsSlabs = 8;
constexpr int kDim0SlabsT = 20;
constexpr int kDim0ChunkRows = (kDim0Slabs + kDim0LdsSlabs) * 512 / 16;   // 896
constexpr int kDim0ChunkRowsT = kDim0SlabsT * 512 / 16;                    // 640
// Upper limit on the chunk count of a team (the library also keeps it at
// most the CU count, so that a team fits among the resident workgroups).
constexpr int kDim0MaxTeam = 128;
// Largest dim0 grid launched at once; past it the workgroups loop.
constexpr int64_t kDim0MaxGrid = int64_t(1) << 22;

// Upper bound on the chunks of all chunked groups: a group of s > C rows
// (C = chunk_rows) has ceil(s / C) <= floor(s / C) + 1 chunks, and there are
// at most M / (C + 1) such groups.
inline int64_t dim0_chunk_bound(int64_t M, int64_t chunk_rows) {
    if (M <= chunk_rows) return 0;
    return M / chunk_rows + M / (chunk_rows + 1);
}

// Tiles of one group of R rows (the rule of the kernel's tile search), with
// C = chunk_rows: n(w) = ceil(K / w') strips of width w' = min(w, 8 << max_lt)
// with w = 4096 columns for R <= C/32, 2048 up to C/16, 1024 up to C/8, 512
// up to C/4, 256 up to C/2 and 128 up to C. A taller group has c = ceil(R / C) chunks on n(128) strips:
// c * n(128) tiles as a team (c <= team_max), else 2 * c * n(128).
inline int64_t dim0_group_tiles(int64_t R, int64_t K, int64_t team_max, int max_lt,
                                int64_t chunk_rows) {
    const int64_t wmax = int64_t(8) << max_lt;
    auto n = [K, wmax](int64_t w) {
        const int64_t wc = w < wmax ? w : wmax;
        return (K + wc - 1) / wc;
    };
    if (R <= chunk_rows / 32) return n(4096);
    if (R <= chunk_rows / 16) return n(2048);
    if (R <= chunk_rows / 8) return n(1024);
    if (R <= chunk_rows / 4) return n(512);
    if (R <= chunk_rows / 2) return n(256);
    if (R <= chunk_rows) return n(128);
    const int64_t c = (R + chunk_rows - 1) / chunk_rows;
    return (c <= team_max ? 1 : 2) * c * n(128);
}

// Upper bound on the dim0 tiles for any offsets, from (M, K, G) alone.
//
// tiles(R) is a step function of R, so every group has n(1024) tiles plus at
// most rho * R more, where rho is the largest (tiles(R) - n(1024)) / R over
// the first row count R of each step with R <= M (inside a step the ratio
// falls as R grows). The rows of all groups add up to at most M, hence
//     tiles <= G * n(1024) + floor(rho * M).
// tiles(R) never falls as R grows, so no group has more than tiles(M), and
// tiles <= G * tiles(M) as well; the bound is the smaller of the two.
// Team steps: rho falls with the chunk count c unless K <= 128, so all of
// them (2 <= c <= team_max <= 128) are scanned; past team_max only the
// first. A strip-width cap (max_lt) only merges steps, so the same rows
// bound it.
inline int64_t dim0_tile_bound(int64_t M, int64_t K, int64_t G, int64_t team_max, int max_lt,
                               int64_t chunk_rows) {
    const int64_t base = dim0_group_tiles(0, K, team_max, max_lt, chunk_rows);
    int64_t extra = 0;
    auto step = [&](int64_t first_rows) {
        if (first_rows > M) return;
        const int64_t num = dim0_group_tiles(first_rows, K, team_max, max_lt, chunk_rows) - base;
        const int64_t e = M * num / first_rows;
        if (e > extra) extra = e;
    };
    step(chunk_rows / 32 + 1);
    step(chunk_rows / 16 + 1);
    step(chunk_rows / 8 + 1);
    step(chunk_rows / 4 + 1);
    step(chunk_rows / 2 + 1);
    // chunked groups have at least 2 chunks (more than chunk_rows rows)
    const int64_t last = team_max + 1 > 2 ? team_max + 1 : 2;
    for (int64_t c = 2; c <= last; ++c) step(chunk_rows * (c - 1) + 1);
    const int64_t spread = G * base + extra;
    const int64_t one = G * dim0_group_tiles(M, K, team_max, max_lt, chunk_rows);
    return spread < one ? spread : one;
}

// Widest strips the launch may use (log2 of 8-column units per strip, 3..9;
// at most 7, 1024 columns, for the transposed kernel, chunk_rows =
// kDim0ChunkRowsT). Never wider than K needs. A tiny problem also gets narrower strips, down
// to 64 columns, until G groups of M / G rows would make at least one tile
// per CU: otherwise a handful of tiles leaves most CUs idle. Only then:
// strips under 256 bytes of bf16 per row stream poorly, and problems with a
// few hundred tiles already run faster on the wide ones.
inline int dim0_lt_cap(int64_t M, int64_t K, int64_t G, int64_t team_max, int64_t cus,
                       int64_t chunk_rows) {
    int lt = 3;
    const int max_lt = chunk_rows == kDim0ChunkRowsT ? 7 : 9;
    while (lt < max_lt && (int64_t(8) << lt) < K) ++lt;
    if (G < 1) return lt;
    const int64_t want = cus;
    while (lt > 3 && G * dim0_group_tiles(M / G, K, team_max, lt, chunk_rows) < want) --lt;
    return lt;
}

// Whether the transposed kernel deals its tiles to the 8 XCDs by column
// range: every strip width (at most 8 << lt_cap columns) must divide K / 8.
// The caller then keeps teams to at most cus / 8 chunks (a quarter of the
// workgroups one XCD holds at once), since a team's tiles all run on one
// XCD.
inline bool dim0_xcd_split(int64_t K, int lt_cap, int64_t cus) {
    return cus >= 64 && cus % 8 == 0 && K > 0 && K % (int64_t(64) << lt_cap) == 0;
}

// dim0 workspace (needed only when M > kDim0ChunkRowsT), in two 256-byte
// aligned regions: one 32-bit counter per (chunk row, 128-column strip), then
// the column maxima of every chunk row, one 64-bit word per column pair
// (a presence tag in the high half, two 16-bit magnitude patterns in the
// low half). A team of chunk tiles (one chunked group, one strip) uses the
// counter at (its first chunk row, its strip) and the words of its chunk rows
// in its strip. Sized for the smaller chunks (dim0_t's), so one workspace
// serves both kernels. Zero-filled before first use; every launch leaves it
// zero-filled again (see mgs_dim0.hip).
struct Dim0Workspace {
    int64_t chunks;      // chunk rows
    int64_t strips;      // 128-column strips, ceil(K / 128)
    size_t ctr_off, max_off, bytes;
};

inline Dim0Workspace dim0_workspace(int64_t M, int64_t K) {
    Dim0Workspace w;
    w.chunks = dim0_chunk_bound(M, kDim0ChunkRowsT);
    w.strips = (K + 127) / 128;
    w.ctr_off = 0;
    w.max_off = ((size_t)(w.chunks * w.strips) * sizeof(uint32_t) + 255) / 256 * 256;
    w.bytes = w.chunks > 0 ? w.max_off + (size_t)(w.chunks * (K / 2)) * sizeof(uint64_t) : 0;
    return w;
}

}  // namespace mgs
