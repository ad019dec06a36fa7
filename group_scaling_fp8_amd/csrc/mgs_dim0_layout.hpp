// mgs_dim0_layout.hpp — dim0 tiling constants, the grid bound and the
// workspace layout (host code with no HIP dependency).
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mgs {

// dim0 tiling: 512-thread workgroups holding 16-byte vectors of the tile,
// per thread kDim0Slabs in registers (10240 vectors, 160 KiB of bf16) and
// kDim0LdsSlabs more in LDS (4096 vectors, 64 KiB); the transposed kernel
// uses the same LDS, once its rows are cast, as its output stage. A group of
// at most chunk_rows rows (the rows of a full 128-column tile, 896) is one
// tile per column strip. A taller group is cut into chunks of at most
// chunk_rows rows on 128-column strips: a team of chunk tiles per strip when
// the chunk count is at most the team limit, else a column-maximum tile and
// a casting tile per chunk and strip. Strip widths step at lt_rows / 2^k
// rows: lt_rows = 896 in dim0; 640, the register rows of a 128-column tile,
// in the transposed kernel, whose tiles cost more the more rows they hold
// (each passes through its LDS stage). Strips are at most 4096 columns wide
// (8 << kDim0MaxLt), 1024 in the transposed kernel (its stage holds strips of
// at most that width).
constexpr int kDim0Slabs = 20;
constexpr int kDim0LdsSlabs = 8;
constexpr int kDim0SlabsT = 20;
constexpr int kDim0ChunkRows = (kDim0Slabs + kDim0LdsSlabs) * 512 / 16;   // 896
constexpr int kDim0ChunkRowsT = (kDim0SlabsT + kDim0LdsSlabs) * 512 / 16; // 896
constexpr int kDim0LtRows = kDim0ChunkRows;                                // 896
constexpr int kDim0LtRowsT = kDim0SlabsT * 512 / 16;                       // 640
constexpr int kDim0MaxLt = 9;
constexpr int kDim0MaxLtT = 7;
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
// C = chunk_rows and L = lt_rows: n(w) = ceil(K / w') strips of width
// w' = min(w, 8 << max_lt) with w = 4096 columns for R <= L/32, 2048 up to
// L/16, 1024 up to L/8, 512 up to L/4, 256 up to L/2 and 128 up to C. A
// taller group has c = ceil(R / C) chunks on n(128) strips: c * n(128) tiles
// as a team (c <= team_max), else 2 * c * n(128).
inline int64_t dim0_group_tiles(int64_t R, int64_t K, int64_t team_max, int max_lt,
                                int64_t chunk_rows, int64_t lt_rows) {
    const int64_t wmax = int64_t(8) << max_lt;
    auto n = [K, wmax](int64_t w) {
        const int64_t wc = w < wmax ? w : wmax;
        return (K + wc - 1) / wc;
    };
    if (R <= lt_rows / 32) return n(4096);
    if (R <= lt_rows / 16) return n(2048);
    if (R <= lt_rows / 8) return n(1024);
    if (R <= lt_rows / 4) return n(512);
    if (R <= lt_rows / 2) return n(256);
    if (R <= chunk_rows) return n(128);
    const int64_t c = (R + chunk_rows - 1) / chunk_rows;
    return (c <= team_max ? 1 : 2) * c * n(128);
}

// Upper bound on the dim0 tiles for any offsets, from (M, K, G) alone.
//
// Every group has base = tiles(0) tiles plus extra(R) = tiles(R) - base more,
// a step function of its rows R that never falls as R grows. Its least
// concave majorant f is the upper hull of the first row count of each step
// (0, then L/32 + 1 .. L/2 + 1 for L = lt_rows, then C * (c - 1) + 1 for
// groups of c chunks, C = chunk_rows), flat past the last step start at or
// below M. The step starts of teams (c <= team_max) lie on one line, and so
// do those of larger groups (c > team_max), so past the first ones the hull
// needs only each line's ends. f is concave and never falls, and the
// rows of all groups add up to at most M, so by Jensen's inequality
//     tiles <= G * base + G * f(M / G).
// No group has more than tiles(M) tiles either, so tiles <= G * tiles(M); the
// bound is the smaller of the two. A strip-width cap (max_lt) only merges
// steps, so the same points bound it.
inline int64_t dim0_tile_bound(int64_t M, int64_t K, int64_t G, int64_t team_max, int max_lt,
                               int64_t chunk_rows, int64_t lt_rows) {
    if (G < 1) return 0;
    auto tiles = [&](int64_t r) { return dim0_group_tiles(r, K, team_max, max_lt, chunk_rows, lt_rows); };
    const int64_t base = tiles(0);
    struct Pt {
        int64_t x, y;
    };
    Pt pts[16 + kDim0MaxTeam];
    int n = 0;
    pts[n++] = {0, 0};
    auto add = [&](int64_t r) {
        if (r <= M && r > pts[n - 1].x) pts[n++] = {r, tiles(r) - base};
    };
    auto chunks = [&](int64_t c) {      // the first rows of a group of c >= 2 chunks
        if (c >= 2 && c <= M / chunk_rows + 1) add(chunk_rows * (c - 1) + 1);
    };
    for (int k = 32; k >= 2; k /= 2) add(lt_rows / k + 1);
    const int64_t team = team_max < kDim0MaxTeam ? (team_max > 0 ? team_max : 0) : kDim0MaxTeam;
    for (int64_t c = 2; c <= team + 2; ++c) chunks(c);
    chunks(team_max);                   // the last team, then the first larger groups
    chunks(team_max + 1);
    chunks(team_max + 2);
    if (M >= 1) add(chunk_rows * ((M - 1) / chunk_rows) + 1);   // the last step start at or below M
    // upper hull: drop a point that lies on or below the line between its neighbours
    Pt h[16 + kDim0MaxTeam];
    int m = 0;
    for (int i = 0; i < n; ++i) {
        const Pt c = pts[i];
        while (m >= 2) {
            const Pt a = h[m - 2], b = h[m - 1];
            if ((__int128)(b.y - a.y) * (c.x - a.x) > (__int128)(c.y - a.y) * (b.x - a.x)) break;
            --m;
        }
        h[m++] = c;
    }
    // G * f(M / G): the hull segment holding M / G (x <= M, G <= 2^31: no overflow)
    int i = 0;
    while (i + 1 < m && G * h[i + 1].x <= M) ++i;
    __int128 gf = (__int128)G * h[i].y;
    if (i + 1 < m)
        gf += (__int128)(h[i + 1].y - h[i].y) * (M - G * h[i].x) / (h[i + 1].x - h[i].x);
    const __int128 spread = (__int128)G * base + gf;
    const __int128 one = (__int128)G * tiles(M);
    const __int128 b = spread < one ? spread : one;
    return b > (__int128)INT64_MAX ? INT64_MAX : (int64_t)b;
}

// Widest strips the launch may use (log2 of 8-column units per strip, 3 to
// max_lt: kDim0MaxLt, or kDim0MaxLtT for the transposed kernel). Never wider
// than K needs. A tiny problem also gets narrower strips, down to 64
// columns, until G groups of M / G rows would make at least one tile per CU:
// otherwise a handful of tiles leaves most CUs idle. Only then: strips under
// 256 bytes of bf16 per row stream poorly, and problems with a few hundred
// tiles already run faster on the wide ones.
inline int dim0_lt_cap(int64_t M, int64_t K, int64_t G, int64_t team_max, int64_t cus,
                       int64_t chunk_rows, int64_t lt_rows, int max_lt) {
    int lt = 3;
    while (lt < max_lt && (int64_t(8) << lt) < K) ++lt;
    if (G < 1) return lt;
    const int64_t want = cus;
    while (lt > 3 && G * dim0_group_tiles(M / G, K, team_max, lt, chunk_rows, lt_rows) < want) --lt;
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
// in its strip. Both kernels cut groups into the same chunks, so one
// workspace serves both. Zero-filled before first use; every launch leaves it
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
