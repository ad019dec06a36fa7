// mgs_dim0.hip — per-token-group scaling along dim0 on gfx950.
//
// Method: "[moe training] use smaller block sizes for per group scaling
// kernels to improve perf", description (per-token-group scaling along dim0:
// one scale per (group, column)) and its kernel-argument dict (448, 1e-12,
// power-of-two rounding). That page's fix was filling every compute unit
// when groups are small. Here every workgroup gets a tile of about the same
// size whatever the group sizes, so the grid scales with M * K and not with
// the group count.
//
// One launch, one tile per workgroup. The host sizes the grid with an upper
// bound from (M, K, G) (it never reads the offsets); workgroups past the real
// tile count exit as soon as they find no tile. Every wave finds its tile by
// itself from the offsets (64 groups at a time: scalar loads in dim0, one
// vector load in dim0_t; DPP scans and a ballot), so nothing stands between
// the launch and the tile's loads.
// Offsets are sanitised on the fly: end[g] = min(max(off[0..g]), M), clamped
// below at 0, so any offsets array gives in-range rows.
//
// A 512-thread workgroup holds up to kSlabs 16-byte vectors per thread in
// registers (160 KiB of bf16) and kLdsSlabs more in LDS (64 KiB, loaded
// straight from global memory with global_load_lds), and every byte of x is
// loaded once into them. One CU alone streams only a few tens of GB/s, so
// HBM is full only while every CU has loads in flight; holding 224 KiB per
// tile lets a group of up to 896 rows (C below) be one tile and gives
// 449-896-row groups strips of 256 and 128 columns instead of chunk teams.
// The transposed kernel reuses the same LDS as its output stage once the
// rows held there are cast. A tile is rows of one group times a strip of
// 8 * tpr columns, tpr lanes per row:
//   * class A, R <= C rows: one tile per strip. tpr is the widest power of
//     two in [16, 512] whose tile fits (short groups get strips up to 4096
//     columns; up to 1024 in the transposed kernel, whose LDS stage holds
//     strips of at most that width, and which picks widths as if tiles held
//     only their 640 register rows: its tiles cost more the more rows they
//     hold). Load -> column amax -> scale -> cast from registers -> store.
//     No strip is narrower than 128 columns unless K is, or the launch would
//     otherwise have fewer tiles than CUs (lt_cap, from dim0_lt_cap): rows of
//     128 bytes stream far worse than rows of 256.
//   * class T, R > C rows and at most team_max chunks: the group is cut
//     into c = ceil(R / C) chunks of about R / c rows (in the transposed
//     kernel rounded to 128 rows, with boundaries on 128-row lines of x where
//     the last chunk allows) on 128-column strips, and the c tiles of a strip
//     are consecutive in the grid (a team). Each loads its chunk,
//     writes the chunk's column maxima to a workspace, waits for the maxima
//     of the other chunks of its strip, and casts its chunk from registers.
//     team_max is at most the CU count: with two resident workgroups per CU
//     and workgroups started in grid order, the first resident workgroups
//     always hold a whole team, which finishes and frees room for the rest.
//   * class C, more chunks than that: a column-maximum tile and a casting
//     tile per (chunk, strip). All column-maximum tiles come first in the
//     grid; a casting tile waits for its strip's maxima before its own loads,
//     and casts its chunk (a chunk is read twice).
// Maxima go through the workspace as 64-bit words, each holding a presence
// tag next to the maxima of two columns, written and read as single relaxed
// device-scope atomics. A word is read and written whole, so a reader that
// sees the tag sees the maxima: no fence or flag is needed. Every wait is
// bounded: past it the tile computes the column amax of the whole group from
// x itself, so the result never depends on the order in which workgroups run.
// The workspace is all zero between launches, so a tagged word can only be
// this launch's. Every tile of a team (a chunked group on one strip: its
// chunk tiles, and in class C its column-maximum tiles) counts itself on the
// team's counter once it has read every word it needs and its own words are
// stored; the counter wraps back to zero on the team's last tile, which then
// clears the team's words. No state outlives a launch, so calls need nothing
// from the host, and a captured graph replays with no extra node.
// Tile order: all column-maximum tiles, then every group's own tiles in
// group order: class A strip by strip; class T strip by strip with the chunks
// of a strip together; class C chunk by chunk with strips fastest.
#include "mgs_device.hpp"
#include "mgs_kernels.hpp"

#include <map>
#include <mutex>
#if defined(MGS_TILE_TRACE)
#include "mgs_trace.h"
#endif

namespace mgs {

#if defined(MGS_TILE_TRACE)
// Tile timeline, in trace builds only (libmgs_trace.so). For each tile item
// i < kTraceTiles that casts (column-maximum tiles of class C are not
// recorded; with the transposed kernel's XCD split, record 8 i + x holds
// item i of XCD x), eight 64-bit words: five s_memrealtime stamps (100 MHz) at the
// item's start, the tile found, its loads and column maxima done (a team
// tile: after the team's maxima came in; a class C casting tile: after its
// strip's maxima came in and its loads), the reduction across the workgroup
// done, and its stores issued; then the workgroup's placement (HW_ID << 32 |
// XCC_ID), class << 60 | chunk << 32 | rows, and group << 40 | strip << 16 |
// strip width in columns. Each launch overwrites the items it runs.
constexpr int kTraceTiles = 16384;
__device__ unsigned long long g_tile_trace[kTraceTiles * 8];
#define MGS_TRACE_STAMP(v) const unsigned long long v = __builtin_amdgcn_s_memrealtime()
#else
#define MGS_TRACE_STAMP(v)
#endif

namespace {

constexpr int kThreads = 512;
constexpr int kLdsSlabs = kDim0LdsSlabs;              // vectors per thread in LDS
// vectors per thread in registers
template <bool kT>
constexpr int reg_slabs() { return kT ? kDim0SlabsT : kDim0Slabs; }
// Rows of a full 128-column tile (16 lanes per row, 32 rows per slab): the
// chunk size, and 8x / 4x / 2x the rows of the 1024 / 512 / 256-column steps.
template <bool kT>
constexpr int rows_w128() { return kThreads * (reg_slabs<kT>() + kLdsSlabs) / 16; }
static_assert(rows_w128<false>() == kDim0ChunkRows, "dim0 chunk size mismatch");
static_assert(rows_w128<true>() == kDim0ChunkRowsT, "dim0_t chunk size mismatch");
static_assert(kDim0ChunkRows % 8 == 0 && kDim0ChunkRowsT % 8 == 0, "strip steps");
constexpr int kStreamSlabs = 4;                       // rows in flight per lane for streamed rows

enum { kClassA = 0, kClassT = 1, kClassC = 2 };

struct Tile {
    int g;          // group, or -1 when this workgroup has no tile
    int maxima;     // 1: class C column-maximum tile (writes no output)
    int cls;        // kClassA / kClassT / kClassC
    int lt;         // log2 of lanes per row (3..9)
    int strip;      // column strip index (strip width 8 << lt)
    int c, nc;      // chunk index and chunk count (classes T, C), else 0 and 1
    int r0, r1;     // rows of this tile (the chunk for classes T, C)
    int g0, g1;     // rows of the whole group
    int cbase;      // classes T, C: workspace row of the group's first chunk
};

// Per-lane view of one group: rows, class, strips, chunks and tile counts.
struct GroupInfo {
    int start, R, lt, cls, ns, nc;
    int cnt_x;      // column-maximum tiles
    int cnt_m;      // own tiles
    int chunks;     // workspace rows (classes T, C)
};

// Strip widths step at kLtRows / 2^k rows (the rows of a full 128-column
// tile that the kernel likes best: all of them in dim0, the register rows in
// the transposed kernel); groups of more than kRows rows are cut into chunks.
template <int kRows, int kLtRows>
__device__ __forceinline__ GroupInfo group_info(int start, int end, bool valid, int K, int team_max,
                                                int lt_cap) {
    GroupInfo gi;
    gi.start = start;
    gi.R = end - start;
    const int R = gi.R;
    gi.nc = 1;
    if (R > kRows) {
        gi.lt = 4;
        gi.nc = (R + kRows - 1) / kRows;
        gi.cls = gi.nc <= team_max ? kClassT : kClassC;
    } else {
        gi.lt = R <= kLtRows / 32 ? 9 : (R <= kLtRows / 16 ? 8 : (R <= kLtRows / 8 ? 7 :
                (R <= kLtRows / 4 ? 6 : (R <= kLtRows / 2 ? 5 : 4))));
        gi.cls = kClassA;
    }
    // no strip wider than needed to cover K
    gi.lt = min(gi.lt, lt_cap);
    gi.ns = (K + (8 << gi.lt) - 1) >> (gi.lt + 3);
    gi.chunks = (valid && gi.cls != kClassA) ? gi.nc : 0;
    gi.cnt_x = (valid && gi.cls == kClassC) ? gi.nc * gi.ns : 0;
    gi.cnt_m = valid ? gi.nc * gi.ns : 0;
    return gi;
}

// Inclusive prefix sum over a wave with DPP: row shifts 1, 2, 4, 8 inside
// each 16-lane row, then the row_bcast:15 / row_bcast:31 carries.
__device__ __forceinline__ int wave_prefix_sum_dpp(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);
    return v;
}

// v in lane L becomes the wave-uniform value e (the lane an immediate: a
// second scalar operand would break the one-scalar-read limit of VALU
// instructions on this target).
template <int L>
__device__ __forceinline__ void write_lane(int& v, int e) {
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(v) : "s"(e), "n"(L));
}

// Lanes L .. L + 15 of v from p[L .. L + 15] (one 64-byte scalar load).
template <int L>
__device__ __forceinline__ void write_lanes16(int& v, const int32_t* __restrict__ p) {
    int e[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) e[k] = p[L + k];
    write_lane<L + 0>(v, e[0]);   write_lane<L + 1>(v, e[1]);   write_lane<L + 2>(v, e[2]);
    write_lane<L + 3>(v, e[3]);   write_lane<L + 4>(v, e[4]);   write_lane<L + 5>(v, e[5]);
    write_lane<L + 6>(v, e[6]);   write_lane<L + 7>(v, e[7]);   write_lane<L + 8>(v, e[8]);
    write_lane<L + 9>(v, e[9]);   write_lane<L + 10>(v, e[10]); write_lane<L + 11>(v, e[11]);
    write_lane<L + 12>(v, e[12]); write_lane<L + 13>(v, e[13]); write_lane<L + 14>(v, e[14]);
    write_lane<L + 15>(v, e[15]);
}

// The lane number, computed where it is used: the compiler cannot hoist it,
// so addresses derived from it do not stay live (and spill) across the
// whole kernel.
__device__ __forceinline__ int lane_here() {
    int lane;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane));
    return lane;
}

// threadIdx.x through an opaque copy, for the same reason.
__device__ __forceinline__ int tid_here() {
    int tid;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));
    return tid;
}

// Lane i's raw group end for group base + i: off[base + i] (or the equal
// group's end), M past the last group. kScalar: the offsets come in through
// scalar loads, 16 at a time, and are written into lanes with v_writelane.
// A vector load queues in the CU's memory pipeline behind the tile loads of
// the other workgroup on the CU; a scalar load takes the scalar cache
// instead. (The transposed kernel keeps the vector load: there the scalar
// form measured slower and needed a register spill.)
template <bool kScalar>
__device__ __forceinline__ int group_end_raw(const int32_t* __restrict__ off, int base, int G, int M,
                                             int uniform_rows) {
    // (the lane through lane_here: computed here, not hoisted out of the
    // tile loop and kept, or spilled, through the whole kernel)
    const int lane = lane_here();
    if (uniform_rows >= 0) {
        const int g = base + lane;
        return g < G ? (g + 1) * uniform_rows : M;
    }
    if (!kScalar) {
        const int g = base + lane;
        return g < G ? off[g] : M;
    }
    int v = M;
    const int n = min(G - base, kWave);
    const int32_t* p = off + base;
    if (n == kWave) {
        write_lanes16<0>(v, p);
        write_lanes16<16>(v, p);
        write_lanes16<32>(v, p);
        write_lanes16<48>(v, p);
        return v;
    }
    for (int j = 0; j < n; ++j) {
        const int e = p[j];
        v = lane == j ? e : v;
    }
    return v;
}

// Fills t from lane src's group, tile `local` inside that group. src is
// wave-uniform, so the fields land in scalar registers.
template <int kRows, int kLine>
__device__ __forceinline__ void take_tile(Tile& t, const GroupInfo& gi, int chunk_incl, int src,
                                          int g, int local, int maxima, int row_align) {
    const int ns = __builtin_amdgcn_readlane(gi.ns, src);
    const int nc = __builtin_amdgcn_readlane(gi.nc, src);
    const int start = __builtin_amdgcn_readlane(gi.start, src);
    const int R = __builtin_amdgcn_readlane(gi.R, src);
    t.g = g;
    t.maxima = maxima;
    t.cls = __builtin_amdgcn_readlane(gi.cls, src);
    t.lt = __builtin_amdgcn_readlane(gi.lt, src);
    t.nc = nc;
    t.g0 = start;
    t.g1 = start + R;
    if (t.cls == kClassA) {          // one tile per strip: no division
        t.c = 0;
        t.strip = local;
        t.r0 = t.g0;
        t.r1 = t.g1;
        t.cbase = 0;
        return;
    }
    // class T: the chunks of a strip together; class C: strips fastest. One
    // division and plain selects: stores into t.strip or t.c chosen by class
    // made the compiler keep the Tile in scratch memory.
    const bool team = t.cls == kClassT;
    const int den = team ? nc : ns;
    const int quo = local / den;
    const int rem = local - quo * den;
    t.strip = team ? quo : rem;
    t.c = team ? rem : quo;
    // Chunk rows: R / nc rounded up to row_align and kLine (powers of two;
    // kLine = 128 rows, a q_t line, in the transposed kernel, else 1). kRows
    // is a multiple of both, so cs <= kRows, and (nc - 1) * cs < R since
    // R > (nc - 1) * kRows: the last chunk is never empty. With kLine > 1 the
    // boundaries also move onto multiples of kLine rows of x when the last
    // chunk still fits (chunk 0 then starts short), so that chunk tiles share
    // no q_t line.
    static_assert(kRows % kLine == 0 && (kLine & (kLine - 1)) == 0, "chunk rounding");
    const int align = kLine > row_align ? kLine : row_align;
    const int cs = ((R + nc - 1) / nc + align - 1) & -align;
    int s0 = start;
    if (kLine > 1) {
        const int lead = start & (kLine - 1);
        if (R + lead - (nc - 1) * cs <= kRows) s0 = start - lead;
    }
    t.r0 = t.c == 0 ? start : min(s0 + t.c * cs, t.g1);
    t.r1 = t.c == nc - 1 ? t.g1 : min(s0 + (t.c + 1) * cs, t.g1);
    t.cbase = __builtin_amdgcn_readlane(chunk_incl, src) - __builtin_amdgcn_readlane(gi.chunks, src);
}

// Tile number `target` of the order described at the top of this file. Run
// by every wave of the workgroup; all lanes return the same tile.
// Group ends come from off (uniform_rows < 0), or are (g + 1) * uniform_rows
// (equal groups, e.g. the experts of a 3D weight, with no offsets array).
template <int kRows, int kLtRows, bool kScalar, int kLine>
__device__ Tile find_tile(const int32_t* __restrict__ off, int G, int M, int K, int team_max,
                          int lt_cap, bool maybe_c, int row_align, int uniform_rows, int target) {
    const int lane = threadIdx.x & (kWave - 1);
    Tile t;
    t.g = -1;
    // One pass finds a column-maximum tile, or an own tile provided there are
    // no column-maximum tiles at all (their count is known only at the end).
    int carry_end = 0, carry_x = 0, carry_m = 0, carry_ch = 0;
    for (int base = 0; base < G; base += kWave) {
        const int g = base + lane;
        const int raw = min(max(group_end_raw<kScalar>(off, base, G, M, uniform_rows), 0), M) & -row_align;
        const int end = max((int)wave_prefix_max((uint32_t)raw), carry_end);
        // the previous lane's end (wave_shr:1); lane 0 keeps carry_end
        const int start = __builtin_amdgcn_update_dpp(carry_end, end, 0x138, 0xF, 0xF, false);
        const GroupInfo gi = group_info<kRows, kLtRows>(start, end, g < G, K, team_max, lt_cap);
        const int incl_x = maybe_c ? wave_prefix_sum_dpp(gi.cnt_x) + carry_x : 0;
        const int incl_m = wave_prefix_sum_dpp(gi.cnt_m) + carry_m;
        const int incl_ch = wave_prefix_sum_dpp(gi.chunks) + carry_ch;
        const uint64_t hx =
            maybe_c ? __ballot(gi.cnt_x > 0 && target >= incl_x - gi.cnt_x && target < incl_x) : 0ull;
        if (hx) {
            const int src = __ffsll((unsigned long long)hx) - 1;
            const int local = target - (__builtin_amdgcn_readlane(incl_x, src) -
                                        __builtin_amdgcn_readlane(gi.cnt_x, src));
            take_tile<kRows, kLine>(t, gi, incl_ch, src, base + src, local, 1, row_align);
            return t;
        }
        if (t.g < 0) {
            const uint64_t hm = __ballot(gi.cnt_m > 0 && target >= incl_m - gi.cnt_m && target < incl_m);
            if (hm) {
                const int src = __ffsll((unsigned long long)hm) - 1;
                const int local = target - (__builtin_amdgcn_readlane(incl_m, src) -
                                            __builtin_amdgcn_readlane(gi.cnt_m, src));
                take_tile<kRows, kLine>(t, gi, incl_ch, src, base + src, local, 0, row_align);
            }
        }
        if (t.g >= 0 && !maybe_c) return t;
        carry_end = __builtin_amdgcn_readlane(end, kWave - 1);
        carry_x = __builtin_amdgcn_readlane(incl_x, kWave - 1);
        carry_m = __builtin_amdgcn_readlane(incl_m, kWave - 1);
        carry_ch = __builtin_amdgcn_readlane(incl_ch, kWave - 1);
    }
    if (carry_x == 0) return t;
    // There are column-maximum tiles, and target lies past them: search the
    // own tiles again with their count taken off.
    target -= carry_x;
    t.g = -1;
    carry_end = carry_m = carry_ch = 0;
    for (int base = 0; base < G; base += kWave) {
        const int g = base + lane;
        const int raw = min(max(group_end_raw<kScalar>(off, base, G, M, uniform_rows), 0), M) & -row_align;
        const int end = max((int)wave_prefix_max((uint32_t)raw), carry_end);
        const int start = __builtin_amdgcn_update_dpp(carry_end, end, 0x138, 0xF, 0xF, false);
        const GroupInfo gi = group_info<kRows, kLtRows>(start, end, g < G, K, team_max, lt_cap);
        const int incl_m = wave_prefix_sum_dpp(gi.cnt_m) + carry_m;
        const int incl_ch = wave_prefix_sum_dpp(gi.chunks) + carry_ch;
        const uint64_t hm = __ballot(gi.cnt_m > 0 && target >= incl_m - gi.cnt_m && target < incl_m);
        if (hm) {
            const int src = __ffsll((unsigned long long)hm) - 1;
            const int local = target - (__builtin_amdgcn_readlane(incl_m, src) -
                                        __builtin_amdgcn_readlane(gi.cnt_m, src));
            take_tile<kRows, kLine>(t, gi, incl_ch, src, base + src, local, 0, row_align);
            return t;
        }
        carry_end = __builtin_amdgcn_readlane(end, kWave - 1);
        carry_m = __builtin_amdgcn_readlane(incl_m, kWave - 1);
        carry_ch = __builtin_amdgcn_readlane(incl_ch, kWave - 1);
    }
    return t;
}

// Words of the LDS scratch of find_tile_wide: block maxima, block totals
// (column-maximum tiles, own tiles, chunk rows), the found flag and the tile.
constexpr int kWaves = kThreads / kWave;
constexpr int kSearchMax = 0;
constexpr int kSearchTot = kWaves;
constexpr int kSearchFlag = 4 * kWaves;
constexpr int kSearchTile = 4 * kWaves + 1;
constexpr int kSearchWords = kSearchTile + 12;

// find_tile for launches of more than 64 groups (at most 1024): the
// workgroup's 8 waves take 8 contiguous blocks of 64 or 128 groups and scan
// them at once, then combine the blocks' maxima of the group ends and their
// tile and chunk totals through LDS (three barriers); the wave that holds
// the target publishes its tile. Same order, same tiles as find_tile; run by
// every wave, and every lane returns the same tile.
template <int kRows, int kLtRows, bool kScalar, int kLine>
__device__ Tile find_tile_wide(const int32_t* __restrict__ off, int G, int M, int K, int team_max,
                               int lt_cap, bool maybe_c, int row_align, int uniform_rows, int target,
                               int* sx) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
    // groups per wave: 64 up to 512 groups, else 128
    const int np = G > kWaves * kWave ? 2 : 1;
    const int b0 = w * np * kWave;
    // ends, block by block: the running max inside this wave's block
    int end[2], start[2];
    int carry = 0;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        end[p] = 0;
        const int base = b0 + p * kWave;
        if (p < np && base < G) {
            const int raw = min(max(group_end_raw<kScalar>(off, base, G, M, uniform_rows), 0), M) & -row_align;
            end[p] = max((int)wave_prefix_max((uint32_t)raw), carry);
            carry = __builtin_amdgcn_readlane(end[p], kWave - 1);
        }
    }
    if (lane == 0) {
        sx[kSearchMax + w] = carry;
        if (w == 0) sx[kSearchFlag] = 0;
    }
    __syncthreads();
    int carry_end = 0;
    for (int v = 0; v < w; ++v) carry_end = max(carry_end, sx[kSearchMax + v]);
    // group rules and the block's prefix sums, from the global running max
    GroupInfo gi[2];
    int incl_x[2], incl_m[2], incl_ch[2];
    int cx = 0, cm = 0, cch = 0;
    int prev_end = carry_end;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int base = b0 + p * kWave;
        const int e = max(end[p], carry_end);
        start[p] = __builtin_amdgcn_update_dpp(prev_end, e, 0x138, 0xF, 0xF, false);
        gi[p] = group_info<kRows, kLtRows>(start[p], e, p < np && base + lane < G, K, team_max, lt_cap);
        incl_x[p] = maybe_c ? wave_prefix_sum_dpp(gi[p].cnt_x) + cx : 0;
        incl_m[p] = wave_prefix_sum_dpp(gi[p].cnt_m) + cm;
        incl_ch[p] = wave_prefix_sum_dpp(gi[p].chunks) + cch;
        prev_end = __builtin_amdgcn_readlane(e, kWave - 1);
        cx = __builtin_amdgcn_readlane(incl_x[p], kWave - 1);
        cm = __builtin_amdgcn_readlane(incl_m[p], kWave - 1);
        cch = __builtin_amdgcn_readlane(incl_ch[p], kWave - 1);
    }
    if (lane == 0) {
        sx[kSearchTot + 3 * w] = cx;
        sx[kSearchTot + 3 * w + 1] = cm;
        sx[kSearchTot + 3 * w + 2] = cch;
    }
    __syncthreads();
    int base_x = 0, base_m = 0, base_ch = 0, total_x = 0;
    for (int v = 0; v < kWaves; ++v) {
        const int tx = sx[kSearchTot + 3 * v];
        total_x += tx;
        if (v < w) {
            base_x += tx;
            base_m += sx[kSearchTot + 3 * v + 1];
            base_ch += sx[kSearchTot + 3 * v + 2];
        }
    }
    // column-maximum tiles come first; own tiles are numbered after them
    const bool maxima = maybe_c && target < total_x;
    const int tgt = maxima ? target : target - total_x;
    Tile t;
    t.g = -1;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int cnt = maxima ? gi[p].cnt_x : gi[p].cnt_m;
        const int incl = (maxima ? base_x + incl_x[p] : base_m + incl_m[p]);
        const uint64_t h = __ballot(p < np && cnt > 0 && tgt >= incl - cnt && tgt < incl);
        if (h && t.g < 0) {
            const int src = __ffsll((unsigned long long)h) - 1;
            const int local = tgt - (__builtin_amdgcn_readlane(incl, src) - __builtin_amdgcn_readlane(cnt, src));
            take_tile<kRows, kLine>(t, gi[p], base_ch + incl_ch[p], src, b0 + p * kWave + src, local,
                                      maxima ? 1 : 0, row_align);
        }
    }
    if (t.g >= 0 && lane == 0) {
        int* d = sx + kSearchTile;
        d[0] = t.g;  d[1] = t.maxima;  d[2] = t.cls;  d[3] = t.lt;  d[4] = t.strip;  d[5] = t.c;
        d[6] = t.nc; d[7] = t.r0;      d[8] = t.r1;   d[9] = t.g0;  d[10] = t.g1;    d[11] = t.cbase;
        sx[kSearchFlag] = 1;
    }
    __syncthreads();
    Tile r;
    r.g = -1;
    if (__builtin_amdgcn_readfirstlane(sx[kSearchFlag])) {
        const int* d = sx + kSearchTile;
        r.g = __builtin_amdgcn_readfirstlane(d[0]);
        r.maxima = __builtin_amdgcn_readfirstlane(d[1]);
        r.cls = __builtin_amdgcn_readfirstlane(d[2]);
        r.lt = __builtin_amdgcn_readfirstlane(d[3]);
        r.strip = __builtin_amdgcn_readfirstlane(d[4]);
        r.c = __builtin_amdgcn_readfirstlane(d[5]);
        r.nc = __builtin_amdgcn_readfirstlane(d[6]);
        r.r0 = __builtin_amdgcn_readfirstlane(d[7]);
        r.r1 = __builtin_amdgcn_readfirstlane(d[8]);
        r.g0 = __builtin_amdgcn_readfirstlane(d[9]);
        r.g1 = __builtin_amdgcn_readfirstlane(d[10]);
        r.cbase = __builtin_amdgcn_readfirstlane(d[11]);
    }
    return r;
}

__device__ __forceinline__ void max4(uint4& m, const uint4& t) {
    m.x = mag_max2(m.x, t.x);
    m.y = mag_max2(m.y, t.y);
    m.z = mag_max2(m.z, t.z);
    m.w = mag_max2(m.w, t.w);
}

// Column amax over every lane that shares this lane's 8 columns (same
// tx = lane mod tpr), returned in every lane: xor shuffles inside the wave,
// then one partial per (wave, tx) through LDS (per (row, tx) when a row spans
// waves) and one barrier. Ends with every thread reading red: a barrier must
// come before red is written again.
__device__ __forceinline__ uint4 block_column_amax(uint4 m, int tpr, uint4* red) {
    for (int d = tpr; d < kWave; d <<= 1) {
        m.x = mag_max2(m.x, __shfl_xor(m.x, d, kWave));
        m.y = mag_max2(m.y, __shfl_xor(m.y, d, kWave));
        m.z = mag_max2(m.z, __shfl_xor(m.z, d, kWave));
        m.w = mag_max2(m.w, __shfl_xor(m.w, d, kWave));
    }
    const int lane = lane_here();
    const int tid = tid_here();
    int parts;
    if (tpr <= kWave) {
        parts = kThreads / kWave;
        if (lane < tpr) red[(tid / kWave) * tpr + lane] = m;
    } else {
        parts = kThreads / tpr;
        red[tid] = m;
    }
    __syncthreads();
    const int tx = tid & (tpr - 1);
    uint4 a = make_uint4(0u, 0u, 0u, 0u);
    for (int p = 0; p < parts; ++p) max4(a, red[p * tpr + tx]);
    return a;
}

// Whether ok holds in every thread of the workgroup: a ballot per wave, one
// LDS word per wave, one barrier. (HIP's __syncthreads_and reduces over the
// flat thread id, which keeps the y and z thread ids in registers through
// the whole kernel.) Called at most once per tile item: vote is written again
// only in a later item, after the item's closing barrier.
__device__ __forceinline__ bool block_all(bool ok, int* vote) {
    const unsigned long long bad = __ballot(!ok);
    if (lane_here() == 0) vote[threadIdx.x / kWave] = bad == 0ull;
    __syncthreads();
    int all = 1;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) all &= vote[w];
    return all != 0;
}

struct TileGeom {
    int tpr, tx, ty, rps, col;
    bool col_ok;
    bool full_width;    // every lane's columns lie inside K (uniform)
};

__device__ __forceinline__ TileGeom tile_geom(const Tile& t, int K) {
    TileGeom q;
    q.tpr = 1 << t.lt;
    q.tx = threadIdx.x & (q.tpr - 1);
    q.ty = threadIdx.x >> t.lt;
    q.rps = kThreads >> t.lt;
    q.col = t.strip * (q.tpr * 8) + q.tx * 8;
    q.col_ok = q.col < K;
    q.full_width = (t.strip + 1) * (q.tpr * 8) <= K;
    return q;
}

// Tile row held in vector s by a lane of row index ty. Plain layout: rows
// s * rps + ty. Quad layout (transposed output): vectors 4j .. 4j + 3 hold
// four consecutive rows 4 * (j * rps + ty) + 0..3, so that a lane can turn
// them into 4-byte column words.
template <bool kQuad>
__device__ __forceinline__ int slab_row(int s, int rps, int ty) {
    return kQuad ? 4 * ((s >> 2) * rps + ty) + (s & 3) : s * rps + ty;
}

// Loads rows [r0, r0 + nrows) of this lane's 8 columns into registers.
// A lane's rows sit at slab_row(s, rps, 0) plus a fixed lane offset, so the
// addresses are one lane base plus a uniform step per slab; slabs whose rows
// all exist for every lane of a full-width strip skip the per-lane checks.
template <bool kQuad>
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, int64_t K, int r0, int nrows,
                                          const TileGeom& q, uint4 (&v)[reg_slabs<kQuad>()]) {
    constexpr int kSlabs = reg_slabs<kQuad>();
    const int lane_row = slab_row<kQuad>(0, q.rps, q.ty);
    const int last_lane_row = slab_row<kQuad>(0, q.rps, q.rps - 1);
    const uint16_t* p = x + (int64_t)(r0 + lane_row) * K + q.col;
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
        v[s] = make_uint4(0u, 0u, 0u, 0u);
        const int r_s = slab_row<kQuad>(s, q.rps, 0);
        if (r_s + last_lane_row < nrows && q.full_width) {
            v[s] = load_stream(p);
        } else if (r_s < nrows) {
            if (r_s + lane_row < nrows && q.col_ok) v[s] = load_stream(p);
        }
        if (s + 1 < kSlabs)
            p += (int64_t)(slab_row<kQuad>(s + 1, q.rps, 0) - r_s) * K;
    }
}

typedef __attribute__((address_space(3))) void lds_void;

// Slabs kSlabs .. kSlabs + kLdsSlabs - 1 (rows slab_row(kSlabs + e, rps,
// ty)) go straight from global memory into LDS (global_load_lds_dwordx4:
// lane i of a wave writes 16 bytes at the wave's LDS base + 16 i), so thread
// t owns ext[e * kThreads + t]. Lanes whose row or columns do not exist load
// nothing, and ext_slab masks them.
// In the quad layout tile rows are whole quads (the transposed kernel's rows
// and row starts are multiples of 16), so a quad's first row decides for all
// four of its vectors.
template <bool kQuad>
__device__ __forceinline__ int ext_check_row(int e, int rps, int ty) {
    return slab_row<kQuad>(reg_slabs<kQuad>() + (kQuad ? e & ~3 : e), rps, ty);
}

template <bool kQuad>
__device__ __forceinline__ void load_tile_ext(const uint16_t* __restrict__ x, int64_t K, int r0,
                                              int nrows, const TileGeom& q, uint4* ext) {
    constexpr int kSlabs = reg_slabs<kQuad>();
    const int wave = threadIdx.x / kWave;
    const uint16_t* p = x + (int64_t)(r0 + slab_row<kQuad>(kSlabs, q.rps, q.ty)) * K + q.col;
#pragma unroll
    for (int e = 0; e < kLdsSlabs; ++e) {
        const int r = ext_check_row<kQuad>(e, q.rps, q.ty);
        if (r < nrows && q.col_ok)
            __builtin_amdgcn_global_load_lds(p, (lds_void*)(ext + e * kThreads + wave * kWave), 16, 0,
                                             kLoadNontemporal);
        if (e + 1 < kLdsSlabs)
            p += (int64_t)(slab_row<kQuad>(kSlabs + e + 1, q.rps, 0) - slab_row<kQuad>(kSlabs + e, q.rps, 0)) * K;
    }
}

template <bool kQuad>
__device__ __forceinline__ uint4 ext_slab(const uint4* ext, int e, int nrows, const TileGeom& q) {
    if (ext_check_row<kQuad>(e, q.rps, q.ty) < nrows && q.col_ok)
        return ext[e * kThreads + threadIdx.x];
    return make_uint4(0u, 0u, 0u, 0u);
}

// Running column amax of rows [r0, r0 + nrows) of this lane's columns,
// streamed through a few registers.
__device__ __forceinline__ void stream_amax(const uint16_t* __restrict__ x, int64_t K, int r0, int nrows,
                                            const TileGeom& q, uint4& m) {
    for (int base = 0; base < nrows; base += kStreamSlabs * q.rps) {
        uint4 u[kStreamSlabs];
#pragma unroll
        for (int b = 0; b < kStreamSlabs; ++b) {
            u[b] = make_uint4(0u, 0u, 0u, 0u);
            const int rr = base + b * q.rps + q.ty;
            if (rr < nrows && q.col_ok) u[b] = load_stream(x + (int64_t)(r0 + rr) * K + q.col);
        }
#pragma unroll
        for (int b = 0; b < kStreamSlabs; ++b) max4(m, u[b]);
    }
}

__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Tag of a word that holds this launch's maxima (the workspace is zero
// between launches).
constexpr uint64_t kWordPresent = uint64_t(1) << 32;

// Wave 0 of a tile of a team, after the tile's last read of maxima words and
// once its own words are stored: counts the tile on the team's counter, which
// wraps to zero on the team's last tile (an atomic increment with bound
// team_size - 1). Returns the count before (lane 0); the value is first used
// after the tile's final barrier, so the increment's round trip overlaps the
// tile's stores.
__device__ __forceinline__ uint32_t team_tile_done(uint32_t* ctr, uint32_t team_size) {
    uint32_t old = 0;
    if ((threadIdx.x & (kWave - 1)) == 0)
        old = __builtin_amdgcn_atomic_inc32(ctr, team_size - 1u, __ATOMIC_RELAXED, "agent");
    return old;
}

// The words of this lane's 8 columns for chunk c of the tile's group.
__device__ __forceinline__ uint64_t* chunk_words(uint64_t* ws_max, const Tile& t, int c, int64_t K,
                                                 const TileGeom& q) {
    return ws_max + (((int64_t)(t.cbase + c) * K + q.col) >> 1);
}

// Publishes this chunk's column maxima (threads 0..tpr-1 hold them).
__device__ __forceinline__ void publish_maxima(uint64_t* ws_max, const Tile& t, int64_t K,
                                               const TileGeom& q, uint4 m) {
    if (threadIdx.x < q.tpr && q.col_ok) {
        uint64_t* dst = chunk_words(ws_max, t, t.c, K, q);
        store_agent(dst, kWordPresent | m.x);
        store_agent(dst + 1, kWordPresent | m.y);
        store_agent(dst + 2, kWordPresent | m.z);
        store_agent(dst + 3, kWordPresent | m.w);
    }
}

// Wave 0 of the team's last tile: clears the words of the team's chunk rows
// in its strip (one word per column pair: 4 << lt words per row, at most 64
// since chunked groups have strips of at most 128 columns).
__device__ __forceinline__ void clear_team_words(uint64_t* ws_max, const Tile& t, int64_t K) {
    const int lane = threadIdx.x & (kWave - 1);
    const int per_strip = 4 << t.lt;
    const int64_t w = (int64_t)t.strip * per_strip + lane;
    if (lane >= per_strip || w >= K / 2) return;
    for (int c = 0; c < t.nc; ++c) store_agent(ws_max + (int64_t)(t.cbase + c) * (K / 2) + w, 0ull);
}

// Folds into m the maxima of chunks ty, ty + rps, ... of the tile's strip,
// waiting until each word is present. Returns false if the wait ran out
// (then m is incomplete) or was skipped (spin_ticks < 0).
__device__ __forceinline__ bool gather_maxima(uint64_t* ws_max, const Tile& t, int64_t K,
                                              const TileGeom& q, long long spin_ticks, uint4& m) {
    if (spin_ticks < 0) return false;
    if (!q.col_ok) return true;
    const long long t0 = wall_clock64();
    for (int c = q.ty; c < t.nc; c += q.rps) {
        const uint64_t* src = chunk_words(ws_max, t, c, K, q);
        uint64_t w0, w1, w2, w3;
        for (;;) {
            w0 = load_agent(src);
            w1 = load_agent(src + 1);
            w2 = load_agent(src + 2);
            w3 = load_agent(src + 3);
            if ((w0 & w1 & w2 & w3) & kWordPresent) break;
            if (wall_clock64() - t0 > spin_ticks) return false;
            __builtin_amdgcn_s_sleep(8);
        }
        max4(m, make_uint4((uint32_t)w0, (uint32_t)w1, (uint32_t)w2, (uint32_t)w3));
    }
    return true;
}

// Staging of the transposed tile in LDS: per tile column a row of pw 4-byte
// words (a power of two, at least 8), word u holding the four consecutive
// rows row_a + 4u .. + 3. The 4-word group of a word index is XOR-swizzled
// with the lane's column block within its aligned block of min(pw, 64)
// words, so that the lanes of a wave writing one row quad spread over the
// banks. The register rows pass in two phases with pw = 4 * rps (room for
// four quads: 8 << lt columns x 4 * (512 >> lt) words, 16384 words at any
// strip width); the two quads of the LDS rows pass before them with
// pw = 2 * rps, in half of that.
constexpr int kStageWords = kLdsSlabs * kThreads * 4;     // 64 KiB, the LDS rows' space
static_assert(kStageWords == 16384, "stage size");
static_assert(kLdsSlabs == 8 && reg_slabs<true>() == 20,
              "the stage takes the LDS rows as quads 5..6, the register rows as quads 0..2 and 3..4");
__device__ __forceinline__ int stage_pitch(int rps) { return 4 * rps; }
__device__ __forceinline__ int stage_swizzle(int col_block, int pw) {
    const int groups = (pw < 64 ? pw : 64) >> 2;
    return (col_block & (groups - 1)) << 2;
}

// Stores rows [row_a, row_b) of the tile's ncols columns from the stage to
// q_t (qstrip: the strip's first q_t row at the tile's first row) in pieces
// of 16 rows of one column, consecutive lanes along the rows of a column:
// c = p / npc by a multiply-shift, exact since p < ncols * npc <= 3072 and
// npc <= 48.
__device__ __forceinline__ void store_staged(const uint32_t* stage, int pw, int ncols, int row_a,
                                             int row_b, uint8_t* qstrip, int64_t M) {
    const int npc = (row_b - row_a) >> 4;
    const uint32_t inv = ((1u << 20) + (uint32_t)npc - 1u) / (uint32_t)npc;
    const int total = ncols * npc;
    uint8_t* qbase = qstrip + row_a;
    for (int p = threadIdx.x; p < total; p += kThreads) {
        const int c = (int)(((uint32_t)p * inv) >> 20);
        const int k = p - c * npc;
        const uint4 val = *reinterpret_cast<const uint4*>(stage + c * pw + ((4 * k) ^ stage_swizzle(c >> 3, pw)));
        // an ordinary store: a group's run of a q_t row starts on a 16-byte
        // boundary only, and L2 merges the two tiles' parts of a shared line
        // (nontemporal partial lines cost far more)
        *reinterpret_cast<uint4*>(qbase + (int64_t)c * M + 16 * k) = val;
    }
}

// One tile: load, column amax (across chunk tiles when the group is cut),
// scales, cast. kT: q is (K, M) and scales (K, G), the transposes of dim0's
// outputs, written through the LDS stage.
template <bool kT>
__device__ __forceinline__ void dim0_body(
        const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ off, int G,
        int pow2, uint8_t* __restrict__ q, float* __restrict__ scales, int n_tiles, int team_max,
        int lt_cap, int maybe_c, uint32_t* __restrict__ ws_ctr, uint64_t* __restrict__ ws_max,
        long long spin_ticks, int uniform_rows, int xcd_split, uint4* red, uint32_t* stage, uint4* ext,
        int* search, int* vote) {
    constexpr int kRowAlign = kT ? 16 : 1;
    constexpr int kRows = rows_w128<kT>();
    constexpr int kLtRows = kT ? kDim0LtRowsT : kDim0LtRows;
    constexpr int kLine = kT ? 128 : 1;      // chunk boundaries on q_t lines (transposed output)
    constexpr int kSlabs = reg_slabs<kT>();
    const bool wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x) < kWave;

    // xcd_split: the dispatcher deals workgroups to the 8 XCDs in turn, and
    // XCD x takes the tiles of columns [x K/8, (x + 1) K/8) in their usual
    // order: the tiling of a K/8-column problem, shifted. Every strip width
    // divides K/8 (the host checks), so each column, and each output row of
    // the transposed kernel, is written from one XCD only.
    const int xcol = xcd_split ? (int)(blockIdx.x & 7) : 0;
    const int Ks = xcd_split ? K >> 3 : K;
    const unsigned first = xcd_split ? blockIdx.x >> 3 : blockIdx.x;
    const unsigned stride = xcd_split ? gridDim.x >> 3 : gridDim.x;
    // n_tiles < 2^31 and gridDim.x <= 2^22, so the unsigned sum never wraps
    for (unsigned item = first; item < (unsigned)n_tiles; item += stride) {
        MGS_TRACE_STAMP(tr0);
        Tile t = G > kWave
                     ? find_tile_wide<kRows, kLtRows, !kT, kLine>(off, G, M, Ks, team_max, lt_cap, maybe_c,
                                                                 kRowAlign, uniform_rows, (int)item, search)
                     : find_tile<kRows, kLtRows, !kT, kLine>(off, G, M, Ks, team_max, lt_cap, maybe_c,
                                                            kRowAlign, uniform_rows, (int)item);
        if (t.g < 0) break;      // later items of this workgroup lie past the last tile too
        t.strip += xcol * (Ks >> (t.lt + 3));
        const TileGeom geo = tile_geom(t, K);
        MGS_TRACE_STAMP(tr1);
        const int nrows = t.r1 - t.r0;      // at most the register capacity in every class
        // a team: the tiles of one chunked group on one strip (class C: its
        // column-maximum tiles too), with one counter in the workspace
        const bool chunked = t.cls != kClassA;
        const uint32_t team_size = t.cls == kClassT ? (uint32_t)t.nc : 2u * (uint32_t)t.nc;
        // (strips of chunked groups are 128 columns wide, or 64 in launches
        // that narrow every strip; a chunked group has at least two chunk
        // rows, so its ceil(K / 64) counters fit in its rows' slots)
        uint32_t* team_ctr = ws_ctr + (int64_t)t.cbase * ((K + 127) >> 7) + t.strip;

        uint4 m = make_uint4(0u, 0u, 0u, 0u);
        if (t.cls == kClassC && !t.maxima) {
            // casting tile of a class C group: its strip's maxima were written
            // by tiles earlier in the grid; wait for them before the tile's own
            // loads, so that no tile data sits in registers meanwhile
            const bool ok = gather_maxima(ws_max, t, K, geo, spin_ticks, m);
            if (!block_all(ok, vote)) {
                m = make_uint4(0u, 0u, 0u, 0u);
                stream_amax(x, K, t.g0, t.g1 - t.g0, geo, m);
            }
        }

        uint4 v[kSlabs];
        load_tile<kT>(x, K, t.r0, nrows, geo, v);
        // rows past the registers': into LDS
        const bool use_ext = kSlabs * geo.rps < nrows;
        if (use_ext) load_tile_ext<kT>(x, K, t.r0, nrows, geo, ext);
        if (t.cls != kClassC || t.maxima) {
#pragma unroll
            for (int s = 0; s < kSlabs; ++s)
                if (slab_row<kT>(s, geo.rps, 0) < nrows) max4(m, v[s]);
        }
        if (use_ext) {
            // every load of this thread, the LDS ones included, has landed
            __builtin_amdgcn_s_waitcnt(0);
            if (t.cls != kClassC || t.maxima) {
#pragma unroll
                for (int e = 0; e < kLdsSlabs; ++e) max4(m, ext_slab<kT>(ext, e, nrows, geo));
            }
        }

        if (t.maxima) {
            // class C column-maximum tile: publish this chunk's column maxima
            m = block_column_amax(m, geo.tpr, red);
            publish_maxima(ws_max, t, K, geo, m);
            uint32_t before = 0;
            if (wave0) {
                // this wave's words are stored before the tile counts as done
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                before = team_tile_done(team_ctr, team_size);
            }
            __syncthreads();      // ends this item's reads of red
            if (wave0 && __builtin_amdgcn_readfirstlane(before) + 1u == team_size)
                clear_team_words(ws_max, t, K);
            continue;
        }
        if (t.cls == kClassT) {
            // team tile: publish this chunk's maxima, then combine the team's
            m = block_column_amax(m, geo.tpr, red);
            publish_maxima(ws_max, t, K, geo, m);
            m = make_uint4(0u, 0u, 0u, 0u);
            // a complete gather has read this tile's own words back, so they
            // are stored before the tile counts as done
            const bool ok = gather_maxima(ws_max, t, K, geo, spin_ticks, m);
            if (!block_all(ok, vote)) {
                // the team's maxima did not come in time: the column amax of
                // the whole group from x
                m = make_uint4(0u, 0u, 0u, 0u);
                stream_amax(x, K, t.g0, t.g1 - t.g0, geo, m);
                if (wave0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
        }
        MGS_TRACE_STAMP(tr2);
        m = block_column_amax(m, geo.tpr, red);
        MGS_TRACE_STAMP(tr3);

        // every lane derives its own 8 scales; lanes of row 0 store them
        const bool p2 = pow2 != 0;
        const float s0 = group_scale(m.x & 0xFFFFu, p2), s1 = group_scale(m.x >> 16, p2);
        const float s2 = group_scale(m.y & 0xFFFFu, p2), s3 = group_scale(m.y >> 16, p2);
        const float s4 = group_scale(m.z & 0xFFFFu, p2), s5 = group_scale(m.z >> 16, p2);
        const float s6 = group_scale(m.w & 0xFFFFu, p2), s7 = group_scale(m.w >> 16, p2);
        if (!kT) {
            if (geo.col_ok) {
                if (geo.ty == 0 && t.c == 0) {
                    float4* dst = reinterpret_cast<float4*>(scales + (int64_t)t.g * K + geo.col);
                    dst[0] = make_float4(s0, s1, s2, s3);
                    dst[1] = make_float4(s4, s5, s6, s7);
                }
                // one lane base, advanced by a uniform step of rps rows
                uint8_t* qb = q + (int64_t)(t.r0 + geo.ty) * K + geo.col;
                const int64_t step = (int64_t)geo.rps * K;
#pragma unroll
                for (int s = 0; s < kSlabs; ++s) {
                    const int r_s = s * geo.rps;
                    if (r_s < nrows && r_s + geo.ty < nrows)
                        store_stream(qb, cast8_group(v[s], s0, s1, s2, s3, s4, s5, s6, s7));
                    qb += step;
                }
                if (use_ext) {
#pragma unroll
                    for (int e = 0; e < kLdsSlabs; ++e) {
                        if ((kSlabs + e) * geo.rps + geo.ty < nrows)
                            store_stream(qb, cast8_group(ext[e * kThreads + threadIdx.x], s0, s1, s2, s3,
                                                         s4, s5, s6, s7));
                        qb += step;
                    }
                }
            }
        } else {
            if (geo.col_ok && geo.ty == 0 && t.c == 0) {
                float* dst = scales + (int64_t)geo.col * G + t.g;
                dst[0] = s0;
                dst[(int64_t)G] = s1;
                dst[2 * (int64_t)G] = s2;
                dst[3 * (int64_t)G] = s3;
                dst[4 * (int64_t)G] = s4;
                dst[5 * (int64_t)G] = s5;
                dst[6 * (int64_t)G] = s6;
                dst[7 * (int64_t)G] = s7;
            }
            // Tile rows and their starts are multiples of 16, so every quad
            // is whole and every output piece is 16 aligned bytes.
            const int W = geo.tpr * 8;
            const int ncols = min(W, K - t.strip * W);
            uint8_t* qstrip = q + (int64_t)(t.strip * W) * M + t.r0;
            if (use_ext) {
                // The rows in LDS (quads 5 and 6) go first, so that all of the
                // LDS is free for the stage afterwards. Cast in place: slot e
                // of this thread (e < 4) takes the cast of its vectors e and
                // e + 4, so the upper half of the LDS (vectors 4..7) is free
                // once every thread has read its own.
                uint2* own = reinterpret_cast<uint2*>(ext + threadIdx.x);
#pragma unroll
                for (int e = 0; e < kLdsSlabs; ++e) {
                    const uint2 c = cast8_group(ext_slab<true>(ext, e, nrows, geo), s0, s1, s2, s3, s4, s5,
                                                s6, s7);
                    own[(e & 3) * 2 * kThreads + (e >> 2)] = c;
                }
                __syncthreads();
                uint32_t* st = reinterpret_cast<uint32_t*>(ext + 4 * kThreads);   // 32 KiB
                const int pw = 2 * geo.rps;           // two quads of rows per column
                uint32_t* col_base = st + geo.tx * 8 * pw;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = 4 * ((kSlabs / 4 + h) * geo.rps + geo.ty);
                    if (row < nrows && geo.col_ok) {
                        const uint2 b0 = own[0 * 2 * kThreads + h], b1 = own[1 * 2 * kThreads + h];
                        const uint2 b2 = own[2 * 2 * kThreads + h], b3 = own[3 * 2 * kThreads + h];
                        uint32_t lo[4], hi[4];
                        transpose4x4(b0.x, b1.x, b2.x, b3.x, lo);
                        transpose4x4(b0.y, b1.y, b2.y, b3.y, hi);
                        const int w = (h * geo.rps + geo.ty) ^ stage_swizzle(geo.tx, pw);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            col_base[j * pw + w] = lo[j];
                            col_base[(j + 4) * pw + w] = hi[j];
                        }
                    }
                }
                __syncthreads();
                store_staged(st, pw, ncols, kSlabs * geo.rps,
                             min(4 * (kSlabs / 4 + 2) * geo.rps, nrows), qstrip, M);
                __syncthreads();      // the stage's reads are done
            }
            // The register rows in two phases through the stage: row quads
            // 0..2, then 3..4.
            const int pw = stage_pitch(geo.rps);
            for (int ph = 0; ph < 2; ++ph) {
                const int qa = ph ? 3 : 0, qb = ph ? 5 : 3;
                const int row_a = 4 * qa * geo.rps;
                if (row_a >= nrows) break;
                const int row_b = min(4 * qb * geo.rps, nrows);
                if (ph) __syncthreads();      // the stage's first-phase reads are done
                uint32_t* col_base = stage + geo.tx * 8 * pw;
#pragma unroll
                for (int qd = 0; qd < kSlabs / 4; ++qd) {
                    if ((qd >= 3) != (ph == 1)) continue;
                    const int row = 4 * (qd * geo.rps + geo.ty);
                    if (row < nrows && geo.col_ok) {
                        const uint2 b0 = cast8_group(v[4 * qd + 0], s0, s1, s2, s3, s4, s5, s6, s7);
                        const uint2 b1 = cast8_group(v[4 * qd + 1], s0, s1, s2, s3, s4, s5, s6, s7);
                        const uint2 b2 = cast8_group(v[4 * qd + 2], s0, s1, s2, s3, s4, s5, s6, s7);
                        const uint2 b3 = cast8_group(v[4 * qd + 3], s0, s1, s2, s3, s4, s5, s6, s7);
                        uint32_t lo[4], hi[4];
                        transpose4x4(b0.x, b1.x, b2.x, b3.x, lo);
                        transpose4x4(b0.y, b1.y, b2.y, b3.y, hi);
                        const int w = ((qd - qa) * geo.rps + geo.ty) ^ stage_swizzle(geo.tx, pw);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            col_base[j * pw + w] = lo[j];
                            col_base[(j + 4) * pw + w] = hi[j];
                        }
                    }
                }
                __syncthreads();
                store_staged(stage, pw, ncols, row_a, row_b, qstrip, M);
            }
        }
#if defined(MGS_TILE_TRACE)
        // with the XCD split every XCD numbers its own tiles: record i holds
        // tile item i / 8 of XCD i % 8
        const unsigned rec = xcd_split ? item * 8u + (unsigned)xcol : item;
        if (threadIdx.x == 0 && rec < (unsigned)kTraceTiles) {
            MGS_TRACE_STAMP(tr4);
            unsigned hw, xcc;
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
            asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
            unsigned long long* d = g_tile_trace + 8 * (size_t)rec;
            d[0] = tr0;
            d[1] = tr1;
            d[2] = tr2;
            d[3] = tr3;
            d[4] = tr4;
            d[5] = ((unsigned long long)hw << 32) | xcc;
            d[6] = ((unsigned long long)t.cls << 60) | ((unsigned long long)t.c << 32) | (unsigned)nrows;
            d[7] = ((unsigned long long)t.g << 40) | ((unsigned long long)t.strip << 16) |
                   (unsigned)(8 << t.lt);
        }
#endif
        uint32_t before = 0;
        if (chunked && wave0) before = team_tile_done(team_ctr, team_size);
        __syncthreads();     // red (and the stage) are rewritten by the next item
        if (chunked && wave0 && __builtin_amdgcn_readfirstlane(before) + 1u == team_size)
            clear_team_words(ws_max, t, K);
    }
}

}  // namespace

// ws layout (Dim0Workspace): a counter per (chunk row, 128-column strip),
// then maxima[chunk row][K / 2] 64-bit words (presence tag << 32 | two 16-bit
// magnitude patterns).
__global__ __launch_bounds__(kThreads, 4) void dim0_kernel(
        const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ off, int G,
        int pow2, uint8_t* __restrict__ q, float* __restrict__ scales, int n_tiles, int team_max,
        int lt_cap, int maybe_c, uint32_t* __restrict__ ws_ctr, uint64_t* __restrict__ ws_max,
        long long spin_ticks, int uniform_rows, int xcd_split) {
    __shared__ uint4 red[kThreads];
    __shared__ uint4 ext[kLdsSlabs * kThreads];     // 64 KiB: the tile's rows past the registers
    __shared__ int search[kSearchWords];
    __shared__ int vote[kWaves];
    dim0_body<false>(x, M, K, off, G, pow2, q, scales, n_tiles, team_max, lt_cap, maybe_c, ws_ctr,
                     ws_max, spin_ticks, uniform_rows, xcd_split, red, nullptr, ext, search, vote);
}

// The same per-group scaling with transposed outputs: qT (K, M), scalesT (K, G).
__global__ __launch_bounds__(kThreads, 4) void dim0t_kernel(
        const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ off, int G,
        int pow2, uint8_t* __restrict__ q, float* __restrict__ scales, int n_tiles, int team_max,
        int lt_cap, int maybe_c, uint32_t* __restrict__ ws_ctr, uint64_t* __restrict__ ws_max,
        long long spin_ticks, int uniform_rows, int xcd_split) {
    __shared__ uint4 red[kThreads];
    __shared__ uint4 ext[kLdsSlabs * kThreads];     // 64 KiB: rows past the registers, then the stage
    __shared__ int search[kSearchWords];
    __shared__ int vote[kWaves];
    dim0_body<true>(x, M, K, off, G, pow2, q, scales, n_tiles, team_max, lt_cap, maybe_c, ws_ctr,
                    ws_max, spin_ticks, uniform_rows, xcd_split, red, reinterpret_cast<uint32_t*>(ext),
                    ext, search, vote);
}

// Zero fill of n 16-byte words (a fresh workspace; no memset node, so the
// same call also works inside a captured graph).
__global__ __launch_bounds__(256) void zero_kernel(uint4* __restrict__ p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Workgroups of dim0_kernel the device holds at once (two per CU by design:
// 72 KiB of LDS and at most 128 VGPRs each), from the runtime's occupancy
// query, kept per device; 0 if the query fails.
int dim0_resident(int cus) {
    static std::mutex mu;
    static std::map<int, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(dev);
        if (it != cache.end()) return it->second;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dim0_kernel, kThreads, 0) != hipSuccess ||
            per_cu < 1)
        return 0;
    const int resident = per_cu * (cus > 0 ? cus : 1);
    std::lock_guard<std::mutex> lock(mu);
    cache[dev] = resident;
    return resident;
}

hipError_t launch_dim0(const uint16_t* x, int M, int K, const int32_t* off, int G, int uniform_rows,
                       bool pow2, bool transposed, uint8_t* q, float* scales, int team_max, int lt_cap,
                       bool xcd_split, void* ws, long long spin_ticks, int cus, hipStream_t stream) {
    const int64_t chunk_rows = transposed ? kDim0ChunkRowsT : kDim0ChunkRows;
    const int64_t lt_rows = transposed ? kDim0LtRowsT : kDim0LtRows;
    // with xcd_split every XCD runs the tiling of K / 8 columns
    const int64_t n_tiles =
        dim0_tile_bound(M, xcd_split ? K / 8 : K, G, team_max, lt_cap, chunk_rows, lt_rows);
    if (n_tiles >= INT32_MAX) return hipErrorInvalidValue;
    const int64_t per = n_tiles < (xcd_split ? kDim0MaxGrid / 8 : kDim0MaxGrid)
                            ? n_tiles : (xcd_split ? kDim0MaxGrid / 8 : kDim0MaxGrid);
    int64_t grid = xcd_split ? 8 * per : per;
    // One group in one to three rounds of tiles (by the bound): one resident
    // round of workgroups instead, each walking its tiles b, b + grid, ...
    // with no exit, dispatch and start between them. Other launches keep one
    // workgroup per tile, which lets the hardware dispatcher balance tiles:
    // a fixed share of them was slower for groups of unequal size and for
    // equal experts alike. Teams stay consecutive in the tile order and hold
    // fewer tiles than the grid, so the lowest tile in progress always has
    // every teammate started or done.
    if (!transposed && !xcd_split && G == 1) {
        const int resident = dim0_resident(cus);
        if (resident > 0 && grid > resident && grid <= 3 * (int64_t)resident) grid = resident;
    }
    const Dim0Workspace w = dim0_workspace(M, K);
    char* base = static_cast<char*>(ws);
    uint32_t* ws_ctr = base ? reinterpret_cast<uint32_t*>(base + w.ctr_off) : nullptr;
    uint64_t* ws_max = base ? reinterpret_cast<uint64_t*>(base + w.max_off) : nullptr;
    // a group can need column-maximum tiles only if M rows make more chunks
    // than a team may have
    const int maybe_c = (int64_t)M > chunk_rows * team_max ? 1 : 0;
    hipLaunchKernelGGL(transposed ? dim0t_kernel : dim0_kernel, dim3((unsigned)grid), dim3(kThreads),
                       0, stream, x, M, K, off, G, pow2 ? 1 : 0, q, scales, (int)n_tiles, team_max,
                       lt_cap, maybe_c, ws_ctr, ws_max, spin_ticks, uniform_rows, xcd_split ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream) {
    const int64_t n = (int64_t)(bytes / 16);
    if (n == 0) return hipSuccess;
    const int64_t blocks = n / 256 + 1 < 1024 ? n / 256 + 1 : 1024;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       static_cast<uint4*>(p), n);
    return hipGetLastError();
}

}  // namespace mgs

#if defined(MGS_TILE_TRACE)
// Trace builds only: the tile timeline of the last dim0-family launches (see
// g_tile_trace). Return hipError_t codes.
extern "C" int mgs_tile_trace_capacity(void) { return mgs::kTraceTiles; }

extern "C" int mgs_tile_trace_clear(void) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(mgs::g_tile_trace));
    if (e != hipSuccess) return (int)e;
    e = hipMemset(p, 0, sizeof(mgs::g_tile_trace));
    if (e != hipSuccess) return (int)e;
    return (int)hipDeviceSynchronize();
}

namespace mgs {
namespace {
__global__ void tile_trace_stamp_kernel(unsigned long long* dst) {
    if (threadIdx.x == 0) *dst = __builtin_amdgcn_s_memrealtime();
}
}  // namespace
}  // namespace mgs

extern "C" int mgs_tile_trace_stamp(void* dst, void* stream) {
    if (!dst || (reinterpret_cast<uintptr_t>(dst) & 7)) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mgs::tile_trace_stamp_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream),
                       static_cast<unsigned long long*>(dst));
    return (int)hipGetLastError();
}

extern "C" int mgs_tile_trace_read(void* dst, int64_t bytes) {
    if (!dst || bytes < 0 || (size_t)bytes > sizeof(mgs::g_tile_trace)) return (int)hipErrorInvalidValue;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return (int)e;
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(mgs::g_tile_trace), (size_t)bytes, 0,
                                    hipMemcpyDeviceToHost);
}
#endif
