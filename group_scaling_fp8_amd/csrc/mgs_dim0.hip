// mgs_dim0.hip — per-token-group scaling along dim0 on gfx950.
//
// Method: "[moe training] use smaller block sizes for per group scaling
// kernels to improve perf", description (per-token-group scaling along dim0:
// one scale per (group, column)) and its kernel-argument dict (448, 1e-12,
// power-of-two rounding). That page's fix was filling every compute unit
// when groups are small; here every (group, 128-column strip) pair is its
// own workgroup, and tall groups are split into row chunks, so the grid
// scales with M and K rather than with the group count.
//
// Work decomposition (all decided on the device from the offsets, so the
// host never reads them):
//   * A group of at most kChunkRows rows is one chunk. A taller group is cut
//     into ceil(rows / kChunkRows) near-equal chunks.
//   * Workgroup item = (chunk, strip of 128 columns). 256 threads: 16 lanes
//     per row, each lane holding 8 columns (one 16-byte load), 16 rows per
//     slab, up to 32 slabs held in registers. So a whole chunk (<= 512 rows
//     x 128 columns, 128 KiB of bf16) is read from HBM exactly once.
//   * Single-chunk groups: load -> column amax -> scale -> cast from
//     registers -> store. One pass.
//   * Multi-chunk groups: a first kernel writes each chunk's column amax to
//     a workspace; the main kernel combines the group's partials, then
//     re-reads its chunk and casts. This second read is the only extra
//     traffic, and only tall groups pay it.
#include "mgs_device.hpp"
#include "mgs_kernels.hpp"

namespace mgs {

namespace {

constexpr int kThreads = 256;
constexpr int kTpr = 16;                   // lanes per row
constexpr int kRowsPerSlab = kThreads / kTpr;
constexpr int kSlabs = kDim0Slabs;
constexpr int kChunkRows = kRowsPerSlab * kSlabs;
constexpr int kStripCols = kTpr * 8;
static_assert(kChunkRows == kDim0ChunkRows, "chunk size mismatch");
static_assert(kStripCols == kDim0StripCols, "strip width mismatch");

struct Chunk {
    int g;          // group index, or -1 if the item does not exist
    int c;          // chunk index within the group
    int nc;         // chunks in the group
    int big_base;   // index of the group's first chunk among tall-group chunks
    int r0, r1;     // rows of this chunk
};

// One wave walks the group table in tiles of 64 groups and finds chunk
// `target`, counting all chunks (tall_only = false) or only the chunks of
// groups taller than kChunkRows (tall_only = true). Offsets are sanitised
// on the fly: end[g] = min(max(off[0..g]), M), clamped below at 0, so any
// offsets array gives in-range rows.
__device__ void find_chunk(const int32_t* __restrict__ off, int G, int M, int target,
                           bool tall_only, Chunk* out) {
    const int lane = threadIdx.x & (kWave - 1);
    int carry_end = 0, carry_cnt = 0, carry_big = 0;
    for (int base = 0; base < G; base += kWave) {
        const int g = base + lane;
        int raw = g < G ? off[g] : M;
        raw = min(max(raw, 0), M);
        const int end = max(wave_prefix_imax(raw), carry_end);
        int start = __shfl_up(end, 1, kWave);
        if (lane == 0) start = carry_end;
        const int size = end - start;
        const int nc = (g < G) ? (size <= kChunkRows ? 1 : (size + kChunkRows - 1) / kChunkRows) : 0;
        const int nbig = (size > kChunkRows) ? nc : 0;
        const int cnt = tall_only ? nbig : nc;
        const int incl = wave_prefix_sum(cnt) + carry_cnt;
        const int bincl = wave_prefix_sum(nbig) + carry_big;
        const bool hit = cnt > 0 && target >= incl - cnt && target < incl;
        if (hit) {
            const int c = target - (incl - cnt);
            const int cs = (size + nc - 1) / nc;
            out->g = g;
            out->c = c;
            out->nc = nc;
            out->big_base = bincl - nbig;
            out->r0 = min(start + c * cs, end);
            out->r1 = min(start + (c + 1) * cs, end);
        }
        if (__any(hit)) return;
        carry_end = __shfl(end, kWave - 1, kWave);
        carry_cnt = __shfl(incl, kWave - 1, kWave);
        carry_big = __shfl(bincl, kWave - 1, kWave);
    }
    if (lane == 0) out->g = -1;
}

// Loads the chunk's rows of this lane's 8 columns into registers (zeros for
// rows past the chunk or columns past K).
__device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ x, int64_t K, int r0,
                                           int nrows, int ty, int64_t col, bool col_ok,
                                           uint4 (&v)[kSlabs]) {
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
        v[s] = make_uint4(0u, 0u, 0u, 0u);
        if (s * kRowsPerSlab < nrows) {
            const int rr = s * kRowsPerSlab + ty;
            if (rr < nrows && col_ok)
                v[s] = *reinterpret_cast<const uint4*>(x + (int64_t)(r0 + rr) * K + col);
        }
    }
}

// Per-lane column amax of the chunk held in registers, as four packed pairs
// of 15-bit magnitudes (lane tx holds columns 8tx..8tx+7).
__device__ __forceinline__ uint4 lane_column_amax(const uint4 (&v)[kSlabs], int nrows) {
    uint32_t m0 = 0, m1 = 0, m2 = 0, m3 = 0;
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
        if (s * kRowsPerSlab < nrows) {
            m0 = mag_max2(m0, v[s].x);
            m1 = mag_max2(m1, v[s].y);
            m2 = mag_max2(m2, v[s].z);
            m3 = mag_max2(m3, v[s].w);
        }
    }
    return make_uint4(m0, m1, m2, m3);
}

// Combines the per-lane values of all lanes that share a column set (same
// tx, every ty) and returns the result in threads 0..kTpr-1.
__device__ __forceinline__ uint4 block_column_amax(uint4 m, uint4 (*red)[kTpr]) {
    // lanes tx, tx+16, tx+32, tx+48 of a wave share columns
#pragma unroll
    for (int d = kTpr; d < kWave; d <<= 1) {
        m.x = mag_max2(m.x, __shfl_xor(m.x, d, kWave));
        m.y = mag_max2(m.y, __shfl_xor(m.y, d, kWave));
        m.z = mag_max2(m.z, __shfl_xor(m.z, d, kWave));
        m.w = mag_max2(m.w, __shfl_xor(m.w, d, kWave));
    }
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    if (lane < kTpr) red[wave][lane] = m;
    __syncthreads();
    uint4 r = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x < kTpr) {
#pragma unroll
        for (int w = 0; w < kThreads / kWave; ++w) {
            const uint4 t = red[w][threadIdx.x];
            r.x = mag_max2(r.x, t.x);
            r.y = mag_max2(r.y, t.y);
            r.z = mag_max2(r.z, t.z);
            r.w = mag_max2(r.w, t.w);
        }
    }
    return r;
}

}  // namespace

// First pass for groups taller than one chunk: each (tall chunk, strip)
// writes its 8-per-lane column amax (one uint32 per column) to
// ws[tall_chunk * K + column].
__global__ __launch_bounds__(kThreads) void dim0_tall_partials_kernel(
        const uint16_t* __restrict__ x, int M, int64_t K, const int32_t* __restrict__ off,
        int G, int n_strips, uint32_t* __restrict__ ws) {
    __shared__ Chunk info;
    __shared__ uint4 red[kThreads / kWave][kTpr];
    const int target = blockIdx.x / n_strips;
    const int strip = blockIdx.x % n_strips;
    if (threadIdx.x < kWave) find_chunk(off, G, M, target, true, &info);
    __syncthreads();
    if (info.g < 0) return;
    const int tx = threadIdx.x % kTpr, ty = threadIdx.x / kTpr;
    const int64_t col = (int64_t)strip * kStripCols + tx * 8;
    const bool col_ok = col < K;
    const int nrows = info.r1 - info.r0;
    uint4 v[kSlabs];
    load_chunk(x, K, info.r0, nrows, ty, col, col_ok, v);
    const uint4 m = block_column_amax(lane_column_amax(v, nrows), red);
    if (threadIdx.x < kTpr && col_ok) {
        uint32_t* dst = ws + (int64_t)(info.big_base + info.c) * K + col;
        reinterpret_cast<uint4*>(dst)[0] = make_uint4(m.x & 0xFFFFu, m.x >> 16, m.y & 0xFFFFu, m.y >> 16);
        reinterpret_cast<uint4*>(dst)[1] = make_uint4(m.z & 0xFFFFu, m.z >> 16, m.w & 0xFFFFu, m.w >> 16);
    }
}

// Main pass: one workgroup per (chunk, strip) of every group, empty groups
// included (they write their scale row).
__global__ __launch_bounds__(kThreads) void dim0_main_kernel(
        const uint16_t* __restrict__ x, int M, int64_t K, const int32_t* __restrict__ off,
        int G, int n_strips, int pow2, uint8_t* __restrict__ q, float* __restrict__ scales,
        const uint32_t* __restrict__ ws) {
    __shared__ Chunk info;
    __shared__ uint4 red[kThreads / kWave][kTpr];
    __shared__ float s_scale[kTpr][8];
    const int target = blockIdx.x / n_strips;
    const int strip = blockIdx.x % n_strips;
    if (threadIdx.x < kWave) find_chunk(off, G, M, target, false, &info);
    __syncthreads();
    if (info.g < 0) return;
    const int tx = threadIdx.x % kTpr, ty = threadIdx.x / kTpr;
    const int64_t col = (int64_t)strip * kStripCols + tx * 8;
    const bool col_ok = col < K;
    const int nrows = info.r1 - info.r0;
    const bool tall = info.nc > 1;

    uint4 v[kSlabs];
    load_chunk(x, K, info.r0, nrows, ty, col, col_ok, v);

    // Column amax: from the registers for a single-chunk group, else from
    // the tall-group partials (chunks spread over the ty lanes).
    uint4 m = make_uint4(0u, 0u, 0u, 0u);
    if (!tall) {
        m = lane_column_amax(v, nrows);
    } else if (col_ok) {
        for (int c = ty; c < info.nc; c += kRowsPerSlab) {
            const uint4* src = reinterpret_cast<const uint4*>(ws + (int64_t)(info.big_base + c) * K + col);
            const uint4 a = src[0], b = src[1];
            m.x = mag_max2(m.x, a.x | (a.y << 16));
            m.y = mag_max2(m.y, a.z | (a.w << 16));
            m.z = mag_max2(m.z, b.x | (b.y << 16));
            m.w = mag_max2(m.w, b.z | (b.w << 16));
        }
    }
    m = block_column_amax(m, red);
    if (threadIdx.x < kTpr) {
        const bool p2 = pow2 != 0;
        float s[8];
        s[0] = group_scale(m.x & 0xFFFFu, p2);
        s[1] = group_scale(m.x >> 16, p2);
        s[2] = group_scale(m.y & 0xFFFFu, p2);
        s[3] = group_scale(m.y >> 16, p2);
        s[4] = group_scale(m.z & 0xFFFFu, p2);
        s[5] = group_scale(m.z >> 16, p2);
        s[6] = group_scale(m.w & 0xFFFFu, p2);
        s[7] = group_scale(m.w >> 16, p2);
#pragma unroll
        for (int i = 0; i < 8; ++i) s_scale[threadIdx.x][i] = s[i];
        if (col_ok && info.c == 0) {
            float4* dst = reinterpret_cast<float4*>(scales + (int64_t)info.g * K + col);
            dst[0] = make_float4(s[0], s[1], s[2], s[3]);
            dst[1] = make_float4(s[4], s[5], s[6], s[7]);
        }
    }
    __syncthreads();
    if (!col_ok) return;
    const float s0 = s_scale[tx][0], s1 = s_scale[tx][1], s2 = s_scale[tx][2], s3 = s_scale[tx][3];
    const float s4 = s_scale[tx][4], s5 = s_scale[tx][5], s6 = s_scale[tx][6], s7 = s_scale[tx][7];
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
        if (s * kRowsPerSlab < nrows) {
            const int rr = s * kRowsPerSlab + ty;
            if (rr < nrows) {
                const uint2 o = cast8(v[s], s0, s1, s2, s3, s4, s5, s6, s7);
                *reinterpret_cast<uint2*>(q + (int64_t)(info.r0 + rr) * K + col) = o;
            }
        }
    }
}

hipError_t launch_dim0(const uint16_t* x, int M, int64_t K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, uint32_t* ws, int64_t tall_chunk_bound,
                       hipStream_t stream) {
    const int n_strips = (int)((K + kStripCols - 1) / kStripCols);
    if (tall_chunk_bound > 0) {
        const int64_t blocks = tall_chunk_bound * n_strips;
        hipLaunchKernelGGL(dim0_tall_partials_kernel, dim3((unsigned)blocks), dim3(kThreads), 0,
                           stream, x, M, K, off, G, n_strips, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t chunks = dim0_chunk_bound(M, G);
    const int64_t blocks = chunks * n_strips;
    hipLaunchKernelGGL(dim0_main_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, M,
                       K, off, G, n_strips, pow2 ? 1 : 0, q, scales, ws);
    return hipGetLastError();
}

}  // namespace mgs
