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
// Tiling (all decided on the device from the offsets; the host never reads
// them). A workgroup has 512 threads and holds up to kSlabs 16-byte vectors
// per thread in registers (160 KiB of bf16). Its tile is R rows of one group
// times a strip of 8 * tpr columns, with tpr lanes per row:
//   * class A, R <= 1280 rows: one pass. tpr is the widest power of two in
//     [16, 128] whose tile still fits (short groups get strips up to 1024
//     columns wide), or 8 (64-column strips) for groups of 641..1280 rows.
//     Load -> column amax -> scale -> cast from registers -> store.
//   * class B, 1280 < R <= 5120: 64-column strips; the first 1280 rows stay in
//     registers and the rest is read twice (once for the amax, once for the
//     cast).
//   * class C, R > 5120: the group is cut into chunks of at most 640 rows
//     (128-column strips). A first kernel writes every chunk's column amax
//     to a workspace; the main kernel combines them, then casts its chunk
//     from registers. The chunk is read twice. That kernel is launched only
//     when M > 5120.
// Items are numbered group by group (chunk by chunk, strips fastest inside a
// group) and the workgroups are persistent: workgroup b takes items b,
// b + grid, ..., so workgroups that run at the same time read neighbouring
// strips of the same rows. Every workgroup builds the group plan once, in
// LDS, so an item costs no global lookup.
#include "mgs_device.hpp"
#include "mgs_kernels.hpp"

namespace mgs {

namespace {

constexpr int kThreads = 512;
constexpr int kSlabs = kDim0Slabs;                    // vectors per thread
constexpr int kCap = kThreads * kSlabs;               // vectors per tile
constexpr int kRowsW64 = kCap / 8;                    // 1280 rows at 64 columns
constexpr int kRowsW128 = kCap / 16;                  // 640 rows at 128 columns
static_assert(kRowsW128 == kDim0HugeChunkRows, "chunk size mismatch");
static_assert(kRowsW64 * 4 == kDim0HugeRows, "huge-group threshold mismatch");

enum { kClassA = 0, kClassB = 1, kClassC = 2 };

struct Tile {
    int g;          // group, or -1 when the item does not exist
    int cls;        // kClassA / kClassB / kClassC
    int lt;         // log2 of lanes per row (3..7)
    int strip;      // column strip index (strip width 8 << lt)
    int c, nc;      // chunk index and chunk count (class C), else 0 and 1
    int r0, r1;     // rows of this tile (the chunk for class C)
    int cbase;      // class C: index of the group's first chunk in the workspace
};

// Log2 lanes per row for a group of R rows, and its class.
__device__ __forceinline__ void choose_tiling(int R, int K, int* lt_out, int* cls_out) {
    int lt, cls;
    if (R > kDim0HugeRows) {
        lt = 4;
        cls = kClassC;
    } else if (R > kRowsW64) {
        lt = 3;
        cls = kClassB;
    } else if (R > kRowsW128) {
        lt = 3;
        cls = kClassA;
    } else {
        lt = 7;
        while (lt > 4 && R * (1 << lt) > kCap) --lt;
        cls = kClassA;
    }
    // no strip wider than needed to cover K
    while (lt > 3 && (8 << (lt - 1)) >= K) --lt;
    *lt_out = lt;
    *cls_out = cls;
}

// Per-workgroup plan of every group, in LDS: first row, rows, class, log2
// lanes per row, strip count, chunk count, end of its item range and (class C)
// index of its first chunk in the workspace. Built once per workgroup by
// wave 0. Offsets are sanitised on the fly: end[g] = min(max(off[0..g]), M),
// clamped below at 0, so any offsets array gives in-range rows.
struct Plan {
    int start[kMaxGroups];
    int rows[kMaxGroups];
    int code[kMaxGroups];     // cls | lt << 4
    int iend[kMaxGroups];     // inclusive prefix of items, in group order
    int cbase[kMaxGroups];    // class C: first workspace chunk of the group
    int total;
};

// huge_only: count only the class C chunks (the partial-amax kernel's items)
__device__ void build_plan(const int32_t* __restrict__ off, int G, int M, int K, bool huge_only,
                           Plan* p) {
    if (threadIdx.x >= kWave) return;
    const int lane = threadIdx.x;
    int carry_end = 0, carry_cnt = 0, carry_chunks = 0;
    for (int base = 0; base < G; base += kWave) {
        const int g = base + lane;
        int raw = g < G ? off[g] : M;
        raw = min(max(raw, 0), M);
        const int end = max(wave_prefix_imax(raw), carry_end);
        int start = __shfl_up(end, 1, kWave);
        if (lane == 0) start = carry_end;
        const int R = end - start;
        int lt, cls;
        choose_tiling(R, K, &lt, &cls);
        const int ns = (K + (8 << lt) - 1) / (8 << lt);
        const int nc = cls == kClassC ? (R + kRowsW128 - 1) / kRowsW128 : 1;
        const int chunks_c = (g < G && cls == kClassC) ? nc : 0;
        int cnt = 0;
        if (g < G) cnt = huge_only ? chunks_c * ns : nc * ns;
        const int incl = wave_prefix_sum(cnt) + carry_cnt;
        const int cincl = wave_prefix_sum(chunks_c) + carry_chunks;
        if (g < G) {
            p->start[g] = start;
            p->rows[g] = R;
            p->code[g] = cls | (lt << 4);
            p->iend[g] = incl;
            p->cbase[g] = cincl - chunks_c;
        }
        carry_end = __shfl(end, kWave - 1, kWave);
        carry_cnt = __shfl(incl, kWave - 1, kWave);
        carry_chunks = __shfl(cincl, kWave - 1, kWave);
    }
    if (lane == 0) p->total = carry_cnt;
}

// Tile of item `item` (item < p->total): the group is the first g with
// iend[g] > item; inside a group items run chunk by chunk, strips fastest.
__device__ __forceinline__ Tile tile_of(const Plan* p, int G, int K, int item) {
    int lo = 0, hi = G - 1;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (p->iend[mid] > item) hi = mid; else lo = mid + 1;
    }
    Tile t;
    const int g = lo;
    const int code = p->code[g];
    t.g = g;
    t.cls = code & 15;
    t.lt = code >> 4;
    const int ns = (K + (8 << t.lt) - 1) / (8 << t.lt);
    const int R = p->rows[g], start = p->start[g];
    t.nc = t.cls == kClassC ? (R + kRowsW128 - 1) / kRowsW128 : 1;
    const int local = item - (p->iend[g] - t.nc * ns);
    t.c = local / ns;
    t.strip = local - t.c * ns;
    if (t.cls == kClassC) {
        const int cs = (R + t.nc - 1) / t.nc;
        t.r0 = min(start + t.c * cs, start + R);
        t.r1 = min(start + (t.c + 1) * cs, start + R);
    } else {
        t.r0 = start;
        t.r1 = start + R;
    }
    t.cbase = p->cbase[g];
    return t;
}

__device__ __forceinline__ void max4(uint4& m, const uint4& t) {
    m.x = mag_max2(m.x, t.x);
    m.y = mag_max2(m.y, t.y);
    m.z = mag_max2(m.z, t.z);
    m.w = mag_max2(m.w, t.w);
}

// Column amax over every lane that shares this lane's 8 columns (same
// tx = lane mod tpr). The result is valid in threads 0..tpr-1.
__device__ __forceinline__ uint4 block_column_amax(uint4 m, int tpr, uint4* red) {
    for (int d = tpr; d < kWave; d <<= 1) {
        m.x = mag_max2(m.x, __shfl_xor(m.x, d, kWave));
        m.y = mag_max2(m.y, __shfl_xor(m.y, d, kWave));
        m.z = mag_max2(m.z, __shfl_xor(m.z, d, kWave));
        m.w = mag_max2(m.w, __shfl_xor(m.w, d, kWave));
    }
    red[threadIdx.x] = m;
    __syncthreads();
    uint4 a = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x < tpr) {
        const int stride = tpr > kWave ? tpr : kWave;
        for (int k = threadIdx.x; k < kThreads; k += stride) max4(a, red[k]);
    }
    return a;
}

struct TileGeom {
    int tpr, tx, ty, rps, col;
    bool col_ok;
};

__device__ __forceinline__ TileGeom tile_geom(const Tile& t, int K) {
    TileGeom q;
    q.tpr = 1 << t.lt;
    q.tx = threadIdx.x & (q.tpr - 1);
    q.ty = threadIdx.x >> t.lt;
    q.rps = kThreads >> t.lt;
    q.col = t.strip * (q.tpr * 8) + q.tx * 8;
    q.col_ok = q.col < K;
    return q;
}

// Loads the first nreg rows of the tile into registers (zeros elsewhere).
__device__ __forceinline__ void load_tile(const uint16_t* __restrict__ x, int64_t K, int r0, int nreg,
                                          const TileGeom& q, uint4 (&v)[kSlabs]) {
#pragma unroll
    for (int s = 0; s < kSlabs; ++s) {
        v[s] = make_uint4(0u, 0u, 0u, 0u);
        if (s * q.rps < nreg) {
            const int rr = s * q.rps + q.ty;
            if (rr < nreg && q.col_ok)
                v[s] = *reinterpret_cast<const uint4*>(x + (int64_t)(r0 + rr) * K + q.col);
        }
    }
}

constexpr int kStreamSlabs = 4;     // rows in flight per lane for streamed (class B) rows

}  // namespace

// Class C first pass: column amax of every (chunk, 128-column strip) of the
// groups taller than kDim0HugeRows, to ws[chunk * K + column]. Persistent:
// workgroup b takes items b, b + grid, ...; it exits at once when no group
// is that tall.
__global__ __launch_bounds__(kThreads) void dim0_huge_partials_kernel(
        const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ off, int G,
        uint32_t* __restrict__ ws) {
    __shared__ Plan plan;
    __shared__ uint4 red[kThreads];
    build_plan(off, G, M, K, true, &plan);
    __syncthreads();
    for (int item = blockIdx.x; item < plan.total; item += gridDim.x) {
        const Tile t = tile_of(&plan, G, K, item);
        const TileGeom q = tile_geom(t, K);
        const int nrows = t.r1 - t.r0;
        uint4 v[kSlabs];
        load_tile(x, K, t.r0, nrows, q, v);
        uint4 m = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int s = 0; s < kSlabs; ++s)
            if (s * q.rps < nrows) max4(m, v[s]);
        m = block_column_amax(m, q.tpr, red);
        if (threadIdx.x < q.tpr && q.col_ok) {
            uint32_t* dst = ws + (int64_t)(t.cbase + t.c) * K + q.col;
            reinterpret_cast<uint4*>(dst)[0] = make_uint4(m.x & 0xFFFFu, m.x >> 16, m.y & 0xFFFFu, m.y >> 16);
            reinterpret_cast<uint4*>(dst)[1] = make_uint4(m.z & 0xFFFFu, m.z >> 16, m.w & 0xFFFFu, m.w >> 16);
        }
        __syncthreads();     // red is reused by the next item
    }
}

// Main pass, persistent: workgroup b takes items b, b + grid, ... of every
// group, empty groups included (they write their scale row).
__global__ __launch_bounds__(kThreads) void dim0_main_kernel(
        const uint16_t* __restrict__ x, int M, int K, const int32_t* __restrict__ off, int G,
        int pow2, uint8_t* __restrict__ q, float* __restrict__ scales,
        const uint32_t* __restrict__ ws) {
    __shared__ Plan plan;
    __shared__ uint4 red[kThreads];
    __shared__ float s_scale[128 * 8];
    build_plan(off, G, M, K, false, &plan);
    __syncthreads();
    const bool p2 = pow2 != 0;
    for (int item = blockIdx.x; item < plan.total; item += gridDim.x) {
        const Tile t = tile_of(&plan, G, K, item);
        const TileGeom geo = tile_geom(t, K);
        const int nrows = t.r1 - t.r0;
        const int nreg = min(nrows, geo.rps * kSlabs);     // rows held in registers

        uint4 v[kSlabs];
        load_tile(x, K, t.r0, nreg, geo, v);

        uint4 m = make_uint4(0u, 0u, 0u, 0u);
        if (t.cls == kClassC) {
            // column amax of the whole group from the first pass's partials
            if (geo.col_ok) {
                for (int c = geo.ty; c < t.nc; c += geo.rps) {
                    const uint4* src = reinterpret_cast<const uint4*>(ws + (int64_t)(t.cbase + c) * K + geo.col);
                    const uint4 a = src[0], b = src[1];
                    max4(m, make_uint4(a.x | (a.y << 16), a.z | (a.w << 16), b.x | (b.y << 16), b.z | (b.w << 16)));
                }
            }
        } else {
            // class B: rows past the register capacity are streamed for the amax
            for (int base = nreg; base < nrows; base += kStreamSlabs * geo.rps) {
                uint4 u[kStreamSlabs];
#pragma unroll
                for (int b = 0; b < kStreamSlabs; ++b) {
                    u[b] = make_uint4(0u, 0u, 0u, 0u);
                    const int rr = base + b * geo.rps + geo.ty;
                    if (rr < nrows && geo.col_ok)
                        u[b] = *reinterpret_cast<const uint4*>(x + (int64_t)(t.r0 + rr) * K + geo.col);
                }
#pragma unroll
                for (int b = 0; b < kStreamSlabs; ++b) max4(m, u[b]);
            }
#pragma unroll
            for (int s = 0; s < kSlabs; ++s)
                if (s * geo.rps < nreg) max4(m, v[s]);
        }
        m = block_column_amax(m, geo.tpr, red);

        if (threadIdx.x < geo.tpr) {
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
            for (int i = 0; i < 8; ++i) s_scale[threadIdx.x * 8 + i] = s[i];
            if (geo.col_ok && t.c == 0) {
                float4* dst = reinterpret_cast<float4*>(scales + (int64_t)t.g * K + geo.col);
                dst[0] = make_float4(s[0], s[1], s[2], s[3]);
                dst[1] = make_float4(s[4], s[5], s[6], s[7]);
            }
        }
        __syncthreads();
        if (geo.col_ok) {
            const float* ss = s_scale + geo.tx * 8;
            const float s0 = ss[0], s1 = ss[1], s2 = ss[2], s3 = ss[3];
            const float s4 = ss[4], s5 = ss[5], s6 = ss[6], s7 = ss[7];
#pragma unroll
            for (int s = 0; s < kSlabs; ++s) {
                if (s * geo.rps < nreg) {
                    const int rr = s * geo.rps + geo.ty;
                    if (rr < nreg)
                        *reinterpret_cast<uint2*>(q + (int64_t)(t.r0 + rr) * K + geo.col) =
                            cast8(v[s], s0, s1, s2, s3, s4, s5, s6, s7);
                }
            }
            // class B: second read of the streamed rows
            for (int base = nreg; base < nrows; base += kStreamSlabs * geo.rps) {
                uint4 u[kStreamSlabs];
#pragma unroll
                for (int b = 0; b < kStreamSlabs; ++b) {
                    u[b] = make_uint4(0u, 0u, 0u, 0u);
                    const int rr = base + b * geo.rps + geo.ty;
                    if (rr < nrows) u[b] = *reinterpret_cast<const uint4*>(x + (int64_t)(t.r0 + rr) * K + geo.col);
                }
#pragma unroll
                for (int b = 0; b < kStreamSlabs; ++b) {
                    const int rr = base + b * geo.rps + geo.ty;
                    if (rr < nrows)
                        *reinterpret_cast<uint2*>(q + (int64_t)(t.r0 + rr) * K + geo.col) =
                            cast8(u[b], s0, s1, s2, s3, s4, s5, s6, s7);
                }
            }
        }
        __syncthreads();     // s_scale and red are reused by the next item
    }
}

hipError_t launch_dim0(const uint16_t* x, int M, int K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, uint32_t* ws, int grid, hipStream_t stream) {
    if (M > kDim0HugeRows) {
        hipLaunchKernelGGL(dim0_huge_partials_kernel, dim3((unsigned)grid), dim3(kThreads), 0,
                           stream, x, M, K, off, G, ws);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(dim0_main_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, x, M, K,
                       off, G, pow2 ? 1 : 0, q, scales, ws);
    return hipGetLastError();
}

}  // namespace mgs
