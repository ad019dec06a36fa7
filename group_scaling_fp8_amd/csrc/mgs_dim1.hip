// mgs_dim1.hip — per-group rowwise scaling (groups along dim1) on gfx950.
//
// Method: "[moe fp8 training] test and bench new faster method for per group
// rowwise scaling", Summary: one scale per (row, token group) of a row-major
// tensor whose token groups run along the contiguous dim. The slow kernel on
// that page lost its time to uncoalesced accesses; here every access runs
// along the contiguous dim:
//   * a workgroup (256 threads) owns whole rows; lane l of wave w holds the
//     16-byte vectors w*64 + l + 256*j (j < V), so each load instruction
//     reads 1 KiB of a row contiguously;
//   * group boundaries are multiples of 16 columns (token-group alignment
//     16, "[moe training] use smaller block sizes ..." test source), so a
//     vector never straddles two groups;
//   * per-(row, group) amax is a segmented reduction: the key
//     (group << 16) | max|x| of each vector goes through a 64-lane prefix
//     max (DPP), which never mixes groups because group ids grow along the
//     row; the last lane of each group segment then does one LDS atomic max;
//   * the row stays in registers between the amax and the cast (single pass)
//     whenever it fits in 256 * V * 8 columns. Longer rows are processed in
//     column chunks and re-read for the cast.
#include "mgs_device.hpp"
#include "mgs_kernels.hpp"

namespace mgs {

namespace {

constexpr int kThreads = 256;

// Group of the vector starting at column col: the first g with end[g] > col,
// or G if none (columns past the last offset belong to no group).
__device__ __forceinline__ int group_of(const int* s_end, int G, int col) {
    int lo = 0, hi = G;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_end[mid] > col) hi = mid; else lo = mid + 1;
    }
    return lo;
}

template <int V>
__global__ __launch_bounds__(kThreads) void dim1_kernel(
        const uint16_t* __restrict__ x, int64_t M, int K, const int32_t* __restrict__ off, int G,
        int pow2, uint8_t* __restrict__ q, float* __restrict__ scales, int rows_per_block) {
    extern __shared__ int smem[];
    int* s_end = smem;                                                   // G
    uint32_t* s_amax = reinterpret_cast<uint32_t*>(smem + G);           // G
    float* s_scale = reinterpret_cast<float*>(smem + 2 * G);            // G

    const int lane = threadIdx.x & (kWave - 1);
    if (threadIdx.x < kWave) {
        // sanitised end offsets: running max of the clamped raw values
        int carry = 0;
        for (int base = 0; base < G; base += kWave) {
            const int g = base + lane;
            int raw = g < G ? off[g] : K;
            raw = min(max(raw, 0), K);
            const int end = max(wave_prefix_imax(raw), carry);
            if (g < G) s_end[g] = end;
            carry = __shfl(end, kWave - 1, kWave);
        }
    }
    for (int t = threadIdx.x; t < G; t += kThreads) s_amax[t] = 0u;
    __syncthreads();

    const int64_t row0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t row1 = min(row0 + rows_per_block, M);
    const int chunk_cols = kThreads * V * 8;
    const int n_cc = (K + chunk_cols - 1) / chunk_cols;
    const bool p2 = pow2 != 0;

    int gid[V];
    bool tail[V];
    auto map_slots = [&](int cc) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int col = cc * chunk_cols + (threadIdx.x + j * kThreads) * 8;
            int g = G;
            bool t = false;
            if (col < K) {
                g = group_of(s_end, G, col);
                t = (g < G) && (lane == kWave - 1 || col + 8 >= s_end[g]);
            }
            gid[j] = g;
            tail[j] = t;
        }
    };
    auto load_slots = [&](const uint16_t* xr, int cc, uint4 (&v)[V]) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int col = cc * chunk_cols + (threadIdx.x + j * kThreads) * 8;
            v[j] = make_uint4(0u, 0u, 0u, 0u);
            if (gid[j] < G) v[j] = *reinterpret_cast<const uint4*>(xr + col);
        }
    };
    auto amax_slots = [&](const uint4 (&v)[V]) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            uint32_t key = 0u;
            if (gid[j] < G) key = ((uint32_t)gid[j] << 16) | mag_fold(mag_max8(0u, v[j]));
            key = wave_prefix_max(key);
            if (tail[j]) atomicMax(&s_amax[gid[j]], key & 0xFFFFu);
        }
    };
    auto cast_slots = [&](uint8_t* qr, int cc, const uint4 (&v)[V]) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            if (gid[j] < G) {
                const int col = cc * chunk_cols + (threadIdx.x + j * kThreads) * 8;
                *reinterpret_cast<uint2*>(qr + col) = cast8(v[j], s_scale[gid[j]]);
            }
        }
    };

    uint4 v[V];
    if (n_cc == 1) map_slots(0);
    for (int64_t row = row0; row < row1; ++row) {
        const uint16_t* xr = x + row * (int64_t)K;
        uint8_t* qr = q + row * (int64_t)K;
        for (int cc = 0; cc < n_cc; ++cc) {
            if (n_cc > 1) map_slots(cc);
            load_slots(xr, cc, v);
            amax_slots(v);
        }
        __syncthreads();
        for (int t = threadIdx.x; t < G; t += kThreads) {
            const float s = group_scale(s_amax[t], p2);
            s_scale[t] = s;
            scales[row * G + t] = s;
            s_amax[t] = 0u;
        }
        __syncthreads();
        for (int cc = 0; cc < n_cc; ++cc) {
            if (n_cc > 1) {
                map_slots(cc);
                load_slots(xr, cc, v);      // second read of long rows
            }
            cast_slots(qr, cc, v);
        }
    }
}

template <int V>
hipError_t launch_v(const uint16_t* x, int64_t M, int K, const int32_t* off, int G, bool pow2,
                    uint8_t* q, float* scales, hipStream_t stream) {
    // Enough workgroups to fill 256 CUs several times over, a few rows each.
    int64_t rpb = M / (256 * 8);
    rpb = rpb < 1 ? 1 : (rpb > 64 ? 64 : rpb);
    const int64_t blocks = (M + rpb - 1) / rpb;
    const size_t shmem = (size_t)3 * G * sizeof(int);
    hipLaunchKernelGGL(dim1_kernel<V>, dim3((unsigned)blocks), dim3(kThreads), shmem, stream, x, M,
                       K, off, G, pow2 ? 1 : 0, q, scales, (int)rpb);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dim1(const uint16_t* x, int64_t M, int K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, hipStream_t stream) {
    const int vecs_per_thread = (K / 8 + kThreads - 1) / kThreads;
    if (vecs_per_thread <= 1) return launch_v<1>(x, M, K, off, G, pow2, q, scales, stream);
    if (vecs_per_thread <= 2) return launch_v<2>(x, M, K, off, G, pow2, q, scales, stream);
    if (vecs_per_thread <= 4) return launch_v<4>(x, M, K, off, G, pow2, q, scales, stream);
    if (vecs_per_thread <= 6) return launch_v<6>(x, M, K, off, G, pow2, q, scales, stream);
    if (vecs_per_thread <= 9) return launch_v<9>(x, M, K, off, G, pow2, q, scales, stream);
    if (vecs_per_thread <= 12) return launch_v<12>(x, M, K, off, G, pow2, q, scales, stream);
    return launch_v<16>(x, M, K, off, G, pow2, q, scales, stream);
}

}  // namespace mgs
