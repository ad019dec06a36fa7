// mgs_dim1.hip — per-group rowwise scaling (groups along dim1) on gfx950.
//
// Method: "[moe fp8 training] test and bench new faster method for per group
// rowwise scaling", Summary: one scale per (row, token group) of a row-major
// tensor whose token groups run along the contiguous dim. The slow kernel on
// that page lost its time to uncoalesced accesses; here every access runs
// along the contiguous dim.
//   * One workgroup owns one row at a time. It is sized to the row: NT
//     threads (a multiple of 64, at most 1024) with V 16-byte vectors each,
//     NT * V * 8 >= K. Lane t holds vectors t + NT*j, so each load
//     instruction of a wave reads 1 KiB of the row contiguously. Few vectors
//     per thread and many waves per row keep more bytes in flight than a few
//     long-running waves would.
//   * Workgroups are persistent over rows (row = block, block + grid, ...)
//     and load the next row while the current one is reduced and cast.
//   * Group boundaries are multiples of 16 columns (token-group alignment 16,
//     test source in "[moe training] use smaller block sizes for per group
//     scaling kernels to improve perf"), so a vector never straddles two
//     groups. A vector -> (group, last-vector-of-group) table is built once
//     per workgroup in LDS.
//   * Per-(row, group) amax is a segmented reduction: the key
//     (group << 16) | max|x| of every vector goes through a 64-lane prefix max
//     (DPP), which never mixes groups because group ids grow along the row;
//     the last lane of each group segment in a wave then does one LDS atomic
//     max.
//   * Rows longer than NT * V * 8 (K > 32768 with NT = 1024, V = 4) are done
//     in column chunks; their cast re-reads the row (the only extra traffic).
#include "mgs_device.hpp"
#include "mgs_kernels.hpp"

#include <map>
#include <mutex>

namespace mgs {

namespace {

constexpr uint32_t kNoGroup = 0x7FFFu;     // vector past the last group end
constexpr uint32_t kTailBit = 0x8000u;     // last vector of its group

// Group of the vector starting at column col: the first g with end[g] > col,
// or G if there is none.
__device__ __forceinline__ int group_of(const int* s_end, int G, int col) {
    int lo = 0, hi = G;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (s_end[mid] > col) hi = mid; else lo = mid + 1;
    }
    return lo;
}

template <int V>
__global__ __launch_bounds__(1024) void dim1_kernel(
        const uint16_t* __restrict__ x, int64_t M, int K, const int32_t* __restrict__ off, int G,
        int pow2, uint8_t* __restrict__ q, float* __restrict__ scales) {
    extern __shared__ int smem[];
    const int NT = blockDim.x;
    const int nvec = K / 8;
    int* s_end = smem;                                               // G
    uint32_t* s_amax = reinterpret_cast<uint32_t*>(smem + G);        // G
    float* s_scale = reinterpret_cast<float*>(smem + 2 * G);         // G
    uint16_t* vtab = reinterpret_cast<uint16_t*>(smem + 3 * G);      // nvec
    const int lane = threadIdx.x & (kWave - 1);

    if (threadIdx.x < kWave) {
        // sanitised end offsets: running max of the raw values clamped to [0, K]
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
    for (int t = threadIdx.x; t < G; t += NT) s_amax[t] = 0u;
    __syncthreads();
    for (int vi = threadIdx.x; vi < nvec; vi += NT) {
        const int c = vi * 8;
        const int g = group_of(s_end, G, c);
        uint32_t e = kNoGroup;
        if (g < G) e = (uint32_t)g | ((c + 8 >= s_end[g]) ? kTailBit : 0u);
        vtab[vi] = (uint16_t)e;
    }
    __syncthreads();

    const int chunk_vecs = NT * V;
    const int n_cc = (nvec + chunk_vecs - 1) / chunk_vecs;
    const bool p2 = pow2 != 0;

    uint32_t e[V];
    auto map_slots = [&](int cc) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const int vi = cc * chunk_vecs + threadIdx.x + NT * j;
            e[j] = vi < nvec ? vtab[vi] : kNoGroup;
        }
    };
    auto load_slots = [&](int64_t row, int cc, uint4 (&v)[V]) {
        const uint16_t* xr = x + row * (int64_t)K;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            v[j] = make_uint4(0u, 0u, 0u, 0u);
            if ((e[j] & kNoGroup) != kNoGroup) {
                const int vi = cc * chunk_vecs + threadIdx.x + NT * j;
                v[j] = load_stream(xr + (int64_t)vi * 8);
            }
        }
    };
    auto amax_slots = [&](const uint4 (&v)[V]) {
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const uint32_t gid = e[j] & kNoGroup;
            uint32_t key = 0u;
            if (gid != kNoGroup) key = (gid << 16) | mag_fold(mag_max8(0u, v[j]));
            key = wave_prefix_max(key);
            if (gid != kNoGroup && ((e[j] & kTailBit) || lane == kWave - 1))
                atomicMax(&s_amax[gid], key & 0xFFFFu);
        }
    };
    auto cast_slots = [&](int64_t row, int cc, const uint4 (&v)[V]) {
        uint8_t* qr = q + row * (int64_t)K;
#pragma unroll
        for (int j = 0; j < V; ++j) {
            const uint32_t gid = e[j] & kNoGroup;
            if (gid != kNoGroup) {
                const int vi = cc * chunk_vecs + threadIdx.x + NT * j;
                // a plain store: measured faster here than a nontemporal one
                *reinterpret_cast<uint2*>(qr + (int64_t)vi * 8) = cast8_group(v[j], s_scale[gid]);
            }
        }
    };
    auto scales_of_row = [&](int64_t row) {
        for (int g = threadIdx.x; g < G; g += NT) {
            const float s = group_scale(s_amax[g], p2);
            s_scale[g] = s;
            scales[row * G + g] = s;
            s_amax[g] = 0u;
        }
    };

    if (n_cc == 1) {
        // Whole row in registers; the next row is loaded before this one is
        // reduced and cast.
        map_slots(0);
        uint4 v[V], vn[V];
        int64_t row = blockIdx.x;
        if (row < M) load_slots(row, 0, vn);
        for (; row < M; row += gridDim.x) {
#pragma unroll
            for (int j = 0; j < V; ++j) v[j] = vn[j];
            if (row + gridDim.x < M) load_slots(row + gridDim.x, 0, vn);
            amax_slots(v);
            __syncthreads();
            scales_of_row(row);
            __syncthreads();
            cast_slots(row, 0, v);
        }
    } else {
        // Long rows: amax over column chunks, then re-read each chunk to cast.
        uint4 v[V];
        for (int64_t row = blockIdx.x; row < M; row += gridDim.x) {
            for (int cc = 0; cc < n_cc; ++cc) {
                map_slots(cc);
                load_slots(row, cc, v);
                amax_slots(v);
            }
            __syncthreads();
            scales_of_row(row);
            __syncthreads();
            for (int cc = 0; cc < n_cc; ++cc) {
                map_slots(cc);
                load_slots(row, cc, v);
                cast_slots(row, cc, v);
            }
        }
    }
}

// Workgroups of dim1_kernel<V> resident per CU for a launch shape, from the
// runtime's occupancy query, kept per (device, threads, LDS bytes): the query
// costs more than the rest of a call's host work.
template <int V>
int resident_per_cu(int threads, size_t shmem) {
    struct Key {
        int dev, threads;
        size_t shmem;
        bool operator<(const Key& o) const {
            return dev != o.dev ? dev < o.dev : threads != o.threads ? threads < o.threads : shmem < o.shmem;
        }
    };
    static std::mutex mu;
    static std::map<Key, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const Key key{dev, threads, shmem};
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, dim1_kernel<V>, threads, shmem) !=
            hipSuccess || per_cu < 1)
        per_cu = 1;
    std::lock_guard<std::mutex> lock(mu);
    cache[key] = per_cu;
    return per_cu;
}

template <int V>
hipError_t launch_v(const uint16_t* x, int64_t M, int K, const int32_t* off, int G, bool pow2,
                    uint8_t* q, float* scales, int threads, int cus, hipStream_t stream) {
    const size_t shmem = (size_t)3 * G * sizeof(int) + (size_t)(K / 8) * sizeof(uint16_t) + 16;
    // One round of workgroups: as many as fit on the GPU at once, each
    // walking M / blocks rows with the next row in flight. A second round
    // (twice the resident count) measured 2 us slower at (8192, 16640):
    // the workgroups that start late finish late.
    const int per_cu = resident_per_cu<V>(threads, shmem);
    const int64_t resident = (int64_t)per_cu * (cus > 0 ? cus : 1);
    const int64_t blocks = M < resident ? M : resident;
    hipLaunchKernelGGL(dim1_kernel<V>, dim3((unsigned)blocks), dim3(threads), shmem, stream, x, M,
                       K, off, G, pow2 ? 1 : 0, q, scales);
    return hipGetLastError();
}

// Rows of no columns: every group of every row is empty, so each of the
// n = M * G scales is the amax = 0 value.
__global__ __launch_bounds__(256) void empty_rows_kernel(float* __restrict__ scales, int64_t n,
                                                          int pow2) {
    const float s = group_scale(0u, pow2 != 0);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) scales[i] = s;
}

}  // namespace

hipError_t launch_dim1(const uint16_t* x, int64_t M, int K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, int cus, hipStream_t stream) {
    if (K == 0) {
        const int64_t n = M * G;
        const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
        hipLaunchKernelGGL(empty_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, scales, n,
                           pow2 ? 1 : 0);
        return hipGetLastError();
    }
    const int nvec = K / 8;
    // Smallest V whose workgroup (a multiple of 64 threads) fits in 1024
    // threads; rows longer than 1024 * 4 vectors use V = 4 in column chunks.
    for (int v = 1; v <= 4; ++v) {
        const int threads = ((nvec + v - 1) / v + kWave - 1) / kWave * kWave;
        if (threads <= 1024 || v == 4) {
            const int t = threads > 1024 ? 1024 : threads;
            switch (v) {
                case 1: return launch_v<1>(x, M, K, off, G, pow2, q, scales, t, cus, stream);
                case 2: return launch_v<2>(x, M, K, off, G, pow2, q, scales, t, cus, stream);
                case 3: return launch_v<3>(x, M, K, off, G, pow2, q, scales, t, cus, stream);
                default: return launch_v<4>(x, M, K, off, G, pow2, q, scales, t, cus, stream);
            }
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace mgs
