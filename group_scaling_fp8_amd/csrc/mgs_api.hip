// mgs_api.hip — the C ABI of libmgs.so (declared in include/mgs.h): host-side
// argument checks, the dim0 workspace, and stream-ordered launches.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "mgs.h"
#include "mgs_kernels.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
    if (e == hipSuccess) return MGS_OK;
    g_last_hip_error = (int)e;
    return MGS_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Device workspace of dim0 for groups taller than 640 rows (layout in
// Dim0Workspace), one per (device, stream) so that concurrent streams never
// share it. It grows on demand and lives until process exit. gen is the last
// generation number handed to a kernel on that stream (1 .. 2^31 - 1).
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
    uint32_t gen = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace>* g_ws = nullptr;

// Returns the workspace of the current device and `stream` with at least
// `bytes` bytes and the generation number of this call (0 when the stream is
// capturing a graph: then the kernel reads it from the epoch word).
// A new or regrown buffer is zeroed in stream order, and so is the whole
// buffer whenever the host counter wraps.
hipError_t dim0_workspace_for(hipStream_t stream, const mgs::Dim0Workspace& layout, bool capturing,
                              void** out, uint32_t* gen) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (!g_ws) g_ws = new std::map<std::pair<int, hipStream_t>, Workspace>();
    Workspace& w = (*g_ws)[std::make_pair(dev, stream)];
    if (w.bytes < layout.bytes) {
        // no allocation while a graph is being captured
        if (capturing) return hipErrorStreamCaptureUnsupported;
        if (w.ptr) {
            // earlier work on this stream may still read the old buffer
            e = hipStreamSynchronize(stream);
            if (e != hipSuccess) return e;
            e = hipFree(w.ptr);
            if (e != hipSuccess) return e;
            w.ptr = nullptr;
            w.bytes = 0;
        }
        e = hipMalloc(&w.ptr, layout.bytes);
        if (e != hipSuccess) {
            w.ptr = nullptr;
            return e;
        }
        e = hipMemsetAsync(w.ptr, 0, layout.bytes, stream);
        if (e != hipSuccess) return e;
        w.bytes = layout.bytes;
        w.gen = 0;
    }
    *out = w.ptr;
    if (capturing) {
        *gen = 0;
        return hipSuccess;
    }
    if (w.gen >= 0x7FFFFFFFu) {
        // wrapped: clear the workspace so that no stale word can hold the
        // next generation
        e = hipMemsetAsync(w.ptr, 0, w.bytes, stream);
        if (e != hipSuccess) return e;
        w.gen = 0;
    }
    *gen = ++w.gen;
    return hipSuccess;
}

// MGS_FLAG_VALIDATE: the offsets, copied to the host in stream order, must be
// non-decreasing multiples of `align` in [0, extent] ending at extent.
int validate_offsets(const int32_t* offsets, int32_t n_groups, int64_t extent, int align,
                     hipStream_t stream) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cap);
    if (e != hipSuccess) return hip_status(e);
    if (cap != hipStreamCaptureStatusNone) return MGS_ERR_UNSUPPORTED;
    std::vector<int32_t> h((size_t)n_groups);
    e = hipMemcpyAsync(h.data(), offsets, (size_t)n_groups * sizeof(int32_t), hipMemcpyDeviceToHost,
                       stream);
    if (e != hipSuccess) return hip_status(e);
    e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_status(e);
    int64_t prev = 0;
    for (int32_t g = 0; g < n_groups; ++g) {
        const int64_t v = h[(size_t)g];
        if (v < prev || v > extent || v % align != 0) return MGS_ERR_INVALID_ARG;
        prev = v;
    }
    return prev == extent ? MGS_OK : MGS_ERR_INVALID_ARG;
}

// A stand-in for the offsets pointer of calls that have none (equal groups):
// well aligned, never dereferenced.
const int32_t* const kNoOffsets = reinterpret_cast<const int32_t*>(uintptr_t(256));

int check_grouped(const void* x, int64_t M, int64_t K, const int32_t* offsets, int32_t n_groups,
                  uint32_t flags, const void* q, const float* scales) {
    if (M < 0 || K < 0) return MGS_ERR_INVALID_ARG;
    if (n_groups < 1) return MGS_ERR_INVALID_ARG;
    if (n_groups > MGS_MAX_GROUPS) return MGS_ERR_UNSUPPORTED;
    if (flags & ~(MGS_FLAG_POW2_SCALE | MGS_FLAG_VALIDATE)) return MGS_ERR_INVALID_ARG;
    if (!offsets || !aligned(offsets, 4)) return MGS_ERR_INVALID_ARG;
    if (M > INT32_MAX || K > INT32_MAX) return MGS_ERR_UNSUPPORTED;  // offsets are int32
    if (M * K > 0) {
        if (!x || !q || !aligned(x, 16) || !aligned(q, 8)) return MGS_ERR_INVALID_ARG;
    }
    (void)scales;
    return MGS_OK;
}

}  // namespace

namespace mgs {

struct DeviceInfo {
    long long spin_ticks;   // 20 ms of the device wall clock
    int team_max;           // min(kDim0MaxTeam, CU count)
    int cus;                // compute units
};

DeviceInfo device_info() {
    static std::mutex mu;
    static std::map<int, DeviceInfo> per_device;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DeviceInfo{2000000, 1, 1};
    std::lock_guard<std::mutex> lock(mu);
    auto it = per_device.find(dev);
    if (it != per_device.end()) return it->second;
    int khz = 0, cus = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        khz = 100000;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 1;
    DeviceInfo d{20LL * khz, cus < kDim0MaxTeam ? cus : kDim0MaxTeam, cus};
    per_device[dev] = d;
    return d;
}

// Bound on a dim0 tile's wait for maxima written by other tiles: 20 ms of
// device wall clock. MGS_DIM0_SPIN_TICKS overrides it (a negative value
// skips the wait, which exercises the path where a tile computes the maxima
// itself).
long long dim0_spin_ticks(const DeviceInfo& d) {
    if (const char* v = getenv("MGS_DIM0_SPIN_TICKS")) return atoll(v);
    return d.spin_ticks;
}

// Most chunks of a group cast as a team: min(128, CU count).
// MGS_DIM0_TEAM_MAX lowers it (at least 1), which sends tall groups through
// the column-maximum tiles instead.
int dim0_team_max(const DeviceInfo& d) {
    if (const char* v = getenv("MGS_DIM0_TEAM_MAX")) {
        const int t = atoi(v);
        if (t >= 1 && t < d.team_max) return t;
    }
    return d.team_max;
}

// Both dim0 entry points: q (M, K) and scales (G, K), or their transposes.
// uniform_rows >= 0: n_groups equal groups of uniform_rows rows and no offsets.
int quant_groups_dim0(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                      int32_t n_groups, uint32_t flags, void* q, float* scales, void* stream,
                      bool transposed, int64_t uniform_rows = -1) {
    const bool uniform = uniform_rows >= 0;
    int st = check_grouped(x, M, K, uniform ? kNoOffsets : offsets, n_groups, flags, q, scales);
    if (st != MGS_OK) return st;
    if (K % 8 != 0) return MGS_ERR_INVALID_ARG;
    if (transposed && (M % 16 != 0 || (M * K > 0 && !aligned(q, 16)))) return MGS_ERR_INVALID_ARG;
    if (K == 0) return MGS_OK;
    if (!scales || !aligned(scales, transposed ? 4 : 16)) return MGS_ERR_INVALID_ARG;
    if ((flags & MGS_FLAG_VALIDATE) && !uniform) {
        st = validate_offsets(offsets, n_groups, M, transposed ? 16 : 1,
                              reinterpret_cast<hipStream_t>(stream));
        if (st != MGS_OK) return st;
    }
    const mgs::DeviceInfo dinfo = mgs::device_info();
    const int team_max = mgs::dim0_team_max(dinfo);
    const int64_t chunk_rows = transposed ? mgs::kDim0ChunkRowsT : mgs::kDim0ChunkRows;
    const int lt_cap = mgs::dim0_lt_cap(M, K, n_groups, team_max, dinfo.cus, chunk_rows);
    if (mgs::dim0_tile_bound(M, K, n_groups, team_max, lt_cap, chunk_rows) >= INT32_MAX)
        return MGS_ERR_UNSUPPORTED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const mgs::Dim0Workspace layout = mgs::dim0_workspace(M, K);
    void* ws = nullptr;
    uint32_t gen = 0;
    if (layout.chunks > 0) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(s, &cap);
        if (e != hipSuccess) return hip_status(e);
        const bool capturing = cap != hipStreamCaptureStatusNone;
        e = dim0_workspace_for(s, layout, capturing, &ws, &gen);
        if (e == hipErrorStreamCaptureUnsupported) return MGS_ERR_UNSUPPORTED;
        if (e != hipSuccess) return hip_status(e);
        if (capturing) {
            e = mgs::launch_dim0_epoch_bump(ws, s);
            if (e != hipSuccess) return hip_status(e);
        }
    }
    return hip_status(mgs::launch_dim0(static_cast<const uint16_t*>(x), (int)M, (int)K, offsets,
                                       n_groups, (int)uniform_rows,
                                       (flags & MGS_FLAG_POW2_SCALE) != 0, transposed,
                                       static_cast<uint8_t*>(q), scales, team_max, lt_cap, ws, gen,
                                       mgs::dim0_spin_ticks(dinfo), s));
}

}  // namespace mgs

extern "C" {

int mgs_quant_groups_dim0(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                          int32_t n_groups, uint32_t flags, void* q, float* scales,
                          void* stream) {
    return mgs::quant_groups_dim0(x, M, K, offsets, n_groups, flags, q, scales, stream, false);
}

int mgs_quant_groups_dim0_t(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                            int32_t n_groups, uint32_t flags, void* q_t, float* scales_t,
                            void* stream) {
    return mgs::quant_groups_dim0(x, M, K, offsets, n_groups, flags, q_t, scales_t, stream, true);
}

int mgs_quant_experts_dim1(const void* w, int64_t E, int64_t D1, int64_t D2, uint32_t flags,
                           void* q, float* scales, void* stream) {
    if (E < 1 || D1 < 0) return MGS_ERR_INVALID_ARG;
    if (E > MGS_MAX_GROUPS || D1 > INT32_MAX / E) return MGS_ERR_UNSUPPORTED;
    return mgs::quant_groups_dim0(w, E * D1, D2, nullptr, (int32_t)E, flags, q, scales, stream, false,
                                  D1);
}

int mgs_quant_groups_dim1(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                          int32_t n_groups, uint32_t flags, void* q, float* scales,
                          void* stream) {
    int st = check_grouped(x, M, K, offsets, n_groups, flags, q, scales);
    if (st != MGS_OK) return st;
    if (K % 16 != 0) return MGS_ERR_INVALID_ARG;
    if (K > MGS_DIM1_MAX_K) return MGS_ERR_UNSUPPORTED;
    if (M == 0 || K == 0) return MGS_OK;
    if (!scales || !aligned(scales, 4)) return MGS_ERR_INVALID_ARG;
    if (flags & MGS_FLAG_VALIDATE) {
        st = validate_offsets(offsets, n_groups, K, 16, reinterpret_cast<hipStream_t>(stream));
        if (st != MGS_OK) return st;
    }
    return hip_status(mgs::launch_dim1(static_cast<const uint16_t*>(x), M, (int)K, offsets,
                                       n_groups, (flags & MGS_FLAG_POW2_SCALE) != 0,
                                       static_cast<uint8_t*>(q), scales, mgs::device_info().cus,
                                       reinterpret_cast<hipStream_t>(stream)));
}

int mgs_mx_quant_dim0(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                      int32_t n_groups, int mode, void* q, uint8_t* scales_e8m0, void* stream) {
    (void)offsets;
    (void)n_groups;
    if (M < 0 || K < 0 || K % 32 != 0) return MGS_ERR_INVALID_ARG;
    if (mode != MGS_MX_FLOOR && mode != MGS_MX_RCEIL) return MGS_ERR_INVALID_ARG;
    if (M == 0 || K == 0) return MGS_OK;
    if (M > INT64_MAX / K) return MGS_ERR_UNSUPPORTED;
    if (!x || !q || !scales_e8m0 || !aligned(x, 16) || !aligned(q, 8)) return MGS_ERR_INVALID_ARG;
    return hip_status(mgs::launch_mx(static_cast<const uint16_t*>(x), M * K, mode == MGS_MX_RCEIL,
                                     static_cast<uint8_t*>(q), scales_e8m0,
                                     reinterpret_cast<hipStream_t>(stream)));
}

int mgs_mx_quant_dim1(const void* x, int64_t M, int64_t K, int mode, void* q_t, uint8_t* scales_t,
                      void* stream) {
    if (M < 0 || K < 0 || M % 32 != 0 || K % 8 != 0) return MGS_ERR_INVALID_ARG;
    if (mode != MGS_MX_FLOOR && mode != MGS_MX_RCEIL) return MGS_ERR_INVALID_ARG;
    if (M == 0 || K == 0) return MGS_OK;
    if (M > INT64_MAX / K) return MGS_ERR_UNSUPPORTED;
    if (!x || !q_t || !scales_t || !aligned(x, 16) || !aligned(q_t, 8)) return MGS_ERR_INVALID_ARG;
    return hip_status(mgs::launch_mx_dim1(static_cast<const uint16_t*>(x), M, K, mode == MGS_MX_RCEIL,
                                          static_cast<uint8_t*>(q_t), scales_t,
                                          reinterpret_cast<hipStream_t>(stream)));
}

int mgs_mx_dequant_dim0(const void* q, const uint8_t* scales_e8m0, int64_t M, int64_t K, void* y,
                        void* stream) {
    if (M < 0 || K < 0 || K % 32 != 0) return MGS_ERR_INVALID_ARG;
    if (M == 0 || K == 0) return MGS_OK;
    if (M > INT64_MAX / K) return MGS_ERR_UNSUPPORTED;
    if (!q || !scales_e8m0 || !y || !aligned(q, 16) || !aligned(y, 16)) return MGS_ERR_INVALID_ARG;
    return hip_status(mgs::launch_mx_dequant(static_cast<const uint8_t*>(q), scales_e8m0, M * K,
                                             static_cast<uint16_t*>(y),
                                             reinterpret_cast<hipStream_t>(stream)));
}

int mgs_cast_e4m3(const float* in, int64_t n, uint8_t* out, void* stream) {
    if (n < 0 || n % 4 != 0) return MGS_ERR_INVALID_ARG;
    if (n == 0) return MGS_OK;
    if (!in || !out || !aligned(in, 16) || !aligned(out, 4)) return MGS_ERR_INVALID_ARG;
    return hip_status(mgs::launch_cast(in, n, out, reinterpret_cast<hipStream_t>(stream)));
}

int mgs_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    if (bytes < 0 || bytes % 16 != 0) return MGS_ERR_INVALID_ARG;
    if (bytes == 0) return MGS_OK;
    if (!src || !dst || !aligned(src, 16) || !aligned(dst, 16)) return MGS_ERR_INVALID_ARG;
    return hip_status(mgs::launch_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream)));
}

const char* mgs_status_string(int status) {
    switch (status) {
        case MGS_OK: return "ok";
        case MGS_ERR_INVALID_ARG: return "invalid argument";
        case MGS_ERR_UNSUPPORTED: return "unsupported";
        case MGS_ERR_HIP: return "HIP error";
        default: return "unknown status";
    }
}

int mgs_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
