// mgs_api.hip — the C ABI of libmgs.so (declared in include/mgs.h): host-side
// argument checks, the dim0 workspace, and stream-ordered launches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
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

// The library's own dim0 workspace, used only by calls that pass none: one
// per (device, stream), so that calls on different streams never share one.
// It only grows. A grown workspace replaces the old one for later calls, but
// the old buffer is kept until process exit (graphs captured earlier may
// still use it), so nothing is ever freed and nothing waits for the stream.
// A new buffer is zero-filled by a kernel queued on the stream before the
// call's own kernel.
struct Workspace {
    void* ptr = nullptr;
    size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, Workspace>* g_ws = nullptr;
std::vector<void*>* g_ws_retired = nullptr;

hipError_t own_workspace(hipStream_t stream, size_t need, bool capturing, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (!g_ws) {
        g_ws = new std::map<std::pair<int, hipStream_t>, Workspace>();
        g_ws_retired = new std::vector<void*>();
    }
    Workspace& w = (*g_ws)[std::make_pair(dev, stream)];
    if (w.bytes < need) {
        // no allocation while a graph is being captured
        if (capturing) return hipErrorStreamCaptureUnsupported;
        void* p = nullptr;
        e = hipMalloc(&p, need);
        if (e != hipSuccess) return e;
        e = mgs::launch_zero(p, need, stream);
        if (e != hipSuccess) {
            g_ws_retired->push_back(p);
            return e;
        }
        if (w.ptr) g_ws_retired->push_back(w.ptr);
        w.ptr = p;
        w.bytes = need;
    }
    *out = w.ptr;
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

// Per-device constants, read from the runtime once per device. Two threads
// may both fill an entry the first time; they write the same values.
constexpr int kMaxDevices = 64;
DeviceInfo g_dev_info[kMaxDevices];
std::atomic<int> g_dev_ready[kMaxDevices];

DeviceInfo device_info() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return DeviceInfo{2000000, 1, 1};
    if (g_dev_ready[dev].load(std::memory_order_acquire)) return g_dev_info[dev];
    int khz = 0, cus = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        khz = 100000;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 1;
    const DeviceInfo d{20LL * khz, cus < kDim0MaxTeam ? cus : kDim0MaxTeam, cus};
    g_dev_info[dev] = d;
    g_dev_ready[dev].store(1, std::memory_order_release);
    return d;
}

// Overrides of two dim0 launch parameters, for tests only (mgs_test_quant_dim0).
struct Dim0Knobs {
    long long spin_ticks;   // wait bound in wall-clock ticks; -1: no wait; below -1: the default
    int team_max;           // 1 .. the device's limit lowers it (taller groups go to class C); else the default
};

// The dim0 workspace of mgs_quant_groups_dim0_noalloc: a fixed array in the
// code object, one copy per device, alive until the process ends. In host
// code `scratch` only names the symbol: its device address comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to a kernel.
constexpr size_t kScratchBytes = size_t(MGS_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint64_t scratch[kScratchBytes / sizeof(uint64_t)];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];
bool g_scratch_cleared[kMaxDevices];

// This device's copy of scratch, cleared in stream order the first time an
// eager call needs it. A call being captured before that also queues the
// clear (into its graph, so every replay starts from a clear array) without
// counting it as done, since the graph may never run.
hipError_t device_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    if (!g_scratch_cleared[dev]) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        e = hipStreamIsCapturing(stream, &cap);
        if (e != hipSuccess) return e;
        e = launch_zero(g_scratch_ptr[dev], kScratchBytes, stream);
        if (e != hipSuccess) return e;
        if (cap == hipStreamCaptureStatusNone) g_scratch_cleared[dev] = true;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

// Every dim0-family entry point: q (M, K) and scales (G, K), or their
// transposes. uniform_rows >= 0: n_groups equal groups of uniform_rows rows
// and no offsets. ws == null && ws_bytes == 0: the library's own workspace
// (use_scratch: the static scratch instead, never an allocation).
int quant_groups_dim0(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                      int32_t n_groups, uint32_t flags, void* q, float* scales, void* ws,
                      int64_t ws_bytes, void* stream, bool transposed, int64_t uniform_rows,
                      const Dim0Knobs* knobs, bool use_scratch = false) {
    const bool uniform = uniform_rows >= 0;
    int st = check_grouped(x, M, K, uniform ? kNoOffsets : offsets, n_groups, flags, q, scales);
    if (st != MGS_OK) return st;
    if (K % 8 != 0) return MGS_ERR_INVALID_ARG;
    if (transposed && (M % 16 != 0 || (M * K > 0 && !aligned(q, 16)))) return MGS_ERR_INVALID_ARG;
    if (ws_bytes < 0 || (!ws && ws_bytes != 0) || (ws && !aligned(ws, 256))) return MGS_ERR_INVALID_ARG;
    if (K == 0) return MGS_OK;
    if (!scales || !aligned(scales, transposed ? 4 : 16)) return MGS_ERR_INVALID_ARG;
    const mgs::Dim0Workspace layout = mgs::dim0_workspace(M, K);
    if (ws && (size_t)ws_bytes < layout.bytes) return MGS_ERR_INVALID_ARG;
    if (use_scratch && layout.bytes > kScratchBytes) return MGS_ERR_UNSUPPORTED;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if ((flags & MGS_FLAG_VALIDATE) && !uniform) {
        st = validate_offsets(offsets, n_groups, M, transposed ? 16 : 1, s);
        if (st != MGS_OK) return st;
    }
    const mgs::DeviceInfo dinfo = mgs::device_info();
    int team_max = dinfo.team_max;
    long long spin_ticks = dinfo.spin_ticks;
    if (knobs) {
        if (knobs->team_max >= 1 && knobs->team_max < team_max) team_max = knobs->team_max;
        if (knobs->spin_ticks >= -1) spin_ticks = knobs->spin_ticks;
    }
    const int64_t chunk_rows = transposed ? mgs::kDim0ChunkRowsT : mgs::kDim0ChunkRows;
    const int64_t lt_rows = transposed ? mgs::kDim0LtRowsT : mgs::kDim0LtRows;
    const int max_lt = transposed ? mgs::kDim0MaxLtT : mgs::kDim0MaxLt;
    int lt_cap = mgs::dim0_lt_cap(M, K, n_groups, team_max, dinfo.cus, chunk_rows, lt_rows, max_lt);
    // the transposed kernel deals its tiles to XCDs by column range when the
    // strips allow it, so that the 128-byte lines of q_t that two groups share
    // are written from one L2 (with teams that fit one XCD)
    bool xcd_split = false;
    if (transposed) {
        const int team_xcd = team_max < dinfo.cus / 8 ? team_max : (dinfo.cus / 8 > 0 ? dinfo.cus / 8 : 1);
        const int lt_xcd = mgs::dim0_lt_cap(M, K, n_groups, team_xcd, dinfo.cus, chunk_rows, lt_rows,
                                            max_lt);
        if (mgs::dim0_xcd_split(K, lt_xcd, dinfo.cus)) {
            xcd_split = true;
            team_max = team_xcd;
            lt_cap = lt_xcd;
        }
    }
    if (mgs::dim0_tile_bound(M, K, n_groups, team_max, lt_cap, chunk_rows, lt_rows) >= INT32_MAX)
        return MGS_ERR_UNSUPPORTED;
    void* w = ws;
    if (layout.bytes == 0) {
        w = nullptr;            // no chunked group possible: the kernels never touch it
    } else if (use_scratch) {
        hipError_t e = device_scratch(s, &w);
        if (e != hipSuccess) return hip_status(e);
    } else if (!w) {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing(s, &cap);
        if (e != hipSuccess) return hip_status(e);
        e = own_workspace(s, layout.bytes, cap != hipStreamCaptureStatusNone, &w);
        if (e == hipErrorStreamCaptureUnsupported) return MGS_ERR_UNSUPPORTED;
        if (e != hipSuccess) return hip_status(e);
    }
    return hip_status(mgs::launch_dim0(static_cast<const uint16_t*>(x), (int)M, (int)K, offsets,
                                       n_groups, (int)uniform_rows,
                                       (flags & MGS_FLAG_POW2_SCALE) != 0, transposed,
                                       static_cast<uint8_t*>(q), scales, team_max, lt_cap, xcd_split, w,
                                       spin_ticks, dinfo.cus, s));
}

int quant_experts(const void* w, int64_t E, int64_t D1, int64_t D2, uint32_t flags, void* q,
                  float* scales, void* ws, int64_t ws_bytes, void* stream, const Dim0Knobs* knobs) {
    if (E < 1 || D1 < 0) return MGS_ERR_INVALID_ARG;
    if (E > MGS_MAX_GROUPS || D1 > INT32_MAX / E) return MGS_ERR_UNSUPPORTED;
    return quant_groups_dim0(w, E * D1, D2, nullptr, (int32_t)E, flags, q, scales, ws, ws_bytes, stream,
                             false, D1, knobs);
}

}  // namespace mgs

extern "C" {

int mgs_dim0_workspace_bytes(int64_t M, int64_t K, int64_t* bytes) {
    if (!bytes || M < 0 || K < 0) return MGS_ERR_INVALID_ARG;
    if (M > INT32_MAX || K > INT32_MAX) return MGS_ERR_UNSUPPORTED;
    *bytes = (int64_t)mgs::dim0_workspace(M, K).bytes;
    return MGS_OK;
}

int mgs_quant_groups_dim0(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                          int32_t n_groups, uint32_t flags, void* q, float* scales,
                          void* stream) {
    return mgs::quant_groups_dim0(x, M, K, offsets, n_groups, flags, q, scales, nullptr, 0, stream,
                                  false, -1, nullptr);
}

int mgs_quant_groups_dim0_ws(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                             int32_t n_groups, uint32_t flags, void* q, float* scales,
                             void* workspace, int64_t workspace_bytes, void* stream) {
    return mgs::quant_groups_dim0(x, M, K, offsets, n_groups, flags, q, scales, workspace,
                                  workspace_bytes, stream, false, -1, nullptr);
}

int mgs_quant_groups_dim0_t(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                            int32_t n_groups, uint32_t flags, void* q_t, float* scales_t,
                            void* workspace, int64_t workspace_bytes, void* stream) {
    return mgs::quant_groups_dim0(x, M, K, offsets, n_groups, flags, q_t, scales_t, workspace,
                                  workspace_bytes, stream, true, -1, nullptr);
}

int mgs_quant_experts_dim1(const void* w, int64_t E, int64_t D1, int64_t D2, uint32_t flags,
                           void* q, float* scales, void* workspace, int64_t workspace_bytes,
                           void* stream) {
    return mgs::quant_experts(w, E, D1, D2, flags, q, scales, workspace, workspace_bytes, stream,
                              nullptr);
}

int mgs_quant_groups_dim0_noalloc(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                                  int32_t n_groups, uint32_t flags, void* q, float* scales,
                                  void* stream) {
    return mgs::quant_groups_dim0(x, M, K, offsets, n_groups, flags, q, scales, nullptr, 0, stream,
                                  false, -1, nullptr, true);
}

int mgs_test_quant_dim0(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                        int32_t n_groups, int64_t uniform_rows, uint32_t flags, int transposed,
                        void* q, float* scales, void* workspace, int64_t workspace_bytes,
                        int64_t spin_ticks, int32_t team_max, void* stream) {
    const mgs::Dim0Knobs knobs{(long long)spin_ticks, (int)team_max};
    if (uniform_rows >= 0) {
        if (transposed) return MGS_ERR_INVALID_ARG;
        if (M < 0 || (uniform_rows > 0 && M % uniform_rows != 0) || (uniform_rows == 0 && M != 0))
            return MGS_ERR_INVALID_ARG;
        const int64_t E = n_groups;
        if (uniform_rows * E != M) return MGS_ERR_INVALID_ARG;
        return mgs::quant_experts(x, E, uniform_rows, K, flags, q, scales, workspace, workspace_bytes,
                                  stream, &knobs);
    }
    return mgs::quant_groups_dim0(x, M, K, offsets, n_groups, flags, q, scales, workspace,
                                  workspace_bytes, stream, transposed != 0, -1, &knobs);
}

int mgs_quant_groups_dim1(const void* x, int64_t M, int64_t K, const int32_t* offsets,
                          int32_t n_groups, uint32_t flags, void* q, float* scales,
                          void* stream) {
    int st = check_grouped(x, M, K, offsets, n_groups, flags, q, scales);
    if (st != MGS_OK) return st;
    if (K % 16 != 0) return MGS_ERR_INVALID_ARG;
    if (K > MGS_DIM1_MAX_K) return MGS_ERR_UNSUPPORTED;
    if (M == 0) return MGS_OK;
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
    if (!x || !q_t || !scales_t || !aligned(x, 16) || !aligned(q_t, 16)) return MGS_ERR_INVALID_ARG;
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
