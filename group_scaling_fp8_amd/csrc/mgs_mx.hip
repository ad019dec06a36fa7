// mgs_mx.hip — MX-style block-32 cast along the last dim, E8M0 scales, on
// gfx950; plus the standalone E4M3 cast and a calibration copy kernel.
//
// Method: "[mxfp8 moe training] fix mxfp8 a2a bench script; set mxfp8 a2a
// scaling type to RCEIL" — investigation comment (the mxfp8 dim0 cast as one
// fused kernel) and Summary (RCEIL scaling type, fp32 -> e8m0 cast). E8M0 as
// in the OCP MX spec (byte = exponent + 127).
//
// Blocks of 32 run along the last dim and K % 32 == 0, so block b of the
// flattened tensor is elements [32b, 32b + 32) and its scale is byte b of the
// flattened (M, K/32) scale array: the kernel is a flat stream that never
// needs the row index. Four consecutive lanes own one block (8 elements, one
// 16-byte load each), so every load instruction reads 1 KiB contiguously;
// the block amax is two lane swaps. The exponent comes from the bits of the
// 15-bit bf16 magnitude of the amax (no log2):
//   biased exponent Eb = amax15 >> 7, mantissa m = amax15 & 0x7F;
//   FLOOR: byte = Eb - 8;  RCEIL: byte = Eb - 8 + (m > 96)  (1 + m/128 > 1.75)
//   byte = max(byte, 0)   (e >= -127; zero and subnormal amax land here)
// and the multiplier 2^-e = 2^(127 - byte) is built as binary32 bits
// (254 - byte) << 23, always a normal number for finite bf16 input, so
// x * 2^-e is exact unless it is too small to matter for E4M3.
#include "mgs_device.hpp"
#include "mgs_kernels.hpp"

namespace mgs {

namespace {

constexpr int kThreads = 256;
constexpr int kMxVecs = 4;   // 16-byte vectors per lane per workgroup

__global__ __launch_bounds__(kThreads) void mx_kernel(const uint16_t* __restrict__ x, int64_t n_vec,
                                                      int rceil, uint8_t* __restrict__ q,
                                                      uint8_t* __restrict__ scales) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kMxVecs) + threadIdx.x;
    const int lane = threadIdx.x & (kWave - 1);
    uint4 v[kMxVecs];
#pragma unroll
    for (int j = 0; j < kMxVecs; ++j) {
        const int64_t vi = base + (int64_t)j * kThreads;
        v[j] = make_uint4(0u, 0u, 0u, 0u);
        if (vi < n_vec) v[j] = load_stream(reinterpret_cast<const uint4*>(x) + vi);
    }
#pragma unroll
    for (int j = 0; j < kMxVecs; ++j) {
        const int64_t vi = base + (int64_t)j * kThreads;
        uint32_t m = mag_fold(mag_max8(0u, v[j]));
        m = max(m, (uint32_t)__shfl_xor((int)m, 1, kWave));
        m = max(m, (uint32_t)__shfl_xor((int)m, 2, kWave));
        int byte = (int)(m >> 7) - 8 + ((rceil != 0 && (m & 0x7Fu) > 96u) ? 1 : 0);
        byte = max(byte, 0);
        const float mult = __uint_as_float((uint32_t)(254 - byte) << 23);
        if (vi < n_vec) {
            store_stream(reinterpret_cast<uint2*>(q) + vi, cast8(v[j], mult));
            if ((lane & 3) == 0) scales[vi >> 2] = (uint8_t)byte;
        }
    }
}

__global__ __launch_bounds__(kThreads) void cast_kernel(const float4* __restrict__ in, int64_t n4,
                                                        uint32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n4) {
        const float4 f = in[i];
        out[i] = e4m3x4(f.x, f.y, f.z, f.w);
    }
}

constexpr int kCopyVecs = 4;

__global__ __launch_bounds__(kThreads) void copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n16) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kCopyVecs) + threadIdx.x;
    uint4 v[kCopyVecs];
#pragma unroll
    for (int j = 0; j < kCopyVecs; ++j) {
        const int64_t i = base + (int64_t)j * kThreads;
        v[j] = make_uint4(0u, 0u, 0u, 0u);
        if (i < n16) v[j] = src[i];
    }
#pragma unroll
    for (int j = 0; j < kCopyVecs; ++j) {
        const int64_t i = base + (int64_t)j * kThreads;
        if (i < n16) dst[i] = v[j];
    }
}

}  // namespace

hipError_t launch_mx(const uint16_t* x, int64_t n_elems, bool rceil, uint8_t* q, uint8_t* scales,
                     hipStream_t stream) {
    const int64_t n_vec = n_elems / 8;
    const int64_t per_block = (int64_t)kThreads * kMxVecs;
    const int64_t blocks = (n_vec + per_block - 1) / per_block;
    hipLaunchKernelGGL(mx_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, x, n_vec,
                       rceil ? 1 : 0, q, scales);
    return hipGetLastError();
}

hipError_t launch_cast(const float* in, int64_t n, uint8_t* out, hipStream_t stream) {
    const int64_t n4 = n / 4;
    const int64_t blocks = (n4 + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const float4*>(in), n4, reinterpret_cast<uint32_t*>(out));
    return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
    const int64_t n16 = bytes / 16;
    const int64_t per_block = (int64_t)kThreads * kCopyVecs;
    const int64_t blocks = (n16 + per_block - 1) / per_block;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(src), reinterpret_cast<uint4*>(dst), n16);
    return hipGetLastError();
}

}  // namespace mgs
