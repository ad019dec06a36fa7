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

// ---- MX dequantisation ------------------------------------------------------
// y = bf16(E4M3(q) * 2^(byte - 127)) per block of 32: the receiving side of
// the quantise -> all-to-all -> dequantise pipeline. A lane takes 16 codes
// (one 16-byte load, half a block, so lanes 2i and 2i + 1 share a scale
// byte) and writes 16 bf16 values with two ordinary 16-byte stores (at the
// MX shape: 6.3 TB/s, against 4.7 TB/s with nontemporal stores; one vector
// per lane beats two or four). The fp8 -> fp32 conversion is exact and so is
// the product with a power of two (4 significant bits, binary32 subnormals
// kept), so the only rounding is nearest-even to bf16.
typedef float f32x2 __attribute__((ext_vector_type(2)));
constexpr int kDqVecs = 1;   // 16-byte code vectors per lane per workgroup

// 2^(byte - 127) in binary32: normal for byte >= 1, the subnormal 2^-127 for
// byte 0; byte 0xFF is NaN (OCP MX E8M0).
__device__ __forceinline__ float e8m0_value(uint32_t byte) {
    if (byte == 0xFFu) return __uint_as_float(0x7FC00000u);
    return __uint_as_float(byte ? byte << 23 : 0x00400000u);
}

// bf16 bits of f rounded to nearest even (overflow to infinity); NaN -> 0x7FC0.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t b = __float_as_uint(f);
    if ((b & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// Codes in bytes 0-1 (kHi = false) or 2-3 (kHi = true) of w, scaled, as two
// packed bf16 values (the lower byte in the low half).
template <bool kHi>
__device__ __forceinline__ uint32_t dequant2(uint32_t w, float s) {
    const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
    return bf16_rne(f.x * s) | (bf16_rne(f.y * s) << 16);
}

__global__ __launch_bounds__(kThreads) void mx_dequant_kernel(const uint4* __restrict__ q,
                                                              const uint8_t* __restrict__ scales,
                                                              int64_t n16, uint4* __restrict__ y) {
    const int64_t base = (int64_t)blockIdx.x * (kThreads * kDqVecs) + threadIdx.x;
    uint4 v[kDqVecs];
    uint32_t sb[kDqVecs];
#pragma unroll
    for (int j = 0; j < kDqVecs; ++j) {
        const int64_t vi = base + (int64_t)j * kThreads;
        v[j] = make_uint4(0u, 0u, 0u, 0u);
        sb[j] = 0u;
        if (vi < n16) {
            v[j] = load_stream(q + vi);
            sb[j] = scales[vi >> 1];
        }
    }
#pragma unroll
    for (int j = 0; j < kDqVecs; ++j) {
        const int64_t vi = base + (int64_t)j * kThreads;
        if (vi < n16) {
            const float s = e8m0_value(sb[j]);
            const uint4 a = make_uint4(dequant2<false>(v[j].x, s), dequant2<true>(v[j].x, s),
                                       dequant2<false>(v[j].y, s), dequant2<true>(v[j].y, s));
            const uint4 b = make_uint4(dequant2<false>(v[j].z, s), dequant2<true>(v[j].z, s),
                                       dequant2<false>(v[j].w, s), dequant2<true>(v[j].w, s));
            y[2 * vi] = a;
            y[2 * vi + 1] = b;
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

hipError_t launch_mx_dequant(const uint8_t* q, const uint8_t* scales, int64_t n_elems, uint16_t* y,
                             hipStream_t stream) {
    const int64_t n16 = n_elems / 16;
    const int64_t per_block = (int64_t)kThreads * kDqVecs;
    const int64_t blocks = (n16 + per_block - 1) / per_block;
    hipLaunchKernelGGL(mx_dequant_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint4*>(q), scales, n16, reinterpret_cast<uint4*>(y));
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
