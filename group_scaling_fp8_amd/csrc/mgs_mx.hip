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
constexpr int kMxVecs = 2;   // 16-byte vectors per lane per workgroup (2: 314 us at (131072, 5120), 4: 324, 1: 341, 8: 325)

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

// ---- MX cast along dim0 (blocks of 32 rows), transposed output ------------------
// The MX cast of x^T computed from x: q_t (K, M) E4M3 with blocks of 32 along
// its rows and scales_t (K, M/32), the GEMM-ready form. A 1024-thread
// workgroup takes 512 rows x 128 columns; a lane holds 8 consecutive rows of
// 8 columns, so each wave covers exactly one block of 32 rows and a column's
// block amax is two lane swaps (the four lanes of the wave that share its
// columns). A lane casts its 8 x 8 block and transposes it in registers; the
// tile goes through 64 KiB of LDS so that q_t is written in whole 512-byte
// runs of its rows (32 lanes each), and the scales as a column's 16 blocks
// in one 16-byte store. Taller tiles write longer runs of each q_t row:
// 128 / 256 / 512 rows measured 378 / 371 / 364 us at (131072, 5120).
// Tile order: each XCD (the dispatcher deals workgroups to the 8 XCDs in
// turn) takes a contiguous run of tiles, M fastest. A tile writes 16 bytes
// of each of its 128 scale rows; the 8 tiles that fill one 128-byte line of
// a scale row then run on one XCD close together, so its L2 merges them and
// writes whole lines (dealt in turn, every line was written in pieces from
// several L2s).
constexpr int kMxRows = 512;                       // tile rows (M), a multiple of 32
constexpr int kMxCols = 128;                       // tile columns (K)
constexpr int kMxThreads = 2 * kMxRows;            // 16 lanes per 8 rows
constexpr int kMxBlocks = kMxRows / 32;            // blocks of 32 rows per tile column
constexpr int kXcds = 8;
// the LDS word swizzle flips bits 2-4 of a word index inside a column of
// kMxRows / 4 words, and four store passes cover 128 columns of kMxRows / 16 pieces
static_assert(kMxRows % 128 == 0 && kMxThreads <= 1024, "mx_dim1 tile shape");

__global__ __launch_bounds__(kMxThreads) void mx_dim1_kernel(const uint16_t* __restrict__ x, int64_t M,
                                                           int64_t K, int rceil,
                                                           uint8_t* __restrict__ q_t,
                                                           uint8_t* __restrict__ scales_t) {
    const int64_t nm = (M + kMxRows - 1) / kMxRows;
    // workgroup b runs on XCD b % 8: the XCD's run of tiles starts at
    // x * (T / 8) + min(x, T % 8)
    const int64_t n_tiles = (int64_t)gridDim.x;
    const int64_t xcd = blockIdx.x % kXcds, k_in = blockIdx.x / kXcds;
    const int64_t tile = xcd * (n_tiles / kXcds) + min(xcd, n_tiles % kXcds) + k_in;
    const int64_t tile_m = tile % nm, tile_k = tile / nm;
    const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;        // 16 column groups, 64 row groups
    const int64_t row0 = tile_m * kMxRows + 8 * ty;                // this lane's 8 rows
    const int64_t col = tile_k * kMxCols + 8 * tx;                  // and 8 columns
    // M % 32 == 0 and K % 8 == 0: a wave's block and a lane's columns are whole
    const bool ok = row0 < M && col < K;
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        v[i] = make_uint4(0u, 0u, 0u, 0u);
        if (ok) v[i] = load_stream(x + (row0 + i) * K + col);
    }
    // column magnitudes over this lane's rows, then over the wave's four row groups
    uint4 m = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        m.x = mag_max2(m.x, v[i].x);
        m.y = mag_max2(m.y, v[i].y);
        m.z = mag_max2(m.z, v[i].z);
        m.w = mag_max2(m.w, v[i].w);
    }
#pragma unroll
    for (int d = 16; d < kWave; d <<= 1) {
        m.x = mag_max2(m.x, (uint32_t)__shfl_xor((int)m.x, d, kWave));
        m.y = mag_max2(m.y, (uint32_t)__shfl_xor((int)m.y, d, kWave));
        m.z = mag_max2(m.z, (uint32_t)__shfl_xor((int)m.z, d, kWave));
        m.w = mag_max2(m.w, (uint32_t)__shfl_xor((int)m.w, d, kWave));
    }
    const uint32_t a[8] = {m.x & 0xFFFFu, m.x >> 16, m.y & 0xFFFFu, m.y >> 16,
                           m.z & 0xFFFFu, m.z >> 16, m.w & 0xFFFFu, m.w >> 16};
    uint32_t byte[8];
    float mult[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int b = (int)(a[j] >> 7) - 8 + ((rceil != 0 && (a[j] & 0x7Fu) > 96u) ? 1 : 0);
        byte[j] = (uint32_t)max(b, 0);
        mult[j] = __uint_as_float((254u - byte[j]) << 23);
    }
    // stage the cast tile in LDS as column words (four rows each), the word
    // index XOR-swizzled with the lane's column block, and the scale bytes as
    // [column][block]; then store each column's run of its q_t row
    __shared__ uint32_t st[kMxCols * kMxRows / 4];
    __shared__ __attribute__((aligned(16))) uint8_t sst[kMxCols * kMxBlocks];
    const int w = threadIdx.x >> 6;                                 // this wave's block of the tile
    if (ok) {
        uint2 r[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            r[i] = cast8(v[i], mult[0], mult[1], mult[2], mult[3], mult[4], mult[5], mult[6], mult[7]);
        uint32_t lo03[4], lo47[4], hi03[4], hi47[4];     // columns 0-3 / 4-7, rows 0-3 / 4-7
        transpose4x4(r[0].x, r[1].x, r[2].x, r[3].x, lo03);
        transpose4x4(r[4].x, r[5].x, r[6].x, r[7].x, lo47);
        transpose4x4(r[0].y, r[1].y, r[2].y, r[3].y, hi03);
        transpose4x4(r[4].y, r[5].y, r[6].y, r[7].y, hi47);
        const int word = (2 * ty) ^ ((tx & 7) << 2);                // rows 8ty .. 8ty + 7
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<uint2*>(st + (8 * tx + j) * (kMxRows / 4) + word) = make_uint2(lo03[j], lo47[j]);
            *reinterpret_cast<uint2*>(st + (8 * tx + 4 + j) * (kMxRows / 4) + word) = make_uint2(hi03[j], hi47[j]);
        }
        if ((ty & 3) == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) sst[(8 * tx + j) * kMxBlocks + w] = (uint8_t)byte[j];
        }
    }
    __syncthreads();
    const int64_t r0 = tile_m * kMxRows, c0 = tile_k * kMxCols;
    const int rows = (int)min((int64_t)kMxRows, M - r0);            // a multiple of 32
    const int cols = (int)min((int64_t)kMxCols, K - c0);            // a multiple of 8
    const int pieces = rows >> 4;                                    // 16-byte pieces per column
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int idx = threadIdx.x + k * kMxThreads;                // 32 pieces per column, pieces fastest
        const int c = idx / (kMxRows / 16), p = idx % (kMxRows / 16);
        if (c < cols && p < pieces) {
            const uint4 val =
                *reinterpret_cast<const uint4*>(st + c * (kMxRows / 4) + ((4 * p) ^ (((c >> 3) & 7) << 2)));
            store_stream16(q_t + (c0 + c) * M + r0 + 16 * p, val);
        }
    }
    if (threadIdx.x < cols) {
        const int c = threadIdx.x;
        const int64_t nb = M / 32;
        uint8_t* dst = scales_t + (c0 + c) * nb + r0 / 32;
        if (rows == kMxRows && (reinterpret_cast<uintptr_t>(dst) & 15) == 0) {
            // the column's 16 blocks in one 16-byte store
            *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(sst + c * kMxBlocks);
        } else {
            for (int b = 0; b < (rows >> 5); ++b) dst[b] = sst[c * kMxBlocks + b];
        }
    }
}

// ---- MX dequantisation ------------------------------------------------------
// y = bf16(E4M3(q) * 2^(byte - 127)) per block of 32: the receiving side of
// the quantise -> all-to-all -> dequantise pipeline. A wave takes 1024
// consecutive codes: lane l the 8 codes at 8l and the 8 at 512 + 8l (two
// 8-byte loads, each wave instruction 512 contiguous bytes), and writes 16
// bf16 values with two 16-byte nontemporal stores, each wave instruction
// 1 KiB of whole lines of y. The fp8 -> fp32 conversion is exact and so is
// the product with a power of two (4 significant bits, binary32 subnormals
// kept), so the only rounding is nearest-even to bf16.
typedef float f32x2 __attribute__((ext_vector_type(2)));

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

constexpr int kDqUnits = 2;   // units of 8 codes per lane (at (131072, 5120): 2: 318 us, 1: 332, 4: 329, 8: 339)

__global__ __launch_bounds__(kThreads) void mx_dequant_kernel(const uint2* __restrict__ q,
                                                              const uint8_t* __restrict__ scales,
                                                              int64_t n8, uint4* __restrict__ y) {
    // units of 8 codes: this wave's kDqUnits * 64 units start at wave_base
    const int64_t wave_base = ((int64_t)blockIdx.x * kThreads + (threadIdx.x & ~(kWave - 1))) * kDqUnits;
    const int lane = threadIdx.x & (kWave - 1);
    int64_t u[kDqUnits];
#pragma unroll
    for (int h = 0; h < kDqUnits; ++h) u[h] = wave_base + h * kWave + lane;
    uint2 c[kDqUnits];
    uint32_t sb[kDqUnits];
#pragma unroll
    for (int h = 0; h < kDqUnits; ++h) {
        c[h] = make_uint2(0u, 0u);
        sb[h] = 0u;
        if (u[h] < n8) {
            const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q + u[h]));
            c[h] = make_uint2(t.x, t.y);
            sb[h] = scales[u[h] >> 2];           // four units of 8 codes per block of 32
        }
    }
#pragma unroll
    for (int h = 0; h < kDqUnits; ++h) {
        if (u[h] < n8) {
            const float s = e8m0_value(sb[h]);
            store_stream16(y + u[h], make_uint4(dequant2<false>(c[h].x, s), dequant2<true>(c[h].x, s),
                                                dequant2<false>(c[h].y, s), dequant2<true>(c[h].y, s)));
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

hipError_t launch_mx_dim1(const uint16_t* x, int64_t M, int64_t K, bool rceil, uint8_t* q_t,
                          uint8_t* scales_t, hipStream_t stream) {
    const int64_t tiles = ((M + kMxRows - 1) / kMxRows) * ((K + kMxCols - 1) / kMxCols);
    if (tiles > INT32_MAX) return hipErrorInvalidValue;
    hipLaunchKernelGGL(mx_dim1_kernel, dim3((unsigned)tiles), dim3(kMxThreads), 0, stream, x, M, K,
                       rceil ? 1 : 0, q_t, scales_t);
    return hipGetLastError();
}

hipError_t launch_mx_dequant(const uint8_t* q, const uint8_t* scales, int64_t n_elems, uint16_t* y,
                             hipStream_t stream) {
    const int64_t n8 = n_elems / 8;
    const int64_t per_block = (int64_t)kThreads * kDqUnits;
    const int64_t blocks = (n8 + per_block - 1) / per_block;
    hipLaunchKernelGGL(mx_dequant_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       reinterpret_cast<const uint2*>(q), scales, n8, reinterpret_cast<uint4*>(y));
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
