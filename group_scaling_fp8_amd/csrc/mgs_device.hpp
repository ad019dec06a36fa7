// mgs_device.hpp — gfx950 device helpers shared by the quantisation kernels.
//
// Numerics follow the kernel-argument dict of the torch.compile failure
// report on "[moe training] use smaller block sizes for per group scaling
// kernels to improve perf" (fp8 range +-448, EPS 1e-12, optional power-of-two
// scales) and the OCP OFP8 E4M3 / OCP MX E8M0 formats.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgs {

constexpr int kWave = 64;
constexpr int kMaxGroups = 1024;

// ---- bf16 ------------------------------------------------------------------

// A 32-bit word holds two bf16: the low half is the element at the lower
// address. Widening is exact: bf16 is the top half of a binary32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Running max of |x| on packed bf16 pairs. For finite bf16 the magnitude
// order equals the unsigned order of (bits & 0x7FFF), so this is the exact
// fp32 max of |x| in 16-bit form (v_pk_max_u16).
__device__ __forceinline__ uint32_t mag_max2(uint32_t acc, uint32_t w) {
    u16x2 a = __builtin_bit_cast(u16x2, acc);
    u16x2 b = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint32_t mag_max8(uint32_t acc, uint4 v) {
    acc = mag_max2(acc, v.x);
    acc = mag_max2(acc, v.y);
    acc = mag_max2(acc, v.z);
    return mag_max2(acc, v.w);
}

// Max of the two 16-bit halves.
__device__ __forceinline__ uint32_t mag_fold(uint32_t w) {
    return max(w & 0xFFFFu, w >> 16);
}

// ---- streaming global accesses ----------------------------------------------

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Cache-policy argument of __builtin_amdgcn_global_load_lds for a
// nontemporal load (the nt bit, as load_stream's loads carry).
constexpr int kLoadNontemporal = 2;

// 16 bytes of input read once: a nontemporal load, so the streamed input does
// not push reusable lines out of L2 and the Infinity Cache.
__device__ __forceinline__ uint4 load_stream(const void* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// 16 bytes of output written once, with a nontemporal store.
__device__ __forceinline__ void store_stream16(void* p, uint4 v) {
    u32x4 t;
    t.x = v.x;
    t.y = v.y;
    t.z = v.z;
    t.w = v.w;
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}

// 8 bytes of output written once, with a nontemporal store.
__device__ __forceinline__ void store_stream(void* p, uint2 v) {
    u32x2 t;
    t.x = v.x;
    t.y = v.y;
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
}

// ---- byte transposes ----------------------------------------------------------

// Byte transpose of a 4 x 4 block: a, b, c, d hold bytes 0..3 of four
// consecutive rows; word j of out holds byte j of a, b, c, d (low to high).
__device__ __forceinline__ void transpose4x4(uint32_t a, uint32_t b, uint32_t c, uint32_t d,
                                             uint32_t (&out)[4]) {
    // v_perm_b32 picks bytes of {hi, lo}: selector bytes 0..3 address lo,
    // 4..7 address hi
    const uint32_t ab01 = __builtin_amdgcn_perm(b, a, 0x05010400u);   // a0 b0 a1 b1
    const uint32_t ab23 = __builtin_amdgcn_perm(b, a, 0x07030602u);   // a2 b2 a3 b3
    const uint32_t cd01 = __builtin_amdgcn_perm(d, c, 0x05010400u);
    const uint32_t cd23 = __builtin_amdgcn_perm(d, c, 0x07030602u);
    out[0] = __builtin_amdgcn_perm(cd01, ab01, 0x05040100u);           // a0 b0 c0 d0
    out[1] = __builtin_amdgcn_perm(cd01, ab01, 0x07060302u);           // a1 b1 c1 d1
    out[2] = __builtin_amdgcn_perm(cd23, ab23, 0x05040100u);
    out[3] = __builtin_amdgcn_perm(cd23, ab23, 0x07060302u);
}

// ---- per-group scale ---------------------------------------------------------

// amax15 is the bf16 magnitude pattern of the group's max |x|.
// scale = fl32(448 / max(amax, 1e-12)): one IEEE binary32 division (hipcc's
// default division is correctly rounded). Power-of-two mode rounds down by
// clearing the mantissa, exact because the scale is always a normal number
// (amax <= bf16 max gives scale >= ~1.3e-36).
__device__ __forceinline__ float group_scale(uint32_t amax15, bool pow2) {
    const float amax = __uint_as_float(amax15 << 16);
    const float s = 448.0f / fmaxf(amax, 1e-12f);
    uint32_t b = __float_as_uint(s);
    if (pow2) b &= 0xFF800000u;
    return __uint_as_float(b);
}

// ---- E4M3 cast -----------------------------------------------------------------

// Four binary32 values to four E4M3 bytes (little-endian order a, b, c, d):
// clamp to [-448, 448] (v_med3_f32 keeps the sign of zero), then the
// hardware OCP E4M3 conversion, which rounds to nearest even.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Eight bf16 times one scale each: q = E4M3(fl32(x * s)).
__device__ __forceinline__ uint2 cast8(uint4 v, float s0, float s1, float s2, float s3,
                                       float s4, float s5, float s6, float s7) {
    uint2 r;
    r.x = e4m3x4(bf16_lo(v.x) * s0, bf16_hi(v.x) * s1, bf16_lo(v.y) * s2, bf16_hi(v.y) * s3);
    r.y = e4m3x4(bf16_lo(v.z) * s4, bf16_hi(v.z) * s5, bf16_lo(v.w) * s6, bf16_hi(v.w) * s7);
    return r;
}

__device__ __forceinline__ uint2 cast8(uint4 v, float s) {
    return cast8(v, s, s, s, s, s, s, s, s);
}

// Four binary32 values of magnitude below 464 to E4M3 bytes, with no clamp:
// the hardware conversion rounds to nearest even and gives 0x7E / 0xFE for
// every magnitude in [448, 464), the same bytes as clamping first. `spare`
// is any dead register: the first conversion keeps its high half, which the
// second one overwrites, so no zero has to be moved in.
__device__ __forceinline__ uint32_t e4m3x4_below464(float a, float b, float c, float d,
                                                    uint32_t spare) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)spare, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// The per-group cast q = E4M3(fl32(x * s)) of eight bf16, for scales
// s = fl32(448 / max(amax, EPS)) (or that rounded down to a power of two)
// with every |x| <= amax of its slice. Then |fl32(x * s)| < 464, so the clamp
// can be left out: with u = 2^-24, s <= (448 / max(amax, EPS)) (1 + u), hence
// |x * s| <= 448 (1 + u) and its binary32 rounding is at most 448 (1 + 2u).
__device__ __forceinline__ uint2 cast8_group(uint4 v, float s0, float s1, float s2, float s3,
                                             float s4, float s5, float s6, float s7) {
    uint2 r;
    r.x = e4m3x4_below464(bf16_lo(v.x) * s0, bf16_hi(v.x) * s1, bf16_lo(v.y) * s2,
                          bf16_hi(v.y) * s3, v.x);
    r.y = e4m3x4_below464(bf16_lo(v.z) * s4, bf16_hi(v.z) * s5, bf16_lo(v.w) * s6,
                          bf16_hi(v.w) * s7, v.z);
    return r;
}

__device__ __forceinline__ uint2 cast8_group(uint4 v, float s) {
    return cast8_group(v, s, s, s, s, s, s, s, s);
}

// ---- wave primitives ---------------------------------------------------------

// Inclusive prefix max over the 64 lanes of a wave, for non-negative values
// (0 is the identity): four row shifts inside each 16-lane row, then the two
// row broadcasts of the GFX9 DPP set.
__device__ __forceinline__ uint32_t wave_prefix_max(uint32_t v) {
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false)); // row_shr:1
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false)); // row_shr:2
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false)); // row_shr:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false)); // row_shr:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false)); // row_bcast:15
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false)); // row_bcast:31
    return v;
}

// Inclusive prefix sum over a wave (shuffles; used only on group tables).
__device__ __forceinline__ int wave_prefix_sum(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v += o;
    }
    return v;
}

__device__ __forceinline__ int wave_prefix_imax(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(v, d, kWave);
        if (lane >= d) v = max(v, o);
    }
    return v;
}

}  // namespace mgs
