/*
 * mgs_oracle.h — plain, slow, single-threaded CPU reference for per-group
 * fp8 scaling and the MX block-32 cast.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header, table or
 * constant generator with the HIP library.
 *
 * Sources (page titles, then the part of the page):
 *   [ROWWISE]   "[moe fp8 training] test and bench new faster method for per
 *               group rowwise scaling" — Summary (per-group rowwise scales,
 *               transpose method), Benchmarks table (shapes, group counts).
 *   [BLOCKSIZE] "[moe training] use smaller block sizes for per group scaling
 *               kernels to improve perf" — description (per-token-group
 *               scaling along dim0) and the torch.compile failure report,
 *               whose kernel-argument dict fixes fp8_dtype_min = -448,
 *               fp8_dtype_max = 448, EPS = 1e-12 and
 *               round_scales_to_power_of_2; its test source sets the token
 *               group alignment to 16.
 *   [MXA2A]     "[mxfp8 moe training] fix mxfp8 a2a bench script; set mxfp8
 *               a2a scaling type to RCEIL" — Summary (RCEIL scaling type,
 *               fp32 -> e8m0 cast) and the investigation comment (mxfp8
 *               dim0 cast in FLOOR mode).
 *   OCP 8-bit Floating Point Specification (OFP8) rev 1.0, E4M3 format.
 *   OCP Microscaling Formats (MX) Specification v1.0, E8M0 scale format.
 *
 * All arrays are contiguous row-major host arrays. bf16 values are passed as
 * their raw uint16 bit patterns. Offsets are int32 END offsets: group g
 * covers [off[g-1], off[g]) with off[-1] = 0.
 */
#ifndef MGS_ORACLE_H
#define MGS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* OFP8 E4M3 (bias 7, no infinities, S.1111.111 = NaN, max finite 448),
 * round to nearest with ties to even, saturating to +-448. NaN keeps its
 * sign: 0x7F / 0xFF. The argument is the exact real value to encode. */
uint8_t oracle_e4m3_encode(double v);

/* Element-wise oracle_e4m3_encode over n values. */
void oracle_e4m3_encode_array(const double *v, int64_t n, uint8_t *out);

/* oracle_e4m3_encode of the binary32 values whose bit patterns are
 * first, first + 1, ..., first + n - 1 (mod 2^32). */
void oracle_e4m3_encode_f32_bits(uint32_t first, int64_t n, uint8_t *out);

/* Decodes one E4M3 byte to its real value (NaN codes decode to NaN). */
double oracle_e4m3_decode(uint8_t code);

/* bf16 bit pattern -> binary32 value (bf16 is the upper half of binary32). */
float oracle_bf16_to_f32(uint16_t bits);

/* Per-group scale: 448 / max(amax, 1e-12) in IEEE binary32, optionally
 * rounded down to a power of two. */
float oracle_group_scale(float amax, int pow2);

/* Per-group scaling along dim0: x (M, K); groups split the M rows.
 * Writes q (M, K) E4M3 bytes and scales (G, K) fp32. Returns 0, or -1 if
 * the offsets are not a non-decreasing cover of [0, M]. */
int oracle_quant_groups_dim0(const uint16_t *x, int64_t M, int64_t K,
                             const int32_t *offsets, int32_t G, int pow2,
                             uint8_t *q, float *scales);

/* Per-group scaling along dim1: x (M, K); groups split the K columns.
 * Writes q (M, K) E4M3 bytes and scales (M, G) fp32. Same return codes. */
int oracle_quant_groups_dim1(const uint16_t *x, int64_t M, int64_t K,
                             const int32_t *offsets, int32_t G, int pow2,
                             uint8_t *q, float *scales);

/* MX exponent of one block: the e such that the block is scaled by 2^-e.
 * mode 0 = FLOOR: e = floor(log2 amax) - 8 (8 = exponent of the largest
 * power of two not above 448). mode 1 = RCEIL: the smallest integer e with
 * amax <= 448 * 2^e. amax == 0 gives -127. The result is clamped to
 * [-127, 127]; the stored E8M0 byte is e + 127. */
int oracle_mx_exponent(float amax, int mode);

/* MX block-32 cast along the last dim: x (M, K), K % 32 == 0. Writes q (M, K)
 * E4M3 bytes and scales (M, K/32) E8M0 bytes. Returns 0 or -1 on bad args. */
int oracle_mx_quant_dim0(const uint16_t *x, int64_t M, int64_t K, int mode,
                         uint8_t *q, uint8_t *scales);

/* bf16 rounding (nearest even, overflow to infinity) of an exact value. */
uint16_t oracle_f64_to_bf16(double v);

/* MX dequantisation: y (M, K) bf16 = E4M3(q) * 2^(byte - 127) per block of
 * 32 along K ([MXA2A] Summary: the dequantise step after the all-to-all;
 * OCP MX E8M0). Byte 0xFF or a NaN code gives 0x7FC0. Returns -1 unless
 * K % 32 == 0. */
int oracle_mx_dequant_dim0(const uint8_t *q, const uint8_t *scales, int64_t M, int64_t K,
                           uint16_t *y);

#ifdef __cplusplus
}
#endif

#endif
