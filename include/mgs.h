/*
 * mgs.h — MI355X (gfx950) per-group fp8 scaling: C ABI of libmgs.so.
 *
 * The method (page titles, then the part of the page that defines it):
 *   [ROWWISE]   "[moe fp8 training] test and bench new faster method for per
 *               group rowwise scaling" — Summary: per-group rowwise scales of
 *               the backward's grouped GEMM operand, and the transpose
 *               identity between rowwise and colwise per-group scaling.
 *   [BLOCKSIZE] "[moe training] use smaller block sizes for per group scaling
 *               kernels to improve perf" — description: per-token-group
 *               scaling along dim0; torch.compile failure report: kernel
 *               argument dict (fp8_dtype_min -448, fp8_dtype_max 448,
 *               EPS 1e-12, round_scales_to_power_of_2, in-place output) and
 *               the token-group alignment of 16 in its test source.
 *   [MXA2A]     "[mxfp8 moe training] fix mxfp8 a2a bench script; set mxfp8
 *               a2a scaling type to RCEIL" — Summary and investigation
 *               comment: the mxfp8 dim0 cast, FLOOR and RCEIL scaling.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major
 *     arrays owned by the caller; outputs are fully overwritten in place.
 *     bf16 inputs are raw 16-bit patterns (upper halves of binary32).
 *   - `offsets` are int32 END offsets in device memory: group g covers
 *     [off[g-1], off[g]) with off[-1] = 0. They must be non-decreasing and
 *     off[n_groups-1] must equal the grouped extent. They are not checked on
 *     the host (that would need a device sync). The kernels clamp them into
 *     range, so bad offsets give wrong values but no out-of-bounds access.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call is
 *     asynchronous and stream-ordered. Calls are thread-safe.
 *   - Return value: an mgs_status. Argument errors are reported before any
 *     GPU work is queued. MGS_ERR_HIP reports a failed launch or allocation.
 *   - The library reads no environment variables and never synchronises a
 *     stream or the device, except under MGS_FLAG_VALIDATE. It allocates
 *     device memory in one place only: mgs_quant_groups_dim0, and the other
 *     dim0-family calls when given no workspace, keep a workspace of their
 *     own (described there). Every other call, and every call given a
 *     workspace, allocates and frees nothing.
 *   - Numerics: scale = fl32(448 / max(amax, 1e-12)) with one IEEE binary32
 *     division. With MGS_FLAG_POW2_SCALE it is rounded down to a power of
 *     two. q = E4M3(fl32(x * scale)): clamp to [-448, 448], round to
 *     nearest with ties to even (OCP OFP8 E4M3, 0x7E = 448). Subnormals are
 *     preserved, and the sign of zero is kept.
 *   - Inputs must be finite (no NaN or Inf); non-finite inputs are outside
 *     the contract.
 */
#ifndef MGS_H
#define MGS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MGS_OK = 0,
    MGS_ERR_INVALID_ARG = 1,   /* null pointer, bad size, alignment, flag or mode */
    MGS_ERR_UNSUPPORTED = 2,   /* valid but beyond this library's limits */
    MGS_ERR_HIP = 3            /* a HIP launch or allocation failed */
} mgs_status;

#define MGS_FLAG_POW2_SCALE 1u /* round scales down to a power of two */
/* Debug aid for the two grouped entry points: copy the offsets to the host
 * (synchronising the stream) and return MGS_ERR_INVALID_ARG unless they are
 * non-decreasing, within [0, extent], end at the extent (M for dim0, K for
 * dim1) and, for dim1, are multiples of 16. Without it, device offsets are
 * not checked (bad ones give unspecified values, never an out-of-bounds
 * access). MGS_ERR_UNSUPPORTED on a stream that is capturing a graph. */
#define MGS_FLAG_VALIDATE 2u

enum { MGS_MX_FLOOR = 0, MGS_MX_RCEIL = 1 };

#define MGS_MAX_GROUPS 1024    /* n_groups limit of the grouped entry points */
#define MGS_DIM1_MAX_K 131072  /* row length limit of mgs_quant_groups_dim1 */

/*
 * Per-group scaling along dim0 ([BLOCKSIZE] description; constants from the
 * kernel-argument dict of its torch.compile failure report).
 *   x       (M, K) bf16. Groups split the M rows.
 *   offsets n_groups int32 end offsets along M, 1 <= n_groups <= 1024.
 *   flags   0, MGS_FLAG_POW2_SCALE, MGS_FLAG_VALIDATE.
 *   q       (M, K) E4M3 bytes, written.
 *   scales  (n_groups, K) fp32, written. scales[g, k] is the multiplier for
 *           column k of group g. An empty group still gets its row, with the
 *           value for amax = 0 (0x57CBBA10, or 0x57800000 with pow2).
 * Requirements: M >= 0, K >= 0, K % 8 == 0; x 16-byte aligned, q 8-byte
 * aligned, scales 16-byte aligned. M == 0 writes only the scales; K == 0 is a
 * no-op.
 * Tall groups: a group taller than 896 rows is cut into chunks of at most
 * 896 rows (a tile holds 896 rows of 128 columns: 160 KiB in registers and
 * 64 KiB in LDS). The chunks' column maxima pass between workgroups of the
 * one kernel launch through a device workspace of
 * mgs_dim0_workspace_bytes(M, K) bytes (0 when M <= 896, else about
 * M * K / 112 bytes). A tile that waits for other tiles' maxima waits at most
 * about 20 ms of device wall clock; past that it computes them from x
 * itself, so the result never depends on workgroup scheduling.
 * Memory: this call takes no workspace argument (its signature is the one
 * the per-group dim0 cast is known by), so it uses the library's own: one
 * per (device, stream), allocated with hipMalloc and zero-filled by a kernel
 * on the stream the first time a call on that stream needs one, and
 * replaced by a larger one when a later call needs more. Replaced buffers
 * are kept until process exit (graphs captured earlier may still use them);
 * nothing is freed and no stream is synchronised. Inside graph capture no
 * allocation is possible: a capturing call that needs more workspace than
 * its stream has returns MGS_ERR_UNSUPPORTED. mgs_quant_groups_dim0_ws takes
 * the workspace from the caller instead and never allocates. Calls sharing a
 * workspace must not run at the same time (calls on one stream never do).
 * Errors: MGS_ERR_UNSUPPORTED if the tile count bound reaches 2^31.
 */
int mgs_quant_groups_dim0(const void *x, int64_t M, int64_t K,
                          const int32_t *offsets, int32_t n_groups,
                          uint32_t flags, void *q, float *scales,
                          void *stream);

/*
 * Size in bytes of the workspace that the dim0-family calls on an (M, K)
 * input need (mgs_quant_groups_dim0_ws, mgs_quant_groups_dim0_t, and
 * mgs_quant_experts_dim1 with M = E * D1, K = D2): 0 when M <= 896 (no group
 * can be cut into chunks), else, with c = M / 896 + M / 897 chunk rows,
 * round_up(4 * c * ceil(K / 128), 256) + 8 * c * (K / 2).
 * Host only; no GPU work. Returns MGS_ERR_INVALID_ARG for a null `bytes` or
 * negative sizes, MGS_ERR_UNSUPPORTED for M or K over 2^31 - 1.
 */
int mgs_dim0_workspace_bytes(int64_t M, int64_t K, int64_t *bytes);

/*
 * mgs_quant_groups_dim0 with a workspace owned by the caller, the form that
 * leaves every allocation to the caller ([BLOCKSIZE] torch.compile failure
 * report: the kernel writes caller-provided outputs in place, and its
 * constants are launch parameters).
 *   workspace        device memory of at least mgs_dim0_workspace_bytes(M, K)
 *                    bytes, 256-byte aligned, zero-filled by the caller
 *                    before its first use. Every call leaves it zero-filled
 *                    again (each team of workgroups clears the counter and
 *                    the column maxima it used), so it needs no clearing
 *                    between calls and serves calls of any shape that fits
 *                    it. Two calls that may run at the same time (on
 *                    different streams) need two workspaces. NULL with
 *                    workspace_bytes 0 selects the library's own workspace
 *                    (exactly mgs_quant_groups_dim0). When the required size
 *                    is 0 the workspace is not touched.
 *   workspace_bytes  its size.
 * Never allocates, frees or synchronises (MGS_FLAG_VALIDATE aside), so it
 * can be captured into a graph on any stream.
 * Errors: as mgs_quant_groups_dim0, plus MGS_ERR_INVALID_ARG for a workspace
 * that is misaligned or smaller than required, or a NULL workspace with a
 * nonzero size.
 */
int mgs_quant_groups_dim0_ws(const void *x, int64_t M, int64_t K,
                             const int32_t *offsets, int32_t n_groups,
                             uint32_t flags, void *q, float *scales,
                             void *workspace, int64_t workspace_bytes,
                             void *stream);

/*
 * mgs_quant_groups_dim0 for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the workspace is a fixed array of MGS_NOALLOC_SCRATCH_BYTES
 * inside the library's code object, one per device, held until the process
 * ends. Arguments, results and errors are those of mgs_quant_groups_dim0,
 * plus MGS_ERR_UNSUPPORTED when mgs_dim0_workspace_bytes(M, K) exceeds that
 * size (roughly M * K > 1.8e9; inputs with M <= 896 need no workspace at
 * all). Allocates and frees nothing. The first call on a device that needs
 * the array clears it with a kernel queued on the call's stream (a call
 * captured before any eager one puts that clear into its graph); every call
 * leaves it clear again. All calls on one device share the array: calls that
 * may overlap in time (on different streams) race and give wrong results.
 */
#define MGS_NOALLOC_SCRATCH_BYTES (16u << 20)
int mgs_quant_groups_dim0_noalloc(const void *x, int64_t M, int64_t K,
                                  const int32_t *offsets, int32_t n_groups,
                                  uint32_t flags, void *q, float *scales,
                                  void *stream);

/*
 * Per-group scaling along dim0 with transposed outputs ([ROWWISE] Summary:
 * per-group colwise scales computed on one layout give the per-group rowwise
 * scales of its transpose; its stacked change names the transpose method as
 * the way to keep global accesses coalesced). Same values as
 * mgs_quant_groups_dim0, written transposed in one pass, so the result is
 * the rowwise per-group scaling of x^T in GEMM-ready row-major form without
 * x^T ever being stored.
 *   x        (M, K) bf16, token-major. Groups split the M rows.
 *   offsets  n_groups int32 end offsets along M, each a multiple of 16 (the
 *            token-group alignment of [BLOCKSIZE]'s test source),
 *            1 <= n_groups <= 1024. Ends are rounded down to a multiple of
 *            16 on the device, so other offsets give unspecified values but
 *            no out-of-bounds access.
 *   flags    0, MGS_FLAG_POW2_SCALE, MGS_FLAG_VALIDATE.
 *   q_t      (K, M) E4M3 bytes, written: q_t[k, r] = dim0's q[r, k].
 *   scales_t (K, n_groups) fp32, written: scales_t[k, g] = dim0's
 *            scales[g, k]; empty groups get the amax = 0 value.
 *   workspace, workspace_bytes  as for mgs_quant_groups_dim0_ws (NULL, 0:
 *            the library's own workspace).
 * Requirements: M % 16 == 0, K % 8 == 0; x and q_t 16-byte aligned,
 * scales_t 4-byte aligned. M == 0 writes only the scales; K == 0 is a
 * no-op. Tiles, chunks, the bounded wait and errors are as for
 * mgs_quant_groups_dim0_ws (the LDS that holds a tile's last rows is reused
 * as the transposed output stage once they are cast), except that strips
 * are at most 1024 columns wide.
 */
int mgs_quant_groups_dim0_t(const void *x, int64_t M, int64_t K,
                            const int32_t *offsets, int32_t n_groups,
                            uint32_t flags, void *q_t, float *scales_t,
                            void *workspace, int64_t workspace_bytes,
                            void *stream);

/*
 * Per-expert scaling of a 3D expert weight along its dim 1 ([ROWWISE]'s
 * stacked changes: a fused reduction kernel along dim1 for 3d expert weights
 * in the backward pass; [BLOCKSIZE]'s: fp8 rowwise kernels for expert
 * weights). Reading: one scale per (expert, column), from the amax over the
 * expert's D1 rows, fused with the cast -- dim0's per-group scaling of the
 * (E * D1, D2) view with E equal groups of D1 rows, and no offsets array.
 *   w       (E, D1, D2) bf16.
 *   flags   0 or MGS_FLAG_POW2_SCALE (MGS_FLAG_VALIDATE is accepted and
 *           has nothing to check).
 *   q       (E, D1, D2) E4M3 bytes, written.
 *   scales  (E, D2) fp32, written.
 *   workspace, workspace_bytes  as for mgs_quant_groups_dim0_ws with
 *           M = E * D1, K = D2 (NULL, 0: the library's own workspace).
 * Requirements: 1 <= E <= 1024, D1 >= 0, E * D1 < 2^31, D2 % 8 == 0; w
 * 16-byte aligned, q 8-byte aligned, scales 16-byte aligned. Experts taller
 * than 896 rows are cut into chunks exactly as dim0's groups (bounded wait
 * and errors as for mgs_quant_groups_dim0_ws).
 */
int mgs_quant_experts_dim1(const void *w, int64_t E, int64_t D1, int64_t D2,
                           uint32_t flags, void *q, float *scales,
                           void *workspace, int64_t workspace_bytes,
                           void *stream);

/*
 * Per-group rowwise scaling along dim1 ([ROWWISE] Summary).
 *   x       (M, K) bf16. Groups split the K columns.
 *   offsets n_groups int32 end offsets along K. Every offset must be a
 *           multiple of 16 (the token-group alignment of [BLOCKSIZE]'s test
 *           source), 1 <= n_groups <= 1024.
 *   flags   0 or MGS_FLAG_POW2_SCALE.
 *   q       (M, K) E4M3 bytes, written.
 *   scales  (M, n_groups) fp32, written. Empty groups get the amax = 0 value.
 * Requirements: K % 16 == 0, K <= MGS_DIM1_MAX_K (else MGS_ERR_UNSUPPORTED);
 * x 16-byte aligned, q 8-byte aligned, scales 4-byte aligned. M == 0 is a
 * no-op. K == 0 leaves every group empty: nothing is read and q is empty,
 * but all M * n_groups scales are written with the amax = 0 value (x and q
 * may then be NULL).
 */
int mgs_quant_groups_dim1(const void *x, int64_t M, int64_t K,
                          const int32_t *offsets, int32_t n_groups,
                          uint32_t flags, void *q, float *scales,
                          void *stream);

/*
 * MX-style block-32 cast along the last dim ([MXA2A] investigation comment:
 * the mxfp8 dim0 cast; Summary: RCEIL scaling type).
 *   x       (M, K) bf16, K % 32 == 0. Each block of 32 consecutive elements
 *           of a row has amax a. Its exponent e is floor(log2 a) - 8 (FLOOR)
 *           or the smallest integer with a <= 448 * 2^e (RCEIL). e is
 *           clamped to [-127, 127], and a == 0 gives -127.
 *   offsets, n_groups  accepted so that the three calls share a shape. Blocks
 *           never cross a row, so token groups cannot change the result.
 *           They are ignored and may be NULL / 0.
 *   mode    MGS_MX_FLOOR or MGS_MX_RCEIL.
 *   q       (M, K) E4M3 bytes: E4M3(x * 2^-e), saturating, RNE.
 *   scales_e8m0  (M, K/32) bytes: e + 127 (OCP MX E8M0).
 * Requirements: x 16-byte aligned, q 8-byte aligned.
 */
int mgs_mx_quant_dim0(const void *x, int64_t M, int64_t K,
                      const int32_t *offsets, int32_t n_groups, int mode,
                      void *q, uint8_t *scales_e8m0, void *stream);

/*
 * MX-style block-32 cast along dim0, written transposed (the dim1 form of
 * [MXA2A]'s cast benchmark modes: blocks of 32 consecutive rows of one
 * column). The values are mgs_mx_quant_dim0's on x^T, computed from x in
 * one pass without storing x^T.
 *   x         (M, K) bf16, M % 32 == 0, K % 8 == 0.
 *   mode      MGS_MX_FLOOR or MGS_MX_RCEIL (as for mgs_mx_quant_dim0).
 *   q_t       (K, M) E4M3 bytes: q_t[k, r] is x[r, k] cast with the scale
 *             of rows 32 * (r / 32) .. + 31 of column k.
 *   scales_t  (K, M/32) bytes, E8M0 (exponent + 127).
 * Requirements: x and q_t 16-byte aligned. M == 0 or K == 0 is a no-op.
 */
int mgs_mx_quant_dim1(const void *x, int64_t M, int64_t K, int mode,
                      void *q_t, uint8_t *scales_t, void *stream);

/*
 * MX dequantisation along the last dim ([MXA2A] Summary: the dequantise step
 * that follows the all-to-all of mxfp8-quantised tokens; OCP MX E8M0):
 *   q            (M, K) E4M3 bytes, K % 32 == 0.
 *   scales_e8m0  (M, K/32) bytes; block b of row r covers q[r, 32b .. 32b+31].
 *   y            (M, K) bf16, written: y = bf16(E4M3(q) * 2^(byte - 127)),
 *                rounded to nearest even (the product itself is exact);
 *                overflow gives infinity. Byte 0xFF (E8M0 NaN) or an E4M3 NaN
 *                code gives the quiet NaN 0x7FC0.
 * Requirements: q and y 16-byte aligned. M == 0 or K == 0 is a no-op.
 */
int mgs_mx_dequant_dim0(const void *q, const uint8_t *scales_e8m0, int64_t M,
                        int64_t K, void *y, void *stream);

/*
 * The library's own E4M3 cast on its own: out[i] = E4M3(clamp(in[i])), the
 * last step of every entry point above, exposed so it can be checked over
 * 2^32 binary32 inputs. in: n fp32 values, out: n bytes (device). +-Inf
 * saturate to 0x7E / 0xFE; NaN inputs are outside the contract.
 * Requirements: n % 4 == 0, in 16-byte aligned, out 4-byte aligned.
 */
int mgs_cast_e4m3(const float *in, int64_t n, uint8_t *out, void *stream);

/*
 * A plain device-to-device copy kernel of `bytes` bytes (bytes % 16 == 0,
 * both pointers 16-byte aligned), used to calibrate HBM traffic counters
 * against a kernel of known size.
 */
int mgs_copy(const void *src, void *dst, int64_t bytes, void *stream);

/*
 * TEST ONLY (not part of the product interface): the dim0-family cast with
 * two launch parameters overridden, so tests can reach paths that the
 * defaults reach only under rare scheduling.
 *   uniform_rows  -1: groups from offsets (mgs_quant_groups_dim0_ws, or
 *                 mgs_quant_groups_dim0_t when transposed != 0); >= 0:
 *                 n_groups equal groups of that many rows and no offsets
 *                 (mgs_quant_experts_dim1 with E = n_groups, D1 =
 *                 uniform_rows; M must be E * D1, transposed must be 0).
 *   spin_ticks    bound on a tile's wait for other tiles' column maxima, in
 *                 device wall-clock ticks; -1 skips the wait (the waiting
 *                 tile computes the maxima from x); below -1: the default.
 *   team_max      1 up to the library's limit lowers the most chunks a group
 *                 may have and still be cast by one team of workgroups
 *                 (taller groups then read their chunks twice); other
 *                 values: the default.
 * Every other argument is as for the call it stands for.
 */
int mgs_test_quant_dim0(const void *x, int64_t M, int64_t K,
                        const int32_t *offsets, int32_t n_groups,
                        int64_t uniform_rows, uint32_t flags, int transposed,
                        void *q, float *scales, void *workspace,
                        int64_t workspace_bytes, int64_t spin_ticks,
                        int32_t team_max, void *stream);

/* Static text for a status code. */
const char *mgs_status_string(int status);

/* The last HIP error code seen by this library on the calling thread (0 if
 * none); meaningful after a call returned MGS_ERR_HIP. */
int mgs_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MGS_H */
