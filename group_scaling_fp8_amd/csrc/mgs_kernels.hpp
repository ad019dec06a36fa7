// mgs_kernels.hpp — host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mgs_dim0_layout.hpp"

namespace mgs {

// team_max: the most chunks a group may have to be cast as a team (at most
// the CU count, see mgs_dim0.hip). ws: the dim0 workspace (Dim0Workspace
// layout for (M, K), zero-filled; every launch leaves it so), or null when M
// rows cannot make a chunked group. spin_ticks bounds a tile's wait
// for maxima written by other tiles, in device wall-clock ticks; past it the
// tile computes them itself. A negative value skips the wait.
// lt_cap: the widest strips allowed, 8 << lt_cap columns (dim0_lt_cap).
// uniform_rows >= 0: G equal groups of that many rows and no offsets array
// (off unused); -1: group ends from off. transposed: q is (K, M) and scales
// (K, G) (dim0_t); M and the group ends must then be multiples of 16 (ends
// are rounded down to them). xcd_split: XCD x (workgroups x, x + 8, ...)
// takes the tiles of columns [x K/8, (x + 1) K/8); K / 8 must be a multiple
// of the widest strip, 8 << lt_cap columns, and team_max at most the
// workgroups one XCD holds at once, halved (dim0_xcd_split). cus: the
// device's compute units (sizes the resident grid of few-round launches).
hipError_t launch_dim0(const uint16_t* x, int M, int K, const int32_t* off, int G, int uniform_rows,
                       bool pow2, bool transposed, uint8_t* q, float* scales, int team_max, int lt_cap,
                       bool xcd_split, void* ws, long long spin_ticks, int cus, hipStream_t stream);

// Zero fill of bytes / 16 16-byte words at p (16-byte aligned) by a kernel.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t stream);

// cus: compute units of the device; the grid is the workgroups that fit at once.
// K == 0: only the scales are written (every group empty).
hipError_t launch_dim1(const uint16_t* x, int64_t M, int K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, int cus, hipStream_t stream);

hipError_t launch_mx(const uint16_t* x, int64_t n_elems, bool rceil, uint8_t* q, uint8_t* scales,
                     hipStream_t stream);

// blocks of 32 along dim0 (M % 32 == 0), outputs transposed: q_t (K, M),
// scales_t (K, M/32)
hipError_t launch_mx_dim1(const uint16_t* x, int64_t M, int64_t K, bool rceil, uint8_t* q_t,
                          uint8_t* scales_t, hipStream_t stream);

hipError_t launch_mx_dequant(const uint8_t* q, const uint8_t* scales, int64_t n_elems, uint16_t* y,
                             hipStream_t stream);

hipError_t launch_cast(const float* in, int64_t n, uint8_t* out, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

}  // namespace mgs
