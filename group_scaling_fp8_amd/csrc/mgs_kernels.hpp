// mgs_kernels.hpp — host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgs {

// dim0 tiling: 512-thread workgroups holding kDim0Slabs 16-byte vectors per
// thread; groups taller than kDim0HugeRows are cut into chunks of at most
// kDim0HugeChunkRows rows whose column maxima go through a workspace.
constexpr int kDim0Slabs = 20;
constexpr int kDim0HugeRows = 5120;
constexpr int kDim0HugeChunkRows = 640;

// Upper bound on the chunks of groups taller than kDim0HugeRows: such a group
// of s rows has ceil(s / 640) <= s / 640 + 1 chunks, and there are at most
// M / 5121 such groups.
inline int64_t dim0_huge_chunk_bound(int64_t M) {
    if (M <= kDim0HugeRows) return 0;
    return M / kDim0HugeChunkRows + M / (kDim0HugeRows + 1) + 1;
}

// Persistent grid of the dim0 kernels: two 512-thread workgroups per CU.
int dim0_grid();

hipError_t launch_dim0(const uint16_t* x, int M, int K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, uint32_t* ws, int grid, hipStream_t stream);

hipError_t launch_dim1(const uint16_t* x, int64_t M, int K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, hipStream_t stream);

hipError_t launch_mx(const uint16_t* x, int64_t n_elems, bool rceil, uint8_t* q, uint8_t* scales,
                     hipStream_t stream);

hipError_t launch_cast(const float* in, int64_t n, uint8_t* out, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

}  // namespace mgs
