// mgs_kernels.hpp — host-side launchers of the gfx950 kernels (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mgs {

// dim0 tiling: a chunk is up to kDim0ChunkRows rows x kDim0StripCols columns.
constexpr int kDim0Slabs = 32;
constexpr int kDim0ChunkRows = 16 * kDim0Slabs;
constexpr int kDim0StripCols = 128;

// Upper bound on the number of chunks over all groups: a group of s rows
// has ceil(s / C) <= floor(s / C) + 1 chunks (1 if empty).
inline int64_t dim0_chunk_bound(int64_t M, int64_t G) { return M / kDim0ChunkRows + G; }

// Upper bound on the chunks of groups taller than one chunk: each such group
// has s > C rows, so there are at most floor(M / C) of them, and its chunks
// number at most floor(s / C) + 1.
inline int64_t dim0_tall_chunk_bound(int64_t M, int64_t G) {
    const int64_t f = M / kDim0ChunkRows;
    if (M <= kDim0ChunkRows) return 0;
    return f + (G < f ? G : f);
}

hipError_t launch_dim0(const uint16_t* x, int M, int64_t K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, uint32_t* ws, int64_t tall_chunk_bound,
                       hipStream_t stream);

hipError_t launch_dim1(const uint16_t* x, int64_t M, int K, const int32_t* off, int G, bool pow2,
                       uint8_t* q, float* scales, hipStream_t stream);

hipError_t launch_mx(const uint16_t* x, int64_t n_elems, bool rceil, uint8_t* q, uint8_t* scales,
                     hipStream_t stream);

hipError_t launch_cast(const float* in, int64_t n, uint8_t* out, hipStream_t stream);

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t stream);

}  // namespace mgs
