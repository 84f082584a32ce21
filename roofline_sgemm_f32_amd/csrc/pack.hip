// Operand packing for the matrix-core kernel's 16-byte load path.
//
// That path moves four consecutive floats of an operand's contiguous
// dimension per lane, so it needs 16-byte aligned rows and a row length
// (the "run") that is a multiple of 4, or else rows padded with zeros up to
// one.  pack_rows copies a stored rows x cols matrix (any alignment, any
// leading dimension) into a dense rows x ld_dst one, ld_dst = cols rounded
// up to 4, with the extra columns zero: a 16-byte chunk that straddles the
// end of a row then reads zeros, whose products add exactly nothing.
#include <algorithm>

#include "kernels.h"

namespace sgemm {

namespace {
struct PackJob {
    const float* src;
    int64_t rows, cols, ld;
    float* dst;
};

// gridDim.y jobs (one or two matrices).  A workgroup copies whole rows, a
// grid-stride loop over them; lane i moves elements i, i + 256, ... of a
// row, so every load and store instruction covers 256 consecutive bytes
// whatever the source's alignment.  No division per element.
__global__ void __launch_bounds__(256)
pack_rows(PackJob j0, PackJob j1) {
    const PackJob j = blockIdx.y == 0 ? j0 : j1;
    const int64_t ld_dst = (j.cols + 3) / 4 * 4;
    for (int64_t r = blockIdx.x; r < j.rows; r += gridDim.x) {
        const float* s = j.src + r * j.ld;
        float* d = j.dst + r * ld_dst;
        for (int64_t c = threadIdx.x; c < ld_dst; c += blockDim.x) d[c] = c < j.cols ? s[c] : 0.0f;
    }
}
}  // namespace

int64_t packed_ld(int64_t cols) { return (cols + 3) / 4 * 4; }

hipError_t launch_pack(const float* src, int64_t rows, int64_t cols, int64_t ld, float* dst,
                       const float* src2, int64_t rows2, int64_t cols2, int64_t ld2, float* dst2,
                       hipStream_t s) {
    const PackJob j0{src, rows, cols, ld, dst}, j1{src2, rows2, cols2, ld2, dst2};
    // Up to 1024 workgroups per matrix (4 per CU), whole rows each.
    const int64_t rmax = src2 ? std::max(rows, rows2) : rows;
    const unsigned grid = unsigned(std::max<int64_t>(1, std::min<int64_t>(rmax, 1024)));
    hipLaunchKernelGGL(pack_rows, dim3(grid, src2 ? 2 : 1), dim3(256), 0, s, j0, j1);
    return hipGetLastError();
}

}  // namespace sgemm
