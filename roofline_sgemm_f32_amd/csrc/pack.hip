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
// whatever the source's alignment.  For rows longer than two such steps
// the loads of kPackU steps are all issued before their stores, so a row of
// up to 2048 floats costs one memory round trip rather than one per 256
// floats (767 x 769 x 4095 70.5 us per product against 71.7, 513 x 511 x
// 8193 66.5 against 68.8); shorter rows keep the plain loop, which the
// unrolled one slowed (8192 x 13 x 8192: 62.0 against 60.7).  No division
// per element.
constexpr int kPackU = 8;

__global__ void __launch_bounds__(256)
pack_rows(PackJob j0, PackJob j1) {
    const PackJob j = blockIdx.y == 0 ? j0 : j1;
    const int64_t ld_dst = (j.cols + 3) / 4 * 4;
    for (int64_t r = blockIdx.x; r < j.rows; r += gridDim.x) {
        const float* s = j.src + r * j.ld;
        float* d = j.dst + r * ld_dst;
        if (ld_dst <= 2 * 256) {
            for (int64_t c = threadIdx.x; c < ld_dst; c += 256) d[c] = c < j.cols ? s[c] : 0.0f;
            continue;
        }
        for (int64_t c0 = threadIdx.x; c0 < ld_dst; c0 += int64_t(256) * kPackU) {
            float v[kPackU];
#pragma unroll
            for (int u = 0; u < kPackU; u++) {
                const int64_t c = c0 + 256 * u;
                v[u] = c < j.cols ? s[c] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kPackU; u++) {
                const int64_t c = c0 + 256 * u;
                if (c < ld_dst) d[c] = v[u];
            }
        }
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
