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
typedef float v4f __attribute__((ext_vector_type(4)));

struct PackJob {
    const float* src;
    int64_t rows, cols, ld;
    float* dst;
};

// gridDim.y jobs (one or two matrices), each copied by a grid-stride loop
// over its 4-float output chunks.
__global__ void __launch_bounds__(256)
pack_rows(PackJob j0, PackJob j1) {
    const PackJob j = blockIdx.y == 0 ? j0 : j1;
    const int64_t ld_dst = (j.cols + 3) / 4 * 4, q = ld_dst / 4, total = j.rows * q;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / q, c = (i % q) * 4;
        const float* s = j.src + r * j.ld;
        v4f v;
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = c + e < j.cols ? s[c + e] : 0.0f;
        *(v4f*)(j.dst + r * ld_dst + c) = v;
    }
}
}  // namespace

int64_t packed_ld(int64_t cols) { return (cols + 3) / 4 * 4; }

hipError_t launch_pack(const float* src, int64_t rows, int64_t cols, int64_t ld, float* dst,
                       const float* src2, int64_t rows2, int64_t cols2, int64_t ld2, float* dst2,
                       hipStream_t s) {
    const PackJob j0{src, rows, cols, ld, dst}, j1{src2, rows2, cols2, ld2, dst2};
    int64_t chunks = rows * (packed_ld(cols) / 4);
    if (src2) chunks = std::max(chunks, rows2 * (packed_ld(cols2) / 4));
    hipLaunchKernelGGL(pack_rows, dim3(grid_for(ceil_div(chunks, 256)), src2 ? 2 : 1), dim3(256), 0, s,
                       j0, j1);
    return hipGetLastError();
}

}  // namespace sgemm
