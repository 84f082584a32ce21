// Operand packing for the matrix-core kernel's 16-byte load path.
//
// That path moves four consecutive floats of an operand's contiguous
// dimension per lane, so it needs 16-byte aligned rows and a row length
// (the "run") that is a multiple of 4, or else rows padded with zeros up to
// one.  pack_rows copies a stored rows x cols matrix (any alignment, any
// leading dimension) into a dense rows x ld_dst one, ld_dst = cols rounded
// up to 4, with the extra columns zero: a 16-byte chunk that straddles the
// end of a row then reads zeros, whose products add exactly nothing.
#include "kernels.h"

namespace sgemm {

namespace {
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256)
pack_rows(const float* __restrict__ src, int64_t rows, int64_t cols, int64_t ld,
          float* __restrict__ dst, int64_t ld_dst) {
    const int64_t q = ld_dst / 4, total = rows * q;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / q, c = (i % q) * 4;
        const float* s = src + r * ld;
        v4f v;
#pragma unroll
        for (int e = 0; e < 4; e++) v[e] = c + e < cols ? s[c + e] : 0.0f;
        *(v4f*)(dst + r * ld_dst + c) = v;
    }
}
}  // namespace

int64_t packed_ld(int64_t cols) { return (cols + 3) / 4 * 4; }

hipError_t launch_pack(const float* src, int64_t rows, int64_t cols, int64_t ld, float* dst,
                       hipStream_t s) {
    const int64_t ld_dst = packed_ld(cols);
    hipLaunchKernelGGL(pack_rows, dim3(grid_for(ceil_div(rows * (ld_dst / 4), 256))), dim3(256), 0, s,
                       src, rows, cols, ld, dst, ld_dst);
    return hipGetLastError();
}

}  // namespace sgemm
