// Operand packing for the matrix-core kernel's 16-byte load path.
//
// That path moves four consecutive floats of an operand's contiguous
// dimension per lane, so it needs 16-byte aligned rows and a row length
// (the "run") that is a multiple of 4, or else rows padded with zeros up to
// one.  pack_rows copies a stored rows x cols matrix (any alignment, any
// leading dimension) into a dense rows x ld_dst one, ld_dst = packed_ld(cols)
// (a multiple of 4), with the extra columns zero: a 16-byte chunk that
// straddles the end of a row then reads zeros, whose products add exactly
// nothing.
#include <algorithm>

#include "kernels.h"

namespace sgemm {

namespace {
struct PackJob {
    const float* src;
    int64_t rows, cols, ld;
    float* dst;
};

// gridDim.y jobs (one or two matrices).  Lane i moves elements i, i + 256,
// ... of a row, so every load and store instruction covers 256 consecutive
// bytes whatever the source's alignment.  Rows longer than 512 floats go in
// pieces of kPackPiece floats whose loads (kPackU steps) are all issued
// before their stores: one memory round trip per piece rather than one per
// 256 floats (767 x 769 x 4095 70.5 us per product against 71.7, 513 x 511
// x 8193 66.5 against 68.8).  A workgroup takes whole rows in a grid-stride
// loop, except in a matrix of at most one row per CU, whose pieces go to
// workgroups of their own (13 x 8192 x 8191: 59.1 -> 57.0 us); spreading the
// pieces of more rows slowed the copy (767 x 769 x 4095: 70.9 -> 72.6).
// Rows of at most 512 floats keep the plain loop, which the unrolled one
// slowed (8192 x 13 x 8192: 62.0 against 60.7).  No division per element.
constexpr int kPackU = 8;
constexpr int kPackPiece = 256 * kPackU;
constexpr int64_t kPackGrid = 1024;       // workgroups for rows of pieces
constexpr int64_t kPackGridShort = 2048;  // and for rows of at most 512 floats
constexpr int64_t kPackFewRows = 256;     // rows whose pieces are spread

__device__ __forceinline__ void pack_piece(const float* s, float* d, int64_t c0, int64_t cols,
                                           int64_t ld_dst) {
    float v[kPackU];
#pragma unroll
    for (int q = 0; q < kPackU; q++) {
        const int64_t c = c0 + 256 * q;
        v[q] = c < cols ? s[c] : 0.0f;
    }
#pragma unroll
    for (int q = 0; q < kPackU; q++) {
        const int64_t c = c0 + 256 * q;
        if (c < ld_dst) d[c] = v[q];
    }
}

__global__ void __launch_bounds__(256)
pack_rows(PackJob j0, PackJob j1) {
    const PackJob j = blockIdx.y == 0 ? j0 : j1;
    const int64_t ld_dst = packed_ld(j.cols);
    if (ld_dst <= 2 * 256) {
        for (int64_t r = blockIdx.x; r < j.rows; r += gridDim.x) {
            const float* s = j.src + r * j.ld;
            float* d = j.dst + r * ld_dst;
            for (int64_t c = threadIdx.x; c < ld_dst; c += 256) d[c] = c < j.cols ? s[c] : 0.0f;
        }
    } else if (j.rows <= kPackFewRows) {
        const int64_t pieces = (ld_dst + kPackPiece - 1) / kPackPiece;
        for (int64_t u = blockIdx.x; u < j.rows * pieces; u += gridDim.x) {
            const int64_t r = u / pieces;
            pack_piece(j.src + r * j.ld, j.dst + r * ld_dst, (u % pieces) * kPackPiece + threadIdx.x,
                       j.cols, ld_dst);
        }
    } else {
        for (int64_t r = blockIdx.x; r < j.rows; r += gridDim.x)
            for (int64_t c0 = threadIdx.x; c0 < ld_dst; c0 += kPackPiece)
                pack_piece(j.src + r * j.ld, j.dst + r * ld_dst, c0, j.cols, ld_dst);
    }
}
}  // namespace

hipError_t launch_pack(const float* src, int64_t rows, int64_t cols, int64_t ld, float* dst,
                       const float* src2, int64_t rows2, int64_t cols2, int64_t ld2, float* dst2,
                       hipStream_t s) {
    const PackJob j0{src, rows, cols, ld, dst}, j1{src2, rows2, cols2, ld2, dst2};
    // Workgroups: one per row (or piece of a row in a matrix of few rows), at
    // most kPackGridShort (8 per CU) for rows of at most 512 floats and
    // kPackGrid otherwise: the wider grid sped up narrow copies (8192 x 13 x
    // 8192 60.6 -> 59.2 us per product) and slowed long-row ones (800 x 801 x
    // 2047 43.1 -> 44.2).
    auto want = [](int64_t r, int64_t c) {
        const int64_t ld = packed_ld(c);
        if (ld <= 2 * 256) return std::min(r, kPackGridShort);
        return std::min(r <= kPackFewRows ? r * ((ld + kPackPiece - 1) / kPackPiece) : r, kPackGrid);
    };
    const int64_t g = src2 ? std::max(want(rows, cols), want(rows2, cols2)) : want(rows, cols);
    const unsigned grid = unsigned(std::max<int64_t>(1, g));
    hipLaunchKernelGGL(pack_rows, dim3(grid, src2 ? 2 : 1), dim3(256), 0, s, j0, j1);
    return hipGetLastError();
}

}  // namespace sgemm
