// The first rungs of the ladder: one output element per lane.
//
//  k0  one lane per C element, consecutive lanes walk DOWN a column of C
//      (amittech.dev, "3.5 Project: tiled matrix multiplication", stage 0):
//      a wave's A reads and C writes are row-strided - the uncoalesced foil.
//  k1  consecutive lanes walk ALONG a row of C (same page, stage 1): B reads
//      and C writes are contiguous per wave and the A element is uniform
//      across the wave.  On a 64-lane wavefront the workgroup is 64 x 4, so
//      one wave covers 64 consecutive columns of one row (a 16 x 16 block
//      would split a wave over four rows and four 64-byte segments).
//  k2  the same page, stage 2: the workgroup stages a TILE x TILE block of A
//      and of B in LDS per K step (zero-filled past the matrix edge), with a
//      barrier after the loads and another before the next overwrite.
//
//      LDS banking on gfx950: 64 banks of 4 bytes, and a wave's 64 lanes are
//      served together.  A wave of the 32 x 32 workgroup covers two tile rows
//      (lanes 0-31 row ty, lanes 32-63 row ty+1); with a row stride of 32
//      floats the two halves fall in banks b..b+31 and b+32..b+63, so the
//      unpadded tile is already conflict-free, and its 128-byte aligned rows
//      let the inner loop read A four floats at a time.  A wave of the
//      16 x 16 workgroup covers four rows at stride 16: banks 16r..16r+15,
//      again all 64 distinct.  Padding rows by one float (stride 33 or 17)
//      is the comparison point: it stays conflict-free at 32 but loses the
//      vector reads, and at 16 the fourth row wraps onto the first row's
//      banks.
#include "kernels.h"

namespace sgemm {

__global__ void __launch_bounds__(256)
k0_naive(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
         const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
         int64_t tiles_m, int64_t tiles) {
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t row = (t % tiles_m) * 16 + tx;  // x -> row
        const int64_t col = (t / tiles_m) * 16 + ty;  // y -> column
        if (row < M && col < N) {
            float sum = 0.0f;
            for (int64_t k = 0; k < K; k++) sum += A[row * lda + k] * B[k * ldb + col];
            C[row * ldc + col] = sum;
        }
    }
}

__global__ void __launch_bounds__(256)
k1_coalesced(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
             const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
             int64_t tiles_n, int64_t tiles) {
    const int lane = threadIdx.x % 64;
    // The row is the same for the whole wave; say so, so that A is read
    // through the scalar unit once per wave.
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t row = (t / tiles_n) * 4 + wave;
        const int64_t col = (t % tiles_n) * 64 + lane;
        if (row < M && col < N) {
            const float* a = A + row * lda;
            const float* b = B + col;
            float sum = 0.0f;
            for (int64_t k = 0; k < K; k++) sum += a[k] * b[k * ldb];
            C[row * ldc + col] = sum;
        }
    }
}

template <int TILE, int PAD>
__global__ void __launch_bounds__(TILE * TILE)
k2_lds(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
       const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
       int64_t tiles_n, int64_t tiles) {
    __shared__ float As[TILE][TILE + PAD];
    __shared__ float Bs[TILE][TILE + PAD];
    const int tx = threadIdx.x % TILE, ty = threadIdx.x / TILE;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t row = (t / tiles_n) * TILE + ty;
        const int64_t col = (t % tiles_n) * TILE + tx;
        float sum = 0.0f;
        for (int64_t k0 = 0; k0 < K; k0 += TILE) {
            const int64_t ak = k0 + tx, bk = k0 + ty;
            As[ty][tx] = (row < M && ak < K) ? A[row * lda + ak] : 0.0f;
            Bs[ty][tx] = (bk < K && col < N) ? B[bk * ldb + col] : 0.0f;
            __syncthreads();  // the tile is complete before anyone reads it
#pragma unroll
            for (int k = 0; k < TILE; k++) sum += As[ty][k] * Bs[k][tx];
            __syncthreads();  // everyone is done before the next overwrite
        }
        if (row < M && col < N) C[row * ldc + col] = sum;
    }
}

// The general form C = alpha op(A) op(B) + beta C with k1's mapping (lanes
// along a row of C) and 64-bit offsets everywhere; it serves the shapes
// whose per-slab offsets the matrix-core kernel's 32-bit buffer addressing
// cannot reach.
__global__ void __launch_bounds__(256)
k1_general(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
           const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
           bool ta, bool tb, float alpha, float beta, int64_t tiles_n, int64_t tiles) {
    const int lane = threadIdx.x % 64;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t row = (t / tiles_n) * 4 + wave;
        const int64_t col = (t % tiles_n) * 64 + lane;
        if (row < M && col < N) {
            const int64_t a_step = ta ? lda : 1, b_step = tb ? 1 : ldb;
            const float* a = A + (ta ? row : row * lda);
            const float* b = B + (tb ? col * ldb : col);
            float sum = 0.0f;
            for (int64_t k = 0; k < K; k++) sum += a[k * a_step] * b[k * b_step];
            float v = alpha * sum;
            if (beta != 0.0f) v = fmaf(beta, C[row * ldc + col], v);
            C[row * ldc + col] = v;
        }
    }
}

__global__ void __launch_bounds__(256)
scale_c(float* __restrict__ C, int64_t M, int64_t N, int64_t ldc, float beta) {
    const int64_t total = M * N, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        float* p = C + (i / N) * ldc + (i % N);
        *p = beta == 0.0f ? 0.0f : beta * *p;
    }
}

hipError_t launch_k1_general(const GemmArgs& g, hipStream_t s) {
    const int64_t tn = ceil_div(g.N, 64), tiles = tn * ceil_div(g.M, 4);
    hipLaunchKernelGGL(k1_general, dim3(grid_for(tiles)), dim3(256), 0, s, g.M, g.N, g.K, g.A,
                       g.lda, g.B, g.ldb, g.C, g.ldc, g.trans_a, g.trans_b, g.alpha, g.beta, tn,
                       tiles);
    return hipGetLastError();
}

hipError_t launch_scale(float* C, int64_t M, int64_t N, int64_t ldc, float beta, hipStream_t s) {
    hipLaunchKernelGGL(scale_c, dim3(grid_for(ceil_div(M * N, 256))), dim3(256), 0, s, C, M, N, ldc,
                       beta);
    return hipGetLastError();
}

hipError_t launch_k0_naive(const GemmArgs& g, hipStream_t s) {
    const int64_t tm = ceil_div(g.M, 16), tiles = tm * ceil_div(g.N, 16);
    hipLaunchKernelGGL(k0_naive, dim3(grid_for(tiles)), dim3(256), 0, s, g.M, g.N, g.K, g.A,
                       g.lda, g.B, g.ldb, g.C, g.ldc, tm, tiles);
    return hipGetLastError();
}

hipError_t launch_k1_coalesced(const GemmArgs& g, hipStream_t s) {
    const int64_t tn = ceil_div(g.N, 64), tiles = tn * ceil_div(g.M, 4);
    hipLaunchKernelGGL(k1_coalesced, dim3(grid_for(tiles)), dim3(256), 0, s, g.M, g.N, g.K, g.A,
                       g.lda, g.B, g.ldb, g.C, g.ldc, tn, tiles);
    return hipGetLastError();
}

template <int TILE, int PAD>
static hipError_t launch_k2_t(const GemmArgs& g, hipStream_t s) {
    const int64_t tn = ceil_div(g.N, TILE), tiles = tn * ceil_div(g.M, TILE);
    hipLaunchKernelGGL((k2_lds<TILE, PAD>), dim3(grid_for(tiles)), dim3(TILE * TILE), 0, s, g.M,
                       g.N, g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, tn, tiles);
    return hipGetLastError();
}

hipError_t launch_k2_lds(const GemmArgs& g, int tile, int pad, hipStream_t s) {
    if (tile == 16) return pad ? launch_k2_t<16, 1>(g, s) : launch_k2_t<16, 0>(g, s);
    return pad ? launch_k2_t<32, 1>(g, s) : launch_k2_t<32, 0>(g, s);
}

}  // namespace sgemm
