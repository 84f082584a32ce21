// The first rungs of the ladder: one output element per lane.  Stages are
// those of amittech.dev, "3.5 Project: tiled matrix multiplication".
//
//  k0  stage 0 ("the naive baseline"): the stage's 16 x 16 block of lanes
//      with the faster lane index walking DOWN the rows of C.  On a 64-lane
//      wave that is 16 consecutive rows of 4 neighbouring columns, so each k
//      step of a wave reads A from 16 different rows and each store writes 16
//      different rows: 16 cache lines where one would do.  This is the
//      uncoalesced foil.  (With 64 rows of one column per wave instead, the
//      same reads thrash further: 196 ms and 73 GB read at square4096,
//      against 120 ms and 2.7 GB.)
//  k1  stage 1 ("global memory coalescing"): the same four waves turned the
//      other way, a wave's lanes along 64 consecutive COLUMNS of one row.  B
//      reads and C writes are 256 contiguous bytes per wave and the A
//      element is uniform across the wave (a 16 x 16 block, as on a 32-lane
//      machine, would split a 64-lane wave over four rows).
//  k2  stage 2 ("shared memory tiling"): per K step the workgroup stages a
//      TILE x TILE piece of A and of B in LDS, one element per lane each,
//      zero past the matrix edge, and every lane then runs TILE
//      multiply-adds out of LDS; one barrier after staging, one before the
//      next step overwrites the pieces.
//
//      LDS banking on gfx950: 64 banks of 4 bytes, and a wave's 64 lanes are
//      served together.  A wave of the 32 x 32 workgroup covers two tile rows
//      (lanes 0-31 one row, lanes 32-63 the next); with a row stride of 32
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
         int64_t blocks_m, int64_t blocks) {
    const int down = threadIdx.x % 16, across = threadIdx.x / 16;
    // Workgroup block: 16 rows x 16 columns of C, walked over the grid.
    for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x) {
        const int64_t i = (blk % blocks_m) * 16 + down;
        const int64_t j = (blk / blocks_m) * 16 + across;
        if (i >= M || j >= N) continue;
        const float* arow = A + i * lda;
        const float* bcol = B + j;
        float acc = 0.0f;
        for (int64_t k = 0; k < K; k++) acc += arow[k] * bcol[k * ldb];
        C[i * ldc + j] = acc;
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

template <int T, int PAD>
__global__ void __launch_bounds__(T * T)
k2_lds(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
       const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
       int64_t blocks_n, int64_t blocks) {
    constexpr int LD = T + PAD;  // LDS row stride in floats
    __shared__ __attribute__((aligned(16))) float sa[T * LD];
    __shared__ __attribute__((aligned(16))) float sb[T * LD];
    // The lane's output inside the T x T block; c is also the k offset it
    // stages from A, r the one it stages from B.
    const int r = threadIdx.x / T, c = threadIdx.x % T;
    for (int64_t blk = blockIdx.x; blk < blocks; blk += gridDim.x) {
        const int64_t i = (blk / blocks_n) * T + r;
        const int64_t j = (blk % blocks_n) * T + c;
        const bool row_in = i < M, col_in = j < N;
        const float* arow = A + (row_in ? i : 0) * lda;
        float acc = 0.0f;
        for (int64_t kt = 0; kt < K; kt += T) {
            sa[r * LD + c] = row_in && kt + c < K ? arow[kt + c] : 0.0f;
            sb[r * LD + c] = kt + r < K && col_in ? B[(kt + r) * ldb + j] : 0.0f;
            __syncthreads();
            const float* ar = sa + r * LD;
#pragma unroll
            for (int q = 0; q < T; q++) acc += ar[q] * sb[q * LD + c];
            __syncthreads();
        }
        if (row_in && col_in) C[i * ldc + j] = acc;
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
