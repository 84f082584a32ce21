// Third rung: register tiling with an LDS double buffer, on the vector ALUs.
//
// amittech.dev, "3.5 Project: tiled matrix multiplication", section "what
// comes next", names the two steps after one-output-per-lane tiling: each
// lane computing an 8 x 8 block of outputs from registers, and loading the
// next tile while the current one is being used.  The qsysarch.com
// "gemm-kernels" page (section on improving the naive kernel) describes the
// same coarsening with a K x K block per thread strided across the tile.
//
// Here a 256-lane workgroup owns a 128 x 128 tile of C.  Lane (tx, ty) of the
// 16 x 16 arrangement owns rows {4ty..4ty+3, 64+4ty..64+4ty+3} and the same
// pattern of columns, so each K step reads four 16-byte vectors from LDS
// (two of A, two of B) and issues 64 fused multiply-adds.  A is stored
// k-major (transposed) in LDS so that a lane's four rows are contiguous.
// The next K slab is fetched into registers before the current slab's math
// and written to the other LDS buffer after it: one barrier per slab.
// Out-of-range elements load as zero; 64-bit offsets throughout, so every
// shape the interface accepts is addressable.
#include "kernels.h"

namespace sgemm {

namespace {
constexpr int BM = 128, BN = 128, BK = 8, PAD = 4;
typedef float v4f __attribute__((ext_vector_type(4)));
}  // namespace

template <bool VEC>
__global__ void __launch_bounds__(256)
k3_regtile(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
           const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
           int64_t tiles_n, int64_t tiles) {
    __shared__ __attribute__((aligned(16))) float As[2][BK][BM + PAD];
    __shared__ __attribute__((aligned(16))) float Bs[2][BK][BN + PAD];
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;
    // Global -> register staging assignment (fixed per lane).
    const int a_r = tid / 2, a_k = (tid % 2) * 4;   // A: row a_r, k a_k..a_k+3
    const int b_k = tid / 32, b_c = (tid % 32) * 4;  // B: k row b_k, columns b_c..b_c+3

    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const int64_t row0 = (t / tiles_n) * BM, col0 = (t % tiles_n) * BN;
        float acc[8][8];
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < 8; j++) acc[i][j] = 0.0f;

        float ra[4], rb[4];
        auto fetch = [&](int64_t k0) {
            const int64_t ar = row0 + a_r, ak = k0 + a_k;
            const int64_t bk = k0 + b_k, bc = col0 + b_c;
            if (VEC) {
                // Whole 4-vectors are in or out: K and N are multiples of 4.
                v4f va = (ar < M && ak < K) ? *(const v4f*)(A + ar * lda + ak) : v4f{0, 0, 0, 0};
                v4f vb = (bk < K && bc < N) ? *(const v4f*)(B + bk * ldb + bc) : v4f{0, 0, 0, 0};
#pragma unroll
                for (int e = 0; e < 4; e++) { ra[e] = va[e]; rb[e] = vb[e]; }
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    ra[e] = (ar < M && ak + e < K) ? A[ar * lda + ak + e] : 0.0f;
                    rb[e] = (bk < K && bc + e < N) ? B[bk * ldb + bc + e] : 0.0f;
                }
            }
        };
        auto stash = [&](int buf) {
#pragma unroll
            for (int e = 0; e < 4; e++) As[buf][a_k + e][a_r] = ra[e];
            *(v4f*)&Bs[buf][b_k][b_c] = v4f{rb[0], rb[1], rb[2], rb[3]};
        };

        const int64_t nk = (K + BK - 1) / BK;
        if (nk > 0) {
            fetch(0);
            stash(0);
        }
        __syncthreads();
        for (int64_t s = 0; s < nk; s++) {
            const int cur = int(s & 1);
            if (s + 1 < nk) fetch((s + 1) * BK);  // in flight during the math below
#pragma unroll
            for (int k = 0; k < BK; k++) {
                const v4f a0 = *(const v4f*)&As[cur][k][ty * 4];
                const v4f a1 = *(const v4f*)&As[cur][k][64 + ty * 4];
                const v4f b0 = *(const v4f*)&Bs[cur][k][tx * 4];
                const v4f b1 = *(const v4f*)&Bs[cur][k][64 + tx * 4];
                const float a[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
                const float b[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
                for (int i = 0; i < 8; i++)
#pragma unroll
                    for (int j = 0; j < 8; j++) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            // The other buffer was last read before the previous barrier.
            if (s + 1 < nk) stash(cur ^ 1);
            __syncthreads();
        }

#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t r = row0 + (i < 4 ? ty * 4 + i : 64 + ty * 4 + i - 4);
            if (r >= M) continue;
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const int64_t c = col0 + (j < 4 ? tx * 4 + j : 64 + tx * 4 + j - 4);
                if (c < N) C[r * ldc + c] = acc[i][j];
            }
        }
    }
}

hipError_t launch_k3_regtile(const GemmArgs& g, hipStream_t s) {
    const int64_t tn = ceil_div(g.N, BN), tiles = tn * ceil_div(g.M, BM);
    const bool vec = (reinterpret_cast<uintptr_t>(g.A) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && g.lda % 4 == 0 &&
                     g.ldb % 4 == 0 && g.K % 4 == 0 && g.N % 4 == 0;
    if (vec)
        hipLaunchKernelGGL(k3_regtile<true>, dim3(grid_for(tiles)), dim3(256), 0, s, g.M, g.N,
                           g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, tn, tiles);
    else
        hipLaunchKernelGGL(k3_regtile<false>, dim3(grid_for(tiles)), dim3(256), 0, s, g.M, g.N,
                           g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, tn, tiles);
    return hipGetLastError();
}

}  // namespace sgemm
