// Fourth rung: the FP32 matrix-core kernel for gfx950.
//
// amittech.dev, "3.5 Project: tiled matrix multiplication", section "what
// comes next", and the closing paragraph of the qsysarch.com "gemm-kernels"
// page point at the matrix units (AMD's Matrix Fused Multiply-Add) as the
// last step of the ladder.  On CDNA4 one v_mfma_f32_32x32x2_f32 multiplies a
// 32 x 2 slice of A by a 2 x 32 slice of B into a 32 x 32 float accumulator
// held across the wave's 64 lanes (16 registers per lane), at the same FP32
// rate as packed vector FMA but from two operand registers per lane.
//
// Workgroup: 256 lanes = 4 waves in a 2 x 2 arrangement, tile 128 x 128 of C,
// K consumed in slabs of 16.  Each wave owns a 64 x 64 sub-tile = 2 x 2
// MFMA blocks (64 accumulator registers per lane).
//
// Global -> LDS: buffer loads that write LDS directly (buffer_load ... lds),
// so staged data never passes through VGPRs.  Each such load fills a
// contiguous run of LDS (lane L's bytes at L * size), and the lane chooses
// which global element it fetches; that choice implements the LDS layouts
// below.  Elements outside the matrix get an offset past the buffer's range,
// which the hardware returns as zero: edge tiles and the K tail need no
// separate path.  With 16-byte aligned operands whose rows and K, N are
// multiples of 4 floats each lane moves 16 bytes (dwordx4); otherwise 4.
//
// LDS layouts (two stages, double buffered, one barrier per slab):
//   A stage: 128 rows x 16 floats (64 B per row).  The four 16-byte chunks of
//            row r are stored XOR-permuted by swz(r), so that the eight (or
//            sixteen) rows read together by a ds_read_b128 land in distinct
//            banks.
//   B stage: 16 rows x 128 floats, written as 8 blocks of two rows (1 KiB)
//            with a 32-byte gap after each block.  Rows k and k+8, read in
//            the same instruction by the two halves of a wave, then sit 128
//            bytes apart modulo 256 and hit different banks.
//
// MFMA operand mapping.  The 32x32x2 instruction gives lane L the A element
// (i = L % 32, kslot = L / 32) and the B element (kslot = L / 32, j = L % 32).
// Which real k a slot stands for is free as long as A and B agree; here
// kslot s at step t (0..7) is k = 8s + t, so a lane's eight A values of the
// slab are contiguous (two ds_read_b128) and its B values are single floats
// of one column.
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin by id, so ids
// are remapped to give each XCD a contiguous range of tiles, and tiles are
// walked in groups of 8 tile-rows so that concurrently running tiles share A
// and B panels in that XCD's L2.
#include "kernels.h"

namespace sgemm {

namespace {
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int BM = 128, BN = 128, BK = 16;
constexpr int A_STAGE = BM * BK * 4;           // 8192 bytes
constexpr int B_BLOCK = 2 * BN * 4;            // two k-rows, 1024 bytes
constexpr int B_BLOCK_STRIDE = B_BLOCK + 32;   // 1056 bytes
constexpr int B_STAGE = (BK / 2) * B_BLOCK_STRIDE;
constexpr int STAGE = A_STAGE + B_STAGE;       // 16640 bytes
constexpr int GROUP_M = 8;
constexpr unsigned OOB = 0x80000000u;          // offset the buffer range check rejects
constexpr int RSRC_WORD3 = 0x00020000;         // raw buffer, 32-bit data format

// Chunk permutation of A row r (4 chunks of 16 bytes per row).
__device__ __forceinline__ int swz(int r) { return ((r >> 1) & 3) ^ ((r >> 3) & 1); }

// One buffer load that writes LDS directly: lane L's 16 (or 4) bytes go to
// lds + 16 L (or 4 L).
template <bool VEC>
__device__ __forceinline__ void load_lds(__amdgpu_buffer_rsrc_t r, char* lds, unsigned off) {
    if constexpr (VEC)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(lds), 16, off, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, LDS_PTR(lds), 4, off, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)OOB,
                                             RSRC_WORD3);
}
}  // namespace

template <bool VEC>
__global__ void __launch_bounds__(256)
k4_mfma(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
        const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
        int64_t tiles_m, int64_t tiles_n, int64_t tiles) {
    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int li = lane & 31, ls = lane >> 5;

    // Per-lane global element (row/k for A, k/column for B) of each load
    // instruction, fixed for the whole kernel.
    constexpr int NA = VEC ? 2 : 8;  // load instructions per wave per slab, A
    constexpr int NB = VEC ? 2 : 8;  // and B
    int a_r[NA], a_k[NA], b_k[NB], b_c[NB];
    unsigned a_lds[NA], b_lds[NB];
#pragma unroll
    for (int q = 0; q < NA; q++) {
        if (VEC) {
            const int u = wave * 2 + q;             // 16 rows per instruction
            const int r = u * 16 + lane / 4, pc = lane % 4;
            a_r[q] = r;
            a_k[q] = 4 * (pc ^ swz(r));
            a_lds[q] = u * 1024;
        } else {
            const int u = wave * 8 + q;             // 4 rows per instruction
            const int p = u * 64 + lane, r = p / 16, qq = p % 16;
            a_r[q] = r;
            a_k[q] = 4 * ((qq / 4) ^ swz(r)) + qq % 4;
            a_lds[q] = u * 256;
        }
    }
#pragma unroll
    for (int q = 0; q < NB; q++) {
        if (VEC) {
            const int u = wave * 2 + q;             // one two-row block per instruction
            b_k[q] = 2 * u + lane / 32;
            b_c[q] = (lane % 32) * 4;
            b_lds[q] = A_STAGE + u * B_BLOCK_STRIDE;
        } else {
            const int u = wave * 8 + q;             // a quarter block per instruction
            const int o = (u % 4) * 256 + lane * 4;
            b_k[q] = 2 * (u / 4) + o / 512;
            b_c[q] = (o % 512) / 4;
            b_lds[q] = A_STAGE + (u / 4) * B_BLOCK_STRIDE + (u % 4) * 256;
        }
    }

    // Fragment addresses inside a stage (bytes).
    int a_frag[2][2];
#pragma unroll
    for (int mb = 0; mb < 2; mb++) {
        const int r = wm * 64 + mb * 32 + li;
#pragma unroll
        for (int q = 0; q < 2; q++) a_frag[mb][q] = r * 64 + (((2 * ls + q) ^ swz(r)) * 16);
    }
    int b_frag[2];
#pragma unroll
    for (int nb = 0; nb < 2; nb++) b_frag[nb] = A_STAGE + (wn * 64 + nb * 32 + li) * 4;

    const bool direct = (int64_t)gridDim.x == tiles;
    for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        // XCD-contiguous remap of the workgroup id, then grouped tile order.
        int64_t lin = t;
        if (direct) {
            const int64_t q = tiles / 8, rem = tiles % 8, x = t % 8;
            lin = x * q + (x < rem ? x : rem) + t / 8;
        }
        const int64_t per_group = (int64_t)GROUP_M * tiles_n;
        const int64_t first_m = (lin / per_group) * GROUP_M;
        const int64_t gsz = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
        const int64_t tile_m = first_m + (lin % per_group) % gsz;
        const int64_t tile_n = (lin % per_group) / gsz;
        const int64_t row0 = tile_m * BM, col0 = tile_n * BN;

        // Slab-invariant parts of the load offsets.
        unsigned a_off[NA], b_off[NB];
        bool a_ok[NA], b_ok[NB];
#pragma unroll
        for (int q = 0; q < NA; q++) {
            a_ok[q] = row0 + a_r[q] < M;
            a_off[q] = (unsigned)((a_r[q] * lda + a_k[q]) * 4);
        }
#pragma unroll
        for (int q = 0; q < NB; q++) {
            b_ok[q] = col0 + b_c[q] < N;
            b_off[q] = (unsigned)((b_k[q] * ldb + b_c[q]) * 4);
        }

        auto issue = [&](int64_t k0, int stage) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + row0 * lda + k0);
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + k0 * ldb + col0);
            char* base = smem + stage * STAGE;
#pragma unroll
            for (int q = 0; q < NA; q++) {
                const unsigned off = (a_ok[q] && k0 + a_k[q] < K) ? a_off[q] : OOB;
                load_lds<VEC>(ra, base + a_lds[q], off);
            }
#pragma unroll
            for (int q = 0; q < NB; q++) {
                const unsigned off = (b_ok[q] && k0 + b_k[q] < K) ? b_off[q] : OOB;
                load_lds<VEC>(rb, base + b_lds[q], off);
            }
        };

        v16f acc[2][2];
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int nb = 0; nb < 2; nb++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[mb][nb][r] = 0.0f;

        const int64_t nk = (K + BK - 1) / BK;
        if (nk > 0) issue(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int64_t s = 0; s < nk; s++) {
            const char* st = smem + (s & 1) * STAGE;
            v4f a[2][2];
            float b[2][8];
#pragma unroll
            for (int mb = 0; mb < 2; mb++)
#pragma unroll
                for (int q = 0; q < 2; q++) a[mb][q] = *(const v4f*)(st + a_frag[mb][q]);
#pragma unroll
            for (int nb = 0; nb < 2; nb++)
#pragma unroll
                for (int u = 0; u < 8; u++) {
                    const int k = ls * 8 + u;
                    b[nb][u] = *(const float*)(st + b_frag[nb] + (k / 2) * B_BLOCK_STRIDE +
                                               (k % 2) * (BN * 4));
                }
            // All reads of this stage are issued before the next slab's
            // loads, which target the other stage.
            asm volatile("" ::: "memory");
            if (s + 1 < nk) issue((s + 1) * BK, int((s + 1) & 1));
#pragma unroll
            for (int u = 0; u < 8; u++)
#pragma unroll
                for (int mb = 0; mb < 2; mb++)
#pragma unroll
                    for (int nb = 0; nb < 2; nb++)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            a[mb][u / 4][u % 4], b[nb][u], acc[mb][nb], 0, 0, 0);
            // Register-only MFMAs may otherwise be scheduled after the wait
            // and barrier below, which would expose the load latency; tie
            // the accumulators to this point.
#pragma unroll
            for (int mb = 0; mb < 2; mb++)
#pragma unroll
                for (int nb = 0; nb < 2; nb++) asm volatile("" : "+a"(acc[mb][nb]));
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // Accumulator register r of lane L holds row 8*(r/4) + 4*(L/32) + r%4,
        // column L%32 of its 32 x 32 block.
        const bool interior = row0 + BM <= M && col0 + BN <= N;
#pragma unroll
        for (int mb = 0; mb < 2; mb++)
#pragma unroll
            for (int nb = 0; nb < 2; nb++) {
                const int64_t c = col0 + wn * 64 + nb * 32 + li;
                float* cp = C + (row0 + wm * 64 + mb * 32 + ls * 4) * ldc + c;
                if (interior) {
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        cp[((r / 4) * 8 + (r % 4)) * ldc] = acc[mb][nb][r];
                } else {
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int64_t row = row0 + wm * 64 + mb * 32 + (r / 4) * 8 + ls * 4 + (r % 4);
                        if (row < M && c < N) cp[((r / 4) * 8 + (r % 4)) * ldc] = acc[mb][nb][r];
                    }
                }
            }
    }
}

bool k4_supports(const GemmArgs& g) {
    // Largest valid byte offset from a slab's base must stay below OOB.
    const int64_t lim = int64_t(OOB) - 64;
    return ((int64_t)(BM - 1) * g.lda + BK) * 4 < lim && ((int64_t)(BK - 1) * g.ldb + BN) * 4 < lim;
}

hipError_t launch_k4_mfma(const GemmArgs& g, hipStream_t s) {
    const int64_t tm = ceil_div(g.M, BM), tn = ceil_div(g.N, BN), tiles = tm * tn;
    const bool vec = (reinterpret_cast<uintptr_t>(g.A) % 16 == 0) &&
                     (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && g.lda % 4 == 0 &&
                     g.ldb % 4 == 0 && g.K % 4 == 0 && g.N % 4 == 0;
    if (vec)
        hipLaunchKernelGGL(k4_mfma<true>, dim3(grid_for(tiles)), dim3(256), 0, s, g.M, g.N, g.K,
                           g.A, g.lda, g.B, g.ldb, g.C, g.ldc, tm, tn, tiles);
    else
        hipLaunchKernelGGL(k4_mfma<false>, dim3(grid_for(tiles)), dim3(256), 0, s, g.M, g.N, g.K,
                           g.A, g.lda, g.B, g.ldb, g.C, g.ldc, tm, tn, tiles);
    return hipGetLastError();
}

}  // namespace sgemm
