// Fourth rung: the FP32 matrix-core kernel for gfx950.
//
// amittech.dev, "3.5 Project: tiled matrix multiplication", section "what
// comes next", and the closing paragraph of the qsysarch.com "gemm-kernels"
// page point at the matrix units (AMD's Matrix Fused Multiply-Add) as the
// last step of the ladder.  On CDNA4 one v_mfma_f32_32x32x2_f32 multiplies a
// 32 x 2 slice of A by a 2 x 32 slice of B into a 32 x 32 float accumulator
// held across the wave's 64 lanes (16 registers per lane), at the same FP32
// rate as the vector units' peak but from two operand registers per lane.
//
// Structure (geometry and LDS layouts in k4_layout.h):
//  * a workgroup owns a BM x BN tile of C; each wave TM x TN accumulators;
//  * K is consumed in slabs of BK, double-buffered in LDS with one barrier
//    per slab: read this slab's fragments, issue the next slab's loads into
//    the other stage, run the slab's MFMAs, wait for the loads, barrier;
//  * global -> LDS uses buffer loads that write LDS directly
//    (buffer_load_dword[x4] ... lds), so staged data never occupies VGPRs;
//  * elements outside the matrix get a buffer offset past the descriptor's
//    range, which the hardware returns as zero: edge tiles and the K tail run
//    the same code; stores are masked only in edge tiles;
//  * 16-byte loads when both operands are 16-byte aligned and lda, ldb, K, N
//    are multiples of 4, else 4-byte loads (same LDS image either way);
//  * tile order: workgroup ids are dealt to the 8 XCDs round-robin, so ids
//    are remapped to give each XCD a contiguous range of tiles, walked in
//    groups of GROUP_M tile-rows so that resident tiles share A and B panels
//    in that XCD's L2.
#include "k4_layout.h"
#include "kernels.h"

namespace sgemm {

namespace {
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int GROUP_M = 8;
constexpr unsigned OOB = 0x80000000u;  // offset the buffer range check rejects
constexpr int RSRC_WORD3 = 0x00020000; // raw buffer, 32-bit data format
// Largest tile and slab any configuration uses (for the 31-bit offset limit).
constexpr int MAX_BM = 256, MAX_BN = 256, MAX_BK = 32;

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

template <class CF, int OCC>
__global__ void __launch_bounds__(CF::THREADS) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
k4_mfma(int64_t M, int64_t N, int64_t K, const float* __restrict__ A, int64_t lda,
        const float* __restrict__ B, int64_t ldb, float* __restrict__ C, int64_t ldc,
        int64_t tiles_m, int64_t tiles_n, int64_t tiles) {
    constexpr int TM = CF::TM, TN = CF::TN, KH = CF::KH, AQ = CF::A_QUADS;
    __shared__ __attribute__((aligned(1024))) char smem[CF::LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
    const int li = lane & 31, ls = lane >> 5;

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
        const int64_t row0 = (first_m + (lin % per_group) % gsz) * CF::BM;
        const int64_t col0 = ((lin % per_group) / gsz) * CF::BN;

        auto issue = [&](int64_t k0, int stage) {
            const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + row0 * lda + k0);
            const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + k0 * ldb + col0);
            char* base = smem + stage * CF::STAGE;
#pragma unroll
            for (int q = 0; q < CF::A_INSTR_PER_WAVE; q++) {
                const int u = wave * CF::A_INSTR_PER_WAVE + q;
                const int r = CF::a_load_row(u, lane), k = CF::a_load_k(u, lane);
                const bool ok = row0 + r < M && k0 + k < K;
                load_lds<CF::VEC>(ra, base + u * CF::IB,
                                  ok ? (unsigned)((r * lda + k) * 4) : OOB);
            }
#pragma unroll
            for (int q = 0; q < CF::B_INSTR_PER_WAVE; q++) {
                const int u = wave * CF::B_INSTR_PER_WAVE + q;
                const int k = CF::b_load_k(u, lane), c = CF::b_load_col(u, lane);
                const bool ok = k0 + k < K && col0 + c < N;
                load_lds<CF::VEC>(rb, base + CF::b_load_lds(u),
                                  ok ? (unsigned)((k * ldb + c) * 4) : OOB);
            }
        };

        v16f acc[TM][TN];
#pragma unroll
        for (int mb = 0; mb < TM; mb++)
#pragma unroll
            for (int nb = 0; nb < TN; nb++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[mb][nb][r] = 0.0f;

        const int64_t nk = (K + CF::BK - 1) / CF::BK;
        if (nk > 0) issue(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int64_t s = 0; s < nk; s++) {
            const char* st = smem + (s & 1) * CF::STAGE;
            v4f a[TM][AQ];
            float b[TN][KH];
#pragma unroll
            for (int mb = 0; mb < TM; mb++) {
                const int row = wm * TM * 32 + mb * 32 + li;
#pragma unroll
                for (int q = 0; q < AQ; q++)
                    a[mb][q] = *(const v4f*)(st + CF::a_frag(row, ls * AQ + q));
            }
#pragma unroll
            for (int nb = 0; nb < TN; nb++) {
                const int col = wn * TN * 32 + nb * 32 + li;
#pragma unroll
                for (int u = 0; u < KH; u++)
                    b[nb][u] = *(const float*)(st + CF::b_frag(CF::kslot(ls, u), col));
            }
            // All reads of this stage are issued before the next slab's
            // loads, which target the other stage.
            asm volatile("" ::: "memory");
            if (s + 1 < nk) issue((s + 1) * CF::BK, int((s + 1) & 1));
#pragma unroll
            for (int u = 0; u < KH; u++)
#pragma unroll
                for (int mb = 0; mb < TM; mb++)
#pragma unroll
                    for (int nb = 0; nb < TN; nb++)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                            a[mb][u / 4][u % 4], b[nb][u], acc[mb][nb], 0, 0, 0);
            // Register-only MFMAs may otherwise be scheduled after the wait
            // and barrier below, which would expose the load latency; tie
            // the accumulators to this point.
#pragma unroll
            for (int mb = 0; mb < TM; mb++)
#pragma unroll
                for (int nb = 0; nb < TN; nb++) asm volatile("" : "+a"(acc[mb][nb]));
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }

        // Accumulator register r of lane L holds row 8*(r/4) + 4*(L/32) + r%4,
        // column L%32 of its 32 x 32 block.
        const bool interior = row0 + CF::BM <= M && col0 + CF::BN <= N;
#pragma unroll
        for (int mb = 0; mb < TM; mb++)
#pragma unroll
            for (int nb = 0; nb < TN; nb++) {
                const int64_t c = col0 + wn * TN * 32 + nb * 32 + li;
                const int64_t rbase = row0 + wm * TM * 32 + mb * 32 + ls * 4;
                float* cp = C + rbase * ldc + c;
                if (interior) {
#pragma unroll
                    for (int r = 0; r < 16; r++) cp[((r / 4) * 8 + (r % 4)) * ldc] = acc[mb][nb][r];
                } else if (c < N) {
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        if (rbase + (r / 4) * 8 + (r % 4) < M)
                            cp[((r / 4) * 8 + (r % 4)) * ldc] = acc[mb][nb][r];
                }
            }
    }
}

template <class CF, int OCC>
hipError_t launch_k4_cfg(const GemmArgs& g, hipStream_t s) {
    const int64_t tm = ceil_div(g.M, CF::BM), tn = ceil_div(g.N, CF::BN), tiles = tm * tn;
    hipLaunchKernelGGL((k4_mfma<CF, OCC>), dim3(grid_for(tiles)), dim3(CF::THREADS), 0, s, g.M,
                       g.N, g.K, g.A, g.lda, g.B, g.ldb, g.C, g.ldc, tm, tn, tiles);
    return hipGetLastError();
}

bool k4_supports(const GemmArgs& g) {
    // Largest valid byte offset from a slab's base must stay below OOB.
    const int64_t lim = int64_t(OOB) - 64;
    return ((int64_t)(MAX_BM - 1) * g.lda + MAX_BK) * 4 < lim &&
           ((int64_t)(MAX_BK - 1) * g.ldb + MAX_BN) * 4 < lim;
}

static bool vec_ok(const GemmArgs& g) {
    return (reinterpret_cast<uintptr_t>(g.A) % 16 == 0) &&
           (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
           g.K % 4 == 0 && g.N % 4 == 0;
}

// Tile configurations (chosen from a sweep over square 256..8192, skinny and
// unaligned shapes on MI355X):
//  * 128 x 128 tiles, 4 waves of 2 x 2 accumulators, K slabs of 16, 4 waves
//    per SIMD: best once there are at least 1024 tiles (4 per CU), e.g.
//    square 4096 and 8192;
//  * 64 x 64 tiles, 4 waves of 1 accumulator: below that, the larger tile
//    count fills the 256 CUs (square 1024: 2.9x faster than 128 x 128);
//    K slabs of 32 with 16-byte loads, of 16 with 4-byte loads.
template <bool V> using Tile128 = k4::Cfg<2, 2, 2, 2, 16, V>;
using Tile64Vec = k4::Cfg<2, 2, 1, 1, 32, true>;
using Tile64Dword = k4::Cfg<2, 2, 1, 1, 16, false>;

hipError_t launch_k4_tile128(const GemmArgs& g, hipStream_t s) {
    if (vec_ok(g)) return launch_k4_cfg<Tile128<true>, 4>(g, s);
    return launch_k4_cfg<Tile128<false>, 3>(g, s);
}

hipError_t launch_k4_tile64(const GemmArgs& g, hipStream_t s) {
    if (vec_ok(g)) return launch_k4_cfg<Tile64Vec, 4>(g, s);
    return launch_k4_cfg<Tile64Dword, 8>(g, s);
}

hipError_t launch_k4_mfma(const GemmArgs& g, hipStream_t s) {
    const int64_t tiles128 = ceil_div(g.M, 128) * ceil_div(g.N, 128);
    if (vec_ok(g) && tiles128 >= 1024) return launch_k4_cfg<Tile128<true>, 4>(g, s);
    return launch_k4_tile64(g, s);
}

}  // namespace sgemm
