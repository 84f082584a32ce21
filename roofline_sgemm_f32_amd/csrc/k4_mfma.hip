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

template <class CF, int OCC, int GM = GROUP_M, bool XCD_REMAP = true, bool SPLIT = false>
__global__ void __launch_bounds__(CF::THREADS) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
k4_mfma(int M, int N, int K, const float* __restrict__ A, int lda, const float* __restrict__ B,
        int ldb, float* __restrict__ C, int64_t ldc, float alpha, float beta, int tiles_m,
        int tiles_n, int tiles) {
    // 32-bit sizes: the host routes shapes whose sizes, leading dimensions
    // or slab offsets do not fit (k4_supports) to the 64-bit kernel.
    constexpr int TM = CF::TM, TN = CF::TN, KH = CF::KH;
    using LA = typename CF::LA;
    using LB = typename CF::LB;
    __shared__ __attribute__((aligned(1024))) char smem[CF::LDS_BYTES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
    const int li = lane & 31, ls = lane >> 5;

    const bool direct = XCD_REMAP && (int)gridDim.x == tiles;
    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
        // XCD-contiguous remap of the workgroup id, then grouped tile order.
        int lin = t;
        if (direct) {
            const int q = tiles / 8, rem = tiles % 8, x = t % 8;
            lin = x * q + (x < rem ? x : rem) + t / 8;
        }
        const int per_group = GM * tiles_n;
        const int first_m = (lin / per_group) * GM;
        const int gsz = (tiles_m - first_m) < GM ? (tiles_m - first_m) : GM;
        const int row0 = (first_m + (lin % per_group) % gsz) * CF::BM;
        const int col0 = ((lin % per_group) / gsz) * CF::BN;

        auto issue = [&](int k0, int stage) {
            char* base = smem + stage * CF::STAGE;
            if constexpr (CF::A_KMAJOR) {  // A stored M x K
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)row0 * lda + k0);
#pragma unroll
                for (int q = 0; q < CF::A_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::A_INSTR_PER_WAVE + q;
                    const int r = LA::load_row(u, lane), k = LA::load_k(u, lane);
                    const bool ok = row0 + r < M && k0 + k < K;
                    load_lds<CF::VEC>(ra, base + CF::A_BASE + LA::load_lds(u),
                                      ok ? (unsigned)(r * lda + k) * 4u : OOB);
                }
            } else {  // A stored K x M
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)k0 * lda + row0);
#pragma unroll
                for (int q = 0; q < CF::A_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::A_INSTR_PER_WAVE + q;
                    const int k = LA::load_k(u, lane), c = LA::load_col(u, lane);
                    const bool ok = k0 + k < K && row0 + c < M;
                    load_lds<CF::VEC>(ra, base + CF::A_BASE + LA::load_lds(u),
                                      ok ? (unsigned)(k * lda + c) * 4u : OOB);
                }
            }
            if constexpr (CF::B_KMAJOR) {  // B stored N x K
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)col0 * ldb + k0);
#pragma unroll
                for (int q = 0; q < CF::B_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::B_INSTR_PER_WAVE + q;
                    const int r = LB::load_row(u, lane), k = LB::load_k(u, lane);
                    const bool ok = col0 + r < N && k0 + k < K;
                    load_lds<CF::VEC>(rb, base + CF::B_BASE + LB::load_lds(u),
                                      ok ? (unsigned)(r * ldb + k) * 4u : OOB);
                }
            } else {  // B stored K x N
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)k0 * ldb + col0);
#pragma unroll
                for (int q = 0; q < CF::B_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::B_INSTR_PER_WAVE + q;
                    const int k = LB::load_k(u, lane), c = LB::load_col(u, lane);
                    const bool ok = k0 + k < K && col0 + c < N;
                    load_lds<CF::VEC>(rb, base + CF::B_BASE + LB::load_lds(u),
                                      ok ? (unsigned)(k * ldb + c) * 4u : OOB);
                }
            }
        };

        v16f acc[TM][TN];
#pragma unroll
        for (int mb = 0; mb < TM; mb++)
#pragma unroll
            for (int nb = 0; nb < TN; nb++)
#pragma unroll
                for (int r = 0; r < 16; r++) acc[mb][nb][r] = 0.0f;

        const int nk = (K + CF::BK - 1) / CF::BK;
        if (nk > 0) issue(0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        for (int s = 0; s < nk; s++) {
            const char* st = smem + (s & 1) * CF::STAGE;
            // Lane (li, ls) supplies A[row][kslot(ls, u)] and B[kslot(ls, u)][col]
            // for the slab's KH steps u.
            // Fragments are read and consumed in NH parts of KH / NH steps;
            // with NH = 2 only half of them are live at a time.
            constexpr int NH = SPLIT ? 2 : 1, KP = KH / NH;
            auto read_frags = [&](int h, float (&af)[TM][KP], float (&bf)[TN][KP]) {
#pragma unroll
                for (int mb = 0; mb < TM; mb++) {
                    const int row = wm * TM * 32 + mb * 32 + li;
                    if constexpr (CF::A_KMAJOR) {
#pragma unroll
                        for (int q = 0; q < KP / 4; q++) {
                            const v4f v = *(const v4f*)(st + CF::a_elem(row, CF::kslot(ls, h * KP + 4 * q)));
#pragma unroll
                            for (int e = 0; e < 4; e++) af[mb][4 * q + e] = v[e];
                        }
                    } else {
#pragma unroll
                        for (int u = 0; u < KP; u++)
                            af[mb][u] = *(const float*)(st + CF::a_elem(row, CF::kslot(ls, h * KP + u)));
                    }
                }
#pragma unroll
                for (int nb = 0; nb < TN; nb++) {
                    const int col = wn * TN * 32 + nb * 32 + li;
                    if constexpr (CF::B_KMAJOR) {
#pragma unroll
                        for (int q = 0; q < KP / 4; q++) {
                            const v4f v = *(const v4f*)(st + CF::b_elem(CF::kslot(ls, h * KP + 4 * q), col));
#pragma unroll
                            for (int e = 0; e < 4; e++) bf[nb][4 * q + e] = v[e];
                        }
                    } else {
#pragma unroll
                        for (int u = 0; u < KP; u++)
                            bf[nb][u] = *(const float*)(st + CF::b_elem(CF::kslot(ls, h * KP + u), col));
                    }
                }
            };
            auto mfmas = [&](const float (&af)[TM][KP], const float (&bf)[TN][KP]) {
#pragma unroll
                for (int u = 0; u < KP; u++)
#pragma unroll
                    for (int mb = 0; mb < TM; mb++)
#pragma unroll
                        for (int nb = 0; nb < TN; nb++)
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[mb][u], bf[nb][u],
                                                                               acc[mb][nb], 0, 0, 0);
            };
            float af[TM][KP], bf[TN][KP];
            read_frags(0, af, bf);
            // The next slab's loads target the other stage; issue them once
            // the first reads of this stage are out.
            asm volatile("" ::: "memory");
            if (s + 1 < nk) issue((s + 1) * CF::BK, int((s + 1) & 1));
            mfmas(af, bf);
#pragma unroll
            for (int h = 1; h < NH; h++) {
                __builtin_amdgcn_sched_barrier(0);
                read_frags(h, af, bf);
                mfmas(af, bf);
            }
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
        // column L%32 of its 32 x 32 block.  C = alpha * acc (+ beta * C when
        // beta is nonzero; C is not read otherwise).
        const bool interior = row0 + CF::BM <= M && col0 + CF::BN <= N;
        const bool read_c = beta != 0.0f;
#pragma unroll
        for (int mb = 0; mb < TM; mb++)
#pragma unroll
            for (int nb = 0; nb < TN; nb++) {
                const int c = col0 + wn * TN * 32 + nb * 32 + li;
                const int rbase = row0 + wm * TM * 32 + mb * 32 + ls * 4;
                float* cp = C + (int64_t)rbase * ldc + c;
                if (interior && !read_c) {
#pragma unroll
                    for (int r = 0; r < 16; r++)
                        cp[(int64_t)((r / 4) * 8 + (r % 4)) * ldc] = alpha * acc[mb][nb][r];
                } else if (c < N) {
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const int dr = (r / 4) * 8 + (r % 4);
                        if (rbase + dr < M) {
                            float v = alpha * acc[mb][nb][r];
                            if (read_c) v = fmaf(beta, cp[(int64_t)dr * ldc], v);
                            cp[(int64_t)dr * ldc] = v;
                        }
                    }
                }
            }
    }
}

template <class CF, int OCC, bool SPLIT = false>
hipError_t launch_k4_cfg(const GemmArgs& g, hipStream_t s) {
    const int64_t tm = ceil_div(g.M, CF::BM), tn = ceil_div(g.N, CF::BN), tiles = tm * tn;
    hipLaunchKernelGGL((k4_mfma<CF, OCC, GROUP_M, true, SPLIT>), dim3(grid_for(tiles)),
                       dim3(CF::THREADS), 0, s,
                       (int)g.M, (int)g.N, (int)g.K, g.A, (int)g.lda, g.B, (int)g.ldb, g.C, g.ldc,
                       g.alpha, g.beta, (int)tm, (int)tn, (int)tiles);
    return hipGetLastError();
}

// The four storage orientations of (A, B) for one tile configuration.
template <int WM, int WN, int TM, int TN, int BK, bool V, int OCC, bool SPLIT = false>
hipError_t launch_k4_orient(const GemmArgs& g, hipStream_t s) {
    using k4::Cfg;
    if (!g.trans_a && !g.trans_b)
        return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, true, false>, OCC, SPLIT>(g, s);
    if (!g.trans_a && g.trans_b)
        return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, true, true>, OCC, SPLIT>(g, s);
    if (g.trans_a && !g.trans_b)
        return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, false, false>, OCC, SPLIT>(g, s);
    return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, false, true>, OCC, SPLIT>(g, s);
}

// Largest byte offset a slab reaches from its base, per operand orientation.
static bool offsets_fit(bool k_major, int64_t ld) {
    const int64_t lim = int64_t(OOB) - 64;
    return k_major ? ((int64_t)(MAX_BM - 1) * ld + MAX_BK) * 4 < lim
                   : ((int64_t)(MAX_BK - 1) * ld + MAX_BN) * 4 < lim;
}

bool k4_supports(const GemmArgs& g) {
    // 32-bit sizes and tile counts (with room for a tile's overhang), and
    // slab offsets inside the buffer range.
    const int64_t lim = (int64_t(1) << 31) - 1024;
    const int64_t tiles = ceil_div(g.M, 32) * ceil_div(g.N, 32);
    return g.M < lim && g.N < lim && g.K < lim && g.lda < lim && g.ldb < lim && tiles < lim &&
           offsets_fit(!g.trans_a, g.lda) && offsets_fit(g.trans_b, g.ldb);
}

static bool vec_ok(const GemmArgs& g) {
    // 16-byte loads run along each operand's contiguous dimension.
    const int64_t a_run = g.trans_a ? g.M : g.K, b_run = g.trans_b ? g.K : g.N;
    return (reinterpret_cast<uintptr_t>(g.A) % 16 == 0) &&
           (reinterpret_cast<uintptr_t>(g.B) % 16 == 0) && g.lda % 4 == 0 && g.ldb % 4 == 0 &&
           a_run % 4 == 0 && b_run % 4 == 0;
}

// Tile configurations (chosen from a sweep over square 256..8192, skinny and
// unaligned shapes on MI355X):
//  * 128 x 128 tiles, 4 waves of 2 x 2 accumulators, K slabs of 16, 4 waves
//    per SIMD: best once there are at least 1024 tiles (4 per CU), e.g.
//    square 4096 and 8192;
//  * 64 x 64 tiles, 4 waves of 1 accumulator: below that, the larger tile
//    count fills the 256 CUs (square 1024: 2.9x faster than 128 x 128);
//    K slabs of 32 with 16-byte loads (fragments read in two halves: another
//    7 % on square 1024), of 16 with 4-byte loads.
hipError_t launch_k4_tile128(const GemmArgs& g, hipStream_t s) {
    if (vec_ok(g)) return launch_k4_orient<2, 2, 2, 2, 16, true, 4>(g, s);
    return launch_k4_orient<2, 2, 2, 2, 16, false, 3>(g, s);
}

hipError_t launch_k4_tile64(const GemmArgs& g, hipStream_t s) {
    if (vec_ok(g)) return launch_k4_orient<2, 2, 1, 1, 32, true, 4, true>(g, s);
    return launch_k4_orient<2, 2, 1, 1, 16, false, 8>(g, s);
}

hipError_t launch_k4_mfma(const GemmArgs& g, hipStream_t s) {
    const int64_t tiles128 = ceil_div(g.M, 128) * ceil_div(g.N, 128);
    if (vec_ok(g) && tiles128 >= 1024) return launch_k4_orient<2, 2, 2, 2, 16, true, 4>(g, s);
    return launch_k4_tile64(g, s);
}

}  // namespace sgemm
