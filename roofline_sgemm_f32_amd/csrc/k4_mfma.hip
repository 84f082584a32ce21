// Fourth rung: the FP32 matrix-core kernel for gfx950.
//
// amittech.dev, "3.5 Project: tiled matrix multiplication", section "what
// comes next", and the closing paragraph of the qsysarch.com "gemm-kernels"
// page point at the matrix units (AMD's Matrix Fused Multiply-Add) as the
// last step of the ladder.  On CDNA4 one v_mfma_f32_32x32x2_f32 multiplies a
// 32 x 2 slice of A by a 2 x 32 slice of B into a 32 x 32 float accumulator
// held across the wave's 64 lanes (16 registers per lane), at the same FP32
// rate as the vector units' peak but from two operand registers per lane;
// v_mfma_f32_16x16x4_f32 does a 16 x 4 by 4 x 16 product into a 16 x 16
// accumulator (4 registers per lane) at the same rate, and some tile
// configurations build each 32 x 32 block from four of those.
//
// Structure (geometry and LDS layouts in k4_layout.h):
//  * a workgroup owns a BM x BN tile of C; each wave TM x TN accumulators;
//  * K is consumed in slabs of BK through NSTAGE LDS stages (2, or 3 for
//    the 32 x 32 tiles' slabs of 16) with one barrier per slab: read this slab's
//    fragments, issue the loads of the slab NSTAGE - 1 ahead, run the slab's
//    MFMAs, wait for the next slab's loads, barrier;
//  * global -> LDS uses buffer loads that write LDS directly
//    (buffer_load_dword[x4] ... lds), so staged data never occupies VGPRs;
//  * elements outside the matrix get a buffer offset past the descriptor's
//    range, which the hardware returns as zero: edge tiles and the K tail run
//    the same code; stores are masked only in edge tiles;
//  * 16-byte loads when each operand's stored rows are 16-byte aligned and
//    hold whole 4-float chunks (or are zero-padded copies from pack.hip),
//    else 4-byte loads (same LDS image either way);
//  * tile order: workgroup ids are dealt to the 8 XCDs round-robin, so ids
//    are remapped to give each XCD a contiguous range of tiles, walked in
//    groups of GROUP_M tile-rows so that resident tiles share A and B panels
//    in that XCD's L2;
//  * options for small outputs: K groups inside the workgroup (WK) and a
//    split-K mode across workgroups (SPLITK, with a second reduction kernel);
//    for the largest tiles, raised wave priority during the MFMAs (PRIO);
//  * the final C of an unsplit product is stored non-temporally.
// This file holds the kernel and one launcher per tile configuration; which
// configuration and split a product gets is decided in k4_plan.hip.
#include <algorithm>
#include <type_traits>

#include "k4_layout.h"
#include "kernels.h"

namespace sgemm {

namespace {
typedef float v2f __attribute__((ext_vector_type(2)));
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

// Wait until at most N vector-memory operations of this wave are
// outstanding.  Loads complete in issue order, so this means every load but
// the N most recent has landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// wait_vm<n * PER> for a run-time n in [0, MAXN].
template <int PER, int MAXN>
__device__ __forceinline__ void wait_vm_batches(int n) {
    if constexpr (MAXN >= 2) {
        if (n >= 2) { wait_vm<2 * PER>(); return; }
    }
    if constexpr (MAXN >= 1) {
        if (n >= 1) { wait_vm<PER>(); return; }
    }
    wait_vm<0>();
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), (short)0, (int)OOB,
                                             RSRC_WORD3);
}
}  // namespace

// SPLITK: the launch has gridDim.y K-splits; split z covers k in
// [z * kchunk, min(K, (z + 1) * kchunk)) and stores its partial product to the
// M x N slab z of the workspace passed as C (row stride ldc).
// WK: the workgroup holds WK groups of CF's waves over the same tile; group g
// takes slabs g, g + WK, g + 2 WK, ... in LDS stages of its own, and the
// groups' accumulators are added through LDS (group order) by every lane of
// the workgroup, which then stores the tile.  This shortens each wave's chain of dependent MFMAs by
// WK without scratch memory or a second launch.
// UNCHK: how a tile inside C issues the loads of whole slabs: 0 checked
// like every other slab, 1 unchecked behind a branch per slab, 2 unchecked
// in a loop of their own (the last slabs and edge tiles in a checked one).
// PIPE (with SPLIT and UNCHK = 2): in that unchecked loop, the second half's
// fragment reads and the next slab's loads are spread among the first
// MFMAs instead of waiting behind them.
// NOSYNC (K groups of one wave): no barrier per slab.  Such a wave loads
// every element of its group's stages itself and reads only those, so its
// own wait for its loads orders them before its reads, and program order
// (each read consumed before the loads NS - 1 slabs later are issued)
// orders the reads before the next loads into the same stage; the groups
// then run at their own pace until the reduction, which waits for all.
template <class CF, int OCC, int GM = GROUP_M, bool XCD_REMAP = true, bool SPLIT = false,
          bool SPLITK = false, int WK = 1, bool PRIO = false, int UNCHK = 2, bool PIPE = false,
          bool NOSYNC = false>
__global__ void __launch_bounds__(CF::THREADS * WK) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
k4_mfma(int M, int N, int K, const float* __restrict__ A, int lda, const float* __restrict__ B,
        int ldb, float* __restrict__ C, int64_t ldc, float alpha, float beta, int tiles_m,
        int tiles_n, int tiles, int kchunk) {
    // 32-bit sizes: the host routes shapes whose sizes, leading dimensions
    // or slab offsets do not fit (k4_supports) to the 64-bit kernel.
    // MB x NB accumulator blocks per wave (32 x 32, or 16 x 16 with MF16).
    constexpr int MB = CF::MB, NB = CF::NB, KH = CF::KH, NREG = CF::NREG;
    using Acc = typename std::conditional<CF::MF16, v4f, v16f>::type;
    constexpr int WG_WAVES = CF::NWAVES;  // waves of one K group
    // The K groups' partial tiles, rows padded to BN + 8 floats (WK > 1).
    constexpr int RLD = CF::BN + 8;
    constexpr int RED_BYTES = WK > 1 ? WK * CF::BM * RLD * 4 : 0;
    constexpr int LDS_TOTAL = CF::LDS_BYTES * WK > RED_BYTES ? CF::LDS_BYTES * WK : RED_BYTES;
    static_assert(WK >= 1 && WK <= 8 && CF::THREADS * WK <= 1024, "K groups");
    static_assert(LDS_TOTAL <= 160 * 1024, "LDS per workgroup");
    // OCC waves per SIMD make OCC * 4 / (waves per workgroup) resident
    // workgroups per CU, and their LDS must fit the CU's 160 KiB.
    static_assert((OCC * 4 / (CF::NWAVES * WK)) * LDS_TOTAL <= 160 * 1024,
                  "occupancy target exceeds the CU's LDS");
    if constexpr (SPLITK) {
        const int z = blockIdx.y, k0 = z * kchunk;
        K = K - k0 < kchunk ? K - k0 : kchunk;
        A += CF::A_KMAJOR ? (int64_t)k0 : (int64_t)k0 * lda;
        B += CF::B_KMAJOR ? (int64_t)k0 : (int64_t)k0 * ldb;
        C += (int64_t)z * M * ldc;
    }
    using LA = typename CF::LA;
    using LB = typename CF::LB;
    __shared__ __attribute__((aligned(1024))) char smem[LDS_TOTAL];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kg = WK > 1 ? wave_all / WG_WAVES : 0;       // K group
    const int wave = WK > 1 ? wave_all % WG_WAVES : wave_all;  // wave within the group
    const int wm = wave / CF::WAVES_N, wn = wave % CF::WAVES_N;
    const int li = CF::MF16 ? lane & 15 : lane & 31, ls = CF::MF16 ? lane >> 4 : lane >> 5;

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

        // Loads of one slab.  CHECK: elements outside the matrix get the
        // offset the buffer's range check turns into zero.  A tile wholly
        // inside C with a whole slab left in K needs no check; skipping it
        // takes about 40 scalar and vector instructions out of every slab
        // of the 128 x 256 configuration.  Measured on MI355X against the
        // checked-only kernel: square 4096 0.961 -> 0.956 ms, 8192 7.63 ->
        // 7.60, 6144 3.34 -> 3.31, 3072 0.469 -> 0.452, 3001 x 4099 x 2048
        // 0.431 -> 0.421, 768 x 1024 x 1024 18.9 -> 17.3 us; square 256 4.69
        // -> 4.85 us.  Part of these differences follows the code's
        // placement rather than the instructions removed: the checked-only
        // kernel built with its loops aligned to 64 bytes measures within
        // 0.3 % of this one on all of these shapes.
        auto issue_slab = [&](auto check, int k0, int stage) {
            constexpr bool CHECK = decltype(check)::value;
            char* base = smem + (stage * WK + kg) * CF::STAGE;
            if constexpr (CF::A_KMAJOR) {  // A stored M x K
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)row0 * lda + k0);
#pragma unroll
                for (int q = 0; q < CF::A_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::A_INSTR_PER_WAVE + q;
                    const int r = LA::load_row(u, lane), k = LA::load_k(u, lane);
                    const unsigned off = (unsigned)(r * lda + k) * 4u;
                    load_lds<CF::VEC>(ra, base + CF::A_BASE + LA::load_lds(u),
                                      !CHECK || (row0 + r < M && k0 + k < K) ? off : OOB);
                }
            } else {  // A stored K x M
                const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)k0 * lda + row0);
#pragma unroll
                for (int q = 0; q < CF::A_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::A_INSTR_PER_WAVE + q;
                    const int k = LA::load_k(u, lane), c = LA::load_col(u, lane);
                    const unsigned off = (unsigned)(k * lda + c) * 4u;
                    load_lds<CF::VEC>(ra, base + CF::A_BASE + LA::load_lds(u),
                                      !CHECK || (k0 + k < K && row0 + c < M) ? off : OOB);
                }
            }
            if constexpr (CF::B_KMAJOR) {  // B stored N x K
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)col0 * ldb + k0);
#pragma unroll
                for (int q = 0; q < CF::B_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::B_INSTR_PER_WAVE + q;
                    const int r = LB::load_row(u, lane), k = LB::load_k(u, lane);
                    const unsigned off = (unsigned)(r * ldb + k) * 4u;
                    load_lds<CF::VEC>(rb, base + CF::B_BASE + LB::load_lds(u),
                                      !CHECK || (col0 + r < N && k0 + k < K) ? off : OOB);
                }
            } else {  // B stored K x N
                const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (int64_t)k0 * ldb + col0);
#pragma unroll
                for (int q = 0; q < CF::B_INSTR_PER_WAVE; q++) {
                    const int u = wave * CF::B_INSTR_PER_WAVE + q;
                    const int k = LB::load_k(u, lane), c = LB::load_col(u, lane);
                    const unsigned off = (unsigned)(k * ldb + c) * 4u;
                    load_lds<CF::VEC>(rb, base + CF::B_BASE + LB::load_lds(u),
                                      !CHECK || (k0 + k < K && col0 + c < N) ? off : OOB);
                }
            }
        };
        const bool tile_inside = row0 + CF::BM <= M && col0 + CF::BN <= N;

        Acc acc[MB][NB];
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++)
#pragma unroll
                for (int r = 0; r < NREG; r++) acc[mb][nb][r] = 0.0f;

        // The group's s-th slab (K slab s * WK + kg) lives in stage s % NS;
        // loads run NS - 1 slabs ahead.  Every wave issues PER load
        // instructions per slab of its group.
        constexpr int NS = CF::NSTAGE;
        constexpr int PER = CF::A_INSTR_PER_WAVE + CF::B_INSTR_PER_WAVE;
        static_assert((NS - 2) * PER <= 63, "outstanding loads fit the vmcnt field");
        const int nk_all = (K + CF::BK - 1) / CF::BK;
        const int iters = (nk_all + WK - 1) / WK;                       // group 0's slab count
        const int nk = kg < nk_all ? (nk_all - kg + WK - 1) / WK : 0;   // this group's
        // The group's last slab wholly inside K, or -1: a tile inside C
        // may load its slabs up to this one unchecked.
        const int t_full = UNCHK > 0 && tile_inside && (K / CF::BK - kg - 1) >= 0
                               ? (K / CF::BK - kg - 1) / WK : -1;
#pragma unroll
        for (int p = 0; p < NS - 1; p++) {
            if (p < nk) {
                if (p <= t_full) issue_slab(std::false_type{}, (p * WK + kg) * CF::BK, p);
                else issue_slab(std::true_type{}, (p * WK + kg) * CF::BK, p);
            }
        }
        // Slab 0 landed: at most min(NS - 2, nk - 1) newer slabs outstanding.
        {
            const int newer = nk - 1 < NS - 2 ? nk - 1 : NS - 2;
            wait_vm_batches<PER, NS - 2>(newer > 0 ? newer : 0);
        }
        static_assert(!NOSYNC || CF::NWAVES == 1, "a K group of several waves shares its stages");
        if constexpr (!NOSYNC) __syncthreads();
        // One slab: its MFMAs, and the loads of the slab NS - 1 ahead
        // (checked or not, after CHECK).
        // WHOLE: the slab NS - 1 ahead exists and is whole (the unchecked loop).
        auto slab_step = [&](int s, auto check, auto whole) {
            const char* st = smem + ((s % NS) * WK + kg) * CF::STAGE;
            // Fragments are read and consumed in NH parts of KH / NH steps;
            // with NH = 2 the second part's reads are issued while the first
            // part's MFMAs run.
            constexpr int NH = SPLIT ? 2 : 1, KP = KH / NH;
            static_assert(!(CF::A_KMAJOR || CF::B_KMAJOR) || KP % 4 == 0, "16-byte fragment reads");
            auto read_frags = [&](int h, float (&af)[MB][KP], float (&bf)[NB][KP]) {
#pragma unroll
                for (int mb = 0; mb < MB; mb++) {
                    const int row = CF::a_row(wm, mb, li);
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
                if constexpr (CF::B_INTERLEAVE) {
                    // The lane's NB columns of one k: one 16- or 8-byte read.
                    using BV = typename std::conditional<NB == 4, v4f, v2f>::type;
                    static_assert(NB == 4 || NB == 2, "interleaved columns");
#pragma unroll
                    for (int u = 0; u < KP; u++) {
                        const BV v = *(const BV*)(st + CF::b_elem(CF::kslot(ls, h * KP + u), CF::b_col(wn, 0, li)));
#pragma unroll
                        for (int nb = 0; nb < NB; nb++) bf[nb][u] = v[nb];
                        // Keep 8-byte reads single: paired into ds_read2_b64,
                        // a lane's two rows would fall on the same banks.
                        if constexpr (NB == 2) asm volatile("" ::: "memory");
                    }
                } else {
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        const int col = CF::b_col(wn, nb, li);
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
                }
            };
            // The MB x NB MFMAs of step u of a half.
            auto mfma_step = [&](int u, const float (&af)[MB][KP], const float (&bf)[NB][KP]) {
#pragma unroll
                for (int mb = 0; mb < MB; mb++)
#pragma unroll
                    for (int nb = 0; nb < NB; nb++) {
                        if constexpr (CF::MF16)
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[mb][u], bf[nb][u],
                                                                               acc[mb][nb], 0, 0, 0);
                        else
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[mb][u], bf[nb][u],
                                                                               acc[mb][nb], 0, 0, 0);
                    }
            };
            auto mfmas = [&](const float (&af)[MB][KP], const float (&bf)[NB][KP]) {
#pragma unroll
                for (int u = 0; u < KP; u++) mfma_step(u, af, bf);
            };
            // LDS read instructions of one half's fragments.
            constexpr int RD = (CF::A_KMAJOR ? MB * KP / 4 : MB * KP) +
                               (CF::B_INTERLEAVE ? KP : CF::B_KMAJOR ? NB * KP / 4 : NB * KP);
            constexpr int MF = MB * NB;  // MFMAs per step
            if constexpr (PIPE && NH == 2 && decltype(whole)::value) {
                static_assert(1 + PER <= 2 * KP * MF, "loads fit between the MFMAs");
                // Both halves' fragments in registers at once.  The order
                // asked of the scheduler: the first half's reads, one MFMA,
                // the second half's reads, then the next slab's loads one
                // after each of the following MFMAs, then the rest.  The
                // second half's reads are then long done when its MFMAs
                // start, and the loads no longer delay the first MFMA.
                // Measured on MI355X against the unpipelined slab (second
                // half read after the first half's MFMAs, loads before them):
                // square 4096 940.5 -> 925.0 us, 8192 7.484 -> 7.329 ms, with
                // A stored K x M 959.8 -> 946.6 us; with every read and load
                // issued before the MFMAs, or one load per MFMA step, no gain.
                float af[MB][KP], bf[NB][KP], af1[MB][KP], bf1[NB][KP];
                if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
                read_frags(0, af, bf);
                read_frags(1, af1, bf1);
                issue_slab(check, ((s + NS - 1) * WK + kg) * CF::BK, (s + NS - 1) % NS);
                mfmas(af, bf);
                mfmas(af1, bf1);
                // Masks: 0x100 LDS reads, 0x008 MFMAs, 0x010 vector-memory
                // instructions.  One scheduling region: the priority change
                // above comes first because it would split it.
                __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
#pragma unroll
                for (int q = 0; q < PER; q++) {
                    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * KP * MF - 1 - PER, 0);
            } else if (WK == 1 || s < nk) {
                float af[MB][KP], bf[NB][KP];
                read_frags(0, af, bf);
                // The slab NS - 1 ahead goes to the stage read in the
                // previous iteration (every wave has passed that iteration's
                // barrier); issue its loads once the first reads of this
                // stage are out.
                asm volatile("" ::: "memory");
                if (s + NS - 1 < nk) {
                    const int k0 = ((s + NS - 1) * WK + kg) * CF::BK, stage = (s + NS - 1) % NS;
                    if constexpr (UNCHK == 1 && decltype(check)::value) {
                        if (s + NS - 1 <= t_full) issue_slab(std::false_type{}, k0, stage);
                        else issue_slab(std::true_type{}, k0, stage);
                    } else {
                        issue_slab(check, k0, stage);
                    }
                }
                if constexpr (PRIO) __builtin_amdgcn_s_setprio(1);
                if constexpr (NH == 2) {
                    // The second half's reads after half of the first
                    // half's MFMAs (into registers of their own): square
                    // 3072 429 -> 425 us, 2048 130.9 -> 129.7, 4608 1.465 ->
                    // 1.457 ms, 3001 x 4099 x 2047 422.5 -> 420.7 us on 64 x 64
                    // tiles; right after the first MFMA step 3001 x 4099 x
                    // 2047 took 438 us.
                    float af1[MB][KP], bf1[NB][KP];
                    mfmas(af, bf);
                    read_frags(1, af1, bf1);
                    mfmas(af1, bf1);
                    __builtin_amdgcn_sched_group_barrier(0x008, MF * KP / 2, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, MF * (2 * KP - KP / 2), 0);
                } else {
                    mfmas(af, bf);
                }
            }
            // Register-only MFMAs may otherwise be scheduled after the wait
            // and barrier below, which would expose the load latency; tie
            // the accumulators to this point.
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
#pragma unroll
                for (int nb = 0; nb < NB; nb++) asm volatile("" : "+a"(acc[mb][nb]));
            if constexpr (PRIO) __builtin_amdgcn_s_setprio(0);
            // Slab s + 1 landed: the slabs after it may stay in flight.
            const int newer = nk - 2 - s < NS - 2 ? nk - 2 - s : NS - 2;
            wait_vm_batches<PER, NS - 2>(newer > 0 ? newer : 0);
            if constexpr (!NOSYNC) __syncthreads();
        };
        // Iterations whose prefetch target is a whole slab of a tile inside
        // C skip the checks; every wave runs `iters` iterations (one barrier
        // each) whichever loop they fall in.
        int s = 0;
        if constexpr (UNCHK == 2) {
            const int s_fast = t_full - (NS - 1) + 1 < iters ? t_full - (NS - 1) + 1 : iters;
            for (; s < s_fast; s++) slab_step(s, std::false_type{}, std::true_type{});
        }
        for (; s < iters; s++) slab_step(s, std::true_type{}, std::false_type{});

        const bool read_c = beta != 0.0f;
        if constexpr (WK > 1) {
            // Every stage is free after the loop's last barrier (with NOSYNC,
            // after the one below).  Each K group
            // leaves its partial tile in LDS (a row of BN floats plus 8, so
            // the two halves of a wave's accumulator writes, four rows apart,
            // fall on disjoint banks); then every lane of the workgroup adds
            // four neighbouring outputs over the groups, in group order, and
            // stores them, 16 bytes at a time where C allows.  (Group 0 alone
            // adding and storing the tile took about 1.6 us of the 23 us of
            // square 1024.)
            constexpr int PER_LANE = CF::BM * CF::BN / (CF::THREADS * WK);
            static_assert(PER_LANE % 4 == 0 && PER_LANE * CF::THREADS * WK == CF::BM * CF::BN,
                          "whole 16-byte chunks per lane");
            if constexpr (NOSYNC) __syncthreads();  // every group past its last slab
            float* red = reinterpret_cast<float*>(smem);
#pragma unroll
            for (int mb = 0; mb < MB; mb++)
#pragma unroll
                for (int nb = 0; nb < NB; nb++)
#pragma unroll
                    for (int r = 0; r < NREG; r++) {
                        const int row = CF::MF16 ? CF::a_row(wm, mb, 0) + ls * 4 + r
                                                 : CF::a_row(wm, mb, 0) + (r / 4) * 8 + ls * 4 + r % 4;
                        const int col = CF::b_col(wn, nb, li);
                        red[(kg * CF::BM + row) * RLD + col] = acc[mb][nb][r];
                    }
            __syncthreads();
            v4f sum[PER_LANE / 4];
#pragma unroll
            for (int q = 0; q < PER_LANE / 4; q++) {
                const int o = (tid + q * CF::THREADS * WK) * 4, row = o / CF::BN, col = o % CF::BN;
                sum[q] = *(const v4f*)(red + row * RLD + col);
#pragma unroll
                for (int g = 1; g < WK; g++) sum[q] += *(const v4f*)(red + (g * CF::BM + row) * RLD + col);
            }
            // The next tile's loads reuse this memory (no next tile: no wait).
            if (t + (int)gridDim.x < tiles) __syncthreads();
            const bool vec_c = (reinterpret_cast<uintptr_t>(C) & 15) == 0 && (ldc & 3) == 0;
#pragma unroll
            for (int q = 0; q < PER_LANE / 4; q++) {
                const int o = (tid + q * CF::THREADS * WK) * 4;
                const int gr = row0 + o / CF::BN, gc = col0 + o % CF::BN;
                float* cp = C + (int64_t)gr * ldc + gc;
                if (tile_inside && !read_c && vec_c) {
                    v4f v;
#pragma unroll
                    for (int e = 0; e < 4; e++) v[e] = alpha * sum[q][e];
                    if constexpr (SPLITK) *(v4f*)cp = v;
                    else __builtin_nontemporal_store(v, (v4f*)cp);
                } else if (gr < M) {
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        if (gc + e < N) {
                            float v = alpha * sum[q][e];
                            if (read_c) v = fmaf(beta, cp[e], v);
                            cp[e] = v;
                        }
                    }
                }
            }
            continue;
        }

        // Accumulator register r of lane L holds row acc_row(L / BLK, r),
        // column L % BLK of its block.  C = alpha * acc (+ beta * C when beta
        // is nonzero; C is not read otherwise).
        const bool interior = tile_inside;
        const bool rows_aligned = (reinterpret_cast<uintptr_t>(C) & 15) == 0 && (ldc & 3) == 0;
        if constexpr (CF::B_INTERLEAVE) {
            // A lane's NB blocks hold NB neighbouring columns of each of its
            // rows: 16- or 8-byte stores (and loads of C when beta is
            // nonzero) where C allows.  Interleaved columns with 4-byte
            // stores wrote partial cache lines and cost 6 % at square 4096;
            // with these, the interleave measured square 4096 0.959 -> 0.948
            // ms, 8192 7.61 -> 7.52, 5632 2.62 -> 2.59 on MI355X (one 16-byte
            // LDS read per k step in place of two two-float reads).
            using CV = typename std::conditional<NB == 4, v4f, v2f>::type;
            if (interior && rows_aligned) {
#pragma unroll
                for (int mb = 0; mb < MB; mb++) {
                    const int rbase = row0 + CF::a_row(wm, mb, 0) + CF::acc_row(ls, 0);
                    float* cp = C + (int64_t)rbase * ldc + col0 + CF::b_col(wn, 0, li);
#pragma unroll
                    for (int r = 0; r < NREG; r++) {
                        CV* d = (CV*)(cp + (int64_t)CF::acc_row(0, r) * ldc);
                        CV v;
#pragma unroll
                        for (int nb = 0; nb < NB; nb++) v[nb] = alpha * acc[mb][nb][r];
                        if (read_c) {
                            const CV c0 = *d;
#pragma unroll
                            for (int nb = 0; nb < NB; nb++) v[nb] = fmaf(beta, c0[nb], v[nb]);
                        }
                        if constexpr (SPLITK) *d = v;
                        else __builtin_nontemporal_store(v, d);
                    }
                }
                continue;
            }
        }
#pragma unroll
        for (int mb = 0; mb < MB; mb++)
#pragma unroll
            for (int nb = 0; nb < NB; nb++) {
                const int c = col0 + CF::b_col(wn, nb, li);
                const int rbase = row0 + CF::a_row(wm, mb, 0) + CF::acc_row(ls, 0);
                float* cp = C + (int64_t)rbase * ldc + c;
                if (interior && !read_c) {
                    // The final C goes out with non-temporal stores (0.1-0.8 %
                    // faster on unsplit products); split partial tiles, which
                    // the reduction reads right back, keep the default policy,
                    // and so do rows that are not 16-byte aligned: their
                    // single-float stores then merge into whole lines in the
                    // L2 (3001 x 4099 x 2047: 52 MB written per product, C
                    // being 49 MB, against 128 MB non-temporal; 420 -> 418 us).
#pragma unroll
                    for (int r = 0; r < NREG; r++) {
                        float* d = cp + (int64_t)(CF::acc_row(0, r)) * ldc;
                        if (SPLITK || !rows_aligned) *d = alpha * acc[mb][nb][r];
                        else __builtin_nontemporal_store(alpha * acc[mb][nb][r], d);
                    }
                } else if (c < N) {
#pragma unroll
                    for (int r = 0; r < NREG; r++) {
                        const int dr = CF::acc_row(0, r);
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

template <class CF, int OCC, bool SPLIT = false, int WK = 1, bool PRIO = false, int UNCHK = 2,
          bool PIPE = false, bool NOSYNC = false>
hipError_t launch_k4_cfg(const GemmArgs& g, hipStream_t s) {
    const int64_t tm = ceil_div(g.M, CF::BM), tn = ceil_div(g.N, CF::BN), tiles = tm * tn;
    hipLaunchKernelGGL((k4_mfma<CF, OCC, GROUP_M, true, SPLIT, false, WK, PRIO, UNCHK, PIPE, NOSYNC>), dim3(grid_for(tiles)),
                       dim3(CF::THREADS * WK), 0, s,
                       (int)g.M, (int)g.N, (int)g.K, g.A, (int)g.lda, g.B, (int)g.ldb, g.C, g.ldc,
                       g.alpha, g.beta, (int)tm, (int)tn, (int)tiles, 0);
    return hipGetLastError();
}

// Split-K second pass: C = alpha * (sum of the S partial slabs, added in
// split order) (+ beta * C when beta is nonzero), the same two roundings the
// unsplit epilogue applies.  Each lane takes four consecutive columns.  W
// holds S slabs of M rows of ldw floats; VW (ldw a multiple of 4, W 16-byte
// aligned) reads a lane's four partial columns as one 16-byte access, also
// past N into a row's padding, whose sums are dropped; VC (N and ldc
// multiples of 4, C 16-byte aligned) moves C the same way.
template <bool VW, bool VC>
__global__ void __launch_bounds__(64)
splitk_reduce(int M, int N, int S, const float* __restrict__ W, int64_t ldw, float* __restrict__ C,
              int64_t ldc, float alpha, float beta) {
    const int nq = (N + 3) / 4;
    const int64_t total = (int64_t)M * nq, slab = (int64_t)M * ldw;
    const bool read_c = beta != 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int r = (int)(i / nq), c = (int)(i % nq) * 4;
        const float* w = W + (int64_t)r * ldw + c;
        float* cp = C + (int64_t)r * ldc + c;
        if constexpr (VW) {
            v4f sum = *(const v4f*)w;
            // Four slabs' loads in flight per step: 8 or 16 measured slower
            // on small outputs (128^2 x 4096, 16 slabs: 9.35 us per product
            // against 10.0 and 11.9), 2 no faster.
#pragma unroll 4
            for (int z = 1; z < S; z++) sum += *(const v4f*)(w + z * slab);
            v4f v;
#pragma unroll
            for (int e = 0; e < 4; e++) v[e] = alpha * sum[e];
            if constexpr (VC) {
                if (read_c) {
                    const v4f c0 = *(const v4f*)cp;
#pragma unroll
                    for (int e = 0; e < 4; e++) v[e] = fmaf(beta, c0[e], v[e]);
                }
                *(v4f*)cp = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (c + e >= N) break;
                    cp[e] = read_c ? fmaf(beta, cp[e], v[e]) : v[e];
                }
            }
        } else {
            for (int e = 0; e < 4 && c + e < N; e++) {
                float sum = w[e];
#pragma unroll 8
                for (int z = 1; z < S; z++) sum += w[z * slab + e];
                float v = alpha * sum;
                if (read_c) v = fmaf(beta, cp[e], v);
                cp[e] = v;
            }
        }
    }
}

hipError_t launch_splitk_reduce(const GemmArgs& g, int splits, const float* ws, int64_t ldw,
                                hipStream_t s) {
    const int64_t total = g.M * ceil_div(g.N, 4);
    const bool vw = ldw % 4 == 0 && reinterpret_cast<uintptr_t>(ws) % 16 == 0;
    const bool vc = g.N % 4 == 0 && g.ldc % 4 == 0 && reinterpret_cast<uintptr_t>(g.C) % 16 == 0;
    // One-wave workgroups: the partial slabs are few and small, so spread
    // them over as many CUs as possible.
    const dim3 grid(grid_for(ceil_div(total, 64)));
    if (vw && vc)
        hipLaunchKernelGGL((splitk_reduce<true, true>), grid, dim3(64), 0, s, (int)g.M, (int)g.N, splits,
                           ws, ldw, g.C, g.ldc, g.alpha, g.beta);
    else if (vw)
        hipLaunchKernelGGL((splitk_reduce<true, false>), grid, dim3(64), 0, s, (int)g.M, (int)g.N, splits,
                           ws, ldw, g.C, g.ldc, g.alpha, g.beta);
    else
        hipLaunchKernelGGL((splitk_reduce<false, false>), grid, dim3(64), 0, s, (int)g.M, (int)g.N, splits,
                           ws, ldw, g.C, g.ldc, g.alpha, g.beta);
    return hipGetLastError();
}

// K split into `splits` chunks of kchunk (a multiple of BK; every chunk
// nonempty): partial products into ws (splits slabs of M rows of
// split_ld(N) floats), then the reduction into C.
template <class CF, int OCC, bool SPLIT = false, int WK = 1, int UNCHK = 2, bool PIPE = false,
          bool NOSYNC = false>
hipError_t launch_k4_cfg_splitk(const GemmArgs& g, int splits, int kchunk, float* ws, hipStream_t s) {
    const int64_t tm = ceil_div(g.M, CF::BM), tn = ceil_div(g.N, CF::BN), tiles = tm * tn;
    const int64_t ldw = split_ld(g.N);
    hipLaunchKernelGGL((k4_mfma<CF, OCC, GROUP_M, true, SPLIT, true, WK, false, UNCHK, PIPE, NOSYNC>), dim3(grid_for(tiles), splits),
                       dim3(CF::THREADS * WK), 0, s,
                       (int)g.M, (int)g.N, (int)g.K, g.A, (int)g.lda, g.B, (int)g.ldb, ws, ldw,
                       1.0f, 0.0f, (int)tm, (int)tn, (int)tiles, kchunk);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_splitk_reduce(g, splits, ws, ldw, s);
}

// The four storage orientations of (A, B) for one tile configuration; with
// splits > 1 (and CAN_SPLIT) the split-K pair of launches.
// OCC_TN: the occupancy target for A stored K x M with B stored K x N.
// Both operands then take the KRows layout, whose stages are larger: in the
// three-stage 32 x 32 configuration with K slabs of 16 a workgroup needs
// 55,296 B of LDS (52,224 B with A stored M x K), so three workgroups would
// need 165,888 B, more than the CU's 160 KiB, and the target drops to 2.
template <int WM, int WN, int TM, int TN, int BK, bool V, int OCC, bool SPLIT = false, int NS = 2,
          int WK = 1, bool CAN_SPLIT = true, int OCC_TN = OCC, int UNCHK = 2, bool MF16 = false,
          bool PIPE = false, bool NOSYNC = false>
hipError_t launch_k4_orient(const GemmArgs& g, hipStream_t s, int splits = 1, int kchunk = 0,
                            float* ws = nullptr) {
    using k4::Cfg;
    if constexpr (CAN_SPLIT) {
        if (splits > 1) {
            if (!g.trans_a && !g.trans_b)
                return launch_k4_cfg_splitk<Cfg<WM, WN, TM, TN, BK, V, true, false, NS, MF16>, OCC, SPLIT, WK, UNCHK, PIPE, NOSYNC>(g, splits, kchunk, ws, s);
            if (!g.trans_a && g.trans_b)
                return launch_k4_cfg_splitk<Cfg<WM, WN, TM, TN, BK, V, true, true, NS, MF16>, OCC, SPLIT, WK, UNCHK, PIPE, NOSYNC>(g, splits, kchunk, ws, s);
            if (g.trans_a && !g.trans_b)
                return launch_k4_cfg_splitk<Cfg<WM, WN, TM, TN, BK, V, false, false, NS, MF16>, OCC_TN, SPLIT, WK, UNCHK, PIPE, NOSYNC>(g, splits, kchunk, ws, s);
            return launch_k4_cfg_splitk<Cfg<WM, WN, TM, TN, BK, V, false, true, NS, MF16>, OCC, SPLIT, WK, UNCHK, PIPE, NOSYNC>(g, splits, kchunk, ws, s);
        }
    }
    if (!g.trans_a && !g.trans_b)
        return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, true, false, NS, MF16>, OCC, SPLIT, WK, false, UNCHK, PIPE, NOSYNC>(g, s);
    if (!g.trans_a && g.trans_b)
        return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, true, true, NS, MF16>, OCC, SPLIT, WK, false, UNCHK, PIPE, NOSYNC>(g, s);
    if (g.trans_a && !g.trans_b)
        return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, false, false, NS, MF16>, OCC_TN, SPLIT, WK, false, UNCHK, PIPE, NOSYNC>(g, s);
    return launch_k4_cfg<Cfg<WM, WN, TM, TN, BK, V, false, true, NS, MF16>, OCC, SPLIT, WK, false, UNCHK, PIPE, NOSYNC>(g, s);
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

// Whether an operand's rows suit 16-byte loads along its run (the stored
// row length): aligned rows, and a run in whole 4-float chunks.
bool rows_vec(const float* p, int64_t ld, int64_t run) {
    return reinterpret_cast<uintptr_t>(p) % 16 == 0 && ld % 4 == 0 && run % 4 == 0;
}

bool vec_ok(const GemmArgs& g) {
    // 16-byte loads run along each operand's contiguous dimension; with
    // padded runs a chunk may straddle the run's end into the zero padding.
    const int64_t a_run = g.trans_a ? g.M : g.K, b_run = g.trans_b ? g.K : g.N;
    const int64_t ra = g.runs_padded ? packed_ld(a_run) : a_run;
    const int64_t rb = g.runs_padded ? packed_ld(b_run) : b_run;
    return rows_vec(g.A, g.lda, ra) && rows_vec(g.B, g.ldb, rb);
}

hipError_t launch_k4_tile128x256(const GemmArgs& g, hipStream_t s) {
    using k4::Cfg;
    // Raised wave priority with the pipelined slab: with A stored K x M it
    // costs 1 % (952 -> 942 us without it) and is off.  As stored it costs
    // 0.3 % (square 4096 929 against 926 us, 8192 7.346 against 7.316 ms) but
    // keeps the two workgroups of a CU in step: without it the L2 misses of
    // square 4096 rise from 388 to 600 MB per launch (FETCH_SIZE), re-reads
    // the Infinity Cache absorbs there and HBM would not at larger sizes.
    // With B stored N x K it is 1.3 % faster (933 against 945 us).
    if (vec_ok(g)) {
        if (!g.trans_a && !g.trans_b) return launch_k4_cfg<Cfg<2, 2, 2, 4, 16, true, true, false>, 2, true, 1, true, 2, true>(g, s);
        if (!g.trans_a) return launch_k4_cfg<Cfg<2, 2, 2, 4, 16, true, true, true>, 2, true, 1, true, 2, true>(g, s);
        if (!g.trans_b) return launch_k4_cfg<Cfg<2, 2, 2, 4, 16, true, false, false>, 2, true, 1, false, 2, true>(g, s);
        return launch_k4_cfg<Cfg<2, 2, 2, 4, 16, true, false, true>, 2, true, 1, true, 2, true>(g, s);
    }
    if (g.trans_a || g.trans_b) return launch_k4_tile128(g, s);
    return launch_k4_cfg<Cfg<2, 2, 2, 4, 16, false>, 2, true, 1, true>(g, s);
}

// The 128 x 128 and 64 x 64 tiles with 16-byte loads run on the 16 x 16 x 4
// instruction: each 32 x 32 block becomes four independent accumulator
// chains.  Measured on MI355X against the 32 x 32 x 2 kernel (integer
// operands bit-identical in all four orientations): 128 x 128 tiles square
// 6144 3.306 -> 3.256 ms, 7168^2 x 1024 0.863 -> 0.846; 64 x 64 tiles
// 3001 x 4099 x 2047 428 -> 421 us, square 3072 450 -> 438, 1536 x 1024 x
// 1024 36.0 -> 34.8, 1280^3 47.3 -> 46.8.  It does not help the K-group
// tiles (square 1024 21.80 against 21.77 us, 1024^2 x 4096 73.4 against
// 73.2), costs 32 x 32 tiles 3-6 % (640^3 9.16 -> 9.69 us) and spills
// registers in the 128 x 256 tile (square 4096 0.942 -> 0.960 ms).
hipError_t launch_k4_tile128(const GemmArgs& g, hipStream_t s) {
    if (vec_ok(g)) return launch_k4_orient<2, 2, 2, 2, 16, true, 4, false, 2, 1, false, 4, 2, true>(g, s);
    return launch_k4_orient<2, 2, 2, 2, 16, false, 3, false, 2, 1, false>(g, s);
}

// The pipelined slab (PIPE) measured slower here: 3001 x 4099 x 2047 423 ->
// 444 us, square 3072 440 -> 443.
hipError_t launch_k4_t64(const GemmArgs& g, hipStream_t s, int splits, int kchunk, float* ws) {
    if (vec_ok(g)) return launch_k4_orient<2, 2, 1, 1, 32, true, 4, true, 2, 1, true, 4, 2, true>(g, s, splits, kchunk, ws);
    return launch_k4_orient<2, 2, 1, 1, 16, false, 8>(g, s, splits, kchunk, ws);
}

hipError_t launch_k4_tile64(const GemmArgs& g, hipStream_t s) { return launch_k4_t64(g, s, 1, 0, nullptr); }

hipError_t launch_k4_t32_wk4(const GemmArgs& g, hipStream_t s, int splits, int kchunk,
                                    float* ws) {
    // Occupancy targets as the LDS allows them (3, 2 and 4 workgroups per
    // CU; a target of 2 for the three-stage slabs of 16 held 768 x 1024 x
    // 1024, 768 tiles, at 21.3 us against 18.7 with 3).
    // With 16-byte loads, K slabs of 16 in three stages (two slabs in
    // flight) when a K group's share is short or two workgroups share each
    // CU: 3-11 % faster than slabs of 32 in two stages on 17 such outputs
    // (square 256 5.07 -> 4.75 us, 320^3 5.79 -> 5.14, 256^2 x 16384 32.0
    // -> 31.1, 512 x 256 x 8192 29.9 -> 28.5); alone on a CU with long
    // shares the extra barriers cost more (64^2 x 65536 22.8 -> 25.3), and
    // 64 x 64 tiles lose 5-15 % with it.
    // Both take the pipelined slab (PIPE): square 256 4.58 -> 4.37 us, 512
    // 6.50 -> 6.02, 640 9.27 -> 8.73, 768 x 1024 x 1024 17.6 -> 16.0,
    // 128^2 x 4096 9.10 -> 8.94.  And no barrier per slab (NOSYNC), except
    // with slabs of 16 and long shares: square 256 4.41 -> 4.18, 512 5.82 ->
    // 5.63, 640 8.72 -> 8.43, 256^2 x 4096 12.6 -> 12.2, 64^2 x 65536 23.1 ->
    // 20.9; with slabs of 16 and shares of 512 it cost 256^2 x 16384 7 %
    // (27.0 -> 28.8 us; groups that drift apart no longer share the 128-byte
    // lines of A that their 64-byte slab rows split).  4-byte loads:
    // NOSYNC too (255^3 6.46 -> 6.27 us, 300 x 1000 x 901 19.3 -> 18.1,
    // 1023 x 1027 x 1024 36.4 -> 35.3, 700 x 901 x 1500 35.6 -> 33.5).
    if (vec_ok(g)) {
        const int64_t share = (splits > 1 ? kchunk : g.K) / 4;
        const int64_t wgs = ceil_div(g.M, 32) * ceil_div(g.N, 32) * (splits > 1 ? splits : 1);
        // More than three per CU: slabs of 16 in two stages, four per CU.
        if (wgs > 3 * 256)
            return launch_k4_orient<1, 1, 1, 1, 16, true, 4, true, 2, 4, true, 4, 2, false, true, true>(g, s, splits, kchunk, ws);
        if (share <= 256)
            return launch_k4_orient<1, 1, 1, 1, 16, true, 3, true, 3, 4, true, 2, 2, false, true, true>(g, s, splits, kchunk, ws);
        if (wgs >= 2 * 256)
            return launch_k4_orient<1, 1, 1, 1, 16, true, 3, true, 3, 4, true, 2, 2, false, true>(g, s, splits, kchunk, ws);
        return launch_k4_orient<1, 1, 1, 1, 32, true, 2, true, 2, 4, true, 2, 2, false, true, true>(g, s, splits, kchunk, ws);
    }
    return launch_k4_orient<1, 1, 1, 1, 16, false, 4, false, 2, 4, true, 4, 2, false, false, true>(g, s, splits, kchunk, ws);
}

// 16-byte loads only (the plan never picks it otherwise: with 4-byte loads
// 64 x 64 tiles with K groups measured slower than 32 x 32 ones).  The
// pipelined slab (PIPE): square 1024 22.2 -> 21.0 us, 1024^2 x 4096 73.7 ->
// 69.1, 896^3 19.7 -> 19.0.
hipError_t launch_k4_t64_wk4(const GemmArgs& g, hipStream_t s, int splits, int kchunk,
                                    float* ws) {
    if (vec_ok(g)) return launch_k4_orient<2, 2, 1, 1, 32, true, 4, true, 2, 4, true, 4, 2, false, true>(g, s, splits, kchunk, ws);
    return launch_k4_t32_wk4(g, s, splits, kchunk, ws);
}

}  // namespace sgemm
