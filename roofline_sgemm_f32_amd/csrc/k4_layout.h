// Tile geometry and LDS layouts of the matrix-core SGEMM kernel (k4_mfma.hip).
//
// Everything here is integer index arithmetic usable on the host too, so the
// layouts can be checked exhaustively on the CPU (every staged element lands
// exactly where a fragment read looks for it, nothing leaves its stage, and
// fragment reads are spread over the LDS banks).
//
// Geometry: WAVES_M x WAVES_N waves per workgroup; each wave owns TM x TN
// blocks of 32 x 32 outputs (one v_mfma_f32_32x32x2_f32 accumulator each).
// The workgroup tile is BM x BN = (WAVES_M*TM*32) x (WAVES_N*TN*32); K is
// consumed in slabs of BK.
//
// Loads (global -> LDS, direct): each load instruction moves 64 lanes x LSIZE
// bytes (16 with VEC, else 4) into a contiguous run of LDS; instruction u of a
// slab covers bytes [u*IB, (u+1)*IB) of the stage's unpadded image, IB = 64 *
// LSIZE.  The lane picks the global element that belongs at its bytes.
//
// A stage: BM rows of BK floats.  Row r's 16-byte chunks are stored permuted:
// physical chunk p holds logical chunk p ^ swz(r).  Sixteen consecutive rows
// read with one ds_read_b128 then cover all 64 banks, and any eight
// consecutive rows cover 32 distinct banks.
//
// B stage: BK rows of BN floats, stored as blocks of 1 KiB (B_RPB rows each)
// followed by a gap of B_GAP bytes.  The two halves of a wave read rows k and
// k + BK/2 in the same instruction; the gap puts them 128 bytes apart modulo
// 256, i.e. on disjoint halves of the 64 banks.
//
// MFMA operand k-slots: lane L of the 32x32x2 instruction supplies A[L%32][s]
// and B[s][L%32], s = L/32.  Slot s at step t (t < BK/2) stands for slab
// column k = s*BK/2 + t, so a lane's A values of one slab are contiguous
// (BK/8 ds_read_b128) and its B values are single floats of one column.
#pragma once
#include <hip/hip_runtime.h>

namespace sgemm {
namespace k4 {

template <int WAVES_M_, int WAVES_N_, int TM_, int TN_, int BK_, bool VEC_>
struct Cfg {
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, TM = TM_, TN = TN_, BK = BK_;
    static constexpr bool VEC = VEC_;
    static constexpr int NWAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * NWAVES;
    static constexpr int BM = WAVES_M * TM * 32, BN = WAVES_N * TN * 32;
    static constexpr int LSIZE = VEC ? 16 : 4;
    static constexpr int IB = 64 * LSIZE;
    // A stage
    static constexpr int A_ROW = BK * 4;
    static constexpr int A_CHUNKS = BK / 4;
    static constexpr int A_STAGE = BM * A_ROW;
    static constexpr int A_INSTR = A_STAGE / IB;
    // B stage
    static constexpr int B_ROW = BN * 4;
    static constexpr int B_RPB = 1024 / B_ROW;
    static constexpr int B_BLOCKS = BK / B_RPB;
    static constexpr int B_GAP = 128 * 2 * B_RPB / BK;
    static constexpr int B_BLOCK_STRIDE = 1024 + B_GAP;
    static constexpr int B_STAGE = B_BLOCKS * B_BLOCK_STRIDE;
    static constexpr int B_INSTR = BK * B_ROW / IB;
    static constexpr int STAGE = A_STAGE + B_STAGE;
    static constexpr int LDS_BYTES = 2 * STAGE;
    static constexpr int A_INSTR_PER_WAVE = A_INSTR / NWAVES;
    static constexpr int B_INSTR_PER_WAVE = B_INSTR / NWAVES;
    static constexpr int KH = BK / 2;       // MFMA steps per slab
    static constexpr int A_QUADS = BK / 8;  // ds_read_b128 per A fragment row block

    static_assert(BK == 16 || BK == 32, "slab depth");
    static_assert(B_ROW <= 1024 && 1024 % B_ROW == 0, "B rows must tile 1 KiB");
    static_assert(BK % B_RPB == 0, "B blocks");
    static_assert(B_GAP >= 16 && B_GAP % 16 == 0, "B gap keeps 16-byte alignment");
    static_assert(A_STAGE % IB == 0 && (BK * B_ROW) % IB == 0, "whole load instructions");
    static_assert(A_INSTR % NWAVES == 0 && B_INSTR % NWAVES == 0, "loads split evenly over waves");
    static_assert(1024 % IB == 0, "a load instruction stays inside one B block");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS per workgroup");

    // Logical chunk c of A row r is stored at physical chunk c ^ swz(r).
    __host__ __device__ static constexpr int swz(int r) {
        return A_CHUNKS == 4 ? (((r >> 1) & 3) ^ ((r >> 3) & 1)) : (((r >> 1) & 7) ^ ((r & 1) << 2));
    }

    // A load: instruction u (0..A_INSTR-1), lane -> the slab element (row, k)
    // of its first float; LDS byte offset is u*IB + lane*LSIZE.
    __host__ __device__ static constexpr int a_load_row(int u, int lane) {
        return (u * IB + lane * LSIZE) / A_ROW;
    }
    __host__ __device__ static constexpr int a_load_k(int u, int lane) {
        const int o = u * IB + lane * LSIZE, r = o / A_ROW, w = o % A_ROW;
        return 4 * ((w / 16) ^ swz(r)) + (w % 16) / 4;
    }
    // B load: instruction u (0..B_INSTR-1), lane -> slab element (k, col);
    // LDS byte offset (within the stage) b_load_lds(u) + lane*LSIZE.
    __host__ __device__ static constexpr int b_load_k(int u, int lane) {
        const int o = u * IB + lane * LSIZE;
        return (o / 1024) * B_RPB + (o % 1024) / B_ROW;
    }
    __host__ __device__ static constexpr int b_load_col(int u, int lane) {
        return ((u * IB + lane * LSIZE) % 1024 % B_ROW) / 4;
    }
    __host__ __device__ static constexpr int b_load_lds(int u) {
        return A_STAGE + (u * IB / 1024) * B_BLOCK_STRIDE + (u * IB) % 1024;
    }
    // Fragment reads (byte offsets within a stage).
    __host__ __device__ static constexpr int a_frag(int row, int chunk) {
        return row * A_ROW + 16 * (chunk ^ swz(row));
    }
    __host__ __device__ static constexpr int b_frag(int k, int col) {
        return A_STAGE + (k / B_RPB) * B_BLOCK_STRIDE + (k % B_RPB) * B_ROW + col * 4;
    }
    // Slab column that k-slot s stands for at MFMA step t.
    __host__ __device__ static constexpr int kslot(int s, int t) { return s * KH + t; }
};

}  // namespace k4
}  // namespace sgemm
