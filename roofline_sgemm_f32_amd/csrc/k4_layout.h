// Tile geometry and LDS layouts of the matrix-core SGEMM kernel (k4_mfma.hip).
//
// Everything here is integer index arithmetic usable on the host too, so the
// layouts can be checked exhaustively on the CPU (every staged element is
// loaded once and lands exactly where a fragment read looks for it, nothing
// leaves its stage, and fragment reads are spread over the LDS banks).
//
// Geometry: WAVES_M x WAVES_N waves per workgroup; each wave owns TM x TN
// blocks of 32 x 32 outputs (one v_mfma_f32_32x32x2_f32 accumulator each, or
// with MF16 four v_mfma_f32_16x16x4_f32 accumulators of 16 x 16).  The
// workgroup tile is BM x BN = (WAVES_M*TM*32) x (WAVES_N*TN*32); K is
// consumed in slabs of BK.
//
// Each operand tile is staged in one of two layouts, after how it is stored
// in memory:
//   KMajor  the operand's rows run along k (A as stored for C = A B, or B
//           stored transposed): ROWS rows of BK floats.  The 16-byte chunks
//           of row r are stored permuted (physical chunk p holds logical
//           chunk p ^ swz(r)), so that sixteen consecutive rows read by one
//           ds_read_b128 cover all 64 banks and any eight cover 32 distinct
//           banks.  A lane's BK/2 values of one row are contiguous.
//   KRows   the operand's rows are k (B as stored, or A stored transposed):
//           BK rows of COLS floats, written as blocks of 1 KiB (RPB rows
//           each) followed by a gap of GAP bytes.  The two halves of a wave
//           read rows k and k + BK/2 in the same instruction; the gap puts
//           them 128 bytes apart modulo 256, on disjoint halves of the 64
//           banks.  A lane reads single floats, or with WIDE eight bytes
//           (two interleaved columns, below), where the gap is doubled: an
//           8-byte read serves 32 lanes at a time, two k-slot groups of 16
//           lanes each covering 128 contiguous bytes, which the doubled gap
//           puts on disjoint halves of the banks.
//
// 16-byte reads (measured on MI355X with SQ_LDS_BANK_CONFLICT): half a wave
// is served in two passes when its lanes L and L + 16 read the same bank
// positions (address modulo 256) and its first 16 lanes 16 distinct ones, in
// four passes otherwise.  The 32 x 32 instruction's reads meet this (lanes L
// and L + 16 read rows 16 apart, or one contiguous 512-byte run); the 16 x 16
// one's do not (lanes L and L + 16 read the same row at the next k-slot),
// and its 16-byte reads of KMajor images and of four interleaved columns
// take four passes per half.  A layout that puts a row's chunks 256 bytes
// apart fixes the reads but spreads each row over lanes 16 apart in every
// load instruction, and measured no faster (square 3072 429 -> 436 us on
// 64 x 64 tiles; square 6144 within 1 % on 128 x 128).
//
// Loads (global -> LDS, direct): each load instruction moves 64 lanes x LSIZE
// bytes (16 with VEC, else 4) into a contiguous run of LDS; instruction u of
// an operand's slab covers bytes [u*IB, (u+1)*IB) of its unpadded image,
// IB = 64 * LSIZE.  The lane picks the global element that belongs at its
// bytes.
//
// MFMA operand k-slots: lane L of the 32x32x2 instruction supplies A[L%32][s]
// and B[s][L%32], s = L/32; of the 16x16x4 one A[L%16][s] and B[s][L%16],
// s = L/16.  Slot s at step t (t < KH = BK/KSLOTS) stands for slab column
// k = s*KH + t.  With four slots the KMajor swizzle still spreads the sixteen
// rows of a slot group over all 64 banks, and the KRows gap puts the four
// groups' rows on disjoint quarters of the banks (16-column runs).
//
// Columns of a wave's accumulator blocks: block nb's column j (the lane's
// L%BLK) is tile column wn*TN*32 + nb*BLK + j, except with B stored K x N
// and NB = 4 blocks (TN = 4, or TN = 2 with MF16) or MF16 with NB = 2
// (B_INTERLEAVE), where it is wn*TN*32 + NB*j + nb: the blocks interleave,
// so a lane's NB values of B of one k are 4*NB contiguous bytes of a KRows
// row (one ds_read_b128 or ds_read_b64) and its NB outputs of one row are
// 4*NB contiguous bytes of C.  (Without it, the compiler pairs the 16 x 16
// blocks' single-float reads into ds_read2_b32, whose two accesses per lane
// overlap the next k-slot group's banks: 25 % of LDS accesses conflicted.)
#pragma once
#include <hip/hip_runtime.h>

namespace sgemm {
namespace k4 {

template <int ROWS_, int BK_, bool VEC_>
struct KMajor {
    static constexpr int ROWS = ROWS_, BK = BK_;
    static constexpr bool KMAJOR = true;
    static constexpr int LSIZE = VEC_ ? 16 : 4, IB = 64 * LSIZE;
    static constexpr int ROW = BK * 4;
    static constexpr int CHUNKS = BK / 4;
    static constexpr int STAGE = ROWS * ROW;
    static constexpr int INSTR = STAGE / IB;
    static_assert(STAGE % IB == 0, "whole load instructions");

    __host__ __device__ static constexpr int swz(int r) {
        return CHUNKS == 4 ? (((r >> 1) & 3) ^ ((r >> 3) & 1)) : (((r >> 1) & 7) ^ ((r & 1) << 2));
    }
    // Load instruction u, lane -> tile element (row, k) of its first float;
    // LDS byte (within this operand's stage) load_lds(u) + lane * LSIZE.
    __host__ __device__ static constexpr int load_row(int u, int lane) { return (u * IB + lane * LSIZE) / ROW; }
    __host__ __device__ static constexpr int load_k(int u, int lane) {
        const int o = u * IB + lane * LSIZE, r = o / ROW, w = o % ROW;
        return 4 * ((w / 16) ^ swz(r)) + (w % 16) / 4;
    }
    __host__ __device__ static constexpr int load_lds(int u) { return u * IB; }
    // Byte of tile element (row, k).
    __host__ __device__ static constexpr int elem(int row, int k) {
        return row * ROW + 16 * ((k / 4) ^ swz(row)) + 4 * (k % 4);
    }
};

template <int COLS_, int BK_, bool VEC_, bool WIDE_ = false>
struct KRows {
    static constexpr int COLS = COLS_, BK = BK_;
    static constexpr bool KMAJOR = false;
    static constexpr int LSIZE = VEC_ ? 16 : 4, IB = 64 * LSIZE;
    static constexpr int ROW = COLS * 4;
    static constexpr int RPB = 1024 / ROW;
    static constexpr int BLOCKS = BK / RPB;
    static constexpr int GAP = (WIDE_ ? 2 : 1) * 128 * 2 * RPB / BK;
    static constexpr int STRIDE = 1024 + GAP;
    static constexpr int STAGE = BLOCKS * STRIDE;
    static constexpr int INSTR = BK * ROW / IB;
    static_assert(ROW <= 1024 && 1024 % ROW == 0, "rows must tile 1 KiB");
    static_assert(BK % RPB == 0, "whole blocks");
    static_assert(GAP >= 16 && GAP % 16 == 0, "gap keeps 16-byte alignment");
    static_assert((BK * ROW) % IB == 0 && 1024 % IB == 0, "whole load instructions");

    // Load instruction u, lane -> tile element (k, col) of its first float.
    __host__ __device__ static constexpr int load_k(int u, int lane) {
        const int o = u * IB + lane * LSIZE;
        return (o / 1024) * RPB + (o % 1024) / ROW;
    }
    __host__ __device__ static constexpr int load_col(int u, int lane) {
        return ((u * IB + lane * LSIZE) % 1024 % ROW) / 4;
    }
    __host__ __device__ static constexpr int load_lds(int u) {
        return (u * IB / 1024) * STRIDE + (u * IB) % 1024;
    }
    // Byte of tile element (k, col).
    __host__ __device__ static constexpr int elem(int k, int col) {
        return (k / RPB) * STRIDE + (k % RPB) * ROW + col * 4;
    }
};

template <bool C, class T, class F> struct pick { using type = T; };
template <class T, class F> struct pick<false, T, F> { using type = F; };

// A_KMAJOR: A stored M x K (k contiguous) rather than K x M.
// B_KMAJOR: B stored N x K (k contiguous) rather than K x N.
// NSTAGE: LDS stages (slabs in flight); loads run NSTAGE - 1 slabs ahead.
// MF16: the wave's 32 x 32 blocks are each computed as four 16 x 16
// accumulators of v_mfma_f32_16x16x4_f32 (four independent chains in place
// of one).
template <int WAVES_M_, int WAVES_N_, int TM_, int TN_, int BK_, bool VEC_, bool A_KMAJOR_ = true,
          bool B_KMAJOR_ = false, int NSTAGE_ = 2, bool MF16_ = false>
struct Cfg {
    static constexpr int WAVES_M = WAVES_M_, WAVES_N = WAVES_N_, TM = TM_, TN = TN_, BK = BK_;
    static constexpr bool VEC = VEC_, A_KMAJOR = A_KMAJOR_, B_KMAJOR = B_KMAJOR_;
    static constexpr int NSTAGE = NSTAGE_;
    static constexpr bool MF16 = MF16_;
    // Accumulator block edge, blocks per wave along M and N, k-slots of one
    // instruction (lane groups), and accumulator registers per lane.
    static constexpr int BLK = MF16 ? 16 : 32;
    static constexpr int MB = TM * 32 / BLK, NB = TN * 32 / BLK;
    static constexpr int KSLOTS = 64 / BLK;
    static constexpr int NREG = BLK * BLK / 64;
    static constexpr int NWAVES = WAVES_M * WAVES_N;
    static constexpr int THREADS = 64 * NWAVES;
    static constexpr int BM = WAVES_M * TM * 32, BN = WAVES_N * TN * 32;
    static constexpr bool B_INTERLEAVE = !B_KMAJOR && (MF16 ? (NB == 2 || NB == 4) : TN == 4);
    using LA = typename pick<A_KMAJOR, KMajor<BM, BK, VEC>, KRows<BM, BK, VEC>>::type;
    using LB = typename pick<B_KMAJOR, KMajor<BN, BK, VEC>,
                             KRows<BN, BK, VEC, MF16 && B_INTERLEAVE && NB == 2>>::type;
    static constexpr int A_BASE = 0, B_BASE = LA::STAGE;
    static constexpr int STAGE = LA::STAGE + LB::STAGE;
    static constexpr int LDS_BYTES = NSTAGE * STAGE;
    static constexpr int A_INSTR_PER_WAVE = LA::INSTR / NWAVES;
    static constexpr int B_INSTR_PER_WAVE = LB::INSTR / NWAVES;
    static constexpr int KH = BK / KSLOTS;  // MFMA steps per slab
    static_assert(BK == 16 || BK == 32, "slab depth");
    static_assert(NSTAGE >= 2 && NSTAGE <= 4, "stages");
    static_assert(LA::INSTR % NWAVES == 0 && LB::INSTR % NWAVES == 0, "loads split evenly over waves");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS per workgroup");

    // Slab column that k-slot s stands for at MFMA step t.
    __host__ __device__ static constexpr int kslot(int s, int t) { return s * KH + t; }
    // Tile row and column of a wave's accumulator blocks (lane index
    // j = L % BLK).
    __host__ __device__ static constexpr int a_row(int wm, int mb, int j) { return wm * TM * 32 + mb * BLK + j; }
    __host__ __device__ static constexpr int b_col(int wn, int nb, int j) {
        return B_INTERLEAVE ? wn * TN * 32 + NB * j + nb : wn * TN * 32 + nb * BLK + j;
    }
    // Row within its block of accumulator register r of a lane in k-slot
    // group s = L / BLK (its column is L % BLK).
    __host__ __device__ static constexpr int acc_row(int s, int r) {
        return MF16 ? 4 * s + r : 8 * (r / 4) + 4 * s + r % 4;
    }
    // Stage bytes of A(m, k) and B(k, n) for tile-local m, n, k.
    __host__ __device__ static constexpr int a_elem(int m, int k) {
        if constexpr (A_KMAJOR) return A_BASE + LA::elem(m, k);
        else return A_BASE + LA::elem(k, m);
    }
    __host__ __device__ static constexpr int b_elem(int k, int n) {
        if constexpr (B_KMAJOR) return B_BASE + LB::elem(n, k);
        else return B_BASE + LB::elem(k, n);
    }
};

}  // namespace k4
}  // namespace sgemm
