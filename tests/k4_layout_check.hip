// Host-side exhaustive check of the matrix-core kernel's LDS layouts
// (built and run by tests/test_k4_layout.py; no GPU involved).
#include <cstdio>
#include <vector>
#include "../roofline_sgemm_f32_amd/csrc/k4_layout.h"

using namespace sgemm::k4;
static int failures = 0;
#define CHECK(cond, ...) do { if (!(cond)) { if (failures < 20) { printf(__VA_ARGS__); printf("\n"); } failures++; } } while (0)

// One operand: its load instructions put every tile element (major, k) into
// the LDS byte that elem() names, exactly once, inside [0, STAGE).
template <class L>
void check_operand(const char* name, int major_extent) {
    std::vector<int> seen(major_extent * L::BK, 0);
    for (int u = 0; u < L::INSTR; u++) {
        CHECK(L::load_lds(u) % 16 == 0, "%s load base align", name);
        for (int lane = 0; lane < 64; lane++)
            for (int e = 0; e < L::LSIZE / 4; e++) {
                int mj, k, at;
                if constexpr (L::KMAJOR) {
                    mj = L::load_row(u, lane); k = L::load_k(u, lane) + e;
                    at = L::elem(mj, k);
                } else {
                    k = L::load_k(u, lane); mj = L::load_col(u, lane) + e;
                    at = L::elem(k, mj);
                }
                CHECK(mj >= 0 && mj < major_extent && k >= 0 && k < L::BK, "%s load outside tile (%d,%d)", name, mj, k);
                if (mj < 0 || mj >= major_extent || k < 0 || k >= L::BK) continue;
                seen[mj * L::BK + k]++;
                const int lds = L::load_lds(u) + lane * L::LSIZE + 4 * e;
                CHECK(lds >= 0 && lds + 4 <= L::STAGE, "%s lds outside stage", name);
                CHECK(lds == at, "%s element (%d,%d) loaded to %d, read at %d", name, mj, k, lds, at);
            }
    }
    for (size_t i = 0; i < seen.size(); i++) CHECK(seen[i] == 1, "%s element %zu loaded %d times", name, i, seen[i]);
}

// Bank model of one LDS read instruction of a wave, from measurements on
// MI355X (SQ_LDS_BANK_CONFLICT over SQ_LDS_IDX_ACTIVE, 64 banks of 4 bytes):
//  * 4 bytes per lane: all 64 lanes at once, on distinct banks;
//  * 8 bytes: 32 consecutive lanes at a time, on distinct banks;
//  * 16 bytes: half a wave in two passes, which needs the half's first 16
//    lanes on 16 distinct 16-byte bank positions (address / 16 mod 16) and
//    lane L + 16 on the same position as lane L (four 256-byte runs of 16
//    lanes take 4 cycles when congruent modulo 256, 6 when one is shifted or
//    permuted, 8 when both halves differ).
// Returns whether the read is conflict-free.
static bool read_ok(const int (&off)[64], int width) {
    if (width == 4 || width == 8) {
        const int per = 256 / width;
        for (int g = 0; g < 64 / per; g++) {
            std::vector<int> bank(64, 0);
            for (int l = per * g; l < per * (g + 1); l++)
                for (int e = 0; e < width / 4; e++) bank[(off[l] / 4 + e) % 64]++;
            for (int b = 0; b < 64; b++) if (bank[b] > 1) return false;
        }
        return true;
    }
    for (int h = 0; h < 2; h++) {
        std::vector<int> pos(16, 0);
        for (int i = 0; i < 16; i++) {
            const int l = 32 * h + i;
            pos[(off[l] / 16) % 16]++;
            if ((off[l] / 16) % 16 != (off[l + 16] / 16) % 16) return false;
        }
        for (int q = 0; q < 16; q++) if (pos[q] != 1) return false;
    }
    return true;
}

// Fragment reads of one operand by one wave: lane l reads
// (major = base + l % BLK, k = kslot(l / BLK, t)).  KMajor: ds_read_b128 of
// four consecutive k per 4 steps; KRows: ds_read_b32 per step, or with
// interleaved columns one read of the NB blocks' columns per step.
template <class CF, bool IS_A>
void check_frags(const char* name) {
    constexpr bool KM = IS_A ? CF::A_KMAJOR : CF::B_KMAJOR;
    constexpr int WAVES = IS_A ? CF::WAVES_M : CF::WAVES_N, T = IS_A ? CF::MB : CF::NB;
    for (int w = 0; w < WAVES; w++)
        for (int blk = 0; blk < T; blk++) {
            auto major = [&](int l) {
                return IS_A ? CF::a_row(w, blk, l % CF::BLK) : CF::b_col(w, blk, l % CF::BLK);
            };
            int off[64];
            if constexpr (!IS_A && CF::B_INTERLEAVE) {
                // One read per k step covers the lane's NB blocks: 4 NB
                // bytes, aligned and contiguous.
                if (blk != 0) continue;
                constexpr int W = 4 * CF::NB;
                for (int t = 0; t < CF::KH; t++) {
                    for (int l = 0; l < 64; l++) {
                        const int k = CF::kslot(l / CF::BLK, t);
                        off[l] = CF::b_elem(k, CF::b_col(w, 0, l % CF::BLK));
                        CHECK(off[l] % W == 0, "%s interleaved read misaligned", name);
                        for (int e = 1; e < CF::NB; e++)
                            CHECK(CF::b_elem(k, CF::b_col(w, e, l % CF::BLK)) == off[l] + 4 * e,
                                  "%s interleaved read not contiguous", name);
                    }
                    // Four interleaved columns under the 16 x 16 instruction:
                    // the same known cost.
                    if (CF::MF16 && W == 16) {
                        CHECK(!read_ok(off, W), "%s expected the known 16-byte read conflict", name);
                        continue;
                    }
                    CHECK(read_ok(off, W), "%s interleaved read bank conflict w=%d t=%d", name, w, t);
                }
            } else if constexpr (KM) {
                for (int q = 0; q < CF::KH / 4; q++) {
                    for (int l = 0; l < 64; l++) {
                        const int mj = major(l), k = CF::kslot(l / CF::BLK, 4 * q);
                        off[l] = IS_A ? CF::a_elem(mj, k) : CF::b_elem(k, mj);
                        CHECK(off[l] % 16 == 0, "%s frag b128 misaligned", name);
                        // the 4 values of the read are k..k+3
                        for (int e = 1; e < 4; e++) {
                            const int o2 = IS_A ? CF::a_elem(mj, k + e) : CF::b_elem(k + e, mj);
                            CHECK(o2 == off[l] + 4 * e, "%s frag b128 not contiguous", name);
                        }
                    }
                    // The 16 x 16 instruction's 16-byte reads of KMajor
                    // images take four passes per half wave, a known cost
                    // (see k4_layout.h) the layout accepts for coalesced loads.
                    if (CF::MF16) {
                        CHECK(!read_ok(off, 16), "%s expected the known 16-byte read conflict", name);
                        continue;
                    }
                    CHECK(read_ok(off, 16), "%s b128 bank conflict w=%d blk=%d q=%d", name, w, blk, q);
                }
            } else {
                for (int t = 0; t < CF::KH; t++) {
                    for (int l = 0; l < 64; l++) {
                        const int mj = major(l), k = CF::kslot(l / CF::BLK, t);
                        off[l] = IS_A ? CF::a_elem(mj, k) : CF::b_elem(k, mj);
                    }
                    CHECK(read_ok(off, 4), "%s b32 bank conflict w=%d blk=%d t=%d", name, w, blk, t);
                }
            }
        }
}

template <class CF>
void check(const char* name) {
    const int failures_before = failures;
    check_operand<typename CF::LA>(name, CF::BM);
    check_operand<typename CF::LB>(name, CF::BN);
    // A and B stages do not overlap; both stages fit the allocation.
    CHECK(CF::B_BASE >= CF::LA::STAGE && CF::B_BASE + CF::LB::STAGE == CF::STAGE, "%s stage split", name);
    std::vector<int> seenK(CF::BK, 0);
    for (int s = 0; s < CF::KSLOTS; s++) for (int t = 0; t < CF::KH; t++) seenK[CF::kslot(s, t)]++;
    for (int k = 0; k < CF::BK; k++) CHECK(seenK[k] == 1, "%s kslot %d", name, k);
    check_frags<CF, true>(name);
    check_frags<CF, false>(name);
    // Each wave's accumulator blocks cover its rows and columns exactly once.
    for (int w = 0; w < CF::WAVES_M; w++) {
        std::vector<int> seen(CF::TM * 32, 0);
        for (int mb = 0; mb < CF::MB; mb++)
            for (int j = 0; j < CF::BLK; j++) seen[CF::a_row(w, mb, j) - w * CF::TM * 32]++;
        for (int r = 0; r < CF::TM * 32; r++) CHECK(seen[r] == 1, "%s row map w=%d r=%d", name, w, r);
    }
    for (int w = 0; w < CF::WAVES_N; w++) {
        std::vector<int> seen(CF::TN * 32, 0);
        for (int nb = 0; nb < CF::NB; nb++)
            for (int j = 0; j < CF::BLK; j++) seen[CF::b_col(w, nb, j) - w * CF::TN * 32]++;
        for (int c = 0; c < CF::TN * 32; c++) CHECK(seen[c] == 1, "%s column map w=%d c=%d", name, w, c);
    }
    // The accumulator registers of a block's 64 lanes (row acc_row(l / BLK,
    // r), column l % BLK) hold each of its BLK x BLK outputs once.
    {
        std::vector<int> seen(CF::BLK * CF::BLK, 0);
        for (int l = 0; l < 64; l++)
            for (int r = 0; r < CF::NREG; r++) {
                const int row = CF::acc_row(l / CF::BLK, r);
                CHECK(row >= 0 && row < CF::BLK, "%s accumulator row %d", name, row);
                if (row >= 0 && row < CF::BLK) seen[row * CF::BLK + l % CF::BLK]++;
            }
        for (int i = 0; i < CF::BLK * CF::BLK; i++) CHECK(seen[i] == 1, "%s accumulator element %d", name, i);
    }
    printf("%-39s BMxBN=%3dx%-3d BK=%d threads=%4d LDS=%6d A_instr/wave=%d B_instr/wave=%d%s\n", name,
           CF::BM, CF::BN, CF::BK, CF::THREADS, CF::LDS_BYTES, CF::A_INSTR_PER_WAVE, CF::B_INSTR_PER_WAVE,
           failures > failures_before ? "  FAILED" : "");
}

#define CFG1(wm, wn, tm, tn, bk, v, ak, bk2) \
    check<Cfg<wm, wn, tm, tn, bk, v, ak, bk2>>("Cfg<" #wm "," #wn "," #tm "," #tn "," #bk "," #v "," #ak "," #bk2 ">");
#define CFG(wm, wn, tm, tn, bk)                                                                   \
    CFG1(wm, wn, tm, tn, bk, true, true, false) CFG1(wm, wn, tm, tn, bk, false, true, false)     \
    CFG1(wm, wn, tm, tn, bk, true, true, true) CFG1(wm, wn, tm, tn, bk, false, true, true)       \
    CFG1(wm, wn, tm, tn, bk, true, false, false) CFG1(wm, wn, tm, tn, bk, false, false, false)   \
    CFG1(wm, wn, tm, tn, bk, true, false, true) CFG1(wm, wn, tm, tn, bk, false, false, true)

// The same with the 16 x 16 x 4 instruction (four k-slot lane groups).
#define CFG1M(wm, wn, tm, tn, bk, v, ak, bk2) \
    check<Cfg<wm, wn, tm, tn, bk, v, ak, bk2, 2, true>>("Cfg<" #wm "," #wn "," #tm "," #tn "," #bk "," #v "," #ak "," #bk2 ",MF16>");
#define CFGM(wm, wn, tm, tn, bk)                                                                    \
    CFG1M(wm, wn, tm, tn, bk, true, true, false) CFG1M(wm, wn, tm, tn, bk, false, true, false)     \
    CFG1M(wm, wn, tm, tn, bk, true, true, true) CFG1M(wm, wn, tm, tn, bk, false, true, true)       \
    CFG1M(wm, wn, tm, tn, bk, true, false, false) CFG1M(wm, wn, tm, tn, bk, false, false, false)   \
    CFG1M(wm, wn, tm, tn, bk, true, false, true) CFG1M(wm, wn, tm, tn, bk, false, false, true)

int main() {
    CFG(2, 2, 2, 2, 16)
    CFG(2, 2, 1, 1, 16)
    CFG(2, 2, 1, 1, 32)
    CFG(2, 2, 2, 1, 16)
    CFG(2, 2, 1, 2, 16)
    CFG(4, 2, 2, 2, 16)
    CFG(2, 4, 2, 2, 16)
    CFG(2, 2, 2, 2, 32)
    CFG(1, 1, 1, 1, 16)
    CFG(2, 1, 1, 1, 16)
    CFG(1, 2, 1, 1, 16)
    CFG(4, 2, 1, 2, 16)
    CFG(2, 4, 2, 1, 16)
    CFG(4, 2, 1, 2, 32)
    CFG(2, 2, 2, 4, 16)
    CFG(1, 1, 1, 1, 32)
    CFGM(2, 2, 2, 2, 16)
    CFGM(2, 2, 1, 1, 16)
    CFGM(2, 2, 1, 1, 32)
    // (32 x 32 tiles with slabs of 16 are left out: there the 32-column
    // KRows image puts k-slot groups 0 and 1 on the same banks, a two-way
    // conflict on every b32 read; no launcher builds that configuration.)
    CFGM(1, 1, 1, 1, 32)
    CFGM(2, 2, 2, 4, 16)
    printf("failures: %d\n", failures);
    return failures ? 1 : 0;
}
