// Host-side exhaustive check of the matrix-core kernel's LDS layouts
// (built and run by tests/test_k4_layout.py; no GPU involved).
#include <cstdio>
#include <vector>
#include "../roofline_sgemm_f32_amd/csrc/k4_layout.h"

using namespace sgemm::k4;
static int failures = 0;
#define CHECK(cond, ...) do { if (!(cond)) { if (failures < 20) { printf(__VA_ARGS__); printf("\n"); } failures++; } } while (0)

template <class C>
void check(const char* name) {
    // A: every slab element loaded exactly once, at the byte its fragment read uses.
    std::vector<int> seenA(C::BM * C::BK, 0);
    for (int u = 0; u < C::A_INSTR; u++)
        for (int lane = 0; lane < 64; lane++)
            for (int e = 0; e < C::LSIZE / 4; e++) {
                const int r = C::a_load_row(u, lane), k = C::a_load_k(u, lane) + e;
                CHECK(r >= 0 && r < C::BM && k >= 0 && k < C::BK, "%s A load out of slab r=%d k=%d", name, r, k);
                if (r < 0 || r >= C::BM || k < 0 || k >= C::BK) continue;
                seenA[r * C::BK + k]++;
                const int lds = u * C::IB + lane * C::LSIZE + 4 * e;
                CHECK(lds < C::A_STAGE, "%s A lds out of region", name);
                CHECK(lds == C::a_frag(r, k / 4) + 4 * (k % 4), "%s A element (%d,%d) at %d, read at %d", name, r, k, lds, C::a_frag(r, k / 4) + 4 * (k % 4));
            }
    for (int i = 0; i < C::BM * C::BK; i++) CHECK(seenA[i] == 1, "%s A element %d loaded %d times", name, i, seenA[i]);
    // B likewise.
    std::vector<int> seenB(C::BK * C::BN, 0);
    for (int u = 0; u < C::B_INSTR; u++)
        for (int lane = 0; lane < 64; lane++)
            for (int e = 0; e < C::LSIZE / 4; e++) {
                const int k = C::b_load_k(u, lane), c = C::b_load_col(u, lane) + e;
                CHECK(k >= 0 && k < C::BK && c >= 0 && c < C::BN, "%s B load out of slab", name);
                if (k < 0 || k >= C::BK || c < 0 || c >= C::BN) continue;
                seenB[k * C::BN + c]++;
                const int lds = C::b_load_lds(u) + lane * C::LSIZE + 4 * e;
                CHECK(lds >= C::A_STAGE && lds + 4 <= C::STAGE, "%s B lds out of region", name);
                CHECK(lds == C::b_frag(k, c), "%s B element (%d,%d) at %d, read at %d", name, k, c, lds, C::b_frag(k, c));
            }
    for (int i = 0; i < C::BK * C::BN; i++) CHECK(seenB[i] == 1, "%s B element %d loaded %d times", name, i, seenB[i]);
    // Load instructions split over waves; each instruction's base is 16-byte aligned.
    for (int u = 0; u < C::B_INSTR; u++) CHECK(C::b_load_lds(u) % 16 == 0, "%s B base align", name);
    // k-slots cover the slab once.
    std::vector<int> seenK(C::BK, 0);
    for (int s = 0; s < 2; s++) for (int t = 0; t < C::KH; t++) seenK[C::kslot(s, t)]++;
    for (int k = 0; k < C::BK; k++) CHECK(seenK[k] == 1, "%s kslot %d", name, k);
    // Fragment reads: within the stage, and spread over 64 banks of 4 bytes.
    for (int wm = 0; wm < C::WAVES_M; wm++)
        for (int mb = 0; mb < C::TM; mb++)
            for (int q = 0; q < C::A_QUADS; q++) {
                // ds_read_b128: 16 lanes at a time must hit 16 distinct 16-byte bank groups.
                for (int g = 0; g < 4; g++) {
                    std::vector<int> slot(16, 0);
                    for (int l = 16 * g; l < 16 * g + 16; l++) {
                        const int row = wm * C::TM * 32 + mb * 32 + (l & 31);
                        const int off = C::a_frag(row, (l >> 5) * C::A_QUADS + q);
                        CHECK(off >= 0 && off + 16 <= C::A_STAGE, "%s A frag out of region", name);
                        slot[(off / 16) % 16]++;
                    }
                    for (int s = 0; s < 16; s++) CHECK(slot[s] <= 1, "%s A frag bank conflict wm=%d mb=%d q=%d g=%d", name, wm, mb, q, g);
                }
            }
    for (int wn = 0; wn < C::WAVES_N; wn++)
        for (int nb = 0; nb < C::TN; nb++)
            for (int t = 0; t < C::KH; t++) {
                std::vector<int> bank(64, 0);
                for (int l = 0; l < 64; l++) {
                    const int col = wn * C::TN * 32 + nb * 32 + (l & 31);
                    const int off = C::b_frag(C::kslot(l >> 5, t), col);
                    CHECK(off >= C::A_STAGE && off + 4 <= C::STAGE, "%s B frag out of region", name);
                    bank[(off / 4) % 64]++;
                }
                for (int b = 0; b < 64; b++) CHECK(bank[b] <= 1, "%s B frag bank conflict wn=%d nb=%d t=%d", name, wn, nb, t);
            }
    printf("%-28s BMxBN=%3dx%-3d BK=%d threads=%4d LDS=%6d A_instr/wave=%d B_instr/wave=%d\n", name,
           C::BM, C::BN, C::BK, C::THREADS, C::LDS_BYTES, C::A_INSTR_PER_WAVE, C::B_INSTR_PER_WAVE);
}

#define CFG(wm, wn, tm, tn, bk)                                                   \
    check<Cfg<wm, wn, tm, tn, bk, true>>("Cfg<" #wm "," #wn "," #tm "," #tn "," #bk ",vec>"); \
    check<Cfg<wm, wn, tm, tn, bk, false>>("Cfg<" #wm "," #wn "," #tm "," #tn "," #bk ",dword>");

int main() {
    CFG(2, 2, 2, 2, 16)
    CFG(1, 1, 1, 1, 16)
    CFG(2, 1, 1, 1, 16)
    CFG(1, 2, 1, 1, 16)
    CFG(1, 1, 1, 1, 32)
    CFG(2, 2, 1, 1, 16)
    CFG(2, 2, 2, 1, 16)
    CFG(2, 2, 1, 2, 16)
    CFG(4, 2, 2, 2, 16)
    CFG(2, 4, 2, 2, 16)
    CFG(2, 2, 2, 2, 32)
    CFG(2, 2, 1, 1, 32)
    CFG(4, 2, 2, 2, 32)
    printf("failures: %d\n", failures);
    return failures ? 1 : 0;
}
