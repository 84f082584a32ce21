// Shape-dependent plan of the matrix-core kernel (host side): which tile
// configuration of k4_mfma.hip runs a product, whether K is split across
// workgroups, and the packing pre-pass for operands the 16-byte loads cannot
// read as stored.  The choices come from sweeps on MI355X, recorded below
// with the shapes that decided them.
#include <algorithm>

#include "kernels.h"

namespace sgemm {

// Tile configurations, chosen from sweeps on MI355X (square 256..8192,
// K-heavy 64^2 x 65536 .. 1024^2 x 4096, skinny and unaligned shapes; every
// sweep row checked bit-exact against a reference on integer data):
//  * T128: 128 x 128 tiles, 4 waves of 2 x 2 accumulators, K slabs of 16,
//    4 waves per SIMD: with at least two rounds of 1024 tiles (4 per CU) or
//    whole rounds (square 6144: 3.34 ms against 3.62 on 64 x 64; 7168: 5.56
//    against 5.72), and for transposed operands at square 4096;
//  * T64: 64 x 64 tiles, 4 waves of 1 accumulator, K slabs of 32 with
//    16-byte loads (fragments read in two halves: 7 % on square 1024), of 16
//    with 4-byte loads: from 512 tiles up (more than 256 with 16-byte loads
//    and more than 256 tiles of 32 x 32), when the larger tiles would leave
//    a partial round (square 3072 0.488 ms against 0.575 on 128 x 128; 4608
//    1.60 against 1.68; 5120 2.11 against 2.17; 3001 x 4099 x 2047);
//  * T64_WK4: the same tile with 4 K groups (16 waves, one workgroup per CU
//    by LDS): up to 256 such tiles with 16-byte loads (square 1024: 23.9 us
//    against 24.2; 1024^2 x 4096: 79.8 against 86.9).  Between 256 and 512
//    tiles a second round of these workgroups costs more than the groups
//    save, and plain 64 x 64 tiles win (1536 x 1024 x 1024: 40.2 us against
//    45.3; 1280^3: 49.3 against 54.7; 1408^2 x 2048: 76.5 against 83.0);
//  * T32_WK4: 32 x 32 tiles, one wave per K group, 4 groups: outputs of at
//    most 256 such tiles (square 256: 5.0 us against 7.9; square 512: 6.9
//    against 13.2), and with 4-byte loads below 512 tiles of 64 x 64 as well
//    (1024 x 1027 x 1024: 41.5 against 52.0).  A wave's chain of dependent
//    matrix instructions is what bounds these shapes: 32 x 32 tiles give more
//    workgroups, K groups shorten each chain.  With K <= 2048 also up to 768
//    tiles, unsplit (three workgroups per CU, one round), in place of 64 x 64
//    tiles with K groups or a split (640^3 16.3 us -> 10.3, 704^3 17.5 ->
//    11.0, 512 x 1024 x 1024 17.7 -> 14.3, 768 x 1024 x 1280 28.1 -> 22.6,
//    1024 x 768 x 2048 35.5 -> 33.5, 640^2 x 1536 21.9 -> 20.5).  Two
//    shapes measured 1-2 % slower under the rule (640^2 x 2048 25.8 ->
//    26.1, 768^2 x 2048 32.6 -> 33.3); a carve-out for them would need a
//    third bound on K x tiles that no other shape supports, and the rule's
//    gains elsewhere are 5-20 %, so it keeps them.  On packed
//    copies only up to K = 1024 (800 x 801 x 2047 41.5 us split on 64 x 64
//    tiles against 43.8); with longer K (512 x 768 x 4096 35.9 -> 44.3) the
//    64 x 64 choice stays.  From 769 to 1024 tiles these run four per CU
//    with slabs of 16 in two stages (one round), once K groups of one wave
//    ran without per-slab barriers: square 1024 23.2 -> 21.9 us, 896^3 19.0
//    -> 18.4, 800 x 1024 x 1024 22.9 -> 20.2, 1024^2 x 2048 39.9 -> 39.4
//    (earlier, with barriers and three per CU in two rounds, 896^3 21.3 ->
//    24.0 and 1024^3 23.7 -> 26.6 against 64 x 64 tiles).
//  * T128x256: 128 x 256 tiles (4 waves of 2 x 4 accumulators, 2 waves per
//    SIMD, fragments read in halves, raised wave priority during the
//    matrix instructions except with A stored K x M) when the tiles fill
//    whole rounds of 2 per CU, or
//    the last round at least 3/4: square 4096 0.956 ms against 0.990 on
//    128 x 128, 8192 7.57 against 7.79 ms, 5632 2.63 against 2.71; with a
//    smaller last round (square 3072, 4608, 6144) it is the slowest of the
//    three.  Stored transposes take it too (square 8192 with B stored N x K
//    8.11 -> 7.68 ms, A stored K x M 7.90 -> 7.74; square 4096 with A stored
//    K x M 1.006 -> 0.980; both transposed within 0.3 %).

// Split-K on top of the tile choice, when the tiles alone leave the chip
// underused (same sweeps, timed as back-to-back calls so that the second
// launch, about 2.5 us, counts).
//  * 32 x 32 tiles with K groups: with T tiles, up to ceil(512 / T) splits,
//    each keeping at least 256 of K, and only when a workgroup's share of K
//    shrinks by at least 512 (64^2 x 65536: 1316 us unsplit on 64 x 64
//    tiles, 28 us on 32 x 32 with 32 splits; 128^2 x 4096: 85 -> 11.6 us;
//    256^2 x 16384: 333 -> 32 us; 256^2 x 2048: 44 -> 11 us).
//  * 64 x 64 tiles (16-byte loads, fewer than 1024 tiles, i.e. under 4 per
//    CU): the split count from a cost model, below, when it saves at least
//    5 % over the unsplit choice.  At most 16 splits of at least 512 of K.
// Chunks are whole slabs.
namespace {
constexpr int kCUs = 256;
// Sustained rate of one CU running n = 1..4 of the 64 x 64 workgroups, and
// of one CU running the 4-K-group 64 x 64 workgroup, in FLOP per us; fixed
// cost of a launch, and the split reduction's launch and bandwidth (bytes
// per us).  Fitted to sweeps of 64..2048 x 64..16384 x 1024..16384 outputs
// on MI355X (mean error 2 %).
constexpr double kRate64[5] = {0.0, 0.405e6, 0.462e6, 0.475e6, 0.487e6};
constexpr double kRate64Wk4 = 0.43e6;
constexpr double kLaunchUs = 4.0, kReduceUs = 2.5, kReduceBytesPerUs = 5e6;

// Estimated time of T 64 x 64 tiles over S chunks of kc of K: each CU runs
// c = ceil(T S / 256) workgroups one after another at the rate c of them
// sustain together, plus the reduction (S partial products read, C written).
double t64_time_us(const GemmArgs& g, int64_t T, int64_t kc, int64_t S) {
    const int64_t c = ceil_div(T * S, kCUs);
    double t = kLaunchUs + double(c) * double(kc) * 8192.0 / kRate64[c < 4 ? c : 4];
    if (S > 1) t += kReduceUs + 4.0 * double(g.M) * double(g.N) * double(S + 1) / kReduceBytesPerUs;
    return t;
}

// Chunk count for 64 x 64 tiles by the model (1: no split pays).  wk4: the
// unsplit choice is the 4-K-group workgroup (one per CU) rather than plain
// 64 x 64 tiles.
int64_t t64_model_splits(const GemmArgs& g, int64_t T, bool wk4) {
    const double base = wk4 ? kLaunchUs + double(g.K) * 8192.0 / kRate64Wk4 : t64_time_us(g, T, g.K, 1);
    double best = 0.95 * base;
    int64_t pick = 1;
    for (int64_t s = 2; s <= 16; s++) {
        const int64_t kc = ceil_div(ceil_div(g.K, s), 32) * 32;
        if (kc < 512) break;
        const int64_t se = ceil_div(g.K, kc);
        const double t = t64_time_us(g, T, kc, se);
        if (t < best) {
            best = t;
            pick = se;
        }
    }
    return pick;
}
}  // namespace

SplitPlan k4_plan(const GemmArgs& g, int requested) {
    const bool vec = vec_ok(g);
    const int64_t bk = vec ? 32 : 16;
    const int64_t T128 = ceil_div(g.M, 128) * ceil_div(g.N, 128);
    const int64_t T64 = ceil_div(g.M, 64) * ceil_div(g.N, 64);
    const int64_t T32 = ceil_div(g.M, 32) * ceil_div(g.N, 32);
    const int64_t T256 = ceil_div(g.M, 128) * ceil_div(g.N, 256);
    int cfg;
    int64_t tiles;
    // Large tiles pay off only when the workgroups fill their rounds: a
    // partial last round of 128 x 256 (2 per CU) costs about a full one, of
    // 128 x 128 (4 per CU) about its share.  They must also be mostly full
    // themselves (at least 7/8 of the tiles' area inside C): an edge tile
    // does a whole tile's matrix work, so a narrow output wastes most of it
    // (65536 x 128 x 1024: 251 us on 128 x 256, 156 on 64 x 64; 65536 x 64 x
    // 4096: 961 against 335; 32768 x 320 x 2048: 485 against 360).
    const double area = double(g.M) * double(g.N);
    const bool full256 = area >= 0.875 * double(T256) * 128.0 * 256.0;
    const bool full128 = area >= 0.875 * double(T128) * 128.0 * 128.0;
    if (vec && full256 && T256 >= 512 &&
        (T256 % 512 == 0 || T256 % 512 >= 384)) {
        cfg = K4_T128X256;
        tiles = T256;
    } else if (vec && full128 && (T128 >= 2048 || (T128 >= 1024 && T128 % 1024 == 0))) {
        cfg = K4_T128;
        tiles = T128;
    } else if (T64 >= 512 || (vec && T64 > 256 && T32 > 256)) {
        cfg = K4_T64;
        tiles = T64;
    } else if (T32 <= 256 || !vec || (T32 <= 4 * kCUs && g.K <= (g.runs_padded ? 1024 : 2048))) {
        cfg = K4_T32_WK4;
        tiles = T32;
    } else {
        cfg = K4_T64_WK4;
        tiles = T64;
    }
    // Under 4 workgroups of 64 x 64 per CU: the model's split, if any.
    int64_t model_S = 1;
    if (requested <= 0 && vec && (cfg == K4_T64 || cfg == K4_T64_WK4) && T64 < 4 * kCUs) {
        model_S = t64_model_splits(g, T64, cfg == K4_T64_WK4);
        if (model_S > 1) cfg = K4_T64;
    }
    int64_t S = requested;
    if (S <= 0) {
        S = model_S;
        if (cfg == K4_T32_WK4) {
            S = std::min<int64_t>(std::min(ceil_div(512, tiles), g.K / 256), 32);
            if ((S >= 2 && g.K - ceil_div(g.K, S) < 512) || tiles > 256) S = 1;
        }
    }
    // 128 x 128 and 128 x 256 tiles have no split variant: a requested split
    // runs on 64 x 64.
    if (S > 1 && (cfg == K4_T128 || cfg == K4_T128X256)) cfg = K4_T64;
    S = std::min(S, ceil_div(g.K, bk));
    if (S <= 1) return {1, g.K, 0, cfg};
    const int64_t kc = ceil_div(ceil_div(g.K, S), bk) * bk;
    S = ceil_div(g.K, kc);
    return {(int)S, kc, S * g.M * split_ld(g.N), cfg};
}

static hipError_t launch_plan(const GemmArgs& g, const SplitPlan& p, float* ws, hipStream_t s) {
    const int kc = (int)p.kchunk;
    switch (p.cfg) {
        case K4_T128: return launch_k4_tile128(g, s);
        case K4_T128X256: return launch_k4_tile128x256(g, s);
        case K4_T64_WK4: return launch_k4_t64_wk4(g, s, p.splits, kc, ws);
        case K4_T32_WK4: return launch_k4_t32_wk4(g, s, p.splits, kc, ws);
        default: return launch_k4_t64(g, s, p.splits, kc, ws);
    }
}

// Packing pre-pass: operands that do not suit 16-byte loads are copied into
// zero-padded aligned rows (pack.hip) when the output is large enough for a
// 64 x 64 or larger tile configuration, where the 16-byte path pays for the
// copy (3001 x 4099 x 2047: 0.488 ms on 4-byte loads, 0.437 ms + 0.02 ms of
// packing on 16-byte ones; 4095 x 4097 x 4093: 1.295 -> 1.158 + 0.04 ms).
// Smaller outputs keep 4-byte loads.
namespace {
struct PackPlan {
    bool pack_a = false, pack_b = false;
    int64_t a_rows = 0, a_run = 0, b_rows = 0, b_run = 0;
    size_t a_bytes = 0, b_bytes = 0;  // each copy rounded up to 256 bytes
    GemmArgs gp;                      // the product on the copies
    SplitPlan p;                      // and its plan
};
}  // namespace

// Whether an eager shape-chosen call packs g's operands first, and then how.
// The plan depends on the copies' addresses only through their 16-byte
// alignment, which the workspace layout gives; until the copies exist gp
// holds an aligned placeholder address for them.
static bool packing_plan(const GemmArgs& g, PackPlan* pk) {
    if (vec_ok(g)) return false;
    GemmArgs gp = g;
    gp.runs_padded = true;
    pk->a_rows = g.trans_a ? g.K : g.M;
    pk->a_run = g.trans_a ? g.M : g.K;
    pk->b_rows = g.trans_b ? g.N : g.K;
    pk->b_run = g.trans_b ? g.K : g.N;
    pk->pack_a = !rows_vec(g.A, g.lda, pk->a_run);
    pk->pack_b = !rows_vec(g.B, g.ldb, pk->b_run);
    if (pk->pack_a) {
        gp.A = reinterpret_cast<const float*>(uintptr_t(256));
        gp.lda = packed_ld(pk->a_run);
        pk->a_bytes = (size_t(pk->a_rows * gp.lda) * sizeof(float) + 255) / 256 * 256;
    }
    if (pk->pack_b) {
        gp.B = reinterpret_cast<const float*>(uintptr_t(256));
        gp.ldb = packed_ld(pk->b_run);
        pk->b_bytes = (size_t(pk->b_rows * gp.ldb) * sizeof(float) + 255) / 256 * 256;
    }
    if (!k4_supports(gp)) return false;
    // Worth a copy launch: outputs of at least 512 tiles of 64 x 64; or a
    // product moving 64 MB or more whose copies are at most 1/8 of that, as
    // when a narrow or thin operand is the only unaligned one (8192 x 13 x
    // 8192: 82 -> 61 us; 13 x 8192 x 8191); or 4 GFLOP or more with copies
    // of at most 64 MB and 1 byte per 100 FLOP (767 x 769 x 4095: 91 -> 72
    // us; 1025 x 1025 x 2047: 78 -> 70), or with K >= 1536 from 1 GFLOP
    // (511 x 513 x 4095: 72 -> 42 us; 800 x 801 x 2047: 48.3 -> 43.3; 767 x
    // 769 x 2047: 48.1 -> 43.6).  The copy launch and the wait for it cost
    // about 9 us at 8 MB, so it did not pay for shorter K (1023^3: 32.2 ->
    // 33.0 us; 1024 x 1027 x 1024: 41.6 -> 42.1; 1023^2 x 511: 19.3 -> 20.7),
    // nor where a large operand of a memory-bound product is copied (1 x 8191
    // x 8192: 79 -> 144).
    const double moved = 4.0 * (double(g.M) * g.K + double(g.K) * g.N + double(g.M) * g.N);
    const double flop = 2.0 * double(g.M) * double(g.N) * double(g.K);
    const double copied = double(pk->a_bytes + pk->b_bytes);
    const bool big_output = ceil_div(g.M, 64) * ceil_div(g.N, 64) >= 512;
    const bool thin_copy = moved >= 64e6 && copied <= moved / 8;
    const bool heavy = (flop >= 4e9 || (flop >= 1e9 && g.K >= 1536)) && copied <= 64e6 &&
                       copied <= flop / 100;
    if (!big_output && !thin_copy && !heavy) return false;
    pk->p = k4_plan(gp, 0);
    pk->gp = gp;
    return true;
}

static hipError_t launch_packed(const GemmArgs& g, hipStream_t s, bool* done,
                                const FixedScratch* fixed) {
    *done = false;
    PackPlan pk;
    if (!packing_plan(g, &pk)) return hipSuccess;
    // Workspace: A's copy, B's copy, then the split's partial products,
    // each on a 256-byte boundary.
    size_t p_bytes = pk.p.splits > 1 ? size_t(pk.p.ws_floats) * sizeof(float) : 0;
    Workspace ws;
    char* base;
    if (fixed) {
        // A fixed scratch too small for the partial products runs the packed
        // product unsplit; too small for the copies, the 4-byte path.
        if (pk.a_bytes + pk.b_bytes + p_bytes > fixed->bytes) {
            if (pk.a_bytes + pk.b_bytes > fixed->bytes) return hipSuccess;
            pk.p.splits = 1;
            p_bytes = 0;
        }
        base = reinterpret_cast<char*>(fixed->ptr);
    } else {
        if (workspace_acquire(pk.a_bytes + pk.b_bytes + p_bytes, s, &ws) != hipSuccess) {
            (void)hipGetLastError();
            return hipSuccess;  // no workspace: the 4-byte path
        }
        base = static_cast<char*>(ws.ptr);
    }
    float* pa = reinterpret_cast<float*>(base);
    float* pb = reinterpret_cast<float*>(base + pk.a_bytes);
    float* pp = pk.p.splits > 1 ? reinterpret_cast<float*>(base + pk.a_bytes + pk.b_bytes) : nullptr;
    // One launch packs both operands when both need it.
    hipError_t e;
    if (pk.pack_a && pk.pack_b)
        e = launch_pack(g.A, pk.a_rows, pk.a_run, g.lda, pa, g.B, pk.b_rows, pk.b_run, g.ldb, pb, s);
    else if (pk.pack_a)
        e = launch_pack(g.A, pk.a_rows, pk.a_run, g.lda, pa, nullptr, 0, 0, 0, nullptr, s);
    else
        e = launch_pack(g.B, pk.b_rows, pk.b_run, g.ldb, pb, nullptr, 0, 0, 0, nullptr, s);
    GemmArgs gp = pk.gp;
    if (pk.pack_a) gp.A = pa;
    if (pk.pack_b) gp.B = pb;
    if (e == hipSuccess) e = launch_plan(gp, pk.p, pp, s);
    *done = true;
    if (fixed) return e;
    const hipError_t f = workspace_release(&ws, s);
    return e != hipSuccess ? e : f;
}

// Thin products (one side of C at most 8) stream their large operand on the
// vector units (thin.hip) when it is stored with K on the long axis (B
// stored K x N for M <= 8, A stored M x K for N <= 8; in 16-byte loads, or
// 4-byte ones for rows that are not whole 16-byte chunks: 16384 x 1 x 16383
// 314 -> 176 us, 2 x 65535 x 4096 698 -> 178, against the matrix cores'
// 4-byte path) and is large enough: 384 MB or more;
// for N <= 4, 256 MB; for a single column, 16 MB.  Measured against the
// matrix-core path, whose 32 x 32 tiles stream the operand too (MI355X,
// back-to-back launches, us): 1 x 16384 x 16384 290 -> 168, 16384 x 8 x
// 16384 296 -> 187, 2 x 65536 x 4096 286 -> 174, 100000 x 4 x 1024 127 ->
// 80, 8192 x 4 x 8192 56 -> 51, 8192 x 1 x 8192 79 -> 48; at 268 MB the
// thin kernels were no faster for M <= 8 or 5 <= N <= 8 (1 x 8192 x 8192
// 55 -> 55, 8192 x 8 x 8192 56 -> 62): the fixed costs of the split and of
// staging B weigh more there.  thin_n runs workgroups of 8 waves that keep
// two steps' loads in flight, except for one or two columns of C with
// M >= 16384, where 4 waves of one step each were faster (100000 x 1 x
// 4096 300 -> 274, 65536 x 2 x 4096 204 -> 181, 16384 x 1 x 16384 168 ->
// 162).  K is split so that about 1024 workgroups keep loads in flight; a
// chunk keeps at least 256 of K (thin_m) or one 1024-k piece (thin_n).
static ThinPlan thin_plan_direct(const GemmArgs& g, bool transposed) {
    ThinPlan t;
    constexpr int64_t kTarget = 1024, kMinBytes = int64_t(384) << 20;
    constexpr int64_t kMinFewColumns = int64_t(256) << 20, kMinColumn = int64_t(16) << 20;
    // thin_n's grid has one work-item per 1/16 row (4 rows a wave), which
    // must stay under the 2^32 work-items a dispatch can count.
    constexpr int64_t kMaxThinRows = int64_t(1) << 27;
    int64_t groups = 0, min_chunk = 0, quantum = 4;
    // The lower thresholds for few columns are where the matrix-core path
    // reads the small operand with 4-byte loads; a transposed product's
    // original keeps 16-byte loads there (1 x 8192 x 8192 with B stored N x K:
    // 48.7 us on the matrix cores, 50.0 on thin_n).
    const int64_t min_n = transposed ? kMinBytes : g.N == 1 ? kMinColumn : g.N <= 4 ? kMinFewColumns : kMinBytes;
    // A streamed operand whose rows are not whole 16-byte chunks leaves the
    // matrix cores their 4-byte path, which the thin kernels beat from
    // 16 MB for up to 4 rows or columns of C (us: 1 x 8191 x 8192 76 -> 60,
    // 8192 x 4 x 8191 76 -> 52, 8192 x 3 x 4095 41.8 -> 27.9, 1 x 4095 x 4096
    // 25.5 -> 21.1) but not for 8 (8 x 4095 x 4096 25.7 -> 27.7).
    const bool few_m = g.M <= 4 && !rows_vec(g.B, g.ldb, g.N);
    const bool few_n = g.N <= 4 && !rows_vec(g.A, g.lda, g.K);
    if (g.M <= 8 && !g.trans_b && 4 * g.K * g.N >= (few_m ? kMinColumn : kMinBytes)) {
        t.kind = ThinPlan::THIN_M;
        groups = ceil_div(g.N, 256);
        min_chunk = 256;
    } else if (g.N <= 8 && !g.trans_a && 4 * g.M * g.K >= (few_n ? kMinColumn : min_n) &&
               g.M <= kMaxThinRows) {
        t.kind = ThinPlan::THIN_N;
        t.waves = g.N <= 2 && g.M >= 16384 ? 4 : 8;
        groups = ceil_div(g.M, 4 * t.waves);
        min_chunk = 1024;
        quantum = 1024;
    } else {
        return t;
    }
    int64_t S = std::min<int64_t>(std::min(ceil_div(kTarget, groups), g.K / min_chunk), 64);
    if (S < 1) S = 1;
    const int64_t kc = ceil_div(ceil_div(g.K, S), quantum) * quantum;
    t.splits = (int)ceil_div(g.K, kc);
    t.kchunk = t.splits > 1 ? kc : g.K;
    t.ws_floats = t.splits > 1 ? t.splits * g.M * g.N : 0;
    return t;
}

// A large operand stored with K contiguous on the other side (B stored
// N x K with M <= 8, A stored K x M with N <= 8) is streamed by the same
// kernels on the transposed product, whose result they store transposed,
// from 384 MB (MI355X, us: 1 x 16384 x 16384 with B stored N x K 268 ->
// 167, 16384 x 1 x 16384 with A stored K x M 290 -> 164, 8 x 16384 x 16384
// 270 -> 207, 16384 x 8 x 16384 286 -> 184, 2 x 65536 x 4096 265 -> 187).
ThinPlan thin_plan(const GemmArgs& g) {
    ThinPlan t = thin_plan_direct(g, false);
    if (t.kind != ThinPlan::NONE || (g.M > 8 && g.N > 8)) return t;
    t = thin_plan_direct(swapped(g), true);
    t.swap = t.kind != ThinPlan::NONE;
    return t;
}

PlanInfo plan_info(const GemmArgs& g, int requested) {
    PlanInfo info;
    if (requested == 0) {
        const ThinPlan t = thin_plan(g);
        if (t.kind != ThinPlan::NONE) {
            info.engine = 2;
            const GemmArgs gt = t.swap ? swapped(g) : g;
            int tm = t.kind == ThinPlan::THIN_M ? (int)gt.M : 4 * t.waves;
            int tn = t.kind == ThinPlan::THIN_M ? 256 : (int)gt.N;
            if (t.swap) std::swap(tm, tn);
            info.tile_m = tm;
            info.tile_n = tn;
            info.k_groups = t.kind == ThinPlan::THIN_M ? 4 : 1;
            info.splits = t.splits;
            info.kchunk = t.kchunk;
            return info;
        }
    }
    PackPlan pk;
    info.packed = requested == 0 && packing_plan(g, &pk);
    const SplitPlan p = info.packed ? pk.p : k4_plan(g, requested);
    static const int dims[][3] = {
        {128, 128, 1},  // K4_T128
        {64, 64, 1},    // K4_T64
        {64, 64, 4},    // K4_T64_WK4
        {32, 32, 4},    // K4_T32_WK4
        {128, 256, 1},  // K4_T128X256
    };
    static_assert(K4_T128 == 0 && K4_T64 == 1 && K4_T64_WK4 == 2 && K4_T32_WK4 == 3 && K4_T128X256 == 4,
                  "table order");
    info.engine = 1;
    info.tile_m = dims[p.cfg][0];
    info.tile_n = dims[p.cfg][1];
    info.k_groups = dims[p.cfg][2];
    info.splits = p.splits;
    info.kchunk = p.kchunk;
    return info;
}

// Whether work on s is being captured into a graph.  The workspace paths
// (split-K, packing) allocate stream-ordered memory and order uses across
// streams with an event, which a capture cannot take part in; captured
// calls run the unsplit kernel on the operands as stored instead, so every
// entry point can be captured.
static bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) {
        (void)hipGetLastError();
        return false;
    }
    return st != hipStreamCaptureStatusNone;
}

size_t k4_split_scratch_bytes(const GemmArgs& g, int requested) {
    const SplitPlan p = k4_plan(g, requested);
    return p.splits > 1 ? size_t(p.ws_floats) * sizeof(float) : 0;
}

hipError_t launch_k4_mfma(const GemmArgs& g, hipStream_t s, int requested, bool thin_ok,
                          const FixedScratch* fixed) {
    // A fixed scratch needs no allocation and no ordering across streams,
    // so captured calls may use it too.
    const bool in_graph = !fixed && capturing(s);
    if (requested == 0 && thin_ok) {
        ThinPlan t = thin_plan(g);
        if (t.kind != ThinPlan::NONE) {
            Workspace ws;
            float* buf = nullptr;
            bool pooled = false;
            if (t.splits > 1) {
                const size_t bytes = size_t(t.ws_floats) * sizeof(float);
                if (fixed) {
                    if (bytes <= fixed->bytes) buf = fixed->ptr;
                } else if (!in_graph) {
                    if (workspace_acquire(bytes, s, &ws) == hipSuccess) {
                        buf = static_cast<float*>(ws.ptr);
                        pooled = true;
                    } else {
                        (void)hipGetLastError();
                    }
                }
                // Captured, or no scratch: one chunk gives the same product.
                if (!buf) {
                    t.splits = 1;
                    t.kchunk = g.K;
                }
            }
            const hipError_t e = launch_thin(g, t, buf, s);
            if (!pooled) return e;
            const hipError_t f = workspace_release(&ws, s);
            return e != hipSuccess ? e : f;
        }
    }
    if (requested == 0 && !in_graph) {
        bool done;
        const hipError_t e = launch_packed(g, s, &done, fixed);
        if (done || e != hipSuccess) return e;
    }
    SplitPlan p = k4_plan(g, requested);
    if (in_graph || (fixed && size_t(p.ws_floats) * sizeof(float) > fixed->bytes)) p.splits = 1;
    if (p.splits <= 1) return launch_plan(g, p, nullptr, s);
    if (fixed) return launch_plan(g, p, fixed->ptr, s);
    Workspace ws;
    if (workspace_acquire(size_t(p.ws_floats) * sizeof(float), s, &ws) != hipSuccess) {
        // No workspace: the unsplit kernel gives the same product.
        (void)hipGetLastError();
        p.splits = 1;
        return launch_plan(g, p, nullptr, s);
    }
    const hipError_t e = launch_plan(g, p, static_cast<float*>(ws.ptr), s);
    const hipError_t f = workspace_release(&ws, s);
    return e != hipSuccess ? e : f;
}

}  // namespace sgemm
