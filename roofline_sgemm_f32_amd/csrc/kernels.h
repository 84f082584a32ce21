// Internal launcher interface between the C ABI (api.hip) and the kernels.
// Every launcher enqueues on the given stream and returns the launch status;
// arguments have already been validated by the caller.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <mutex>

namespace sgemm {

// C = alpha * op(A) * op(B) + beta * C, row-major.  trans_a: A is stored
// K x M (else M x K); trans_b: B is stored N x K (else K x N).  beta == 0
// means C is not read.
struct GemmArgs {
    int64_t M, N, K;
    const float* A;
    int64_t lda;
    const float* B;
    int64_t ldb;
    float* C;
    int64_t ldc;
    bool trans_a = false, trans_b = false;
    float alpha = 1.0f, beta = 0.0f;
    // Rows of A and B as stored hold their run rounded up to 4 floats, the
    // extra ones zero (packed operands: see pack.hip).
    bool runs_padded = false;
};

// Upper bound on the number of workgroups a launch uses; kernels loop over
// tiles beyond it, which keeps grid * block within the 32-bit dispatch size.
constexpr int64_t kMaxGrid = int64_t(1) << 20;

// Copy probe: workgroup count limit (grid * block stays below 2^32 work-items
// for blocks of up to 1024 lanes).
constexpr int64_t kMaxCopyGrid = int64_t(1) << 22;
constexpr int kCopyBlock = 64;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline unsigned grid_for(int64_t tiles) { return unsigned(tiles < kMaxGrid ? tiles : kMaxGrid); }

hipError_t launch_k0_naive(const GemmArgs& g, hipStream_t s);
hipError_t launch_k1_coalesced(const GemmArgs& g, hipStream_t s);
hipError_t launch_k2_lds(const GemmArgs& g, int tile, int pad, hipStream_t s);
hipError_t launch_k3_regtile(const GemmArgs& g, hipStream_t s);
// Scratch memory fixed by the caller (the static scratch of the entry point
// that allocates nothing): when given, the launches use it in place of the
// library's workspace, and a plan whose scratch does not fit in `bytes`
// runs without it (unpacked, or unsplit).
struct FixedScratch {
    float* ptr = nullptr;
    size_t bytes = 0;
};
// Tile size and K split chosen by shape; requested_splits > 0 asks for that
// many K chunks (at most; 1 = never split).  thin_ok: a shape-chosen call
// (requested_splits == 0) may run the thin-product kernels on the vector
// units (thin.hip); otherwise every product runs on the matrix cores.
hipError_t launch_k4_mfma(const GemmArgs& g, hipStream_t s, int requested_splits = 0,
                          bool thin_ok = true, const FixedScratch* fixed = nullptr);
// Bytes of scratch an eager call with this split request would use for its
// partial products (requested_splits >= 2; 0 when the plan does not split).
size_t k4_split_scratch_bytes(const GemmArgs& g, int requested_splits);
// Devices the per-device tables (workspace, static scratch) can serve.
constexpr int kMaxDevices = 64;
// Size of the library's static device scratch (static_scratch.hip).
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
// The static scratch of the device that runs `s`: its device address (found
// once per device) and size.
hipError_t static_scratch(hipStream_t s, FixedScratch* out);
// Plan of the matrix-core kernel for a shape: tile configuration (cfg, an
// internal id) and K split, `splits` chunks of kchunk (the last one shorter)
// whose partial products take ws_floats floats of workspace.
struct SplitPlan {
    int splits;
    int64_t kchunk, ws_floats;
    int cfg;
};
// requested_splits 0: split by shape; > 0: at most that many chunks.
SplitPlan k4_plan(const GemmArgs& g, int requested_splits);
// Thin products on the vector units (thin.hip): M <= 8 (B streamed) or
// N <= 8 (A streamed), in `splits` K chunks of kchunk whose partial
// products take ws_floats floats of workspace; thin_n workgroups of `waves`
// waves (8, or 4 for N <= 2), 4 rows of C each.  swap: the plan is for the
// transposed product C^T = op(B)^T op(A)^T (swapped(g)), whose kernels store
// C^T into C transposed; that is how a large operand stored with K
// contiguous on the other side (B stored N x K for M <= 8, A stored K x M
// for N <= 8) is streamed.
struct ThinPlan {
    enum Kind { NONE, THIN_M, THIN_N } kind = NONE;
    int splits = 1, waves = 8;
    bool swap = false;
    int64_t kchunk = 0, ws_floats = 0;
};
// The transposed product C^T = op(B)^T op(A)^T, with C^T held in C (its
// element (j, i) at C[i * ldc + j]).
inline GemmArgs swapped(const GemmArgs& g) {
    GemmArgs t = g;
    t.M = g.N;
    t.N = g.M;
    t.A = g.B;
    t.lda = g.ldb;
    t.trans_a = !g.trans_b;
    t.B = g.A;
    t.ldb = g.lda;
    t.trans_b = !g.trans_a;
    return t;
}
// Whether a shape-chosen call takes the thin path, and how.
ThinPlan thin_plan(const GemmArgs& g);
// What an eager call with this K-split request runs (requested 0: shape-
// chosen): engine 1 the matrix-core kernel, 2 the thin vector kernels; the
// workgroup's C tile and K groups; whether operands are packed first; the
// K chunks.
struct PlanInfo {
    int engine = 0, tile_m = 0, tile_n = 0, k_groups = 0;
    bool packed = false;
    int splits = 0;
    int64_t kchunk = 0;
};
PlanInfo plan_info(const GemmArgs& g, int requested);
hipError_t launch_thin(const GemmArgs& g, const ThinPlan& p, float* ws, hipStream_t s);
// Split-K second pass: C = alpha * (sum of the `splits` dense M x N slabs of
// ws, added in slab order) (+ beta * C).
// C from `splits` partial slabs in ws, each M rows of ldw floats (C's
// columns first), added in slab order; alpha and beta as the unsplit
// epilogue applies them.
hipError_t launch_splitk_reduce(const GemmArgs& g, int splits, const float* ws, int64_t ldw,
                                hipStream_t s);
// Row length of the matrix-core kernel's split partial slabs: N rounded up
// to 4 floats, so the reduction reads them in 16-byte accesses.
inline int64_t split_ld(int64_t N) { return (N + 3) / 4 * 4; }
// Scratch memory for launches that need it: the device's cached buffer,
// held (with the device's workspace lock) from acquire to release; every
// launch that uses it goes on stream s in between.
struct Workspace {
    void* ptr = nullptr;
    bool own = false;  // a one-off buffer, freed stream-ordered on release
    int dev = 0;
    std::unique_lock<std::mutex> lock;
};
hipError_t workspace_acquire(size_t bytes, hipStream_t s, Workspace* ws);
hipError_t workspace_release(Workspace* ws, hipStream_t s);
// Tile configurations of the matrix-core kernel (k4_mfma.hip), as the plan
// (k4_plan.hip) names them: 128 x 128, 64 x 64, 64 x 64 with 4 K groups,
// 32 x 32 with 4 K groups, 128 x 256.
enum K4Cfg { K4_T128, K4_T64, K4_T64_WK4, K4_T32_WK4, K4_T128X256 };
hipError_t launch_k4_tile128(const GemmArgs& g, hipStream_t s);
hipError_t launch_k4_tile64(const GemmArgs& g, hipStream_t s);
// 128 x 256 tiles for A and B as stored (transposed operands: 128 x 128).
hipError_t launch_k4_tile128x256(const GemmArgs& g, hipStream_t s);
// The configurations with a split-K mode: splits > 1 runs `splits` chunks of
// kchunk of K into ws (splits * M * N floats), then the reduction into C.
hipError_t launch_k4_t64(const GemmArgs& g, hipStream_t s, int splits, int kchunk, float* ws);
hipError_t launch_k4_t32_wk4(const GemmArgs& g, hipStream_t s, int splits, int kchunk, float* ws);
hipError_t launch_k4_t64_wk4(const GemmArgs& g, hipStream_t s, int splits, int kchunk, float* ws);
// Whether the matrix-core kernel's 32-bit buffer offsets can address this shape.
bool k4_supports(const GemmArgs& g);
// Whether rows of `run` floats at stride ld from p suit 16-byte loads
// (aligned rows, whole 4-float chunks), and whether both operands do.
bool rows_vec(const float* p, int64_t ld, int64_t run);
bool vec_ok(const GemmArgs& g);
hipError_t launch_zero(float* C, int64_t M, int64_t N, int64_t ldc, hipStream_t s);
// C = beta * C (zeros when beta == 0, C then not read).
hipError_t launch_scale(float* C, int64_t M, int64_t N, int64_t ldc, float beta, hipStream_t s);
// General (transposes, alpha, beta) one-output-per-lane kernel with 64-bit
// offsets: the fallback for shapes the matrix-core kernel cannot address.
hipError_t launch_k1_general(const GemmArgs& g, hipStream_t s);
// Row length of a packed copy: cols rounded up to 4 floats, or for rows of
// at least 256 floats to 32 (128-byte rows, so that a tile's row segments do
// not straddle an extra cache line: 3001 x 4099 x 2047 423.4 -> 421.8 us,
// 1025 x 1025 x 2047 66.1 -> 65.2, 513 x 511 x 8193 62.9 -> 61.6).  Shared by
// the copy kernel and the host, which sizes and reads the copies.
__host__ __device__ inline int64_t packed_ld(int64_t cols) {
    return cols >= 256 ? (cols + 31) / 32 * 32 : (cols + 3) / 4 * 4;
}
// Copy a stored rows x cols matrix (leading dimension ld, any alignment)
// into dst as rows x packed_ld(cols), zero-padded; dst 16-byte aligned.  A
// second matrix (src2 not null) is packed by the same launch.
hipError_t launch_pack(const float* src, int64_t rows, int64_t cols, int64_t ld, float* dst,
                       const float* src2, int64_t rows2, int64_t cols2, int64_t ld2, float* dst2,
                       hipStream_t s);
hipError_t launch_copy(float* dst, const float* src, int64_t n, int block, int64_t grid, hipStream_t s);
int64_t copy_default_grid(int64_t n, int block);
hipError_t launch_probe_valu(float* out, int64_t iters, float x, float y, int64_t blocks, int block,
                             hipStream_t s);
hipError_t launch_probe_mfma(float* out, const float* a_vals, const float* b_vals, int64_t iters,
                             int64_t blocks, hipStream_t s);

}  // namespace sgemm
