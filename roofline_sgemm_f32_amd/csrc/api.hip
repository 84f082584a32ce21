// C ABI entry points: argument validation (host only, before any HIP call),
// variant dispatch and launch-status reporting.  The interface contract is
// documented in include/sgemm.h.
#include "../../include/sgemm.h"
#include "kernels.h"

using sgemm::GemmArgs;

namespace {

thread_local int g_last_hip_error = 0;

int launch_status(hipError_t e) {
    if (e == hipSuccess) return SGEMM_OK;
    g_last_hip_error = int(e);
    return SGEMM_ERR_LAUNCH;
}

// Byte range [lo, hi) spanned by a rows x cols row-major view (rows, cols > 0).
void span(const void* p, int64_t rows, int64_t cols, int64_t ld, uintptr_t* lo, uintptr_t* hi) {
    *lo = reinterpret_cast<uintptr_t>(p);
    *hi = *lo + uintptr_t(((rows - 1) * ld + cols) * int64_t(sizeof(float)));
}

bool overlaps(uintptr_t alo, uintptr_t ahi, uintptr_t blo, uintptr_t bhi) {
    return alo < bhi && blo < ahi;
}

int validate(int variant, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
             const float* B, int64_t ldb, const float* C, int64_t ldc) {
    if (variant < 0 || variant >= SGEMM_VARIANT_COUNT) return SGEMM_ERR_VARIANT;
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_DIM;
    // Keep every element offset, and (rows - 1) * ld + cols, inside int64.
    const int64_t lim = int64_t(1) << 40;
    if (M > lim || N > lim || K > lim) return SGEMM_ERR_DIM;
    const int64_t k1 = K > 1 ? K : 1, n1 = N > 1 ? N : 1;
    if (lda < k1 || ldb < n1 || ldc < n1) return SGEMM_ERR_LD;
    if (lda > lim || ldb > lim || ldc > lim) return SGEMM_ERR_LD;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (C == nullptr) return SGEMM_ERR_NULLPTR;
    if (K > 0) {
        if (A == nullptr || B == nullptr) return SGEMM_ERR_NULLPTR;
        uintptr_t clo, chi, alo, ahi, blo, bhi;
        span(C, M, N, ldc, &clo, &chi);
        span(A, M, K, lda, &alo, &ahi);
        span(B, K, N, ldb, &blo, &bhi);
        if (overlaps(clo, chi, alo, ahi) || overlaps(clo, chi, blo, bhi)) return SGEMM_ERR_ALIAS;
    }
    return SGEMM_OK;
}

// Validation of the general entry point (row-major; see include/sgemm.h):
// flags, sizes and leading dimensions, then pointers.
int validate_ex_shape(int ta, int tb, int64_t M, int64_t N, int64_t K, int64_t lda, int64_t ldb,
                      int64_t ldc) {
    if ((ta != SGEMM_OP_N && ta != SGEMM_OP_T) || (tb != SGEMM_OP_N && tb != SGEMM_OP_T))
        return SGEMM_ERR_ARG;
    if (M < 0 || N < 0 || K < 0) return SGEMM_ERR_DIM;
    const int64_t lim = int64_t(1) << 40;
    if (M > lim || N > lim || K > lim) return SGEMM_ERR_DIM;
    const int64_t m1 = M > 1 ? M : 1, n1 = N > 1 ? N : 1, k1 = K > 1 ? K : 1;
    if (lda < (ta ? m1 : k1) || ldb < (tb ? k1 : n1) || ldc < n1) return SGEMM_ERR_LD;
    if (lda > lim || ldb > lim || ldc > lim) return SGEMM_ERR_LD;
    return SGEMM_OK;
}

int validate_ex(int ta, int tb, int64_t M, int64_t N, int64_t K, float alpha, const float* A,
                int64_t lda, const float* B, int64_t ldb, const float* C, int64_t ldc) {
    const int v = validate_ex_shape(ta, tb, M, N, K, lda, ldb, ldc);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    if (C == nullptr) return SGEMM_ERR_NULLPTR;
    if (K > 0 && alpha != 0.0f) {
        if (A == nullptr || B == nullptr) return SGEMM_ERR_NULLPTR;
        uintptr_t clo, chi, alo, ahi, blo, bhi;
        span(C, M, N, ldc, &clo, &chi);
        if (ta) span(A, K, M, lda, &alo, &ahi); else span(A, M, K, lda, &alo, &ahi);
        if (tb) span(B, N, K, ldb, &blo, &bhi); else span(B, K, N, ldb, &blo, &bhi);
        if (overlaps(clo, chi, alo, ahi) || overlaps(clo, chi, blo, bhi)) return SGEMM_ERR_ALIAS;
    }
    return SGEMM_OK;
}

int choose_auto(const GemmArgs& g) {
    // The matrix-core kernel handles every shape whose per-slab offsets fit
    // its 32-bit buffer addressing; the register-tiled kernel (64-bit
    // offsets) takes the rest.
    return sgemm::k4_supports(g) ? SGEMM_K4_MFMA : SGEMM_K3_REGTILE_DB;
}

}  // namespace

extern "C" {

int sgemm_f32_variant(int variant, int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                      const float* B, int64_t ldb, float* C, int64_t ldc, void* stream) {
    const int v = validate(variant, M, N, K, A, lda, B, ldb, C, ldc);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const GemmArgs g{M, N, K, A, lda, B, ldb, C, ldc};
    if (K == 0) return launch_status(sgemm::launch_zero(C, M, N, ldc, s));
    if (variant == SGEMM_AUTO) {
        // AUTO may also take the thin-product kernels (vector units) for
        // products with one side of C at most 8.
        if (choose_auto(g) == SGEMM_K4_MFMA) return launch_status(sgemm::launch_k4_mfma(g, s, 0, true));
        return launch_status(sgemm::launch_k3_regtile(g, s));
    }
    switch (variant) {
        case SGEMM_K0_NAIVE: return launch_status(sgemm::launch_k0_naive(g, s));
        case SGEMM_K1_COALESCED: return launch_status(sgemm::launch_k1_coalesced(g, s));
        case SGEMM_K2_LDS_TILED: return launch_status(sgemm::launch_k2_lds(g, 32, 0, s));
        case SGEMM_K2_LDS_TILED16: return launch_status(sgemm::launch_k2_lds(g, 16, 0, s));
        case SGEMM_K2_LDS_TILED_PAD1: return launch_status(sgemm::launch_k2_lds(g, 32, 1, s));
        case SGEMM_K2_LDS_TILED16_PAD1: return launch_status(sgemm::launch_k2_lds(g, 16, 1, s));
        case SGEMM_K3_REGTILE_DB: return launch_status(sgemm::launch_k3_regtile(g, s));
        case SGEMM_K4_MFMA:
            if (!sgemm::k4_supports(g)) return SGEMM_ERR_UNSUPPORTED;
            // Always the matrix cores (tile, K split and packing by shape).
            return launch_status(sgemm::launch_k4_mfma(g, s, 0, false));
        case SGEMM_K4_MFMA_TILE128:
            if (!sgemm::k4_supports(g)) return SGEMM_ERR_UNSUPPORTED;
            return launch_status(sgemm::launch_k4_tile128(g, s));
        case SGEMM_K4_MFMA_TILE64:
            if (!sgemm::k4_supports(g)) return SGEMM_ERR_UNSUPPORTED;
            return launch_status(sgemm::launch_k4_tile64(g, s));
        case SGEMM_K4_MFMA_TILE128X256:
            if (!sgemm::k4_supports(g)) return SGEMM_ERR_UNSUPPORTED;
            return launch_status(sgemm::launch_k4_tile128x256(g, s));
        default: return SGEMM_ERR_VARIANT;
    }
}

int sgemm_f32(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda, const float* B,
              int64_t ldb, float* C, int64_t ldc, void* stream) {
    return sgemm_f32_variant(SGEMM_AUTO, M, N, K, A, lda, B, ldb, C, ldc, stream);
}

int sgemm_f32_ex_split(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                       const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                       float* C, int64_t ldc, int splits, void* stream) {
    if (splits < 0 || splits > SGEMM_MAX_SPLITS) return SGEMM_ERR_ARG;
    const int v = validate_ex(transa, transb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0 || alpha == 0.0f) return launch_status(sgemm::launch_scale(C, M, N, ldc, beta, s));
    GemmArgs g{M, N, K, A, lda, B, ldb, C, ldc};
    g.trans_a = transa == SGEMM_OP_T;
    g.trans_b = transb == SGEMM_OP_T;
    g.alpha = alpha;
    g.beta = beta;
    if (sgemm::k4_supports(g)) return launch_status(sgemm::launch_k4_mfma(g, s, splits));
    return launch_status(sgemm::launch_k1_general(g, s));
}

int sgemm_f32_ex_split_noalloc(int transa, int transb, int64_t M, int64_t N, int64_t K,
                               float alpha, const float* A, int64_t lda, const float* B,
                               int64_t ldb, float beta, float* C, int64_t ldc, int splits,
                               void* stream) {
    static_assert(sgemm::kStaticScratchBytes == size_t(SGEMM_STATIC_SCRATCH_BYTES),
                  "header and library agree on the static scratch size");
    if (splits < 0 || splits > SGEMM_MAX_SPLITS) return SGEMM_ERR_ARG;
    const int v = validate_ex(transa, transb, M, N, K, alpha, A, lda, B, ldb, C, ldc);
    if (v != SGEMM_OK) return v;
    if (M == 0 || N == 0) return SGEMM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0 || alpha == 0.0f) return launch_status(sgemm::launch_scale(C, M, N, ldc, beta, s));
    GemmArgs g{M, N, K, A, lda, B, ldb, C, ldc};
    g.trans_a = transa == SGEMM_OP_T;
    g.trans_b = transb == SGEMM_OP_T;
    g.alpha = alpha;
    g.beta = beta;
    if (!sgemm::k4_supports(g)) return launch_status(sgemm::launch_k1_general(g, s));
    // An explicit split whose partial products exceed the scratch is refused
    // before any HIP call.
    if (splits >= 2 && sgemm::k4_split_scratch_bytes(g, splits) > sgemm::kStaticScratchBytes)
        return SGEMM_ERR_SCRATCH;
    sgemm::FixedScratch fs;
    const hipError_t e = sgemm::static_scratch(s, &fs);
    if (e != hipSuccess) return launch_status(e);
    return launch_status(sgemm::launch_k4_mfma(g, s, splits, true, &fs));
}

int sgemm_f32_ex(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                 const float* A, int64_t lda, const float* B, int64_t ldb, float beta, float* C,
                 int64_t ldc, void* stream) {
    return sgemm_f32_ex_split(transa, transb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, 0,
                              stream);
}

int sgemm_f32_colmajor(int transa, int transb, int64_t m, int64_t n, int64_t k, float alpha,
                       const float* A, int64_t lda, const float* B, int64_t ldb, float beta,
                       float* C, int64_t ldc, void* stream) {
    // A column-major m x n matrix read row-major is its transpose, so
    // C = op(A) op(B) (column-major) is C^T = op(B)^T op(A)^T (row-major):
    // the operands swap places and keep their transpose flags.
    return sgemm_f32_ex(transb, transa, n, m, k, alpha, B, ldb, A, lda, beta, C, ldc, stream);
}

int sgemm_auto_variant(int64_t M, int64_t N, int64_t K, const float* A, int64_t lda,
                       const float* B, int64_t ldb, float* C, int64_t ldc) {
    const int v = validate(SGEMM_AUTO, M, N, K, A, lda, B, ldb, C, ldc);
    if (v != SGEMM_OK) return -v;
    const GemmArgs g{M, N, K, A, lda, B, ldb, C, ldc};
    return choose_auto(g);
}

int sgemm_split_plan(int transa, int transb, int64_t M, int64_t N, int64_t K, const float* A,
                     int64_t lda, const float* B, int64_t ldb, int splits, int64_t* kchunk) {
    if (splits < 0 || splits > SGEMM_MAX_SPLITS) return -SGEMM_ERR_ARG;
    const int v = validate_ex_shape(transa, transb, M, N, K, lda, ldb, N > 1 ? N : 1);
    if (v != SGEMM_OK) return -v;
    GemmArgs g{M, N, K, A, lda, B, ldb, nullptr, N > 1 ? N : 1};
    g.trans_a = transa == SGEMM_OP_T;
    g.trans_b = transb == SGEMM_OP_T;
    sgemm::PlanInfo p;
    p.splits = 1;
    p.kchunk = K;
    if (M > 0 && N > 0 && K > 0 && sgemm::k4_supports(g)) p = sgemm::plan_info(g, splits);
    if (kchunk) *kchunk = p.kchunk;
    return p.splits;
}

int sgemm_plan_config(int transa, int transb, int64_t M, int64_t N, int64_t K, const float* A,
                      int64_t lda, const float* B, int64_t ldb, int* engine, int* tile_m,
                      int* tile_n, int* k_groups, int* packed, int64_t* kchunk) {
    const int v = validate_ex_shape(transa, transb, M, N, K, lda, ldb, N > 1 ? N : 1);
    if (v != SGEMM_OK) return -v;
    GemmArgs g{M, N, K, A, lda, B, ldb, nullptr, N > 1 ? N : 1};
    g.trans_a = transa == SGEMM_OP_T;
    g.trans_b = transb == SGEMM_OP_T;
    sgemm::PlanInfo p;
    if (M > 0 && N > 0 && K > 0 && sgemm::k4_supports(g)) p = sgemm::plan_info(g, 0);
    if (engine) *engine = p.engine;
    if (tile_m) *tile_m = p.tile_m;
    if (tile_n) *tile_n = p.tile_n;
    if (k_groups) *k_groups = p.k_groups;
    if (packed) *packed = p.packed ? 1 : 0;
    if (kchunk) *kchunk = p.kchunk;
    return p.splits;
}

int sgemm_copy_f32_launch(float* dst, const float* src, int64_t n, int block, int64_t grid,
                          void* stream) {
    if (n < 0) return SGEMM_ERR_ARG;
    if (block < 64 || block > 1024 || block % 64 != 0) return SGEMM_ERR_ARG;
    if (grid < 1 || grid > sgemm::kMaxCopyGrid) return SGEMM_ERR_ARG;
    if (n == 0) return SGEMM_OK;
    if (dst == nullptr || src == nullptr) return SGEMM_ERR_NULLPTR;
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
    const uintptr_t bytes = uintptr_t(n) * sizeof(float);
    if (overlaps(d, d + bytes, s, s + bytes)) return SGEMM_ERR_ALIAS;
    return launch_status(sgemm::launch_copy(dst, src, n, block, grid,
                                            static_cast<hipStream_t>(stream)));
}

int sgemm_copy_f32(float* dst, const float* src, int64_t n, void* stream) {
    const int block = sgemm::kCopyBlock;
    return sgemm_copy_f32_launch(dst, src, n, block, sgemm::copy_default_grid(n, block), stream);
}

int sgemm_probe_valu_f32(float* out, int64_t blocks, int block, int64_t iters, float x, float y,
                         void* stream) {
    if (blocks < 1 || blocks > sgemm::kMaxGrid) return SGEMM_ERR_ARG;
    if (block < 64 || block > 1024 || block % 64 != 0) return SGEMM_ERR_ARG;
    if (iters < 0) return SGEMM_ERR_ARG;
    if (out == nullptr) return SGEMM_ERR_NULLPTR;
    return launch_status(sgemm::launch_probe_valu(out, iters, x, y, blocks, block,
                                                  static_cast<hipStream_t>(stream)));
}

int sgemm_probe_mfma_f32(float* out, const float* a_vals, const float* b_vals, int64_t blocks,
                         int64_t iters, void* stream) {
    if (blocks < 1 || blocks > sgemm::kMaxGrid) return SGEMM_ERR_ARG;
    if (iters < 0) return SGEMM_ERR_ARG;
    if (out == nullptr || a_vals == nullptr || b_vals == nullptr) return SGEMM_ERR_NULLPTR;
    return launch_status(sgemm::launch_probe_mfma(out, a_vals, b_vals, iters, blocks,
                                                  static_cast<hipStream_t>(stream)));
}

const char* sgemm_status_string(int status) {
    switch (status) {
        case SGEMM_OK: return "ok";
        case SGEMM_ERR_DIM: return "invalid dimension (M, N and K must be >= 0)";
        case SGEMM_ERR_LD: return "invalid leading dimension (lda >= max(1,K), ldb and ldc >= max(1,N))";
        case SGEMM_ERR_NULLPTR: return "null operand pointer";
        case SGEMM_ERR_VARIANT: return "unknown kernel variant";
        case SGEMM_ERR_ALIAS: return "output overlaps an input";
        case SGEMM_ERR_LAUNCH: return "kernel launch failed";
        case SGEMM_ERR_UNSUPPORTED: return "variant cannot address this shape";
        case SGEMM_ERR_ARG: return "invalid argument";
        case SGEMM_ERR_SCRATCH: return "the requested split needs more than the static scratch holds";
        default: return "unknown status";
    }
}

const char* sgemm_variant_name(int variant) {
    switch (variant) {
        case SGEMM_AUTO: return "auto";
        case SGEMM_K1_COALESCED: return "k1_coalesced";
        case SGEMM_K2_LDS_TILED: return "k2_lds_tiled32";
        case SGEMM_K2_LDS_TILED16_PAD1: return "k2_lds_tiled16_pad1";
        case SGEMM_K3_REGTILE_DB: return "k3_regtile_db";
        case SGEMM_K4_MFMA: return "k4_mfma";
        case SGEMM_K2_LDS_TILED16: return "k2_lds_tiled16";
        case SGEMM_K2_LDS_TILED_PAD1: return "k2_lds_tiled32_pad1";
        case SGEMM_K0_NAIVE: return "k0_naive";
        case SGEMM_K4_MFMA_TILE128: return "k4_mfma_tile128";
        case SGEMM_K4_MFMA_TILE64: return "k4_mfma_tile64";
        case SGEMM_K4_MFMA_TILE128X256: return "k4_mfma_tile128x256";
        default: return nullptr;
    }
}

int sgemm_last_hip_error(void) { return g_last_hip_error; }

int sgemm_abi_version(void) { return SGEMM_ABI_VERSION; }

}  // extern "C"
