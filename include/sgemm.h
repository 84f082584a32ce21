/*
 * sgemm.h - C ABI of the MI355X (gfx950) single-precision matrix multiply.
 *
 * Operation (amittech.dev, "3.5 Project: tiled matrix multiplication",
 * sections "the numeric background" and "starter scaffolding"): for
 * row-major float matrices, C = A * B, i.e.
 *
 *     C[i*ldc + j] = sum_{k<K} A[i*lda + k] * B[k*ldb + j],   0<=i<M, 0<=j<N,
 *
 * costing 2*M*N*K floating-point operations.  The page works with square
 * N x N matrices and asks the code to accept any N; this interface takes the
 * general M x K by K x N shape with BLAS-style leading dimensions.  C is
 * overwritten and never read (the course's library call passes alpha = 1 and
 * beta = 0; section "the reference ceiling").  Accumulation is in float.
 *
 * Shapes and layout
 *   M, N, K >= 0.  M == 0 or N == 0: nothing is done and SGEMM_OK returned.
 *   K == 0: C (M x N) is set to zero.
 *   lda >= max(1, K), ldb >= max(1, N), ldc >= max(1, N); elements between a
 *   row's end and the next row's start are neither read (A, B) nor written
 *   (C).  Pointers need only 4-byte alignment; 16-byte alignment with lda,
 *   ldb, K and N multiples of 4 selects wider loads internally.
 *
 * Ownership, memory and synchronisation (per entry point)
 *   A, B and C are device pointers owned by the caller (for example the data
 *   of torch tensors); the library never frees or keeps them.  Every entry
 *   point enqueues its work on ``stream`` (a hipStream_t; NULL means the null
 *   stream) and returns without waiting for that work; a device fault
 *   surfaces at the caller's next synchronisation.
 *
 *   The caller-owns-everything reading of the course's scaffolding (the
 *   harness allocates every buffer) holds for sgemm_f32_variant with the
 *   ladder variants 1-3, 5-8 and 9-11, for the copy and compute probes, and
 *   for sgemm_f32_ex_split_noalloc: they allocate no device memory and never
 *   synchronise.  The shape-chosen paths depart from it in one place, a
 *   library workspace:
 *     - sgemm_f32 and SGEMM_AUTO, SGEMM_K4_MFMA, sgemm_f32_ex,
 *       sgemm_f32_colmajor and sgemm_f32_ex_split use scratch device memory
 *       when their plan (sgemm_plan_config) splits K across workgroups
 *       (partial products), packs unaligned operands into zero-padded
 *       aligned copies first (for example the 3001 x 4099 x 2047 product,
 *       whose packed copies take about 58 MB), or splits a thin product's K;
 *     - that scratch is one buffer per device, allocated stream-ordered from
 *       a memory pool the library creates, on first need, grown on demand
 *       up to 256 MiB and kept until the process ends; a larger request gets
 *       a buffer of its own, freed stream-ordered after its call;
 *     - calls that use it on one device take it in turn (a host lock around
 *       their launches).  While every such call has used one stream, the
 *       stream alone orders them.  The first such call on a second stream
 *       synchronises the whole device once (hipDeviceSynchronize: it must
 *       not coincide with a graph capture on another thread); from then on
 *       a call on another stream than the previous one waits for it on the
 *       GPU through an event;
 *     - if the workspace cannot be allocated, the same product runs without
 *       it (unsplit, unpacked), and so do calls made while ``stream`` is
 *       being captured into a graph.
 *   Every other case of these entry points (products that neither split nor
 *   pack, K == 0, alpha == 0) allocates nothing and never synchronises.
 *
 * Errors
 *   Arguments are validated on the host before any HIP call; a bad argument
 *   returns a nonzero sgemm_status_t and enqueues nothing.  A failed launch
 *   returns SGEMM_ERR_LAUNCH; sgemm_last_hip_error() then gives the HIP error
 *   code of the calling thread's last failure.  The library never exits or
 *   aborts the process.
 */
#ifndef SGEMM_MI355X_H
#define SGEMM_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel ladder.  Every variant computes the same product and accepts every
 * shape the validation above accepts (the SGEMM_K4_MFMA variants excepted,
 * see SGEMM_ERR_UNSUPPORTED); they differ in how they use the chip.  Stages
 * are those of amittech.dev, "3.5 Project: tiled matrix multiplication",
 * section "what we build - the GEMM ladder".  Variants 0-4 are the ladder
 * proper; 5-11 are comparison points. */
typedef enum sgemm_variant {
    SGEMM_AUTO = 0,               /* pick per shape: the SGEMM_K4_MFMA path, or for products with
                                     one side of C at most 8 and a large operand the thin-product
                                     kernels on the vector units (sgemm_plan_config, engine 2);
                                     the register-tiled kernel for shapes beyond the matrix-core
                                     kernel's 32-bit offsets */
    SGEMM_K1_COALESCED = 1,       /* section "stage 1 - global memory coalescing": one output per
                                     lane, the 64 lanes of a wave along a row of C (coalesced B
                                     and C, wave-uniform A) */
    SGEMM_K2_LDS_TILED = 2,       /* section "stage 2 - shared memory tiling": 32 x 32 LDS tiles of
                                     A and B per K step, one output per lane */
    SGEMM_K3_REGTILE_DB = 3,      /* section "what comes next" (register tiling, double
                                     buffering) and qsysarch.com "gemm-kernels", section
                                     "improving the naive multiplier" (several outputs per
                                     thread): 128 x 128 workgroup tile, 8 x 8 outputs per lane in
                                     VGPRs, LDS double buffer */
    SGEMM_K4_MFMA = 4,            /* section "what comes next" (the matrix units): FP32 matrix-core
                                     kernel (v_mfma_f32_32x32x2_f32), direct global->LDS loads;
                                     128 x 256, 128 x 128, 64 x 64 or 32 x 32 workgroup tiles, K
                                     split and operand packing chosen by shape.  Always the
                                     matrix cores (never the thin-product kernels of AUTO) */
    SGEMM_K2_LDS_TILED16 = 5,     /* as K2 with 16 x 16 tiles (the section's TILE = 16 vs 32
                                     comparison, "acceptance criteria") */
    SGEMM_K2_LDS_TILED_PAD1 = 6,  /* as K2 with rows padded by one float (LDS bank comparison) */
    SGEMM_K0_NAIVE = 7,           /* section "stage 0 - the naive baseline": one output per lane,
                                     the lanes of a wave down a column of C (uncoalesced) */
    SGEMM_K2_LDS_TILED16_PAD1 = 8,/* as K2_LDS_TILED16 with rows padded by one float */
    SGEMM_K4_MFMA_TILE128 = 9,    /* K4 with 128 x 128 tiles whatever the shape, unsplit, unpacked */
    SGEMM_K4_MFMA_TILE64 = 10,    /* K4 with 64 x 64 tiles whatever the shape, unsplit, unpacked */
    SGEMM_K4_MFMA_TILE128X256 = 11, /* K4 with 128 x 256 tiles whatever the shape (128 x 128 for
                                     transposed operands without 16-byte loads), unsplit */
    SGEMM_VARIANT_COUNT = 12
} sgemm_variant_t;

typedef enum sgemm_status {
    SGEMM_OK = 0,
    SGEMM_ERR_DIM = 1,         /* a negative M, N or K */
    SGEMM_ERR_LD = 2,          /* lda < max(1,K), ldb < max(1,N) or ldc < max(1,N) */
    SGEMM_ERR_NULLPTR = 3,     /* a NULL operand that the shape requires */
    SGEMM_ERR_VARIANT = 4,     /* unknown variant */
    SGEMM_ERR_ALIAS = 5,       /* C's byte range overlaps A's or B's */
    SGEMM_ERR_LAUNCH = 6,      /* the HIP launch failed (see sgemm_last_hip_error) */
    SGEMM_ERR_UNSUPPORTED = 7, /* the explicit variant cannot index this shape (AUTO always can) */
    SGEMM_ERR_ARG = 8,         /* another invalid argument (copy probe: n < 0, bad block or grid) */
    SGEMM_ERR_SCRATCH = 9      /* sgemm_f32_ex_split_noalloc: the requested K split's partial
                                  products need more than SGEMM_STATIC_SCRATCH_BYTES */
} sgemm_status_t;

/* C = A * B with the variant chosen per shape.  Same as
 * sgemm_f32_variant(SGEMM_AUTO, ...). */
int sgemm_f32(int64_t M, int64_t N, int64_t K,
              const float *A, int64_t lda,
              const float *B, int64_t ldb,
              float *C, int64_t ldc, void *stream);

/* C = A * B with an explicit ladder variant (sgemm_variant_t). */
int sgemm_f32_variant(int variant, int64_t M, int64_t N, int64_t K,
                      const float *A, int64_t lda,
                      const float *B, int64_t ldb,
                      float *C, int64_t ldc, void *stream);

/* Operand orientation for the general entry points. */
typedef enum sgemm_op { SGEMM_OP_N = 0, SGEMM_OP_T = 1 } sgemm_op_t;

/* General form, row-major: C = alpha * op(A) * op(B) + beta * C, with op(A)
 * M x K and op(B) K x N (the BLAS operation of the course's library call in
 * amittech.dev, "3.5 Project: tiled matrix multiplication", section "the
 * reference ceiling", here in row-major storage).
 *   transa == SGEMM_OP_N: A is stored M x K, lda >= max(1, K);
 *   transa == SGEMM_OP_T: A is stored K x M, lda >= max(1, M) (op(A) = A^T);
 *   transb == SGEMM_OP_N: B is stored K x N, ldb >= max(1, N);
 *   transb == SGEMM_OP_T: B is stored N x K, ldb >= max(1, K);
 *   ldc >= max(1, N).
 * beta == 0: C is written without being read (NaN in C does not
 * propagate).  K == 0 or alpha == 0: A and B are not read and C = beta * C.
 * C may be read and written in place; it must not overlap A or B when they
 * are read (SGEMM_ERR_ALIAS).  Other conventions as sgemm_f32; an invalid
 * transa / transb is SGEMM_ERR_ARG. */
int sgemm_f32_ex(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                 const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                 float *C, int64_t ldc, void *stream);

/* sgemm_f32_ex with a K-split request: the small-shape path.  Workgroups
 * are dealt from a queue to compute units with free resources, and the grid
 * size does not by itself occupy the chip (qsysarch.com "gemm-kernels",
 * section "Understanding the naive matrix multiplier"): an output of few
 * 64 x 64 tiles leaves most of the 256 compute units idle however long K is.
 * Split-K cuts K into chunks of whole slabs that run as separate workgroups;
 * each stores its partial product to a workspace of chunks x M rows of N
 * floats (rows rounded up to a multiple of 4),
 * and a second kernel adds the partials in chunk order and applies alpha and
 * beta.  The partial products live in the library workspace (see "Ownership,
 * memory and synchronisation" above); a call made while `stream` is being
 * captured into a graph runs unsplit and unpacked.
 *   splits == 0: chosen by shape (what sgemm_f32 and sgemm_f32_ex do);
 *   splits == 1: never split;
 *   2 <= splits <= SGEMM_MAX_SPLITS: at most that many chunks (fewer when K
 *     has fewer slabs).
 * Other values give SGEMM_ERR_ARG.  Shapes the matrix-core kernel cannot
 * address (32-bit offsets) run unsplit on the 64-bit kernel.  A split result
 * differs from the unsplit one only in the order of the additions (same
 * error bound).  Other arguments and conventions as sgemm_f32_ex. */
#define SGEMM_MAX_SPLITS 64
int sgemm_f32_ex_split(int transa, int transb, int64_t M, int64_t N, int64_t K, float alpha,
                       const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                       float *C, int64_t ldc, int splits, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * operation and arguments as sgemm_f32_ex_split, with the library's static
 * device scratch in place of its workspace.  It calls no allocator and
 * never synchronises, captured or not.
 *   The scratch is a static device array of SGEMM_STATIC_SCRATCH_BYTES that
 *   every device the library runs on holds until the process ends.
 *   splits == 0 or 1: the shape's plan, except that packing, a K split or a
 *   thin product's split runs only when its scratch fits (otherwise the same
 *   product runs unpacked or unsplit, on the matrix cores or the thin
 *   kernels as chosen);
 *   2 <= splits <= SGEMM_MAX_SPLITS: partial products that would exceed the
 *   scratch give SGEMM_ERR_SCRATCH before any HIP call.
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents (nothing in it needs to start at zero); calls that overlap
 * in time on one device (from different streams or threads) race on it, so
 * a caller issues them on one stream or orders them itself. */
#define SGEMM_STATIC_SCRATCH_BYTES (64 * 1024 * 1024)
int sgemm_f32_ex_split_noalloc(int transa, int transb, int64_t M, int64_t N, int64_t K,
                               float alpha, const float *A, int64_t lda, const float *B,
                               int64_t ldb, float beta, float *C, int64_t ldc, int splits,
                               void *stream);

/* The K split sgemm_f32_ex_split(transa, transb, M, N, K, ..., splits, ...)
 * would run with these operands (host-only decision, no HIP call; the
 * pointers enter only through their alignment): the number of K chunks
 * (1 = unsplit), with the chunk length in *kchunk when kchunk is not NULL
 * (the last chunk takes the rest of K); or minus the status code of invalid
 * flags, sizes, leading dimensions or splits (C's leading dimension is taken
 * as max(1, N)). */
int sgemm_split_plan(int transa, int transb, int64_t M, int64_t N, int64_t K,
                     const float *A, int64_t lda, const float *B, int64_t ldb,
                     int splits, int64_t *kchunk);

/* The kernel configuration a shape-chosen call (sgemm_f32, sgemm_f32_ex, or
 * sgemm_f32_ex_split with splits == 0, not under graph capture) runs for
 * these operands: host-only, no HIP call; the pointers enter only through
 * their alignment.  Writes the engine (*engine: 1 = the matrix-core kernel,
 * 2 = the thin-product kernels on the vector units, for M <= 8 or N <= 8
 * when the large operand is 384 MB or more, 256 MB or more for 2 <= N <= 4,
 * or 16 MB or more for N == 1; stored with K contiguous on the other side,
 * 384 MB or more), the
 * workgroup's C tile (*tile_m x *tile_n), the number of K ranges one
 * workgroup splits its work into (*k_groups), whether the operands are
 * first copied into zero-padded aligned rows (*packed, 1 or 0) and the K
 * chunk length (*kchunk); any of these pointers may be NULL.  Returns the
 * number of K chunks across workgroups (1 = unsplit); 0, with the outputs
 * zero, when the call launches neither (an empty product, K == 0, or a
 * shape only the 64-bit kernel can address); or minus the status code of
 * invalid flags, sizes or leading dimensions (C's leading dimension taken
 * as max(1, N)).  Matrix-core tiles are among 128 x 256, 128 x 128, 64 x 64
 * and 32 x 32; which configuration a shape gets follows measurements on
 * MI355X and may change between library versions. */
int sgemm_plan_config(int transa, int transb, int64_t M, int64_t N, int64_t K,
                      const float *A, int64_t lda, const float *B, int64_t ldb, int *engine,
                      int *tile_m, int *tile_n, int *k_groups, int *packed, int64_t *kchunk);

/* The same operation in column-major storage (the BLAS and cuBLAS
 * convention): C (m x n, ldc >= max(1, m)) = alpha * op(A) op(B) + beta * C,
 * op(A) m x k, op(B) k x n; A is m x k (lda >= max(1, m)) or, transposed,
 * k x m (lda >= max(1, k)); B is k x n (ldb >= max(1, k)) or n x k
 * (ldb >= max(1, n)).  Computed as the row-major product
 * C^T = op(B)^T op(A)^T, i.e. sgemm_f32_ex(transb, transa, n, m, k, alpha,
 * B, ldb, A, lda, beta, C, ldc, stream) - the operand swap the course uses
 * to run its row-major product through a column-major library. */
int sgemm_f32_colmajor(int transa, int transb, int64_t m, int64_t n, int64_t k, float alpha,
                       const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                       float *C, int64_t ldc, void *stream);

/* Device-to-device copy dst[i] = src[i], 0 <= i < n, with a grid-stride loop:
 * the HBM bandwidth probe of amittech.dev, "7.3 Bandwidths and peak rate -
 * exercises", exercise 2 (it moves 2 * n * 4 bytes).  dst and src are device
 * pointers owned by the caller and must not overlap (SGEMM_ERR_ALIAS).
 * n == 0 does nothing.  Default launch shape. */
int sgemm_copy_f32(float *dst, const float *src, int64_t n, void *stream);

/* The same copy with an explicit launch shape, for the exercise's block and
 * grid sweep: block is the workgroup size (a multiple of 64, 64..1024), grid
 * the number of workgroups (1..2^22).  Invalid values give SGEMM_ERR_ARG. */
int sgemm_copy_f32_launch(float *dst, const float *src, int64_t n,
                          int block, int64_t grid, void *stream);

/* Compute-roof probes (amittech.dev, "7.3 Bandwidths and peak rate -
 * exercises", exercise 5: register-only multiply-add chains that measure the
 * sustained arithmetic rate).
 *
 * sgemm_probe_valu_f32: blocks x block lanes (block a multiple of 64 in
 * 64..1024, blocks in 1..2^20); lane t runs 32 independent chains, chain j
 * starting at (j + 1) / 16 and updated iters times as acc = fmaf(acc, x, y)
 * with x and y held in vector registers, and writes the 32 final values to
 * out[32 t .. 32 t + 31].  out is a device buffer of blocks * block * 32
 * floats owned by the caller.  Work: blocks * block * iters * 32 * 2 FLOP.
 *
 * sgemm_probe_mfma_f32: blocks workgroups of 4 waves (1..2^20).  Every wave
 * accumulates iters products A * B (A 32 x 2 with A[i][k] = a_vals[i + 32 k],
 * B 2 x 32 with B[k][j] = b_vals[j + 32 k]; a_vals and b_vals are device
 * arrays of 64 floats) into 4 independent 32 x 32 float accumulators with the
 * FP32 matrix instruction, and writes accumulator q of wave w row-major to
 * out[(4 w + q) * 1024 ...].  out holds blocks * 16 * 1024 floats.  Work:
 * blocks * 16 * iters * 4096 FLOP.
 *
 * Both validate their arguments (SGEMM_ERR_ARG, SGEMM_ERR_NULLPTR) before
 * any HIP call and enqueue on stream without synchronising. */
int sgemm_probe_valu_f32(float *out, int64_t blocks, int block, int64_t iters,
                         float x, float y, void *stream);
int sgemm_probe_mfma_f32(float *out, const float *a_vals, const float *b_vals,
                         int64_t blocks, int64_t iters, void *stream);

/* Static description of a status code (never NULL). */
const char *sgemm_status_string(int status);

/* Static name of a variant ("auto", "k1_coalesced", ...), or NULL if unknown. */
const char *sgemm_variant_name(int variant);

/* The variant SGEMM_AUTO would run for this shape and these pointers
 * (host-only decision, no HIP call), or minus the status code when the
 * arguments are invalid. */
int sgemm_auto_variant(int64_t M, int64_t N, int64_t K,
                       const float *A, int64_t lda, const float *B, int64_t ldb,
                       float *C, int64_t ldc);

/* hipError_t of the calling thread's last SGEMM_ERR_LAUNCH (0 if none). */
int sgemm_last_hip_error(void);

/* ABI version of this header (incremented on incompatible change). */
int sgemm_abi_version(void);

#define SGEMM_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* SGEMM_MI355X_H */
