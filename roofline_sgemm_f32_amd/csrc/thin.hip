// Thin products on the vector units: one dimension of C of at most 8.
//
// With M <= 8 (or N <= 8) the product reads the large operand once and does
// at most 16 FLOP per 4-byte element of it, far under the MI355X ridge of
// about 20 FLOP per byte, so the memory roof binds (amittech.dev, "7.3
// Bandwidths and peak rate - exercises", exercises 4 and 6: a kernel's
// intensity against the ridge decides which roof applies), and a 32 x 32
// matrix-core tile would mostly multiply padding.  These kernels stream the
// large operand along its contiguous dimension, one pass, in 16-byte loads
// (4-byte ones, each wave instruction still 256 contiguous bytes, when its
// rows are not whole 16-byte chunks), and keep the small one close:
//  * thin_m (M <= 8, B stored K x N): lane owns 4 columns of C, so a wave's
//    loads of one row of B are 1 KB contiguous; the M values of A a step
//    needs are the same for every lane (scalar loads).  The workgroup's four
//    waves take four consecutive K ranges of the chunk and add their partial
//    columns in wave order through LDS.
//  * thin_n (N <= 8, A stored M x K): a wave owns 4 rows of C and its lanes
//    split K, 4 k per lane per step, UN steps' loads in flight; the
//    workgroup (WAVES waves: 8 with UN 2, or 4 with UN 1 for long A of one or
//    two columns) stages B (K x N or N x K) through LDS, k-major per column,
//    in pieces of 1024 k.  Lane partial sums are added by a fixed butterfly
//    across the wave.
// Both take a K chunk per gridDim.y: with one chunk they write C
// (alpha * sum, then fmaf(beta, C, .) when beta != 0, as every other path);
// with several they write dense partial slabs that a reduction adds in
// chunk order.  Every order is fixed, so a call is bit-reproducible.  With
// tc they store C transposed: the plan runs a product whose large operand
// is stored with K contiguous on the other side as its transpose.
#include <algorithm>

#include "kernels.h"

namespace sgemm {

namespace {
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kThinThreads = 256;   // thin_m: four waves
constexpr int kThinMUnroll = 8;     // rows of B in flight per lane (16 B each)
constexpr int kThinNRows = 4;       // rows of A (and C) per wave in thin_n
constexpr int kThinNPiece = 1024;   // k per LDS piece of B in thin_n

// Store n values of C from a lane, element e at c[e * step]: alpha * v
// (+ beta * C).  step 1 stores a row segment; step ldc stores it into a
// column of C, where a transposed product keeps its result.
__device__ __forceinline__ void store_c(float* c, int64_t step, const float* v, int n, float alpha,
                                        float beta) {
    for (int e = 0; e < n; e++) {
        float r = alpha * v[e];
        if (beta != 0.0f) r = fmaf(beta, c[e * step], r);
        c[e * step] = r;
    }
}
}  // namespace

// out: C (ldo = ldc) when slab == 0, else the workspace, chunk z at
// out + z * slab with ldo = N.  VB: N % 4 == 0 and B's rows 16-byte
// aligned, a lane's four columns consecutive (one 16-byte load per row);
// otherwise they are 64 apart (four 4-byte loads, each wave instruction
// still 256 contiguous bytes) and any N.
template <int MR, bool TA, bool VB>
__global__ void __launch_bounds__(kThinThreads)
thin_m(int N, int K, int kchunk, const float* __restrict__ A, int64_t lda,
       const float* __restrict__ B, int64_t ldb, float* __restrict__ out, int64_t ldo, int64_t slab,
       float alpha, float beta, bool tc) {
    __shared__ v4f red[3][64][MR];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    // Column of the lane's component e.
    auto col = [&](int e) { return VB ? (blockIdx.x * 64 + lane) * 4 + e : blockIdx.x * 256 + lane + 64 * e; };
    auto load_row = [&](const float* rowp) -> v4f {
        if constexpr (VB) {
            return __builtin_nontemporal_load(reinterpret_cast<const v4f*>(rowp + col(0)));
        } else {
            v4f b;
#pragma unroll
            for (int e = 0; e < 4; e++) b[e] = col(e) < N ? __builtin_nontemporal_load(rowp + col(e)) : 0.0f;
            return b;
        }
    };
    const int z = blockIdx.y;
    const int kc0 = z * kchunk, kc1 = min(K, kc0 + kchunk);
    // Wave w takes the w-th quarter of the chunk.
    const int q = (kc1 - kc0 + 3) / 4;
    const int k0 = min(kc1, kc0 + w * q), k1 = min(kc1, k0 + q);
    v4f acc[MR];
#pragma unroll
    for (int m = 0; m < MR; m++) acc[m] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    if (col(0) < N) {
        const float* bp = B + (int64_t)k0 * ldb;
        int k = k0;
        for (; k + kThinMUnroll <= k1; k += kThinMUnroll) {
            v4f b[kThinMUnroll];
#pragma unroll
            for (int u = 0; u < kThinMUnroll; u++) b[u] = load_row(bp + (int64_t)u * ldb);
#pragma unroll
            for (int u = 0; u < kThinMUnroll; u++)
#pragma unroll
                for (int m = 0; m < MR; m++) {
                    const float a = TA ? A[(int64_t)(k + u) * lda + m] : A[(int64_t)m * lda + k + u];
                    acc[m] += a * b[u];
                }
            bp += (int64_t)kThinMUnroll * ldb;
        }
        for (; k < k1; k++, bp += ldb) {
            const v4f b = load_row(bp);
#pragma unroll
            for (int m = 0; m < MR; m++) {
                const float a = TA ? A[(int64_t)k * lda + m] : A[(int64_t)m * lda + k];
                acc[m] += a * b;
            }
        }
    }
    // Waves 1..3 hand their partial columns to wave 0, which adds them in
    // wave (= k) order.
    if (w > 0) {
#pragma unroll
        for (int m = 0; m < MR; m++) red[w - 1][lane][m] = acc[m];
    }
    __syncthreads();
    if (w > 0 || col(0) >= N) return;
#pragma unroll
    for (int v = 0; v < 3; v++)
#pragma unroll
        for (int m = 0; m < MR; m++) acc[m] += red[v][lane][m];
    if (slab) {
        float* o = out + (int64_t)z * slab;
#pragma unroll
        for (int m = 0; m < MR; m++) {
            if constexpr (VB) {
                *reinterpret_cast<v4f*>(o + (int64_t)m * ldo + col(0)) = acc[m];
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++)
                    if (col(e) < N) o[(int64_t)m * ldo + col(e)] = acc[m][e];
            }
        }
    } else {
#pragma unroll
        for (int m = 0; m < MR; m++) {
            if constexpr (VB) {
                const float v[4] = {acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
                if (tc)
                    store_c(out + (int64_t)col(0) * ldo + m, ldo, v, 4, alpha, beta);
                else
                    store_c(out + (int64_t)m * ldo + col(0), 1, v, 4, alpha, beta);
            } else {
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    if (col(e) >= N) break;
                    const float v = acc[m][e];
                    store_c(tc ? out + (int64_t)col(e) * ldo + m : out + (int64_t)m * ldo + col(e), 1, &v, 1,
                            alpha, beta);
                }
            }
        }
    }
}

// out as in thin_m (ldo = ldc, or N for the workspace).  VA: K % 4 == 0 and
// A's rows 16-byte aligned (16-byte loads); otherwise 4-byte loads.  B
// element (k, n) is B[k * ldb + n], or B[n * ldb + k] when TB.
template <int NR, bool TB, int WAVES, int UN, bool VA>
__global__ void __launch_bounds__(64 * WAVES)
thin_n(int M, int K, int kchunk, const float* __restrict__ A, int64_t lda,
       const float* __restrict__ B, int64_t ldb, float* __restrict__ out, int64_t ldo, int64_t slab,
       float alpha, float beta, bool tc) {
    // B piece, k-major per column; the pad keeps the 16-byte reads of one
    // column's k run conflict-free across columns.
    __shared__ __attribute__((aligned(16))) float bs[NR][kThinNPiece + 4];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int row0 = (blockIdx.x * WAVES + w) * kThinNRows;
    const int z = blockIdx.y;
    const int k0 = z * kchunk, k1 = min(K, k0 + kchunk);
    float acc[kThinNRows][NR];
#pragma unroll
    for (int r = 0; r < kThinNRows; r++)
#pragma unroll
        for (int n = 0; n < NR; n++) acc[r][n] = 0.0f;
    const float* ap[kThinNRows];
    bool live[kThinNRows];
#pragma unroll
    for (int r = 0; r < kThinNRows; r++) {
        live[r] = row0 + r < M;
        ap[r] = A + (int64_t)(live[r] ? row0 + r : 0) * lda;
    }
    for (int p0 = k0; p0 < k1; p0 += kThinNPiece) {
        const int pk = min(kThinNPiece, k1 - p0);
        __syncthreads();  // the previous piece is consumed
        for (int i = threadIdx.x; i < pk * NR; i += 64 * WAVES) {
            const int k = TB ? i % pk : i / NR, n = TB ? i / pk : i % NR;
            bs[n][k] = TB ? B[(int64_t)n * ldb + p0 + k] : B[(int64_t)(p0 + k) * ldb + n];
        }
        __syncthreads();
        if constexpr (!VA) {
            // Rows of A not in 16-byte chunks: 4-byte loads, lane takes
            // k = p0 + lane + 64 q + 256 t (q < 4), each load 256 contiguous
            // bytes across the wave; any pk.
            for (int kb = 0; kb < pk; kb += 256 * UN) {
                float a[UN][kThinNRows][4];
#pragma unroll
                for (int u = 0; u < UN; u++)
#pragma unroll
                    for (int q = 0; q < 4; q++) {
                        const int kk = kb + 256 * u + 64 * q + lane;
#pragma unroll
                        for (int r = 0; r < kThinNRows; r++)
                            a[u][r][q] = live[r] && kk < pk ? __builtin_nontemporal_load(ap[r] + p0 + kk) : 0.0f;
                    }
#pragma unroll
                for (int u = 0; u < UN; u++) {
                    const int kk = kb + 256 * u + lane;
#pragma unroll
                    for (int n = 0; n < NR; n++) {
                        float b[4];
#pragma unroll
                        for (int q = 0; q < 4; q++) b[q] = kk + 64 * q < pk ? bs[n][kk + 64 * q] : 0.0f;
#pragma unroll
                        for (int r = 0; r < kThinNRows; r++)
                            acc[r][n] += a[u][r][0] * b[0] + a[u][r][1] * b[1] + a[u][r][2] * b[2] + a[u][r][3] * b[3];
                    }
                }
            }
            continue;
        }
        // Lane takes k = p0 + 4 lane + 256 t, UN steps t per batch with all
        // their loads issued first.  pk is a multiple of 4.
        for (int kb = 0; kb < pk; kb += 256 * UN) {
            v4f a[UN][kThinNRows];
#pragma unroll
            for (int u = 0; u < UN; u++) {
                const int kk = kb + 256 * u + 4 * lane;
#pragma unroll
                for (int r = 0; r < kThinNRows; r++)
                    a[u][r] = live[r] && kk < pk
                                  ? __builtin_nontemporal_load(reinterpret_cast<const v4f*>(ap[r] + p0 + kk))
                                  : v4f{0.0f, 0.0f, 0.0f, 0.0f};
            }
#pragma unroll
            for (int u = 0; u < UN; u++) {
                const int kk = kb + 256 * u + 4 * lane;
                if (kk >= pk) continue;
#pragma unroll
                for (int n = 0; n < NR; n++) {
                    const v4f b = *reinterpret_cast<const v4f*>(&bs[n][kk]);
#pragma unroll
                    for (int r = 0; r < kThinNRows; r++)
                        acc[r][n] += a[u][r][0] * b[0] + a[u][r][1] * b[1] + a[u][r][2] * b[2] + a[u][r][3] * b[3];
                }
            }
        }
    }
    // Butterfly over the wave: afterwards every lane holds the sums.
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1)
#pragma unroll
        for (int r = 0; r < kThinNRows; r++)
#pragma unroll
            for (int n = 0; n < NR; n++) acc[r][n] += __shfl_xor(acc[r][n], d, 64);
    // Lane r writes row row0 + r.
#pragma unroll
    for (int r = 0; r < kThinNRows; r++) {
        if (lane != r || !live[r]) continue;
        if (slab) {
            float* o = out + (int64_t)z * slab + (int64_t)(row0 + r) * ldo;
#pragma unroll
            for (int n = 0; n < NR; n++) o[n] = acc[r][n];
        } else {
            if (tc)
                store_c(out + (row0 + r), ldo, acc[r], NR, alpha, beta);
            else
                store_c(out + (int64_t)(row0 + r) * ldo, 1, acc[r], NR, alpha, beta);
        }
    }
}

namespace {
template <int MR>
hipError_t launch_thin_m_r(const GemmArgs& g, int splits, int kchunk, float* ws, bool tc, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(g.N, 256), (unsigned)splits);
    float* out = splits > 1 ? ws : g.C;
    const int64_t ldo = splits > 1 ? g.N : g.ldc, slab = splits > 1 ? g.M * g.N : 0;
    const bool vb = rows_vec(g.B, g.ldb, g.N);
    if (g.trans_a && vb)
        hipLaunchKernelGGL((thin_m<MR, true, true>), grid, dim3(kThinThreads), 0, s, (int)g.N, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
    else if (vb)
        hipLaunchKernelGGL((thin_m<MR, false, true>), grid, dim3(kThinThreads), 0, s, (int)g.N, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
    else if (g.trans_a)
        hipLaunchKernelGGL((thin_m<MR, true, false>), grid, dim3(kThinThreads), 0, s, (int)g.N, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
    else
        hipLaunchKernelGGL((thin_m<MR, false, false>), grid, dim3(kThinThreads), 0, s, (int)g.N, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
    return hipGetLastError();
}

template <int NR, int WAVES, int UN>
void launch_thin_n_w(const GemmArgs& g, int splits, int kchunk, float* ws, bool tc, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(g.M, WAVES * kThinNRows), (unsigned)splits);
    float* out = splits > 1 ? ws : g.C;
    const int64_t ldo = splits > 1 ? g.N : g.ldc, slab = splits > 1 ? g.M * g.N : 0;
    const bool va = rows_vec(g.A, g.lda, g.K);
    if (g.trans_b && va)
        hipLaunchKernelGGL((thin_n<NR, true, WAVES, UN, true>), grid, dim3(64 * WAVES), 0, s, (int)g.M, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
    else if (va)
        hipLaunchKernelGGL((thin_n<NR, false, WAVES, UN, true>), grid, dim3(64 * WAVES), 0, s, (int)g.M, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
    else if (g.trans_b)
        hipLaunchKernelGGL((thin_n<NR, true, WAVES, UN, false>), grid, dim3(64 * WAVES), 0, s, (int)g.M, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
    else
        hipLaunchKernelGGL((thin_n<NR, false, WAVES, UN, false>), grid, dim3(64 * WAVES), 0, s, (int)g.M, (int)g.K,
                           kchunk, g.A, g.lda, g.B, g.ldb, out, ldo, slab, g.alpha, g.beta, tc);
}

template <int NR>
hipError_t launch_thin_n_r(const GemmArgs& g, const ThinPlan& p, float* ws, hipStream_t s) {
    if constexpr (NR <= 2) {
        if (p.waves == 4) {
            launch_thin_n_w<NR, 4, 1>(g, p.splits, (int)p.kchunk, ws, p.swap, s);
            return hipGetLastError();
        }
    }
    if (p.waves != 8) return hipErrorInvalidValue;
    launch_thin_n_w<NR, 8, 2>(g, p.splits, (int)p.kchunk, ws, p.swap, s);
    return hipGetLastError();
}

// Split reduction of a transposed thin product: the partial slabs hold the
// M x N product dense (M x N of the transposed problem), and element (r, j)
// of their sum goes to C[j * ldc + r]; lanes run along r, so C is written
// in runs of consecutive floats.  Slabs are added in order, alpha and beta
// applied as in splitk_reduce.
__global__ void __launch_bounds__(256)
thin_reduce_t(int M, int N, int S, const float* __restrict__ W, float* __restrict__ C, int64_t ldc,
              float alpha, float beta) {
    const int64_t total = (int64_t)M * N, slab = total;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t j = i / M, r = i % M;
        const float* w = W + r * N + j;
        float sum = w[0];
        for (int z = 1; z < S; z++) sum += w[z * slab];
        float v = alpha * sum;
        float* c = C + j * ldc + r;
        if (beta != 0.0f) v = fmaf(beta, *c, v);
        *c = v;
    }
}
}  // namespace

hipError_t launch_thin(const GemmArgs& g0, const ThinPlan& p, float* ws, hipStream_t s) {
    // A swapped plan runs the transposed product, stored transposed.
    const GemmArgs g = p.swap ? swapped(g0) : g0;
    hipError_t e;
    if (p.kind == ThinPlan::THIN_M) {
        switch (g.M) {
            case 1: e = launch_thin_m_r<1>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            case 2: e = launch_thin_m_r<2>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            case 3: e = launch_thin_m_r<3>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            case 4: e = launch_thin_m_r<4>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            case 5: e = launch_thin_m_r<5>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            case 6: e = launch_thin_m_r<6>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            case 7: e = launch_thin_m_r<7>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            case 8: e = launch_thin_m_r<8>(g, p.splits, (int)p.kchunk, ws, p.swap, s); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (g.N) {
            case 1: e = launch_thin_n_r<1>(g, p, ws, s); break;
            case 2: e = launch_thin_n_r<2>(g, p, ws, s); break;
            case 3: e = launch_thin_n_r<3>(g, p, ws, s); break;
            case 4: e = launch_thin_n_r<4>(g, p, ws, s); break;
            case 5: e = launch_thin_n_r<5>(g, p, ws, s); break;
            case 6: e = launch_thin_n_r<6>(g, p, ws, s); break;
            case 7: e = launch_thin_n_r<7>(g, p, ws, s); break;
            case 8: e = launch_thin_n_r<8>(g, p, ws, s); break;
            default: return hipErrorInvalidValue;
        }
    }
    if (e != hipSuccess || p.splits <= 1) return e;
    if (!p.swap) return launch_splitk_reduce(g, p.splits, ws, g.N, s);
    const int64_t total = g.M * g.N;
    hipLaunchKernelGGL(thin_reduce_t, dim3(grid_for(ceil_div(total, 256))), dim3(256), 0, s, (int)g.M,
                       (int)g.N, p.splits, ws, g.C, g.ldc, g.alpha, g.beta);
    return hipGetLastError();
}

}  // namespace sgemm
