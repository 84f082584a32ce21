// Compute-roof probes: how fast can the chip retire FP32 multiply-adds when
// nothing else is in the way?
//
// amittech.dev, "7.3 Bandwidths and peak rate - exercises", exercise 5: each
// lane runs long register-only chains acc = acc * x + y over several
// independent accumulators, enough lanes to fill the machine, and the FLOP
// count is lanes x iterations x chains x 2.  probe_valu is that kernel
// with 32 chains per lane, plain (unpacked) v_fma_f32.  Its multiplier and
// addend are held in vector registers: with one of them a scalar operand,
// as a kernel argument would naturally be, the same chains retire at about
// half the rate (72 against 129 TFLOP/s on MI355X at 32 waves per CU), so
// a probe in that form measures the operand path, not the vector ALU's
// roof.
//
// probe_mfma is the same question for the matrix cores: every wave issues
// back-to-back v_mfma_f32_32x32x2_f32 into 4 independent 32 x 32
// accumulators (2 x 32 x 32 x 2 FLOP each).  The A and B operand values come
// from memory (lane L supplies A[L%32][L/32] and B[L/32][L%32]), and every
// wave writes its four accumulators back as row-major 32 x 32 matrices, using
// the same register-to-(row, column) map as the matrix-core SGEMM: register r
// of lane L is row 8*(r/4) + 4*(L/32) + r%4, column L%32.  The output is
// therefore also a check of that map.
#include "kernels.h"

namespace sgemm {

namespace {
typedef float v16f __attribute__((ext_vector_type(16)));
constexpr int kValuChains = 32;
constexpr int kMfmaAcc = 4;
}  // namespace

__global__ void __launch_bounds__(1024)
probe_valu(float* __restrict__ out, int64_t iters, float x, float y) {
    // Move x and y into vector registers (the empty asm takes them as VGPR
    // operands, so the multiply-adds below read VGPRs only).
    float xv = x, yv = y;
    asm volatile("" : "+v"(xv), "+v"(yv));
    float acc[kValuChains];
#pragma unroll
    for (int j = 0; j < kValuChains; j++) acc[j] = 0.0625f * (float)(j + 1);
    for (int64_t i = 0; i < iters; i++) {
#pragma unroll
        for (int j = 0; j < kValuChains; j++) acc[j] = fmaf(acc[j], xv, yv);
    }
    const int64_t lane = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
    for (int j = 0; j < kValuChains; j++) out[lane * kValuChains + j] = acc[j];
}

__global__ void __launch_bounds__(256)
probe_mfma(float* __restrict__ out, const float* __restrict__ a_vals,
           const float* __restrict__ b_vals, int64_t iters) {
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const float a = a_vals[lane], b = b_vals[lane];
    v16f acc[kMfmaAcc];
#pragma unroll
    for (int q = 0; q < kMfmaAcc; q++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[q][r] = 0.0f;
    for (int64_t i = 0; i < iters; i++) {
#pragma unroll
        for (int q = 0; q < kMfmaAcc; q++)
            acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[q], 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < kMfmaAcc; q++) {
        float* o = out + (wave * kMfmaAcc + q) * 1024;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const int row = (r / 4) * 8 + (lane / 32) * 4 + (r % 4), col = lane % 32;
            o[row * 32 + col] = acc[q][r];
        }
    }
}

hipError_t launch_probe_valu(float* out, int64_t iters, float x, float y, int64_t blocks, int block,
                             hipStream_t s) {
    hipLaunchKernelGGL(probe_valu, dim3((unsigned)blocks), dim3(block), 0, s, out, iters, x, y);
    return hipGetLastError();
}

hipError_t launch_probe_mfma(float* out, const float* a_vals, const float* b_vals, int64_t iters,
                             int64_t blocks, hipStream_t s) {
    hipLaunchKernelGGL(probe_mfma, dim3((unsigned)blocks), dim3(256), 0, s, out, a_vals, b_vals,
                       iters);
    return hipGetLastError();
}

}  // namespace sgemm
