// HBM bandwidth probe and the K == 0 fill.
//
// The copy follows amittech.dev, "7.3 Bandwidths and peak rate - exercises",
// exercise 2: out[i] = in[i] with a grid-stride loop, so that any launch
// shape covers any length; its traffic is one read and one write of each
// element.  When both pointers are 16-byte aligned each lane moves float4
// vectors and the last n % 4 elements are copied singly; otherwise every
// element is copied singly.
//
// Shape measured on MI355X (2 GiB per copy): one-wave workgroups with one
// float4 per lane per trip and non-temporal loads and stores (streamed past
// the caches, since nothing is reused) sustain 6.7 TB/s; grid-stride loops
// over a few thousand 256-lane workgroups stay near 4.5-5 TB/s, and lanes
// that each own several consecutive vectors fall to 1-2.5 TB/s.
#include "kernels.h"

namespace sgemm {

namespace {
typedef float v4f __attribute__((ext_vector_type(4)));
}

__global__ void copy_vec4(v4f* __restrict__ dst, const v4f* __restrict__ src, int64_t n4,
                          float* __restrict__ dtail, const float* __restrict__ stail, int tail) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
    if (blockIdx.x == 0 && (int)threadIdx.x < tail) dtail[threadIdx.x] = stail[threadIdx.x];
}

__global__ void copy_scalar(float* __restrict__ dst, const float* __restrict__ src, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

__global__ void fill_zero(float* __restrict__ C, int64_t M, int64_t N, int64_t ldc) {
    const int64_t total = M * N, stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride)
        C[(i / N) * ldc + (i % N)] = 0.0f;
}

int64_t copy_default_grid(int64_t n, int block) {
    // One trip per lane when the grid allows it (see the measurement above);
    // longer arrays loop.
    const int64_t want = ceil_div(n / 4 + 1, block);
    return want < kMaxCopyGrid ? want : kMaxCopyGrid;
}

hipError_t launch_copy(float* dst, const float* src, int64_t n, int block, int64_t grid,
                       hipStream_t s) {
    const bool vec = reinterpret_cast<uintptr_t>(dst) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(src) % 16 == 0;
    if (vec) {
        const int64_t n4 = n / 4;
        const int tail = int(n - n4 * 4);
        hipLaunchKernelGGL(copy_vec4, dim3((unsigned)grid), dim3(block), 0, s,
                           reinterpret_cast<v4f*>(dst), reinterpret_cast<const v4f*>(src), n4,
                           dst + n4 * 4, src + n4 * 4, tail);
    } else {
        hipLaunchKernelGGL(copy_scalar, dim3((unsigned)grid), dim3(block), 0, s, dst, src, n);
    }
    return hipGetLastError();
}

hipError_t launch_zero(float* C, int64_t M, int64_t N, int64_t ldc, hipStream_t s) {
    const int64_t grid = ceil_div(M * N, 256);
    hipLaunchKernelGGL(fill_zero, dim3(grid_for(grid)), dim3(256), 0, s, C, M, N, ldc);
    return hipGetLastError();
}

}  // namespace sgemm
