// misc.hip — small state kernels (token slots, counters, fills).  Plain fill kernels are used
// instead of memset nodes so that everything the step does can be captured into a graph.
#include "kernels.h"

namespace tsd {
namespace {

__global__ void k_copy_i32(int* __restrict__ d, const int* __restrict__ s, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) d[i] = s[i];
}
template <class T>
__global__ void k_fill(T* d, T v, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) d[i] = v;
}
__global__ void k_gather_i32(int* __restrict__ d, const int* __restrict__ s, int rows, int cols, long long stride)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * cols) return;
    const int r = i / cols, c = i - r * cols;
    d[i] = s[r * stride + c];
}
__global__ void k_copy_bytes(uint8_t* __restrict__ d, const uint8_t* __restrict__ s, size_t n)
{
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) d[i] = s[i];
}

template <class T>
hipError_t fill(T* d, T v, size_t n, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    const size_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_fill<T>, dim3((unsigned)blocks), dim3(256), 0, st, d, v, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_copy_i32(int* dst, const int* src, int n, hipStream_t st)
{
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_copy_i32, dim3((n + 255) / 256), dim3(256), 0, st, dst, src, n);
    return hipGetLastError();
}
hipError_t launch_gather_i32(int* dst, const int* src, int rows, int cols, long long src_stride, hipStream_t st)
{
    const int n = rows * cols;
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_gather_i32, dim3((n + 255) / 256), dim3(256), 0, st, dst, src, rows, cols, src_stride);
    return hipGetLastError();
}
hipError_t launch_fill_i32(int* d, int v, int n, hipStream_t st) { return fill<int>(d, v, (size_t)n, st); }
hipError_t launch_fill_u32(unsigned int* d, unsigned int v, int n, hipStream_t st) { return fill<unsigned int>(d, v, (size_t)n, st); }
hipError_t launch_fill_u64(unsigned long long* d, unsigned long long v, int n, hipStream_t st)
{
    return fill<unsigned long long>(d, v, (size_t)n, st);
}
hipError_t launch_fill_f32(float* d, float v, size_t n, hipStream_t st) { return fill<float>(d, v, n, st); }
hipError_t launch_copy_bytes(void* dst, const void* src, size_t n, hipStream_t st)
{
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_copy_bytes, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (uint8_t*)dst,
                       (const uint8_t*)src, n);
    return hipGetLastError();
}

}  // namespace tsd
