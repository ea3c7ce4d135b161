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

// one workgroup: every id is checked before any is copied, so a rejected input changes nothing
__global__ __launch_bounds__(256) void k_set_input(int* __restrict__ d, const int* __restrict__ s, int rows, int cols,
                                                   long long stride, int lim0, int lim1, uint32_t* err)
{
    __shared__ int bad;
    if (threadIdx.x == 0) bad = (int)*err;
    __syncthreads();
    const int n = rows * cols;
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int r = i / cols, c = i - r * cols;
        const int v = s[r * stride + c];
        if (v < 0 || v >= (c == 0 ? lim0 : lim1)) atomicOr(&bad, 2);
    }
    __syncthreads();
    if (bad) {
        if (threadIdx.x == 0 && (bad & 2)) *err = 1u;
        return;
    }
    for (int i = threadIdx.x; i < n; i += blockDim.x) {
        const int r = i / cols, c = i - r * cols;
        d[i] = s[r * stride + c];
    }
}
__global__ void k_check_ids(const int* __restrict__ s, long long n, int cols, int lim0, int lim1, uint32_t* err)
{
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const int c = (int)(i % cols), v = s[i];
    if (v < 0 || v >= (c == 0 ? lim0 : lim1)) *err = 1u;
}
__global__ void k_set_pos(int* pos, int v, const uint32_t* err)
{
    if (threadIdx.x == 0 && *err == 0u) *pos = v;
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
hipError_t launch_set_input(int* dst, const int* src, int rows, int cols, long long src_stride, int lim0, int lim1,
                            uint32_t* err, hipStream_t st)
{
    if (rows * cols <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_set_input, dim3(1), dim3(256), 0, st, dst, src, rows, cols, src_stride, lim0, lim1, err);
    return hipGetLastError();
}
hipError_t launch_check_ids(const int* src, int rows, int n, int cols, int lim0, int lim1, uint32_t* err, hipStream_t st)
{
    const long long total = (long long)rows * n * cols;
    if (total <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_check_ids, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, src, total, cols, lim0, lim1,
                       err);
    return hipGetLastError();
}
hipError_t launch_set_pos(int* pos, int value, const uint32_t* err, hipStream_t st)
{
    hipLaunchKernelGGL(k_set_pos, dim3(1), dim3(64), 0, st, pos, value, err);
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
