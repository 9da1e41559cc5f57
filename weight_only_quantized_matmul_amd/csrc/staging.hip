// Kernel copies for the host-pointer calls (staging.h): a call's activations
// (tens of KiB to a few MiB) reach the device, and its outputs come back,
// through pinned host buffers mapped into the device's address space, read
// or written by these kernels over the bus, in place of two DMA transfers
// whose set-up latency is larger than the copy itself at these sizes.
#include "staging.h"

#include <algorithm>

namespace wq {
namespace {

__global__ __launch_bounds__(256) void stage_copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst,
                                                         size_t n4, const float *__restrict__ src_tail,
                                                         float *__restrict__ dst_tail, int tail) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride) dst[i] = src[i];
    if (blockIdx.x == 0 && (int)threadIdx.x < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

} // namespace

hipError_t launch_stage_copy(const float *src, float *dst, size_t n, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const size_t n4 = n / 4;
    const int tail = (int)(n - 4 * n4);
    const unsigned grid = (unsigned)std::max<size_t>(1, std::min<size_t>((n4 + 255) / 256, 1024));
    hipLaunchKernelGGL(stage_copy_kernel, dim3(grid), dim3(256), 0, st, reinterpret_cast<const float4 *>(src),
                       reinterpret_cast<float4 *>(dst), n4, src + 4 * n4, dst + 4 * n4, tail);
    return hipGetLastError();
}

} // namespace wq
