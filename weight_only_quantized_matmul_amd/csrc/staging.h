// Copies between the host-pointer calls' pinned, device-mapped staging
// buffers and device memory, done by a kernel on the call's stream.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>

namespace wq {

// dst[i] = src[i] for i < n; src and dst 16-byte aligned (either may be the
// device address of pinned host memory).
hipError_t launch_stage_copy(const float *src, float *dst, size_t n, hipStream_t st);

} // namespace wq
