// Stream-read calibration: the practical HBM read ceiling for a given byte
// count and launch shape, measured with the same load instruction the GEMV
// streams its weights with (128-bit, non-temporal). Every 16-byte granule of
// the buffer is read exactly once; each wave owns one contiguous chunk and
// keeps L loads of 1 KiB (64 lanes x 16 bytes) in flight, issued before any
// of them is consumed. The loaded words are folded with exclusive-or into
// one word per lane, written to `out` so the loads cannot be removed.
#include "wq_internal.h"

namespace wq {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int L>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, long n16, long per_wave,
                                                          uint32_t *__restrict__ out) {
    const long wave = (long)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const long begin = wave * per_wave;                 // granules
    const long end = begin + per_wave < n16 ? begin + per_wave : n16;
    uint32_t acc = 0;
    long g = begin;
    for (; g + 64L * L <= end; g += 64L * L) {
        u32x4 v[L];
#pragma unroll
        for (int j = 0; j < L; ++j) v[j] = __builtin_nontemporal_load(p + g + 64L * j + lane);
#pragma unroll
        for (int j = 0; j < L; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
    }
    for (; g + lane < end; g += 64) {  // tail of the chunk, one 1 KiB step at a time
        const u32x4 v = __builtin_nontemporal_load(p + g + lane);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    out[wave * 64 + lane] = acc;
}

} // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, int waves, int loads, uint32_t *out, hipStream_t st) {
    const long n16 = (long)(bytes / 16);
    const long per_wave = (n16 + waves - 1) / waves;
    const dim3 grid((unsigned)(waves / 4)), block(256);
    const u32x4 *p = reinterpret_cast<const u32x4 *>(buf);
    switch (loads) {
#define WQ_SR(L)                                                                              \
    case L:                                                                                   \
        hipLaunchKernelGGL(stream_read_kernel<L>, grid, block, 0, st, p, n16, per_wave, out); \
        break;
        WQ_SR(1) WQ_SR(2) WQ_SR(4) WQ_SR(5) WQ_SR(8) WQ_SR(9) WQ_SR(12) WQ_SR(16) WQ_SR(18) WQ_SR(24) WQ_SR(36)
#undef WQ_SR
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace wq
