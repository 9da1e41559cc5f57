// LDS-tiled dequant + fp32 MFMA path for S beyond the register GEMV.
//
// y[s,o] = scale[o] * sum_i dequant(W[o,i]) * x[s,i]
//   (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四, qmatmul.comp
//    header; dequant rules from colibri-analysis "CUDA 后端", section 1,
//    weight_at; batched rows moving to matrix units once there are enough of
//    them: colibri docs "CUDA backend (Linux)", section "The GPU-resident
//    pipeline")
//
// With many activation rows the work is a dense [S x I] * [I x O]
// contraction, so it runs on the matrix cores:
//  * a 256-thread block owns a 64 (s) x 64 (o) output tile; its four waves
//    each own a 32 x 32 quarter made of 2 x 2 v_mfma_f32_16x16x4_f32 tiles;
//  * the contraction runs over the weight fields in device order (see the
//    layout in wq_internal.h); per 32-position K step the block stages the
//    matching activations (gathered as runs of four consecutive elements)
//    and the weight tile, dequantized once to exact fp32 values, in LDS
//    (double-buffered, rows padded by 4 floats so a 16-lane row group reads
//    16 distinct banks);
//  * within a 16-column group lane group g = lane/16 reads columns
//    4g..4g+3 with one 128-bit LDS read and feeds them to four MFMAs, so each
//    MFMA sees one column per lane group; A and B use the same column order;
//  * the per-row scale is applied in the epilogue, after the sum;
//  * tiles are handed out XCD by XCD (blocks are dispatched round-robin over
//    the 8 XCDs), consecutive tiles of one XCD sharing a weight tile so it is
//    fetched into that XCD's L2 once.
#include "wq_internal.h"

namespace wq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 64, BN = 64, BK = 32, LDK = BK + 4;

// Weight bytes covering 8 consecutive elements, dequantized to exact floats.
template <int FMT>
__device__ __forceinline__ void load_w8(const uint8_t *__restrict__ row, long stride, long k0, float (&q)[8]) {
    if constexpr (FMT == WQ_F32) {
        const long bo = k0 * 4;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (bo + 16 * h < stride) v = *reinterpret_cast<const u32x4 *>(row + bo + 16 * h);
            q[4 * h + 0] = __uint_as_float(v.x);
            q[4 * h + 1] = __uint_as_float(v.y);
            q[4 * h + 2] = __uint_as_float(v.z);
            q[4 * h + 3] = __uint_as_float(v.w);
        }
    } else if constexpr (FMT == WQ_I8) {
        u32x2 v = {0u, 0u};
        if (k0 < stride) v = *reinterpret_cast<const u32x2 *>(row + k0);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)(int)(int8_t)((e < 4 ? v.x : v.y) >> (8 * (e & 3)));
    } else if constexpr (FMT == WQ_I4) {
        const long bo = k0 / 2;
        uint32_t v = 0x88888888u;
        if (bo < stride) v = *reinterpret_cast<const uint32_t *>(row + bo);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)((int)((v >> (4 * e)) & 0xFu) - 8);
    } else {
        const long bo = k0 / 4;
        uint32_t v = 0xAAAAu;
        if (bo < stride) v = *reinterpret_cast<const uint16_t *>(row + bo);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)((int)((v >> (2 * e)) & 0x3u) - 2);
    }
}

// Activations for the 8 field positions [P0, P0 + 8) of a row (two runs of
// four consecutive elements, located through the device layout).
template <int FMT>
__device__ __forceinline__ void load_x8(const float *__restrict__ x, int S, int I, int nfull, bool vec_ok, int s,
                                        long P0, float (&v)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    if (s >= S) return;
    const float *xs = x + (long)s * I;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const long e0 = elem_of_pos4(FMT, P0 + 4 * h, nfull);
        if (vec_ok && e0 + 4 <= I) {
            const float4 a = *reinterpret_cast<const float4 *>(xs + e0);
            v[4 * h] = a.x; v[4 * h + 1] = a.y; v[4 * h + 2] = a.z; v[4 * h + 3] = a.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (e0 + u < I) v[4 * h + u] = xs[e0 + u];
        }
    }
}

template <int FMT>
__global__ __launch_bounds__(256) void tiled_kernel(TiledArgs a) {
    __shared__ __attribute__((aligned(16))) float As[2][BM][LDK];
    __shared__ __attribute__((aligned(16))) float Bs[2][BN][LDK];

    // XCD-aware tile order: block b runs on XCD b % 8; XCD x owns a contiguous
    // range of tiles, walked with s fastest so consecutive tiles share W.
    const int nt = a.tiles_s * a.tiles_o;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = nt >> 3, extra = nt & 7;
    const int t = xcd * base + min(xcd, extra) + local;
    const int ts = t % a.tiles_s, to = t / a.tiles_s;
    const int s0 = ts * BM, o0 = to * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int lrow = tid >> 2;        // staging row 0..63
    const int lcol = (tid & 3) * 8;   // staging column 0,8,16,24

    const bool vec_ok = ((a.I & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
    const int wrow = o0 + lrow;
    const uint8_t *wrow_p = a.w + (long)min(wrow, a.O - 1) * a.stride;
    const bool wrow_ok = wrow < a.O;

    float xv[8], wq[8];
    auto fetch = [&](long k0) {
        load_x8<FMT>(a.x, a.S, a.I, a.nfull, vec_ok, s0 + lrow, k0 + lcol, xv);
        if (wrow_ok) {
            load_w8<FMT>(wrow_p, a.stride, k0 + lcol, wq);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) wq[e] = 0.0f;
        }
    };
    auto stash = [&](int buf) {
        *reinterpret_cast<float4 *>(&As[buf][lrow][lcol]) = make_float4(xv[0], xv[1], xv[2], xv[3]);
        *reinterpret_cast<float4 *>(&As[buf][lrow][lcol + 4]) = make_float4(xv[4], xv[5], xv[6], xv[7]);
        *reinterpret_cast<float4 *>(&Bs[buf][lrow][lcol]) = make_float4(wq[0], wq[1], wq[2], wq[3]);
        *reinterpret_cast<float4 *>(&Bs[buf][lrow][lcol + 4]) = make_float4(wq[4], wq[5], wq[6], wq[7]);
    };

    f32x4 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // every field position of a row, in device order (the layout permutes
    // elements inside 1 KiB blocks; positions past I may hold real elements)
    const long npos = (FMT == WQ_F32) ? (long)a.I : (long)(a.stride) * (FMT == WQ_I8 ? 1 : FMT == WQ_I4 ? 2 : 4);
    const int nk = (int)((npos + BK - 1) / BK);
    fetch(0);
    stash(0);
    __syncthreads();
    const int g = lane >> 4, li = lane & 15;
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) fetch((long)(kt + 1) * BK);
#pragma unroll
        for (int kg = 0; kg < BK / 16; ++kg) {
            f32x4 av[2], bv[2];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                av[mi] = *reinterpret_cast<const f32x4 *>(&As[buf][wm * 32 + mi * 16 + li][kg * 16 + 4 * g]);
#pragma unroll
            for (int ni = 0; ni < 2; ++ni)
                bv[ni] = *reinterpret_cast<const f32x4 *>(&Bs[buf][wn * 32 + ni * 16 + li][kg * 16 + 4 * g]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < 2; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[mi][j], bv[ni][j], acc[mi][ni], 0, 0, 0);
        }
        if (kt + 1 < nk) stash(buf ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds rows 4*(lane/16) + r, column lane % 16 of each 16x16 tile
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
        const int o = o0 + wn * 32 + ni * 16 + li;
        if (o >= a.O) continue;
        const float sc = a.scales[o];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + wm * 32 + mi * 16 + 4 * g + r;
                if (s < a.S) a.y[(long)s * a.O + o] = sc * acc[mi][ni][r];
            }
    }
}

} // namespace

TiledPlan plan_tiled(int fmt, int O, int I, int S) {
    (void)fmt;
    (void)I;
    TiledPlan p;
    p.tiles_s = (S + p.bm - 1) / p.bm;
    p.tiles_o = (O + p.bn - 1) / p.bn;
    p.grid = p.tiles_s * p.tiles_o;
    return p;
}

hipError_t launch_tiled(int fmt, const TiledPlan &p, const TiledArgs &a, hipStream_t st) {
    switch (fmt) {
    case WQ_F32: hipLaunchKernelGGL(tiled_kernel<WQ_F32>, dim3(p.grid), dim3(p.block), 0, st, a); break;
    case WQ_I8: hipLaunchKernelGGL(tiled_kernel<WQ_I8>, dim3(p.grid), dim3(p.block), 0, st, a); break;
    case WQ_I4: hipLaunchKernelGGL(tiled_kernel<WQ_I4>, dim3(p.grid), dim3(p.block), 0, st, a); break;
    case WQ_I2: hipLaunchKernelGGL(tiled_kernel<WQ_I2>, dim3(p.grid), dim3(p.block), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

} // namespace wq
