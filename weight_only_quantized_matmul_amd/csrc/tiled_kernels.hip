// LDS-tiled dequant + MFMA path for S beyond the register GEMV.
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
//  * a 256-thread block owns a BM (s) x BN (o) output tile, BM = 32*WM and
//    BN = 32*WN; its four waves (2 x 2) each own WM x WN 16x16 fragments;
//  * the contraction runs over the weight fields in device order (see the
//    layout in wq_internal.h); per BK-position step the block stages the
//    matching activations and the weight tile, dequantized once, in LDS
//    (double-buffered, rows padded by 16 bytes) while the next step's global
//    data is already in registers;
//  * the per-row scale is applied in the epilogue, after the sum;
//  * tiles are handed out XCD by XCD (blocks are dispatched round-robin over
//    the 8 XCDs), consecutive tiles of one XCD sharing a weight tile so it is
//    fetched into that XCD's L2 once.
//
// Two operand modes:
//  * fp32 (any weight format, the only one for f32 weights): activations are
//    gathered from x in runs of four consecutive elements, operands stay
//    fp32, v_mfma_f32_16x16x4_f32 (lane group g = lane/16 reads positions
//    4g..4g+3 of a 16-position group with one 128-bit LDS read and feeds them
//    to four MFMAs; A and B use the same order, so the sum is unchanged);
//  * bf16x3 (quantized weights): a pre-pass splits every activation exactly
//    into three bf16 parts by truncation (x = b1 + b2 + b3: b1 keeps the top
//    8 significant bits, b2 the next 8 of the remainder, b3 the last 8) and
//    writes them as three planes in the weights' field order; the integer
//    codes are exact in bf16, and v_mfma_f32_16x16x32_bf16 accumulates
//    b1*q + b2*q + b3*q in fp32 with every product exact: fp32-level
//    results at the bf16 matrix rate, and the split is done once per
//    activation instead of once per output tile.
//
// Few activation rows (S <= 16, bf16x3): 16 x 128 tiles whose eight waves
// sit side by side along o and share each K step's activation fragments
// through LDS (tiled_x3o_kernel). When the tiles alone leave the chip short
// of waves, K is split across blocks: each stores fp32 partials and a small
// kernel adds them in fixed order (splitk_sum_kernel).
#include <climits>

#include "wq_internal.h"

namespace wq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// XCD-aware tile order: block b runs on XCD b % 8; XCD x owns a contiguous
// range of work items, walked with the K chunk fastest, then s, so the
// blocks of one tile (and consecutive tiles, which share W) meet in one L2.
// Returns the work item's K chunk (0 without split K).
__device__ __forceinline__ int tile_origin(const TiledArgs &a, int bm, int bn, int &s0, int &o0) {
    const int ks = a.ksplit;
    const int nt = a.tiles_s * a.tiles_o * ks;
    const int b = blockIdx.x;
    const int xcd = b & 7, local = b >> 3;
    const int base = nt >> 3, extra = nt & 7;
    const int t = xcd * base + min(xcd, extra) + local;
    const int tile = t / ks;
    s0 = (tile % a.tiles_s) * bm;
    o0 = (tile / a.tiles_s) * bn;
    return t - tile * ks;
}

// Epilogue: lane holds rows 4*(lane/16) + r, column lane % 16 of each 16x16
// fragment; the row scale multiplies the finished sum.
template <int WM, int WN>
__device__ __forceinline__ void store_tile(const TiledArgs &a, const f32x4 (&acc)[WM][WN], int s0, int o0, int wm,
                                           int wn, int g, int li) {
#pragma unroll
    for (int n = 0; n < WN; ++n) {
        const int o = o0 + wn * 16 * WN + n * 16 + li;
        if (o >= a.O) continue;
        const float sc = a.scales[o];
#pragma unroll
        for (int m = 0; m < WM; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + wm * 16 * WM + m * 16 + 4 * g + r;
                if (s < a.S) a.y[(long)s * a.O + o] = sc * acc[m][n][r];
            }
    }
}

// ===========================================================================
// fp32 mode

constexpr int BK32 = 32;

// Weight fields at the 8 positions [P0, P0 + 8) of a row, dequantized.
template <int FMT>
__device__ __forceinline__ void load_w8(const uint8_t *__restrict__ row, long stride, long P0, float (&q)[8]) {
    if constexpr (FMT == WQ_F32) {
        const long bo = P0 * 4;
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
        if (P0 < stride) v = *reinterpret_cast<const u32x2 *>(row + P0);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)(int)(int8_t)((e < 4 ? v.x : v.y) >> (8 * (e & 3)));
    } else if constexpr (FMT == WQ_I4) {
        const long bo = P0 / 2;
        uint32_t v = 0x88888888u;
        if (bo < stride) v = *reinterpret_cast<const uint32_t *>(row + bo);
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = (float)((int)((v >> (4 * e)) & 0xFu) - 8);
    } else {
        const long bo = P0 / 4;
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

template <int WM, int WN>
struct F32Cfg {
    static constexpr int BM = 32 * WM, BN = 32 * WN;
    static constexpr int LDA = BK32 + 4;                  // floats per LDS row
    static constexpr int A_FLOATS = BM * LDA, B_FLOATS = BN * LDA;
    static constexpr int STAGE_FLOATS = A_FLOATS + B_FLOATS;
    static constexpr int LDS_BYTES = 2 * STAGE_FLOATS * 4;
    static constexpr int XU = BM * BK32 / 8 / 256;          // activation units (8 positions) per thread
    static constexpr int WU = (BN * BK32 / 8 + 255) / 256;  // weight units per thread (last may be partial)
};

template <int FMT, int WM, int WN>
__global__ __launch_bounds__(256) void tiled_f32_kernel(TiledArgs a) {
    using C = F32Cfg<WM, WN>;
    constexpr int BM = C::BM, BN = C::BN, LDA = C::LDA;
    extern __shared__ __attribute__((aligned(16))) float ldsf[];

    int s0, o0;
    const int kc = tile_origin(a, BM, BN, s0, o0);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int g = lane >> 4, li = lane & 15;

    const bool vec_ok = ((a.I & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
    // every field position of a row, in device order (the layout permutes
    // elements inside 1 KiB blocks; positions past I may hold real elements)
    const long npos = (FMT == WQ_F32) ? (long)a.I : (long)(a.stride) * (FMT == WQ_I8 ? 1 : FMT == WQ_I4 ? 2 : 4);
    const int nk = (int)((npos + BK32 - 1) / BK32);
    // this block's K steps [kb, ke) (all of them without split K)
    const int kb = (int)((long)kc * nk / a.ksplit), ke = (int)((long)(kc + 1) * nk / a.ksplit);

    // staging: unit u covers tile row u / 4, positions 8 * (u % 4) .. +8 of the K step
    float xv[C::XU][8], wv[C::WU][8];
    auto fetch = [&](long k0) {
#pragma unroll
        for (int j = 0; j < C::XU; ++j) {
            const int u = tid + 256 * j;
            load_x8<FMT>(a.x, a.S, a.I, a.nfull, vec_ok, s0 + u / 4, k0 + 8 * (u % 4), xv[j]);
        }
#pragma unroll
        for (int j = 0; j < C::WU; ++j) {
            const int u = tid + 256 * j;
            const int row = o0 + u / 4;
            if (u < BN * 4 && row < a.O) {
                load_w8<FMT>(a.w + (long)row * a.stride, a.stride, k0 + 8 * (u % 4), wv[j]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) wv[j][e] = 0.0f;
            }
        }
    };
    auto stash = [&](int buf) {
        float *As = ldsf + buf * C::STAGE_FLOATS;
        float *Bs = As + C::A_FLOATS;
#pragma unroll
        for (int j = 0; j < C::XU; ++j) {
            const int u = tid + 256 * j;
            float *d = As + (u / 4) * LDA + 8 * (u % 4);
            *reinterpret_cast<float4 *>(d) = make_float4(xv[j][0], xv[j][1], xv[j][2], xv[j][3]);
            *reinterpret_cast<float4 *>(d + 4) = make_float4(xv[j][4], xv[j][5], xv[j][6], xv[j][7]);
        }
#pragma unroll
        for (int j = 0; j < C::WU; ++j) {
            const int u = tid + 256 * j;
            if (u < BN * 4) {
                float *d = Bs + (u / 4) * LDA + 8 * (u % 4);
                *reinterpret_cast<float4 *>(d) = make_float4(wv[j][0], wv[j][1], wv[j][2], wv[j][3]);
                *reinterpret_cast<float4 *>(d + 4) = make_float4(wv[j][4], wv[j][5], wv[j][6], wv[j][7]);
            }
        }
    };

    f32x4 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    fetch((long)kb * BK32);
    stash(0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
        const int buf = (kt - kb) & 1;
        if (kt + 1 < ke) fetch((long)(kt + 1) * BK32);
        const float *As = ldsf + buf * C::STAGE_FLOATS;
        const float *Bs = As + C::A_FLOATS;
#pragma unroll
        for (int kg = 0; kg < BK32 / 16; ++kg) {
            f32x4 av[WM], bv[WN];
#pragma unroll
            for (int m = 0; m < WM; ++m)
                av[m] = *reinterpret_cast<const f32x4 *>(As + (wm * 16 * WM + m * 16 + li) * LDA + kg * 16 + 4 * g);
#pragma unroll
            for (int n = 0; n < WN; ++n)
                bv[n] = *reinterpret_cast<const f32x4 *>(Bs + (wn * 16 * WN + n * 16 + li) * LDA + kg * 16 + 4 * g);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int m = 0; m < WM; ++m)
#pragma unroll
                    for (int n = 0; n < WN; ++n)
                        acc[m][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[m][j], bv[n][j], acc[m][n], 0, 0, 0);
        }
        if (kt + 1 < ke) stash(buf ^ 1);
        __syncthreads();
    }
    if (a.ksplit == 1) {
        store_tile<WM, WN>(a, acc, s0, o0, wm, wn, g, li);
        return;
    }
    // split K: this chunk's unscaled sums; splitk_sum_kernel adds the chunks
    const long pstride = (long)a.S * a.O;
#pragma unroll
    for (int n = 0; n < WN; ++n) {
        const int o = o0 + wn * 16 * WN + n * 16 + li;
        if (o >= a.O) continue;
#pragma unroll
        for (int m = 0; m < WM; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + wm * 16 * WM + m * 16 + 4 * g + r;
                if (s < a.S) a.part[kc * pstride + (long)s * a.O + o] = acc[m][n][r];
            }
    }
}

// ===========================================================================
// bf16x3 mode

// Upper halves of two fp32 bit patterns whose values are exact in bf16.
__device__ __forceinline__ uint32_t bf16_pair(uint32_t lo_bits, uint32_t hi_bits) {
    return (lo_bits >> 16) | (hi_bits & 0xFFFF0000u);
}

// Activations -> three bf16 planes in device field order, each stored
// fragment-major: the block for rows [16 sg, 16 sg + 16) and positions
// [32 kc, 32 kc + 32) is 1 KiB, holding at 16-byte slot l = li + 16 g the
// eight positions 32 kc + 8 g .. +8 of row 16 sg + li. That is the operand
// layout of v_mfma_f32_16x16x32_bf16, so the MFMA kernel loads a fragment
// as one contiguous, fully coalesced 1 KiB access. Thread t fills slot t % 64
// of block t / 64 (blocks ordered with kc fastest); rows past S, elements
// past I and positions past the row's fields are written as zeros, so every
// element of the planes is rewritten on every call.
template <int FMT, int NP = 3>
__global__ __launch_bounds__(256) void split_x_kernel(const float *__restrict__ x, int S, int I, int nfull,
                                                      int vec_ok, int sp, int kp, long plane,
                                                      uint16_t *__restrict__ xp) {
    const long t = (long)blockIdx.x * 256 + threadIdx.x;

    const int kcs = kp / 32;
    if (t >= (long)sp / 16 * kcs * 64) return;
    const int l = (int)(t & 63), li = l & 15, g = l >> 4;
    const long blk = t >> 6;
    const int s = (int)(blk / kcs) * 16 + li;
    const long P = (blk % kcs) * 32 + 8 * g;
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    if (s < S) {
        const float *xs = x + (long)s * I;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const long e0 = elem_of_pos4(FMT, P + 4 * h, nfull);
            if (vec_ok && e0 + 4 <= I) {
                const float4 q = *reinterpret_cast<const float4 *>(xs + e0);
                v[4 * h] = q.x; v[4 * h + 1] = q.y; v[4 * h + 2] = q.z; v[4 * h + 3] = q.w;
            } else {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (e0 + u < I) v[4 * h + u] = xs[e0 + u];
            }
        }
    }
    const long off = t * 8;
    if constexpr (NP == 1) {  // one plane: each activation rounded to the nearest bf16 (ties to even)
        uint32_t b[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t u = __float_as_uint(v[e]);
            b[e] = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
        }
        *reinterpret_cast<u32x4 *>(xp + off) =
            u32x4{bf16_pair(b[0], b[1]), bf16_pair(b[2], b[3]), bf16_pair(b[4], b[5]), bf16_pair(b[6], b[7])};
        return;
    }
    uint32_t b1[8], b2[8], b3[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t hb = __float_as_uint(v[e]) & 0xFFFF0000u;
        const float r = v[e] - __uint_as_float(hb);  // exact
        const uint32_t mb = __float_as_uint(r) & 0xFFFF0000u;
        b1[e] = hb;
        b2[e] = mb;
        b3[e] = __float_as_uint(r - __uint_as_float(mb));  // exact, at most 8 significant bits
    }
    *reinterpret_cast<u32x4 *>(xp + off) =
        u32x4{bf16_pair(b1[0], b1[1]), bf16_pair(b1[2], b1[3]), bf16_pair(b1[4], b1[5]), bf16_pair(b1[6], b1[7])};
    *reinterpret_cast<u32x4 *>(xp + plane + off) =
        u32x4{bf16_pair(b2[0], b2[1]), bf16_pair(b2[2], b2[3]), bf16_pair(b2[4], b2[5]), bf16_pair(b2[6], b2[7])};
    *reinterpret_cast<u32x4 *>(xp + 2 * plane + off) =
        u32x4{bf16_pair(b3[0], b3[1]), bf16_pair(b3[2], b3[3]), bf16_pair(b3[4], b3[5]), bf16_pair(b3[6], b3[7])};
}

// Raw weight bits for the 8 field positions [P0, P0 + 8) of a row (P0 a
// multiple of 8). Positions past the row's stride are read from the row's
// last bytes instead: the activation planes are zero there, so whatever
// codes are read contribute exact zeros.
template <int FMT>
struct RawW;
template <>
struct RawW<WQ_I8> {
    u32x2 v;
    __device__ __forceinline__ void load(const uint8_t *__restrict__ row, long stride, long P0) {
        v = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(row + min(P0, stride - 8)));
    }
    __device__ __forceinline__ int code(int e) const {
        return (int)(int8_t)((e < 4 ? v.x : v.y) >> (8 * (e & 3)));
    }
};
template <>
struct RawW<WQ_I4> {
    uint32_t v;
    __device__ __forceinline__ void load(const uint8_t *__restrict__ row, long stride, long P0) {
        v = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(row + min(P0 / 2, stride - 4)));
    }
    // nibble c stands for c - 8: flipping its top bit gives the same value as
    // a signed 4-bit field
    __device__ __forceinline__ int code(int e) const {
        return (int)((v ^ 0x88888888u) << (28 - 4 * e)) >> 28;
    }
};
template <>
struct RawW<WQ_I2> {
    uint32_t v;
    __device__ __forceinline__ void load(const uint8_t *__restrict__ row, long stride, long P0) {
        v = __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(row + min(P0 / 4, stride - 2)));
    }
    // code c stands for c - 2: the same value as a signed 2-bit field with
    // its top bit flipped
    __device__ __forceinline__ int code(int e) const {
        return (int)((v ^ 0xAAAAu) << (30 - 2 * e)) >> 30;
    }
};

// Eight decoded codes as bf16 (exact: |code| <= 128 has at most 8 significant bits).
template <int FMT>
__device__ __forceinline__ u32x4 codes_bf16x8(const RawW<FMT> &w) {
    uint32_t f[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = __float_as_uint((float)w.code(e));
    return u32x4{bf16_pair(f[0], f[1]), bf16_pair(f[2], f[3]), bf16_pair(f[4], f[5]), bf16_pair(f[6], f[7])};
}

// bf16x3 tile: the block's WAVES waves are stacked along s. Wave w owns rows
// [16*WM*w, 16*WM*(w+1)) of the block's BM = 16*WM*WAVES rows and all
// BN = 16*WN columns, so its activation rows are its own: their fragments
// are loaded from the planes straight into registers (MFMA operand layout,
// one step ahead), and only the dequantized weight tile, shared by all the
// waves, goes through LDS. Eight waves per block give two waves per SIMD,
// which hide each other's load latency.
template <int WAVES, int WM, int WN, int BK_>
struct X3Cfg {
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = 16 * WM * WAVES, BN = 16 * WN, BK = BK_;
    static constexpr int KH = BK / 32;               // 32-position MFMA steps per K step
    // 16-byte operand reads (lane l: row l % 16, chunk l / 16) hit distinct
    // banks when the row stride is an odd multiple of 32 bytes (160 or 288 here)
    static constexpr int LDB = BK + 16;              // bf16 per LDS row
    static constexpr int CH = BK / 8;                // 16-byte chunks per row per step
    static constexpr int WU = (BN * CH + THREADS - 1) / THREADS; // weight chunks per thread
    static constexpr int BROWS = WU * THREADS / CH;  // LDS rows written (>= BN; the rest are never read)
    static constexpr int STAGE = BROWS * LDB;        // bf16 per stage
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static_assert((WU * THREADS) % CH == 0 && BROWS >= BN, "weight chunks must fill whole rows");
    static_assert(kTiledKAlign % BK == 0 && ((LDB * 2 / 32) & 1) == 1, "K step and LDS row stride");
};

constexpr int gcd_c(int x, int y) { return y == 0 ? x : gcd_c(y, x % y); }

// bf16x3 pipeline depths (measured on the 512 x 6144 x 6144 int8 prefill:
// deeper activation prefetch and 2..8 weight sets all ran within 3%)
constexpr int kX3ActPrefetch = 1;  // activation fragments loaded this many K steps ahead
constexpr int kX3WeightSets = 4;   // weight-code register sets (loaded kX3WeightSets - 1 steps ahead)

// PD: activation fragments are loaded PD steps ahead (PD + 1 register sets);
// NW: weight codes are loaded NW - 1 steps before they are staged (NW sets)
// GS: group-wise scales (rows in natural order, gs a multiple of BK, 64 or
// 128; the planner takes 128-deep steps only when gs % 128 == 0): each K step
// lies in one group; the steps of a group accumulate into
// separate fragments, which are added to the accumulators times the group
// scale of their output column when the group ends.
// NP: activation planes (3: the exact split; 1: x rounded to bf16).
template <int FMT, int WAVES, int WM, int WN, int BK_, int PD, int NW, bool GS, int NP = 3>
__global__ __launch_bounds__(64 * WAVES) void tiled_x3_kernel(TiledArgs a) {
    using C = X3Cfg<WAVES, WM, WN, BK_>;
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, LDB = C::LDB, CH = C::CH, KH = C::KH;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds16[];

    int s0, o0;
    const int kc = tile_origin(a, BM, BN, s0, o0);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int nk = a.kp / BK;
    // this block's K steps [kb, ke) (all of them without split K)
    const int kb = (int)((long)kc * nk / a.ksplit), ke = (int)((long)(kc + 1) * nk / a.ksplit);

    // A fragments of one step: [m][plane][32-position part], lane (li, g)
    // holds row 16m + li, positions 32 * part + 8g .. +8 of the step: one
    // 1 KiB block of the fragment-major planes each
    typedef u32x4 AFrag[WM][NP][KH];
    const int kcs = a.kp / 32;
    const uint16_t *ap = a.xp + ((long)(s0 / 16 + WM * wave) * kcs) * 512 + lane * 8;
    auto load_a = [&](int kt, AFrag &af) {
#pragma unroll
        for (int m = 0; m < WM; ++m)
#pragma unroll
            for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                for (int h = 0; h < KH; ++h)
                    af[m][pl][h] = *reinterpret_cast<const u32x4 *>(ap + pl * a.plane +
                                                                     ((long)m * kcs + KH * kt + h) * 512);
    };

    // Weight codes travel through a ring of NW register sets: step j's raw
    // codes sit in set j % NW, loaded NW - 1 steps before they are stored to
    // LDS (they mostly come from HBM, and loads retire in issue order, so a
    // short distance would also hold up the activation loads behind them).
    // Weight rows past O are read from row O - 1: they only feed output
    // columns that are never stored.
    typedef RawW<FMT> WSet[C::WU];
    auto load_w = [&](int kt, WSet &w) {
        const long k0 = (long)kt * BK;
#pragma unroll
        for (int j = 0; j < C::WU; ++j) {
            const int u = tid + C::THREADS * j;
            const int row = min(o0 + u / CH, a.O - 1);
            w[j].load(a.w + (long)row * a.stride, a.stride, k0 + 8 * (u % CH));
        }
    };
    auto stash_w = [&](int buf, const WSet &w) {
        uint16_t *st = lds16 + buf * C::STAGE;
#pragma unroll
        for (int j = 0; j < C::WU; ++j) {
            const int u = tid + C::THREADS * j;
            *reinterpret_cast<u32x4 *>(st + (u / CH) * LDB + 8 * (u % CH)) = codes_bf16x8<FMT>(w[j]);
        }
    };

    f32x4 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // One K step kt: A of step kt in `cur`, B of step kt in LDS buffer
    // kt & 1. The weights of step kt + 1 (`wnext`) go to the other buffer,
    // released by the previous barrier; activations of step kt + PD and
    // weights of step kt + NW are loaded (clamped: the last steps reload
    // data nobody reads).
    f32x4 tacc[WM][WN];  // GS: the current group's sums
    auto iter = [&](int kt, const AFrag &cur, AFrag &nxt, const WSet &wnext, WSet &wload) {
        const int buf = (kt - kb) & 1;
        load_a(min(kt + PD, ke - 1), nxt);
        float gsc[WN];
        bool group_ends = false;
        if constexpr (GS) {
            static_assert(BK % kGroupAlign == 0, "a group-scaled K step covers whole 64-position blocks");
            const long first = (long)kt * BK;
            const int grp = min((int)(first / a.gs), a.ng - 1);
            group_ends = (first + BK) % a.gs == 0 || kt + 1 == nk;  // wave-uniform
#pragma unroll
            for (int n = 0; n < WN; ++n) gsc[n] = a.scales[(long)grp * a.O + min(o0 + 16 * n + li, a.O - 1)];
            if (first % a.gs == 0) {
#pragma unroll
                for (int m = 0; m < WM; ++m)
#pragma unroll
                    for (int n = 0; n < WN; ++n) tacc[m][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        auto &dst = *(GS ? &tacc : &acc);
        const uint16_t *Bs = lds16 + buf * C::STAGE;
#pragma unroll
        for (int h = 0; h < KH; ++h) {
            bf16x8 bv[WN];
#pragma unroll
            for (int n = 0; n < WN; ++n)
                bv[n] = *reinterpret_cast<const bf16x8 *>(Bs + (16 * n + li) * LDB + 32 * h + 8 * g);
            if (h == KH / 2) {
                stash_w(buf ^ 1, wnext);
                load_w(min(kt + NW, ke - 1), wload);
            }
#pragma unroll
            for (int pl = 0; pl < NP; ++pl)
#pragma unroll
                for (int m = 0; m < WM; ++m) {
                    const bf16x8 av = __builtin_bit_cast(bf16x8, cur[m][pl][h]);
#pragma unroll
                    for (int n = 0; n < WN; ++n)
                        dst[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[n], dst[m][n], 0, 0, 0);
                }
        }
        if constexpr (GS) {
            if (group_ends) {
#pragma unroll
                for (int m = 0; m < WM; ++m)
#pragma unroll
                    for (int n = 0; n < WN; ++n)
#pragma unroll
                        for (int r = 0; r < 4; ++r) acc[m][n][r] = fmaf(gsc[n], tacc[m][n][r], acc[m][n][r]);
            }
        }
        __syncthreads();
    };

    // Step j uses activation set j % (PD + 1) and weight set j % NW; the
    // loop body covers U steps so that every index is a constant.
    constexpr int U = (PD + 1) * NW / gcd_c(PD + 1, NW);
    AFrag af[PD + 1];
    WSet wg[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) load_w(min(kb + i, ke - 1), wg[i]);
    stash_w(0, wg[0]);
#pragma unroll
    for (int i = 0; i < PD; ++i) load_a(min(kb + i, ke - 1), af[i]);
    __syncthreads();
    int kt = kb;
    for (; kt + U <= ke; kt += U) {
#pragma unroll
        for (int i = 0; i < U; ++i)
            iter(kt + i, af[i % (PD + 1)], af[(i + PD) % (PD + 1)], wg[(i + 1) % NW], wg[i % NW]);
    }
#pragma unroll
    for (int i = 0; i + 1 < U; ++i)
        if (kt + i < ke) iter(kt + i, af[i % (PD + 1)], af[(i + PD) % (PD + 1)], wg[(i + 1) % NW], wg[i % NW]);

    // epilogue: lane holds rows 4g + r, column li of each 16x16 fragment
    if (a.ksplit == 1) {
#pragma unroll
        for (int n = 0; n < WN; ++n) {
            const int o = o0 + 16 * n + li;
            if (o >= a.O) continue;
            const float sc = GS ? 1.0f : a.scales[o];
#pragma unroll
            for (int m = 0; m < WM; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = s0 + 16 * WM * wave + 16 * m + 4 * g + r;
                    if (s < a.S) a.y[(long)s * a.O + o] = sc * acc[m][n][r];
                }
        }
        return;
    }
    // split K: store this chunk's sums; splitk_sum_kernel adds the chunks
    const long pstride = (long)a.S * a.O;
#pragma unroll
    for (int n = 0; n < WN; ++n) {
        const int o = o0 + 16 * n + li;
        if (o >= a.O) continue;
#pragma unroll
        for (int m = 0; m < WM; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int s = s0 + 16 * WM * wave + 16 * m + 4 * g + r;
                if (s < a.S) a.part[kc * pstride + (long)s * a.O + o] = acc[m][n][r];
            }
    }
}

// Split K: y[s][o] = scale[o] * (sum over chunks c = 0.. of part[c][s][o]),
// the chunks added in order (deterministic; exact partial sums stay exact).
// Runs after the tiled kernel on the same stream.
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float *__restrict__ part, int ks, long n, int O,
                                                         const float *__restrict__ scales, float *__restrict__ y) {
    for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long)gridDim.x * 256) {
        float t = 0.0f;
        for (int c = 0; c < ks; ++c) t += part[c * n + i];
        y[i] = scales[i % O] * t;
    }
}

// bf16x3 tile for few activation rows (S <= 16): the block's WAVES waves
// sit side by side along o. The block's 16 activation rows are shared: each
// K step's fragments (3 planes x 2 halves x 64 lanes x 16 bytes) are loaded
// once per block and staged in LDS next to the weight tile, instead of
// every wave loading them itself (which made the activation stream ~12x the
// int2 weight bytes). Wave w owns columns [16 WN w, 16 WN (w + 1)) of the
// block's BN = 16 WN WAVES. K steps of 64 positions.
template <int WAVES, int WN>
struct X3OCfg {
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int BM = 16, BN = 16 * WN * WAVES, BK = 64, KH = 2;
    static constexpr int LDB = BK + 16;
    static constexpr int CH = BK / 8;
    static constexpr int WU = (BN * CH + THREADS - 1) / THREADS;
    static constexpr int BROWS = WU * THREADS / CH;
    static constexpr int WSTAGE = BROWS * LDB;                // bf16 per weight stage
    static constexpr int ACH = 3 * KH * 64;                   // 16-byte activation chunks per step
    static constexpr int AU = (ACH + THREADS - 1) / THREADS;  // per thread
    static constexpr int STAGE = WSTAGE + ACH * 8;            // bf16 per stage (weights, then activations)
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static_assert((WU * THREADS) % CH == 0 && BROWS >= BN, "weight chunks must fill whole rows");
    static_assert(kTiledKAlign % BK == 0 && ((LDB * 2 / 32) & 1) == 1, "K step and LDS row stride");
};

template <int FMT, int WAVES, int WN, int NW, bool GS>
__global__ __launch_bounds__(64 * WAVES) void tiled_x3o_kernel(TiledArgs a) {
    using C = X3OCfg<WAVES, WN>;
    constexpr int BM = C::BM, BN = C::BN, BK = C::BK, LDB = C::LDB, CH = C::CH, KH = C::KH;
    extern __shared__ __attribute__((aligned(16))) uint16_t lds16[];

    int s0, o0;
    const int kc = tile_origin(a, BM, BN, s0, o0);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4, li = lane & 15;
    const int nk = a.kp / BK;
    const int kb = (int)((long)kc * nk / a.ksplit), ke = (int)((long)(kc + 1) * nk / a.ksplit);

    // activation chunk c of step kt: plane c / 128, half (c / 64) % 2, lane slot c % 64
    const int kcs = a.kp / 32;
    const uint16_t *ab = a.xp + (long)(s0 / 16) * kcs * 512;
    typedef u32x4 ARaw[C::AU];
    auto load_a = [&](int kt, ARaw &r) {
#pragma unroll
        for (int j = 0; j < C::AU; ++j) {
            const int c = tid + C::THREADS * j;
            if (c < C::ACH)
                r[j] = *reinterpret_cast<const u32x4 *>(ab + (c >> 7) * a.plane +
                                                        ((long)KH * kt + ((c >> 6) & 1)) * 512 + (c & 63) * 8);
        }
    };
    auto stash_a = [&](int buf, const ARaw &r) {
        uint16_t *st = lds16 + buf * C::STAGE + C::WSTAGE;
#pragma unroll
        for (int j = 0; j < C::AU; ++j) {
            const int c = tid + C::THREADS * j;
            if (c < C::ACH) *reinterpret_cast<u32x4 *>(st + c * 8) = r[j];
        }
    };
    typedef RawW<FMT> WSet[C::WU];
    auto load_w = [&](int kt, WSet &w) {
        const long k0 = (long)kt * BK;
#pragma unroll
        for (int j = 0; j < C::WU; ++j) {
            const int u = tid + C::THREADS * j;
            const int row = min(o0 + u / CH, a.O - 1);
            w[j].load(a.w + (long)row * a.stride, a.stride, k0 + 8 * (u % CH));
        }
    };
    auto stash_w = [&](int buf, const WSet &w) {
        uint16_t *st = lds16 + buf * C::STAGE;
#pragma unroll
        for (int j = 0; j < C::WU; ++j) {
            const int u = tid + C::THREADS * j;
            *reinterpret_cast<u32x4 *>(st + (u / CH) * LDB + 8 * (u % CH)) = codes_bf16x8<FMT>(w[j]);
        }
    };

    f32x4 acc[WN], tacc[WN];
#pragma unroll
    for (int n = 0; n < WN; ++n) acc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Step kt reads stage (kt - kb) & 1 and fills the other one: the weights
    // of step kt + 1 (set wnext, loaded NW - 1 steps ago) and its
    // activations (ar, loaded one step ago); then requests the weights of
    // step kt + NW (into the set just consumed) and the activations of step
    // kt + 2 (clamped: the last steps reload data nobody reads).
    ARaw ar;
    auto iter = [&](int kt, const WSet &wnext, WSet &wload) {
        const int buf = (kt - kb) & 1;
        float gsc[WN];
        bool group_ends = false;
        if constexpr (GS) {
            const long first = (long)kt * BK;
            const int grp = min((int)(first / a.gs), a.ng - 1);
            group_ends = (first + BK) % a.gs == 0 || kt + 1 == nk;  // wave-uniform
#pragma unroll
            for (int n = 0; n < WN; ++n)
                gsc[n] = a.scales[(long)grp * a.O + min(o0 + 16 * (WN * wave + n) + li, a.O - 1)];
            if (first % a.gs == 0) {
#pragma unroll
                for (int n = 0; n < WN; ++n) tacc[n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
        auto &dst = *(GS ? &tacc : &acc);
        const uint16_t *Bs = lds16 + buf * C::STAGE;
        const uint16_t *As = Bs + C::WSTAGE;
#pragma unroll
        for (int h = 0; h < KH; ++h) {
            bf16x8 bv[WN], av[3];
#pragma unroll
            for (int n = 0; n < WN; ++n)
                bv[n] = *reinterpret_cast<const bf16x8 *>(Bs + (16 * (WN * wave + n) + li) * LDB + 32 * h + 8 * g);
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
                av[pl] = *reinterpret_cast<const bf16x8 *>(As + ((pl * KH + h) * 64 + lane) * 8);
            if (h == KH / 2) {
                stash_w(buf ^ 1, wnext);
                stash_a(buf ^ 1, ar);
                load_w(min(kt + NW, ke - 1), wload);
                load_a(min(kt + 2, ke - 1), ar);
            }
#pragma unroll
            for (int pl = 0; pl < 3; ++pl)
#pragma unroll
                for (int n = 0; n < WN; ++n)
                    dst[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[pl], bv[n], dst[n], 0, 0, 0);
        }
        if constexpr (GS) {
            if (group_ends) {
#pragma unroll
                for (int n = 0; n < WN; ++n)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[n][r] = fmaf(gsc[n], tacc[n][r], acc[n][r]);
            }
        }
        __syncthreads();
    };

    WSet wg[NW];
#pragma unroll
    for (int i = 0; i < NW; ++i) load_w(min(kb + i, ke - 1), wg[i]);
    load_a(kb, ar);
    stash_w(0, wg[0]);
    stash_a(0, ar);
    load_a(min(kb + 1, ke - 1), ar);
    __syncthreads();
    int kt = kb;
    for (; kt + NW <= ke; kt += NW) {
#pragma unroll
        for (int i = 0; i < NW; ++i) iter(kt + i, wg[(i + 1) % NW], wg[i % NW]);
    }
#pragma unroll
    for (int i = 0; i + 1 < NW; ++i)
        if (kt + i < ke) iter(kt + i, wg[(i + 1) % NW], wg[i % NW]);

    // epilogue: lane holds rows 4g + r, column li of each 16x16 fragment
    const long pstride = (long)a.S * a.O;
#pragma unroll
    for (int n = 0; n < WN; ++n) {
        const int o = o0 + 16 * (WN * wave + n) + li;
        if (o >= a.O) continue;
        const float sc = (GS || a.ksplit > 1) ? 1.0f : a.scales[o];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int s = s0 + 4 * g + r;
            if (s >= a.S) continue;
            if (a.ksplit == 1) a.y[(long)s * a.O + o] = sc * acc[n][r];
            else a.part[kc * pstride + (long)s * a.O + o] = acc[n][r];
        }
    }
}

// ===========================================================================
// launch

template <typename K>
hipError_t raise_lds_limit(K kernel, int bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    return hipFuncSetAttribute(reinterpret_cast<const void *>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               bytes);
}

template <int FMT, int WM, int WN>
hipError_t launch_f32(const TiledPlan &p, const TiledArgs &a, hipStream_t st) {
    using C = F32Cfg<WM, WN>;
    static_assert(C::LDS_BYTES <= 160 * 1024, "tile does not fit in LDS");
    static const hipError_t lim = raise_lds_limit(&tiled_f32_kernel<FMT, WM, WN>, C::LDS_BYTES);
    if (lim != hipSuccess) return lim;
    hipLaunchKernelGGL((tiled_f32_kernel<FMT, WM, WN>), dim3(p.grid), dim3(256), C::LDS_BYTES, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.ksplit == 1) return e;
    const long n = (long)a.S * a.O;
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)std::min<long>((n + 255) / 256, 4096)), dim3(256), 0, st,
                       a.part, a.ksplit, n, a.O, a.scales, a.y);
    return hipGetLastError();
}

template <int FMT, int WAVES, int WM, int WN, int BK, int PD, bool GS = false, int NP = 3>
hipError_t launch_x3(const TiledPlan &p, const TiledArgs &a, hipStream_t st) {
    using C = X3Cfg<WAVES, WM, WN, BK>;
    constexpr int NW = kX3WeightSets;
    static_assert(C::LDS_BYTES <= 160 * 1024, "tile does not fit in LDS");
    static const hipError_t lim =
        raise_lds_limit(&tiled_x3_kernel<FMT, WAVES, WM, WN, BK, PD, NW, GS, NP>, C::LDS_BYTES);
    if (lim != hipSuccess) return lim;
    const int vec_ok = ((a.I & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
    const long slots = (long)p.sp * p.kp / 8;  // one thread per 16-byte fragment slot
    hipLaunchKernelGGL((split_x_kernel<FMT, NP>), dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, st, a.x, a.S,
                       a.I, a.nfull, vec_ok, p.sp, p.kp, (long)p.sp * p.kp, const_cast<uint16_t *>(a.xp));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tiled_x3_kernel<FMT, WAVES, WM, WN, BK, PD, NW, GS, NP>), dim3(p.grid), dim3(C::THREADS),
                       C::LDS_BYTES, st, a);
    e = hipGetLastError();
    if (e != hipSuccess || a.ksplit == 1) return e;
    const long n = (long)a.S * a.O;
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)std::min<long>((n + 255) / 256, 4096)), dim3(256), 0, st,
                       a.part, a.ksplit, n, a.O, a.scales, a.y);
    return hipGetLastError();
}

template <int FMT, int WAVES, int WN, bool GS = false>
hipError_t launch_x3o(const TiledPlan &p, const TiledArgs &a, hipStream_t st) {
    using C = X3OCfg<WAVES, WN>;
    constexpr int NW = kX3WeightSets;
    static_assert(C::LDS_BYTES <= 64 * 1024, "tile does not fit the default LDS limit");
    const int vec_ok = ((a.I & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
    const long slots = (long)p.sp * p.kp / 8;
    hipLaunchKernelGGL((split_x_kernel<FMT>), dim3((unsigned)((slots + 255) / 256)), dim3(256), 0, st, a.x, a.S,
                       a.I, a.nfull, vec_ok, p.sp, p.kp, (long)p.sp * p.kp, const_cast<uint16_t *>(a.xp));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((tiled_x3o_kernel<FMT, WAVES, WN, NW, GS>), dim3(p.grid), dim3(C::THREADS), C::LDS_BYTES, st,
                       a);
    e = hipGetLastError();
    if (e != hipSuccess || a.ksplit == 1) return e;
    const long n = (long)a.S * a.O;
    hipLaunchKernelGGL(splitk_sum_kernel, dim3((unsigned)std::min<long>((n + 255) / 256, 4096)), dim3(256), 0, st,
                       a.part, a.ksplit, n, a.O, a.scales, a.y);
    return hipGetLastError();
}

// Compiled tile shapes {bm, bn, bk}; the first entry is the large-problem
// default, the last the small-problem default.
struct Shape {
    int bm, bn, bk;
};
constexpr Shape kX3Shapes[] = {{128, 96, 64}, {128, 96, 128}, {64, 64, 64}, {16, 128, 64}, {64, 192, 64},
                               {64, 64, 128}};
constexpr Shape kF32Shapes[] = {{128, 96, 32}, {64, 64, 32}};

template <int FMT>
hipError_t launch_fmt(const TiledPlan &p, const TiledArgs &a, hipStream_t st) {
    if constexpr (FMT != WQ_F32) {
        if (p.mode == kTiledBF16) {  // one rounded plane; no 16-row tile
            if (a.gs > 0) {
                if (p.bm == 128 && p.bk == 128) return launch_x3<FMT, 8, 1, 6, 128, kX3ActPrefetch, true, 1>(p, a, st);
                if (p.bm == 128) return launch_x3<FMT, 8, 1, 6, 64, kX3ActPrefetch, true, 1>(p, a, st);
                if (p.bn == 192) return launch_x3<FMT, 4, 1, 12, 64, kX3ActPrefetch, true, 1>(p, a, st);
                if (p.bk == 128) return launch_x3<FMT, 4, 1, 4, 128, kX3ActPrefetch, true, 1>(p, a, st);
                return launch_x3<FMT, 4, 1, 4, 64, kX3ActPrefetch, true, 1>(p, a, st);
            }
            if (p.bm == 128) {
                if (p.bk == 128) return launch_x3<FMT, 8, 1, 6, 128, kX3ActPrefetch, false, 1>(p, a, st);
                return launch_x3<FMT, 8, 1, 6, 64, kX3ActPrefetch, false, 1>(p, a, st);
            }
            if (p.bn == 192) return launch_x3<FMT, 4, 1, 12, 64, kX3ActPrefetch, false, 1>(p, a, st);
            if (p.bk == 128) return launch_x3<FMT, 4, 1, 4, 128, kX3ActPrefetch, false, 1>(p, a, st);
            return launch_x3<FMT, 4, 1, 4, 64, kX3ActPrefetch, false, 1>(p, a, st);
        }
        if (p.mode == kTiledBF16X3 && a.gs > 0) {  // group-wise scales: K steps within one group
            if (p.bm == 128 && p.bk == 128) return launch_x3<FMT, 8, 1, 6, 128, kX3ActPrefetch, true>(p, a, st);
            if (p.bm == 128) return launch_x3<FMT, 8, 1, 6, 64, kX3ActPrefetch, true>(p, a, st);
            if (p.bm == 16) return launch_x3o<FMT, 8, 1, true>(p, a, st);
            if (p.bn == 192) return launch_x3<FMT, 4, 1, 12, 64, kX3ActPrefetch, true>(p, a, st);
            if (p.bk == 128) return launch_x3<FMT, 4, 1, 4, 128, kX3ActPrefetch, true>(p, a, st);
            return launch_x3<FMT, 4, 1, 4, 64, kX3ActPrefetch, true>(p, a, st);
        }
        if (p.mode == kTiledBF16X3) {
            if (p.bm == 128) {
                if (p.bk == 128) return launch_x3<FMT, 8, 1, 6, 128, kX3ActPrefetch>(p, a, st);
                return launch_x3<FMT, 8, 1, 6, 64, kX3ActPrefetch>(p, a, st);
            }
            if (p.bm == 16) return launch_x3o<FMT, 8, 1>(p, a, st);
            if (p.bn == 192) return launch_x3<FMT, 4, 1, 12, 64, kX3ActPrefetch>(p, a, st);
            if (p.bk == 128) return launch_x3<FMT, 4, 1, 4, 128, kX3ActPrefetch>(p, a, st);
            return launch_x3<FMT, 4, 1, 4, 64, kX3ActPrefetch>(p, a, st);
        }
    }
    if (p.bm == 128) return launch_f32<FMT, 4, 3>(p, a, st);
    return launch_f32<FMT, 2, 2>(p, a, st);
}

} // namespace

namespace {

// The rest of a plan for one tile shape: tile counts, block size, the
// bf16x3 planes and split K.
TiledPlan plan_shape(TiledPlan p, const Shape &sh, int fmt, int O, int I, int S, int gs) {
    p.bm = sh.bm;
    p.bn = sh.bn;
    p.bk = sh.bk;
    p.tiles_s = (S + p.bm - 1) / p.bm;
    p.tiles_o = (O + p.bn - 1) / p.bn;
    p.grid = p.tiles_s * p.tiles_o;
    p.block = (p.mode != kTiledF32 && (p.bm == 128 || p.bm == 16)) ? 512 : 256;  // 64-row tiles: four waves
    if (p.mode == kTiledF32) {
        // fp32 mode: no planes; split K as below when the tiles leave the
        // chip short of waves (f32 12288 x 6144 at S = 9: 192 tiles)
        const long npos = fmt == WQ_F32 ? (long)I : round_up(row_bytes(fmt, I), kRowAlign) * elems_per_byte(fmt);
        const int nk = (int)((npos + BK32 - 1) / BK32);
        const int waves = p.grid * (p.block / 64);
        if (gs == 0 && waves < kTiledSplitWaves && nk >= 2 * kTiledMinChunk) {
            int ks = (kTiledSplitWaves + waves - 1) / waves;
            ks = std::min(ks, nk / kTiledMinChunk);
            if (ks > 1 && (long)ks * S * O <= (long)INT_MAX) {
                p.ksplit = ks;
                p.grid *= ks;
                p.part_off = 0;
                p.ws_bytes = (size_t)ks * S * O * sizeof(float);
            }
        }
    }
    if (p.mode != kTiledF32) {
        const long stride = round_up(row_bytes(fmt, I), kRowAlign);
        const long npos = stride * elems_per_byte(fmt);
        p.kp = (int)round_up(npos, kTiledKAlign);
        // plane rows: the 16-row tile reads 16-row blocks only; the larger
        // tiles read up to 128-row multiples
        p.sp = (int)round_up(S, p.bm == 16 ? 16 : kTiledSAlign);
        p.ws_bytes = (size_t)(p.mode == kTiledBF16 ? 1 : 3) * p.sp * p.kp * sizeof(uint16_t);
        // Split K when the tiles alone leave the chip short of blocks (few
        // activation rows): each K chunk of at least kTiledMinChunk steps
        // becomes a block of its own. Group-scaled tensors keep whole rows.
        const int nk = p.kp / p.bk;
        // (the 16-row tile's eight waves share one activation stage: it takes
        // twice the waves, measured 3-5 % faster than four-wave blocks)
        const int waves = p.grid * (p.block / 64);
        const int target = p.bm == 16 ? 2 * kTiledSplitWaves : kTiledSplitWaves;
        if (gs == 0 && waves < target && nk >= 2 * kTiledMinChunk) {
            int ks = (target + waves - 1) / waves;
            ks = std::min(ks, nk / kTiledMinChunk);
            if (ks > 1 && (long)ks * S * O <= (long)INT_MAX) {
                p.ksplit = ks;
                p.grid *= ks;
                p.part_off = round_up((long)p.ws_bytes, 256);
                p.ws_bytes = p.part_off + (size_t)ks * S * O * sizeof(float);
            }
        }
    }
    return p;
}

// Share of the last round of resident waves that a plan fills (1: its
// waves make whole rounds of kTiledSplitWaves).
double round_fill(const TiledPlan &p) {
    const long waves = (long)p.grid * (p.block / 64);
    const long rounds = (waves + kTiledSplitWaves - 1) / kTiledSplitWaves;
    return (double)waves / (double)(rounds * kTiledSplitWaves);
}

} // namespace

TiledPlan plan_tiled(int fmt, int O, int I, int S, int mode, int shape, int gs) {
    TiledPlan p;
    // the bf16 split needs exact integer codes (quantized formats); f32 weights
    // stay fp32; group-scaled tensors always take the bf16x3 kernel
    p.mode = fmt == WQ_F32 ? kTiledF32
             : mode == kTiledBF16 ? kTiledBF16
             : (mode == kTiledBF16X3 || gs > 0) ? kTiledBF16X3 : kTiledF32;
    // plane sizes are kept in int: rows near the int limit take the fp32 mode
    if ((long)S > INT_MAX - kTiledSAlign || (long)I > INT_MAX / 2 - 4 * kTiledKAlign) p.mode = kTiledF32;
    if (p.mode != kTiledF32) {
        const bool a16 = p.mode == kTiledBF16;  // no 16-row tile (its kernel reads three planes)
        for (const Shape &c : kX3Shapes)
            if (shape == c.bm * 1000000 + c.bn * 1000 + c.bk && (gs == 0 || gs % c.bk == 0) &&
                !(a16 && c.bm == 16))
                return plan_shape(p, c, fmt, O, I, S, gs);
        // S <= 16: 16 x 128 tiles of eight waves side by side along o,
        // sharing the activation fragments (tiled_x3o_kernel). 17..64: 64 x
        // 192 tiles of four waves (each 16 x 192: a third of the activation
        // reads of 64 x 64 tiles) unless their grid, split K included, fills
        // its last round of resident waves clearly worse (by more than 0.2)
        // than the 64 x 64 tiles' (us:
        // int4 12288 x 6144 at S = 33 / 64 47.2 / 53.3 vs 55.1 / 59.4, int8
        // 6144 x 6144 35.7 / 38.3 vs 39.1 / 41.1; int2 16384 x 8192 at S = 40
        // 82.2 on 516 blocks vs 69.8 on 512). Above, the 128 x 96 tiles of
        // eight waves (one block per CU; 64 x 192 measured 5-10 % slower
        // there) on the same test against the 64 x 64 tiles (int4 at S = 96
        // 65.8 vs 80.2, int8 at S = 128 44.8 vs 62.9; int2 at S = 96 139.6 on
        // 342 big blocks vs 115.7 on 512 small ones; int4 14336 x 4096 at
        // S = 512 207.5 on 600 big blocks, fill 0.78, vs 255 on 1792 small
        // ones, fill 0.88).
        if (S <= 16) return plan_shape(p, a16 ? kX3Shapes[2] : kX3Shapes[3], fmt, O, I, S, gs);
        // One rounded plane above 64 rows: 128 x 96 tiles with 128-deep K
        // steps (half the barriers per product), whatever the fill (us,
        // 128x96x128 / 128x96x64 / 64x64x64: int8 6144 x 6144 at S = 512
        // 64.1 / 73.1 / 86.5, at S = 128 32.3 / 35.1 / 40.9; int4 12288 x 6144
        // at S = 96 41.7 / 47.0 / 52.7; int4 14336 x 4096 at S = 512 100.2 /
        // 115.4 / 127.9; int2 16384 x 8192 at S = 96 66.0 / 81.5 / 78.4).
        // Group scales need steps within one group (gs % 128 == 0 here).
        if (a16 && S > 64 && gs % 128 == 0) return plan_shape(p, kX3Shapes[1], fmt, O, I, S, gs);
        // ... and 64 x 64 tiles, also 128 deep, for 17..64 rows (us, 64x64x128 /
        // 64x192x64: int4 12288 x 6144 at S = 40 34.5 / 41.5, at S = 48 36.3 /
        // 43.7; int8 6144 x 6144 at S = 64 28.6 / 34.3). 64 x 192 tiles 128
        // deep run one wave per SIMD and lost everywhere (5-50 %).
        if (a16 && gs % 128 == 0) return plan_shape(p, kX3Shapes[5], fmt, O, I, S, gs);
        // bf16x3: where the 64 x 64 tiles win above 64 rows they step 128 deep
        // (int2 16384 x 8192 at S = 96 106.2 against 114.9 us); at 17..64 rows
        // 128-deep 64 x 64 tiles lost to 64 x 192 ones (int4 at S = 40 54.0 /
        // 48.6, int8 at S = 64 39.7 / 38.3).
        const TiledPlan small =
            plan_shape(p, S > 64 && gs % 128 == 0 ? kX3Shapes[5] : kX3Shapes[2], fmt, O, I, S, gs);
        // The large tiles above 64 rows step 128 deep in K unless a group
        // holds fewer or an odd number of 64-position blocks (us, 128x96x128 / 128x96x64 in this mode:
        // int8 6144 x 6144 at S = 512 109.2 / 114.3, at S = 128 43.1 / 45.2;
        // int4 12288 x 6144 at S = 96 62.6 / 66.6; int4 14336 x 4096 at
        // S = 512 197.6 / 207.7).
        const Shape &big = gs % 128 == 0 ? kX3Shapes[1] : kX3Shapes[0];
        const TiledPlan large = plan_shape(p, S <= 64 ? kX3Shapes[4] : big, fmt, O, I, S, gs);
        return round_fill(large) + 0.2 >= round_fill(small) ? large : small;
    }
    // fp32: big tiles (128 x 96, 4 x 3 fragments per wave) when there are enough of them
    const long big = (long)((S + 127) / 128) * ((O + 95) / 96);
    Shape sh = (S >= 128 && big >= 128) ? kF32Shapes[0] : kF32Shapes[1];
    for (const Shape &c : kF32Shapes)
        if (shape == c.bm * 1000000 + c.bn * 1000 + c.bk) sh = c;
    return plan_shape(p, sh, fmt, O, I, S, gs);
}

hipError_t launch_tiled(int fmt, const TiledPlan &p, const TiledArgs &a, hipStream_t st) {
    switch (fmt) {
    case WQ_F32: return launch_fmt<WQ_F32>(p, a, st);
    case WQ_I8: return launch_fmt<WQ_I8>(p, a, st);
    case WQ_I4: return launch_fmt<WQ_I4>(p, a, st);
    case WQ_I2: return launch_fmt<WQ_I2>(p, a, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace wq
