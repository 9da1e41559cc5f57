// Register GEMV for S <= 8 and its grouped (many tensors, one launch) form.
//
// y[s,o] = scale[o] * sum_i dequant(W[o,i]) * x[s,i]
//   (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四, qmatmul.comp
//    header; dequant rules from colibri-analysis "CUDA 后端", section 1,
//    weight_at; scale after the sum, same section, quant_matmul)
//
// Design (gfx950, wave64):
//  * A "team" of 1..8 waves owns a set of consecutive output rows. Each lane
//    owns fixed byte slices of every row: slot k covers bytes
//    [(k*team_lanes + lane)*LW, +LW), so one wave-wide load is LW*64
//    contiguous bytes (1 KiB for LW = 16) of the row, read once, non-temporal.
//  * The activations of a lane's columns are loaded once into registers
//    (SMAX rows of them) and reused for every row the team processes; the
//    weight stream is the only per-row memory traffic.
//  * Dequantization happens in registers on 32-bit words. For int4 and int2
//    the code offset is folded out of the inner loop: codes are converted
//    unshifted (byte masks + v_cvt_f32_ubyteN, with the activations of the
//    higher fields pre-divided by 16 / 4^k, exact powers of two) and
//    offset * sum(x) is subtracted once per lane. The lane's sum(x) is formed
//    in the same order as the FMA chain, so a row whose codes all decode to
//    zero gives exactly 0.
//  * Lanes are reduced with DPP (quad_perm, row_shr, row_bcast) instead of an
//    LDS tree; teams of several waves add their wave totals through LDS in a
//    fixed order, so results are deterministic.
#include "wq_internal.h"

namespace wq {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int FMT> struct FmtInfo;
template <> struct FmtInfo<WQ_F32> { static constexpr int EPW = 1;  static constexpr int OFF = 0; };
template <> struct FmtInfo<WQ_I8>  { static constexpr int EPW = 4;  static constexpr int OFF = 0; };
template <> struct FmtInfo<WQ_I4>  { static constexpr int EPW = 8;  static constexpr int OFF = 8; };
template <> struct FmtInfo<WQ_I2>  { static constexpr int EPW = 16; static constexpr int OFF = 2; };

// Factor applied to the activation that meets element e (0..EPW-1) of a word,
// compensating the unshifted field position used by the folded dequant.
template <int FMT> __device__ constexpr float x_prescale(int e) {
    if (FMT == WQ_I4) return (e & 1) ? 0.0625f : 1.0f;
    if (FMT == WQ_I2) {
        const int f = e & 3;
        return f == 0 ? 1.0f : f == 1 ? 0.25f : f == 2 ? 0.0625f : 0.015625f;
    }
    return 1.0f;
}

template <int LW> __device__ __forceinline__ void load_w(const uint8_t *p, uint32_t (&v)[LW / 4]) {
    if constexpr (LW == 16) {
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    } else if constexpr (LW == 8) {
        const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
        v[0] = t.x; v[1] = t.y;
    } else {
        v[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
    }
}

// Keeps the compiler from pushing a byte mask into each field extraction
// (which would turn one v_cvt_f32_ubyteN into v_bfe_u32 + v_cvt_f32_ubyte0).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// acc[s] += sum over the EPW elements of one word of code * xw[e][s].
template <int FMT, int SMAX>
__device__ __forceinline__ void word_fma(uint32_t w, const float (*xw)[SMAX], float (&acc)[SMAX]) {
    if constexpr (FMT == WQ_F32) {
        const float q = __uint_as_float(w);
#pragma unroll
        for (int s = 0; s < SMAX; ++s) acc[s] = __builtin_fmaf(q, xw[0][s], acc[s]);
    } else if constexpr (FMT == WQ_I8) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float q = (float)(int)(int8_t)(w >> (8 * b));
#pragma unroll
            for (int s = 0; s < SMAX; ++s) acc[s] = __builtin_fmaf(q, xw[b][s], acc[s]);
        }
    } else if constexpr (FMT == WQ_I4) {
        const uint32_t lo = opaque(w & 0x0F0F0F0Fu);  // even elements, code in bits 0..3 of each byte
        const uint32_t hi = opaque(w & 0xF0F0F0F0u);  // odd elements, 16 * code
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float cl = (float)((lo >> (8 * b)) & 0xFFu);
            const float ch = (float)((hi >> (8 * b)) & 0xFFu);
#pragma unroll
            for (int s = 0; s < SMAX; ++s) {
                acc[s] = __builtin_fmaf(cl, xw[2 * b][s], acc[s]);
                acc[s] = __builtin_fmaf(ch, xw[2 * b + 1][s], acc[s]);
            }
        }
    } else {  // WQ_I2
        const uint32_t m0 = opaque(w & 0x03030303u);
        const uint32_t m1 = opaque(w & 0x0C0C0C0Cu);
        const uint32_t m2 = opaque(w & 0x30303030u);
        const uint32_t m3 = opaque(w & 0xC0C0C0C0u);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float c0 = (float)((m0 >> (8 * b)) & 0xFFu);
            const float c1 = (float)((m1 >> (8 * b)) & 0xFFu);
            const float c2 = (float)((m2 >> (8 * b)) & 0xFFu);
            const float c3 = (float)((m3 >> (8 * b)) & 0xFFu);
#pragma unroll
            for (int s = 0; s < SMAX; ++s) {
                acc[s] = __builtin_fmaf(c0, xw[4 * b + 0][s], acc[s]);
                acc[s] = __builtin_fmaf(c1, xw[4 * b + 1][s], acc[s]);
                acc[s] = __builtin_fmaf(c2, xw[4 * b + 2][s], acc[s]);
                acc[s] = __builtin_fmaf(c3, xw[4 * b + 3][s], acc[s]);
            }
        }
    }
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

// Sum over the 64 lanes; the total lands in lane 63.
__device__ __forceinline__ float wave_sum_lane63(float v) {
    v += dpp_move<0xB1>(v);        // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v);        // quad_perm [2,3,0,1]
    v += dpp_move<0x114>(v);       // row_shr:4
    v += dpp_move<0x118>(v);       // row_shr:8
    v += dpp_move<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_move<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// One team processes rows [row_begin, row_end).
template <int FMT, int SMAX, int LW, int KMAX, int R>
__device__ __forceinline__ void team_rows(const uint8_t *__restrict__ w, long stride,
                                          const float *__restrict__ scales,
                                          const float *__restrict__ x, float *__restrict__ y, int O,
                                          int I, int S, int K, int team, int tl, int wave_in_team,
                                          int row_begin, int row_end, float *red) {
    constexpr int EPW = FmtInfo<FMT>::EPW;
    constexpr int OFF = FmtInfo<FMT>::OFF;
    constexpr int WPC = LW / 4;     // 32-bit words per lane load
    constexpr int EPC = WPC * EPW;  // elements per lane load
    const int team_lanes = team * 64;
    const int lane = threadIdx.x & 63;

    // ---- stage this lane's activations in registers (pre-scaled), and sum(x)
    float xr[KMAX][EPC][SMAX];
    float sx[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) sx[s] = 0.0f;
    const bool vec_ok = ((I & 3) == 0) && ((reinterpret_cast<uintptr_t>(x) & 15) == 0);
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const long cb = (long)(k * team_lanes + tl) * LW;
        const long e0 = cb / 4 * EPW;
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            float v[EPC];
#pragma unroll
            for (int e = 0; e < EPC; ++e) v[e] = 0.0f;
            if (k < K && s < S) {
                const float *xs = x + (long)s * I + e0;
                if (vec_ok && e0 + EPC <= I) {
#pragma unroll
                    for (int e = 0; e < EPC; e += 4) {
                        const float4 t = *reinterpret_cast<const float4 *>(xs + e);
                        v[e] = t.x; v[e + 1] = t.y; v[e + 2] = t.z; v[e + 3] = t.w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPC; ++e)
                        if (e0 + e < I) v[e] = xs[e];
                }
            }
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                xr[k][e][s] = v[e] * x_prescale<FMT>(e % EPW);
                if constexpr (OFF != 0) sx[s] += v[e];
            }
        }
    }

    // ---- stream rows
    for (int row0 = row_begin; row0 < row_end; row0 += R) {
        uint32_t wv[R][KMAX][WPC];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int o = min(row0 + r, row_end - 1);
            const uint8_t *p = w + (long)o * stride;
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                const long cb = (long)(k * team_lanes + tl) * LW;
                if (k < K && cb < stride) {
                    load_w<LW>(p + cb, wv[r][k]);
                } else {
#pragma unroll
                    for (int j = 0; j < WPC; ++j) wv[r][k][j] = 0u;
                }
            }
        }
        float acc[R][SMAX];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int s = 0; s < SMAX; ++s) acc[r][s] = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (k < K) {
#pragma unroll
                    for (int j = 0; j < WPC; ++j) word_fma<FMT, SMAX>(wv[r][k][j], &xr[k][j * EPW], acc[r]);
                }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int s = 0; s < SMAX; ++s) {
                float t = acc[r][s];
                if constexpr (OFF != 0) t -= (float)OFF * sx[s];
                acc[r][s] = wave_sum_lane63(t);
            }
        if (team == 1) {
            if (lane == 63) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int o = row0 + r;
                    if (o < row_end) {
                        const float sc = scales[o];
#pragma unroll
                        for (int s = 0; s < SMAX; ++s)
                            if (s < S) y[(long)s * O + o] = sc * acc[r][s];
                    }
                }
            }
        } else {
            if (lane == 63) {
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int s = 0; s < SMAX; ++s) red[(wave_in_team * R + r) * SMAX + s] = acc[r][s];
            }
            __syncthreads();
            if (wave_in_team == 0 && lane < R * SMAX) {
                const int r = lane / SMAX, s = lane % SMAX;
                float t = 0.0f;
                for (int wv2 = 0; wv2 < team; ++wv2) t += red[(wv2 * R + r) * SMAX + s];
                const int o = row0 + r;
                if (o < row_end && s < S) y[(long)s * O + o] = scales[o] * t;
            }
            __syncthreads();
        }
    }
}

constexpr int kMaxTeam = 8;

template <int FMT, int SMAX, int LW, int KMAX, int R>
__global__ __launch_bounds__(512) void gemv_kernel(GemvArgs a) {
    __shared__ float red[kMaxTeam * R * SMAX];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int team_in_block = wave / a.team;
    const int wave_in_team = wave - team_in_block * a.team;
    const int team_id = blockIdx.x * a.teams_per_block + team_in_block;
    const int row_begin = team_id * a.rows_per_team;
    if (row_begin >= a.O) return;  // uniform over the team (and the block when team > 1)
    const int row_end = min(a.O, row_begin + a.rows_per_team);
    team_rows<FMT, SMAX, LW, KMAX, R>(a.w, a.stride, a.scales, a.x, a.y, a.O, a.I, a.S, a.k, a.team,
                                      wave_in_team * 64 + lane, wave_in_team, row_begin, row_end, red);
}

template <int FMT, int SMAX, int LW, int KMAX, int R>
__global__ __launch_bounds__(256) void grouped_kernel(GroupedArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int item_id = blockIdx.x * 4 + wave;
    if (item_id >= a.n_items) return;
    const WorkItem it = a.items[item_id];
    const int p = __builtin_amdgcn_readfirstlane(it.p);
    const int S = a.S[p];
    if (S <= 0) return;
    const GroupDesc d = a.desc[p];
    team_rows<FMT, SMAX, LW, KMAX, R>(d.w, d.stride, d.scales, a.x[p], a.y[p], d.O, d.I, S, it.k, 1, lane, 0,
                                      it.row_begin, it.row_end, nullptr);
}

// ---- compiled shapes -------------------------------------------------------
// (fmt, S bucket) -> bytes per lane load, load slots, rows in flight.
// Register budget: KMAX * (LW/4 * EPW) * SMAX activation registers
// (64 for f32/int8, 128 for int4/int2).
#define WQ_SHAPES(X)                                   \
    X(WQ_F32, 1, 16, 16, 1) X(WQ_F32, 2, 16, 8, 2)     \
    X(WQ_F32, 4, 16, 4, 2) X(WQ_F32, 8, 16, 2, 2)      \
    X(WQ_I8, 1, 16, 4, 2) X(WQ_I8, 2, 16, 2, 2)        \
    X(WQ_I8, 4, 16, 1, 4) X(WQ_I8, 8, 8, 1, 4)         \
    X(WQ_I4, 1, 16, 4, 2) X(WQ_I4, 2, 16, 2, 2)        \
    X(WQ_I4, 4, 16, 1, 4) X(WQ_I4, 8, 8, 1, 4)         \
    X(WQ_I2, 1, 16, 2, 4) X(WQ_I2, 2, 16, 1, 4)        \
    X(WQ_I2, 4, 8, 1, 4) X(WQ_I2, 8, 4, 1, 4)

} // namespace

int gemv_smax_bucket(int S) {
    if (S <= 1) return 1;
    if (S <= 2) return 2;
    if (S <= 4) return 4;
    if (S <= 8) return 8;
    return 0;
}

GemvShape gemv_shape(int fmt, int smax) {
#define WQ_SHAPE_CASE(F, SM, LW, KM, R) \
    if (fmt == F && smax == SM) return GemvShape{LW, KM, R};
    WQ_SHAPES(WQ_SHAPE_CASE)
#undef WQ_SHAPE_CASE
    return GemvShape{0, 0, 0};
}

GemvPlan plan_gemv(int fmt, int O, int I, int S, int cus, int waves_per_cu) {
    GemvPlan p;
    p.fmt = fmt;
    p.smax = gemv_smax_bucket(S);
    if (p.smax == 0 || O <= 0 || I <= 0) return p;
    const GemvShape sh = gemv_shape(fmt, p.smax);
    if (sh.lw == 0) return p;
    p.lw = sh.lw;
    p.kmax = sh.kmax;
    p.r = sh.r;
    const long stride = round_up(row_bytes(fmt, I), kRowAlign);
    const long per_wave = 64L * sh.lw * sh.kmax;
    long team = (stride + per_wave - 1) / per_wave;
    if (team > kMaxTeam) return p;  // row too long for the register GEMV
    p.team = (int)team;
    p.k = (int)((stride + 64L * p.lw * p.team - 1) / (64L * p.lw * p.team));
    p.teams_per_block = (p.team == 1) ? 4 : 1;
    p.block = 64 * p.team * p.teams_per_block;
    // teams: enough waves to keep HBM busy, each with at least R rows
    const long want_teams = std::max(1L, (long)cus * waves_per_cu / p.team);
    const long max_teams = (O + p.r - 1) / p.r;
    long teams = std::min(want_teams, max_teams);
    long rpt = (O + teams - 1) / teams;
    rpt = (rpt + p.r - 1) / p.r * p.r;
    teams = (O + rpt - 1) / rpt;
    p.rows_per_team = (int)rpt;
    p.grid = (int)((teams + p.teams_per_block - 1) / p.teams_per_block);
    p.ok = true;
    return p;
}

hipError_t launch_gemv(const GemvPlan &p, const GemvArgs &a, hipStream_t st) {
#define WQ_LAUNCH_CASE(F, SM, LW, KM, R)                                                   \
    if (p.fmt == F && p.smax == SM) {                                                      \
        hipLaunchKernelGGL((gemv_kernel<F, SM, LW, KM, R>), dim3(p.grid), dim3(p.block), 0, \
                           st, a);                                                         \
        return hipGetLastError();                                                          \
    }
    WQ_SHAPES(WQ_LAUNCH_CASE)
#undef WQ_LAUNCH_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_grouped(int fmt, const GroupedPlan &p, const GroupedArgs &a, hipStream_t st) {
#define WQ_GLAUNCH_CASE(F, SM, LW, KM, R)                                                      \
    if (fmt == F && p.smax == SM) {                                                            \
        hipLaunchKernelGGL((grouped_kernel<F, SM, LW, KM, R>), dim3(p.grid), dim3(p.block), 0, \
                           st, a);                                                             \
        return hipGetLastError();                                                              \
    }
    WQ_SHAPES(WQ_GLAUNCH_CASE)
#undef WQ_GLAUNCH_CASE
    return hipErrorInvalidValue;
}

} // namespace wq
