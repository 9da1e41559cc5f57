// Few activation rows (S <= 32) on the matrix cores: planner and launches.
// The kernel and its design notes are in skinny_kernel.h; the 4-wave
// variants for 17 <= S <= 32 are compiled in skinny_wide_*.hip.
#include "skinny_kernel.h"

namespace wq {

// 16 waves of one 16-row block (for few output rows) keep every value in
// registers at four waves per SIMD (from the compiled register counts).
constexpr bool skinny_wide_ok(int fmt, int m, int rpl) {
    return (m == 1 && rpl == 1) || (m == 2 && rpl == 2) || (m == 1 && rpl == 2 && fmt != WQ_I8) ||
           (m == 2 && rpl == 3 && fmt == WQ_I2);
}
namespace {

template <int FMT, int M, int RPL>
hipError_t launch_mr(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
    const dim3 grid(p.grid), block(64 * p.waves);
    if (a.gs > 0) {  // group-wise scales: two chunks in flight
#define WQ_SKG(NB_, W_)                                                                                         \
    if constexpr (skinny_gs_ok(FMT, M, RPL, NB_, W_)) {                                                         \
        if (p.nb == NB_ && p.waves == W_ && p.ring == 2) {                                                      \
            hipLaunchKernelGGL((skinny_kernel<FMT, M, RPL, NB_, W_, 2, skinny_nbuf(M, NB_, W_), true>), grid, \
                               block, 0, st, a);                                                                \
            return hipGetLastError();                                                                           \
        }                                                                                                       \
    }
        WQ_SKG(1, 8) WQ_SKG(2, 8) WQ_SKG(3, 8) WQ_SKG(4, 8) WQ_SKG(3, 4) WQ_SKG(4, 4)
#undef WQ_SKG
        return hipErrorInvalidValue;
    }
#define WQ_SK(NB_, W_, R_)                                                                           \
    if (p.nb == NB_ && p.waves == W_ && p.ring == R_) {                                              \
        hipLaunchKernelGGL((skinny_kernel<FMT, M, RPL, NB_, W_, R_, skinny_nbuf(M, NB_, W_)>), grid, \
                           block, 0, st, a);                                                         \
        return hipGetLastError();                                                                    \
    }
#define WQ_SKR(NB_, R_) \
    if constexpr (skinny_max_ring(FMT, M, RPL, NB_) >= R_) WQ_SK(NB_, 8, R_)
    WQ_SKR(1, 2) WQ_SKR(2, 2) WQ_SKR(3, 2) WQ_SKR(4, 2)
    WQ_SKR(1, 4) WQ_SKR(2, 4) WQ_SKR(3, 4) WQ_SKR(4, 4)
    WQ_SKR(1, 6) WQ_SKR(2, 6) WQ_SKR(3, 6) WQ_SKR(4, 6)
#define WQ_SKW(NB_, W_) \
    if constexpr (skinny_wide_ok(FMT, M, RPL)) WQ_SK(NB_, W_, 2)
    WQ_SKW(1, 16)
#undef WQ_SKW
#undef WQ_SKR
#undef WQ_SK
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_f(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
    switch (p.m * 10 + p.rpl) {
    case 11: return launch_mr<FMT, 1, 1>(p, a, st);
    case 12: return launch_mr<FMT, 1, 2>(p, a, st);
    case 22: return launch_mr<FMT, 2, 2>(p, a, st);
    case 23: return launch_mr<FMT, 2, 3>(p, a, st);
    case 33: return launch_mr<FMT, 3, 3>(p, a, st);
    case 34: return launch_mr<FMT, 3, 4>(p, a, st);
    default:  // 4-wave blocks, S > 16
        if (a.gs > 0) return hipErrorInvalidValue;
        return FMT == WQ_I8 ? launch_skinny_wide_i8(p, a, st)
             : FMT == WQ_I4 ? launch_skinny_wide_i4(p, a, st)
                            : launch_skinny_wide_i2(p, a, st);
    }
}

} // namespace

SkinnyPlan plan_skinny(int fmt, int O, int I, int S, int cus, int ring, int gs) {
    SkinnyPlan p;
    if ((fmt != WQ_I8 && fmt != WQ_I4 && fmt != WQ_I2) || O <= 0 || I < 4 || I % 4 != 0 || S < 1 ||
        S > kSkinnyMaxS)
        return p;
    // group-wise scales: a chunk's positions in one group, the 8-wave tiles
    if (gs < 0 || (gs > 0 && (S > 16 || gs % (fmt == WQ_I2 ? 2 * kChunk : kChunk) != 0 ||
                              (long)O * ((I + gs - 1) / gs) >= (1L << 31))))
        return p;
    const long stride = round_up(row_bytes(fmt, I), kRowAlign);
    const long npos = stride * elems_per_byte(fmt);
    long nchunks = (npos + kChunk - 1) / kChunk;
    nchunks = round_up(nchunks, 2);
    if (S <= 16) {
        p.m = S <= 5 ? 1 : S <= 10 ? 2 : 3;
        p.rpl = (S + 3) / 4;
        // Output blocks per block (of the compiled ones): the fewest rounds
        // of one block per CU, weighed against bigger blocks (each block also
        // loads and splits all of x, about one output block's worth): cost =
        // rounds * (1 + nb). A second round costs more than idle CUs: int8
        // 6144 x 6144 at S = 8, 16.3 us on 192 blocks of 32 rows against 20.5
        // on 384 of 16; int4 6144 x 6144 13.2 against 18.3.
        const long row_blocks = ((long)O + 15) / 16;
        p.nb = 1;
        p.waves = 8;
        if (row_blocks < cus) {  // few output rows: more waves per block share each row's chunks
            if (skinny_wide_ok(fmt, p.m, p.rpl) && gs == 0) p.waves = 16;
        } else {
            long best = -1;
            for (int nb = 1; nb <= 4; ++nb) {
                if (skinny_max_ring(fmt, p.m, p.rpl, nb) == 0) continue;
                if (gs > 0 && !skinny_gs_ok(fmt, p.m, p.rpl, nb, 8)) continue;
                const long blocks = (row_blocks + nb - 1) / nb;
                const long cost = (blocks + cus - 1) / cus * (1 + nb);
                if (best < 0 || cost < best) {
                    best = cost;
                    p.nb = nb;
                }
            }
            // group-scaled three-fragment tiles: when the 8-wave blocks that
            // keep their registers take more than one round, 4-wave blocks
            // of three or four output blocks at one wave per SIMD
            if (gs > 0 && p.m == 3 && (row_blocks + p.nb - 1) / p.nb > cus) {
                for (int nb = 3; nb <= 4; ++nb)
                    if (skinny_gs_ok(fmt, p.m, p.rpl, nb, 4) && (row_blocks + nb - 1) / nb <= cus) {
                        p.nb = nb;
                        p.waves = 4;
                        break;
                    }
            }
        }
        // two chunks of loads in flight (the fastest measured), or a deeper
        // spill-free ring when asked for
        const int deepest = skinny_max_ring(fmt, p.m, p.rpl, p.nb);
        p.ring = (p.waves == 8 && gs == 0 && (ring == 4 || ring == 6)) ? std::min(ring, deepest) : 2;
    } else {
        // 17 <= S <= 32: four waves per block (their operand buffers fit in
        // LDS; one block per CU), compiled tiles (m, rpl) = (4, 5), (5, 6),
        // (6, 8). The fewest output blocks per block that keep the grid to
        // one block per CU (a second round of blocks costs more than bigger
        // blocks: int2 16384 x 8192 at S = 20, 37.6 us with 4 output blocks,
        // 57.0 with 2, 62.8 with 3); where no compiled size does, m >= 5
        // leaves it to the tiled kernel (within 3 % at S = 24: 66.6 vs
        // 65.0 us on two rounds of 4-wave blocks; faster at S = 32: 68.1 vs
        // 81.2 us).
        p.m = S <= 20 ? 4 : S <= 24 ? 5 : 6;
        p.rpl = S <= 20 ? 5 : S <= 24 ? 6 : 8;
        const int nbmax = p.m == 6 ? 3 : 4;
        const long row_blocks = ((long)O + 15) / 16;
        p.nb = 0;
        for (int nb = 1; nb <= nbmax && p.nb == 0; ++nb)
            if ((row_blocks + nb - 1) / nb <= cus) p.nb = nb;
        if (p.nb == 0) {
            if (p.m >= 5) return p;
            p.nb = nbmax;
        }
        p.waves = 4;
        p.ring = 2;
    }
    p.grid = (O + 16 * p.nb - 1) / (16 * p.nb);
    const long per_wave = (nchunks + p.waves - 1) / p.waves;
    p.chunks_per_wave = (int)round_up(per_wave, 2);
    p.nchunks = (int)nchunks;
    // 32-bit offsets inside the kernel
    p.ok = (long)O * stride < (1L << 31) && (long)S * I < (1L << 29) && nchunks * kChunk < (1L << 30);
    return p;
}

hipError_t launch_skinny(int fmt, const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
    switch (fmt) {
    case WQ_I8: return launch_f<WQ_I8>(p, a, st);
    case WQ_I4: return launch_f<WQ_I4>(p, a, st);
    case WQ_I2: return launch_f<WQ_I2>(p, a, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace wq
