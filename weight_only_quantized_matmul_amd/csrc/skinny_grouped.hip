// Grouped few-rows launch (skinny_group.h): every block finds its tensor in
// the launch's descriptor table and runs the few-rows kernel's block body
// (skinny_kernel.h) on it. One tile (stacked fragments and activation runs
// per lane) for the whole launch, sized for its largest S: a tensor with
// fewer rows leaves the extra operand rows zero, as a single launch does
// for S below its tile.
#include <climits>

#include "skinny_group.h"
#include "skinny_kernel.h"

namespace wq {

namespace {

template <int FMT, int M, int RPL, int NB, bool GS, int WAVES = 8>
__global__ __launch_bounds__(64 * WAVES) void skinny_group_kernel(SkinnyGroupArgs ga) {
    // the block's tensor (wave-uniform scan of at most kSkinnyGroupMax entries)
    const int b = blockIdx.x;
    int t = 0;
    while (t + 1 < ga.n && ga.t[t].block_end <= b) ++t;
    const SkinnyGroupDesc &d = ga.t[t];
    SkinnyArgs a;
    a.w = d.w;
    a.scales = d.scales;
    a.x = d.x;
    a.y = d.y;
    a.stride = d.stride;
    a.nfull = d.nfull;
    a.O = d.O;
    a.I = d.I;
    a.S = d.S;
    a.chunks_per_wave = d.chunks_per_wave;
    a.nchunks = d.nchunks;
    a.gscales_t = d.gscales_t;
    a.gs = d.gs;
    a.ng = d.ng;
    skinny_block<FMT, M, RPL, NB, WAVES, 2, skinny_nbuf(M, NB, WAVES), GS>(a, b - (t > 0 ? ga.t[t - 1].block_end : 0));
}

template <int FMT, int M, int RPL>
hipError_t launch_group_mr(const SkinnyGroupPlan &p, const SkinnyGroupArgs &a, hipStream_t st) {
#define WQ_SKGR(NB_)                                                                                          \
    if constexpr (skinny_ring_ok(FMT, M, RPL, NB_)) {                                                         \
        if (p.nb == NB_ && !p.gs) {                                                                           \
            hipLaunchKernelGGL((skinny_group_kernel<FMT, M, RPL, NB_, false>), dim3(p.grid), dim3(512), 0, st, \
                               a);                                                                            \
            return hipGetLastError();                                                                         \
        }                                                                                                     \
    }                                                                                                         \
    if constexpr (skinny_ring_ok(FMT, M, RPL, NB_) && skinny_gs_ok(FMT, M, RPL, NB_, 8)) {                    \
        if (p.nb == NB_ && p.gs) {                                                                            \
            hipLaunchKernelGGL((skinny_group_kernel<FMT, M, RPL, NB_, true>), dim3(p.grid), dim3(512), 0, st,  \
                               a);                                                                            \
            return hipGetLastError();                                                                         \
        }                                                                                                     \
    }
    WQ_SKGR(1) WQ_SKGR(2) WQ_SKGR(3) WQ_SKGR(4)
#undef WQ_SKGR
    return hipErrorInvalidValue;
}

// 17 <= S <= 32: 4-wave blocks at one wave per SIMD (the tiles of the
// single-tensor launch), one scale per row
template <int FMT, int M, int RPL>
hipError_t launch_group_wide(const SkinnyGroupPlan &p, const SkinnyGroupArgs &a, hipStream_t st) {
    if (p.gs || p.waves != 4) return hipErrorInvalidValue;
#define WQ_SKGW(NB_)                                                                                        \
    if (p.nb == NB_) {                                                                                      \
        hipLaunchKernelGGL((skinny_group_kernel<FMT, M, RPL, NB_, false, 4>), dim3(p.grid), dim3(256), 0, st, \
                           a);                                                                              \
        return hipGetLastError();                                                                           \
    }
    WQ_SKGW(1) WQ_SKGW(2) WQ_SKGW(3)
    if constexpr (M <= 5) { WQ_SKGW(4) }  // (m = 6 with four blocks would spill)
#undef WQ_SKGW
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_group_f(const SkinnyGroupPlan &p, const SkinnyGroupArgs &a, hipStream_t st) {
    switch (p.m * 10 + p.rpl) {
    case 45: return launch_group_wide<FMT, 4, 5>(p, a, st);
    case 56: return launch_group_wide<FMT, 5, 6>(p, a, st);
    case 68: return launch_group_wide<FMT, 6, 8>(p, a, st);
    case 11: return launch_group_mr<FMT, 1, 1>(p, a, st);
    case 12: return launch_group_mr<FMT, 1, 2>(p, a, st);
    case 22: return launch_group_mr<FMT, 2, 2>(p, a, st);
    case 23: return launch_group_mr<FMT, 2, 3>(p, a, st);
    case 33: return launch_group_mr<FMT, 3, 3>(p, a, st);
    case 34: return launch_group_mr<FMT, 3, 4>(p, a, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

SkinnyGroupPlan plan_skinny_group(int fmt, SkinnyGroupDesc *t, int n, int cus, bool gs) {
    SkinnyGroupPlan p;
    if ((fmt != WQ_I8 && fmt != WQ_I4 && fmt != WQ_I2) || n < 1 || n > kSkinnyGroupMax) return p;
    p.gs = gs;
    int smax = 0;
    for (int i = 0; i < n; ++i) {
        const SkinnyGroupDesc &d = t[i];
        if (d.S < 1 || d.S > kSkinnyMaxS || d.O <= 0 || d.I < 4 || d.I % 4 != 0) return p;
        if ((long)d.O * d.stride >= (1L << 31) || (long)d.S * d.I >= (1L << 29)) return p;
        if (gs && (d.gscales_t == nullptr || d.gs <= 0 || d.ng < 1 || d.gs % (fmt == WQ_I2 ? 2 * kChunk : kChunk) != 0 ||
                   (long)d.O * d.ng >= (1L << 31)))
            return p;
        smax = std::max(smax, d.S);
    }
    if (smax <= 16) {
        p.m = smax <= 5 ? 1 : smax <= 10 ? 2 : 3;
        p.rpl = (smax + 3) / 4;
        p.waves = 8;
    } else {  // the single-tensor launch's 4-wave tiles
        if (gs) return p;
        p.m = smax <= 20 ? 4 : smax <= 24 ? 5 : 6;
        p.rpl = smax <= 20 ? 5 : smax <= 24 ? 6 : 8;
        p.waves = 4;
    }
    // output blocks per block: the fewest rounds of one block per CU, weighed
    // against bigger blocks (each loads all of its tensor's x), as for one tensor
    long best = -1;
    for (int nb = 1; nb <= 4; ++nb) {
        if (p.waves == 8 && (!skinny_ring_ok(fmt, p.m, p.rpl, nb) || (gs && !skinny_gs_ok(fmt, p.m, p.rpl, nb, 8))))
            continue;
        if (p.waves == 4 && p.m == 6 && nb == 4) continue;
        long blocks = 0;
        for (int i = 0; i < n; ++i) blocks += ((long)t[i].O + 16 * nb - 1) / (16 * nb);
        const long cost = (blocks + cus - 1) / cus * (1 + nb);
        if (best < 0 || cost < best) {
            best = cost;
            p.nb = nb;
        }
    }
    if (p.nb == 0) return p;
    long end = 0;
    for (int i = 0; i < n; ++i) {
        SkinnyGroupDesc &d = t[i];
        const long npos = (long)d.stride * elems_per_byte(fmt);
        const long nchunks = round_up((npos + kChunk - 1) / kChunk, 2);
        if (nchunks * kChunk >= (1L << 30)) return p;
        d.nchunks = (int)nchunks;
        d.chunks_per_wave = (int)round_up((nchunks + p.waves - 1) / p.waves, 2);
        end += ((long)d.O + 16 * p.nb - 1) / (16 * p.nb);
        d.block_end = (int)end;
    }
    if (end > INT_MAX) return p;
    p.grid = (int)end;
    p.ok = true;
    return p;
}

hipError_t launch_skinny_group(int fmt, const SkinnyGroupPlan &p, const SkinnyGroupArgs &a, hipStream_t st) {
    if (!p.ok || a.n < 1 || a.n > kSkinnyGroupMax) return hipErrorInvalidValue;
    switch (fmt) {
    case WQ_I8: return launch_group_f<WQ_I8>(p, a, st);
    case WQ_I4: return launch_group_f<WQ_I4>(p, a, st);
    case WQ_I2: return launch_group_f<WQ_I2>(p, a, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace wq
