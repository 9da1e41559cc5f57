// Grouped few-rows launch: the tensors of a group (one format, 2..16
// activation rows each) in one launch of the few-rows matrix-core kernel
// (grouped expert matmuls of a mixture-of-experts step with several tokens
// per expert; grouped expert handling at prefill: colibri docs "CUDA
// backend (Linux)", section "The GPU-resident pipeline").
#pragma once
#include "wq_internal.h"

namespace wq {

// One tensor of a grouped few-rows launch; blocks [block_end of the previous
// entry, block_end) work on it (16 * nb output rows each).
struct SkinnyGroupDesc {
    const uint8_t *w;
    const float *scales;
    const float *x;
    float *y;
    int stride, nfull, O, I, S, nchunks, chunks_per_wave, block_end;
    // launches with group-wise scales: ng x O group-major scales and the
    // group size (a tensor with one scale per row: its scales, gs = 1 << 30,
    // ng = 1)
    const float *gscales_t;
    int gs, ng;
};

constexpr int kSkinnyGroupMax = 32;  // tensors per launch (2 KiB of kernel arguments)

struct SkinnyGroupArgs {
    int n;
    SkinnyGroupDesc t[kSkinnyGroupMax];
};

struct SkinnyGroupPlan {
    bool ok = false;
    int m = 0, rpl = 0, nb = 0;  // tile for the largest S of the launch
    int waves = 8;               // 8-wave blocks up to S = 16, 4-wave blocks above
    bool gs = false;             // the group-scaled kernel (per-chunk accumulators)
    int grid = 0;
};

// Plan for n tensors (S[i] >= 1) of one format; fills each
// descriptor's nchunks, chunks_per_wave and block_end (the caller fills the
// pointers, shape, S and, with gs, the group fields). Not ok when a tensor
// cannot take the few-rows kernel (S > 32, or S > 16 with group scales,
// I % 4 != 0, 32-bit offsets, a group size that is not a multiple of a
// chunk's span).
SkinnyGroupPlan plan_skinny_group(int fmt, SkinnyGroupDesc *t, int n, int cus, bool gs = false);
hipError_t launch_skinny_group(int fmt, const SkinnyGroupPlan &p, const SkinnyGroupArgs &a, hipStream_t st);

// The activation step of several experts' gated feed-forward in one launch:
// h_e[j] = silu(h_e[j]) * u_e[j] for j < count_e (h_e holds the gate
// product on entry, u_e the up product).
struct GatedGroupArgs {
    int n;
    struct {
        float *h;
        const float *u;
        int count;
    } e[kSkinnyGroupMax];
};
hipError_t launch_gated_group(const GatedGroupArgs &a, int max_count, hipStream_t st);

} // namespace wq
