// Internal declarations of libwqmm: tensor/group objects, launch plans and
// kernel argument blocks shared by the runtime and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "wqmm.h"

namespace wq {

constexpr uint32_t kTensorMagic = 0x57515431u; // "WQT1"
constexpr uint32_t kGroupMagic = 0x57514731u;  // "WQG1"
constexpr int kRowAlign = 16;                  // device row stride alignment (bytes)
constexpr int kGroupMaxPerLaunch = 64;         // problems passed by value per grouped launch

// Bits per stored element, by format code.
inline int fmt_bits(int fmt) {
    switch (fmt) {
    case WQ_F32: return 32;
    case WQ_I8: return 8;
    case WQ_I4: return 4;
    case WQ_I2: return 2;
    default: return 0;
    }
}

inline long row_bytes(int fmt, long I) {
    int b = fmt_bits(fmt);
    if (b == 0 || I < 0) return -1;
    return (I * b + 7) / 8;
}

inline long round_up(long v, long a) { return (v + a - 1) / a * a; }

} // namespace wq

struct wq_tensor {
    uint32_t magic;
    int device, fmt, O, I;
    long rb;      // packed host row bytes
    long stride;  // device row stride (rb rounded up to kRowAlign; padding zeroed)
    uint8_t *d_w;
    float *d_scales;
    size_t bytes; // device bytes held (weights + scales)
};

namespace wq {

// ---------------------------------------------------------------------------
// Register GEMV (S <= 8): plan and arguments.

struct GemvPlan {
    int fmt = 0;
    int smax = 0;   // S bucket the kernel is compiled for (1, 2, 4, 8)
    int lw = 0;     // bytes per lane per weight load (16, 8 or 4)
    int kmax = 0;   // load slots per lane per row compiled in
    int k = 0;      // load slots used for this row length
    int r = 0;      // rows in flight per team iteration
    int team = 0;   // waves cooperating on one row
    int teams_per_block = 0;
    int block = 0;
    int grid = 0;
    int rows_per_team = 0;
    bool ok = false;
};

struct GemvArgs {
    const uint8_t *w;
    const float *scales;
    const float *x;
    float *y;
    long stride;
    int O, I, S;
    int k;             // load slots per lane per row
    int team;          // waves per team
    int teams_per_block;
    int rows_per_team;
};

// Kernel shape for (fmt, S bucket): bytes per lane load, compiled slot count
// and rows in flight. Row coverage per wave = 64 * lw * kmax bytes.
struct GemvShape {
    int lw, kmax, r;
};
GemvShape gemv_shape(int fmt, int smax);
int gemv_smax_bucket(int S); // 1,2,4,8 or 0 if S > 8

GemvPlan plan_gemv(int fmt, int O, int I, int S, int cus, int waves_per_cu);
hipError_t launch_gemv(const GemvPlan &p, const GemvArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Grouped GEMV: one launch over several tensors of one format.

struct GroupDesc {
    const uint8_t *w;
    const float *scales;
    long stride;
    int O, I;
};

struct WorkItem {
    int p;         // problem index within the launch
    int row_begin;
    int row_end;
    int k;         // load slots for this problem's rows
};

struct GroupedArgs {
    const GroupDesc *desc;  // device table, indexed by problem (launch-local)
    const WorkItem *items;  // device table, one per wave
    int n_items;
    int pad;
    const float *x[kGroupMaxPerLaunch];
    float *y[kGroupMaxPerLaunch];
    int S[kGroupMaxPerLaunch];
};

struct GroupedPlan {
    bool ok = false;
    int smax = 0, lw = 0, kmax = 0, r = 0;
    int n_items = 0, grid = 0, block = 256;
};

hipError_t launch_grouped(int fmt, const GroupedPlan &p, const GroupedArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// LDS-tiled dequant + fp32 MFMA path (any S).

struct TiledArgs {
    const uint8_t *w;
    const float *scales;
    const float *x;
    float *y;
    long stride;
    int O, I, S;
    int tiles_s, tiles_o;
};

struct TiledPlan {
    int bm = 64, bn = 64, bk = 32;
    int tiles_s = 0, tiles_o = 0, grid = 0, block = 256;
};

TiledPlan plan_tiled(int fmt, int O, int I, int S);
hipError_t launch_tiled(int fmt, const TiledPlan &p, const TiledArgs &a, hipStream_t st);

} // namespace wq

struct wq_group {
    uint32_t magic;
    int device, fmt, G;
    std::vector<wq_tensor *> ts;
    std::vector<wq::GroupDesc> h_desc;
    wq::GroupDesc *d_desc;
    // per S bucket (index 0..3 for 1,2,4,8): work table on the device
    struct Bucket {
        bool built = false;
        wq::GroupedPlan plan;
        std::vector<int> first_item;           // per launch chunk: first item index
        std::vector<int> n_items;              // per launch chunk
        wq::WorkItem *d_items = nullptr;
    } buckets[4];
};
