// Internal declarations of libwqmm: tensor/group objects, the device weight
// layout, launch plans and kernel argument blocks shared by the runtime and
// the kernel files.
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
constexpr int kMaxTeam = 8;                    // waves that may share one row
constexpr int kTeamChunk = 32;                 // rows a team collects in LDS between barriers

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

// ---------------------------------------------------------------------------
// Device weight layout (library-private).
//
// Rows are stored one after another with a stride rounded up to 16 bytes
// (padding zeroed). f32 rows keep their natural order. For int8/int4/int2
// every complete 1024-byte block of a row is a permutation of its bytes:
// with epb elements per byte and G = 16 * epb elements per 16-byte granule,
// field n (0 <= n < G, low bits of a byte first, bytes in order) of granule
// lambda (0 <= lambda < 64) holds element
//
//     block_base + 256 * (n / 4) + 4 * lambda + (n % 4).
//
// A wave whose 64 lanes read the 64 granules of a block therefore needs, for
// each n / 4, the 256 consecutive activations [block_base + 256 m, +256):
// every activation load is one fully coalesced 1 KiB access, and the
// activations live in registers in the same order as the weight fields.
// Four consecutive fields n = 4m .. 4m+3 are four consecutive elements, and
// each stored byte holds whole consecutive elements, so the permutation moves
// bytes only. The last partial block of a row (if any) keeps natural order.
constexpr int kBlockBytes = 1024;

// Elements per byte, or 0 for f32 (4 bytes per element).
__host__ __device__ inline int elems_per_byte(int fmt) {
    return fmt == WQ_I8 ? 1 : fmt == WQ_I4 ? 2 : fmt == WQ_I2 ? 4 : 0;
}

// Full permuted blocks per row.
__host__ __device__ inline int full_blocks(int fmt, long rb) {
    return elems_per_byte(fmt) == 0 ? 0 : (int)(rb / kBlockBytes);
}

// Source byte (natural order, within the row) of device byte p.
__host__ __device__ inline long natural_byte_of(int fmt, long p, int nfull) {
    const int epb = elems_per_byte(fmt);
    if (epb == 0 || p >= (long)nfull * kBlockBytes) return p;
    const long base = p / kBlockBytes * kBlockBytes;
    const int r = (int)(p - base);
    const int lambda = r >> 4, q = r & 15;
    const int n0 = q * epb;                                 // first field of the byte
    const long e0 = 256L * (n0 >> 2) + 4 * lambda + (n0 & 3); // element within the block
    return base + e0 / epb;
}

// Element index of the first of four consecutive fields starting at field
// position P (P a multiple of 4) of a row; positions count fields in device
// order (P = byte * epb + field; for f32, P = byte / 4).
__host__ __device__ inline long elem_of_pos4(int fmt, long P, int nfull) {
    const int epb = elems_per_byte(fmt);
    if (epb == 0) return P;
    const long per_block = (long)kBlockBytes * epb;
    if (P >= (long)nfull * per_block) return P;
    const long b = P / per_block;
    const int r = (int)(P - b * per_block);
    const int G = 16 * epb;
    const int lambda = r / G, n = r % G;
    return b * per_block + 256L * (n >> 2) + 4 * lambda;
}

} // namespace wq

struct wq_tensor {
    uint32_t magic;
    int device, fmt, O, I;
    long rb;      // packed host row bytes
    long stride;  // device row stride (rb rounded up to kRowAlign; padding zeroed)
    int nfull;    // permuted 1 KiB blocks per row (0 for group-scaled tensors: natural order)
    int gs;       // group size of the scales (0: one scale per row)
    int ng;       // scales per row (1, or ceil(I / gs))
    uint8_t *d_w;
    float *d_scales;   // O x ng floats (row-major: one row's groups together)
    float *d_scales_t; // gs > 0: the same scales group-major, ng x O (tiled path)
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
    int d = 0;      // rows in flight per wave (ring depth)
    int team = 0;   // waves cooperating on one row
    int teams_per_block = 0;
    int block = 0;
    int grid = 0;
    int rows_per_team = 0;
    bool ok = false;
};

// Group-wise scales (gs > 0): rows are in natural element order, gs is a
// multiple of kGroupAlign, so every lane slot (at most 64 elements) and every
// 64-position tiled K step lies inside one group. The GEMV reads
// scales[o * ng + g]; the tiled kernel reads a group-major copy,
// scales[g * O + o], so one tile's rows share cache lines.
constexpr int kGroupAlign = 64;

struct GemvArgs {
    const uint8_t *w;
    const float *scales;
    const float *x;
    float *y;
    long stride;
    int nfull;
    int gs, ng;       // group-wise scales (gs == 0: one scale per row)
    int O, I, S;
    int k;             // load slots per lane per row
    int team;          // waves per team
    int teams_per_block;
    int rows_per_team;
    // paired rows (gated feed-forward): up rows and scales; O then counts
    // virtual rows (2 x output rows) and y receives silu(g) * u, S x O/2
    const uint8_t *w2 = nullptr;
    const float *scales2 = nullptr;
};

// Kernel shape for (fmt, S bucket): bytes per lane load, compiled slot count,
// ring depth of the grouped launch (d) and of the single-tensor GEMV (dg),
// and the GEMV's default waves per CU (wg). Row coverage per wave =
// 64 * lw * kmax bytes.
struct GemvShape {
    int lw, kmax, d, dg, wg;
};
GemvShape gemv_shape(int fmt, int smax);

// Rows in flight per wave for a row that needs ks of the kmax load slots a
// shape compiles: a shorter row's ring reuses the registers of the unused
// slots for more rows (d * kmax / ks rounded down to 1x, 2x or 4x), so each
// wave keeps about the same number of bytes in flight.
__host__ __device__ constexpr int ring_depth(int kmax, int d, int ks) {
    return d * (kmax >= 4 * ks ? 4 : kmax >= 2 * ks ? 2 : 1);
}
int gemv_smax_bucket(int S); // 1,2,4,8 or 0 if S > 8

// Up to the shape's slots per lane, a team of waves sharing a longer row.
// waves_per_cu <= 0: the shape's default.
GemvPlan plan_gemv(int fmt, int O, int I, int S, int cus, int waves_per_cu);
hipError_t launch_gemv(const GemvPlan &p, const GemvArgs &a, hipStream_t st);  // a.gs, a.w2 select the variant

// h[j] = silu(h[j]) * u[j], j < n (gated feed-forward after separate gate and up matmuls)
hipError_t launch_gated_inplace(float *h, const float *u, long n, hipStream_t st);

// ---------------------------------------------------------------------------
// Grouped GEMV: one launch over several tensors of one format.

struct GroupDesc {
    const uint8_t *w;
    const float *scales;
    const uint8_t *w2;      // paired groups: the up tensor (same shape); else null
    const float *scales2;
    long stride;
    int nfull;
    int O, I;  // output rows (a paired problem has 2 * O virtual rows)
    int pad;
};

struct WorkItem {
    int p;         // problem index within the launch
    int row_begin; // rows (virtual rows for a paired group)
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
    int smax = 0, lw = 0, kmax = 0, d = 0;
    int n_items = 0, grid = 0, block = 256;
};

// xv: every activation pointer 16-byte aligned and every I a multiple of 4.
// pair: every problem is a (gate, up) pair and y receives silu(g) * u.
// ks: the slot count (WorkItem::k, 1..p.kmax) shared by every item of the
// launch, or 0 when the launch mixes slot counts (each item carries its own).
hipError_t launch_grouped(int fmt, const GroupedPlan &p, const GroupedArgs &a, bool xv, bool pair, int ks,
                          hipStream_t st);

// ---------------------------------------------------------------------------
// LDS-tiled dequant + MFMA path (any S).

struct TiledArgs {
    const uint8_t *w;
    const float *scales;
    const float *x;
    float *y;
    long stride;
    int nfull;
    int gs, ng;       // group-wise scales (gs == 0: one scale per row)
    int O, I, S;
    int tiles_s, tiles_o;
    // bf16x3 mode: workspace holding the three activation planes
    const uint16_t *xp;
    long plane;  // bf16 elements per plane (sp * kp)
    int kp;      // bf16 elements per plane row
    // split K (bf16x3, ksplit > 1): block (tile, c) sums K steps
    // [c * nk / ksplit, (c + 1) * nk / ksplit) into part[c][S][O]; a
    // second kernel adds the ksplit partials in order c = 0.. and writes y
    int ksplit = 1;
    float *part = nullptr;
};

constexpr int kTiledF32 = 0;     // fp32 operands, v_mfma_f32_16x16x4_f32
constexpr int kTiledBF16X3 = 1;  // exact 3-way bf16 split of x, v_mfma_f32_16x16x32_bf16
constexpr int kTiledBF16 = 2;    // opt-in: x rounded to the nearest bf16 (one plane), same MFMA
constexpr int kTiledKAlign = 128; // plane rows padded (with zeros) to this many positions
constexpr int kTiledSAlign = 128; // planes padded (with zero rows) to this many rows

struct TiledPlan {
    int mode = kTiledF32;
    int bm = 64, bn = 64, bk = 32;
    int tiles_s = 0, tiles_o = 0, grid = 0, block = 256;
    int sp = 0, kp = 0;   // bf16x3: plane rows and row length
    int ksplit = 1;       // bf16x3: K chunks per tile (grid = tiles * ksplit)
    size_t part_off = 0;  // split K: byte offset of the partials in the workspace
    size_t ws_bytes = 0;  // device workspace the call needs (bf16x3: 3 planes, bf16: 1 [+ partials])
};
constexpr int kTiledSplitWaves = 2048;  // split K until the grid holds this many waves (8 per CU)
constexpr int kTiledMinChunk = 4;       // K steps per chunk at least

// shape: 0 picks by size; bm * 1000000 + bn * 1000 + bk forces a compiled tile shape
// gs > 0 (group-wise scales) always takes the bf16x3 mode
TiledPlan plan_tiled(int fmt, int O, int I, int S, int mode, int shape, int gs = 0);
hipError_t launch_tiled(int fmt, const TiledPlan &p, const TiledArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Few activation rows (S <= 32) on the matrix cores: one launch, no
// workspace (skinny_kernel.h, skinny_kernels.hip, skinny_wide_*.hip). Needs x
// 16-byte aligned and I % 4 == 0.

struct SkinnyArgs {
    const uint8_t *w;
    const float *scales;
    const float *x;
    float *y;
    long stride;
    int nfull;
    int O, I, S;
    int chunks_per_wave;  // 128-position chunks each wave streams (even)
    int nchunks;          // chunks per row (even): chunks past it hold no field positions
    // group-wise scales (gs > 0): ng x O, group-major; scales is then unused
    const float *gscales_t = nullptr;
    int gs = 0, ng = 1;
};

constexpr int kSkinnyMaxS = 32;  // activation rows the few-rows kernel takes at most

struct SkinnyPlan {
    bool ok = false;
    int m = 0;       // stacked operand fragments: 1 (S <= 5), 2 (S <= 10), 3 (S <= 16), 4..6 (S <= 32)
    int rpl = 0;     // activation runs per lane per chunk: ceil(S / 4) (5, 6 or 8 above S = 16)
    int nb = 0;      // 16-row output blocks per block
    int waves = 0;   // waves per block, each streaming its own chunks of the rows
    int ring = 0;    // chunks of loads in flight per wave
    int grid = 0;
    int nchunks = 0;          // chunks per row (even)
    int chunks_per_wave = 0;
};
// ring: 4 or 6 asks for that many chunks of loads in flight per wave (capped
// at the deepest spill-free ring; 8-wave blocks only), else 2
// gs > 0: group-wise scales (S <= 16 and gs a multiple of the positions one
// chunk spans: 128 for int8/int4, 256 for int2; otherwise not ok).
SkinnyPlan plan_skinny(int fmt, int O, int I, int S, int cus, int ring, int gs = 0);
hipError_t launch_skinny(int fmt, const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st);

// ---------------------------------------------------------------------------
// Stream-read calibration: `waves` waves (a multiple of 4) each read one
// contiguous chunk of the buffer with `loads` 1 KiB loads in flight; out
// receives 64 words per wave.
hipError_t launch_stream_read(const void *buf, size_t bytes, int waves, int loads, uint32_t *out, hipStream_t st);

// ---------------------------------------------------------------------------
// Upload: natural packed rows (O x rb, device) -> device layout (O x stride).
hipError_t launch_relayout(int fmt, const uint8_t *src, uint8_t *dst, int O, long rb, long stride, int nfull,
                           hipStream_t st);

} // namespace wq

struct wq_group {
    uint32_t magic;
    int device, fmt, G;
    std::vector<wq_tensor *> ts;
    std::vector<wq_tensor *> ts2;  // paired (gated feed-forward) group: the up tensors; else empty
    std::vector<wq::GroupDesc> h_desc;
    wq::GroupDesc *d_desc;
    bool has_gs = false;  // a group-scaled tensor is present: one launch per tensor
    // per S bucket (index 0..3 for 1,2,4,8): work table on the device
    struct Bucket {
        bool built = false;
        wq::GroupedPlan plan;
        // per launch segment (the problems of one chunk of at most
        // kGroupMaxPerLaunch problems, whatever their row lengths):
        std::vector<int> seg_chunk;            // chunk index (problems chunk*64 ..)
        std::vector<int> first_item;           // first item index
        std::vector<int> n_items;
        std::vector<int> ks;                   // slot count of every item of the segment, or 0 (mixed)
        std::vector<uint64_t> mask;            // problems of the chunk in the segment
        wq::WorkItem *d_items = nullptr;
    } buckets[4];
};
