// Few activation rows (S <= 32) on the matrix cores, one launch, no workspace:
// the kernel template, included by the planner (skinny_kernels.hip) and by
// the 4-wave instantiations for 17 <= S <= 32 (skinny_wide_*.hip).
//
// y[s,o] = scale[o] * sum_i dequant(W[o,i]) * x[s,i]
//   (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四, qmatmul.comp
//    header; dequant rules from colibri-analysis "CUDA 后端", section 1,
//    weight_at; batched rows on matrix units: colibri docs "CUDA backend
//    (Linux)", section "The GPU-resident pipeline")
//
// With 2..32 activation rows the register GEMV spends S vector FMAs on
// every weight element and becomes ALU-bound; here the products run on
// v_mfma_f32_16x16x32_bf16 and the vector ALUs only decode the weights
// (about two instructions per element) and split the activations.
//
//  * Exact operands. Every activation is split by truncation into three
//    bf16 parts, x = b1 + b2 + b3 (b1 the top 8 significant bits, b2 the
//    next 8 of the remainder, b3 the rest: both subtractions are exact), and
//    every code becomes its exact value q (|q| <= 128 has at most 8
//    significant bits) -- int4 and int2 as 16 * q and 64 * q, the factor
//    removed from the finished sum. Each MFMA product b * q is exact; only
//    the fp32 accumulation rounds, so the error is bounded by
//    sum |q * x| like any fp32 sum.
//  * Planes stacked into the MFMA's 16 rows: stacked row p * S + s holds
//    part p of activation row s, so S <= 5 needs one MFMA per 16 x 32 weight
//    tile (S <= 10 two, S <= 16 three, up to six for S <= 32); y[s] adds rows
//    s, S + s and 2S + s.
//  * Weights straight into operand registers, in the device layout that the
//    GEMV streams (no second copy): the contraction runs over field
//    positions, and a lane's 16-byte load of one row holds, for its group
//    of 8 positions per k-step, the codes of several consecutive k-steps;
//    the activations are paired with the same positions.
//  * A block of WAVES waves owns 16 * NB output rows and deals the rows'
//    128-position chunks to its waves in pairs, in turn (neighbouring pairs
//    go to different waves, so the block reads each row front to back);
//    each wave streams its pairs with the weight and activation loads of R
//    chunks in flight, splits its activations into a wave-private LDS
//    buffer laid out as MFMA operands (all 64 lanes split; no block barrier
//    per step), and the waves' partial tiles are added through LDS at the
//    end in fixed order (deterministic; no split-K kernel and no second
//    launch).
//  * Group-wise scales (GS): a chunk's positions lie in one group when the
//    group size is a multiple of the positions a chunk spans (128; int2 256),
//    so each chunk's MFMAs go to fresh accumulators that are then added to
//    the running tile times the group scale of their column (the output
//    row), read from the group-major copy of the scales with the chunk's
//    loads.
//  * The operand buffer is swizzled so that any 8 consecutive lanes touch 8
//    distinct 16-byte bank groups, both when they write it (two stacked rows
//    x four k-groups) and when the MFMA reads it (eight rows of one
//    k-group); chunks alternate between two buffers where LDS allows, so the
//    split of one chunk need not wait for the MFMA reads of the one before.
#pragma once
#include <algorithm>
#include <type_traits>

#include "wq_internal.h"

namespace wq {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 128;  // field positions per chunk: four 32-position MFMA k-steps

// Per format: elements per byte, 16-byte weight loads per chunk per lane
// and o-block (int2: one load serves two chunks), and the power of two the
// decoded codes carry.
template <int FMT> struct SkF;
template <> struct SkF<WQ_I8> { static constexpr int EPB = 1; static constexpr int LOADS2 = 4; static constexpr float UNSCALE = 1.0f; };
template <> struct SkF<WQ_I4> { static constexpr int EPB = 2; static constexpr int LOADS2 = 2; static constexpr float UNSCALE = 0.0625f; };
template <> struct SkF<WQ_I2> { static constexpr int EPB = 4; static constexpr int LOADS2 = 1; static constexpr float UNSCALE = 0.015625f; };
// (LOADS2: 16-byte loads per two chunks)

// First field position of k-step j of chunk c for lane group g (8
// consecutive positions follow). int8 / int4: a lane group covers 32
// positions of a chunk (one 32-byte / 16-byte run of its row); int2: one
// 16-byte load of a lane group covers 64 positions, 32 of each of two chunks.
template <int FMT> __device__ __forceinline__ int chunk_pos(int c, int g, int j) {
    if constexpr (FMT == WQ_I2) return 256 * (c >> 1) + 64 * g + 32 * (c & 1) + 8 * j;
    return kChunk * c + 32 * g + 8 * j;
}

// Byte offset in the row of 16-byte weight load u (0 .. LOADS2-1) of the
// chunk pair starting at chunk c2 (even), for lane group g.
template <int FMT> __device__ __forceinline__ int load_byte(int c2, int g, int u) {
    if constexpr (FMT == WQ_I8) return 128 * (c2 + (u >> 1)) + 32 * g + 16 * (u & 1);
    if constexpr (FMT == WQ_I4) return 64 * (c2 + u) + 16 * g;
    return 64 * (c2 >> 1) + 16 * g;
}

__device__ __forceinline__ uint32_t pack_hi(uint32_t lo_bits, uint32_t hi_bits) {
    // bytes [lo.2, lo.3, hi.2, hi.3]: the bf16 (upper) halves of two fp32
    // values that bf16 represents exactly
    return __builtin_amdgcn_perm(hi_bits, lo_bits, 0x07060302u);
}

__device__ __forceinline__ uint32_t sbyte_f32(uint32_t w, int b) {
    return __float_as_uint((float)(int)(int8_t)(w >> (8 * b)));  // one SDWA conversion
}

// Keeps a value in a register (stops the compiler from folding masks into
// each field extraction).
__device__ __forceinline__ uint32_t reg(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// B operand of one k-step: the 8 codes of field positions 8j' .. 8j' + 7 as
// bf16 values of (a power of two times) q, positions ascending.
// int4: one dword of 8 nibbles -> 16 * q.
__device__ __forceinline__ u32x4 b_frag_i4(uint32_t w) {
    const uint32_t t = w ^ 0x88888888u;              // each nibble: two's complement of q
    const uint32_t ev = reg((t << 4) & 0xF0F0F0F0u);  // byte b = 16 * q of position 2b
    const uint32_t od = reg(t & 0xF0F0F0F0u);         // byte b = 16 * q of position 2b + 1
    u32x4 r;
    r.x = pack_hi(sbyte_f32(ev, 0), sbyte_f32(od, 0));
    r.y = pack_hi(sbyte_f32(ev, 1), sbyte_f32(od, 1));
    r.z = pack_hi(sbyte_f32(ev, 2), sbyte_f32(od, 2));
    r.w = pack_hi(sbyte_f32(ev, 3), sbyte_f32(od, 3));
    return r;
}
// int8: two dwords of 4 bytes -> q.
__device__ __forceinline__ u32x4 b_frag_i8(uint32_t w0, uint32_t w1) {
    u32x4 r;
    r.x = pack_hi(sbyte_f32(w0, 0), sbyte_f32(w0, 1));
    r.y = pack_hi(sbyte_f32(w0, 2), sbyte_f32(w0, 3));
    r.z = pack_hi(sbyte_f32(w1, 0), sbyte_f32(w1, 1));
    r.w = pack_hi(sbyte_f32(w1, 2), sbyte_f32(w1, 3));
    return r;
}
// int2: one dword of 16 codes (two k-steps) -> 64 * q; lo = positions 0..7.
__device__ __forceinline__ void b_frag_i2(uint32_t w, u32x4 &lo, u32x4 &hi) {
    const uint32_t t = w ^ 0xAAAAAAAAu;  // each field: two's complement of q
    // m[f] byte b = 64 * q of position 4b + f
    const uint32_t m0 = reg((t << 6) & 0xC0C0C0C0u), m1 = reg((t << 4) & 0xC0C0C0C0u);
    const uint32_t m2 = reg((t << 2) & 0xC0C0C0C0u), m3 = reg(t & 0xC0C0C0C0u);
    lo.x = pack_hi(sbyte_f32(m0, 0), sbyte_f32(m1, 0));
    lo.y = pack_hi(sbyte_f32(m2, 0), sbyte_f32(m3, 0));
    lo.z = pack_hi(sbyte_f32(m0, 1), sbyte_f32(m1, 1));
    lo.w = pack_hi(sbyte_f32(m2, 1), sbyte_f32(m3, 1));
    hi.x = pack_hi(sbyte_f32(m0, 2), sbyte_f32(m1, 2));
    hi.y = pack_hi(sbyte_f32(m2, 2), sbyte_f32(m3, 2));
    hi.z = pack_hi(sbyte_f32(m0, 3), sbyte_f32(m1, 3));
    hi.w = pack_hi(sbyte_f32(m2, 3), sbyte_f32(m3, 3));
}

// Chunks per permuted 1 KiB block of a row (a chunk never straddles one).
template <int FMT> constexpr int kChunksPerBlock = FMT == WQ_I8 ? 8 : FMT == WQ_I4 ? 16 : 32;

// Element index of field position chunk_pos(c, g, j) + 4 q inside the
// permuted blocks (device layout: field n of 16-byte granule lambda of a
// block holds element 256 (n / 4) + 4 lambda + n % 4), split into a part
// that depends on the chunk only (wave-uniform) and one that depends on
// the lane's (g, j, q) only.
template <int FMT> __device__ __forceinline__ int elem_chunk_part(int c) {
    if constexpr (FMT == WQ_I4) return ((c >> 4) << 11) + ((c & 15) << 4);
    if constexpr (FMT == WQ_I2) return ((c >> 5) << 12) + (((c >> 1) & 15) << 4) + ((c & 1) << 11);
    return ((c >> 3) << 10) + ((c & 7) << 5);
}
template <int FMT> __device__ __forceinline__ int elem_lane_part(int g, int j, int q) {
    if constexpr (FMT == WQ_I4 || FMT == WQ_I2) return (g << 2) + ((2 * j + q) << 8);
    return (g << 3) + ((j >> 1) << 2) + ((2 * (j & 1) + q) << 8);
}

// 16-byte slot of stacked row rho, k-step j and k-group g in an operand
// buffer (1 KiB per fragment of 16 rows and k-step; the MFMA's lane li + 16 g
// reads row li of k-group g): inside its k-group the row is rotated by
// S j + 2 g (see the bank-conflict note at the top).
__device__ __forceinline__ int opnd_slot(int rho, int j, int g, int S) {
    return ((rho >> 4) * 4 + j) * 64 + 16 * g + (((rho & 15) + S * j + 2 * g) & 15);
}

// Group of the field positions of chunk c (all in one group, see GS above).
template <int FMT> __device__ __forceinline__ int chunk_group(int c, int gs, int ng) {
    return min(chunk_pos<FMT>(c, 0, 0) / gs, ng - 1);
}

// M: stacked operand fragments (3 S <= 16 M); RPL: 8-position activation
// runs per lane per chunk (16 S runs per chunk, so RPL = ceil(S / 4));
// NB: 16-row output blocks per wave (and block); WAVES: waves per block,
// each streaming its own chunks; R: chunks of loads in flight (even);
// NBUF: operand buffers per wave (1 or 2); GS: group-wise scales.
// The work of one block: output rows [16 NB blk, 16 NB (blk + 1)) of a.
template <int FMT, int M, int RPL, int NB, int WAVES, int R, int NBUF, bool GS>
__device__ __forceinline__ void skinny_block(const SkinnyArgs &a, int blk) {
    static_assert(R % 2 == 0, "the load ring advances by chunk pairs");
    static_assert(NBUF == 1 || NBUF == 2, "one or two operand buffers");
    constexpr int L2 = SkF<FMT>::LOADS2;
    constexpr int ABUF = M * 4 * 1024;                // bytes of one operand buffer
    constexpr int RED = WAVES * NB * M * 1024;        // bytes of the partial tiles
    constexpr int LDS = WAVES * NBUF * ABUF > RED ? WAVES * NBUF * ABUF : RED;
    __shared__ __align__(16) uint8_t lds[LDS];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int S = a.S, O = a.O, I = a.I;
    const int o0 = blk * (16 * NB);
    const int stride = (int)a.stride;
    // chunk pairs are dealt to the waves in turn (pair k of this wave is
    // pair wave + WAVES k of the row), so at any time the block's waves read
    // neighbouring pieces of its rows; pairs past the row are skipped and
    // their loads re-read the row's last pair (cache hits, never used)
    const int np_row = a.nchunks / 2;
    const int npairs = a.chunks_per_wave / 2;  // pairs per wave
    const int c_full = a.nfull * kChunksPerBlock<FMT>;  // chunks inside the permuted blocks
    auto pair_c2 = [&](int k) { return 2 * min(wave + WAVES * k, np_row - 1); };
    auto pair_live = [&](int k) { return wave + WAVES * k < np_row; };

    // 32-bit byte offsets from the tensor's base (O * stride < 2^31): the
    // rows this lane reads (clamped: rows past O are read, never stored)
    uint32_t roff[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) roff[b] = (uint32_t)min(o0 + 16 * b + li, O - 1) * (uint32_t)stride;
    const uint32_t lane_w = (FMT == WQ_I8 ? 32u : 16u) * (uint32_t)g;  // lane group's bytes in a chunk
    const uint32_t last16 = (uint32_t)stride - 16u;

    // operand buffers: rows >= 3S stay zero for the whole call
    u32x4 *abuf = reinterpret_cast<u32x4 *>(lds + wave * NBUF * ABUF);
#pragma unroll
    for (int i = 0; i < NBUF * M * 4; ++i) abuf[i * 64 + lane] = u32x4{0u, 0u, 0u, 0u};
    // the MFMA read slots of this lane, per k-step (fragment m adds 256 m)
    int rd_slot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rd_slot[j] = opnd_slot(li, j, g, S);

    // run r = lane + 64 i: k-group r % 4 (four lanes read 64 contiguous
    // bytes of an activation row), run index t = r / 4, which is activation
    // row t % S of k-step t / S (runs t >= 4 S are loaded and never stored)
    int run_g[RPL], run_j[RPL], run_slot[RPL][3];
    uint32_t run_x[RPL][2];   // activation offset (floats) of the run inside the permuted blocks, less the chunk part
    uint32_t run_xn[RPL][2];  // the same in natural order (past the blocks), less the chunk's first position
    bool run_live[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const int t = (lane >> 2) + 16 * i;
        const int rs = t % S;
        run_g[i] = lane & 3;
        run_j[i] = min(t / S, 3);
        run_live[i] = t < 4 * S;
#pragma unroll
        for (int p = 0; p < 3; ++p) run_slot[i][p] = opnd_slot(p * S + rs, run_j[i], run_g[i], S);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            run_x[i][q] = (uint32_t)(rs * I + elem_lane_part<FMT>(run_g[i], run_j[i], q));
            run_xn[i][q] = (uint32_t)(rs * I + (int)(chunk_pos<FMT>(0, run_g[i], run_j[i]) + 4 * q));
        }
    }

    // ---- loads of one chunk pair: weights (NB x L2 16-byte loads) and the
    // activation runs of both chunks (2 x RPL runs of two 16-byte loads).
    // Every load is issued unconditionally (addresses clamped inside the
    // row / the activations), so the compiler's wait counts stay exact.
    auto load_w = [&](u32x4 (&wv)[L2][NB], int c2) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < L2; ++u) {
            const uint32_t off = min((uint32_t)load_byte<FMT>(c2, 0, u) + lane_w, last16);
#pragma unroll
            for (int b = 0; b < NB; ++b)
                wv[u][b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(a.w + (roff[b] + off)));
        }
    };
    // GS: the group scale of this lane's column (output row, clamped like
    // the weight rows) for both chunks of a pair
    uint32_t scol[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) scol[b] = (uint32_t)min(o0 + 16 * b + li, O - 1);
    auto load_s = [&](float (&sv)[2][NB], int c2) __attribute__((always_inline)) {
        if constexpr (GS) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t gbase = (uint32_t)chunk_group<FMT>(c2 + h, a.gs, a.ng) * (uint32_t)O;
#pragma unroll
                for (int b = 0; b < NB; ++b) sv[h][b] = a.gscales_t[gbase + scol[b]];
            }
        }
    };
    const uint32_t xlast = (uint32_t)(S * I - 4);
    auto load_x = [&](f32x4 (&xv)[2][RPL][2], int c2) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = c2 + h;
            const bool full = c < c_full;  // wave-uniform
            const uint32_t cp = full ? (uint32_t)elem_chunk_part<FMT>(c) : (uint32_t)chunk_pos<FMT>(c, 0, 0);
#pragma unroll
            for (int i = 0; i < RPL; ++i)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const uint32_t e = min(cp + (full ? run_x[i][q] : run_xn[i][q]), xlast);
                    xv[h][i][q] = *reinterpret_cast<const f32x4 *>(a.x + e);
                }
        }
    };

    f32x4 acc[NB][M];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[b][m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    constexpr int RP = R / 2;  // chunk pairs in flight
    u32x4 wring[RP][L2][NB];
    f32x4 xring[RP][2][RPL][2];
    float sring[RP][2][NB];  // GS only
#pragma unroll
    for (int p = 0; p < RP; ++p) {
        load_x(xring[p], pair_c2(p));
        load_w(wring[p], pair_c2(p));
        load_s(sring[p], pair_c2(p));
    }

    // ---- one chunk: split its activations into an operand buffer, then
    // 4 k-steps x NB o-blocks x M stacked fragments of MFMAs. Inside the
    // permuted blocks (FULL) every run lies inside the row (I % 4 == 0 and
    // the blocks hold exactly the first elements); past them (natural
    // order) a run lies inside or outside [0, I) and is masked. The same
    // wave writes and reads each buffer: its LDS operations complete in
    // order, and the buffer's accesses may alias, so the compiler keeps them
    // in program order.
    auto do_chunk = [&](auto full_c, const f32x4 (&xv)[RPL][2], const u32x4 (&wv)[L2][NB],
                        const float (&sv)[NB], int c, int h) __attribute__((always_inline)) {
        constexpr bool FULL = decltype(full_c)::value;
        u32x4 *buf = abuf + (NBUF == 2 ? h : 0) * (ABUF / 16);
        const int cpos = chunk_pos<FMT>(c, 0, 0);
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            float v[8];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                f32x4 t = xv[i][q];
                if constexpr (!FULL) {
                    const bool in = cpos + chunk_pos<FMT>(0, run_g[i], run_j[i]) + 4 * q < I;
                    t = in ? t : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                }
                v[4 * q + 0] = t.x;
                v[4 * q + 1] = t.y;
                v[4 * q + 2] = t.z;
                v[4 * q + 3] = t.w;
            }
            uint32_t pl[3][8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t hb = __float_as_uint(v[e]) & 0xFFFF0000u;
                const float r1 = v[e] - __uint_as_float(hb);  // exact
                const uint32_t mb = __float_as_uint(r1) & 0xFFFF0000u;
                pl[0][e] = hb;
                pl[1][e] = mb;
                pl[2][e] = __float_as_uint(r1 - __uint_as_float(mb));  // exact, <= 8 significant bits
            }
            if (run_live[i]) {
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    buf[run_slot[i][p]] = u32x4{pack_hi(pl[p][0], pl[p][1]), pack_hi(pl[p][2], pl[p][3]),
                                                pack_hi(pl[p][4], pl[p][5]), pack_hi(pl[p][6], pl[p][7])};
            }
        }
        f32x4 tmp[NB][M];  // GS: this chunk's sums (one group)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 av[M];
#pragma unroll
            for (int m = 0; m < M; ++m) av[m] = __builtin_bit_cast(bf16x8, buf[m * 256 + rd_slot[j]]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                u32x4 bw;
                if constexpr (FMT == WQ_I4) {
                    const u32x4 &ld = wv[h][b];
                    bw = b_frag_i4(j == 0 ? ld.x : j == 1 ? ld.y : j == 2 ? ld.z : ld.w);
                } else if constexpr (FMT == WQ_I8) {
                    const u32x4 &ld = wv[2 * h + (j >> 1)][b];
                    bw = (j & 1) ? b_frag_i8(ld.z, ld.w) : b_frag_i8(ld.x, ld.y);
                } else {
                    // one dword holds k-steps j and j ^ 1 of this chunk
                    const u32x4 &ld = wv[0][b];
                    const uint32_t d = h == 0 ? ((j >> 1) ? ld.y : ld.x) : ((j >> 1) ? ld.w : ld.z);
                    u32x4 lo, hi;
                    b_frag_i2(d, lo, hi);
                    bw = (j & 1) ? hi : lo;
                }
                const bf16x8 bv = __builtin_bit_cast(bf16x8, bw);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    if constexpr (GS)
                        tmp[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av[m], bv, j == 0 ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : tmp[b][m], 0, 0, 0);
                    else
                        acc[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], bv, acc[b][m], 0, 0, 0);
                }
            }
        }
        if constexpr (GS) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int m = 0; m < M; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[b][m][r] = __builtin_fmaf(sv[b], tmp[b][m][r], acc[b][m][r]);
        }
    };
    auto chunk = [&](const f32x4 (&xv)[RPL][2], const u32x4 (&wv)[L2][NB], const float (&sv)[NB], int c, int h)
        __attribute__((always_inline)) {
        if (c < c_full) do_chunk(std::true_type{}, xv, wv, sv, c, h);  // wave-uniform branch
        else do_chunk(std::false_type{}, xv, wv, sv, c, h);
    };

    // (the pair checks are wave-uniform: skipping work changes no load count)
    int kk = 0;
    for (; kk + RP < npairs; kk += RP) {
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const int k = kk + p;
            if (pair_live(k)) {
                const int c2 = 2 * (wave + WAVES * k);
                chunk(xring[p][0], wring[p], sring[p][0], c2, 0);
                chunk(xring[p][1], wring[p], sring[p][1], c2 + 1, 1);
            }
            // refill this slot with the wave's pair RP pairs ahead
            load_x(xring[p], pair_c2(k + RP));
            load_w(wring[p], pair_c2(k + RP));
            load_s(sring[p], pair_c2(k + RP));
        }
    }
#pragma unroll
    for (int p = 0; p < RP; ++p) {  // the last round: nothing left to load
        const int k = kk + p;
        if (k < npairs && pair_live(k)) {
            const int c2 = 2 * (wave + WAVES * k);
            chunk(xring[p][0], wring[p], sring[p][0], c2, 0);
            chunk(xring[p][1], wring[p], sring[p][1], c2 + 1, 1);
        }
    }

    // ---- add the waves' partial tiles (and the three planes) in fixed order
    __syncthreads();  // every wave is done with its operand buffers
    float *red = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int m = 0; m < M; ++m)
            reinterpret_cast<f32x4 *>(red)[((wave * NB + b) * M + m) * 64 + lane] = acc[b][m];
    __syncthreads();
    for (int idx = threadIdx.x; idx < S * 16 * NB; idx += 64 * WAVES) {
        const int s = idx / (16 * NB), oc = idx % (16 * NB);
        const int o = o0 + oc;
        if (o >= O) continue;
        const int b = oc >> 4, col = oc & 15;
        float sum = 0.0f;
        for (int w = 0; w < WAVES; ++w)
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                const int rho = p * S + s;
                const int lc = ((rho & 15) >> 2) * 16 + col;
                sum += red[(((w * NB + b) * M + (rho >> 4)) * 64 + lc) * 4 + (rho & 3)];
            }
        a.y[(long)s * O + o] = GS ? sum * SkF<FMT>::UNSCALE : a.scales[o] * (sum * SkF<FMT>::UNSCALE);
    }
}

template <int FMT, int M, int RPL, int NB, int WAVES, int R, int NBUF, bool GS = false>
__global__ __launch_bounds__(64 * WAVES) void skinny_kernel(SkinnyArgs a) {
    skinny_block<FMT, M, RPL, NB, WAVES, R, NBUF, GS>(a, blockIdx.x);
}

// LDS of a block: the waves' operand buffers (nbuf each), reused for the
// partial tiles.
constexpr int skinny_lds_bytes(int m, int nb, int waves, int nbuf) {
    return waves * nbuf * m * 4096 > waves * nb * m * 1024 ? waves * nbuf * m * 4096 : waves * nb * m * 1024;
}
// Two operand buffers per wave where they fit in the CU's 160 KiB of LDS.
constexpr int skinny_nbuf(int m, int nb, int waves) {
    return skinny_lds_bytes(m, nb, waves, 2) <= 160 * 1024 ? 2 : 1;
}

// 4-wave blocks for 17 <= S <= 32: (m, rpl) = (4, 5) for S <= 20, (5, 6) for
// S <= 24, (6, 8) for S <= 32, nb = 1..4 (1..3 for m = 6): the operand
// buffers of four waves fit in LDS, one wave per SIMD holds the larger
// tiles in registers.
template <int FMT, int M, int RPL>
hipError_t launch_wide_mr(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
#define WQ_SKW4(NB_)                                                                                         \
    if (p.nb == NB_) {                                                                                       \
        hipLaunchKernelGGL((skinny_kernel<FMT, M, RPL, NB_, 4, 2, skinny_nbuf(M, NB_, 4)>), dim3(p.grid),    \
                           dim3(256), 0, st, a);                                                             \
        return hipGetLastError();                                                                            \
    }
    WQ_SKW4(1) WQ_SKW4(2) WQ_SKW4(3)
    if constexpr (M <= 5) { WQ_SKW4(4) }  // (m = 6 with four blocks would spill)
#undef WQ_SKW4
    return hipErrorInvalidValue;
}
template <int FMT>
hipError_t launch_wide(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
    if (p.waves != 4 || p.ring != 2) return hipErrorInvalidValue;
    switch (p.m * 10 + p.rpl) {
    case 45: return launch_wide_mr<FMT, 4, 5>(p, a, st);
    case 56: return launch_wide_mr<FMT, 5, 6>(p, a, st);
    case 68: return launch_wide_mr<FMT, 6, 8>(p, a, st);
    default: return hipErrorInvalidValue;
    }
}

} // namespace

// Deepest ring (chunks of loads in flight per wave) whose kernel keeps every
// value in registers (no spills at two waves per SIMD), from the compiled
// register counts: the ring holds a chunk pair's weights (LOADS2 x NB
// 16-byte loads) and activation runs (2 x RPL x 32 bytes); 0: not compiled.
constexpr int skinny_max_ring(int fmt, int m, int rpl, int nb) {
    // [format][(m, rpl) = (1,1) (1,2) (2,2) (2,3) (3,3) (3,4)][nb - 1]
    constexpr signed char kRing[3][6][4] = {
        {{6, 6, 6, 4}, {6, 6, 4, 2}, {6, 4, 2, 2}, {4, 2, 2, 2}, {4, 2, 2, 0}, {4, 2, 0, 0}},   // int8
        {{6, 6, 6, 6}, {6, 6, 6, 4}, {6, 6, 4, 4}, {6, 4, 2, 2}, {6, 4, 2, 0}, {4, 2, 2, 0}},   // int4
        {{6, 6, 6, 6}, {6, 6, 6, 6}, {6, 6, 6, 4}, {6, 4, 4, 2}, {6, 4, 2, 0}, {4, 2, 2, 0}}};  // int2
    const int f = fmt == WQ_I8 ? 0 : fmt == WQ_I4 ? 1 : fmt == WQ_I2 ? 2 : -1;
    const int mr = m * 10 + rpl;
    const int k = mr == 11 ? 0 : mr == 12 ? 1 : mr == 22 ? 2 : mr == 23 ? 3 : mr == 33 ? 4 : mr == 34 ? 5 : -1;
    return f < 0 || k < 0 || nb < 1 || nb > 4 ? 0 : kRing[f][k][nb - 1];
}

// Tiles with at least the default two chunks of loads in flight.
constexpr bool skinny_ring_ok(int fmt, int m, int rpl, int nb) { return skinny_max_ring(fmt, m, rpl, nb) >= 2; }

// Group-scaled tiles (fresh accumulators per chunk beside the running ones)
// that keep every value in registers with two chunks in flight (from the
// compiled register counts): 8-wave blocks at two waves per SIMD, and for
// three stacked fragments (11 <= S <= 16) also 4-wave blocks at one wave per
// SIMD, whose larger register file holds three or four output blocks.
constexpr bool skinny_gs_ok(int fmt, int m, int rpl, int nb, int waves) {
    if (fmt < WQ_I8 || fmt > WQ_I2 || m < 1 || m > 3 || rpl < 1 || rpl > 4 || nb < 1 || nb > 4) return false;
    if (waves == 4) return m == 3 && nb >= 3;
    if (waves != 8) return false;
    if (m * nb <= 6) return true;
    const int k = m * 100 + rpl * 10 + nb;
    return k == 224 || k == 333 || (k == 234 && fmt != WQ_I8) || (k == 343 && fmt == WQ_I2);
}

hipError_t launch_skinny_wide_i8(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st);
hipError_t launch_skinny_wide_i4(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st);
hipError_t launch_skinny_wide_i2(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st);

} // namespace wq

