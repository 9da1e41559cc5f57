// Few activation rows (S <= 16) on the matrix cores, one launch, no workspace.
//
// y[s,o] = scale[o] * sum_i dequant(W[o,i]) * x[s,i]
//   (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四, qmatmul.comp
//    header; dequant rules from colibri-analysis "CUDA 后端", section 1,
//    weight_at; batched rows on matrix units: colibri docs "CUDA backend
//    (Linux)", section "The GPU-resident pipeline")
//
// With 2..16 activation rows the register GEMV spends S vector FMAs on
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
//    tile (S <= 10 two, S <= 16 three); y[s] adds rows s, S + s and 2S + s.
//  * Weights straight into operand registers, in the device layout that the
//    GEMV streams (no second copy): the contraction runs over field
//    positions, and a lane's 16-byte load of one row holds, for its group
//    of 8 positions per k-step, the codes of several consecutive k-steps;
//    the activations are paired with the same positions.
//  * A block of WAVES waves owns 16 * NB output rows and splits the row's
//    128-position chunks between its waves; each wave streams its own
//    chunks with the weight and activation loads of R chunks in flight,
//    splits its activations into a wave-private LDS buffer laid out as MFMA
//    operands (all 64 lanes split; no block barrier per step), and the
//    waves' partial tiles are added through LDS at the end in fixed order
//    (deterministic; no split-K kernel and no second launch).
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
template <int FMT> __device__ __forceinline__ long chunk_pos(long c, int g, int j) {
    if constexpr (FMT == WQ_I2) return 256L * (c >> 1) + 64 * g + 32 * (c & 1) + 8 * j;
    return (long)kChunk * c + 32 * g + 8 * j;
}

// Byte offset in the row of 16-byte weight load u (0 .. LOADS2-1) of the
// chunk pair starting at chunk c2 (even), for lane group g.
template <int FMT> __device__ __forceinline__ long load_byte(long c2, int g, int u) {
    if constexpr (FMT == WQ_I8) return 128L * (c2 + (u >> 1)) + 32 * g + 16 * (u & 1);
    if constexpr (FMT == WQ_I4) return 64L * (c2 + u) + 16 * g;
    return 64L * (c2 >> 1) + 16 * g;
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

template <int M> struct SkBucket {
    static constexpr int SMAX = M == 1 ? 5 : M == 2 ? 10 : 16;  // activation rows of the bucket
    static constexpr int RPL = (16 * SMAX + 63) / 64;           // 8-position runs per lane per chunk
};

// NB: 16-row output blocks per wave (and block); WAVES: waves per block,
// each streaming its own chunks; R: chunks of loads in flight (even).
template <int FMT, int M, int NB, int WAVES, int R>
__global__ __launch_bounds__(64 * WAVES) void skinny_kernel(SkinnyArgs a) {
    static_assert(R % 2 == 0, "the load ring advances by chunk pairs");
    constexpr int RPL = SkBucket<M>::RPL;
    constexpr int L2 = SkF<FMT>::LOADS2;
    constexpr int ABUF = M * 4 * 1024;                // bytes of one wave's operand buffer
    constexpr int RED = WAVES * NB * M * 1024;        // bytes of the partial tiles
    constexpr int LDS = WAVES * ABUF > RED ? WAVES * ABUF : RED;
    __shared__ __align__(16) uint8_t lds[LDS];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int li = lane & 15, g = lane >> 4;
    const int S = a.S, O = a.O, I = a.I;
    const int o0 = blockIdx.x * (16 * NB);
    const long stride = a.stride;
    const long c_begin = (long)wave * a.chunks_per_wave;
    const int npairs = a.chunks_per_wave / 2;

    // the rows this lane reads (clamped: rows past O are read, never stored)
    const uint8_t *rowp[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) rowp[b] = a.w + (long)min(o0 + 16 * b + li, O - 1) * stride;

    // operand buffer: rows >= 3S stay zero for the whole call
    uint8_t *abuf = lds + wave * ABUF;
#pragma unroll
    for (int i = 0; i < M * 4; ++i) reinterpret_cast<u32x4 *>(abuf)[i * 64 + lane] = u32x4{0u, 0u, 0u, 0u};

    // ---- loads of one chunk pair: weights (NB x L2 16-byte loads) and the
    // activation runs of both chunks (2 x RPL runs of two 16-byte loads).
    // Every load is issued unconditionally (addresses clamped inside the
    // row / the activations), so the compiler's wait counts stay exact.
    const long last16 = stride - 16;
    auto load_w = [&](u32x4 (&wv)[L2][NB], long c2) {
#pragma unroll
        for (int u = 0; u < L2; ++u) {
            const long off = min(load_byte<FMT>(c2, g, u), last16);
#pragma unroll
            for (int b = 0; b < NB; ++b) wv[u][b] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(rowp[b] + off));
        }
    };
    // run r = lane + 64 i of a chunk: g fastest (four lanes read 64
    // contiguous bytes of an activation row), then the row s, then the
    // k-step j (runs r >= 16 S are loaded, clamped, and never stored)
    int run_s[RPL], run_g[RPL], run_j[RPL];
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
        const int r = lane + 64 * i;
        run_g[i] = r & 3;
        run_s[i] = (r >> 2) % S;
        run_j[i] = min((r >> 2) / S, 3);
    }
    auto load_x = [&](f32x4 (&xv)[2][RPL][2], long c2) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < RPL; ++i) {
                const long P = chunk_pos<FMT>(c2 + h, run_g[i], run_j[i]);
                const float *xs = a.x + (long)run_s[i] * I;
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const long e = elem_of_pos4(FMT, P + 4 * q, a.nfull);
                    xv[h][i][q] = *reinterpret_cast<const f32x4 *>(xs + min(e, (long)I - 4));
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
#pragma unroll
    for (int p = 0; p < RP; ++p) {
        load_x(xring[p], c_begin + 2 * p);
        load_w(wring[p], c_begin + 2 * p);
    }

    // ---- one chunk: split its activations into the operand buffer, then
    // 4 k-steps x NB o-blocks x M stacked fragments of MFMAs
    auto do_chunk = [&](const f32x4 (&xv)[RPL][2], const u32x4 (&wv)[L2][NB], long c, int h) {
#pragma unroll
        for (int i = 0; i < RPL; ++i) {
            const int r = lane + 64 * i;
            const int rs = run_s[i], rg = run_g[i], rj = run_j[i];
            const long P = chunk_pos<FMT>(c, rg, rj);
            float v[8];
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const long e = elem_of_pos4(FMT, P + 4 * q, a.nfull);
                const bool in = e < I;  // a run lies inside or outside the row (I % 4 == 0)
                v[4 * q + 0] = in ? xv[i][q].x : 0.0f;
                v[4 * q + 1] = in ? xv[i][q].y : 0.0f;
                v[4 * q + 2] = in ? xv[i][q].z : 0.0f;
                v[4 * q + 3] = in ? xv[i][q].w : 0.0f;
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
            if (r < 16 * S) {
#pragma unroll
                for (int p = 0; p < 3; ++p) {
                    const int rho = p * S + rs;
                    const int slot = ((rho >> 4) * 4 + rj) * 64 + (rho & 15) + 16 * rg;
                    reinterpret_cast<u32x4 *>(abuf)[slot] =
                        u32x4{pack_hi(pl[p][0], pl[p][1]), pack_hi(pl[p][2], pl[p][3]), pack_hi(pl[p][4], pl[p][5]),
                              pack_hi(pl[p][6], pl[p][7])};
                }
            }
        }
        // the same wave reads the buffer back: LDS operations of one wave
        // complete in order; keep the compiler from moving reads above writes
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            bf16x8 av[M];
#pragma unroll
            for (int m = 0; m < M; ++m)
                av[m] = __builtin_bit_cast(bf16x8, reinterpret_cast<const u32x4 *>(abuf)[(m * 4 + j) * 64 + lane]);
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
                for (int m = 0; m < M; ++m)
                    acc[b][m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[m], bv, acc[b][m], 0, 0, 0);
            }
        }
        asm volatile("" ::: "memory");  // the next chunk's writes stay after these reads
    };

    int pp = 0;
    for (; pp + RP < npairs; pp += RP) {
#pragma unroll
        for (int p = 0; p < RP; ++p) {
            const long c2 = c_begin + 2 * (pp + p);
            do_chunk(xring[p][0], wring[p], c2, 0);
            do_chunk(xring[p][1], wring[p], c2 + 1, 1);
            // refill this slot with the chunk pair R chunks ahead
            load_x(xring[p], c2 + R);
            load_w(wring[p], c2 + R);
        }
    }
#pragma unroll
    for (int p = 0; p < RP; ++p) {  // the last pairs: nothing left to load
        const long c2 = c_begin + 2 * (pp + p);
        do_chunk(xring[p][0], wring[p], c2, 0);
        do_chunk(xring[p][1], wring[p], c2 + 1, 1);
    }

    // ---- add the waves' partial tiles (and the three planes) in fixed order
    __syncthreads();  // every wave is done with its operand buffer
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
        a.y[(long)s * O + o] = a.scales[o] * (sum * SkF<FMT>::UNSCALE);
    }
}

template <int FMT, int M>
hipError_t launch_m(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
    const dim3 grid(p.grid), block(64 * p.waves);
#define WQ_SK(NB_, W_, R_)                                                                      \
    if (p.nb == NB_ && p.waves == W_ && p.ring == R_) {                                         \
        hipLaunchKernelGGL((skinny_kernel<FMT, M, NB_, W_, R_>), grid, block, 0, st, a);       \
        return hipGetLastError();                                                               \
    }
    // (16-wave blocks leave 128 registers per lane: one fragment only)
    if constexpr (M == 1) WQ_SK(1, 16, 2)
    WQ_SK(1, 8, 2) WQ_SK(2, 8, 2) WQ_SK(3, 8, 2)
    if constexpr (!(FMT == WQ_I8 && M == 3)) WQ_SK(4, 8, 2)  // (int8, three fragments: 4 blocks spill)
#undef WQ_SK
    return hipErrorInvalidValue;
}

template <int FMT>
hipError_t launch_f(const SkinnyPlan &p, const SkinnyArgs &a, hipStream_t st) {
    if (p.m == 1) return launch_m<FMT, 1>(p, a, st);
    if (p.m == 2) return launch_m<FMT, 2>(p, a, st);
    return launch_m<FMT, 3>(p, a, st);
}

} // namespace

SkinnyPlan plan_skinny(int fmt, int O, int I, int S, int cus) {
    SkinnyPlan p;
    if ((fmt != WQ_I8 && fmt != WQ_I4 && fmt != WQ_I2) || O <= 0 || I < 4 || I % 4 != 0 || S < 1 || S > 16)
        return p;
    p.m = S <= 5 ? 1 : S <= 10 ? 2 : 3;
    const long stride = round_up(row_bytes(fmt, I), kRowAlign);
    const long npos = stride * elems_per_byte(fmt);
    long nchunks = (npos + kChunk - 1) / kChunk;
    nchunks = round_up(nchunks, 2);
    // output blocks: as many rows per block as still gives every CU a block
    const int nbmax = (fmt == WQ_I8 && p.m == 3) ? 3 : 4;
    p.nb = 0;
    for (int nb = nbmax; nb >= 1; --nb)
        if ((O + 16 * nb - 1) / (16 * nb) >= cus) {
            p.nb = nb;
            break;
        }
    if (p.nb == 0) {  // few output rows: more waves per block share each row's chunks
        p.nb = 1;
        p.waves = p.m == 1 ? 16 : 8;
    } else {
        p.waves = 8;
    }
    p.ring = 2;
    p.grid = (O + 16 * p.nb - 1) / (16 * p.nb);
    const long per_wave = (nchunks + p.waves - 1) / p.waves;
    p.chunks_per_wave = (int)round_up(per_wave, p.ring);
    p.nchunks = (int)nchunks;
    p.ok = (long)p.chunks_per_wave * p.waves < (1L << 30);
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
