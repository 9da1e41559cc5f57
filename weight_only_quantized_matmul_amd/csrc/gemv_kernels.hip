// Register GEMV for S <= 8 and its grouped (many tensors, one launch) form.
//
// y[s,o] = scale[o] * sum_i dequant(W[o,i]) * x[s,i]
//   (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四, qmatmul.comp
//    header; dequant rules from colibri-analysis "CUDA 后端", section 1,
//    weight_at; scale after the sum, same section, quant_matmul)
//
// Design (gfx950, wave64):
//  * A "team" of 1..8 waves owns rows [row_begin, row_begin + rows_per_team).
//    Lane slot k covers the row bytes [(k*team_lanes + lane)*LW, +LW): one
//    wave-wide load is LW*64 contiguous bytes (1 KiB for LW = 16), read once,
//    non-temporal.
//  * With the device layout (see wq_internal.h) the activations that meet a
//    lane's weight fields are 4-element runs that are contiguous across the
//    wave, so each lane's activations are staged once into registers with
//    fully coalesced 16-byte loads and reused for every row of the team.
//  * Each wave keeps D rows of weights in flight (a register ring): row r is
//    reduced while rows r+1..r+D-1 are still arriving, and its registers are
//    refilled with row r+D right after. Reloads in the steady state are
//    unconditional so the wait counts stay exact.
//  * Dequantization happens in registers on 32-bit words, and every code
//    becomes its exact value q = code - offset before it meets an
//    activation, so each product q * x is exact and the rounding of the sum
//    is bounded by sum |q * x| (the offset is never folded into a separate
//    offset * sum(x) term, whose rounding would scale with sum |code * x|).
//    One activation row (S = 1): one and-or of a word leaves two codes in
//    the mantissas of its 16-bit halves under the f16 exponent of 1024
//    (half value 1024 + code * 2^k, exact); one packed f16 subtraction of
//    1024 + offset * 2^k leaves 2^k * q in each half, exact, and
//    v_fma_mix_f32 widens that half inside the FMA. Several rows: an
//    exclusive-or turns every field into the two's complement of q, a shift
//    and mask place it at the top of a byte (byte = 2^k * q), and one
//    sign-extending byte conversion per code feeds the S plain FMAs. The
//    activations meeting a field scaled by 2^k are pre-divided by 2^k
//    (exact). A row whose codes all decode to zero therefore gives exactly
//    0.
//  * Lanes are reduced four rows at a time with gfx950's lane-half and
//    lane-quarter swaps (v_permlane32_swap, v_permlane16_swap) and DPP
//    (quad_perm, row_shr) instead of an LDS tree; teams of several waves add
//    their wave totals through LDS in a
//    fixed order, so results are deterministic. Row scales are read with
//    scalar loads (the row index is wave-uniform), which do not wait on the
//    weight stream.
//  * Paired rows (gated feed-forward): the ring walks virtual rows 2o and
//    2o + 1, gate row o and up row o of two tensors of one shape, so both
//    dot products of an output meet the same staged activations and end in
//    the same epilogue, which writes h = silu(g) * u instead of g and u
//    (SiLU gating: the reading taken for the gated up-projection shader that
//    colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端" names in its learning
//    goals and section recap without giving its activation).
#include "skinny_group.h"
#include "wq_internal.h"


namespace wq {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <int FMT> struct FmtInfo;
template <> struct FmtInfo<WQ_F32> { static constexpr int EPW = 1; };
template <> struct FmtInfo<WQ_I8>  { static constexpr int EPW = 4; };
template <> struct FmtInfo<WQ_I4>  { static constexpr int EPW = 8; };
template <> struct FmtInfo<WQ_I2>  { static constexpr int EPW = 16; };


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

// How int4 / int2 codes reach the FMAs. MIX: two codes per and-or and one
// packed f16 subtraction, as f16 halves holding 2^k * q that v_fma_mix_f32
// widens inside the FMA -- fewest instructions per element when each code
// meets one activation row. Otherwise (several activation rows) each code is
// converted once, from a byte holding 2^k * q, and meets the rows in plain
// v_fmac_f32. (Measured: at S = 1 the mixed form is the faster one; at S = 4
// the plain FMAs are, the conversion being shared by the rows.)
template <int FMT, int SMAX> constexpr bool kMix = (FMT == WQ_I4 || FMT == WQ_I2) && SMAX == 1;

// Factor applied to the activation that meets field e (0..EPW-1) of a word:
// 2^-k for a field whose dequantized value is carried as 2^k * q.
template <int FMT, int SMAX> __device__ constexpr float x_prescale(int e) {
    if (FMT == WQ_I4) return kMix<FMT, SMAX> ? ((e & 1) ? 0.0625f : 1.0f) : 0.0625f;
    if (FMT == WQ_I2) {
        if (!kMix<FMT, SMAX>) return 0.015625f;
        const int f = e & 3;
        return f == 0 ? 1.0f : f == 1 ? 0.25f : f == 2 ? 0.0625f : 0.015625f;
    }
    return 1.0f;
}

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

// Keeps a value in a register as computed: stops the compiler from pushing a
// byte mask into each field extraction, and keeps constants that
// three-operand instructions need in registers.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// Two fields of v, selected by mask (each inside mantissa bits 0..9 of its
// 16-bit half, value f * 2^k), as the exact f16 pair 2^k * (f - off): the
// and-or gives halves 1024 + 2^k * f (below 2048, so exact), and one packed
// f16 subtraction of 1024 + 2^k * off leaves an integer of magnitude below
// 2048, exact as well. The mask and the exponent bits are passed in
// registers (opaque values) so that the and-or is one v_and_or_b32: a
// three-operand instruction takes no literal constants on this target.
template <int BIAS>
__device__ __forceinline__ half2v exact_pair(uint32_t v, uint32_t mask, uint32_t expo) {
    const half2v b = __builtin_bit_cast(half2v, (v & mask) | expo);
    constexpr _Float16 c = (_Float16)(1024 + BIAS);
    return b - half2v{c, c};
}

// With the mixed form at S = 1, int4 / int2 sums run in two independent
// chains (fields in the low and in the high f16 half of the masked words),
// so consecutive mixed FMAs do not depend on each other (back to back they
// need a wait state); each chain visits its fields in ascending order. With
// several activation rows the rows already give independent chains.
template <int FMT, int SMAX> constexpr int kChains = kMix<FMT, SMAX> ? 2 : 1;
template <int FMT, int SMAX> __device__ constexpr int field_chain(int e) {
    return !kMix<FMT, SMAX> ? 0 : FMT == WQ_I4 ? (e >= 4) : (e >= 8);
}

// acc[c][s] += sum over the fields e of chain c of one word of
// q * xw[e][s] (xw pre-scaled by x_prescale, so each product is q * x).
template <int FMT, int SMAX>
__device__ __forceinline__ void word_fma(uint32_t w, const float (*xw)[SMAX], float (&acc)[kChains<FMT, SMAX>][SMAX]) {
    if constexpr (FMT == WQ_F32) {
        const float q = __uint_as_float(w);
#pragma unroll
        for (int s = 0; s < SMAX; ++s) acc[0][s] = __builtin_fmaf(q, xw[0][s], acc[0][s]);
    } else if constexpr (FMT == WQ_I8) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float q = (float)(int)(int8_t)(w >> (8 * b));
#pragma unroll
            for (int s = 0; s < SMAX; ++s) acc[0][s] = __builtin_fmaf(q, xw[b][s], acc[0][s]);
        }
    } else if constexpr (FMT == WQ_I4 && !kMix<FMT, SMAX>) {
        // nibble ^ 8 is the 4-bit two's complement of q = nibble - 8; moved
        // to the top of its byte it reads as the signed byte 16 * q
        const uint32_t v = w ^ 0x88888888u;
        const uint32_t lo = opaque((v << 4) & 0xF0F0F0F0u);  // even fields
        const uint32_t hi = opaque(v & 0xF0F0F0F0u);         // odd fields
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float cl = (float)(int)(int8_t)(lo >> (8 * b));
            const float ch = (float)(int)(int8_t)(hi >> (8 * b));
#pragma unroll
            for (int s = 0; s < SMAX; ++s) {
                acc[0][s] = __builtin_fmaf(cl, xw[2 * b][s], acc[0][s]);
                acc[0][s] = __builtin_fmaf(ch, xw[2 * b + 1][s], acc[0][s]);
            }
        }
    } else if constexpr (FMT == WQ_I2 && !kMix<FMT, SMAX>) {
        // code ^ 2 is the 2-bit two's complement of q = code - 2; at the top
        // of its byte it reads as the signed byte 64 * q
        const uint32_t v = w ^ 0xAAAAAAAAu;
        const uint32_t m[4] = {opaque((v << 6) & 0xC0C0C0C0u), opaque((v << 4) & 0xC0C0C0C0u),
                               opaque((v << 2) & 0xC0C0C0C0u), opaque(v & 0xC0C0C0C0u)};
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const float c = (float)(int)(int8_t)(m[f] >> (8 * b));  // 64 * q
#pragma unroll
                for (int s = 0; s < SMAX; ++s)
                    acc[0][s] = __builtin_fmaf(c, xw[4 * b + f][s], acc[0][s]);
            }
    } else if constexpr (FMT == WQ_I4) {
        // Fields 2b and 2b + 1 are the low and high nibble of byte b; q[j]
        // holds field j in its low half (chain 0) and field j + 4 in its
        // high half (chain 1), the odd fields as 16 * q.
        const uint32_t t = w >> 8;  // bytes 1 and 3 into the low byte of each half
        const uint32_t e = opaque(0x64006400u), m0 = opaque(0x000F000Fu), m1 = opaque(0x00F000F0u);
        const half2v q[4] = {exact_pair<8>(w, m0, e), exact_pair<128>(w, m1, e), exact_pair<8>(t, m0, e),
                             exact_pair<128>(t, m1, e)};
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int hi = 0; hi < 2; ++hi)
#pragma unroll
                for (int s = 0; s < SMAX; ++s)
                    acc[hi][s] = __builtin_fmaf(hi ? (float)q[j].y : (float)q[j].x, xw[4 * hi + j][s], acc[hi][s]);
    } else {  // WQ_I2: fields 4b..4b + 3 in bit pairs 0-1 .. 6-7 of byte b, as 4^f * q
        const uint32_t v[2] = {w, w >> 8};
        const uint32_t e = opaque(0x64006400u);
        const uint32_t m[4] = {opaque(0x00030003u), opaque(0x000C000Cu), opaque(0x00300030u), opaque(0x00C000C0u)};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const half2v q[4] = {exact_pair<2>(v[h], m[0], e), exact_pair<8>(v[h], m[1], e),
                                 exact_pair<32>(v[h], m[2], e), exact_pair<128>(v[h], m[3], e)};
#pragma unroll
            for (int f = 0; f < 4; ++f)
#pragma unroll
                for (int hi = 0; hi < 2; ++hi)
#pragma unroll
                    for (int s = 0; s < SMAX; ++s)
                        acc[hi][s] = __builtin_fmaf(hi ? (float)q[f].y : (float)q[f].x, xw[8 * hi + 4 * h + f][s],
                                                    acc[hi][s]);
        }
    }
}

// A load of one fp32 value at a wave-uniform address through the scalar data
// cache (s_load). A vector load there would queue behind the weight loads in
// flight (vector loads complete in order) and its wait would drain the ring.
// Only for data no kernel writes while this one runs (row scales).
__device__ __forceinline__ float uniform_ld(const float *p) {
    return *(const __attribute__((address_space(4))) float *)p;
}

// silu(g) * u with silu(z) = z / (1 + e^-z), in fp32 (expf from the device
// math library; a very negative g gives -0 * u).
__device__ __forceinline__ float gated(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_move(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, true));
}

// Sums of N values over the 64 lanes, up to four values per register:
// v_permlane32_swap exchanges the upper lane half of value a with the lower
// half of value b, so one add leaves a's half sums in lanes 0..31 and b's in
// 32..63; v_permlane16_swap does the same for 16-lane quarters of two such
// registers, and four DPP steps finish each 16-lane row. Every value is
// summed in the same order whatever N and whatever its place in a register
// (a missing partner is a zero), so launches with different ring depths give
// identical sums. One or two values take a register each (independent
// chains, and their totals share a lane); four or more share registers.
// Total i ends in lane sum_lane<N>(i) of v[i]. About 10 VALU instructions per
// four values, against 32 for four separate butterflies.
template <int N> __host__ __device__ constexpr int sum_lane(int i) {
    return N <= 2 ? 15 : (i & 3) == 0 ? 15 : (i & 3) == 1 ? 47 : (i & 3) == 2 ? 31 : 63;
}

__device__ __forceinline__ float swap32_add(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);  // lanes 0..31: a, 32..63: b
}

__device__ __forceinline__ float swap16_add(float a, float b) {
    // a, b from swap32_add: 16-lane rows of the sum hold a.lo, b.lo, a.hi, b.hi
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int N> __device__ __forceinline__ void wave_sums_rows(float (&v)[N]) {
    constexpr int P = N <= 2 ? 1 : 4;  // values per register
    constexpr int G = (N + P - 1) / P;
    // value in place p (0..3) of register g, or -1
    auto slot = [](int g, int p) { return P == 1 ? (p == 0 ? g : -1) : (g * 4 + p < N ? g * 4 + p : -1); };
    float q[2 * G], r[G];
#pragma unroll
    for (int j = 0; j < 2 * G; ++j) {
        const int a = slot(j / 2, 2 * (j % 2)), b = slot(j / 2, 2 * (j % 2) + 1);
        q[j] = (a < 0 && b < 0) ? 0.0f : swap32_add(a < 0 ? 0.0f : v[a], b < 0 ? 0.0f : v[b]);
    }
#pragma unroll
    for (int g = 0; g < G; ++g) r[g] = swap16_add(q[2 * g], q[2 * g + 1]);
    // rows of r[g]: places 0, 2, 1, 3; the registers' steps interleave so
    // independent DPP adds sit back to back
#pragma unroll
    for (int g = 0; g < G; ++g) r[g] += dpp_move<0xB1>(r[g]);   // quad_perm [1,0,3,2]
#pragma unroll
    for (int g = 0; g < G; ++g) r[g] += dpp_move<0x4E>(r[g]);   // quad_perm [2,3,0,1]
#pragma unroll
    for (int g = 0; g < G; ++g) r[g] += dpp_move<0x114>(r[g]);  // row_shr:4
#pragma unroll
    for (int g = 0; g < G; ++g) r[g] += dpp_move<0x118>(r[g]);  // row_shr:8: lane 15 of each row
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = r[i / P];
}

// One team processes rows [row_begin, row_begin + rpt) (rows >= O are not
// stored). red: LDS scratch of 2 * kMaxTeam * D * SMAX floats, used when
// team > 1 (then the block is exactly one team).
// GS: group-wise scales (rows in natural order; scales[row * ng + i / gs]);
// each lane slot lies in one group, so a slot's partial sum is scaled once.
// PAIR: O counts virtual rows (twice the output rows); virtual row 2o is row
// o of (w, scales), 2o + 1 row o of (w2, scales2); y is S x O/2 and receives
// gated(g, u). D is even, row_begin and rpt are multiples of D.
//
template <int FMT, int SMAX, int LW, int KMAX, int D, bool XV, bool GS = false, bool PAIR = false>
__device__ __forceinline__ void team_rows(const uint8_t *__restrict__ w, long stride, int nfull,
                                          const float *__restrict__ scales, const float *__restrict__ x,
                                          float *__restrict__ y, int O, int I, int S, int team, int tl,
                                          int wave_in_team, int row_begin, int rpt, float *red, int gs = 0,
                                          int ng = 1, const uint8_t *__restrict__ w2 = nullptr,
                                          const float *__restrict__ scales2 = nullptr) {
    static_assert(!PAIR || D % 2 == 0, "paired rows need an even ring depth");
    // KMAX is the exact number of load slots per lane: every slot is loaded
    // unconditionally (a slot past the row re-reads the row start, see
    // below), which keeps the compiler's memory wait counts exact.
    constexpr int K = KMAX;
    constexpr int EPW = FmtInfo<FMT>::EPW;
    constexpr int WPC = LW / 4;     // 32-bit words per lane load
    constexpr int EPC = WPC * EPW;  // fields per lane load
    const int team_lanes = team * 64;
    const int lane = threadIdx.x & 63;
    const int row_last = min(O, row_begin + rpt) - 1;

    // Byte offset of slot k inside a row. A lane whose slice starts past the
    // row (only possible in the last slot) re-reads the row start: its
    // activations are zero, so quantized codes contribute nothing; f32
    // values are zeroed explicitly (inf * 0 would not vanish). Offsets are
    // 32-bit so loads use a wave-uniform base plus a per-lane offset.
    uint32_t cb[KMAX];
    bool live[KMAX];
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const uint32_t c = (uint32_t)(k * team_lanes + tl) * LW;
        live[k] = c < (uint32_t)stride;
        cb[k] = live[k] ? c : 0u;
    }

    // ---- stage this lane's activations in registers (pre-scaled), and sum(x).
    // Phase 1 issues every load in straight-line code (indices clamped into
    // the row, so no lane branches); phase 2 masks, pre-scales and sums in
    // place once the data is there.
    float xr[KMAX][EPC][SMAX];
    // The 4-field runs of one slot lie in a single 16-byte granule, so their
    // first elements form an arithmetic progression: step 256 inside a
    // permuted block, step 4 in natural order (f32 rows, last partial block).
    int xb[KMAX], xs_step[KMAX];
    bool lane_in = true;  // every run of every slot of this lane lies inside x
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int c = (k * team_lanes + tl) * LW;  // this slot's first byte
        if (FMT == WQ_F32 || c >= nfull * kBlockBytes) {
            xb[k] = (FMT == WQ_F32) ? c / 4 : c * (EPW / 4);
            xs_step[k] = 4;
        } else {
            const int r = c & (kBlockBytes - 1);
            const int n0 = (r & 15) * (EPW / 4);  // first field of the slot in its granule
            xb[k] = (c - r) * (EPW / 4) + 256 * (n0 >> 2) + 4 * (r >> 4);
            xs_step[k] = 256;
        }
        lane_in = lane_in && live[k] && xb[k] + xs_step[k] * (EPC / 4 - 1) + 4 <= I;
    }
    // wave-uniform: no activation of this wave needs masking
    const bool wave_in = __builtin_amdgcn_ballot_w64(!lane_in) == 0;
#define WQ_XE(k, g) (xb[k] + xs_step[k] * (g))
    // The weight ring: D rows of this wave's weights in registers.
    uint32_t ring[D][KMAX][WPC];
    float gring[D][KMAX];  // GS: the group scale of each slot, per row in flight
    int grp[KMAX];         // GS: group of each slot (clamped: dead slots have zero activations)
#pragma unroll
    for (int k = 0; k < KMAX; ++k) grp[k] = GS ? min(xb[k] / max(gs, 1), ng - 1) : 0;
    auto load_row = [&](uint32_t (&b)[KMAX][WPC], float (&gv)[KMAX], int row) {
        const long r = min(row, row_last);
        // wave-uniform tensor, row and scale pointer
        const long rr = PAIR ? (r >> 1) : r;
        const uint8_t *wb = (PAIR && (r & 1)) ? w2 : w;
        const float *sb = (PAIR && (r & 1)) ? scales2 : scales;
        const uint8_t *p = wb + rr * stride;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) load_w<LW>(p + cb[k], b[k]);
        if constexpr (GS) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) gv[k] = sb[rr * ng + grp[k]];
        }
    };
    // The activations are requested first, straight from global memory (an
    // LDS copy per block measured slower: its barrier holds back the weight
    // stream), then the first D weight rows; vector loads complete in order,
    // so staging the activations waits for them alone.
    if constexpr (XV) {  // x 16-byte aligned and I % 4 == 0: a run is entirely inside or outside the row
        const uint32_t last4 = (uint32_t)(I - 4) * 4u;  // clamp: runs past the row are masked below
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const uint32_t b4 = (uint32_t)xb[k] * 4u, st4 = (uint32_t)xs_step[k] * 4u;
#pragma unroll
            for (int s = 0; s < SMAX; ++s)
                if (SMAX == 1 || s < S) {
                    const char *xs = reinterpret_cast<const char *>(x + (long)s * I);  // wave-uniform base
#pragma unroll
                    for (int g = 0; g < EPC / 4; ++g) {
                        const uint32_t off = min(b4 + st4 * (uint32_t)g, last4);
                        float4 t = *reinterpret_cast<const float4 *>(xs + off);
                        if (!wave_in) {  // runs past the row (or of a dead slot) are zero
                            const bool in = live[k] && WQ_XE(k, g) + 4 <= I;
                            t.x = in ? t.x : 0.0f;
                            t.y = in ? t.y : 0.0f;
                            t.z = in ? t.z : 0.0f;
                            t.w = in ? t.w : 0.0f;
                        }
                        xr[k][4 * g][s] = t.x;
                        xr[k][4 * g + 1][s] = t.y;
                        xr[k][4 * g + 2][s] = t.z;
                        xr[k][4 * g + 3][s] = t.w;
                    }
                } else {  // activation rows past S contribute zero
#pragma unroll
                    for (int e = 0; e < EPC; ++e) xr[k][e][s] = 0.0f;
                }
        }
    } else {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
#pragma unroll
            for (int s = 0; s < SMAX; ++s)
                if (SMAX == 1 || s < S) {
                    const float *xs = x + (long)s * I;
#pragma unroll
                    for (int e = 0; e < EPC; ++e) {
                        const int ei = WQ_XE(k, e / 4) + (e & 3);
                        xr[k][e][s] = xs[(live[k] && ei < I) ? ei : 0];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < EPC; ++e) xr[k][e][s] = 0.0f;
                }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load_row(ring[d], gring[d], row_begin + d);
        __builtin_amdgcn_sched_barrier(0);  // rows issued in ring order (waits count whole rows)
    }

    // (16-byte activation runs are already zero where they leave the row)
    constexpr int NC = kChains<FMT, SMAX>;
    if (XV || wave_in) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
#pragma unroll
            for (int s = 0; s < SMAX; ++s)
#pragma unroll
                for (int e = 0; e < EPC; ++e) xr[k][e][s] *= x_prescale<FMT, SMAX>(e % EPW);
    } else if constexpr (!XV) {
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
#pragma unroll
            for (int s = 0; s < SMAX; ++s)
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    const int ei = WQ_XE(k, e / 4) + (e & 3);
                    const bool in = live[k] && ei < I;
                    xr[k][e][s] = (in ? xr[k][e][s] : 0.0f) * x_prescale<FMT, SMAX>(e % EPW);
                }
    }
#undef WQ_XE

    // This lane's partial sums of one row (reduced over the wave later, for
    // all rows of a ring pass at once).
    auto row_partials = [&](uint32_t (&b)[KMAX][WPC], const float (&gv)[KMAX], float (&part)[SMAX]) {
        if constexpr (FMT == WQ_F32) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k)
                if (!live[k]) {
#pragma unroll
                    for (int j = 0; j < WPC; ++j) b[k][j] = 0u;
                }
        }
        float acc[NC][SMAX];  // code sums per chain (not GS)
        float gacc[SMAX];     // GS: sum of the group-scaled slot sums
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            gacc[s] = 0.0f;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c][s] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < KMAX; ++k)
            if (k < K) {
                if constexpr (GS) {
                    // the slot's sum times its group scale
                    float t[NC][SMAX];
#pragma unroll
                    for (int c = 0; c < NC; ++c)
#pragma unroll
                        for (int s = 0; s < SMAX; ++s) t[c][s] = 0.0f;
#pragma unroll
                    for (int j = 0; j < WPC; ++j) word_fma<FMT, SMAX>(b[k][j], &xr[k][j * EPW], t);
#pragma unroll
                    for (int s = 0; s < SMAX; ++s) {
                        float u = 0.0f;
#pragma unroll
                        for (int c = 0; c < NC; ++c) u += t[c][s];
                        gacc[s] = fmaf(gv[k], u, gacc[s]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < WPC; ++j) word_fma<FMT, SMAX>(b[k][j], &xr[k][j * EPW], acc);
                }
            }
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
            float t = 0.0f;
            if constexpr (GS) {
                t = gacc[s];
            } else {
#pragma unroll
                for (int c = 0; c < NC; ++c) t += acc[c][s];
            }
            part[s] = t;
        }
    };

    // The wave totals of part[d][s]: paired rows reduce the gate (even d)
    // and up (odd d) values separately, so both totals of an output sit in
    // the same lane.
    constexpr int NS = PAIR ? D / 2 * SMAX : D * SMAX;
    auto tot_lane = [&](int d, int s) { return sum_lane<NS>(PAIR ? (d >> 1) * SMAX + s : d * SMAX + s); };
    auto reduce = [&](float (&part)[D][SMAX]) {
        if constexpr (PAIR) {
            float gv[NS], uv[NS];
#pragma unroll
            for (int d = 0; d < D; d += 2)
#pragma unroll
                for (int s = 0; s < SMAX; ++s) {
                    gv[(d >> 1) * SMAX + s] = part[d][s];
                    uv[(d >> 1) * SMAX + s] = part[d + 1][s];
                }
            wave_sums_rows(gv);
            wave_sums_rows(uv);
#pragma unroll
            for (int d = 0; d < D; d += 2)
#pragma unroll
                for (int s = 0; s < SMAX; ++s) {
                    part[d][s] = gv[(d >> 1) * SMAX + s];
                    part[d + 1][s] = uv[(d >> 1) * SMAX + s];
                }
        } else {
            wave_sums_rows(reinterpret_cast<float(&)[D * SMAX]>(part));
        }
    };

    // Finish D rows starting at row0: lane tot_lane(d, s) of part[d][s]
    // holds this wave's total.
    int pb = 0;
    const int Oy = PAIR ? O / 2 : O;  // output rows (row stride of y)
    int cpos = 0;  // rows of the open chunk (team > 1, not PAIR)
    auto finish = [&](int row0, float (&part)[D][SMAX], int nvalid, bool last) {
        if constexpr (PAIR) {
            if (team == 1) {
#pragma unroll
                for (int d = 0; d < D; d += 2) {
                    if (d < nvalid) {
                        const int o = (row0 + d) >> 1;
                        const int oc = min(o, Oy - 1);
                        const float sg = GS ? 1.0f : uniform_ld(scales + oc);
                        const float su = GS ? 1.0f : uniform_ld(scales2 + oc);
                        if (row0 + d <= row_last) {
#pragma unroll
                            for (int s = 0; s < SMAX; ++s)
                                if (lane == tot_lane(d, s) && s < S)
                                    y[(long)s * Oy + o] = gated(sg * part[d][s], su * part[d + 1][s]);
                        }
                    }
                }
            } else {
                float *rbuf = red + pb * (kMaxTeam * D * SMAX);
#pragma unroll
                for (int d = 0; d < D; ++d)
#pragma unroll
                    for (int s = 0; s < SMAX; ++s)
                        if (lane == tot_lane(d, s)) rbuf[(wave_in_team * D + d) * SMAX + s] = part[d][s];
                float sg[D / 2], su[D / 2];
#pragma unroll
                for (int j = 0; j < D / 2; ++j) {
                    const int oc = min((row0 >> 1) + j, Oy - 1);
                    sg[j] = GS ? 1.0f : uniform_ld(scales + oc);
                    su[j] = GS ? 1.0f : uniform_ld(scales2 + oc);
                }
                __syncthreads();
                if (wave_in_team == 0 && lane < (D / 2) * SMAX) {
                    const int j = lane / SMAX, s = lane % SMAX;
                    const int d = 2 * j;
                    float tg = 0.0f, tu = 0.0f;
                    for (int w2i = 0; w2i < team; ++w2i) {
                        tg += rbuf[(w2i * D + d) * SMAX + s];
                        tu += rbuf[(w2i * D + d + 1) * SMAX + s];
                    }
                    float g = sg[0], u = su[0];
#pragma unroll
                    for (int jj = 1; jj < D / 2; ++jj) {
                        g = (j == jj) ? sg[jj] : g;
                        u = (j == jj) ? su[jj] : u;
                    }
                    if (d < nvalid && row0 + d <= row_last && s < S)
                        y[(long)s * Oy + ((row0 + d) >> 1)] = gated(g * tg, u * tu);
                }
                pb ^= 1;
            }
            return;
        }
        if (team == 1) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                if (d < nvalid) {
                    const int row = row0 + d;
                    const float sc = GS ? 1.0f : uniform_ld(scales + min(row, O - 1));
                    if (row <= row_last) {
#pragma unroll
                        for (int s = 0; s < SMAX; ++s)
                            if (lane == tot_lane(d, s) && s < S) y[(long)s * O + row] = sc * part[d][s];
                    }
                }
            }
        } else {
            // Several waves share each row: their totals (and the row scales)
            // collect in LDS over a chunk of kTeamChunk rows, and the block
            // syncs once per chunk; wave 0 then adds the team's totals in
            // wave order. Two chunk buffers: the barrier that closes chunk
            // n + 1 also tells that wave 0 has read chunk n.
            float *cbuf = red + pb * (kTeamChunk * kMaxTeam * SMAX);
            float *sbuf = red + 2 * (kTeamChunk * kMaxTeam * SMAX) + pb * kTeamChunk;
#pragma unroll
            for (int d = 0; d < D; ++d)
#pragma unroll
                for (int s = 0; s < SMAX; ++s)
                    if (lane == tot_lane(d, s)) cbuf[((cpos + d) * kMaxTeam + wave_in_team) * SMAX + s] = part[d][s];
            if (wave_in_team == 0) {
#pragma unroll
                for (int d = 0; d < D; ++d) {
                    const float sc = GS ? 1.0f : uniform_ld(scales + min(row0 + d, O - 1));  // scalar load
                    if (lane == 63) sbuf[cpos + d] = sc;
                }
            }
            cpos += D;
            if (cpos + D > kTeamChunk || last) {  // the chunk holds kTeamChunk / D whole passes
                __syncthreads();
                if (wave_in_team == 0) {
                    const int crow0 = row0 + D - cpos;  // first row of the chunk
                    for (int j = lane; j < cpos * SMAX; j += 64) {
                        const int r = j / SMAX, s = j % SMAX;
                        const int row = crow0 + r;
                        float t = 0.0f;
                        for (int w2 = 0; w2 < team; ++w2) t += cbuf[(r * kMaxTeam + w2) * SMAX + s];
                        if (r < cpos - D + nvalid && row <= row_last && s < S) y[(long)s * O + row] = sbuf[r] * t;
                    }
                }
                pb ^= 1;
                cpos = 0;
            }
        }
    };

    // ---- stream rows through the ring
    int i = 0;
    for (; i + D < rpt; i += D) {
        float part[D][SMAX];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            row_partials(ring[d], gring[d], part[d]);
            load_row(ring[d], gring[d], row_begin + i + d + D);
            // keep the refill of this ring slot right here: left to itself
            // the scheduler sinks it below the next row's arithmetic, and the
            // wave then has no weight load in flight between ring passes
            __builtin_amdgcn_sched_barrier(0);
        }
        reduce(part);
        finish(row_begin + i, part, D, false);
    }
    {
        float part[D][SMAX];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (i + d < rpt) {
                row_partials(ring[d], gring[d], part[d]);
            } else {
#pragma unroll
                for (int s = 0; s < SMAX; ++s) part[d][s] = 0.0f;
            }
        }
        reduce(part);
        finish(row_begin + i, part, rpt - i, true);
    }
}

template <int FMT, int SMAX, int LW, int KS, int D, bool XV, bool GS = false, bool PAIR = false>
__global__ __launch_bounds__(512) void gemv_kernel(GemvArgs a) {
    // team > 1: two chunk buffers of totals and scales (paired rows: two
    // ring passes of totals, which fit in the same space)
    __shared__ float red[2 * kTeamChunk * kMaxTeam * SMAX + 2 * kTeamChunk];
    static_assert(2 * kMaxTeam * D * SMAX <= 2 * kTeamChunk * kMaxTeam * SMAX, "paired reduction space");
    static_assert(D <= kTeamChunk, "a chunk holds whole ring passes");
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int team_in_block = wave / a.team;
    const int wave_in_team = wave - team_in_block * a.team;
    const int team_id = blockIdx.x * a.teams_per_block + team_in_block;
    const int row_begin = team_id * a.rows_per_team;
    if (row_begin >= a.O) return;  // uniform over the team (and the block when team > 1)
    team_rows<FMT, SMAX, LW, KS, D, XV, GS, PAIR>(a.w, a.stride, a.nfull, a.scales, a.x, a.y, a.O, a.I, a.S, a.team,
                                                  wave_in_team * 64 + lane, wave_in_team, row_begin,
                                                  a.rows_per_team, red, a.gs, a.ng, a.w2, a.scales2);
}

// PAIR: every problem is a (gate, up) pair; its work items count virtual rows.
// KS > 0: every item of the launch has KS load slots, and the kernel's
// registers are those of its rows. KS == 0: the items of one launch may need
// any slot count 1..KMAX (rows of different lengths, e.g. the gate/up and
// down projections of a mixture-of-experts layer in one launch); each wave
// takes the code path compiled for its item's count, and the registers are
// those of the longest rows present in the compiled set.
template <int FMT, int SMAX, int LW, int KMAX, int D, bool XV, bool PAIR, int KS>
__global__ __launch_bounds__(256) void grouped_kernel(GroupedArgs a) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int item_id = blockIdx.x * 4 + wave;
    if (item_id >= a.n_items) return;
    const WorkItem it = a.items[item_id];
    const int k = __builtin_amdgcn_readfirstlane(it.k);
    const int p = __builtin_amdgcn_readfirstlane(it.p);
    const int S = a.S[p];
    if (S <= 0) return;
    const GroupDesc d = a.desc[p];
    const int r0 = __builtin_amdgcn_readfirstlane(it.row_begin);
    const int nr = __builtin_amdgcn_readfirstlane(it.row_end - it.row_begin);
#define WQ_RUN(KU)                                                                                               \
    team_rows<FMT, SMAX, LW, KU, ring_depth(KMAX, D, KU), XV, false, PAIR>(                                    \
        d.w, d.stride, d.nfull, d.scales, a.x[p], a.y[p], PAIR ? 2 * d.O : d.O, d.I, S, 1, lane, 0, r0, nr, nullptr, \
        0, 1, d.w2, d.scales2)
    if constexpr (KS > 0) {
        if (k == KS) WQ_RUN(KS);  // (a table built for another slot count runs nothing)
    } else {
        if (k == 1) WQ_RUN(1);
        if constexpr (KMAX >= 2) if (k == 2) WQ_RUN(2);
        if constexpr (KMAX >= 3) if (k == 3) WQ_RUN(3);
        if constexpr (KMAX >= 4) if (k == 4) WQ_RUN(4);
    }
#undef WQ_RUN
}

// ---- compiled shapes -------------------------------------------------------
// (fmt, S bucket) -> bytes per lane load, load slots, ring depth of the
// grouped launch, ring depth and default waves per CU of the single-tensor
// GEMV. Registers: activations KMAX * (LW/4 * EPW) * SMAX, ring
// D * KMAX * LW/4. int4 at S = 1 runs one wave per SIMD with a 4-row ring:
// half the activation staging of 8 waves per CU and enough rows in flight
// (9.0 us vs 9.6 for dense_gemv); the grouped launches keep 2 rows and 8
// waves per CU (their expert rows are few per wave).
#define WQ_SHAPES(X)                                                   \
    X(WQ_F32, 1, 16, 4, 2, 2, 8) X(WQ_F32, 2, 16, 4, 2, 2, 8)          \
    X(WQ_F32, 4, 16, 4, 2, 2, 8) X(WQ_F32, 8, 16, 4, 2, 2, 8)          \
    X(WQ_I8, 1, 16, 4, 2, 2, 8) X(WQ_I8, 2, 16, 2, 2, 2, 8)            \
    X(WQ_I8, 4, 16, 1, 4, 4, 8) X(WQ_I8, 8, 8, 1, 4, 4, 8)             \
    X(WQ_I4, 1, 16, 4, 2, 4, 4) X(WQ_I4, 2, 16, 1, 2, 2, 8)            \
    X(WQ_I4, 4, 16, 1, 4, 4, 8) X(WQ_I4, 8, 8, 1, 4, 4, 8)             \
    X(WQ_I2, 1, 16, 1, 2, 2, 8) X(WQ_I2, 2, 8, 1, 4, 4, 8)             \
    X(WQ_I2, 4, 8, 1, 4, 4, 8) X(WQ_I2, 8, 4, 1, 4, 4, 8)

__global__ void relayout_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst, int fmt, int O,
                                long rb, long stride, int nfull) {
    const long n = (long)O * stride;
    for (long i = blockIdx.x * (long)blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
        const long o = i / stride, p = i - o * stride;
        dst[i] = p < rb ? src[o * rb + natural_byte_of(fmt, p, nfull)] : (uint8_t)0;
    }
}

// The same for expert blockIdx.y of a launch over several experts.
__global__ void gated_group_kernel(GatedGroupArgs a) {
    float *h = a.e[blockIdx.y].h;
    const float *u = a.e[blockIdx.y].u;
    const int n = a.e[blockIdx.y].count;
    for (int j = blockIdx.x * 256 + threadIdx.x; j < n; j += gridDim.x * 256) h[j] = gated(h[j], u[j]);
}

// h[j] = gated(h[j], u[j]): the activation step of the gated feed-forward
// when gate and up ran as separate matmuls (h holds g on entry).
__global__ void gated_inplace_kernel(float *__restrict__ h, const float *__restrict__ u, long n) {
    for (long j = blockIdx.x * (long)blockDim.x + threadIdx.x; j < n; j += (long)gridDim.x * blockDim.x)
        h[j] = gated(h[j], u[j]);
}

} // namespace

hipError_t launch_gated_group(const GatedGroupArgs &a, int max_count, hipStream_t st) {
    if (a.n <= 0 || max_count <= 0) return hipSuccess;
    const dim3 grid((unsigned)std::min((max_count + 255) / 256, 64), (unsigned)a.n);
    hipLaunchKernelGGL(gated_group_kernel, grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_gated_inplace(float *h, const float *u, long n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int block = 256;
    const int grid = (int)std::min<long>((n + block - 1) / block, 4096);
    hipLaunchKernelGGL(gated_inplace_kernel, dim3(grid), dim3(block), 0, st, h, u, n);
    return hipGetLastError();
}

int gemv_smax_bucket(int S) {
    if (S <= 1) return 1;
    if (S <= 2) return 2;
    if (S <= 4) return 4;
    if (S <= 8) return 8;
    return 0;
}

GemvShape gemv_shape(int fmt, int smax) {
#define WQ_SHAPE_CASE(F, SM, LW, KM, D, DG, WG) \
    if (fmt == F && smax == SM) return GemvShape{LW, KM, D, DG, WG};
    WQ_SHAPES(WQ_SHAPE_CASE)
#undef WQ_SHAPE_CASE
    return GemvShape{0, 0, 0, 0, 0};
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
    const long stride = round_up(row_bytes(fmt, I), kRowAlign);
    // Slots per lane: up to kmax, a team of waves sharing a longer row.
    // Group-scaled tensors take the same shape (measured against one-slot
    // teams at 8 waves per CU, µs: int4 12288 x 6144 gs = 128 11.0 vs 12.7,
    // int8 6144 x 6144 8.8 vs 9.3, int2 16384 x 8192 15.5 both).
    const long per_wave = 64L * sh.lw * sh.kmax;
    const long team = (stride + per_wave - 1) / per_wave;
    if (team > kMaxTeam) return p;  // row too long for the register GEMV
    p.team = (int)team;
    p.k = (int)((stride + 64L * p.lw * p.team - 1) / (64L * p.lw * p.team));
    p.d = ring_depth(sh.kmax, sh.dg, p.k);
    p.teams_per_block = (p.team == 1) ? 4 : 1;
    p.block = 64 * p.team * p.teams_per_block;
    // teams: enough waves to keep HBM busy, rows per team a multiple of the ring depth
    const int wpc = waves_per_cu > 0 ? waves_per_cu : sh.wg;
    const long want_teams = std::max(1L, (long)cus * wpc / p.team);
    long teams = std::min(want_teams, ((long)O + p.d - 1) / p.d);
    long rpt = ((long)O + teams - 1) / teams;
    rpt = (rpt + p.d - 1) / p.d * p.d;
    teams = ((long)O + rpt - 1) / rpt;
    p.rows_per_team = (int)rpt;
    p.grid = (int)((teams + p.teams_per_block - 1) / p.teams_per_block);
    p.ok = true;
    return p;
}

// DG: the ring depth of the single-tensor GEMV (the plan's, see plan_gemv).
template <int F, int SM, int LW, int KM, int DG>
hipError_t launch_gemv_k(const GemvPlan &p, const GemvArgs &a, bool xv, hipStream_t st) {
    // exact slot count: 1..KM; 16-byte activation loads when x allows (xv)
#define WQ_GO(KS, GS_, PAIR_)                                                                                   \
    do {                                                                                                        \
        constexpr int RD = ring_depth(KM, DG, KS);                                                              \
        if (xv)                                                                                                 \
            hipLaunchKernelGGL((gemv_kernel<F, SM, LW, KS, RD, true, GS_, PAIR_>), dim3(p.grid), dim3(p.block), \
                               0, st, a);                                                                       \
        else                                                                                                    \
            hipLaunchKernelGGL((gemv_kernel<F, SM, LW, KS, RD, false, GS_, PAIR_>), dim3(p.grid), dim3(p.block),\
                               0, st, a);                                                                       \
        return hipGetLastError();                                                                               \
    } while (0)
#define WQ_K(KS)                                                     \
    if constexpr (KS <= KM) {                                        \
        if (p.k == KS) {                                             \
            if (a.w2 != nullptr) {                                   \
                if (a.gs > 0) return hipErrorInvalidValue;           \
                WQ_GO(KS, false, true);                              \
            }                                                        \
            if constexpr (F != WQ_F32) {                             \
                if (a.gs > 0) WQ_GO(KS, true, false);                \
            }                                                        \
            WQ_GO(KS, false, false);                                 \
        }                                                            \
    }
    WQ_K(1) WQ_K(2) WQ_K(3) WQ_K(4)
#undef WQ_K
#undef WQ_GO
    return hipErrorInvalidValue;
}

hipError_t launch_gemv(const GemvPlan &p, const GemvArgs &a, hipStream_t st) {
    const bool xv = (a.I % 4 == 0) && ((reinterpret_cast<uintptr_t>(a.x) & 15) == 0);
#define WQ_LAUNCH_CASE(F, SM, LW, KM, D, DG, WG) \
    if (p.fmt == F && p.smax == SM) return launch_gemv_k<F, SM, LW, KM, DG>(p, a, xv, st);
    WQ_SHAPES(WQ_LAUNCH_CASE)
#undef WQ_LAUNCH_CASE
    return hipErrorInvalidValue;
}

template <int F, int SM, int LW, int KM, int D>
hipError_t launch_grouped_k(const GroupedPlan &p, const GroupedArgs &a, bool xv, bool pair, int ks,
                            hipStream_t st) {
#define WQ_GK(KU)                                                                                         \
    if constexpr (KU <= KM) {                                                                             \
        if (ks == KU) {                                                                                   \
            if (pair && xv)                                                                               \
                hipLaunchKernelGGL((grouped_kernel<F, SM, LW, KM, D, true, true, KU>), dim3(p.grid),      \
                                   dim3(p.block), 0, st, a);                                              \
            else if (pair)                                                                                \
                hipLaunchKernelGGL((grouped_kernel<F, SM, LW, KM, D, false, true, KU>), dim3(p.grid),     \
                                   dim3(p.block), 0, st, a);                                              \
            else if (xv)                                                                                  \
                hipLaunchKernelGGL((grouped_kernel<F, SM, LW, KM, D, true, false, KU>), dim3(p.grid),     \
                                   dim3(p.block), 0, st, a);                                              \
            else                                                                                          \
                hipLaunchKernelGGL((grouped_kernel<F, SM, LW, KM, D, false, false, KU>), dim3(p.grid),    \
                                   dim3(p.block), 0, st, a);                                              \
            return hipGetLastError();                                                                     \
        }                                                                                                 \
    }
    WQ_GK(0) WQ_GK(1) WQ_GK(2) WQ_GK(3) WQ_GK(4)
#undef WQ_GK
    return hipErrorInvalidValue;
}

hipError_t launch_grouped(int fmt, const GroupedPlan &p, const GroupedArgs &a, bool xv, bool pair, int ks,
                          hipStream_t st) {
#define WQ_GLAUNCH_CASE(F, SM, LW, KM, D, DG, WG) \
    if (fmt == F && p.smax == SM) return launch_grouped_k<F, SM, LW, KM, D>(p, a, xv, pair, ks, st);
    WQ_SHAPES(WQ_GLAUNCH_CASE)
#undef WQ_GLAUNCH_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_relayout(int fmt, const uint8_t *src, uint8_t *dst, int O, long rb, long stride, int nfull,
                           hipStream_t st) {
    const long n = (long)O * stride;
    const int block = 256;
    const long want = (n + block - 1) / block;
    const int grid = (int)std::min<long>(std::max<long>(want, 1), 65536);
    hipLaunchKernelGGL(relayout_kernel, dim3(grid), dim3(block), 0, st, src, dst, fmt, O, rb, stride, nfull);
    return hipGetLastError();
}

} // namespace wq
