/*
 * CPU oracle for the weight-only quantized matmul.
 *
 * TEST INFRASTRUCTURE ONLY. Tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library; the product library never does.
 * It shares no source, header, table or helper with the HIP library.
 *
 * What it computes (colibri "第 8 章 · 02 CUDA/Metal/Vulkan 三后端", section 四,
 * the qmatmul.comp header; colibri-analysis "CUDA 后端", section 1, the
 * quant_matmul and weight_at descriptions):
 *
 *     y[s,o] = scale[o] * sum_{i=0}^{I-1} dequant(W[o,i]) * x[s,i]
 *
 * with the per-row scale applied once, after the sum over i.
 *
 * Arithmetic: every product q*x is exact in IEEE double (q has at most 8 bits,
 * x at most 24). The sum runs in ascending i in double, the result is
 * multiplied by the scale in double and rounded once to float.
 *
 * Readings of the pages used here (they are silent or truncated on these):
 *   - format codes 0 = f32, 1 = int8, 2 = int4, 3 = int2 (the Vulkan tensor
 *     description lists 0/1/2 and stops; row_bytes names exactly f32, int8,
 *     int4, int2, so int2 takes the next code);
 *   - int8 is two's complement with no offset;
 *   - int4: two elements per byte, the even element in the low nibble,
 *     value = nibble - 8;
 *   - int2: four elements per byte, element 4j+k in bits 2k..2k+1 of byte j,
 *     value = code - 2;
 *   - each row occupies ceil(I * bits / 8) bytes; unused high bits of a row's
 *     last byte are ignored;
 *   - f32 weights may come without scales; a NULL scale array means 1.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_I8 1
#define ORACLE_I4 2
#define ORACLE_I2 3

/* Bytes one packed row of I elements occupies (colibri-analysis "CUDA 后端",
 * section 1, row_bytes). Returns -1 for an unknown format or I < 0. */
long oracle_row_bytes(int fmt, long I)
{
    if (I < 0)
        return -1;
    switch (fmt) {
    case ORACLE_F32: return 4 * I;
    case ORACLE_I8: return I;
    case ORACLE_I4: return (I + 1) / 2;
    case ORACLE_I2: return (I + 3) / 4;
    default: return -1;
    }
}

/* Dequantized value of element i of one packed row (colibri-analysis
 * "CUDA 后端", section 1, weight_at: int4 minus 8, int2 minus 2). */
double oracle_weight(int fmt, const unsigned char *row, long i)
{
    switch (fmt) {
    case ORACLE_F32: {
        float f;
        memcpy(&f, row + 4 * i, sizeof f); /* little-endian host */
        return (double)f;
    }
    case ORACLE_I8: {
        int v = row[i];
        if (v >= 128)
            v -= 256;
        return (double)v;
    }
    case ORACLE_I4: {
        int byte = row[i / 2];
        int nib = (i % 2 == 0) ? (byte & 0xF) : ((byte >> 4) & 0xF);
        return (double)(nib - 8);
    }
    case ORACLE_I2: {
        int byte = row[i / 4];
        int code = (byte >> (2 * (int)(i % 4))) & 0x3;
        return (double)(code - 2);
    }
    default:
        return NAN;
    }
}

/*
 * y[s*O + o] = fl32(scale[o] * sum_i q[o,i] * x[s*I + i])  for s < S, o < O.
 *
 * w:      O packed rows, row o starting at w + o * row_stride (row_stride >=
 *         oracle_row_bytes(fmt, I)).
 * scales: O floats, or NULL (f32 only) for scale 1.
 * x:      S x I floats, row-major.
 * y:      S x O floats, row-major (written).
 * absb:   optional S x O doubles receiving sum_i |scale[o] * q[o,i] * x[s,i]|,
 *         the magnitude the acceptance bound is stated against.
 * nthreads: OpenMP threads over output rows o (results do not depend on it).
 *
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_matmul(int fmt, long O, long I, const unsigned char *w, long row_stride,
                  const float *scales, const float *x, long S, float *y, double *absb,
                  int nthreads)
{
    long rb = oracle_row_bytes(fmt, I);
    if (rb < 0 || O < 0 || S < 0 || row_stride < rb)
        return -1;
    if (scales == NULL && fmt != ORACLE_F32)
        return -1;
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long o = 0; o < O; ++o) {
        const unsigned char *row = w + o * row_stride;
        double scale = scales ? (double)scales[o] : 1.0;
        for (long s = 0; s < S; ++s) {
            const float *xs = x + s * I;
            double acc = 0.0, mag = 0.0;
            for (long i = 0; i < I; ++i) {
                double q = oracle_weight(fmt, row, i);
                double t = q * (double)xs[i];
                acc += t;
                mag += fabs(t);
            }
            y[s * O + o] = (float)(acc * scale);
            if (absb)
                absb[s * O + o] = mag * fabs(scale);
        }
    }
    return 0;
}

/*
 * Group-wise scales: one scale per (row o, group of gs consecutive columns).
 * The Vulkan tensor description ("三后端", section 三) carries a group-size
 * field next to the scales; the CUDA tensor there has per-row scales only.
 * Reading taken here: columns [g*gs, (g+1)*gs) of row o use
 * scales[o*ng + g], ng = ceil(I/gs) (the last group may be shorter), and
 *
 *     y[s,o] = fl32( sum_g scales[o,g] * sum_{i in group g} q[o,i] * x[s,i] )
 *
 * Each group's sum runs in ascending column order in double, is multiplied
 * by its scale in double and added to the row total in ascending group
 * order; one rounding to float at the end. absb receives
 * sum_i |scales[o, i/gs] * q[o,i] * x[s,i]|.
 *
 * scales: O x ng floats, row-major (required). gs >= 1.
 * Returns 0, or -1 on an invalid argument.
 */
int oracle_matmul_gs(int fmt, long O, long I, const unsigned char *w, long row_stride,
                     const float *scales, long gs, const float *x, long S, float *y, double *absb,
                     int nthreads)
{
    long rb = oracle_row_bytes(fmt, I);
    if (rb < 0 || O < 0 || S < 0 || row_stride < rb || gs < 1 || scales == NULL)
        return -1;
    long ng = (I + gs - 1) / gs;
    if (nthreads < 1)
        nthreads = 1;

#pragma omp parallel for schedule(static) num_threads(nthreads)
    for (long o = 0; o < O; ++o) {
        const unsigned char *wrow = w + o * row_stride;
        const float *srow = scales + o * ng;
        for (long s = 0; s < S; ++s) {
            const float *xrow = x + s * I;
            double total = 0.0, magnitude = 0.0;
            for (long g = 0; g < ng; ++g) {
                long first = g * gs, end = first + gs < I ? first + gs : I;
                double group_sum = 0.0, group_mag = 0.0;
                for (long c = first; c < end; ++c) {
                    double prod = oracle_weight(fmt, wrow, c) * (double)xrow[c];
                    group_sum += prod;
                    group_mag += fabs(prod);
                }
                double gscale = (double)srow[g];
                total += gscale * group_sum;
                magnitude += fabs(gscale) * group_mag;
            }
            y[s * O + o] = (float)total;
            if (absb)
                absb[s * O + o] = magnitude;
        }
    }
    return 0;
}

/*
 * SiLU-gated product of a mixture-of-experts feed-forward step. colibri
 * "第 8 章 · 02 CUDA/Metal/Vulkan 三后端" (learning goals and section recap)
 * names a gated up-projection shader, qmatmul_gate_up.comp, but shows neither
 * its body nor its activation; the reading taken is SiLU gating (SwiGLU):
 *
 *     h[j] = fl32( silu(g[j]) * u[j] ),   silu(z) = z / (1 + exp(-z)),
 *
 * evaluated in double from the float inputs (g = gate rows . x, u = up rows . x).
 */
void oracle_silu_mul(const float *g, const float *u, long n, float *h)
{
    for (long j = 0; j < n; ++j) {
        double z = (double)g[j];
        double silu = z / (1.0 + exp(-z));
        h[j] = (float)(silu * (double)u[j]);
    }
}
