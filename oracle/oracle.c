/*
 * oracle.c -- plain f64 CPU oracle (test infrastructure only; see oracle.h).
 *
 * Written from the definitions on the Metal Compute Kernels page of the S-MoE
 * docs.  Nothing here is blocked, fused or reordered: every weight is
 * dequantised on its own, and every sum runs in ascending index order with a
 * single f64 accumulator.  The only parallelism is an OpenMP loop over
 * independent output rows, which does not change any sum.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Affine zero point of a b-bit code: the midpoint of 0 .. 2^b-1.  The page
 * ("Fused FFN Kernels", affine weight definition) gives 7.5 at Q4 and 1.5 at Q2. */
static double zero_point(int bits)
{
    return bits == 4 ? 7.5 : 1.5;
}

static int check(int bits, int group, long rows, long cols)
{
    if (bits != 4 && bits != 2) return -1;
    if (rows <= 0 || cols <= 0 || group <= 0) return -1;
    if (cols % group) return -1;
    if ((cols * bits) % 8) return -1;
    return 0;
}

/* Code of column j in a packed row: 4-bit codes low nibble first, 2-bit codes
 * from the least significant bit pair up. */
static unsigned code_at(const uint8_t *row, int bits, long j)
{
    if (bits == 4)
        return (row[j / 2] >> (4 * (j % 2))) & 0xFu;
    return (row[j / 4] >> (2 * (j % 4))) & 0x3u;
}

/* w = (code - Z) / Z * s  ("Fused FFN Kernels -- One Simdgroup Per Output Row"). */
static double weight(const uint8_t *codes, const float *scales, int bits, int group,
                     long cols, long r, long j)
{
    const double Z = zero_point(bits);
    const uint8_t *row = codes + r * (cols * bits / 8);
    const double s = (double)scales[r * (cols / group) + j / group];
    return ((double)code_at(row, bits, j) - Z) / Z * s;
}

int oracle_unpack(const uint8_t *codes, int bits, long rows, long cols, uint8_t *out)
{
    if (!codes || !out || check(bits, 1, rows, cols)) return -1;
    for (long r = 0; r < rows; ++r)
        for (long j = 0; j < cols; ++j)
            out[r * cols + j] = (uint8_t)code_at(codes + r * (cols * bits / 8), bits, j);
    return 0;
}

int oracle_dequant(const uint8_t *codes, const float *scales, int bits, int group,
                   long rows, long cols, double *w)
{
    if (!codes || !scales || !w || check(bits, group, rows, cols)) return -1;
    for (long r = 0; r < rows; ++r)
        for (long j = 0; j < cols; ++j)
            w[r * cols + j] = weight(codes, scales, bits, group, cols, r, j);
    return 0;
}

/* A quantised projection y = W x, each weight dequantised explicitly. */
int oracle_qmatvec(const uint8_t *codes, const float *scales, int bits, int group,
                   long rows, long cols, const double *x, double *y)
{
    if (!codes || !scales || !x || !y || check(bits, group, rows, cols)) return -1;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (long j = 0; j < cols; ++j)
            acc += weight(codes, scales, bits, group, cols, r, j) * x[j];
        y[r] = acc;
    }
    return 0;
}

/* SiLU(t) = t * sigmoid(t) = t / (1 + e^-t); the page names SiLU without
 * defining it, and this is the textbook definition. */
double oracle_silu(double t)
{
    return t / (1.0 + exp(-t));
}

/* gate_up of one expert ("Fused FFN Kernels": hidden = SiLU(gate x) * (up x),
 * both projections reading the same input vector). */
int oracle_gate_up(const oracle_qmat *gate, const oracle_qmat *up, int bits, int group,
                   long d_ff, long d_model, const float *x, double *hidden)
{
    if (!gate || !up || !x || !hidden || check(bits, group, d_ff, d_model)) return -1;
    double *xd = malloc(sizeof(double) * d_model);
    double *g = malloc(sizeof(double) * d_ff);
    double *u = malloc(sizeof(double) * d_ff);
    int rc = -1;
    if (!xd || !g || !u) goto out;
    for (long j = 0; j < d_model; ++j) xd[j] = (double)x[j];
    if (oracle_qmatvec(gate->codes, gate->scales, bits, group, d_ff, d_model, xd, g)) goto out;
    if (oracle_qmatvec(up->codes, up->scales, bits, group, d_ff, d_model, xd, u)) goto out;
    for (long i = 0; i < d_ff; ++i) hidden[i] = oracle_silu(g[i]) * u[i];
    rc = 0;
out:
    free(xd); free(g); free(u);
    return rc;
}

/* down of one expert ("Fused FFN Kernels": out = down_proj . hidden, shape d_model). */
int oracle_down(const oracle_qmat *down, int bits, int group, long d_model, long d_ff,
                const double *hidden, double *out)
{
    if (!down || !hidden || !out || check(bits, group, d_model, d_ff)) return -1;
    return oracle_qmatvec(down->codes, down->scales, bits, group, d_model, d_ff, hidden, out);
}

/* Routed experts over a token batch.  Each token goes through every listed
 * expert ("Token-Batch Fused FFN": one expert applied to many token rows);
 * the expert outputs are combined with the router weights, experts ascending.
 * The pages describe no combine step; a router-weighted sum is the reading. */
int oracle_expert_ffn(const oracle_expert *experts, int n_experts, const float *route_w,
                      int bits, int group, long d_model, long d_ff, long T,
                      const float *x, double *out)
{
    if (!experts || !x || !out || n_experts <= 0 || T <= 0) return -1;
    if (check(bits, group, d_ff, d_model) || check(bits, group, d_model, d_ff)) return -1;
    double *h = malloc(sizeof(double) * d_ff);
    double *y = malloc(sizeof(double) * d_model);
    int rc = -1;
    if (!h || !y) goto out;
    for (long t = 0; t < T; ++t) {
        double *o = out + t * d_model;
        for (long j = 0; j < d_model; ++j) o[j] = 0.0;
        for (int e = 0; e < n_experts; ++e) {
            const oracle_expert *ex = &experts[e];
            if (oracle_gate_up(&ex->gate, &ex->up, bits, group, d_ff, d_model,
                               x + t * d_model, h)) goto out;
            if (oracle_down(&ex->down, bits, group, d_model, d_ff, h, y)) goto out;
            const double r = route_w ? (double)route_w[t * n_experts + e] : 1.0;
            for (long j = 0; j < d_model; ++j) o[j] += r * y[j];
        }
    }
    rc = 0;
out:
    free(h); free(y);
    return rc;
}

/* Routed experts: token t goes through the top_k experts listed for it, each
 * listed slot being one expert application ("Token-Batch Fused FFN": the
 * tokens that chose an expert are run through it together; per token, its
 * experts' outputs are combined with the router weights).
 *   out[t][:] = sum over slots j < top_k, ascending, of w[t][j] * FFN_{ids[t][j]}(x[t]);
 * a slot whose id is outside [0, n_experts) adds nothing. */
int oracle_routed_ffn(const oracle_expert *experts, int n_experts, int bits, int group, long d_model,
                      long d_ff, long T, int top_k, const int *ids, const float *w, const float *x,
                      double *out)
{
    if (!experts || !ids || !w || !x || !out || n_experts <= 0 || T <= 0 || top_k <= 0) return -1;
    if (check(bits, group, d_ff, d_model) || check(bits, group, d_model, d_ff)) return -1;
    double *h = malloc(sizeof(double) * d_ff);
    double *y = malloc(sizeof(double) * d_model);
    int rc = -1;
    if (!h || !y) goto out;
    for (long t = 0; t < T; ++t) {
        double *o = out + t * d_model;
        for (long j = 0; j < d_model; ++j) o[j] = 0.0;
        for (int s = 0; s < top_k; ++s) {
            const int e = ids[t * top_k + s];
            if (e < 0 || e >= n_experts) continue;
            const oracle_expert *ex = &experts[e];
            if (oracle_gate_up(&ex->gate, &ex->up, bits, group, d_ff, d_model,
                               x + t * d_model, h)) goto out;
            if (oracle_down(&ex->down, bits, group, d_model, d_ff, h, y)) goto out;
            const double r = (double)w[t * top_k + s];
            for (long j = 0; j < d_model; ++j) o[j] += r * y[j];
        }
    }
    rc = 0;
out:
    free(h); free(y);
    return rc;
}

/* IEEE 754 binary16 to double, from the format's definition: sign bit 15,
 * exponent bits 10..14 with bias 15, fraction bits 0..9.  An exponent field of
 * 0 is a subnormal, fraction * 2^-24; 31 is an infinity (fraction 0) or a NaN;
 * otherwise the value is (1024 + fraction) * 2^(exponent - 25).  Every
 * binary16 value is exactly a binary32 value.  Used for the 2-byte scale
 * layout, which the kernels' callers may pass instead of f32 scales. */
static double f16_value(uint16_t h)
{
    const int sign = h >> 15, e = (h >> 10) & 0x1F, m = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

int oracle_f16_widen(const uint16_t *h, long n, float *out)
{
    if (!h || !out || n < 0) return -1;
    for (long i = 0; i < n; ++i) out[i] = (float)f16_value(h[i]);
    return 0;
}

/* bf16 bits to f32: the bf16 pattern is the upper half of the f32 pattern, so
 * widening is exact ("Coalesced Dense Matvec -- the Same Contract for bf16"). */
static double bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_matvec_bf16(const uint16_t *W, long rows, long cols, const float *x, double *y)
{
    if (!W || !x || !y || rows <= 0 || cols <= 0) return -1;
#pragma omp parallel for schedule(static)
    for (long r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (long j = 0; j < cols; ++j)
            acc += bf16_value(W[r * cols + j]) * (double)x[j];
        y[r] = acc;
    }
    return 0;
}
