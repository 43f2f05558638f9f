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

/* Threads of the row loops from now on (n >= 1); results do not depend on it. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
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

/* ------------------------------------------------------------------------
 * Decode attention block (S-MoE docs, Metal Compute Kernels page, section
 * "GPU-Resident Decode Attention": the Q/K/V projections, a per-head QK RMS
 * norm with 1e-6 added to the mean of squares, RoPE, K/V appended to the KV
 * cache, causal GQA attention for the new token, and the output projection).
 * ------------------------------------------------------------------------ */

/* y[h][d] = x[h][d] / sqrt(mean over d of x[h][d]^2 + eps) * w[d], each of
 * n_heads rows of hd values on its own.  The gain w (one per dimension,
 * shared by the heads) is the usual learned gain of an RMS norm; the page
 * names the norm and its 1e-6 only. */
int oracle_head_rmsnorm(const double *x, long n_heads, long hd, const float *w, double eps, double *y)
{
    if (!x || !w || !y || n_heads <= 0 || hd <= 0) return -1;
    for (long h = 0; h < n_heads; ++h) {
        const double *xh = x + h * hd;
        double ss = 0.0;
        for (long d = 0; d < hd; ++d) ss += xh[d] * xh[d];
        const double inv = 1.0 / sqrt(ss / (double)hd + eps);
        for (long d = 0; d < hd; ++d) y[h * hd + d] = xh[d] * inv * (double)w[d];
    }
    return 0;
}

/* Rotary position embedding at position pos, in place, each head on its
 * own: for i < hd/2 the pair (a, b) = (x[i], x[i + hd/2]) turns by the angle
 * pos * base^(-2i/hd), giving (a cos - b sin, a sin + b cos).  The page names
 * RoPE only; the half-split pairing and these frequencies are the rotary
 * embedding of the model family the page runs, taken as the reading. */
int oracle_rope(double *x, long n_heads, long hd, long pos, double base)
{
    if (!x || n_heads <= 0 || hd <= 0 || hd % 2 || pos < 0 || !(base > 0.0)) return -1;
    const long half = hd / 2;
    for (long h = 0; h < n_heads; ++h) {
        double *xh = x + h * hd;
        for (long i = 0; i < half; ++i) {
            const double ang = (double)pos * pow(base, -2.0 * (double)i / (double)hd);
            const double cs = cos(ang), sn = sin(ang);
            const double a = xh[i], b = xh[i + half];
            xh[i] = a * cs - b * sn;
            xh[i + half] = a * sn + b * cs;
        }
    }
    return 0;
}

/* Attention of one query per head over cached positions 0 .. n_ctx-1 (the
 * causal window of the newest token), grouped-query: head h reads KV head
 * h / (n_head / n_kv).
 *   s_j = (q_h . K[g][j]) / sqrt(hd),  p = softmax(s),  att[h] = sum_j p_j V[g][j].
 * The softmax is evaluated as exp(s_j - max s) / sum_k exp(s_k - max s).
 * K, V: f32 [n_kv][ctx_stride][hd]. */
int oracle_gqa_attend(const double *q, long n_head, long n_kv, long hd, const float *K, const float *V,
                      long ctx_stride, long n_ctx, double *att)
{
    if (!q || !K || !V || !att || n_head <= 0 || n_kv <= 0 || n_head % n_kv || hd <= 0 || n_ctx <= 0 ||
        n_ctx > ctx_stride)
        return -1;
    double *s = malloc(sizeof(double) * (size_t)n_ctx);
    if (!s) return -1;
    for (long h = 0; h < n_head; ++h) {
        const long g = h / (n_head / n_kv);
        const float *Kg = K + g * ctx_stride * hd, *Vg = V + g * ctx_stride * hd;
        double mx = -INFINITY;
        for (long j = 0; j < n_ctx; ++j) {
            double dot = 0.0;
            for (long d = 0; d < hd; ++d) dot += q[h * hd + d] * (double)Kg[j * hd + d];
            s[j] = dot / sqrt((double)hd);
            if (s[j] > mx) mx = s[j];
        }
        double den = 0.0;
        for (long j = 0; j < n_ctx; ++j) {
            s[j] = exp(s[j] - mx);
            den += s[j];
        }
        for (long d = 0; d < hd; ++d) {
            double acc = 0.0;
            for (long j = 0; j < n_ctx; ++j) acc += s[j] * (double)Vg[j * hd + d];
            att[h * hd + d] = acc / den;
        }
    }
    free(s);
    return 0;
}

/* y = W x for bf16 W and an f64 x. */
static void matvec_bf16_f64(const uint16_t *W, long rows, long cols, const double *x, double *y)
{
    for (long r = 0; r < rows; ++r) {
        double acc = 0.0;
        for (long j = 0; j < cols; ++j) acc += bf16_value(W[r * cols + j]) * x[j];
        y[r] = acc;
    }
}

/* The block for one token at position pos:
 *   q = Wq x, k = Wk x, v = Wv x                   (bf16 weights, f32 x)
 *   q, k: per-head RMS norm (eps 1e-6; gains q_norm, k_norm), then RoPE at pos
 *   K[g][pos] = f32(k_g), V[g][pos] = f32(v_g)      (the cache holds f32)
 *   att = GQA attention over positions 0 .. pos
 *   out = Wo att
 * Wq [n_head*hd][d_model], Wk and Wv [n_kv*hd][d_model], Wo [d_model][n_head*hd].
 * The caches are read at positions < pos and written at pos; nothing else in
 * them changes.  q_rot and att_out (may be NULL) receive the rotated queries
 * and the attention output, [n_head*hd] each. */
int oracle_attn_decode(const uint16_t *wq, const uint16_t *wk, const uint16_t *wv, const uint16_t *wo,
                       const float *q_norm, const float *k_norm, long d_model, long n_head, long n_kv,
                       long hd, const float *x, long pos, double rope_base, float *k_cache, float *v_cache,
                       long ctx_stride, double *out, double *q_rot, double *att_out)
{
    if (!wq || !wk || !wv || !wo || !q_norm || !k_norm || !x || !k_cache || !v_cache || !out ||
        d_model <= 0 || n_head <= 0 || n_kv <= 0 || n_head % n_kv || hd <= 0 || hd % 2 || pos < 0 ||
        pos >= ctx_stride)
        return -1;
    const long nq = n_head * hd, nk = n_kv * hd;
    double *q = malloc(sizeof(double) * (size_t)nq), *k = malloc(sizeof(double) * (size_t)nk);
    double *v = malloc(sizeof(double) * (size_t)nk), *qn = malloc(sizeof(double) * (size_t)nq);
    double *kn = malloc(sizeof(double) * (size_t)nk), *att = malloc(sizeof(double) * (size_t)nq);
    int rc = -1;
    if (!q || !k || !v || !qn || !kn || !att) goto done;
    if (oracle_matvec_bf16(wq, nq, d_model, x, q) || oracle_matvec_bf16(wk, nk, d_model, x, k) ||
        oracle_matvec_bf16(wv, nk, d_model, x, v))
        goto done;
    if (oracle_head_rmsnorm(q, n_head, hd, q_norm, 1e-6, qn) || oracle_head_rmsnorm(k, n_kv, hd, k_norm, 1e-6, kn))
        goto done;
    if (oracle_rope(qn, n_head, hd, pos, rope_base) || oracle_rope(kn, n_kv, hd, pos, rope_base)) goto done;
    for (long g = 0; g < n_kv; ++g)
        for (long d = 0; d < hd; ++d) {
            k_cache[(g * ctx_stride + pos) * hd + d] = (float)kn[g * hd + d];
            v_cache[(g * ctx_stride + pos) * hd + d] = (float)v[g * hd + d];
        }
    if (oracle_gqa_attend(qn, n_head, n_kv, hd, k_cache, v_cache, ctx_stride, pos + 1, att)) goto done;
    matvec_bf16_f64(wo, d_model, nq, att, out);
    if (q_rot) memcpy(q_rot, qn, sizeof(double) * (size_t)nq);
    if (att_out) memcpy(att_out, att, sizeof(double) * (size_t)nq);
    rc = 0;
done:
    free(q);
    free(k);
    free(v);
    free(qn);
    free(kn);
    free(att);
    return rc;
}
