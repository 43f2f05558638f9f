/*
 * oracle.h -- plain f64 CPU oracle for the group-quantised expert FFN, the
 * bf16 dense matvec and the decode attention block.
 *
 * TEST INFRASTRUCTURE ONLY.  This library exists to check the GPU library
 * against.  Only the test suite, the smoke check and the benchmark's CPU
 * baseline load it; the product path never does.  It shares no source with the
 * GPU library: it has its own unpacker, its own dequantiser and its own loops.
 *
 * Everything is computed from the definitions, slowly and in f64:
 *   - each weight is dequantised explicitly, w = (code - Z) / Z * s
 *     (Metal Compute Kernels, S-MoE docs, section "Fused FFN Kernels -- One
 *     Simdgroup Per Output Row": affine codes with Z = 7.5 at 4 bits and 1.5
 *     at 2 bits, one scale per column group);
 *   - each row dot product runs over the columns in ascending order with one
 *     f64 accumulator;
 *   - SiLU(t) = t / (1 + exp(-t)).
 *
 * Packed format (the pages leave the bit order open; this is the reading
 * adopted everywhere in this repository): a row of `cols` codes occupies
 * cols*bits/8 bytes; at 4 bits byte k holds code 2k in its low nibble and code
 * 2k+1 in its high nibble; at 2 bits byte k holds codes 4k..4k+3 starting at
 * the least significant bit pair.  Scales are f32, row-major [rows][cols/group],
 * scale g covering columns g*group .. g*group+group-1 of its row.
 *
 * Return value of every int function: 0 on success, -1 on an argument the
 * definitions do not cover (bits not 2 or 4, a group that does not divide the
 * row, a non-positive size, a NULL pointer).
 */
#ifndef SMOE_ORACLE_H
#define SMOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    const uint8_t *codes;   /* [rows][cols*bits/8] */
    const float *scales;    /* [rows][cols/group]  */
} oracle_qmat;

typedef struct {
    oracle_qmat gate;       /* [d_ff][d_model] */
    oracle_qmat up;         /* [d_ff][d_model] */
    oracle_qmat down;       /* [d_model][d_ff] */
} oracle_expert;

/* Routed experts, token t, for t in [0, T):
 *   out[t][:] = sum over slots s < top_k (ascending) of w[t][s] * FFN_{ids[t][s]}(x[t]),
 * ids and w [T][top_k]; a slot whose id is outside [0, n_experts) adds nothing. */
int oracle_routed_ffn(const oracle_expert *experts, int n_experts, int bits, int group, long d_model,
                      long d_ff, long T, int top_k, const int *ids, const float *w, const float *x,
                      double *out);

/* 2-byte scales: out[i] = the IEEE 754 binary16 value of h[i], widened to f32
 * (exact).  A matrix with 2-byte scales is the matrix whose f32 scales are
 * these values. */
int oracle_f16_widen(const uint16_t *h, long n, float *out);

/* Number of OpenMP threads the oracle's row loops use (1 without OpenMP). */
int oracle_threads(void);
/* Sets the threads of the row loops (results do not depend on it). */
void oracle_set_threads(int n);

/* One code per output byte: out[r*cols + j] = code of row r, column j. */
int oracle_unpack(const uint8_t *codes, int bits, long rows, long cols, uint8_t *out);

/* Explicit dequantisation: w[r*cols + j] = (code - Z) / Z * scale[r][j/group]. */
int oracle_dequant(const uint8_t *codes, const float *scales, int bits, int group,
                   long rows, long cols, double *w);

/* y[r] = sum_j w(r, j) * x[j], j ascending, f64 accumulator. */
int oracle_qmatvec(const uint8_t *codes, const float *scales, int bits, int group,
                   long rows, long cols, const double *x, double *y);

double oracle_silu(double t);

/* hidden[i] = SiLU(g_i) * u_i with g = G x, u = U x (one expert). */
int oracle_gate_up(const oracle_qmat *gate, const oracle_qmat *up, int bits, int group,
                   long d_ff, long d_model, const float *x, double *hidden);

/* out[j] = (D hidden)[j] (one expert). */
int oracle_down(const oracle_qmat *down, int bits, int group, long d_model, long d_ff,
                const double *hidden, double *out);

/* Token t, for t in [0, T):
 *   out[t][:] = sum_e route_w[t][e] * down_e( SiLU(gate_e x[t]) * (up_e x[t]) ),
 * experts in ascending order; route_w == NULL means every weight is 1. */
int oracle_expert_ffn(const oracle_expert *experts, int n_experts, const float *route_w,
                      int bits, int group, long d_model, long d_ff, long T,
                      const float *x, double *out);

/* y[r] = sum_j bf16_to_f32(W[r][j]) * x[j], j ascending, f64 accumulator.
 * W holds raw bf16 bit patterns. */
int oracle_matvec_bf16(const uint16_t *W, long rows, long cols, const float *x, double *y);

/* Decode attention (section "GPU-Resident Decode Attention").
 * Per-head RMS norm: y[h][d] = x[h][d] / sqrt(mean_d x[h][d]^2 + eps) * w[d]. */
int oracle_head_rmsnorm(const double *x, long n_heads, long hd, const float *w, double eps, double *y);

/* RoPE at position pos, in place: pair (x[i], x[i + hd/2]), i < hd/2, turns by
 * pos * base^(-2i/hd):  (a, b) -> (a cos - b sin, a sin + b cos). */
int oracle_rope(double *x, long n_heads, long hd, long pos, double base);

/* att[h] = sum_j softmax_j((q_h . K[g][j]) / sqrt(hd)) V[g][j] over j < n_ctx,
 * g = h / (n_head / n_kv); K, V f32 [n_kv][ctx_stride][hd]. */
int oracle_gqa_attend(const double *q, long n_head, long n_kv, long hd, const float *K, const float *V,
                      long ctx_stride, long n_ctx, double *att);

/* The decode attention block of one token at position pos: q/k/v projections
 * (bf16), per-head RMS norm (eps 1e-6, gains q_norm and k_norm) and RoPE of q
 * and k, K/V rows appended to the f32 caches at pos, GQA attention over
 * positions 0..pos, out = Wo att.  q_rot and att_out may be NULL. */
int oracle_attn_decode(const uint16_t *wq, const uint16_t *wk, const uint16_t *wv, const uint16_t *wo,
                       const float *q_norm, const float *k_norm, long d_model, long n_head, long n_kv,
                       long hd, const float *x, long pos, double rope_base, float *k_cache, float *v_cache,
                       long ctx_stride, double *out, double *q_rot, double *att_out);

#ifdef __cplusplus
}
#endif
#endif
