/*
 * smoe.h -- C ABI of libsmoe.so: the group-quantised routed-expert FFN decode
 * path and its bf16 dense-matvec twin on one AMD Instinct MI355X (gfx950).
 *
 * The operations follow the Metal Compute Kernels page of the S-MoE docs:
 *
 *  - smoe_gate_up   hidden = SiLU(G x) * (U x), gate and up reading one shared
 *                   input vector ("Fused FFN Kernels -- One Simdgroup Per
 *                   Output Row").
 *  - smoe_down      out = D hidden (same section).
 *  - smoe_expert_ffn  the two passes for a group of routed experts in one
 *                   call, expert outputs combined with router weights; one
 *                   token or a batch of tokens ("Fused FFN Kernels" and
 *                   "Token-Batch Fused FFN"; all experts of a group go out in
 *                   one submission as in "Grouped Expert Dispatch").
 *  - matvec_bf16    y = W x with bf16 W and f32 x ("Coalesced Dense Matvec --
 *                   the Same Contract for bf16").
 *  - smoe_routed_ffn  the routed (top-k) token batch: each token through
 *                   its own experts only ("Token-Batch Fused FFN").
 *  - matvec_bf16_batch  several independent bf16 matvecs in one launch
 *                   ("Batched Scout Matvec").
 *  - smoe_attn_decode  one token's attention block: q/k/v projections, QK
 *                   RMS norm, RoPE, KV append, GQA attention, o_proj
 *                   ("GPU-Resident Decode Attention").
 *
 * Weight format (the "Layout assumptions the kernels rely on" contract):
 *   A quantised matrix of rows x cols is a smoe_qmat:
 *     codes  : rows * (cols*bits/8) bytes, row-major, row stride cols*bits/8.
 *              4-bit codes: byte k of a row holds column 2k in the low nibble
 *              and column 2k+1 in the high nibble.  2-bit codes: byte k holds
 *              columns 4k..4k+3 from the least significant bit pair up.
 *              Base address 16-byte aligned; the row stride is then a
 *              multiple of 16 because cols is a multiple of 32 (4-bit) or 64
 *              (2-bit).
 *     scales : rows * (cols/group) values, row-major; scale g of a row covers
 *              columns g*group .. g*group+group-1.  f32 (4-byte aligned) by
 *              default; IEEE binary16 (2-byte aligned) when the call's `bits`
 *              argument has SMOE_SCALE_F16 set.
 *   The weight at (r, j) is (code - Z) / Z * scale, Z = 7.5 at 4 bits and 1.5
 *   at 2 bits.  group must be a multiple of 32 (4-bit) or 64 (2-bit) and
 *   divide cols, so no 16-byte chunk of codes straddles two groups.
 *
 * Activations are f32 throughout (x, hidden, out, y, router weights).  The
 * vectors a kernel stages in 16-byte pieces (x of every call, hidden of
 * smoe_down) must be 16-byte aligned; outputs and router weights 4-byte.
 *
 * Numerics of the one-token (decode) kernels: each 16-byte chunk of the input
 * vector (32 columns at 4 bits, 64 at 2 bits) is carried as 22-bit fixed
 * point with one power-of-two exponent per chunk, so column j is off by at
 * most 2^-22 of its chunk's largest |x|; the code dot products are exact in
 * int32 and the per-chunk epilogue and row sums are f32.  There is no range
 * limit below f32's own: an input of any finite magnitude gives the result to
 * that precision at its own scale.  A non-finite element (NaN or an infinity)
 * makes every row that reads its chunk NaN, which is every output row.
 *
 * Memory and streams: every data pointer is a DEVICE pointer owned by the
 * caller; the library never allocates, frees or copies device memory inside a
 * call.  `stream` is a hipStream_t (NULL = the default stream).  Calls only
 * enqueue work and return; results are ready when the stream reaches them.
 * Scratch memory comes from the caller's workspace, sized by the matching
 * *_workspace() function.  Structures passed by host pointer (smoe_qmat,
 * smoe_expert) are read during the call and may be reused afterwards.
 * A call enqueues kernel launches only (no memset, copy or host callback), so
 * it can be captured into a HIP graph and replayed; a replay reads and writes
 * the addresses the call was captured with, and counters in the workspace are
 * cleared by the call's own kernels on every replay.  Calls on different
 * streams may run at the same time when none of them writes memory another
 * reads or writes (each with its own workspace and outputs).
 *
 * Errors: every call checks all of its arguments on the host before it
 * enqueues anything and returns a negative SMOE_ERR_* code when an argument
 * is outside the contract; in that case nothing was launched.  There is no
 * fallback kernel.  smoe_status_str() gives a message for each code.
 */
#ifndef SMOE_H
#define SMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    SMOE_OK = 0,
    SMOE_ERR_NULL = -1,      /* a required pointer is NULL */
    SMOE_ERR_BITS = -2,      /* bits is not 2 or 4 */
    SMOE_ERR_GROUP = -3,     /* group not a multiple of 32 (4-bit) / 64 (2-bit), or does not divide cols */
    SMOE_ERR_SHAPE = -4,     /* a size is <= 0, not a multiple of the chunk width, or above the kernel limits */
    SMOE_ERR_ALIGN = -5,     /* codes, W, or an f32 input vector read in 16-byte pieces (x, hidden,
                                the KV caches) not 16-byte aligned; other f32 data not 4-byte aligned;
                                a workspace not 256-byte aligned */
    SMOE_ERR_WORKSPACE = -6, /* workspace NULL or smaller than *_workspace() asks for */
    SMOE_ERR_ALIAS = -7,     /* an output range overlaps an input or the workspace */
    SMOE_ERR_DEVICE = -8,    /* current device is not gfx950, or a device query failed */
    SMOE_ERR_LAUNCH = -9,    /* the HIP runtime refused a launch */
};

/* Flag ORed into the `bits` argument of smoe_gate_up, smoe_down and
 * smoe_expert_ffn when every matrix of the call has 2-byte IEEE binary16
 * scales instead of f32 ones.  The scale is widened exactly to f32 and used as
 * an f32 scale would be, so f16 scales give the same results as f32 scales
 * holding the same values.  This 2-byte layout is the reading of the scale
 * bytes that the "Fused FFN Kernels" section's bandwidth figures imply; it
 * cuts the streamed bytes by 5.6% at 4 bits and 10% at 2 bits (group 64). */
#define SMOE_SCALE_F16 0x100
/* Largest n_experts accepted by smoe_expert_ffn in one call. */
#define SMOE_MAX_EXPERTS 16
/* Largest cols of a quantised matrix (d_model for gate/up, d_ff for down). */
#define SMOE_MAX_QCOLS 8192
/* Largest cols of a bf16 matrix. */
#define SMOE_MAX_BF16_COLS 16384
/* Jobs per matvec_bf16_batch call. */
#define SMOE_MAX_BF16_JOBS 16
/* Largest token count T of smoe_expert_ffn. */
#define SMOE_MAX_TOKENS 65536

typedef struct smoe_qmat {
    const uint8_t *codes;
    const void *scales;   /* f32, or f16 with SMOE_SCALE_F16 (see the weight format) */
} smoe_qmat;

typedef struct smoe_expert {
    smoe_qmat gate;   /* [d_ff x d_model] */
    smoe_qmat up;     /* [d_ff x d_model] */
    smoe_qmat down;   /* [d_model x d_ff] */
} smoe_expert;

/*
 * hidden[i] = SiLU((G x)[i]) * (U x)[i],  i < d_ff, for one expert.
 *   gate, up : [d_ff x d_model] quantised matrices (host structs, device data)
 *   x        : f32 [d_model], 16-byte aligned
 *   hidden   : f32 [d_ff], 4-byte aligned, must not overlap x or the weights
 * SiLU(t) = t / (1 + exp(-t)).
 */
int smoe_gate_up(const smoe_qmat *gate, const smoe_qmat *up, int bits, int group,
                 int d_ff, int d_model, const float *x, float *hidden, void *stream);

/*
 * out[j] = (D hidden)[j],  j < d_model, for one expert.
 *   down   : [d_model x d_ff] quantised matrix
 *   hidden : f32 [d_ff], 16-byte aligned
 *   out    : f32 [d_model], 4-byte aligned, must not overlap hidden or the weights
 */
int smoe_down(const smoe_qmat *down, int bits, int group, int d_model, int d_ff,
              const float *hidden, float *out, void *stream);

/*
 * Routed experts over T tokens:
 *   out[t][:] = sum_e route_w[t][e] * down_e( SiLU(gate_e x[t]) * (up_e x[t]) )
 *   experts   : host array of n_experts expert descriptors (1..SMOE_MAX_EXPERTS)
 *   route_w   : f32 [T][n_experts] device array (4-byte aligned), or NULL for
 *               weight 1 everywhere
 *   x         : f32 [T][d_model], 16-byte aligned
 *   out       : f32 [T][d_model], 4-byte aligned, must not overlap x, route_w,
 *               workspace or weights
 *   workspace : device scratch of at least smoe_expert_ffn_workspace(...) bytes,
 *               256-byte aligned.  Every call rewrites what it reads of it;
 *               nothing in it needs to be zero.  Calls that share a workspace
 *               must be ordered (one stream), or they race.
 * T == 1 runs the decode kernels: a gate_up launch that writes every expert's
 * hidden row to the workspace, and a down launch whose blocks each own a range
 * of output rows for all experts and add the experts' f32 rows in ascending
 * expert order in f64, each times its router weight, rounding once to f32
 * (deterministic, no atomics, no range limit).
 * 2 <= T <= SMOE_MAX_TOKENS runs the token-batch kernels on the matrix cores,
 * in which every expert processes every token: for T > 16 an activation pass,
 * a gate_up pass and a down pass that sums the experts in a fixed order
 * (deterministic, no atomics in the sums), for T <= 16 a gate_up pass that
 * stages the activations itself and a down pass.  With few tokens the K
 * dimension of a pass is split over blocks whose partial sums are added in a
 * fixed split order, by a finishing pass or by the last block of the split
 * to finish (one counter per tile in the workspace, zeroed by the call
 * itself).
 * They need group = 32 or 64 at 4 bits and 64 at 2 bits, else SMOE_ERR_GROUP
 * (wider groups are served at T = 1 only).  Activations are carried to the matrix cores
 * as two f16 halves scaled by a power of two per group, about 22 significant
 * bits; non-finite inputs give non-finite outputs.
 * The workspace size depends on (n_experts, d_model, d_ff, T) only; for T > 1
 * nothing in it needs to be zero and every call rewrites it.
 */
size_t smoe_expert_ffn_workspace(int n_experts, int d_model, int d_ff, int T);
int smoe_expert_ffn(const smoe_expert *experts, int n_experts, const float *route_w,
                    int bits, int group, int d_model, int d_ff, int T,
                    const float *x, float *out, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Bytes of the static device scratch array behind smoe_expert_ffn_noalloc
 * (one array per GPU, held until the process ends). */
#define SMOE_NOALLOC_SCRATCH_BYTES (1 << 20)

/*
 * smoe_expert_ffn without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, results and errors as
 * smoe_expert_ffn (the same kernels run), except:
 *   - the scratch memory is a static device array of
 *     SMOE_NOALLOC_SCRATCH_BYTES bytes, one per GPU, in place of the caller's
 *     workspace; a call whose smoe_expert_ffn_workspace(...) size exceeds it
 *     returns SMOE_ERR_WORKSPACE with nothing launched.  Every one-token
 *     (T == 1) call up to the shape limits fits; small token batches fit.
 *   - nothing is allocated, freed or cleared by the host (no hipMalloc,
 *     hipFree, hipMemset or allocating library call); the kernels rewrite
 *     every part of the array they read, so its leftover contents from an
 *     earlier call never matter.
 *   - all calls on one GPU share that GPU's array: calls that may overlap on
 *     one GPU (different streams without ordering, several host threads) race
 *     and give undefined results.  Order them on one stream.
 * The array's device address is looked up once per device, on the first call
 * of any entry point with that device current; SMOE_ERR_DEVICE if that failed.
 */
int smoe_expert_ffn_noalloc(const smoe_expert *experts, int n_experts, const float *route_w,
                            int bits, int group, int d_model, int d_ff, int T,
                            const float *x, float *out, void *stream);

/*
 * y[r] = sum_j float(W[r][j]) * x[j],  r < rows.
 *   W : bf16 bit patterns [rows x cols], 16-byte aligned, cols % 8 == 0
 *   x : f32 [cols]
 *   y : f32 [rows], must not overlap W or x
 *   workspace : may be NULL when matvec_bf16_workspace() returns 0
 */
size_t matvec_bf16_workspace(int rows, int cols);
int matvec_bf16(const uint16_t *W, int rows, int cols, const float *x, float *y,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Routed experts over T tokens ("Token-Batch Fused FFN": per expert, the
 * tokens that chose it run through it together; the experts' outputs of a
 * token are combined with its router weights):
 *   out[t][:] = sum over slots j < top_k, ascending, of
 *               expert_w[t][j] * down_e( SiLU(gate_e x[t]) * (up_e x[t]) ),
 *               e = expert_ids[t][j]
 *   expert_ids : i32 [T][top_k] device array; the ids of one token must be
 *                distinct (as a top-k selection gives: an expert then takes at
 *                most T slots); a slot whose id is outside [0, n_experts) adds
 *                nothing
 *   expert_w   : f32 [T][top_k] device array
 *   x, out     : f32 [T][d_model]; out must not overlap any input or the workspace
 *   workspace  : smoe_routed_ffn_workspace(...) bytes, 256-byte aligned; every
 *                call rewrites it, nothing in it needs to be zero
 * 1 <= T <= SMOE_MAX_TOKENS, 1 <= top_k <= SMOE_MAX_EXPERTS.  Only each slot's
 * expert processes the token: a device pass lists every expert's slots in
 * ascending order, the gate_up and down passes run per expert over those
 * lists on the matrix cores (for T <= 16 and d_ff <= 1536 the streaming
 * kernels of the token batch, an expert's slots being one tile), and a last
 * pass adds each token's slots in slot order (deterministic, no atomics).  Needs group 32 (4-bit) or 64, else
 * SMOE_ERR_GROUP.  `bits` may carry SMOE_SCALE_F16.
 */
size_t smoe_routed_ffn_workspace(int n_experts, int d_model, int d_ff, int T, int top_k);
int smoe_routed_ffn(const smoe_expert *experts, int n_experts, int bits, int group,
                    int d_model, int d_ff, int T, int top_k, const int *expert_ids,
                    const float *expert_w, const float *x, float *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/*
 * Several independent bf16 matvecs in one launch ("Batched Scout Matvec":
 * the matvecs of one layer, such as a projection pair, go out as one
 * submission instead of one each):
 *   y_j = W_j x_j   for j = 0 .. n_jobs-1
 *   jobs   : host array of n_jobs descriptors (1..SMOE_MAX_BF16_JOBS), read
 *            during the call; each job has the contract of matvec_bf16
 *            (W_j bf16 [rows_j x cols_j], 16-byte aligned, cols_j % 8 == 0,
 *            cols_j <= SMOE_MAX_BF16_COLS; x_j f32 [cols_j], 16-byte aligned;
 *            y_j f32 [rows_j], 4-byte aligned).  Jobs may share W or x.
 *   y_j must not overlap any job's W, x or (another job's) y.
 * No workspace.  Each y_j is computed as matvec_bf16 would (within the same
 * tolerance; the summation order may differ).
 */
typedef struct {
    const uint16_t *W;
    const float *x;
    float *y;
    int rows, cols;
} smoe_bf16_job;
int matvec_bf16_batch(const smoe_bf16_job *jobs, int n_jobs, void *stream);

/* Query heads per KV head in smoe_attn_decode. */
#define SMOE_MAX_ATTN_GROUP 16

/*
 * The decode attention block of one token ("GPU-Resident Decode Attention":
 * the layer's attention as one submission with no host round trip):
 *   q = Wq x, k = Wk x, v = Wv x                  (bf16 weights, f32 x)
 *   q and k, per head: RMS norm  y = x / sqrt(mean(x^2) + 1e-6) * gain,
 *     then RoPE at position pos: for i < head_dim/2 the pair
 *     (y[i], y[i + head_dim/2]) turns by pos * rope_base^(-2i/head_dim)
 *   k_cache[g][pos][:] = k_g,  v_cache[g][pos][:] = v_g   (f32)
 *   att[h] = sum_{j <= pos} softmax_j(q_h . K[g][j] / sqrt(head_dim)) V[g][j],
 *     g = h / (n_head / n_kv)
 *   out = Wo att
 * Arguments:
 *   w        : host struct of device pointers: wq bf16 [n_head*head_dim][d_model],
 *              wk and wv bf16 [n_kv*head_dim][d_model], wo bf16
 *              [d_model][n_head*head_dim] (16-byte aligned), q_norm and k_norm
 *              f32 [head_dim]
 *   x        : f32 [d_model], 16-byte aligned
 *   k_cache, v_cache : f32 [n_kv][max_ctx][head_dim], 16-byte aligned, caller
 *              owned; rows 0..pos-1 are read, row pos is written, nothing else
 *              changes
 *   out      : f32 [d_model]; must not overlap any other argument
 *   workspace: smoe_attn_decode_workspace(...) bytes, 256-byte aligned, device
 *              memory the call may overwrite (nothing in it needs to be zero)
 * Limits: d_model % 8 == 0, d_model and n_head*head_dim <= SMOE_MAX_BF16_COLS,
 * n_head % n_kv == 0 with n_head / n_kv <= SMOE_MAX_ATTN_GROUP, head_dim 64 or
 * 128, 0 <= pos < max_ctx, rope_base > 0; else SMOE_ERR_SHAPE.  Four launches
 * on `stream`: the three projections in one; the norm, rotation and append
 * with the attention over 32-position chunks (one block serves a KV head's
 * query heads); the chunk merge in a fixed order (deterministic); o_proj.
 * Rotation angles are formed in f64; everything else is f32.
 */
typedef struct {
    const uint16_t *wq, *wk, *wv, *wo;
    const float *q_norm, *k_norm;
} smoe_attn_weights;
size_t smoe_attn_decode_workspace(int d_model, int n_head, int n_kv, int head_dim, int max_ctx);
int smoe_attn_decode(const smoe_attn_weights *w, int d_model, int n_head, int n_kv, int head_dim,
                     const float *x, int pos, double rope_base, float *k_cache, float *v_cache, int max_ctx,
                     float *out, void *workspace, size_t workspace_bytes, void *stream);

/* Message for a status code (static string). */
const char *smoe_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif
