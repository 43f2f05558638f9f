// Host-side interface between the C ABI (smoe_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace smoe {

// ---------------------------------------------------------------------------
// Decode (one token) launches of the quantised expert FFN
// ---------------------------------------------------------------------------

// Which passes a plan covers: gate_up only, down only, or both (the expert FFN).
enum DecodeMode : int { kGateUpOnly = 0, kDownOnly = 1, kBoth = 2 };

// Lane mapping of the decode launches.  A block has `nw` waves; every wave owns
// whole rows: `lpr` lanes share a row and each owns `nch` of its 16-byte
// chunks (lane lr owns chunks lr, lr + lpr, ...), so a wave covers 64/lpr
// rows per step.  gate_up (cols = d_model) and down (cols = d_ff) each have
// their own lpr / nch.
struct DecodePlan {
    int mode, nw;
    int lpr_g, nch_g;
    int lpr_d, nch_d;
    int d_model, d_ff;
};

struct DecodeArgs {
    QPtr gate[kMaxExperts];
    QPtr up[kMaxExperts];
    QPtr down[kMaxExperts];
    const float *x;          // [d_model]
    float *hidden;           // [n_experts][d_ff]
    const float *route_w;    // [n_experts] or null (weight 1)
    float *out;              // [d_model]
    int d_model, d_ff, group, n_experts;
    int scale_bytes;         // 4: f32 scales, 2: IEEE binary16 scales
    int dn_steps_per_block;  // set by the down launcher: row steps each down block owns
};

bool plan_decode(int mode, int bits, int d_model, int d_ff, int n_experts, DecodePlan *plan);
// `cus` is the device's compute-unit count; the persistent grids are sized from it.
hipError_t launch_gate_up(int bits, const DecodePlan &plan, const DecodeArgs &args, int cus, hipStream_t stream);
hipError_t launch_down(int bits, const DecodePlan &plan, const DecodeArgs &args, int cus, hipStream_t stream);

// ---------------------------------------------------------------------------
// Token-batch (T > 1) launches of the quantised expert FFN (matrix cores)
// ---------------------------------------------------------------------------

// Activations in the workspace are f16 hi/lo halves in sigma order (element
// 8b + i of a row holds column 8b + sigma(i), sigma = 0,4,1,5,2,6,3,7), scaled
// by a power of two: one exponent per token for X, one per (token, group of
// d_ff columns) for the hidden rows, kept as a factor that also holds the
// router weight.
struct TbArgs {
    QPtr gate[kMaxExperts];
    QPtr up[kMaxExperts];
    QPtr down[kMaxExperts];
    const float *x;          // [T][d_model]
    const float *route_w;    // [T][n_experts] or null (weight 1)
    float *out;              // [T][d_model]
    _Float16 *xh, *xl;       // [T][d_model]
    int *xe;                 // [T]
    _Float16 *hh, *hl;       // [n_experts][T][d_ff]
    float *hid;              // streaming path: f32 hidden rows [n_experts][T][d_ff] (over hh and hl)
    float *hf;               // [n_experts][d_ff / group][t_pad]: r[t][e] * 2^e(t, group)
    float *part_gu, *part_dn; // per-tile partial sums of the K splits
    unsigned *cnt_gu, *cnt_dn; // per tile, the K splits done (zeroed by the call's first kernel)
    int n_cnt;               // entries of cnt_gu and cnt_dn together (contiguous)
    // Routed mode (top_k > 0): slot s = t*top_k + j of token
    // t goes to expert ids[s] with weight slot_w[s].  list[e*T + p], p <
    // cnt[e], are expert e's slots in ascending order; the hidden rows,
    // factors and partial sums of expert e are indexed by p instead of the
    // token.  down writes each slot's weighted output row to ys [T*top_k]
    // [d_model] and slot_ok[s] says whether slot s was processed.
    const int *ids;
    const float *slot_w;
    int top_k;
    int *list, *cnt, *slot_ok;
    float *ys;
    int T, t_pad, d_model, d_ff, group, n_experts;
    int scale_bytes;         // 4: f32 scales, 2: IEEE binary16 scales
    int ks_gu, ks_dn;        // K splits over blocks of gate_up and down
};

// Tiling of the token-batch launches: the streaming kernels (T <= 16) or the
// tiled ones with 16*ntt tokens per block, gate_up steps of mg quantisation
// groups and K splits; block counts and dynamic LDS bytes of gate_up and down.
struct TbPlan {
    int stream;
    int mg;
    int ntt;
    int ks_gu;
    long gu_blocks;
    size_t gu_lds;
    int ks_dn;
    long dn_blocks;
    size_t dn_lds;
};

// Token rows of the hidden-row factors are padded to a multiple of this.
constexpr int kTokenPad = 64;

// False if the shape is outside what the token-batch kernels cover (group
// must be 32 or 64 columns at 4 bits, 64 at 2 bits).
bool plan_batch(int bits, int group, int d_model, int d_ff, int n_experts, int T, TbPlan *plan);
// Tiling of the token-batch kernels that depends on the shape only (not
// the group): tokens per tile / 16, tile counts, the largest K splits and the
// partial-sum floats they need in the workspace.
struct BatchSplits {
    int ntt;
    long gu_tiles, dn_tiles;
    int ks_gu, ks_dn;
    size_t gu_part_floats, dn_part_floats;
};
BatchSplits batch_splits(int n_experts, int d_model, int d_ff, int T);
// Routed mode: tiling from the average slots per expert, T * top_k / n_experts.
bool plan_routed(int bits, int group, int d_model, int d_ff, int n_experts, int T, int top_k, TbPlan *plan);
BatchSplits routed_splits(int n_experts, int d_model, int d_ff, int T, int top_k);
hipError_t launch_routed(int bits, const TbPlan &plan, const TbArgs &args, hipStream_t stream);
hipError_t launch_batch(int bits, const TbPlan &plan, const TbArgs &args, hipStream_t stream);

// ---------------------------------------------------------------------------
// Dense bf16 matvec
// ---------------------------------------------------------------------------

// Lane mapping of a bf16 matvec launch: nw waves split a row's chunks into
// slices, lpr lanes share a row, each lane owns nch chunks; a block covers
// (64/lpr)*iter rows.
struct MapConfig {
    int nw, lpr, nch, iter;
    int rows_per_block() const { return (64 / lpr) * iter; }
};

struct Bf16Args {
    const uint16_t *W;     // [rows][cols]
    const float *x;        // [cols]
    float *y;              // [rows]
    int rows, cols;
};

bool choose_bf16map(int chunks, int rows, MapConfig *cfg);
hipError_t launch_matvec_bf16(const MapConfig &cfg, const Bf16Args &a, hipStream_t stream);

// Batched bf16 matvec: up to kMaxBf16Jobs independent jobs in one launch;
// blk_start (filled by the launcher) is the first block of each job.
constexpr int kMaxBf16Jobs = 16;
struct Bf16Job {
    const uint16_t *W;
    const float *x;
    float *y;
    int rows, cols;
};
struct Bf16BatchArgs {
    Bf16Job job[kMaxBf16Jobs];
    int blk_start[kMaxBf16Jobs + 1];
    int n;
};
hipError_t launch_matvec_bf16_batch(const MapConfig &cfg, const Bf16BatchArgs &a, hipStream_t stream);

// Decode attention core (the part between the projections): per-head norm
// and rotation of q and k with the cache append, chunked GQA attention, and
// the chunk merge.  The projections use the bf16 matvec launches.
constexpr int kMaxAttnGroup = 16;   // query heads per KV head
struct AttnArgs {
    const float *q, *k, *v;         // projections: [n_head*hd], [n_kv*hd], [n_kv*hd]
    const float *q_norm, *k_norm;   // RMS norm gains [hd]
    float *k_cache, *v_cache;       // [n_kv][max_ctx][hd]
    float *part_o, *part_ml;        // [n_kv][n_chunks][G][hd], [n_kv][n_chunks][G][2]
    float *att;                     // attention output [n_head*hd]
    double rope_base;
    int n_head, n_kv, head_dim, max_ctx, pos, n_chunks;
};
int attn_chunks(int max_ctx);
hipError_t launch_attn_core(const AttnArgs &a, hipStream_t stream);

}  // namespace smoe
