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
    unsigned long long *row_acc;  // [d_model] exact expert sums, zero on entry and exit (n_experts > 1)
    int d_model, d_ff, group, n_experts;
    int lpr_g, lpr_d;
    int dn_rows_per_wave;    // set by the down launcher
};

bool plan_decode(int mode, int bits, int d_model, int d_ff, int n_experts, DecodePlan *plan);
// `cus` is the device's compute-unit count; the persistent grids are sized from it.
hipError_t launch_gate_up(int bits, const DecodePlan &plan, const DecodeArgs &args, int cus, hipStream_t stream);
hipError_t launch_down(int bits, const DecodePlan &plan, const DecodeArgs &args, int cus, hipStream_t stream);

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

}  // namespace smoe
