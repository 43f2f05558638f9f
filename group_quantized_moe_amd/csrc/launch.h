// Host-side interface between the C ABI (smoe_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace smoe {

// Lane mapping of one matvec launch.  A block has `nw` waves; the chunks
// (16-byte pieces of a packed row) of one row are split into nw contiguous
// slices, one per wave; within a wave, `lpr` lanes share a row and each lane
// owns `nch` chunks of the slice, so 64/lpr rows are in flight per wave step;
// a tile is `iter` such steps, (64/lpr)*iter rows.
struct MapConfig {
    int nw, lpr, nch, iter;
    int rows_per_block() const { return (64 / lpr) * iter; }
};

struct GateUpArgs {
    QPtr gate[kMaxExperts];
    QPtr up[kMaxExperts];
    const float *x;        // [d_model]
    float *hidden;         // [n_experts][d_ff]
    int *counters;         // zeroed for a following combined down launch (may be null)
    int n_counters;
    int d_model, d_ff, group, n_experts;
    int blocks_per_expert; // row tiles per expert
};

struct DownArgs {
    QPtr down[kMaxExperts];
    const float *hidden;   // [n_experts][d_ff]
    const float *route_w;  // [n_experts] or null (weight 1)
    float *out;            // [d_model]
    float *partial;        // [n_experts][d_model], when n_experts > 1
    int *counters;         // [row_blocks], zero on entry, when n_experts > 1
    int d_model, d_ff, group, n_experts;
    int row_blocks;
};

struct Bf16Args {
    const uint16_t *W;     // [rows][cols]
    const float *x;        // [cols]
    float *y;              // [rows]
    int rows, cols;
};

// Picks a lane mapping for rows of `chunks` 16-byte chunks; returns false when
// no supported mapping covers the row.
bool choose_qmap(int bits, int chunks, int rows, int n_experts, MapConfig *cfg);
bool choose_bf16map(int chunks, int rows, MapConfig *cfg);

// `cus` is the device's compute-unit count; the decode kernels size their
// persistent grids from it.
hipError_t launch_gate_up(int bits, const MapConfig &cfg, const GateUpArgs &a, int cus, hipStream_t stream);
hipError_t launch_down(int bits, const MapConfig &cfg, const DownArgs &a, int cus, hipStream_t stream);
hipError_t launch_matvec_bf16(const MapConfig &cfg, const Bf16Args &a, hipStream_t stream);

}  // namespace smoe
