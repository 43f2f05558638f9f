// C ABI of libsmoe.so: host-side argument checks, lane-mapping choice and
// kernel launches.  Every check runs before any HIP call, so an out-of-contract
// argument returns an error with nothing enqueued (and needs no GPU).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "../../include/smoe.h"
#include "launch.h"

static_assert(SMOE_MAX_BF16_JOBS == smoe::kMaxBf16Jobs, "job limit of the header and the kernels");

using smoe::DecodePlan;
using smoe::MapConfig;

namespace {

constexpr int kMaxDevices = 64;

// The scratch memory of smoe_expert_ffn_noalloc: one array per GPU, alive
// until the process ends.  In host code this name is a host-side stand-in,
// not a device address: the device address comes from hipGetSymbolAddress,
// once per device, and only that address is ever handed to a kernel.
static __device__ __align__(256) unsigned char scratch[SMOE_NOALLOC_SCRATCH_BYTES];

// Device properties, queried once per device with that device current (limits
// come from the device, never from constants), and the device address of the
// scratch array on that device (null if the lookup failed).
struct DeviceInfo {
    bool ok;
    int cus;
    void *scratch;
};

DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

int check_device(DeviceInfo *out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SMOE_ERR_DEVICE;
    std::call_once(g_dev_once[dev], [dev] {
        hipDeviceProp_t p;
        DeviceInfo d{false, 0, nullptr};
        if (hipGetDeviceProperties(&p, dev) == hipSuccess) {
            d.ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
            d.cus = p.multiProcessorCount;
        }
        if (d.ok) {
            void *ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess && ptr) d.scratch = ptr;
            else (void)hipGetLastError();   // the failure is reported by the call that needs the array
        }
        g_dev[dev] = d;
    });
    if (!g_dev[dev].ok) return SMOE_ERR_DEVICE;
    if (out) *out = g_dev[dev];
    return SMOE_OK;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) overlap.
bool overlap(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || !na || !nb) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Weight format: the code width and the scale size, from the `bits` argument
// (2 or 4, optionally with SMOE_SCALE_F16 set).
struct Fmt {
    int bits;   // 2 or 4
    int sb;     // bytes per scale: 4 (f32) or 2 (f16)
};

int check_format(int fmt, int group, Fmt *f)
{
    f->bits = fmt & ~SMOE_SCALE_F16;
    f->sb = (fmt & SMOE_SCALE_F16) ? 2 : 4;
    if (f->bits != 4 && f->bits != 2) return SMOE_ERR_BITS;
    const int unit = 128 / f->bits;  // codes in a 16-byte chunk
    if (group <= 0 || group % unit) return SMOE_ERR_GROUP;
    return SMOE_OK;
}

// rows x cols quantised matrix: sizes, group divisibility, pointers, alignment.
int check_qmat(const smoe_qmat *m, const Fmt &f, int group, long rows, long cols)
{
    if (!m || !m->codes || !m->scales) return SMOE_ERR_NULL;
    if (rows <= 0 || cols <= 0 || cols % (128 / f.bits) || cols > SMOE_MAX_QCOLS) return SMOE_ERR_SHAPE;
    if (cols % group) return SMOE_ERR_GROUP;
    if (!aligned(m->codes, 16) || !aligned(m->scales, (uintptr_t)f.sb)) return SMOE_ERR_ALIGN;
    return SMOE_OK;
}

size_t qmat_code_bytes(int bits, long rows, long cols) { return (size_t)rows * cols * bits / 8; }
size_t qmat_scale_bytes(int sb, int group, long rows, long cols) { return (size_t)rows * (cols / group) * sb; }

// out overlaps either array of a quantised matrix.
bool overlaps_qmat(const void *out, size_t nout, const smoe_qmat *m, const Fmt &f, int group, long rows,
                   long cols)
{
    return overlap(out, nout, m->codes, qmat_code_bytes(f.bits, rows, cols)) ||
           overlap(out, nout, m->scales, qmat_scale_bytes(f.sb, group, rows, cols));
}

int launch_status(hipError_t e) { return e == hipSuccess ? SMOE_OK : SMOE_ERR_LAUNCH; }

// Workspace of the decode path (T == 1): the hidden rows f32 [n_experts][d_ff],
// written by gate_up and read by down; nothing in it needs to be zero.
size_t decode_workspace(int n_experts, int d_ff) { return align256((size_t)n_experts * d_ff * 4); }

// Workspace layout of the token-batch path (T > 1), every piece 256-byte aligned:
//   xh, xl  f16 [T][d_model]                 hi/lo halves of the scaled activations
//   xe      i32 [T]                          their per-token exponents
//   hh, hl  f16 [n_experts][T][d_ff]         hi/lo halves of the scaled hidden rows (T <= 16: the
//                                            two together hold the f32 hidden rows [n_experts][T][d_ff])
//   hf      f32 [n_experts][d_ff/group][Tp]  per (expert, group, token) factors, Tp = T rounded up to 64
//   pg, pd  f32                              partial sums of the gate_up / down K splits, per tile
//                                            (T <= 16: of the down pass's chunks, per row group)
//   cnt     u32 [gate_up tiles + down tiles] K splits (chunks) of each tile (row group) done
// Everything is rewritten by each call before it is read (the counters are
// zeroed by the call's first kernel).
struct BatchWorkspace {
    size_t xh, xl, xe, hh, hl, hf, pg, pd, cnt, total;
    int n_cnt, n_cnt_gu;
};

int token_pad(int T) { return (T + smoe::kTokenPad - 1) / smoe::kTokenPad * smoe::kTokenPad; }

BatchWorkspace batch_workspace(int n_experts, int d_model, int d_ff, int T, int group)
{
    BatchWorkspace w;
    const size_t nx = (size_t)T * d_model, nh = (size_t)n_experts * T * d_ff;
    const smoe::BatchSplits bs = smoe::batch_splits(n_experts, d_model, d_ff, T);
    w.xh = 0;
    w.xl = w.xh + align256(nx * 2);
    w.xe = w.xl + align256(nx * 2);
    w.hh = w.xe + align256((size_t)T * 4);
    w.hl = w.hh + align256(nh * 2);
    w.hf = w.hl + align256(nh * 2);
    w.pg = w.hf + align256((size_t)n_experts * (d_ff / group) * token_pad(T) * 4);
    w.pd = w.pg + align256(bs.gu_part_floats * 4);
    w.cnt = w.pd + align256(bs.dn_part_floats * 4);
    w.n_cnt_gu = (int)bs.gu_tiles;
    w.n_cnt = (int)(bs.gu_tiles + bs.dn_tiles);
    w.total = w.cnt + align256((size_t)w.n_cnt * 4);
    return w;
}

// Workspace layout of the routed path, every piece 256-byte aligned:
//   xh, xl, xe                     as the token batch, [T] tokens
//   hh, hl  f16 [n_experts][T][d_ff] hidden rows by position in the expert's slot list (T <= 16:
//                                    the two together hold them as f32 [n_experts][T][d_ff])
//   hf      f32 [n_experts][d_ff/32][Tp] their factors (slot weight * 2^e; T <= 16: the slot
//                                    weights by position, [n_experts][T])
//   pg      f32                      partial sums of the gate_up K splits
//   list    i32 [n_experts][T]       each expert's slots, ascending; cnt i32 [n_experts]
//   ok      i32 [T*top_k]            slot processed
//   ys      f32 [T*top_k][d_model]   weighted output row of each slot
//   tcnt    u32 [gate_up tiles]      K splits of each gate_up tile done
// Everything is rewritten by each call before it is read (the counters are
// zeroed by the call's activation pass).
struct RoutedWorkspace {
    size_t xh, xl, xe, hh, hl, hf, pg, list, cnt, ok, ys, tcnt, total;
    int n_tcnt;
};

RoutedWorkspace routed_workspace(int n_experts, int d_model, int d_ff, int T, int top_k)
{
    RoutedWorkspace w;
    const size_t nx = (size_t)T * d_model, nh = (size_t)n_experts * T * d_ff, ns = (size_t)T * top_k;
    const smoe::BatchSplits bs = smoe::routed_splits(n_experts, d_model, d_ff, T, top_k);
    w.xh = 0;
    w.xl = w.xh + align256(nx * 2);
    w.xe = w.xl + align256(nx * 2);
    w.hh = w.xe + align256((size_t)T * 4);
    w.hl = w.hh + align256(nh * 2);
    w.hf = w.hl + align256(nh * 2);
    w.pg = w.hf + align256((size_t)n_experts * (d_ff / 32) * token_pad(T) * 4);
    w.list = w.pg + align256(bs.gu_part_floats * 4);
    w.cnt = w.list + align256((size_t)n_experts * T * 4);
    w.ok = w.cnt + align256((size_t)n_experts * 4);
    w.ys = w.ok + align256(ns * 4);
    w.tcnt = w.ys + align256(ns * d_model * 4);
    w.n_tcnt = (int)bs.gu_tiles;
    w.total = w.tcnt + align256((size_t)w.n_tcnt * 4);
    return w;
}

// The smallest group the token-batch layout can need (32 columns) gives the
// largest exponent arrays; the workspace size does not depend on the group.
constexpr int kMinBatchGroup = 32;

template <class Args>
void fill_experts(Args &a, const smoe_expert *experts, int n)
{
    for (int e = 0; e < n; ++e) {
        a.gate[e] = {experts[e].gate.codes, experts[e].gate.scales};
        a.up[e] = {experts[e].up.codes, experts[e].up.scales};
        a.down[e] = {experts[e].down.codes, experts[e].down.scales};
    }
}


// Workspace layout of the attention block, every piece 256-byte aligned (f32):
//   q [n_head*hd], k [n_kv*hd], v [n_kv*hd], att [n_head*hd],
//   part_o [n_kv][n_chunks][G][hd], part_ml [n_kv][n_chunks][G][2],
//   n_chunks = max_ctx / 32 rounded up.  Everything is rewritten before it is read.
struct AttnWorkspace {
    size_t q, k, v, att, part_o, part_ml, total;
};

AttnWorkspace attn_workspace(int n_head, int n_kv, int head_dim, int max_ctx)
{
    AttnWorkspace w;
    const size_t nq = (size_t)n_head * head_dim, nk = (size_t)n_kv * head_dim;
    const size_t nc = (size_t)smoe::attn_chunks(max_ctx);
    w.q = 0;
    w.k = w.q + align256(nq * 4);
    w.v = w.k + align256(nk * 4);
    w.att = w.v + align256(nk * 4);
    w.part_o = w.att + align256(nq * 4);
    w.part_ml = w.part_o + align256(nc * nq * 4);
    w.total = w.part_ml + align256(nc * (size_t)n_head * 2 * 4);
    return w;
}

bool attn_shape_ok(int d_model, int n_head, int n_kv, int head_dim, int max_ctx)
{
    if (d_model <= 0 || d_model % 8 || d_model > SMOE_MAX_BF16_COLS) return false;
    if (n_head <= 0 || n_kv <= 0 || n_head % n_kv || n_head / n_kv > SMOE_MAX_ATTN_GROUP) return false;
    if (head_dim != 64 && head_dim != 128) return false;
    if ((long)n_head * head_dim > SMOE_MAX_BF16_COLS || max_ctx <= 0) return false;
    return (long)n_kv * max_ctx * head_dim <= INT_MAX;
}

}  // namespace

extern "C" {

const char *smoe_status_str(int status)
{
    switch (status) {
    case SMOE_OK: return "ok";
    case SMOE_ERR_NULL: return "a required pointer is NULL";
    case SMOE_ERR_BITS: return "bits must be 2 or 4 (optionally with SMOE_SCALE_F16)";
    case SMOE_ERR_GROUP: return "group must be a multiple of 32 (4-bit) or 64 (2-bit) and divide cols";
    case SMOE_ERR_SHAPE: return "a size is out of range or not a multiple of the 16-byte chunk width";
    case SMOE_ERR_ALIGN: return "codes/W must be 16-byte aligned and f32 arrays 4-byte aligned";
    case SMOE_ERR_WORKSPACE: return "workspace missing or smaller than the *_workspace() size";
    case SMOE_ERR_ALIAS: return "an output overlaps an input or the workspace";
    case SMOE_ERR_DEVICE: return "current device is not gfx950 (MI355X) or could not be queried";
    case SMOE_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    default: return "unknown status";
    }
}

int smoe_gate_up(const smoe_qmat *gate, const smoe_qmat *up, int fmt, int group, int d_ff,
                 int d_model, const float *x, float *hidden, void *stream)
{
    Fmt f;
    int rc = check_format(fmt, group, &f);
    if (rc) return rc;
    if (!x || !hidden) return SMOE_ERR_NULL;
    if ((rc = check_qmat(gate, f, group, d_ff, d_model))) return rc;
    if ((rc = check_qmat(up, f, group, d_ff, d_model))) return rc;
    if (!aligned(x, 16) || !aligned(hidden, 4)) return SMOE_ERR_ALIGN;
    const size_t nh = (size_t)d_ff * 4;
    if (overlap(hidden, nh, x, (size_t)d_model * 4) ||
        overlaps_qmat(hidden, nh, gate, f, group, d_ff, d_model) ||
        overlaps_qmat(hidden, nh, up, f, group, d_ff, d_model))
        return SMOE_ERR_ALIAS;
    DecodePlan plan;
    if (!smoe::plan_decode(smoe::kGateUpOnly, f.bits, d_model, d_ff, 1, &plan)) return SMOE_ERR_SHAPE;
    DeviceInfo dev;
    if ((rc = check_device(&dev))) return rc;

    smoe::DecodeArgs a{};
    a.gate[0] = {gate->codes, gate->scales};
    a.up[0] = {up->codes, up->scales};
    a.x = x;
    a.hidden = hidden;
    a.d_model = d_model;
    a.d_ff = d_ff;
    a.group = group;
    a.scale_bytes = f.sb;
    a.n_experts = 1;
    return launch_status(smoe::launch_gate_up(f.bits, plan, a, dev.cus, (hipStream_t)stream));
}

int smoe_down(const smoe_qmat *down, int fmt, int group, int d_model, int d_ff, const float *hidden,
              float *out, void *stream)
{
    Fmt f;
    int rc = check_format(fmt, group, &f);
    if (rc) return rc;
    if (!hidden || !out) return SMOE_ERR_NULL;
    if ((rc = check_qmat(down, f, group, d_model, d_ff))) return rc;
    if (!aligned(hidden, 16) || !aligned(out, 4)) return SMOE_ERR_ALIGN;
    const size_t no = (size_t)d_model * 4;
    if (overlap(out, no, hidden, (size_t)d_ff * 4) ||
        overlaps_qmat(out, no, down, f, group, d_model, d_ff))
        return SMOE_ERR_ALIAS;
    DecodePlan plan;
    if (!smoe::plan_decode(smoe::kDownOnly, f.bits, d_model, d_ff, 1, &plan)) return SMOE_ERR_SHAPE;
    DeviceInfo dev;
    if ((rc = check_device(&dev))) return rc;

    smoe::DecodeArgs a{};
    a.down[0] = {down->codes, down->scales};
    a.hidden = const_cast<float *>(hidden);
    a.out = out;
    a.d_model = d_model;
    a.d_ff = d_ff;
    a.group = group;
    a.scale_bytes = f.sb;
    a.n_experts = 1;
    return launch_status(smoe::launch_down(f.bits, plan, a, dev.cus, (hipStream_t)stream));
}

size_t smoe_expert_ffn_workspace(int n_experts, int d_model, int d_ff, int T)
{
    if (n_experts <= 0 || d_model <= 0 || d_ff <= 0 || T <= 0) return 0;
    if (T == 1) return decode_workspace(n_experts, d_ff);
    if (T > SMOE_MAX_TOKENS) return 0;
    return batch_workspace(n_experts, d_model, d_ff, T, kMinBatchGroup).total;
}

// smoe_expert_ffn, with the caller's workspace or (noalloc) the device's
// static scratch array.
static int expert_ffn(const smoe_expert *experts, int n_experts, const float *route_w, int fmt, int group,
                      int d_model, int d_ff, int T, const float *x, float *out, void *workspace,
                      size_t workspace_bytes, void *stream, bool noalloc)
{
    Fmt f;
    int rc = check_format(fmt, group, &f);
    if (rc) return rc;
    if (!experts || !x || !out) return SMOE_ERR_NULL;
    if (n_experts < 1 || n_experts > SMOE_MAX_EXPERTS || T < 1 || T > SMOE_MAX_TOKENS)
        return SMOE_ERR_SHAPE;
    for (int e = 0; e < n_experts; ++e) {
        if ((rc = check_qmat(&experts[e].gate, f, group, d_ff, d_model))) return rc;
        if ((rc = check_qmat(&experts[e].up, f, group, d_ff, d_model))) return rc;
        if ((rc = check_qmat(&experts[e].down, f, group, d_model, d_ff))) return rc;
    }
    if (!aligned(x, 16) || !aligned(out, 4) || (route_w && !aligned(route_w, 4)))
        return SMOE_ERR_ALIGN;
    smoe::TbPlan tplan{};
    if (T > 1 && !smoe::plan_batch(f.bits, group, d_model, d_ff, n_experts, T, &tplan))
        return SMOE_ERR_GROUP;

    const size_t need = smoe_expert_ffn_workspace(n_experts, d_model, d_ff, T);
    if (noalloc ? need > SMOE_NOALLOC_SCRATCH_BYTES : (!workspace || workspace_bytes < need))
        return SMOE_ERR_WORKSPACE;
    if (!noalloc && !aligned(workspace, 256)) return SMOE_ERR_ALIGN;
    const size_t no = (size_t)T * d_model * 4;
    if (overlap(out, no, x, (size_t)T * d_model * 4) ||
        overlap(out, no, route_w, route_w ? (size_t)T * n_experts * 4 : 0))
        return SMOE_ERR_ALIAS;
    for (int e = 0; e < n_experts; ++e) {
        const smoe_expert &ex = experts[e];
        if (overlaps_qmat(out, no, &ex.gate, f, group, d_ff, d_model) ||
            overlaps_qmat(out, no, &ex.up, f, group, d_ff, d_model) ||
            overlaps_qmat(out, no, &ex.down, f, group, d_model, d_ff))
            return SMOE_ERR_ALIAS;
    }
    if (noalloc) {
        // The device's scratch array (a static device array: no caller
        // buffer can overlap it).
        DeviceInfo dev;
        if ((rc = check_device(&dev))) return rc;
        if (!dev.scratch) return SMOE_ERR_DEVICE;
        workspace = dev.scratch;
        workspace_bytes = SMOE_NOALLOC_SCRATCH_BYTES;
    } else {
        if (overlap(out, no, workspace, need) || overlap(workspace, need, x, (size_t)T * d_model * 4) ||
            overlap(workspace, need, route_w, route_w ? (size_t)T * n_experts * 4 : 0))
            return SMOE_ERR_ALIAS;
        for (int e = 0; e < n_experts; ++e) {
            const smoe_expert &ex = experts[e];
            if (overlaps_qmat(workspace, need, &ex.gate, f, group, d_ff, d_model) ||
                overlaps_qmat(workspace, need, &ex.up, f, group, d_ff, d_model) ||
                overlaps_qmat(workspace, need, &ex.down, f, group, d_model, d_ff))
                return SMOE_ERR_ALIAS;
        }
    }
    hipStream_t st = (hipStream_t)stream;
    if (T > 1) {
        DeviceInfo dev;
        if ((rc = check_device(&dev))) return rc;
        const BatchWorkspace w = batch_workspace(n_experts, d_model, d_ff, T, group);
        char *ws = static_cast<char *>(workspace);
        smoe::TbArgs a{};
        fill_experts(a, experts, n_experts);
        a.x = x;
        a.route_w = route_w;
        a.out = out;
        a.xh = reinterpret_cast<_Float16 *>(ws + w.xh);
        a.xl = reinterpret_cast<_Float16 *>(ws + w.xl);
        a.xe = reinterpret_cast<int *>(ws + w.xe);
        a.hh = reinterpret_cast<_Float16 *>(ws + w.hh);
        a.hl = reinterpret_cast<_Float16 *>(ws + w.hl);
        a.hid = reinterpret_cast<float *>(ws + w.hh);   // f32 rows over hh and hl, which are adjacent
        a.hf = reinterpret_cast<float *>(ws + w.hf);
        a.part_gu = reinterpret_cast<float *>(ws + w.pg);
        a.part_dn = reinterpret_cast<float *>(ws + w.pd);
        a.cnt_gu = reinterpret_cast<unsigned *>(ws + w.cnt);
        a.cnt_dn = a.cnt_gu + w.n_cnt_gu;
        a.n_cnt = w.n_cnt;
        a.T = T;
        a.t_pad = token_pad(T);
        a.d_model = d_model;
        a.d_ff = d_ff;
        a.group = group;
        a.scale_bytes = f.sb;
        a.n_experts = n_experts;
        a.ks_gu = tplan.ks_gu;
        a.ks_dn = tplan.ks_dn;
        return launch_status(smoe::launch_batch(f.bits, tplan, a, st));
    }

    DecodePlan plan;
    if (!smoe::plan_decode(smoe::kBoth, f.bits, d_model, d_ff, n_experts, &plan)) return SMOE_ERR_SHAPE;
    DeviceInfo dev;
    if ((rc = check_device(&dev))) return rc;

    smoe::DecodeArgs a{};
    fill_experts(a, experts, n_experts);
    a.x = x;
    a.hidden = static_cast<float *>(workspace);
    a.route_w = route_w;
    a.out = out;
    a.d_model = d_model;
    a.d_ff = d_ff;
    a.group = group;
    a.scale_bytes = f.sb;
    a.n_experts = n_experts;
    if ((rc = launch_status(smoe::launch_gate_up(f.bits, plan, a, dev.cus, st)))) return rc;
    return launch_status(smoe::launch_down(f.bits, plan, a, dev.cus, st));
}

int smoe_expert_ffn(const smoe_expert *experts, int n_experts, const float *route_w, int fmt,
                    int group, int d_model, int d_ff, int T, const float *x, float *out,
                    void *workspace, size_t workspace_bytes, void *stream)
{
    return expert_ffn(experts, n_experts, route_w, fmt, group, d_model, d_ff, T, x, out, workspace,
                      workspace_bytes, stream, false);
}

int smoe_expert_ffn_noalloc(const smoe_expert *experts, int n_experts, const float *route_w, int fmt,
                            int group, int d_model, int d_ff, int T, const float *x, float *out, void *stream)
{
    return expert_ffn(experts, n_experts, route_w, fmt, group, d_model, d_ff, T, x, out, nullptr, 0, stream,
                      true);
}

size_t smoe_routed_ffn_workspace(int n_experts, int d_model, int d_ff, int T, int top_k)
{
    if (n_experts <= 0 || d_model <= 0 || d_ff <= 0 || T <= 0 || T > SMOE_MAX_TOKENS || top_k <= 0) return 0;
    return routed_workspace(n_experts, d_model, d_ff, T, top_k).total;
}

int smoe_routed_ffn(const smoe_expert *experts, int n_experts, int fmt, int group, int d_model, int d_ff,
                    int T, int top_k, const int *expert_ids, const float *expert_w, const float *x, float *out,
                    void *workspace, size_t workspace_bytes, void *stream)
{
    Fmt f;
    int rc = check_format(fmt, group, &f);
    if (rc) return rc;
    if (!experts || !expert_ids || !expert_w || !x || !out) return SMOE_ERR_NULL;
    if (n_experts < 1 || n_experts > SMOE_MAX_EXPERTS || T < 1 || T > SMOE_MAX_TOKENS || top_k < 1 ||
        top_k > SMOE_MAX_EXPERTS)
        return SMOE_ERR_SHAPE;
    for (int e = 0; e < n_experts; ++e) {
        if ((rc = check_qmat(&experts[e].gate, f, group, d_ff, d_model))) return rc;
        if ((rc = check_qmat(&experts[e].up, f, group, d_ff, d_model))) return rc;
        if ((rc = check_qmat(&experts[e].down, f, group, d_model, d_ff))) return rc;
    }
    if (!aligned(x, 16) || !aligned(out, 4) || !aligned(expert_ids, 4) || !aligned(expert_w, 4))
        return SMOE_ERR_ALIGN;
    smoe::TbPlan plan{};
    if (!smoe::plan_routed(f.bits, group, d_model, d_ff, n_experts, T, top_k, &plan)) return SMOE_ERR_GROUP;
    const size_t need = smoe_routed_ffn_workspace(n_experts, d_model, d_ff, T, top_k);
    if (!workspace || workspace_bytes < need) return SMOE_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SMOE_ERR_ALIGN;
    const size_t no = (size_t)T * d_model * 4, nx = no, ns = (size_t)T * top_k * 4;
    if (overlap(out, no, x, nx) || overlap(out, no, workspace, need) || overlap(out, no, expert_ids, ns) ||
        overlap(out, no, expert_w, ns) || overlap(workspace, need, x, nx) ||
        overlap(workspace, need, expert_ids, ns) || overlap(workspace, need, expert_w, ns))
        return SMOE_ERR_ALIAS;
    for (int e = 0; e < n_experts; ++e) {
        const smoe_expert &ex = experts[e];
        if (overlaps_qmat(out, no, &ex.gate, f, group, d_ff, d_model) ||
            overlaps_qmat(out, no, &ex.up, f, group, d_ff, d_model) ||
            overlaps_qmat(out, no, &ex.down, f, group, d_model, d_ff) ||
            overlaps_qmat(workspace, need, &ex.gate, f, group, d_ff, d_model) ||
            overlaps_qmat(workspace, need, &ex.up, f, group, d_ff, d_model) ||
            overlaps_qmat(workspace, need, &ex.down, f, group, d_model, d_ff))
            return SMOE_ERR_ALIAS;
    }
    DeviceInfo dev;
    if ((rc = check_device(&dev))) return rc;
    const RoutedWorkspace w = routed_workspace(n_experts, d_model, d_ff, T, top_k);
    char *ws = static_cast<char *>(workspace);
    smoe::TbArgs a{};
    fill_experts(a, experts, n_experts);
    a.x = x;
    a.out = out;
    a.xh = reinterpret_cast<_Float16 *>(ws + w.xh);
    a.xl = reinterpret_cast<_Float16 *>(ws + w.xl);
    a.xe = reinterpret_cast<int *>(ws + w.xe);
    a.hh = reinterpret_cast<_Float16 *>(ws + w.hh);
    a.hl = reinterpret_cast<_Float16 *>(ws + w.hl);
    a.hid = reinterpret_cast<float *>(ws + w.hh);   // f32 rows over hh and hl, which are adjacent
    a.hf = reinterpret_cast<float *>(ws + w.hf);
    a.part_gu = reinterpret_cast<float *>(ws + w.pg);
    a.cnt_gu = reinterpret_cast<unsigned *>(ws + w.tcnt);
    a.cnt_dn = nullptr;
    a.n_cnt = w.n_tcnt;
    a.list = reinterpret_cast<int *>(ws + w.list);
    a.cnt = reinterpret_cast<int *>(ws + w.cnt);
    a.slot_ok = reinterpret_cast<int *>(ws + w.ok);
    a.ys = reinterpret_cast<float *>(ws + w.ys);
    a.ids = expert_ids;
    a.slot_w = expert_w;
    a.top_k = top_k;
    a.T = T;
    a.t_pad = token_pad(T);
    a.d_model = d_model;
    a.d_ff = d_ff;
    a.group = group;
    a.scale_bytes = f.sb;
    a.n_experts = n_experts;
    a.ks_gu = plan.ks_gu;
    a.ks_dn = 1;
    return launch_status(smoe::launch_routed(f.bits, plan, a, (hipStream_t)stream));
}

size_t matvec_bf16_workspace(int rows, int cols)
{
    (void)rows;
    (void)cols;
    return 0;
}

int matvec_bf16(const uint16_t *W, int rows, int cols, const float *x, float *y, void *workspace,
                size_t workspace_bytes, void *stream)
{
    (void)workspace;
    (void)workspace_bytes;
    if (!W || !x || !y) return SMOE_ERR_NULL;
    if (rows <= 0 || cols <= 0 || cols % 8 || cols > SMOE_MAX_BF16_COLS) return SMOE_ERR_SHAPE;
    if (!aligned(W, 16) || !aligned(x, 16) || !aligned(y, 4)) return SMOE_ERR_ALIGN;
    const size_t ny = (size_t)rows * 4;
    if (overlap(y, ny, W, (size_t)rows * cols * 2) || overlap(y, ny, x, (size_t)cols * 4))
        return SMOE_ERR_ALIAS;
    MapConfig cfg;
    if (!smoe::choose_bf16map(cols / 8, rows, &cfg)) return SMOE_ERR_SHAPE;
    int rc = check_device(nullptr);
    if (rc) return rc;
    smoe::Bf16Args a{W, x, y, rows, cols};
    return launch_status(smoe::launch_matvec_bf16(cfg, a, (hipStream_t)stream));
}

int matvec_bf16_batch(const smoe_bf16_job *jobs, int n_jobs, void *stream)
{
    if (!jobs) return SMOE_ERR_NULL;
    if (n_jobs < 1 || n_jobs > SMOE_MAX_BF16_JOBS) return SMOE_ERR_SHAPE;
    int max_cols = 0;
    long total_rows = 0;
    for (int j = 0; j < n_jobs; ++j) {
        const smoe_bf16_job &b = jobs[j];
        if (!b.W || !b.x || !b.y) return SMOE_ERR_NULL;
        if (b.rows <= 0 || b.cols <= 0 || b.cols % 8 || b.cols > SMOE_MAX_BF16_COLS) return SMOE_ERR_SHAPE;
        if (!aligned(b.W, 16) || !aligned(b.x, 16) || !aligned(b.y, 4)) return SMOE_ERR_ALIGN;
        max_cols = std::max(max_cols, b.cols);
        total_rows += b.rows;
    }
    for (int j = 0; j < n_jobs; ++j) {
        const size_t ny = (size_t)jobs[j].rows * 4;
        for (int k = 0; k < n_jobs; ++k) {
            const smoe_bf16_job &o = jobs[k];
            if (overlap(jobs[j].y, ny, o.W, (size_t)o.rows * o.cols * 2) ||
                overlap(jobs[j].y, ny, o.x, (size_t)o.cols * 4) ||
                (k != j && overlap(jobs[j].y, ny, o.y, (size_t)o.rows * 4)))
                return SMOE_ERR_ALIAS;
        }
    }
    MapConfig cfg;
    if (total_rows > INT_MAX || !smoe::choose_bf16map(max_cols / 8, (int)total_rows, &cfg)) return SMOE_ERR_SHAPE;
    int rc = check_device(nullptr);
    if (rc) return rc;
    smoe::Bf16BatchArgs a{};
    for (int j = 0; j < n_jobs; ++j)
        a.job[j] = smoe::Bf16Job{jobs[j].W, jobs[j].x, jobs[j].y, jobs[j].rows, jobs[j].cols};
    a.n = n_jobs;
    return launch_status(smoe::launch_matvec_bf16_batch(cfg, a, (hipStream_t)stream));
}

size_t smoe_attn_decode_workspace(int d_model, int n_head, int n_kv, int head_dim, int max_ctx)
{
    if (!attn_shape_ok(d_model, n_head, n_kv, head_dim, max_ctx)) return 0;
    return attn_workspace(n_head, n_kv, head_dim, max_ctx).total;
}

int smoe_attn_decode(const smoe_attn_weights *w, int d_model, int n_head, int n_kv, int head_dim, const float *x,
                     int pos, double rope_base, float *k_cache, float *v_cache, int max_ctx, float *out,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    if (!w || !w->wq || !w->wk || !w->wv || !w->wo || !w->q_norm || !w->k_norm || !x || !k_cache || !v_cache ||
        !out)
        return SMOE_ERR_NULL;
    if (!attn_shape_ok(d_model, n_head, n_kv, head_dim, max_ctx)) return SMOE_ERR_SHAPE;
    if (pos < 0 || pos >= max_ctx || !(rope_base > 0.0) || rope_base > 1e300) return SMOE_ERR_SHAPE;
    if (!aligned(w->wq, 16) || !aligned(w->wk, 16) || !aligned(w->wv, 16) || !aligned(w->wo, 16) ||
        !aligned(w->q_norm, 4) || !aligned(w->k_norm, 4) || !aligned(x, 16) || !aligned(k_cache, 16) ||
        !aligned(v_cache, 16) || !aligned(out, 4))
        return SMOE_ERR_ALIGN;
    const AttnWorkspace ws = attn_workspace(n_head, n_kv, head_dim, max_ctx);
    if (!workspace || workspace_bytes < ws.total) return SMOE_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return SMOE_ERR_ALIGN;
    const size_t nq = (size_t)n_head * head_dim, nk = (size_t)n_kv * head_dim;
    const size_t cache = nk * (size_t)max_ctx * 4;
    // Written ranges (out, the caches, the workspace) against everything else.
    struct Range {
        const void *p;
        size_t n;
    };
    const Range in[] = {{w->wq, nq * d_model * 2}, {w->wk, nk * d_model * 2}, {w->wv, nk * d_model * 2},
                        {w->wo, (size_t)d_model * nq * 2}, {w->q_norm, (size_t)head_dim * 4},
                        {w->k_norm, (size_t)head_dim * 4}, {x, (size_t)d_model * 4}};
    const Range wr[] = {{out, (size_t)d_model * 4}, {k_cache, cache}, {v_cache, cache}, {workspace, ws.total}};
    for (const Range &a : wr) {
        for (const Range &b : in)
            if (overlap(a.p, a.n, b.p, b.n)) return SMOE_ERR_ALIAS;
        for (const Range &b : wr)
            if (&a != &b && overlap(a.p, a.n, b.p, b.n)) return SMOE_ERR_ALIAS;
    }
    MapConfig cfg_qkv, cfg_o;
    if (!smoe::choose_bf16map(d_model / 8, (int)(nq + 2 * nk), &cfg_qkv) ||
        !smoe::choose_bf16map((int)(nq / 8), d_model, &cfg_o))
        return SMOE_ERR_SHAPE;
    int rc = check_device(nullptr);
    if (rc) return rc;
    char *wsb = static_cast<char *>(workspace);
    float *q = reinterpret_cast<float *>(wsb + ws.q), *k = reinterpret_cast<float *>(wsb + ws.k);
    float *v = reinterpret_cast<float *>(wsb + ws.v), *att = reinterpret_cast<float *>(wsb + ws.att);
    const hipStream_t st = (hipStream_t)stream;
    smoe::Bf16BatchArgs b{};
    b.job[0] = smoe::Bf16Job{w->wq, x, q, (int)nq, d_model};
    b.job[1] = smoe::Bf16Job{w->wk, x, k, (int)nk, d_model};
    b.job[2] = smoe::Bf16Job{w->wv, x, v, (int)nk, d_model};
    b.n = 3;
    if ((rc = launch_status(smoe::launch_matvec_bf16_batch(cfg_qkv, b, st)))) return rc;
    smoe::AttnArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.q_norm = w->q_norm;
    a.k_norm = w->k_norm;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.part_o = reinterpret_cast<float *>(wsb + ws.part_o);
    a.part_ml = reinterpret_cast<float *>(wsb + ws.part_ml);
    a.att = att;
    a.rope_base = rope_base;
    a.n_head = n_head;
    a.n_kv = n_kv;
    a.head_dim = head_dim;
    a.max_ctx = max_ctx;
    a.pos = pos;
    a.n_chunks = smoe::attn_chunks(max_ctx);
    if ((rc = launch_status(smoe::launch_attn_core(a, st)))) return rc;
    smoe::Bf16Args o{w->wo, att, out, d_model, (int)nq};
    return launch_status(smoe::launch_matvec_bf16(cfg_o, o, st));
}

}  // extern "C"
