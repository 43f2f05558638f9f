// Decode (one token) kernels for group-quantised expert matrices on gfx950.
//
// What is computed (Metal Compute Kernels, S-MoE docs, "Fused FFN Kernels --
// One Simdgroup Per Output Row"): for a row of affine codes with one scale per
// column group, sum_j w_j x_j with w_j = (code_j - Z)/Z * s equals, group by
// group, s * ((sum code_j x_j) / Z - sum x_j).  The codes therefore enter only
// through the plain dot product sum code_j x_j; the scale and Z are applied once
// per 16-byte chunk (a chunk never straddles a group), and no f32 weight is ever
// formed.  gate_up reads the gate and up rows of an output index against the
// same input, and writes SiLU(g) * u; down reads hidden.
//
// Mapping on the GPU (a redesign for 64-lane waves, not the page's
// one-simdgroup-per-row layout): a block of nw waves covers a tile of rows; the
// chunks of a row are split into nw contiguous slices, one per wave, and inside
// a wave `LPR` lanes share a row, so each lane always reads the same column
// chunk(s).  A lane therefore loads its slice of the input vector into
// registers once and then streams many rows against it: there is no LDS
// traffic for the input in the row loop, every code load is a 16-byte
// coalesced read, and all ITER row steps are issued before any of them is
// consumed.  Row partials are reduced inside the wave with DPP and across
// waves through LDS.  The down kernel runs one block per (row tile, expert)
// and combines the experts' router-weighted outputs deterministically: the
// last block of a row tile to finish sums the experts in ascending order.
#include "launch.h"

#include <cmath>
#include <cstdlib>

namespace smoe {
namespace {

// Fields of a packed byte: field f of a byte (bits BITS*f .. BITS*f+BITS-1)
// holds the code of column F*byte + f.  Masking one field of every byte leaves
// code * 2^(BITS*f) in each byte, which v_cvt_f32_ubyteN converts directly;
// the matching x values are pre-multiplied by 2^-(BITS*f), which is exact.
template <int BITS>
__device__ __forceinline__ void load_vec_chunk(const float *v, int chunk, bool valid, float *xv,
                                               float &xsum)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    constexpr int F = 8 / BITS;
    xsum = 0.0f;
    if (!valid) {
#pragma unroll
        for (int j = 0; j < CPC; ++j) xv[j] = 0.0f;
        return;
    }
    const float4 *src = reinterpret_cast<const float4 *>(v + (size_t)chunk * CPC);
#pragma unroll
    for (int q = 0; q < CPC / 4; ++q) {
        const float4 t = src[q];
        const float vals[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 4 * q + i;
            const int f = j % F;
            xsum += vals[i];
            xv[j] = vals[i] * (1.0f / (float)(1u << (BITS * f)));
        }
    }
}

// sum over the chunk's codes of code * x (x pre-scaled as above).
template <int BITS>
__device__ __forceinline__ float chunk_dot(const uint4 q, const float *xv)
{
    constexpr int F = 8 / BITS;
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
#pragma unroll
        for (int f = 0; f < F; ++f) {
            const uint32_t mask = (((1u << BITS) - 1u) * 0x01010101u) << (BITS * f);
            const uint32_t v = opaque(w[m] & mask);
#pragma unroll
            for (int p = 0; p < 4; ++p)
                acc[m] = fmaf((float)((v >> (8 * p)) & 0xFFu), xv[m * 4 * F + p * F + f], acc[m]);
        }
    }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

template <int BITS, int LPR, int NCH, int ITER>
__global__ __launch_bounds__(512) void k_gate_up(const GateUpArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    constexpr int RS = 64 / LPR;
    constexpr int RB = RS * ITER;
    extern __shared__ float red[];  // [nw][RB][2]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int lr = lane % LPR, slot = lane / LPR;
    const int cpr = a.d_model / CPC;
    const int sl = (cpr + nw - 1) / nw;
    const int e = blockIdx.x / a.blocks_per_expert;
    const int row0 = (blockIdx.x - e * a.blocks_per_expert) * RB;
    const size_t row_bytes = (size_t)a.d_model * BITS / 8;
    const int gpr = a.d_model / a.group;
    const QPtr G = a.gate[e], U = a.up[e];

    if (blockIdx.x == 0)
        for (int i = tid; i < a.n_counters; i += blockDim.x) a.counters[i] = 0;

    int c[NCH], gi[NCH];
    bool valid[NCH];
    float xv[NCH][CPC], xs[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int cs = lr + LPR * k;
        c[k] = wave * sl + cs;
        valid[k] = cs < sl && c[k] < cpr;
        gi[k] = valid[k] ? c[k] * CPC / a.group : 0;
    }

    // Issue every code and scale load of the tile first.
    uint4 qg[ITER][NCH], qu[ITER][NCH];
    float sg[ITER][NCH], su[ITER][NCH];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int r = row0 + slot + RS * it;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            if (valid[k] && r < a.d_ff) {
                const size_t off = (size_t)r * row_bytes + (size_t)c[k] * 16;
                qg[it][k] = load16(G.codes + off);
                qu[it][k] = load16(U.codes + off);
                sg[it][k] = G.scales[(size_t)r * gpr + gi[k]];
                su[it][k] = U.scales[(size_t)r * gpr + gi[k]];
            } else {
                qg[it][k] = qu[it][k] = make_uint4(0, 0, 0, 0);
                sg[it][k] = su[it][k] = 0.0f;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k) load_vec_chunk<BITS>(a.x, c[k], valid[k], xv[k], xs[k]);

#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        float pg = 0.0f, pu = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const float dg = chunk_dot<BITS>(qg[it][k], xv[k]);
            const float du = chunk_dot<BITS>(qu[it][k], xv[k]);
            pg = fmaf(sg[it][k], fmaf(dg, QFormat<BITS>::kInvZ, -xs[k]), pg);
            pu = fmaf(su[it][k], fmaf(du, QFormat<BITS>::kInvZ, -xs[k]), pu);
        }
        pg = lane_group_sum<LPR>(pg);
        pu = lane_group_sum<LPR>(pu);
        if (lr == 0) {
            const int t = wave * RB + slot + RS * it;
            red[2 * t] = pg;
            red[2 * t + 1] = pu;
        }
    }
    __syncthreads();
    for (int t = tid; t < RB; t += blockDim.x) {
        const int r = row0 + t;
        if (r < a.d_ff) {
            float g = 0.0f, u = 0.0f;
            for (int w = 0; w < nw; ++w) {
                g += red[2 * (w * RB + t)];
                u += red[2 * (w * RB + t) + 1];
            }
            a.hidden[(size_t)e * a.d_ff + r] = silu(g) * u;
        }
    }
}

template <int BITS, int LPR, int NCH, int ITER>
__global__ __launch_bounds__(512) void k_down(const DownArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    constexpr int RS = 64 / LPR;
    constexpr int RB = RS * ITER;
    extern __shared__ float red[];  // [nw][RB]
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int lr = lane % LPR, slot = lane / LPR;
    const int E = a.n_experts;
    const int cpr = a.d_ff / CPC;
    const int sl = (cpr + nw - 1) / nw;
    const int rb = blockIdx.x / E, e = blockIdx.x - rb * E;
    const int row0 = rb * RB;
    const size_t row_bytes = (size_t)a.d_ff * BITS / 8;
    const int gpr = a.d_ff / a.group;
    const QPtr D = a.down[e];

    int c[NCH], gi[NCH];
    bool valid[NCH];
    float hv[NCH][CPC], hs[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int cs = lr + LPR * k;
        c[k] = wave * sl + cs;
        valid[k] = cs < sl && c[k] < cpr;
        gi[k] = valid[k] ? c[k] * CPC / a.group : 0;
    }

    uint4 q[ITER][NCH];
    float s[ITER][NCH];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int r = row0 + slot + RS * it;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            if (valid[k] && r < a.d_model) {
                q[it][k] = load16(D.codes + (size_t)r * row_bytes + (size_t)c[k] * 16);
                s[it][k] = D.scales[(size_t)r * gpr + gi[k]];
            } else {
                q[it][k] = make_uint4(0, 0, 0, 0);
                s[it][k] = 0.0f;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NCH; ++k)
        load_vec_chunk<BITS>(a.hidden + (size_t)e * a.d_ff, c[k], valid[k], hv[k], hs[k]);

#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        float py = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const float d = chunk_dot<BITS>(q[it][k], hv[k]);
            py = fmaf(s[it][k], fmaf(d, QFormat<BITS>::kInvZ, -hs[k]), py);
        }
        py = lane_group_sum<LPR>(py);
        if (lr == 0) red[wave * RB + slot + RS * it] = py;
    }
    __syncthreads();

    const float rw = a.route_w ? a.route_w[e] : 1.0f;
    if (E == 1) {
        for (int t = tid; t < RB; t += blockDim.x) {
            const int r = row0 + t;
            if (r < a.d_model) {
                float y = 0.0f;
                for (int w = 0; w < nw; ++w) y += red[w * RB + t];
                a.out[r] = y * rw;
            }
        }
        return;
    }

    // Several experts: publish this expert's weighted rows, then the last block
    // of the row tile adds the experts in ascending order.  The partial rows
    // are written and read with agent-scope atomic accesses, which go through
    // to the device-wide point of coherence instead of staying in one XCD's
    // L2, so no cache-wide write-back or invalidate is needed: each wave waits
    // for its stores to complete before the barrier, and only then does one
    // thread bump the tile's counter.
    for (int t = tid; t < RB; t += blockDim.x) {
        const int r = row0 + t;
        if (r < a.d_model) {
            float y = 0.0f;
            for (int w = 0; w < nw; ++w) y += red[w * RB + t];
            __hip_atomic_store(a.partial + (size_t)e * a.d_model + r, y * rw, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
        s_last = __hip_atomic_fetch_add(&a.counters[rb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == E - 1;
    __syncthreads();
    if (s_last) {
        for (int t = tid; t < RB; t += blockDim.x) {
            const int r = row0 + t;
            if (r < a.d_model) {
                float acc = 0.0f;
                for (int x = 0; x < E; ++x)
                    acc += __hip_atomic_load(a.partial + (size_t)x * a.d_model + r, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
                a.out[r] = acc;
            }
        }
        if (tid == 0) a.counters[rb] = 0;
    }
}

template <int BITS, int LPR, int NCH, int ITER>
hipError_t run_gate_up(const MapConfig &cfg, const GateUpArgs &a, int n_experts, hipStream_t st)
{
    constexpr int RB = (64 / LPR) * ITER;
    const dim3 grid(n_experts * a.blocks_per_expert), block(64 * cfg.nw);
    const size_t shmem = sizeof(float) * 2 * RB * cfg.nw;
    hipLaunchKernelGGL((k_gate_up<BITS, LPR, NCH, ITER>), grid, block, shmem, st, a);
    return hipGetLastError();
}

template <int BITS, int LPR, int NCH, int ITER>
hipError_t run_down(const MapConfig &cfg, const DownArgs &a, hipStream_t st)
{
    constexpr int RB = (64 / LPR) * ITER;
    const dim3 grid(a.n_experts * a.row_blocks), block(64 * cfg.nw);
    const size_t shmem = sizeof(float) * RB * cfg.nw;
    hipLaunchKernelGGL((k_down<BITS, LPR, NCH, ITER>), grid, block, shmem, st, a);
    return hipGetLastError();
}

}  // namespace

// Instantiated mappings (blocks of at most 8 waves): lanes per row 2..32, one or two chunks per lane (4-bit)
// or one (2-bit: a chunk is already 64 codes), 1..8 unrolled row steps.
#define SMOE_QMAP_ITERS(F, B, L, N) F(B, L, N, 1) F(B, L, N, 2) F(B, L, N, 4) F(B, L, N, 8)
#define SMOE_QMAP_LPRS(F, B, N)                                                                \
    SMOE_QMAP_ITERS(F, B, 2, N) SMOE_QMAP_ITERS(F, B, 4, N) SMOE_QMAP_ITERS(F, B, 8, N)         \
    SMOE_QMAP_ITERS(F, B, 16, N) SMOE_QMAP_ITERS(F, B, 32, N)
#define SMOE_QMAP_ALL(F) SMOE_QMAP_LPRS(F, 4, 1) SMOE_QMAP_LPRS(F, 4, 2) SMOE_QMAP_LPRS(F, 2, 1)

static bool qmap_instantiated(int bits, int lpr, int nch, int iter)
{
#define SMOE_HAS(B, L, N, I) if (bits == B && lpr == L && nch == N && iter == I) return true;
    SMOE_QMAP_ALL(SMOE_HAS)
#undef SMOE_HAS
    return false;
}

bool choose_qmap(int bits, int chunks, int rows, int n_experts, MapConfig *cfg)
{
    // Cover the row with nw * lpr * nch lane-chunks, wasting as few lanes as
    // possible, preferring one chunk per lane and blocks of about 8 waves.
    static const int kNw[] = {8, 6, 4, 7, 5, 3, 2, 1};
    static const int kLpr[] = {16, 8, 4, 2, 32};
    double best = 1e30;
    MapConfig pick{0, 0, 0, 0};
    for (int nch = 1; nch <= (bits == 4 ? 2 : 1); ++nch)
        for (int lpr : kLpr)
            for (int nw : kNw) {
                const int sl = (chunks + nw - 1) / nw;
                if (sl > lpr * nch) continue;
                const double waste = 1.0 - (double)chunks / (nw * lpr * nch);
                const double pen = 10.0 * waste + 0.7 * (nch - 1) +
                                   0.25 * std::abs(std::log2((double)nw / 8.0));
                if (pen < best) {
                    best = pen;
                    pick = MapConfig{nw, lpr, nch, 1};
                }
            }
    if (!pick.nw) return false;
    // Unroll as far as the grid still has >= 8 waves per CU (2048 waves).
    const int rs = 64 / pick.lpr;
    for (int iter : {8, 4, 2, 1}) {
        const long blocks = (long)n_experts * ((rows + rs * iter - 1) / (rs * iter));
        if (iter == 1 || blocks * pick.nw >= 2048) {
            pick.iter = iter;
            break;
        }
    }
    if (!qmap_instantiated(bits, pick.lpr, pick.nch, pick.iter)) return false;
    *cfg = pick;
    return true;
}

hipError_t launch_gate_up(int bits, const MapConfig &cfg, const GateUpArgs &a, int n_experts,
                          hipStream_t st)
{
#define SMOE_RUN(B, L, N, I) \
    if (bits == B && cfg.lpr == L && cfg.nch == N && cfg.iter == I) return run_gate_up<B, L, N, I>(cfg, a, n_experts, st);
    SMOE_QMAP_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

hipError_t launch_down(int bits, const MapConfig &cfg, const DownArgs &a, hipStream_t st)
{
#define SMOE_RUN(B, L, N, I) \
    if (bits == B && cfg.lpr == L && cfg.nch == N && cfg.iter == I) return run_down<B, L, N, I>(cfg, a, st);
    SMOE_QMAP_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

}  // namespace smoe
