// Dense bf16 matvec y = W x on gfx950 (Metal Compute Kernels, S-MoE docs,
// "Coalesced Dense Matvec -- the Same Contract for bf16": 16-byte chunks of
// eight bf16 values, widened to f32 by shifting each half of a dword into the
// upper 16 bits, which is exact; f32 input; f32 output).
//
// Same mapping as the quantised kernels: nw waves split a row's chunks into
// contiguous slices, LPR lanes share a row inside a wave, every lane keeps its
// x slice in registers and streams ITER row steps of 16-byte loads issued up
// front; DPP reduction inside the wave, LDS across waves.
//
// The batched form ("Batched Scout Matvec": several independent matvecs of
// one layer in one submission) runs N such matvecs in one launch: the blocks
// are dealt to the jobs in order, each job getting ceil(rows / rows per block)
// of them, all with the lane map of the widest job.
#include "launch.h"

namespace smoe {
namespace {

// Element 2m of a row sits in the low half of dword m, element 2m+1 in the high half.
__device__ __forceinline__ float bf16_chunk_dot(const uint4 q, const float *xv, float acc0)
{
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
    float a0 = acc0, a1 = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        a0 = fmaf(__uint_as_float(w[m] << 16), xv[2 * m], a0);
        a1 = fmaf(__uint_as_float(w[m] & 0xFFFF0000u), xv[2 * m + 1], a1);
    }
    return a0 + a1;
}

// Rows row0 .. row0 + RS*ITER - 1 of y = W x (one block's share).
template <int LPR, int NCH, int ITER>
__device__ __forceinline__ void matvec_rows(const Bf16Args &a, int row0)
{
    constexpr int RS = 64 / LPR;
    constexpr int RB = RS * ITER;
    extern __shared__ float red[];  // [nw][RB]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int lr = lane % LPR, slot = lane / LPR;
    const int cpr = a.cols / 8;
    const int sl = (cpr + nw - 1) / nw;
    const uint8_t *W = reinterpret_cast<const uint8_t *>(a.W);
    const size_t row_bytes = (size_t)a.cols * 2;

    int c[NCH];
    bool valid[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        const int cs = lr + LPR * k;
        c[k] = wave * sl + cs;
        valid[k] = cs < sl && c[k] < cpr;
    }

    // Loads are unconditional from clamped, in-bounds addresses (a divergent
    // "load, else zero" would serialise them); lanes outside the matrix get a
    // zero x slice below, and rows past the end are never stored.
    uint4 q[ITER][NCH];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int r = row0 + slot + RS * it;
        const int rc = r < a.rows ? r : a.rows - 1;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            q[it][k] = load16(W + (size_t)rc * row_bytes + (size_t)(valid[k] ? c[k] : 0) * 16);
    }

    float xv[NCH][8];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
        if (valid[k]) {
            const float4 *src = reinterpret_cast<const float4 *>(a.x + (size_t)c[k] * 8);
            const float4 u = src[0], v = src[1];
            xv[k][0] = u.x; xv[k][1] = u.y; xv[k][2] = u.z; xv[k][3] = u.w;
            xv[k][4] = v.x; xv[k][5] = v.y; xv[k][6] = v.z; xv[k][7] = v.w;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) xv[k][j] = 0.0f;
        }
    }

#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        float acc = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) acc = bf16_chunk_dot(q[it][k], xv[k], acc);
        acc = lane_group_sum<LPR>(acc);
        if (lr == 0) red[wave * RB + slot + RS * it] = acc;
    }
    __syncthreads();
    for (int t = tid; t < RB; t += blockDim.x) {
        const int r = row0 + t;
        if (r < a.rows) {
            float y = 0.0f;
            for (int w = 0; w < nw; ++w) y += red[w * RB + t];
            a.y[r] = y;
        }
    }
}

template <int LPR, int NCH, int ITER>
__global__ __launch_bounds__(512) void k_matvec_bf16(const Bf16Args a)
{
    matvec_rows<LPR, NCH, ITER>(a, blockIdx.x * (64 / LPR) * ITER);
}

// Block b serves the job j with blk_start[j] <= b < blk_start[j + 1].
template <int LPR, int NCH, int ITER>
__global__ __launch_bounds__(512) void k_matvec_bf16_batch(const Bf16BatchArgs a)
{
    const int b = blockIdx.x;
    int j = 0;
    while (j + 1 < a.n && b >= a.blk_start[j + 1]) ++j;
    const Bf16Job &jb = a.job[j];
    const Bf16Args one{jb.W, jb.x, jb.y, jb.rows, jb.cols};
    matvec_rows<LPR, NCH, ITER>(one, (b - a.blk_start[j]) * (64 / LPR) * ITER);
}

template <int LPR, int NCH, int ITER>
hipError_t run_bf16(const MapConfig &cfg, const Bf16Args &a, hipStream_t st)
{
    constexpr int RB = (64 / LPR) * ITER;
    const dim3 grid((a.rows + RB - 1) / RB), block(64 * cfg.nw);
    hipLaunchKernelGGL((k_matvec_bf16<LPR, NCH, ITER>), grid, block, sizeof(float) * RB * cfg.nw, st, a);
    return hipGetLastError();
}

template <int LPR, int NCH, int ITER>
hipError_t run_bf16_batch(const MapConfig &cfg, Bf16BatchArgs a, hipStream_t st)
{
    constexpr int RB = (64 / LPR) * ITER;
    a.blk_start[0] = 0;
    for (int j = 0; j < a.n; ++j) a.blk_start[j + 1] = a.blk_start[j] + (a.job[j].rows + RB - 1) / RB;
    const dim3 grid((unsigned)a.blk_start[a.n]), block(64 * cfg.nw);
    hipLaunchKernelGGL((k_matvec_bf16_batch<LPR, NCH, ITER>), grid, block, sizeof(float) * RB * cfg.nw, st, a);
    return hipGetLastError();
}

}  // namespace

#define SMOE_BMAP_ITERS(F, L, N) F(L, N, 1) F(L, N, 2) F(L, N, 4) F(L, N, 8)
#define SMOE_BMAP_NCHS(F, L) SMOE_BMAP_ITERS(F, L, 1) SMOE_BMAP_ITERS(F, L, 2) SMOE_BMAP_ITERS(F, L, 4) SMOE_BMAP_ITERS(F, L, 8)
#define SMOE_BMAP_ALL(F) SMOE_BMAP_NCHS(F, 4) SMOE_BMAP_NCHS(F, 16) SMOE_BMAP_NCHS(F, 64)

bool choose_bf16map(int chunks, int rows, MapConfig *cfg)
{
    // Up to 16384 rows (the projections of a layer): 64 lanes per row over
    // 8 waves, the fewest chunks per lane that cover the row, and the most
    // row steps a lane loads up front that still give 16384 waves.  Measured
    // against the map below: 4096 x 8192 14.4 -> 13.1 us, 8192 x 4096 13.3 ->
    // 12.7 us; taller matrices (the LM head: 187.6 against 193 us) keep it.
    if (rows <= 16384) {
        const int sl = (chunks + 7) / 8;
        const int nch = sl <= 64 ? 1 : sl <= 128 ? 2 : sl <= 256 ? 4 : 8;
        if (sl <= 64 * nch && 1.0 - (double)chunks / (8 * 64 * nch) <= 0.25) {
            MapConfig m{8, 64, nch, 1};
            for (int iter : {8, 4, 2, 1}) {
                if ((long)rows / iter * 8 >= 16384 && 4 * iter * nch + 8 * nch <= 96) {
                    m.iter = iter;
                    break;
                }
            }
            *cfg = m;
            return true;
        }
    }
    // 16 lanes per row when the slice allows it (short DPP reduction, four rows
    // per wave step), otherwise 4, or 64 for the widest rows; blocks of up to
    // 8 waves, as many as keep every lane busy.
    static const int kNw[] = {8, 4, 6, 2, 1};
    double best = 1e30;
    MapConfig pick{0, 0, 0, 0};
    for (int lpr : {16, 4, 64})
        for (int nch : {1, 2, 4, 8})
            for (int nw : kNw) {
                const int sl = (chunks + nw - 1) / nw;
                if (sl > lpr * nch) continue;
                const double waste = 1.0 - (double)chunks / (nw * lpr * nch);
                const double pen = 10.0 * waste + (lpr == 16 ? 0.0 : 0.5) + 0.05 * nch + (nw == 8 ? 0.0 : 0.3);
                if (pen < best) {
                    best = pen;
                    pick = MapConfig{nw, lpr, nch, 1};
                }
            }
    if (!pick.nw) return false;
    // Row steps whose loads a lane issues up front: the most that still gives
    // 4096 waves, as long as the loads (4 ITER NCH registers) and the x slice
    // (8 NCH) stay within 96 registers, so that two 8-wave blocks fit on a
    // compute unit and one block's reduction overlaps the other's loads
    // (measured: the 151936 x 4096 LM head 244 -> 187 us, 4096 x 8192 15.7 ->
    // 14.5 us).
    const int rs = 64 / pick.lpr;
    for (int iter : {8, 4, 2, 1}) {
        const long blocks = (rows + rs * iter - 1) / (rs * iter);
        if (iter == 1 || (blocks * pick.nw >= 4096 && 4 * iter * pick.nch + 8 * pick.nch <= 96)) {
            pick.iter = iter;
            break;
        }
    }
    *cfg = pick;
    return true;
}

hipError_t launch_matvec_bf16(const MapConfig &cfg, const Bf16Args &a, hipStream_t st)
{
#define SMOE_RUN(L, N, I) \
    if (cfg.lpr == L && cfg.nch == N && cfg.iter == I) return run_bf16<L, N, I>(cfg, a, st);
    SMOE_BMAP_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

hipError_t launch_matvec_bf16_batch(const MapConfig &cfg, const Bf16BatchArgs &a, hipStream_t st)
{
#define SMOE_RUN(L, N, I) \
    if (cfg.lpr == L && cfg.nch == N && cfg.iter == I) return run_bf16_batch<L, N, I>(cfg, a, st);
    SMOE_BMAP_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

}  // namespace smoe
