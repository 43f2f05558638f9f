// Decode (one token) kernels for group-quantised expert matrices on gfx950.
//
// What is computed (Metal Compute Kernels, S-MoE docs, "Fused FFN Kernels --
// One Simdgroup Per Output Row"): for a row of affine codes with one scale per
// column group, sum_j w_j x_j with w_j = (code_j - Z)/Z * s equals, group by
// group, s * (sum_j (code_j - Z) x_j) / Z.  The codes enter only through a plain
// dot product with x; the scale and Z are applied once per 16-byte chunk (a
// chunk never straddles a group) and no f32 weight is ever formed.  gate_up
// reads the gate and up rows of an output index against the same input and
// writes SiLU(g) * u; down reads hidden.
//
// MI355X design (a redesign, not the page's one-simdgroup-per-row layout):
//
//  * Integer dot products.  Each block first quantises the input vector to
//    22-bit fixed point, one exponent per 16-byte chunk of columns
//    (X_j = rint(x_j * 2^k), |X_j| <= 2^22, so the error on a column is at most
//    2^-22 of the chunk's largest |x|), and splits every X_j into six signed
//    4-bit digits, X = sum_p 16^p t_p with t_p in [-8, 7].  The digits are laid
//    out as "planes" that line up nibble for nibble with the packed codes, so
//    one v_dot8_i32_i4 multiplies eight codes by eight digits and accumulates
//    exactly in int32.  A 4-bit code enters as code - 8 (XOR 8 of its nibble);
//    2-bit codes are split into even and odd columns with two masks.  That is
//    about 0.9 VALU instructions per code against about 2.3 for widening codes
//    to f32 and using FMA, which keeps the kernel on the HBM roofline rather
//    than the VALU one.  Per chunk, I = sum_j c_j X_j is exact and the chunk's
//    contribution is s * (float(I) * 2^-k / Z + beta), where beta restores the
//    code offset from the exact digit sum of the chunk.
//
//  * Registers instead of LDS for the vector.  A block of nw waves covers a
//    tile of rows; the chunks of a row are split into nw contiguous slices,
//    one per wave, and inside a wave LPR lanes share a row, so each lane always
//    reads the same column chunk(s) and keeps that chunk's digit planes in
//    registers for the whole kernel.  The row loop touches no LDS except the
//    final cross-wave reduction.
//
//  * Persistent, pipelined blocks.  The grid is sized to what is resident on
//    the device; each block walks its tiles in a grid stride and issues the
//    16-byte code loads and scale loads of the next tile before it computes the
//    current one, so HBM traffic and integer math overlap.
//
//  * Deterministic expert combine.  The down kernel runs blocks bound to one
//    expert; for each row tile, every expert's router-weighted rows are written
//    with agent-scope stores, and the last of the experts' blocks to finish the
//    tile (an agent-scope counter) adds the experts in ascending order.
#include "launch.h"

#include <cmath>
#include <cstdlib>
#include <map>
#include <mutex>
#include <tuple>

namespace smoe {
namespace {

// Per-chunk digit layout.  A chunk is 4 code dwords.  A 4-bit dword holds 8
// codes (one "octet" of columns); a 2-bit dword holds 16 codes, split into the
// even and the odd columns (two octets).  Each octet has 6 digit planes.
template <int BITS>
struct DigitLayout {
    static constexpr int kOctPerDw = BITS == 4 ? 1 : 2;
    static constexpr int kColsPerDw = 8 * kOctPerDw;
    static constexpr int kWordsPerDw = 6 * kOctPerDw;
    static constexpr int kWordsPerChunk = 4 * kWordsPerDw;   // 24 (4-bit) or 48 (2-bit)
};

constexpr uint32_t kDigitBias = 0x888888u;  // adds 8 to each of six nibbles

// Exponent k for a chunk whose largest |x| is m: m * 2^k lies in [2^21, 2^22).
__device__ __forceinline__ int chunk_shift(float m)
{
    return m > 0.0f ? 22 - __builtin_amdgcn_frexp_expf(m) : 0;
}

// Six signed 4-bit digits of X (|X| <= 2^22) packed in nibbles 0..5:
// X + 0x888888 has unsigned nibbles u_p, and t_p = u_p - 8 is the nibble u_p ^ 8
// read as a signed 4-bit value.
__device__ __forceinline__ uint32_t digits6(int X)
{
    return ((uint32_t)X + kDigitBias) ^ kDigitBias;
}

// Quantises one code dword's worth of columns (8 or 16 values) with shift k and
// writes its digit planes to `words` (6 or 12 dwords).  Returns sum of X.
template <int BITS>
__device__ __forceinline__ int make_planes(const float *v, int k, uint32_t *words)
{
    constexpr int OCT = DigitLayout<BITS>::kOctPerDw;
    int sum = 0;
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // 4-bit: columns in order; 2-bit: octet 0 = even columns, octet 1 = odd.
            const float val = v[OCT == 1 ? i : 2 * i + o];
            const int X = (int)__builtin_rintf(__builtin_ldexpf(val, k));
            sum += X;
            w[i] = digits6(X);
        }
#pragma unroll
        for (int p = 0; p < 6; ++p) {
            uint32_t plane = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) plane |= ((w[i] >> (4 * p)) & 0xFu) << (4 * i);
            words[6 * o + p] = plane;
        }
    }
    return sum;
}

// Block-wide: digit planes of a vector of n columns into LDS.
//   cmax   : [n / cols_per_chunk] largest |v| per chunk
//   dwsum  : [n / cols_per_dw]    sum of X per code dword
//   planes : [n / cols_per_dw][words_per_dw]
template <int BITS>
__device__ void build_planes(const float *vec, int n, uint32_t *planes, float *cmax, int *dwsum)
{
    using DL = DigitLayout<BITS>;
    constexpr int kColsPerChunk = 4 * DL::kColsPerDw;
    const int nch = n / kColsPerChunk, ndw = n / DL::kColsPerDw;
    for (int c = threadIdx.x; c < nch; c += blockDim.x) {
        const float4 *src = reinterpret_cast<const float4 *>(vec + (size_t)c * kColsPerChunk);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < kColsPerChunk / 4; ++i) {
            const float4 t = src[i];
            m = fmaxf(m, fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))));
        }
        cmax[c] = m;
    }
    __syncthreads();
    for (int q = threadIdx.x; q < ndw; q += blockDim.x) {
        const int k = chunk_shift(cmax[q >> 2]);
        float v[DL::kColsPerDw];
        const float4 *src = reinterpret_cast<const float4 *>(vec + (size_t)q * DL::kColsPerDw);
#pragma unroll
        for (int i = 0; i < DL::kColsPerDw / 4; ++i) {
            const float4 t = src[i];
            v[4 * i] = t.x; v[4 * i + 1] = t.y; v[4 * i + 2] = t.z; v[4 * i + 3] = t.w;
        }
        uint32_t w[DL::kWordsPerDw];
        dwsum[q] = make_planes<BITS>(v, k, w);
#pragma unroll
        for (int i = 0; i < DL::kWordsPerDw; ++i) planes[(size_t)q * DL::kWordsPerDw + i] = w[i];
    }
    __syncthreads();
}

// A lane's view of one chunk of the vector: its digit planes and the two
// epilogue constants, contribution = s * (float(I) * alpha + beta).
template <int BITS>
struct ChunkVec {
    uint32_t w[DigitLayout<BITS>::kWordsPerChunk];
    float alpha, beta;
};

template <int BITS>
__device__ __forceinline__ void load_chunk_vec(const uint32_t *planes, const float *cmax,
                                               const int *dwsum, int c, bool valid, ChunkVec<BITS> &cv)
{
    // Branch-free: an invalid chunk reads chunk 0 and is zeroed by selects (an
    // early return here makes the compiler spill the struct to scratch).
    using DL = DigitLayout<BITS>;
    const int cc = valid ? c : 0;
    const uint4 *src = reinterpret_cast<const uint4 *>(planes + (size_t)cc * DL::kWordsPerChunk);
#pragma unroll
    for (int i = 0; i < DL::kWordsPerChunk / 4; ++i) {
        const uint4 t = src[i];
        cv.w[4 * i] = valid ? t.x : 0u;
        cv.w[4 * i + 1] = valid ? t.y : 0u;
        cv.w[4 * i + 2] = valid ? t.z : 0u;
        cv.w[4 * i + 3] = valid ? t.w : 0u;
    }
    const int q = 4 * cc;
    const int k = chunk_shift(cmax[cc]);
    const int S = dwsum[q] + dwsum[q + 1] + dwsum[q + 2] + dwsum[q + 3];  // |S| <= 2^28
    const float sx = __builtin_ldexpf((float)S, -k);                        // sum of quantised x
    const float alpha = __builtin_ldexpf(QFormat<BITS>::kInvZ, -k);
    // 4-bit: code - Z = (code - 8) + 1/2, and the dot uses code - 8.
    // 2-bit: code - Z = code - 3/2, and the dot uses code itself.
    const float beta = BITS == 4 ? sx * (0.5f * QFormat<BITS>::kInvZ) : -sx;
    cv.alpha = valid ? alpha : 0.0f;
    cv.beta = valid ? beta : 0.0f;
}

// I = sum over the chunk of c_j * X_j, exact (|I| <= 2^30).  c_j = code - 8 at
// 4 bits, code at 2 bits.  Digit partial sums are combined mod 2^32, which is
// exact because the true I fits in int32.
template <int BITS>
__device__ __forceinline__ int chunk_idot(const uint4 q, const ChunkVec<BITS> &cv)
{
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
    int acc[6] = {0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if constexpr (BITS == 4) {
            const int c = (int)(d[m] ^ 0x88888888u);
#pragma unroll
            for (int p = 0; p < 6; ++p) acc[p] = __builtin_amdgcn_sdot8(c, (int)cv.w[6 * m + p], acc[p], false);
        } else {
            const int lo = (int)(d[m] & 0x33333333u);
            const int hi = (int)((d[m] >> 2) & 0x33333333u);
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                acc[p] = __builtin_amdgcn_sdot8(lo, (int)cv.w[12 * m + p], acc[p], false);
                acc[p] = __builtin_amdgcn_sdot8(hi, (int)cv.w[12 * m + 6 + p], acc[p], false);
            }
        }
    }
    uint32_t u = (uint32_t)acc[0];
#pragma unroll
    for (int p = 1; p < 6; ++p) u += (uint32_t)acc[p] << (4 * p);
    return (int)u;
}

template <int BITS>
__device__ __forceinline__ float chunk_contrib(const uint4 q, float s, const ChunkVec<BITS> &cv)
{
    return s * fmaf((float)chunk_idot<BITS>(q, cv), cv.alpha, cv.beta);
}

// Lane -> chunk mapping shared by both kernels.
template <int LPR, int NCH>
struct LaneMap {
    int lr, slot, c[NCH];
    bool valid[NCH];
    __device__ __forceinline__ explicit LaneMap(int cpr)
    {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
        const int sl = (cpr + nw - 1) / nw;
        lr = lane % LPR;
        slot = lane / LPR;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int cs = lr + LPR * k;
            c[k] = wave * sl + cs;
            valid[k] = cs < sl && c[k] < cpr;
        }
    }
};

// Code and scale registers of one tile of ITER row steps for M matrices.
template <int ITER, int NCH, int M>
struct TileRegs {
    uint4 q[ITER][NCH][M];
    float s[ITER][NCH][M];
};

// Dynamic LDS of both kernels:
//   red    f32 [2][nw][RB][M]   cross-wave partial rows, double-buffered by tile
//   cmax   f32 [nch4]           nch4 = chunks per row rounded up to 4
//   dwsum  i32 [ndw]            ndw = code dwords per row = 4 * chunks
//   planes u32 [ndw][words_per_dw]
template <int BITS>
__host__ __device__ size_t smem_bytes(int nw, int rb, int m, int cols)
{
    const size_t ndw = (size_t)cols / DigitLayout<BITS>::kColsPerDw;
    const size_t nch4 = ((ndw / 4) + 3) & ~size_t(3);
    return sizeof(float) * (2 * (size_t)nw * rb * m) + sizeof(float) * nch4 + sizeof(int) * ndw +
           sizeof(uint32_t) * ndw * DigitLayout<BITS>::kWordsPerDw;
}

template <int BITS>
struct SmemView {
    float *red;
    float *cmax;
    int *dwsum;
    uint32_t *planes;
    __device__ SmemView(unsigned char *base, int nw, int rb, int m, int cols)
    {
        const size_t ndw = (size_t)cols / DigitLayout<BITS>::kColsPerDw;
        const size_t nch4 = ((ndw / 4) + 3) & ~size_t(3);
        red = reinterpret_cast<float *>(base);
        cmax = red + 2 * (size_t)nw * rb * m;
        dwsum = reinterpret_cast<int *>(cmax + nch4);
        planes = reinterpret_cast<uint32_t *>(dwsum + ndw);
    }
};

template <int BITS, int LPR, int NCH, int ITER>
__global__ __launch_bounds__(512) void k_gate_up(const GateUpArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    constexpr int RS = 64 / LPR;
    constexpr int RB = RS * ITER;
    extern __shared__ __align__(16) unsigned char smem[];

    const int tid = threadIdx.x, wave = tid >> 6, nw = blockDim.x >> 6;
    const int cpr = a.d_model / CPC;
    const SmemView<BITS> sm(smem, nw, RB, 2, a.d_model);
    const size_t row_bytes = (size_t)a.d_model * BITS / 8;
    const int gpr = a.d_model / a.group;
    const int ntiles = a.n_experts * a.blocks_per_expert;
    const LaneMap<LPR, NCH> lm(cpr);
    int gi[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) gi[k] = lm.valid[k] ? lm.c[k] * CPC / a.group : 0;

    if (blockIdx.x == 0)
        for (int i = tid; i < a.n_counters; i += blockDim.x) a.counters[i] = 0;

    auto load_tile = [&](TileRegs<ITER, NCH, 2> &t, int tile) {
        const int e = tile / a.blocks_per_expert;
        const int row0 = (tile - e * a.blocks_per_expert) * RB;
        const QPtr G = a.gate[e], U = a.up[e];
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int r = row0 + lm.slot + RS * it;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                if (lm.valid[k] && r < a.d_ff) {
                    const size_t off = (size_t)r * row_bytes + (size_t)lm.c[k] * 16;
                    t.q[it][k][0] = load16(G.codes + off);
                    t.q[it][k][1] = load16(U.codes + off);
                    t.s[it][k][0] = G.scales[(size_t)r * gpr + gi[k]];
                    t.s[it][k][1] = U.scales[(size_t)r * gpr + gi[k]];
                } else {
                    t.q[it][k][0] = t.q[it][k][1] = make_uint4(0, 0, 0, 0);
                    t.s[it][k][0] = t.s[it][k][1] = 0.0f;
                }
            }
        }
    };

    int tile = blockIdx.x;
    TileRegs<ITER, NCH, 2> A, B;
    if (tile < ntiles) load_tile(A, tile);

    build_planes<BITS>(a.x, a.d_model, sm.planes, sm.cmax, sm.dwsum);
    ChunkVec<BITS> cv[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
        load_chunk_vec<BITS>(sm.planes, sm.cmax, sm.dwsum, lm.c[k], lm.valid[k], cv[k]);

    auto compute_tile = [&](const TileRegs<ITER, NCH, 2> &t, int tile, int buf) {
        float *rb = sm.red + buf * (nw * RB * 2);
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            float pg = 0.0f, pu = 0.0f;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                pg += chunk_contrib<BITS>(t.q[it][k][0], t.s[it][k][0], cv[k]);
                pu += chunk_contrib<BITS>(t.q[it][k][1], t.s[it][k][1], cv[k]);
            }
            pg = lane_group_sum<LPR>(pg);
            pu = lane_group_sum<LPR>(pu);
            if (lm.lr == 0) {
                const int i = wave * RB + lm.slot + RS * it;
                rb[2 * i] = pg;
                rb[2 * i + 1] = pu;
            }
        }
        __syncthreads();
        const int e = tile / a.blocks_per_expert;
        const int row0 = (tile - e * a.blocks_per_expert) * RB;
        for (int i = tid; i < RB; i += blockDim.x) {
            const int r = row0 + i;
            if (r < a.d_ff) {
                float g = 0.0f, u = 0.0f;
                for (int w = 0; w < nw; ++w) {
                    g += rb[2 * (w * RB + i)];
                    u += rb[2 * (w * RB + i) + 1];
                }
                a.hidden[(size_t)e * a.d_ff + r] = silu(g) * u;
            }
        }
    };

    // Two-stage pipeline: the next tile's loads are in flight while this one is
    // reduced.  The partial-row buffer alternates, so one barrier per tile
    // suffices (a buffer is rewritten only after the following tile's barrier).
    while (tile < ntiles) {
        const int t1 = tile + gridDim.x;
        if (t1 < ntiles) load_tile(B, t1);
        compute_tile(A, tile, 0);
        if (t1 >= ntiles) break;
        const int t2 = t1 + gridDim.x;
        if (t2 < ntiles) load_tile(A, t2);
        compute_tile(B, t1, 1);
        tile = t2;
    }
}

template <int BITS, int LPR, int NCH, int ITER>
__global__ __launch_bounds__(512) void k_down(const DownArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    constexpr int RS = 64 / LPR;
    constexpr int RB = RS * ITER;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_last;

    const int tid = threadIdx.x, wave = tid >> 6, nw = blockDim.x >> 6;
    const int E = a.n_experts;
    const int cpr = a.d_ff / CPC;
    const SmemView<BITS> sm(smem, nw, RB, 1, a.d_ff);

    // Blocks are bound to one expert: block b serves expert b % E and walks that
    // expert's row tiles with a stride of gridDim.x / E.
    const int e = blockIdx.x % E;
    const int bpe = gridDim.x / E;
    const size_t row_bytes = (size_t)a.d_ff * BITS / 8;
    const int gpr = a.d_ff / a.group;
    const QPtr D = a.down[e];
    const float rw = a.route_w ? a.route_w[e] : 1.0f;
    const LaneMap<LPR, NCH> lm(cpr);
    int gi[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) gi[k] = lm.valid[k] ? lm.c[k] * CPC / a.group : 0;

    auto load_tile = [&](TileRegs<ITER, NCH, 1> &t, int rb) {
        const int row0 = rb * RB;
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int r = row0 + lm.slot + RS * it;
#pragma unroll
            for (int k = 0; k < NCH; ++k) {
                if (lm.valid[k] && r < a.d_model) {
                    t.q[it][k][0] = load16(D.codes + (size_t)r * row_bytes + (size_t)lm.c[k] * 16);
                    t.s[it][k][0] = D.scales[(size_t)r * gpr + gi[k]];
                } else {
                    t.q[it][k][0] = make_uint4(0, 0, 0, 0);
                    t.s[it][k][0] = 0.0f;
                }
            }
        }
    };

    int rb = blockIdx.x / E;
    TileRegs<ITER, NCH, 1> A, B;
    if (rb < a.row_blocks) load_tile(A, rb);

    build_planes<BITS>(a.hidden + (size_t)e * a.d_ff, a.d_ff, sm.planes, sm.cmax, sm.dwsum);
    ChunkVec<BITS> cv[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
        load_chunk_vec<BITS>(sm.planes, sm.cmax, sm.dwsum, lm.c[k], lm.valid[k], cv[k]);

    auto compute_tile = [&](const TileRegs<ITER, NCH, 1> &t, int rb, int buf) {
        float *rbuf = sm.red + buf * (nw * RB);
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            float py = 0.0f;
#pragma unroll
            for (int k = 0; k < NCH; ++k) py += chunk_contrib<BITS>(t.q[it][k][0], t.s[it][k][0], cv[k]);
            py = lane_group_sum<LPR>(py);
            if (lm.lr == 0) rbuf[wave * RB + lm.slot + RS * it] = py;
        }
        __syncthreads();
        const int row0 = rb * RB;
        if (E == 1) {
            for (int i = tid; i < RB; i += blockDim.x) {
                const int r = row0 + i;
                if (r < a.d_model) {
                    float y = 0.0f;
                    for (int w = 0; w < nw; ++w) y += rbuf[w * RB + i];
                    a.out[r] = y * rw;
                }
            }
            return;
        }
        // Publish this expert's weighted rows with agent-scope stores (they go
        // through to the device-wide point of coherence, so no cache-wide
        // write-back is needed), wait for them, then count the expert in; the
        // last expert of the tile adds all experts in ascending order, reading
        // with agent-scope loads.
        for (int i = tid; i < RB; i += blockDim.x) {
            const int r = row0 + i;
            if (r < a.d_model) {
                float y = 0.0f;
                for (int w = 0; w < nw; ++w) y += rbuf[w * RB + i];
                __hip_atomic_store(a.partial + (size_t)e * a.d_model + r, y * rw, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            s_last = __hip_atomic_fetch_add(&a.counters[rb], 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == E - 1;
        __syncthreads();
        if (s_last) {
            for (int i = tid; i < RB; i += blockDim.x) {
                const int r = row0 + i;
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
    };

    while (rb < a.row_blocks) {
        const int r1 = rb + bpe;
        if (r1 < a.row_blocks) load_tile(B, r1);
        compute_tile(A, rb, 0);
        if (r1 >= a.row_blocks) break;
        const int r2 = r1 + bpe;
        if (r2 < a.row_blocks) load_tile(A, r2);
        compute_tile(B, r1, 1);
        rb = r2;
    }
}

// Resident blocks per CU for a kernel at a block size and LDS size, queried
// once per (kernel, block, lds).
int blocks_per_cu(const void *fn, int block, size_t lds)
{
    static std::mutex mu;
    static std::map<std::tuple<const void *, int, size_t>, int> cache;
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_tuple(fn, block, lds);
    auto it = cache.find(key);
    if (it != cache.end()) return it->second;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, block, lds) != hipSuccess || n < 1) n = 1;
    cache[key] = n;
    return n;
}

// Fewest rounds over the resident capacity, with the tiles spread evenly.
long balanced_grid(long tiles, long capacity)
{
    if (capacity < 1) capacity = 1;
    const long rounds = (tiles + capacity - 1) / capacity;
    return (tiles + rounds - 1) / rounds;
}

template <int BITS, int LPR, int NCH, int ITER>
hipError_t run_gate_up(const MapConfig &cfg, const GateUpArgs &a, int cus, hipStream_t st)
{
    constexpr int RB = (64 / LPR) * ITER;
    const int block = 64 * cfg.nw;
    const size_t lds = smem_bytes<BITS>(cfg.nw, RB, 2, a.d_model);
    const void *fn = reinterpret_cast<const void *>(&k_gate_up<BITS, LPR, NCH, ITER>);
    const long tiles = (long)a.n_experts * a.blocks_per_expert;
    const long grid = balanced_grid(tiles, (long)cus * blocks_per_cu(fn, block, lds));
    hipLaunchKernelGGL((k_gate_up<BITS, LPR, NCH, ITER>), dim3((unsigned)grid), dim3(block), lds, st, a);
    return hipGetLastError();
}

template <int BITS, int LPR, int NCH, int ITER>
hipError_t run_down(const MapConfig &cfg, const DownArgs &a, int cus, hipStream_t st)
{
    constexpr int RB = (64 / LPR) * ITER;
    const int block = 64 * cfg.nw;
    const size_t lds = smem_bytes<BITS>(cfg.nw, RB, 1, a.d_ff);
    const void *fn = reinterpret_cast<const void *>(&k_down<BITS, LPR, NCH, ITER>);
    const long cap = (long)cus * blocks_per_cu(fn, block, lds);
    const long per_expert = balanced_grid(a.row_blocks, cap / a.n_experts > 0 ? cap / a.n_experts : 1);
    hipLaunchKernelGGL((k_down<BITS, LPR, NCH, ITER>), dim3((unsigned)(per_expert * a.n_experts)),
                       dim3(block), lds, st, a);
    return hipGetLastError();
}

}  // namespace

// Instantiated mappings (blocks of at most 8 waves): lanes per row 2..32; one or
// two chunks per lane at 4 bits, one at 2 bits (a 2-bit chunk is already 64
// codes); 1 or 2 row steps per tile.
#define SMOE_QMAP_ITERS(F, B, L, N) F(B, L, N, 1) F(B, L, N, 2)
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
    // Two row steps per tile unless the matrix is too small to give a few
    // thousand waves work.
    const int rs = 64 / pick.lpr;
    const long tiles2 = (long)n_experts * ((rows + 2 * rs - 1) / (2 * rs));
    pick.iter = tiles2 * pick.nw >= 4096 ? 2 : 1;
    if (!qmap_instantiated(bits, pick.lpr, pick.nch, pick.iter)) return false;
    *cfg = pick;
    return true;
}

size_t qmap_lds_bytes(int bits, const MapConfig &cfg, int cols, int m)
{
    return bits == 4 ? smem_bytes<4>(cfg.nw, cfg.rows_per_block(), m, cols)
                     : smem_bytes<2>(cfg.nw, cfg.rows_per_block(), m, cols);
}

hipError_t launch_gate_up(int bits, const MapConfig &cfg, const GateUpArgs &a, int cus, hipStream_t st)
{
#define SMOE_RUN(B, L, N, I) \
    if (bits == B && cfg.lpr == L && cfg.nch == N && cfg.iter == I) return run_gate_up<B, L, N, I>(cfg, a, cus, st);
    SMOE_QMAP_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

hipError_t launch_down(int bits, const MapConfig &cfg, const DownArgs &a, int cus, hipStream_t st)
{
#define SMOE_RUN(B, L, N, I) \
    if (bits == B && cfg.lpr == L && cfg.nch == N && cfg.iter == I) return run_down<B, L, N, I>(cfg, a, cus, st);
    SMOE_QMAP_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

}  // namespace smoe
