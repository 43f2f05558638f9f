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
//  * Whole rows per wave.  lpr lanes (8..64, chosen per shape) share a row
//    and lane lr owns chunks lr, lr + lpr, ... of it, so a wave covers 64/lpr
//    rows per step; the row sum is a DPP / lane-shuffle reduction.  A lane
//    always reads the same column chunks, so it copies those chunks' digit
//    planes from LDS into registers once and the row loop touches no LDS and
//    has no barrier.
//
//  * Persistent, pipelined waves.  Each block first builds the digit planes of
//    the vector in LDS (one barrier); its waves then walk their row steps in a
//    grid stride, two steps of 16-byte code loads and scale loads always in
//    flight ahead of the step being reduced.  Loads are issued from clamped,
//    always valid addresses so that no lane's load is conditional.
//
//  * Deterministic expert combine.  down blocks are bound to one expert each.
//    A wave keeps its router-weighted rows in LDS and, at its end, adds each
//    row to a per-row 64-bit accumulator as an exact fixed-point term (2^-32
//    resolution) together with a count; integer addition does not depend on
//    the order of arrival, so the result is bitwise reproducible, and the
//    expert that completes a row's count writes the row and clears the word.
#include "launch.h"

#include <algorithm>
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

// The input vector of a block, one code dword's worth of columns (8 at 4 bits,
// 16 at 2 bits) per thread and group slot: thread t holds dword groups
// t, t + blockDim, ...  Loaded straight into registers at kernel start,
// before any code load is issued, so that waiting for it never waits for the
// (much slower) stream of code loads behind it.
template <int BITS, int GPT>
struct VecRegs {
    float v[GPT][DigitLayout<BITS>::kColsPerDw];
    bool ok[GPT];
};

template <int BITS, int GPT>
__device__ __forceinline__ void load_vec_regs(const float *vec, int n, VecRegs<BITS, GPT> &r)
{
    using DL = DigitLayout<BITS>;
    const int ndw = n / DL::kColsPerDw;
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
        const int q = threadIdx.x + g * blockDim.x;
        r.ok[g] = q < ndw;
        const float4 *src = reinterpret_cast<const float4 *>(vec + (size_t)(q < ndw ? q : ndw - 1) * DL::kColsPerDw);
#pragma unroll
        for (int i = 0; i < DL::kColsPerDw / 4; ++i) {
            const float4 t = src[i];
            r.v[g][4 * i] = t.x; r.v[g][4 * i + 1] = t.y; r.v[g][4 * i + 2] = t.z; r.v[g][4 * i + 3] = t.w;
        }
    }
}

// Largest value over the 4 lanes of an aligned quad (every lane gets it).
__device__ __forceinline__ float quad_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));  // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));  // quad_perm [2,3,0,1]
    return v;
}

// Block-wide: digit planes of the vector held in VecRegs, into LDS.  The four
// code dwords of a chunk belong to four consecutive threads of one wave, so the
// chunk's largest |v| is a quad reduction and one barrier suffices.
//   cmax   : [chunks] largest |v| per chunk
//   dwsum  : [ndw]    sum of X per code dword
//   planes : word w of chunk c at ((w / 4) * chunks + c) * 4 + w % 4, so that
//            consecutive lanes reading consecutive chunks with 16-byte loads hit
//            consecutive LDS addresses (no bank conflicts).
template <int BITS, int GPT>
__device__ void build_planes(const VecRegs<BITS, GPT> &r, int chunks, uint32_t *planes, float *cmax, int *dwsum)
{
    using DL = DigitLayout<BITS>;
#pragma unroll
    for (int g = 0; g < GPT; ++g) {
        const int q = threadIdx.x + g * blockDim.x;
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < DL::kColsPerDw; ++i) m = fmaxf(m, fabsf(r.v[g][i]));
        m = quad_max(m);  // blockDim and the group stride are multiples of 4
        if (!r.ok[g]) continue;
        const int c = q >> 2, dw = q & 3;
        if (dw == 0) cmax[c] = m;
        uint32_t w[DL::kWordsPerDw];
        dwsum[q] = make_planes<BITS>(r.v[g], chunk_shift(m), w);
#pragma unroll
        for (int i = 0; i < DL::kWordsPerDw; ++i) {
            const int word = dw * DL::kWordsPerDw + i;
            planes[((size_t)(word >> 2) * chunks + c) * 4 + (word & 3)] = w[i];
        }
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
__device__ __forceinline__ void load_chunk_vec(const uint32_t *planes, const float *cmax, const int *dwsum,
                                               int chunks, int c, bool valid, ChunkVec<BITS> &cv)
{
    // Branch-free: an invalid chunk reads chunk 0 and is zeroed by selects (an
    // early return here makes the compiler spill the struct to scratch).
    using DL = DigitLayout<BITS>;
    const int cc = valid ? c : 0;
#pragma unroll
    for (int i = 0; i < DL::kWordsPerChunk / 4; ++i) {
        const uint4 t = *reinterpret_cast<const uint4 *>(planes + ((size_t)i * chunks + cc) * 4);
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

// Lane -> chunk mapping of a wave that owns whole rows: lpr lanes (a power of
// two, 8..64, uniform over the launch) share a row, so a wave covers 64/lpr rows
// per step; lane lr owns chunks lr, lr + lpr, ..., lr + (NCH-1)*lpr.
template <int NCH>
struct RowLanes {
    int lr, slot, rs, c[NCH];
    bool valid[NCH];
    __device__ __forceinline__ RowLanes(int cpr, int lpr)
    {
        const int lane = threadIdx.x & 63;
        const int sh = __builtin_ctz(lpr);
        lr = lane & (lpr - 1);
        slot = lane >> sh;
        rs = 64 >> sh;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            c[k] = lr + lpr * k;
            valid[k] = c[k] < cpr;
        }
    }
};

// Sum over aligned groups of lpr lanes (lpr uniform): DPP inside 16-lane rows,
// lane shuffles across rows.
__device__ __forceinline__ float lane_group_sum_rt(float v, int lpr)
{
    if (lpr >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if (lpr >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if (lpr >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if (lpr >= 16) v += dpp<0x140>(v);  // row_mirror
    if (lpr >= 32) v += __shfl_xor(v, 16);
    if (lpr >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Code and scale registers of one wave step (one row per lane group) for M
// matrices.  Loads are issued unconditionally from clamped, always in-bounds
// addresses; `ok` marks the lanes whose load is real, and the scale of any
// other lane is replaced by zero when the step is computed.  (A divergent
// "load, else zero the registers" would make the compiler wait for the load
// before the zeroing write, which serialises the prefetch.)
template <int NCH, int M>
struct StepRegs {
    uint4 q[NCH][M];
    float s[NCH][M];
    bool ok[NCH];
};

// Dynamic LDS: the input vector's digit planes,
//   cmax   f32 [chunks4]        chunks rounded up to 4
//   dwsum  i32 [ndw]            ndw = code dwords per row = 4 * chunks
//   planes u32 [ndw * words_per_dw]
template <int BITS>
__host__ __device__ size_t plane_lds_bytes(int cols)
{
    const size_t ndw = (size_t)cols / DigitLayout<BITS>::kColsPerDw;
    const size_t chunks4 = ((ndw / 4) + 3) & ~size_t(3);
    return sizeof(float) * chunks4 + sizeof(int) * ndw + sizeof(uint32_t) * ndw * DigitLayout<BITS>::kWordsPerDw;
}

template <int BITS>
struct PlaneLds {
    float *cmax;
    int *dwsum;
    uint32_t *planes;
    int chunks;
    __device__ PlaneLds(unsigned char *base, int cols)
    {
        const size_t ndw = (size_t)cols / DigitLayout<BITS>::kColsPerDw;
        const size_t chunks4 = ((ndw / 4) + 3) & ~size_t(3);
        chunks = (int)(ndw / 4);
        cmax = reinterpret_cast<float *>(base);
        dwsum = reinterpret_cast<int *>(cmax + chunks4);
        planes = reinterpret_cast<uint32_t *>(dwsum + ndw);
    }
};

// Code dwords of a vector of up to kMaxQCols columns per thread of a 512-thread block.
constexpr int kBlockThreads = 512;
constexpr int kMaxQCols = 8192;
template <int BITS>
constexpr int kGroupsPerThread = (kMaxQCols / DigitLayout<BITS>::kColsPerDw + kBlockThreads - 1) / kBlockThreads;

// gate_up: hidden[e][i] = SiLU(G_e x)[i] * (U_e x)[i] for every expert.
//
// Blocks are persistent; each block builds the digit planes of x in LDS once,
// every lane copies the planes of its chunks into registers, and from then on
// each wave streams whole rows on its own: no LDS and no barrier in the row
// loop, the codes and scales of the next step are in flight while a step is
// reduced.  Wave steps are numbered expert by expert; global wave w takes steps
// w, w + W, w + 2W, ... of the E * ceil(d_ff / rs) steps.
template <int BITS, int NCH>
__global__ __launch_bounds__(512) void k_gate_up(const DecodeArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    extern __shared__ __align__(16) unsigned char smem[];
    const int nw = blockDim.x >> 6;
    const int cpr = a.d_model / CPC;
    const RowLanes<NCH> rl(cpr, a.lpr_g);
    const PlaneLds<BITS> lds(smem, a.d_model);
    const size_t row_bytes = (size_t)a.d_model * BITS / 8;
    const int gpr = a.d_model / a.group;
    const int spe = (a.d_ff + rl.rs - 1) / rl.rs;  // wave steps per expert
    const int nsteps = a.n_experts * spe;
    const int W = gridDim.x * nw;
    int gi[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) gi[k] = rl.valid[k] ? rl.c[k] * CPC / a.group : 0;

    auto load_step = [&](StepRegs<NCH, 2> &t, int step) {
        const int e = step / spe;
        const int r = (step - e * spe) * rl.rs + rl.slot;
        const int rc = r < a.d_ff ? r : a.d_ff - 1;
        const QPtr G = a.gate[e], U = a.up[e];
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int cc = rl.valid[k] ? rl.c[k] : 0;
            const size_t off = (size_t)rc * row_bytes + (size_t)cc * 16;
            t.q[k][0] = load16(G.codes + off);
            t.q[k][1] = load16(U.codes + off);
            t.s[k][0] = G.scales[(size_t)rc * gpr + gi[k]];
            t.s[k][1] = U.scales[(size_t)rc * gpr + gi[k]];
            t.ok[k] = rl.valid[k] && r < a.d_ff;
        }
    };

    // Order of the prologue: the input vector's loads, then the first two steps'
    // code loads, then the digit planes (which wait only for the vector).  The
    // wave index is made explicitly scalar, so that the step, the expert and the
    // expert's matrix pointers live in SGPRs (scalar loads from the kernel
    // arguments) rather than behind a vector load in front of every step.
    VecRegs<BITS, kGroupsPerThread<BITS>> xr;
    load_vec_regs<BITS>(a.x, a.d_model, xr);
    int step = blockIdx.x * nw + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    StepRegs<NCH, 2> A, B;
    if (step < nsteps) load_step(A, step);
    if (step + W < nsteps) load_step(B, step + W);

    build_planes<BITS>(xr, lds.chunks, lds.planes, lds.cmax, lds.dwsum);
    ChunkVec<BITS> cv[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
        load_chunk_vec<BITS>(lds.planes, lds.cmax, lds.dwsum, lds.chunks, rl.c[k], rl.valid[k], cv[k]);

    auto compute_step = [&](const StepRegs<NCH, 2> &t, int step) {
        float g = 0.0f, u = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            g += chunk_contrib<BITS>(t.q[k][0], t.ok[k] ? t.s[k][0] : 0.0f, cv[k]);
            u += chunk_contrib<BITS>(t.q[k][1], t.ok[k] ? t.s[k][1] : 0.0f, cv[k]);
        }
        g = lane_group_sum_rt(g, a.lpr_g);
        u = lane_group_sum_rt(u, a.lpr_g);
        const int e = step / spe;
        const int r = (step - e * spe) * rl.rs + rl.slot;
        if (rl.lr == 0 && r < a.d_ff) a.hidden[(size_t)e * a.d_ff + r] = silu(g) * u;
    };

    while (step < nsteps) {
        const int s1 = step + W;
        compute_step(A, step);
        if (s1 >= nsteps) break;
        const int s2 = s1 + W;
        if (s2 < nsteps) load_step(A, s2);
        compute_step(B, s1);
        const int s3 = s2 + W;
        if (s3 < nsteps) load_step(B, s3);
        step = s2;
    }
}

// down: out = sum_e r_e * (D_e hidden_e).
//
// Blocks are bound to one expert (block b serves expert b % E) and build that
// expert's hidden digit planes in LDS once; waves then stream whole rows on
// their own as in gate_up.  With one expert the rows go straight to out.  With
// several, the experts' router-weighted rows are summed exactly: each
// contribution is rounded to a multiple of 2^-32 (an error of at most 2^-33 per
// term, far below f32 resolution for outputs of order one, and at most
// E * 2^-33 in absolute terms) and added as a 64-bit integer to a per-row
// accumulator whose top five bits count the experts in.  Integer addition is
// associative, so the sum does not depend on the order in which experts
// arrive: the result is bitwise reproducible.  The expert whose addition
// completes the count converts the exact sum to f32 once, writes out, and
// re-zeroes the accumulator for the next call.  One atomic per row and
// expert, deferred to the end of the wave, is the only cross-block traffic.
// A contribution of magnitude 2^20 or more does not fit the accumulator; it is
// added as a NaN marker so that the row comes out NaN rather than wrong.
constexpr int kAccCountShift = 59;
constexpr unsigned long long kAccBias = 1ull << 52;    // keeps every term non-negative
constexpr unsigned long long kAccNan = 1ull << 58;     // set in the sum when a term overflowed

__device__ __forceinline__ unsigned long long acc_term(float v)
{
    const double t = (double)v * 4294967296.0;  // v * 2^32
    if (!(fabs(t) < 4503599627370496.0))        // |v| < 2^20 (also false for NaN)
        return (1ull << kAccCountShift) | kAccNan;
    return (1ull << kAccCountShift) + kAccBias + (unsigned long long)(long long)__builtin_rint(t);
}

__device__ __forceinline__ float acc_value(unsigned long long sum, int n)
{
    if (sum & kAccNan) return __builtin_nanf("");
    const unsigned long long mag = sum & ((1ull << kAccCountShift) - 1);
    const long long fixed = (long long)(mag - (unsigned long long)n * kAccBias);
    return (float)((double)fixed * (1.0 / 4294967296.0));
}

template <int BITS, int NCH>
__global__ __launch_bounds__(512) void k_down(const DecodeArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    extern __shared__ __align__(16) unsigned char smem[];
    const int nw = blockDim.x >> 6, lane = threadIdx.x & 63;
    const int E = a.n_experts;
    const int cpr = a.d_ff / CPC;
    const RowLanes<NCH> rl(cpr, a.lpr_d);
    const PlaneLds<BITS> lds(smem, a.d_ff);
    const size_t row_bytes = (size_t)a.d_ff * BITS / 8;
    const int gpr = a.d_ff / a.group;
    const int e = blockIdx.x % E;
    const int bpe = gridDim.x / E;                 // blocks per expert
    const int We = bpe * nw;                       // waves per expert
    const int nsteps = (a.d_model + rl.rs - 1) / rl.rs;
    const int w0 = (blockIdx.x / E) * nw + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const QPtr D = a.down[e];
    const float rw = a.route_w ? a.route_w[e] : 1.0f;
    // This wave's router-weighted rows, kept until the deferred combine.
    float *mine = reinterpret_cast<float *>(smem + plane_lds_bytes<BITS>(a.d_ff)) +
                  (threadIdx.x >> 6) * a.dn_rows_per_wave;
    int gi[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) gi[k] = rl.valid[k] ? rl.c[k] * CPC / a.group : 0;

    auto load_step = [&](StepRegs<NCH, 1> &t, int step) {
        const int r = step * rl.rs + rl.slot;
        const int rc = r < a.d_model ? r : a.d_model - 1;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            const int cc = rl.valid[k] ? rl.c[k] : 0;
            t.q[k][0] = load16(D.codes + (size_t)rc * row_bytes + (size_t)cc * 16);
            t.s[k][0] = D.scales[(size_t)rc * gpr + gi[k]];
            t.ok[k] = rl.valid[k] && r < a.d_model;
        }
    };

    if ((int)blockIdx.x >= bpe * E) return;  // whole block idle: no barrier follows for it
    VecRegs<BITS, kGroupsPerThread<BITS>> hr;
    load_vec_regs<BITS>(a.hidden + (size_t)e * a.d_ff, a.d_ff, hr);
    int step = w0;
    StepRegs<NCH, 1> A, B;
    if (step < nsteps) load_step(A, step);
    if (step + We < nsteps) load_step(B, step + We);

    build_planes<BITS>(hr, lds.chunks, lds.planes, lds.cmax, lds.dwsum);
    ChunkVec<BITS> cv[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
        load_chunk_vec<BITS>(lds.planes, lds.cmax, lds.dwsum, lds.chunks, rl.c[k], rl.valid[k], cv[k]);

    auto compute_step = [&](const StepRegs<NCH, 1> &t, int step) {
        float y = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) y += chunk_contrib<BITS>(t.q[k][0], t.ok[k] ? t.s[k][0] : 0.0f, cv[k]);
        y = lane_group_sum_rt(y, a.lpr_d);
        const int r = step * rl.rs + rl.slot;
        if (rl.lr == 0 && r < a.d_model) {
            if (E == 1)
                a.out[r] = y * rw;
            else
                mine[((step - w0) / We) * rl.rs + rl.slot] = y * rw;
        }
    };

    while (step < nsteps) {
        const int s1 = step + We;
        compute_step(A, step);
        if (s1 >= nsteps) break;
        const int s2 = s1 + We;
        if (s2 < nsteps) load_step(A, s2);
        compute_step(B, s1);
        const int s3 = s2 + We;
        if (s3 < nsteps) load_step(B, s3);
        step = s2;
    }

    if (E > 1) {
        // One 64-bit addition per row of this wave, all rows at once (lane j
        // takes the wave's j-th row); the lane that completes a row writes it.
        // The rows were stored to LDS by lanes of this same wave, whose LDS
        // accesses complete in order.
        __builtin_amdgcn_wave_barrier();
        const int my_steps = w0 < nsteps ? (nsteps - 1 - w0) / We + 1 : 0;
        const int my_rows = my_steps * rl.rs;
        for (int j0 = 0; j0 < my_rows; j0 += 64) {
            const int j = j0 + lane;
            if (j < my_rows) {
                const int r = (w0 + (j / rl.rs) * We) * rl.rs + (j % rl.rs);
                if (r < a.d_model) {
                    const unsigned long long term = acc_term(mine[j]);
                    const unsigned long long sum =
                        __hip_atomic_fetch_add(a.row_acc + r, term, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + term;
                    if ((int)(sum >> kAccCountShift) == E) {
                        a.out[r] = acc_value(sum, E);
                        __hip_atomic_store(a.row_acc + r, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            }
        }
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
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, fn, block, lds) != hipSuccess || n < 1) n = 0;
    cache[key] = n;
    return n;
}

template <int BITS, int NCH>
hipError_t run_gate_up(const DecodePlan &p, const DecodeArgs &a, int cus, hipStream_t st)
{
    const int block = 64 * p.nw;
    const size_t lds = plane_lds_bytes<BITS>(a.d_model);
    const void *fn = reinterpret_cast<const void *>(&k_gate_up<BITS, NCH>);
    const long cap = (long)cus * blocks_per_cu(fn, block, lds);
    if (cap < 1) return hipErrorInvalidConfiguration;
    const long steps = (long)a.n_experts * ((a.d_ff + 64 / p.lpr_g - 1) / (64 / p.lpr_g));
    const long grid = std::max(1L, std::min(cap, (steps + p.nw - 1) / p.nw));
    hipLaunchKernelGGL((k_gate_up<BITS, NCH>), dim3((unsigned)grid), dim3(block), lds, st, a);
    return hipGetLastError();
}

template <int BITS, int NCH>
hipError_t run_down(const DecodePlan &p, DecodeArgs a, int cus, hipStream_t st)
{
    const int block = 64 * p.nw;
    const void *fn = reinterpret_cast<const void *>(&k_down<BITS, NCH>);
    const size_t planes = (plane_lds_bytes<BITS>(a.d_ff) + 15) & ~size_t(15);
    // Resident blocks: the occupancy query's answer, but at most two blocks of
    // this size per CU (more were measured not to be co-resident, which puts a
    // second round of blocks after the first).
    const long cap = (long)cus * std::min(2, blocks_per_cu(fn, block, planes + 4096));
    if (cap < a.n_experts) return hipErrorInvalidConfiguration;
    const int rs = 64 / p.lpr_d;
    const long steps = (a.d_model + rs - 1) / rs;
    const long per_expert = std::max(1L, std::min(cap / a.n_experts, (steps + p.nw - 1) / p.nw));
    const long waves = per_expert * p.nw;
    a.dn_rows_per_wave = (int)(((steps + waves - 1) / waves) * rs);
    const size_t lds = planes + (a.n_experts > 1 ? (size_t)p.nw * a.dn_rows_per_wave * sizeof(float) : 0);
    hipLaunchKernelGGL((k_down<BITS, NCH>), dim3((unsigned)(per_expert * a.n_experts)), dim3(block), lds, st, a);
    return hipGetLastError();
}

// Lanes per row and chunks per lane for whole-row waves over `cpr` chunks:
// as few idle lanes as possible, then as few plane registers as possible.
bool row_map(int bits, int cpr, int *lpr_out, int *nch_out)
{
    const int max_nch = bits == 4 ? 4 : 2;
    double best = 1e30;
    int bl = 0, bn = 0;
    for (int nch = 1; nch <= max_nch; ++nch)
        for (int lpr = 8; lpr <= 64; lpr *= 2) {
            if (lpr * nch < cpr) continue;
            const double waste = 1.0 - (double)cpr / ((double)lpr * nch);
            const double pen = 4.0 * waste + 0.5 * (nch - 1) * (bits == 4 ? 1.0 : 2.0);
            if (pen < best) {
                best = pen;
                bl = lpr;
                bn = nch;
            }
        }
    if (!bl) return false;
    *lpr_out = bl;
    *nch_out = bn;
    return true;
}

}  // namespace

bool plan_decode(int mode, int bits, int d_model, int d_ff, int n_experts, DecodePlan *p)
{
    (void)n_experts;
    const int cpc = 128 / bits;
    DecodePlan q{mode, 8, 64, 1, 64, 1, d_model, d_ff};
    if (mode != kDownOnly && !row_map(bits, d_model / cpc, &q.lpr_g, &q.nch_g)) return false;
    if (mode != kGateUpOnly && !row_map(bits, d_ff / cpc, &q.lpr_d, &q.nch_d)) return false;
    *p = q;
    return true;
}

int decode_rows_per_tile(int lpr) { return 64 / lpr; }

hipError_t launch_gate_up(int bits, const DecodePlan &p, const DecodeArgs &a, int cus, hipStream_t st)
{
#define SMOE_RUN(B, N) if (bits == B && p.nch_g == N) return run_gate_up<B, N>(p, a, cus, st);
    SMOE_RUN(4, 1) SMOE_RUN(4, 2) SMOE_RUN(4, 3) SMOE_RUN(4, 4) SMOE_RUN(2, 1) SMOE_RUN(2, 2)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

hipError_t launch_down(int bits, const DecodePlan &p, const DecodeArgs &a, int cus, hipStream_t st)
{
#define SMOE_RUN(B, N) if (bits == B && p.nch_d == N) return run_down<B, N>(p, a, cus, st);
    SMOE_RUN(4, 1) SMOE_RUN(4, 2) SMOE_RUN(4, 3) SMOE_RUN(4, 4) SMOE_RUN(2, 1) SMOE_RUN(2, 2)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

}  // namespace smoe
