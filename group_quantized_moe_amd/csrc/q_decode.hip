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
//  * Whole rows per wave.  LPR lanes (16, 32 or 64, a template parameter)
//    share a row and lane lr owns chunks lr, lr + LPR, ... of it, so a wave
//    covers 64/LPR rows per step and the row sum is a DPP reduction.  A lane
//    always reads the same column chunks, so it copies those chunks' digit
//    planes from LDS into registers once and the row loop touches no LDS and
//    has no barrier.
//
//  * Persistent waves, one step of loads in flight each.  Each block first
//    loads the vector and waits for it, then issues its waves' first steps and
//    builds the digit planes of the vector in LDS (one barrier); each wave then
//    walks a contiguous range of row steps with the next step's 16-byte code
//    loads and scale loads in flight while it reduces the current one (more
//    steps in flight per wave measured slower: the waves of a CU already keep
//    the memory system busy).  Loads come from a uniform base plus a 32-bit lane
//    offset; nothing is loaded past a wave's last step.
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

// 8x8 transpose of nibbles: on return nibble i of w[p] is what nibble p of
// w[i] was.  Three stages swap ever larger blocks between word pairs:
// nibbles between words (2j, 2j+1) with bitfield inserts, then bytes between
// (j, j+2) and 16-bit halves between (j, j+4) with byte permutes.
__device__ __forceinline__ void transpose_nibbles(uint32_t w[8])
{
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
        const uint32_t a = w[j], b = w[j + 1];
        w[j] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
        w[j + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int j = q + (q & 2);   // pairs (0,2) (1,3) (4,6) (5,7)
        const uint32_t a = w[j], b = w[j + 2];
        w[j] = __builtin_amdgcn_perm(b, a, 0x06020400u);      // a.byte0 b.byte0 a.byte2 b.byte2
        w[j + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);  // a.byte1 b.byte1 a.byte3 b.byte3
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t a = w[j], b = w[j + 4];
        w[j] = __builtin_amdgcn_perm(b, a, 0x05040100u);      // low halves
        w[j + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);  // high halves
    }
}

// Quantises one code dword's worth of columns (8 or 16 values) with shift k and
// writes its digit planes to `words` (6 or 12 dwords).  Returns sum of X.
//
// X = rint(v * 2^k) with |X| <= 2^22: adding 1.5 * 2^23 to v * 2^k (|v * 2^k| <
// 2^22) lands in [2^23, 2^24), where floats are the integers, so the one
// rounding of the add is the rounding to the nearest integer and the result's
// bits are 0x4B400000 + X.  X + 0x888888 is then positive and below 2^24, its
// six nibbles u_p = t_p + 8 hold the signed digits of X = sum_p 16^p t_p,
// t_p in [-8, 7], and u_p ^ 8 is t_p as a signed 4-bit value.  The nibble
// transpose gathers digit p of the 8 columns into plane p, nibble i = column i.
template <int BITS>
__device__ __forceinline__ int make_planes(const float *v, int k, uint32_t *words)
{
    constexpr int OCT = DigitLayout<BITS>::kOctPerDw;
    constexpr uint32_t kMagic = 0x4B400000u;   // bits of 1.5 * 2^23
    uint32_t bsum = 0;
#pragma unroll
    for (int o = 0; o < OCT; ++o) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            // 4-bit: columns in order; 2-bit: octet 0 = even columns, octet 1 = odd.
            const float val = v[OCT == 1 ? i : 2 * i + o];
            const uint32_t bits = __float_as_uint(__builtin_ldexpf(val, k) + 12582912.0f);
            bsum += bits;
            w[i] = bits + (kDigitBias - kMagic);
        }
        transpose_nibbles(w);
#pragma unroll
        for (int p = 0; p < 6; ++p) words[6 * o + p] = w[p] ^ 0x88888888u;
    }
    return (int)(bsum - (uint32_t)(8 * OCT) * kMagic);
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
__device__ __forceinline__ uint32_t quad_umax(uint32_t v)
{
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, true));  // quad_perm [1,0,3,2]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, true));  // quad_perm [2,3,0,1]
    return v;
}

// Bit pattern of the largest |v| of a chunk: every finite value is below
// 0x7f800000, an infinity equals it and a NaN lies above it, so the chunk is
// finite exactly when the result is below 0x7f800000.
constexpr uint32_t kInfBits = 0x7f800000u;

// Digit planes of one code dword of a vector (its 8 or 16 values in v) into
// LDS.  The four code dwords of a chunk belong to four consecutive lanes, which
// must all call this together (the chunk's largest |v| is a quad reduction);
// `ok` only gates the stores.
//   cmax   : [chunks] largest |v| per chunk (an infinity or NaN if the chunk
//            holds a non-finite value)
//   dwsum  : [ndw]    sum of X per code dword
//   planes : word w of chunk c at ((w / 4) * chunks + c) * 4 + w % 4, so that
//            consecutive lanes reading consecutive chunks with 16-byte loads hit
//            consecutive LDS addresses (no bank conflicts).
template <int BITS>
__device__ __forceinline__ void plane_dword(const float *v, int q, bool ok, int chunks, uint32_t *planes,
                                            float *cmax, int *dwsum)
{
    using DL = DigitLayout<BITS>;
    uint32_t mb = 0;
#pragma unroll
    for (int i = 0; i < DL::kColsPerDw; ++i) mb = max(mb, __float_as_uint(v[i]) & 0x7fffffffu);
    mb = quad_umax(mb);
    if (!ok) return;
    const int c = q >> 2, dw = q & 3;
    const bool fin = mb < kInfBits;
    if (dw == 0) cmax[c] = __uint_as_float(mb);
    // A non-finite chunk is quantised as zeros; its epilogue constant is NaN.
    float vf[DL::kColsPerDw];
#pragma unroll
    for (int i = 0; i < DL::kColsPerDw; ++i) vf[i] = fin ? v[i] : 0.0f;
    uint32_t w[DL::kWordsPerDw];
    dwsum[q] = make_planes<BITS>(vf, fin ? chunk_shift(__uint_as_float(mb)) : 0, w);
#pragma unroll
    for (int i = 0; i < DL::kWordsPerDw; ++i) {
        const int word = dw * DL::kWordsPerDw + i;
        planes[((size_t)(word >> 2) * chunks + c) * 4 + (word & 3)] = w[i];
    }
}

// Block-wide: digit planes of the vector held in VecRegs, into LDS, then one
// barrier.  blockDim and the group stride are multiples of 4, so the four
// dwords of a chunk sit in four consecutive threads of one wave.
template <int BITS, int GPT>
__device__ void build_planes(const VecRegs<BITS, GPT> &r, int chunks, uint32_t *planes, float *cmax, int *dwsum)
{
#pragma unroll
    for (int g = 0; g < GPT; ++g)
        plane_dword<BITS>(r.v[g], threadIdx.x + g * blockDim.x, r.ok[g], chunks, planes, cmax, dwsum);
    __syncthreads();
}

// A lane's view of one chunk of the vector: its digit planes and the
// epilogue constants, contribution = s * ldexp(float(I) / Z + beta, -k).
// Scaling by 2^-k last keeps a chunk of tiny values (k above 126) from
// underflowing before its sum is formed.
template <int BITS>
struct ChunkVec {
    uint32_t w[DigitLayout<BITS>::kWordsPerChunk];
    float beta;
    int nk;   // -k
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
    const float m = cmax[cc];
    const bool fin = __float_as_uint(m) < kInfBits;
    const int k = fin ? chunk_shift(m) : 0;
    const int S = dwsum[q] + dwsum[q + 1] + dwsum[q + 2] + dwsum[q + 3];  // |S| <= 2^28
    // In units of 2^-k, the chunk's sum of (code - Z) X / Z is I / Z + beta:
    // 4-bit: code - Z = (code - 8) + 1/2 and the dot uses code - 8, so beta = S / (2Z);
    // 2-bit: (code - Z) / Z = code / Z - 1 and the dot uses code itself, so beta = -S.
    const float beta = BITS == 4 ? (float)S * (0.5f * QFormat<BITS>::kInvZ) : -(float)S;
    cv.beta = valid ? (fin ? beta : __builtin_nanf("")) : 0.0f;
    cv.nk = valid ? -k : 0;
}

// I = sum over the chunk of c_j * X_j, exact (|I| <= 2^30).  c_j = code - 8 at
// 4 bits, code at 2 bits.  Digit partial sums are combined mod 2^32, which is
// exact because the true I fits in int32.
// Signed 4-bit dot of 8 lanes' nibbles without an accumulator input (the
// non-accumulating form, so that no register has to be zeroed first).
__device__ __forceinline__ int dot8_first(int a, int b)
{
    int r;
    asm("v_dot8_i32_i4 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

template <int BITS>
__device__ __forceinline__ int chunk_idot(const uint4 q, const ChunkVec<BITS> &cv)
{
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
    int acc[6];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        if constexpr (BITS == 4) {
            const int c = (int)(d[m] ^ 0x88888888u);
#pragma unroll
            for (int p = 0; p < 6; ++p)
                acc[p] = m == 0 ? dot8_first(c, (int)cv.w[p])
                                : __builtin_amdgcn_sdot8(c, (int)cv.w[6 * m + p], acc[p], false);
        } else {
            const int lo = (int)(d[m] & 0x33333333u);
            const int hi = (int)((d[m] >> 2) & 0x33333333u);
#pragma unroll
            for (int p = 0; p < 6; ++p) {
                acc[p] = m == 0 ? dot8_first(lo, (int)cv.w[p])
                                : __builtin_amdgcn_sdot8(lo, (int)cv.w[12 * m + p], acc[p], false);
                acc[p] = __builtin_amdgcn_sdot8(hi, (int)cv.w[12 * m + 6 + p], acc[p], false);
            }
        }
    }
    // I = sum_p 16^p acc_p, by Horner (one shift-add per digit).
    uint32_t u = (uint32_t)acc[5];
#pragma unroll
    for (int p = 4; p >= 0; --p) u = (u << 4) + (uint32_t)acc[p];
    return (int)u;
}

template <int BITS>
__device__ __forceinline__ float chunk_contrib(const uint4 q, float s, const ChunkVec<BITS> &cv)
{
    return s * __builtin_ldexpf(fmaf((float)chunk_idot<BITS>(q, cv), QFormat<BITS>::kInvZ, cv.beta), cv.nk);
}

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

// Lanes of a whole-row wave: LPR lanes share a row and lane lr owns chunks
// lr, lr + LPR, ..., so that each 16-byte load instruction of a wave reads one
// contiguous run of its rows.  Chunks past the row end are idle: their digit
// planes and epilogue constants are zero and their loads read a valid chunk.
template <int NCH, int LPR>
struct RowLanes {
    static constexpr int kRows = 64 / LPR;   // rows per step
    int lr, slot;
    int c[NCH];
    bool valid[NCH];
    unsigned coff[NCH];   // 16 * chunk: code bytes from the start of the row
    unsigned soff[NCH];   // 4 * group of the chunk: scale bytes from the start of the row
    __device__ __forceinline__ RowLanes(int cpr, int cpc, int group)
    {
        const int lane = threadIdx.x & 63;
        lr = lane & (LPR - 1);
        slot = lane / LPR;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            c[k] = lr + LPR * k;
            valid[k] = c[k] < cpr;
            const int cc = valid[k] ? c[k] : cpr - 1;
            coff[k] = 16u * cc;
            soff[k] = 4u * (unsigned)(cc * cpc / group);
        }
    }
    // Lane that holds the row sum after group_sum<LPR>.
    __device__ __forceinline__ bool writer() const { return LPR >= 32 ? lr == LPR - 1 : lr == 0; }
};

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_rows(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}

// Sum over aligned groups of LPR lanes, all in DPP (no LDS).  For LPR <= 16
// every lane of a group gets the sum; for 32 and 64 it lands in the group's
// last lane (row_bcast:15 adds row 0 into row 1 and row 2 into row 3,
// row_bcast:31 adds lane 31 into rows 2 and 3).
template <int LPR>
__device__ __forceinline__ float group_sum(float v)
{
    if constexpr (LPR >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (LPR >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (LPR >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (LPR >= 16) v += dpp<0x140>(v);  // row_mirror
    if constexpr (LPR >= 32) v += dpp_rows<0x142, 0xA>(v);
    if constexpr (LPR >= 64) v += dpp_rows<0x143, 0xC>(v);
    return v;
}

// SiLU(t) = t / (1 + e^-t) with the hardware base-2 exponential and
// reciprocal (each within about one ulp): a few ulp overall, and the right
// limits (t for large t, -0 for very negative t, NaN for NaN).
__device__ __forceinline__ float silu_hw(float t)
{
    const float e = __builtin_amdgcn_exp2f(t * -1.44269504088896341f);
    return t * __builtin_amdgcn_rcpf(1.0f + e);
}

// Code and scale registers of one step: NCH chunks of M matrices for the
// lane's row.  Scales are kept as loaded (f32 bits, or binary16 bits in the
// low half) and widened where they are used: a widening next to the load
// would wait for the load right there.
template <int NCH, int M>
struct Stage {
    uint4 q[NCH][M];
    uint32_t s[NCH][M];
};

template <int SB>
__device__ __forceinline__ float stage_scale(uint32_t bits)
{
    if constexpr (SB == 4)
        return __uint_as_float(bits);
    else
        return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

// Loads of one stage: the lane's row is row0 + slot, clamped to the last row
// (a partial last step re-reads it; its results are never stored).
// Scales are f32 (SB = 4) or IEEE binary16 (SB = 2, widened exactly to f32;
// byte offsets are half the f32 ones).
template <int NCH, int LPR, int M, int SB>
__device__ __forceinline__ void load_stage(Stage<NCH, M> &t, const uint8_t *const *codes, const void *const *scales,
                                           const RowLanes<NCH, LPR> &ln, int row0, int rows, unsigned row_bytes,
                                           int gpr)
{
    const unsigned r = (unsigned)min(row0 + ln.slot, rows - 1);
    const unsigned crow = r * row_bytes, srow = r * (unsigned)gpr * 4u;
#pragma unroll
    for (int m = 0; m < M; ++m) {
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            t.q[k][m] = *reinterpret_cast<const uint4 *>(codes[m] + (crow + ln.coff[k]));
            const uint8_t *sb = reinterpret_cast<const uint8_t *>(scales[m]);
            if constexpr (SB == 4)
                t.s[k][m] = *reinterpret_cast<const uint32_t *>(sb + (srow + ln.soff[k]));
            else
                t.s[k][m] = *reinterpret_cast<const uint16_t *>(sb + ((srow + ln.soff[k]) >> 1));
        }
    }
}

// Row sums of matrix m for the lane's chunks (before the cross-lane sum).
template <int BITS, int NCH, int M, int SB>
__device__ __forceinline__ float stage_dot(const Stage<NCH, M> &t, int m, const ChunkVec<BITS> *cv)
{
    float y = 0.0f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) y += chunk_contrib<BITS>(t.q[k][m], stage_scale<SB>(t.s[k][m]), cv[k]);
    return y;
}

// s_waitcnt vmcnt(0), expcnt and lgkmcnt left alone: every vector memory load
// this wave has issued is in.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Step cursor over the steps of consecutive matrices: `spm` steps of `rs`
// rows per matrix; tracks the matrix index and first row without division.
struct Cursor {
    int m, s;   // matrix, step within it
    __device__ __forceinline__ void init(int step, int spm) { m = step / spm; s = step - m * spm; }
    __device__ __forceinline__ void next(int spm) { if (++s == spm) { s = 0; ++m; } }
};

// gate_up: hidden[e][i] = SiLU(G_e x)[i] * (U_e x)[i] for every expert.
//
// Blocks are persistent.  Each builds the digit planes of x in LDS once (one
// barrier), every lane copies the planes of its chunks into registers, and
// from then on each wave streams whole rows on its own.  Wave w takes a
// contiguous range of the E * ceil(d_ff / rs) row steps (experts in order),
// with DEPTH steps of code and scale loads in flight ahead of the step being
// reduced; the first DEPTH steps are issued before the planes are built.
template <int BITS, int NCH, int LPR, int DEPTH, int SB>
__global__ __launch_bounds__(512) void k_gate_up(const DecodeArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    extern __shared__ __align__(16) unsigned char smem[];
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int cpr = a.d_model / CPC;
    const size_t row_bytes = (size_t)a.d_model * BITS / 8;
    const int gpr = a.d_model / a.group;
    const RowLanes<NCH, LPR> ln(cpr, CPC, a.group);
    const PlaneLds<BITS> lds(smem, a.d_model);
    constexpr int rs = RowLanes<NCH, LPR>::kRows;
    const int spe = (a.d_ff + rs - 1) / rs;
    const int nsteps = a.n_experts * spe;
    const int W = gridDim.x * nw;
    const int wg = blockIdx.x * nw + wave;
    const int sb = (int)((long)wg * nsteps / W), se = (int)((long)(wg + 1) * nsteps / W);

    auto load = [&](Stage<NCH, 2> &t, const Cursor &c) {
        const uint8_t *codes[2] = {a.gate[c.m].codes, a.up[c.m].codes};
        const void *scales[2] = {a.gate[c.m].scales, a.up[c.m].scales};
        load_stage<NCH, LPR, 2, SB>(t, codes, scales, ln, c.s * rs, a.d_ff, (unsigned)row_bytes, gpr);
    };

    // The vector's loads go first and are waited for before the first steps'
    // code loads go out (behind those, the vector's loads took a few
    // microseconds to come back, and the first steps waited for the planes);
    // then the digit planes are built while the code loads are in flight.
    // 2-bit codes: a wave's set-up (the vector, the planes, its chunks'
    // planes) runs at a higher issue priority than the step loops of the
    // other block on its CU, which start first and would otherwise hold back
    // the later block's set-up (the tail of the kernel; Q2 group gate_up
    // 9.4-9.6 -> 9.1 us in kernel traces, the call 18.7 -> 18.3 us
    // event-timed, alternating builds on one GPU).  At 4 bits it measured no
    // faster.
    if constexpr (BITS == 2) __builtin_amdgcn_s_setprio(3);
    VecRegs<BITS, kGroupsPerThread<BITS>> xr;
    load_vec_regs<BITS>(a.x, a.d_model, xr);
    wait_vm_all();
    // Nothing is loaded past the wave's last step: such loads all went to one
    // address and queued there at the end of every wave.
    const bool busy = sb < se;
    // 2-bit codes: a step's loads go out as soon as the previous step's are in,
    // ahead of its arithmetic (two register slots, one step in flight; Q2
    // group 11.3 -> 10.9 us); 4-bit codes: after its arithmetic, through the
    // DEPTH-slot ring (the other order measured 0.3-0.5 us slower there).
    constexpr bool kEarly = BITS == 2;
    constexpr int NS_ = kEarly ? 2 : DEPTH;
    Stage<NCH, 2> S[NS_];
    Cursor cl;
    cl.init(sb, spe);
    int ls = sb;  // step that cl points at
    auto load_next = [&](Stage<NCH, 2> &t) {
        if (ls < se) load(t, cl);
        cl.next(spe);
        ++ls;
    };
    if (busy) {
#pragma unroll
        for (int i = 0; i < (kEarly ? 1 : DEPTH); ++i) load_next(S[i]);
    }

    build_planes<BITS>(xr, lds.chunks, lds.planes, lds.cmax, lds.dwsum);
    ChunkVec<BITS> cv[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k)
        load_chunk_vec<BITS>(lds.planes, lds.cmax, lds.dwsum, lds.chunks, ln.c[k], ln.valid[k], cv[k]);

    if constexpr (BITS == 2) __builtin_amdgcn_s_setprio(0);
    Cursor cc;
    cc.init(sb, spe);
    for (int base = sb; base < se; base += NS_) {
#pragma unroll
        for (int i = 0; i < NS_; ++i) {
            if (base + i < se) {
                if constexpr (kEarly) {
                    wait_vm_all();               // this step's loads (and the last hidden store) are in
                    load_next(S[(i + 1) % NS_]); // the next step's go out first
                }
                float g = stage_dot<BITS, NCH, 2, SB>(S[i], 0, cv);
                float u = stage_dot<BITS, NCH, 2, SB>(S[i], 1, cv);
                g = group_sum<LPR>(g);
                u = group_sum<LPR>(u);
                const int r = cc.s * rs + ln.slot;
                if (ln.writer() && r < a.d_ff) a.hidden[(size_t)cc.m * a.d_ff + r] = silu_hw(g) * u;
                cc.next(spe);
            }
            if constexpr (!kEarly) load_next(S[i]);
        }
    }
}

// One batch of a vector for the wave-level plane build: B code dwords a lane
// (32 values), dword q0 + lane + 64 b in slot b.
template <int BITS>
struct WaveVec {
    static constexpr int kB = 32 / DigitLayout<BITS>::kColsPerDw;
    float v[kB][DigitLayout<BITS>::kColsPerDw];
};

// Loads one batch.  Every slot is loaded (past the end: the last dword again),
// so the number of loads is fixed and the compiler can wait for exactly these
// while loads issued after them stay in flight (a uniform test per slot turns
// those waits into waits for every load).
template <int BITS>
__device__ __forceinline__ void wave_vec_load(const float *vec, int ndw, int q0, WaveVec<BITS> &r)
{
    constexpr int C = DigitLayout<BITS>::kColsPerDw;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < WaveVec<BITS>::kB; ++b) {
        const int q = min(q0 + lane + 64 * b, ndw - 1);
        const float4 *src = reinterpret_cast<const float4 *>(vec + (size_t)q * C);
#pragma unroll
        for (int i = 0; i < C / 4; ++i) {
            const float4 t = src[i];
            r.v[b][4 * i] = t.x; r.v[b][4 * i + 1] = t.y; r.v[b][4 * i + 2] = t.z; r.v[b][4 * i + 3] = t.w;
        }
    }
}

// Digit planes of one batch into the wave's own LDS region (no block barrier).
template <int BITS>
__device__ __forceinline__ void wave_vec_planes(const WaveVec<BITS> &r, int ndw, int q0, const PlaneLds<BITS> &lds)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int b = 0; b < WaveVec<BITS>::kB; ++b) {
        const int q = q0 + lane + 64 * b;
        if (q0 + 64 * b < ndw)  // uniform: a slot is used by every lane's quad or by none
            plane_dword<BITS>(r.v[b], q, q < ndw, lds.chunks, lds.planes, lds.cmax, lds.dwsum);
    }
}

// down: out = sum_e r_e * (D_e hidden_e).
//
// Blocks own output rows: block b covers `spb` row steps (rs rows each) for
// every expert.  Its work is the list of (expert, step) pairs in expert-major
// order, split into contiguous ranges over its waves, so a wave mostly serves
// one expert.  For each expert it serves, a wave issues the loads of the
// expert's hidden vector and right behind them the code and scale loads of
// its first DEPTH steps, so that all of them are in flight together; it
// waits for the hidden vector only, builds its digit planes in the wave's own
// LDS region (no block barrier), copies its chunks' planes into registers
// and reduces its steps as their loads come in, writing each row's sum to an
// LDS slab [E][rows of the block].  After one barrier the block's threads add
// the experts' rows in ascending expert order in f64, each weighted by its
// router weight, and write out.  The sum has a fixed order (bitwise
// reproducible), no atomics and no range limit, and nothing in the workspace
// has to be zero.
template <int BITS, int NCH, int LPR, int SB, int DEPTH>
__global__ __launch_bounds__(512) void k_down(const DecodeArgs a)
{
    constexpr int CPC = QFormat<BITS>::kCodesPerChunk;
    constexpr int rs = RowLanes<NCH, LPR>::kRows;
    extern __shared__ __align__(16) unsigned char smem[];
    const int nw = blockDim.x >> 6;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int E = a.n_experts;
    const int cpr = a.d_ff / CPC;
    const unsigned row_bytes = (unsigned)a.d_ff * BITS / 8;
    const int gpr = a.d_ff / a.group;
    const int ndw = a.d_ff / DigitLayout<BITS>::kColsPerDw;
    const RowLanes<NCH, LPR> ln(cpr, CPC, a.group);
    const int spb = a.dn_steps_per_block;
    const int nsteps = (a.d_model + rs - 1) / rs;
    const int s0 = blockIdx.x * spb;
    const int ns = min(spb, nsteps - s0);   // row steps of this block
    const int items = E * ns;               // (expert, step) pairs, expert-major
    const int ib = (int)((long)wave * items / nw), ie = (int)((long)(wave + 1) * items / nw);
    const size_t pbytes = (plane_lds_bytes<BITS>(a.d_ff) + 15) & ~size_t(15);
    const PlaneLds<BITS> lds(smem + wave * pbytes, a.d_ff);
    const int brows = spb * rs;
    float *slab = reinterpret_cast<float *>(smem + nw * pbytes);   // [E][brows]
    float *rws = slab + E * brows;                                  // [E] router weights
    // The router weights are loaded first and stored to LDS only before the
    // barrier: they are needed after it, and no wait for them sits in front
    // of the first loads.
    const bool rw_lane = (int)threadIdx.x < E;
    const float my_rw = rw_lane ? (a.route_w ? a.route_w[threadIdx.x] : 1.0f) : 0.0f;

    for (int it = ib; it < ie;) {
        const int e = it / ns;
        const int iend = min(ie, (e + 1) * ns);   // this wave's items of expert e
        const int n = iend - it;
        const uint8_t *dcodes[1] = {a.down[e].codes};
        const void *dscales[1] = {a.down[e].scales};
        auto load = [&](Stage<NCH, 1> &t, int item) {
            load_stage<NCH, LPR, 1, SB>(t, dcodes, dscales, ln, (s0 + item - e * ns) * rs, a.d_model, row_bytes,
                                        gpr);
        };
        // 2-bit codes: the expert's set-up (hidden vector, planes, chunk planes)
        // at a raised issue priority over other waves' step loops, as in
        // gate_up (Q2 group 18.3 -> 18.0 us on top of gate_up's change,
        // event-timed, alternating builds on one GPU).
        if constexpr (BITS == 2) __builtin_amdgcn_s_setprio(3);
        const float *hid = a.hidden + (size_t)e * a.d_ff;
        WaveVec<BITS> hv;
        wave_vec_load<BITS>(hid, ndw, 0, hv);
        Stage<NCH, 1> S[DEPTH];
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) load(S[i], it + min(i, n - 1));   // a short range repeats its last step
        // Keeps the code loads above the plane build.
        asm volatile("" ::: "memory");
        wave_vec_planes<BITS>(hv, ndw, 0, lds);
        for (int q0 = 64 * WaveVec<BITS>::kB; q0 < ndw; q0 += 64 * WaveVec<BITS>::kB) {
            wave_vec_load<BITS>(hid, ndw, q0, hv);
            wave_vec_planes<BITS>(hv, ndw, q0, lds);
        }
        // The wave reads its planes back with its own LDS loads, which the LDS
        // serves in order after its stores; this keeps the compiler from
        // hoisting them.
        asm volatile("" ::: "memory");
        ChunkVec<BITS> cv[NCH];
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            load_chunk_vec<BITS>(lds.planes, lds.cmax, lds.dwsum, lds.chunks, ln.c[k], ln.valid[k], cv[k]);

        if constexpr (BITS == 2) __builtin_amdgcn_s_setprio(0);
        // Steps are reduced in order as their loads come in; a slot is
        // reloaded with the step DEPTH further on once it has been reduced.
        for (int base = 0; base < n; base += DEPTH) {
#pragma unroll
            for (int i = 0; i < DEPTH; ++i) {
                const int j = base + i;
                if (j < n) {
                    float y = stage_dot<BITS, NCH, 1, SB>(S[i], 0, cv);
                    y = group_sum<LPR>(y);
                    const int r = (it + j - e * ns) * rs + ln.slot;  // row within the block
                    if (ln.writer() && s0 * rs + r < a.d_model) slab[e * brows + r] = y;
                    if (j + DEPTH < n) load(S[i], it + j + DEPTH);
                }
            }
        }
        it = iend;
    }
    if (rw_lane) rws[threadIdx.x] = my_rw;
    __syncthreads();
    const int nrows = min(ns * rs, a.d_model - s0 * rs);
    for (int t = threadIdx.x; t < nrows; t += blockDim.x) {
        double acc = 0.0;
        for (int e = 0; e < E; ++e) acc += (double)rws[e] * (double)slab[e * brows + t];
        a.out[s0 * rs + t] = (float)acc;
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

template <int BITS, int NCH, int LPR, int DEPTH, int SB>
hipError_t run_gate_up(const DecodePlan &p, const DecodeArgs &a, int cus, hipStream_t st)
{
    const int block = 64 * p.nw;
    const size_t lds = plane_lds_bytes<BITS>(a.d_model);
    const void *fn = reinterpret_cast<const void *>(&k_gate_up<BITS, NCH, LPR, DEPTH, SB>);
    const long cap = (long)cus * blocks_per_cu(fn, block, lds);
    if (cap < 1) return hipErrorInvalidConfiguration;
    const long steps = (long)a.n_experts * ((a.d_ff + 64 / p.lpr_g - 1) / (64 / p.lpr_g));
    const long grid = std::max(1L, std::min(cap, (steps + p.nw - 1) / p.nw));
    hipLaunchKernelGGL((k_gate_up<BITS, NCH, LPR, DEPTH, SB>), dim3((unsigned)grid), dim3(block), lds, st, a);
    return hipGetLastError();
}

// LDS one down block may take: per-wave planes plus the slab and the router
// weights.
constexpr size_t kDownLdsCap = 64 * 1024;

// Steps of loads a down wave keeps in flight: all of its steps of an expert,
// up to 4.
int down_depth(long steps_per_wave) { return steps_per_wave <= 1 ? 1 : steps_per_wave <= 2 ? 2 : 4; }

template <int BITS, int NCH, int LPR, int SB>
hipError_t run_down(const DecodePlan &p, DecodeArgs a, int cus, hipStream_t st)
{
    const int rs = 64 / p.lpr_d;
    const long nsteps = (a.d_model + rs - 1) / rs;
    // One block per CU, each owning an equal share of the row steps.
    const long spb = std::max(1L, (nsteps + cus - 1) / cus);
    const long blocks = (nsteps + spb - 1) / spb;
    const size_t pb = (plane_lds_bytes<BITS>(a.d_ff) + 15) & ~size_t(15);
    const size_t slab = (size_t)a.n_experts * (spb * rs + 1) * sizeof(float);
    // Waves per block: no more than its (expert, step) pairs, and as many
    // per-wave plane regions as fit beside the slab.
    const long items = (long)a.n_experts * spb;
    long nw = std::min<long>(p.nw, items);
    if (slab + pb > kDownLdsCap) return hipErrorInvalidConfiguration;
    nw = std::min<long>(nw, (long)((kDownLdsCap - slab) / pb));
    const size_t lds = nw * pb + slab;
    const int depth = down_depth((items + nw - 1) / nw);
    const void *fn = depth == 1   ? reinterpret_cast<const void *>(&k_down<BITS, NCH, LPR, SB, 1>)
                     : depth == 2 ? reinterpret_cast<const void *>(&k_down<BITS, NCH, LPR, SB, 2>)
                                  : reinterpret_cast<const void *>(&k_down<BITS, NCH, LPR, SB, 4>);
    if (blocks_per_cu(fn, (int)(64 * nw), lds) < 1) return hipErrorInvalidConfiguration;
    a.dn_steps_per_block = (int)spb;
    const dim3 grid((unsigned)blocks), block((unsigned)(64 * nw));
    if (depth == 1)
        hipLaunchKernelGGL((k_down<BITS, NCH, LPR, SB, 1>), grid, block, lds, st, a);
    else if (depth == 2)
        hipLaunchKernelGGL((k_down<BITS, NCH, LPR, SB, 2>), grid, block, lds, st, a);
    else
        hipLaunchKernelGGL((k_down<BITS, NCH, LPR, SB, 4>), grid, block, lds, st, a);
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
        for (int lpr = 16; lpr <= 64; lpr *= 2) {
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

// Among the mappings with the fewest idle lanes, the one with the most chunks
// per lane (the most bytes per step).  down rows are short (d_ff columns), so a
// wave covers several rows per step this way and keeps more bytes in flight.
bool row_map_wide(int bits, int cpr, int *lpr_out, int *nch_out)
{
    const int max_nch = bits == 4 ? 4 : 2;
    double best_waste = 2.0;
    int bl = 0, bn = 0;
    for (int nch = 1; nch <= max_nch; ++nch)
        for (int lpr = 16; lpr <= 64; lpr *= 2) {
            if (lpr * nch < cpr) continue;
            const double waste = 1.0 - (double)cpr / ((double)lpr * nch);
            if (waste < best_waste - 1e-9 || (waste < best_waste + 1e-9 && nch > bn)) {
                best_waste = waste;
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
    if (mode != kGateUpOnly && !row_map_wide(bits, d_ff / cpc, &q.lpr_d, &q.nch_d)) return false;
    *p = q;
    return true;
}

// gate_up: steps in flight per wave (the register ring of code and scale
// loads).  down has its own order: a step's loads go out once the previous
// step's have come back, ahead of its arithmetic.
constexpr int kGateUpDepth = 1;

// Kernels are compiled per (bits, chunks per lane, lanes per row): lanes per
// row 16, 32 or 64; chunks per lane 1..4 (4-bit) or 1..2 (2-bit).
#define SMOE_FOR_LPR(X, B, N) X(B, N, 16) X(B, N, 32) X(B, N, 64)
#define SMOE_FOR_ALL(X)                                                        \
    SMOE_FOR_LPR(X, 4, 1) SMOE_FOR_LPR(X, 4, 2) SMOE_FOR_LPR(X, 4, 3) SMOE_FOR_LPR(X, 4, 4) \
    SMOE_FOR_LPR(X, 2, 1) SMOE_FOR_LPR(X, 2, 2)

hipError_t launch_gate_up(int bits, const DecodePlan &p, const DecodeArgs &a, int cus, hipStream_t st)
{
#define SMOE_RUN(B, N, L)                                                                  \
    if (bits == B && p.nch_g == N && p.lpr_g == L)                                         \
        return a.scale_bytes == 2 ? run_gate_up<B, N, L, kGateUpDepth, 2>(p, a, cus, st)   \
                                  : run_gate_up<B, N, L, kGateUpDepth, 4>(p, a, cus, st);
    SMOE_FOR_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

hipError_t launch_down(int bits, const DecodePlan &p, const DecodeArgs &a, int cus, hipStream_t st)
{
#define SMOE_RUN(B, N, L)                                                                  \
    if (bits == B && p.nch_d == N && p.lpr_d == L)                                         \
        return a.scale_bytes == 2 ? run_down<B, N, L, 2>(p, a, cus, st)                    \
                                  : run_down<B, N, L, 4>(p, a, cus, st);
    SMOE_FOR_ALL(SMOE_RUN)
#undef SMOE_RUN
    return hipErrorInvalidConfiguration;
}

}  // namespace smoe
