// Token-batch routed-expert FFN on the gfx950 matrix cores.
//
// For T tokens X [T][d_model] and each expert e:
//     H_e = SiLU(X G_e^T) * (X U_e^T)        [T][d_ff]
//     out = sum_e diag(r[:, e]) (H_e D_e^T)   [T][d_model]
// (S-MoE docs, Metal Compute Kernels: "Token-Batch Fused FFN", which runs the
// fused gate/up and down passes over many token activations per expert, and
// "Fused FFN Kernels" for the per-group affine form of the dequantised dot
// product).  Every expert processes every token.
//
// Why the contraction can run on f16 MFMA without losing f32 accuracy:
//  * a code c enters the matrix core as the f16 value c - Z (Z = 7.5 or 1.5),
//    which is exact; the scale s/Z is applied per quantisation group afterwards;
//  * activations are scaled by a power of two 2^-e so that every scaled value
//    is below 1 in magnitude (one e per token for X, one per token and group of
//    d_ff columns for the hidden rows), then written as hi + lo with
//    hi = f16(v), lo = f16(v - hi): 22 significant bits, no overflow, and the
//    scaling is undone exactly;
//  * v_mfma_f32_16x16x32_f16 multiplies exactly and accumulates in f32; hi and
//    lo go through two MFMAs into one accumulator per group, and the group's
//    f32 result is multiplied by its scale into the running output.
//
// Launch sequence (one stream), T > 16: k_tb_prep (X -> hi/lo halves +
// per-token exponent), k_tb_gate_up_tiled (both projections, SiLU, hidden rows
// -> hi/lo halves + one factor per (expert, group, token) that folds the
// group's power of two and the router weight), k_tb_down_tiled (all experts
// summed in a fixed order, so the result is deterministic; no atomics in the
// sums), each followed by its finishing pass when its K dimension is split
// over blocks of 32- or 64-token tiles.  T <= 16: k_tb_gate_up_stream (X
// staged per phase of 16 groups into LDS by every block; f32 hidden rows) and
// k_tb_down_stream (hidden rows staged and split per group; the chunks of a
// row group added in the kernel in chunk order).
//
// Orientation: tokens are the MFMA's M side, weight rows its N side.  For
// v_mfma_f32_16x16x32_f16 (lane l, q = l / 16, n = l % 16):
//   A (16 x 32):  token n, k = 8q + i for element i = 0..7   <- activations
//   B (32 x 16):  row n,   k = 8q + i                         <- weight codes
//   D (16 x 16):  tokens 4q + i (i = 0..3), row n             -> outputs
// so a lane needs one scale per row tile and group.  Within one quantisation
// group of 32*KB columns, lane group q owns the 8*KB columns [q*8KB,
// (q+1)*8KB): its codes are one contiguous load, and K-block j uses columns
// q*8KB + 8j + sigma(i), sigma = (0,4,1,5,2,6,3,7), the order in which the
// nibble unpacking yields codes.  Activations are stored in the same order
// (element 8b + i holds column 8b + sigma(i)).
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace smoe {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Half8Parts {
    half2v v[4];
};

// Position of column c (0..7) of an 8-column block in sigma order.
__device__ __forceinline__ int sigma_pos(int c) { return (c & 3) * 2 + (c >> 2); }

// f16 pair (c_a - Z, c_b - Z) from bytes a, b of src picked by sel, whose
// codes sit in their top bits (bits 4..7 of a byte at 4 bits, 6..7 at 2
// bits).  Under the high byte 0x48 (the exponent of 8.0) such a byte reads as
// the f16 value 8 + c/8 (4-bit) or 8 + c/2 (2-bit); one packed FMA then gives
// 8 (8 + c/8) - 71.5 = c - 7.5 or 2 (8 + c/2) - 17.5 = c - 1.5.  Every
// operand and result is an f16 value, so the conversion is exact.
template <int BITS>
__device__ __forceinline__ half2v code_pair(uint32_t src, uint32_t sel)
{
    const uint32_t bits = __builtin_amdgcn_perm(0x48484848u, src, sel);
    const half2v h = __builtin_bit_cast(half2v, bits);
    constexpr float mul = BITS == 4 ? 8.0f : 2.0f;
    constexpr float add = BITS == 4 ? -71.5f : -17.5f;
    return h * (half2v){(_Float16)mul, (_Float16)mul} + (half2v){(_Float16)add, (_Float16)add};
}

// Codes per lane per quantisation group: KB K-blocks of 8 codes.
template <int BITS, int KB>
struct CodeWords {
    static constexpr int kDwords = (KB * BITS + 3) / 4;  // Q4: KB dwords, Q2: KB/2 dwords
    uint32_t w[kDwords];
};

// B fragment of K-block j: the lane's 8 codes in sigma order as f16 (c - Z).
template <int BITS, int KB>
__device__ __forceinline__ half8 code_frag(const CodeWords<BITS, KB> &c, int j)
{
    Half8Parts f;
    if constexpr (BITS == 4) {
        // Nibbles n0..n7 of one dword: lo holds bytes (n0,n2,n4,n6), hi (n1,n3,n5,n7),
        // each nibble in the top half of its byte.
        const uint32_t d = c.w[j];
        const uint32_t lo = (d << 4) & 0xF0F0F0F0u, hi = d & 0xF0F0F0F0u;
        f.v[0] = code_pair<4>(lo, 0x04020400u);  // n0, n4
        f.v[1] = code_pair<4>(hi, 0x04020400u);  // n1, n5
        f.v[2] = code_pair<4>(lo, 0x04030401u);  // n2, n6
        f.v[3] = code_pair<4>(hi, 0x04030401u);  // n3, n7
    } else {
        // 16 two-bit codes c0..c15 per dword; a_k holds bytes (c_k, c_4+k, c_8+k, c_12+k),
        // each code in the top two bits of its byte.
        const uint32_t d = c.w[j >> 1];
        const uint32_t sel = (j & 1) ? 0x04030402u : 0x04010400u;
#pragma unroll
        for (int k = 0; k < 4; ++k) f.v[k] = code_pair<2>((d << (6 - 2 * k)) & 0xC0C0C0C0u, sel);
    }
    return __builtin_bit_cast(half8, f);
}

__device__ __forceinline__ half8 load_half8(const _Float16 *p)
{
    return __builtin_bit_cast(half8, *reinterpret_cast<const uint4 *>(p));
}

__device__ __forceinline__ f32x4 mfma(half8 a, half8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Exponent e with |m| = f * 2^e, f in [0.5, 1) (0 for m == 0): v * 2^-e < 1.
__device__ __forceinline__ int norm_exponent(float m)
{
    int e = 0;
    (void)frexpf(m, &e);
    return e;
}

// Largest value over the 16 lanes of a DPP row (every lane gets it).
__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v));  // row_mirror
    return v;
}

// Buffer loads: a resource (base, byte extent) in scalar registers, a fixed
// per-lane byte offset and a uniform byte offset per step, so that moving to the
// next step writes no vector registers.  Raw buffer (stride 0) with a 32-bit
// data format, as the memory instructions expect for untyped loads.
using BufRes = __amdgpu_buffer_rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ BufRes buf_res(const void *base, size_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)min(bytes, (size_t)0x7fffffff),
                                             0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(BufRes r, unsigned voff, unsigned soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ unsigned buf_load4(BufRes r, unsigned voff, unsigned soff)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

// Raw bits of scale element idx (f32, or binary16 in the low half), and its
// value: the widening is kept apart from the load so that a load issued ahead
// is not waited for where it is issued.
template <int SB>
__device__ __forceinline__ unsigned buf_load_scale_bits(BufRes r, unsigned idx)
{
    if constexpr (SB == 4)
        return buf_load4(r, idx * 4u, 0u);
    else
        return (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, (int)(idx * 2u), 0, 0);
}
// The same at a byte offset: lane part voff, uniform part soff.
template <int SB>
__device__ __forceinline__ unsigned buf_load_scale_at(BufRes r, unsigned voff, unsigned soff)
{
    if constexpr (SB == 4)
        return buf_load4(r, voff, soff);
    else
        return (unsigned)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
template <int SB>
__device__ __forceinline__ float scale_value(unsigned bits)
{
    if constexpr (SB == 4)
        return __uint_as_float(bits);
    else
        return (float)__builtin_bit_cast(_Float16, (unsigned short)bits);
}

// Code unit: the 16 bytes of a row that one lane loads at once, spanning
// kGroups consecutive quantisation groups (two groups of 32 bytes for 4-bit
// codes in 64-column groups; four groups of 16 bytes otherwise).  A
// per-group load would read only 16 or 32 bytes of each 128-byte line per
// instruction, and the cost of these loads goes with the lines an instruction
// touches.  Lane row q (lanes 16q .. 16q+15) loads bytes 16q .. 16q+15 of the
// unit; unit_split then exchanges words between lane rows so that each lane
// holds its column block of every group of the unit.  The column block of
// lane row q is CodeUnit::cb(q): the identity for four groups, rows 1 and 2
// swapped for two.
template <int BITS, int KB>
struct CodeUnit {
    static constexpr int kDw = CodeWords<BITS, KB>::kDwords;   // dwords per lane per group
    static_assert(kDw == 1 || kDw == 2, "code units take 16 or 32 bytes per row and group");
    static constexpr int kGroups = 4 / kDw;
    static __device__ __forceinline__ int cb(int q) { return kDw == 2 ? ((q & 1) << 1) | (q >> 1) : q; }
};

// v_permlane32_swap(x, y) exchanges lanes 32..63 of x with lanes 0..31 of y;
// v_permlane16_swap(x, y) exchanges the odd 16-lane rows of x with the even
// rows of y.  Two groups (lane rows 0, 1 hold group 0, rows 2, 3 group 1, in
// 16-byte halves): swapping dwords 0, 1 of rows 2, 3 with dwords 2, 3 of rows
// 0, 1 leaves every row with 8 bytes of each group, at byte 8 cb(q) of it.
// Four groups (row q holds group q): the 32-lane swap and then the 16-lane
// swap transpose the 4 x 4 dwords, so row q holds dword q of each group.
template <int BITS, int KB>
__device__ __forceinline__ void unit_split(uint4 raw, CodeWords<BITS, KB> (&cw)[CodeUnit<BITS, KB>::kGroups])
{
    const auto a = __builtin_amdgcn_permlane32_swap(raw.x, raw.z, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(raw.y, raw.w, false, false);
    if constexpr (CodeUnit<BITS, KB>::kDw == 2) {
        cw[0].w[0] = a[0];
        cw[0].w[1] = b[0];
        cw[1].w[0] = a[1];
        cw[1].w[1] = b[1];
    } else {
        const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
        const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
        cw[0].w[0] = c[0];
        cw[1].w[0] = c[1];
        cw[2].w[0] = d[0];
        cw[3].w[0] = d[1];
    }
}

// -------------------------------------------------------------------------
// X -> hi/lo halves in sigma order + one exponent per token.  One block of
// 256 threads per token, one pass: each thread keeps up to 4 chunks of 8
// columns in registers (d_model <= 8192), the block finds the row's largest
// |x|, and every chunk is written as two 16-byte stores (hi, lo).
__device__ __forceinline__ void prep_token(const float *__restrict__ x, int cols, _Float16 *__restrict__ xh,
                                           _Float16 *__restrict__ xl, int *__restrict__ xe,
                                           unsigned *__restrict__ cnt, int n_cnt, int tok, int ntok)
{
    __shared__ float s_max[4];
    // The split counters start every call at zero.
    for (int i = tok * 256 + threadIdx.x; i < n_cnt; i += ntok * 256) cnt[i] = 0u;
    const size_t base = (size_t)tok * cols;
    const int nch = cols / 8;
    float v[4][8];
    float m = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = threadIdx.x + 256 * k;
        if (c < nch) {
            const float4 a0 = reinterpret_cast<const float4 *>(x + base)[2 * c];
            const float4 a1 = reinterpret_cast<const float4 *>(x + base)[2 * c + 1];
            v[k][0] = a0.x; v[k][1] = a0.y; v[k][2] = a0.z; v[k][3] = a0.w;
            v[k][4] = a1.x; v[k][5] = a1.y; v[k][6] = a1.z; v[k][7] = a1.w;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[k][i]));
        }
    }
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const int e = norm_exponent(m);
    constexpr int kSigma[8] = {0, 4, 1, 5, 2, 6, 3, 7};   // column at each sigma position
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int c = threadIdx.x + 256 * k;
        if (c < nch) {
            half8 hi, lo;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float sv = ldexpf(v[k][kSigma[i]], -e);
                hi[i] = (_Float16)sv;
                lo[i] = (_Float16)(sv - (float)hi[i]);
            }
            reinterpret_cast<half8 *>(xh + base)[c] = hi;
            reinterpret_cast<half8 *>(xl + base)[c] = lo;
        }
    }
    if (threadIdx.x == 0) xe[tok] = e;
}

__global__ __launch_bounds__(256) void k_tb_prep(const float *__restrict__ x, int cols, _Float16 *__restrict__ xh,
                                                 _Float16 *__restrict__ xl, int *__restrict__ xe,
                                                 unsigned *__restrict__ cnt, int n_cnt)
{
    prep_token(x, cols, xh, xl, xe, cnt, n_cnt, blockIdx.x, gridDim.x);
}

// -------------------------------------------------------------------------
// Kernels (groups of 32 and 64 columns): a block of 8 waves covers a
// tile of TT = 16 * NTT tokens and 128 weight rows (one 16-row tile per wave).
// For each quantisation group (gate_up) or (expert, group) pair (down) the
// block loads the tile's activation halves once, with coalesced 16-byte loads,
// into one of two LDS buffers, and the waves read their MFMA fragments from
// LDS.  One barrier per step: a buffer is refilled only after every wave has
// passed the barrier that ends the step reading it.  The K dimension (the
// groups of d_model, or the (expert, group) pairs) is split over `ks` blocks
// when there would otherwise be too few blocks: each writes its partial sums
// to the workspace, and either the last of a tile's splits to finish or a
// finishing kernel adds them in split order (deterministic) and applies the
// epilogue.
constexpr int kTileWaves = 8;
constexpr int kTileRows = 16 * kTileWaves;

// The hardware hands consecutive workgroups to the 8 XCDs in turn, and each XCD
// has its own L2.  This maps the launch index to a logical one so that the
// blocks an XCD receives are consecutive logical blocks (which share weights);
// a bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_logical(int b, int n)
{
    const int q = n >> 3, r = n & 7, x = b & 7, k = b >> 3;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// LDS activation tiles pad each token row by 16 bytes, so that the 16 token
// rows of a fragment read fall into different banks.
// Cooperative load of one activation tile: TT token rows x MG groups of
// 32 * KB columns of the hi and the lo halves, in pieces of 16 bytes.  A
// thread takes pieces c = tid + 512 i (i < PP); when there are fewer than
// 512 * PP pieces, c wraps round and a piece is loaded and stored twice (same
// value, same place), so every thread issues the same loads.  Piece i of a
// thread is fixed by the thread and i alone: its half (the same for the whole
// wave: a half is a multiple of 64 pieces), its byte offset from the step's
// first column (below 2^30 for T <= 65536 and 8192 columns) and its LDS place.
template <int KB, int NTT, int MG = 1>
struct TileShape {
    static constexpr int kCols = MG * 32 * KB, kPerRow = kCols / 8, kTT = 16 * NTT;
    static constexpr int kPerHalf = kTT * kPerRow, kPieces = 2 * kPerHalf;
    static constexpr int kPP = (kPieces + 511) / 512;
    static constexpr int kStride = kCols + 8;   // halfs per LDS token row
    static constexpr size_t kBytes = (size_t)2 * kTT * kStride * 2;
};

template <int KB, int NTT, int MG = 1>
struct TileRegs {
    uint4 v[TileShape<KB, NTT, MG>::kPP];
};

template <int KB, int NTT, int MG = 1>
struct TileMap {
    static constexpr int PP = TileShape<KB, NTT, MG>::kPP;
    unsigned off[PP];   // global byte offset of the piece within its half
    unsigned lds[PP];   // LDS byte offset of the piece within a tile buffer
    bool lo[PP];        // wave-uniform: the piece belongs to the lo half
};

// Tile rows t0 .. t0+TT-1 of a table of `rows` rows (clamped to the last);
// with a row list (routed mode) tile row p reads table row list[p] / top_k.
template <int KB, int NTT, int MG = 1>
__device__ __forceinline__ void tile_map(TileMap<KB, NTT, MG> &m, int wave, unsigned row_stride_bytes, int t0,
                                         int rows, const int *list = nullptr, int top_k = 1)
{
    using Sh = TileShape<KB, NTT, MG>;
#pragma unroll
    for (int i = 0; i < Sh::kPP; ++i) {
        const int c = (threadIdx.x + 512 * i) % Sh::kPieces;
        const int hl = ((wave * 64 + 512 * i) % Sh::kPieces) / Sh::kPerHalf;
        const int rem = c - hl * Sh::kPerHalf;
        const int tok = rem / Sh::kPerRow, part = rem - tok * Sh::kPerRow;
        const int p = min(t0 + tok, rows - 1);
        const int row = list ? list[p] / top_k : p;
        m.lo[i] = hl != 0;
        m.off[i] = (unsigned)row * row_stride_bytes + (unsigned)part * 16u;
        m.lds[i] = (unsigned)((hl * Sh::kTT + tok) * Sh::kStride + part * 8) * 2u;
    }
}

// The pieces of the step whose first column is `col_bytes` into each row.
template <int KB, int NTT, int MG = 1>
__device__ __forceinline__ void tile_load(TileRegs<KB, NTT, MG> &r, const TileMap<KB, NTT, MG> &m, BufRes hi,
                                          BufRes lo, unsigned col_bytes)
{
#pragma unroll
    for (int i = 0; i < TileShape<KB, NTT, MG>::kPP; ++i)
        r.v[i] = buf_load16(m.lo[i] ? lo : hi, m.off[i], col_bytes);
}

template <int KB, int NTT, int MG = 1>
__device__ __forceinline__ void tile_store(const TileRegs<KB, NTT, MG> &r, const TileMap<KB, NTT, MG> &m,
                                           uint8_t *tile)
{
#pragma unroll
    for (int i = 0; i < TileShape<KB, NTT, MG>::kPP; ++i) *reinterpret_cast<uint4 *>(tile + m.lds[i]) = r.v[i];
}

// A fragments of token tile tt, K-block j of group gi, hi and lo, from an LDS
// tile, for a lane that owns column block cb of the group.
template <int KB, int NTT, int MG = 1>
__device__ __forceinline__ void tile_frags(const uint8_t *tile, int tt, int gi, int j, int cb, half8 &h, half8 &l)
{
    using Sh = TileShape<KB, NTT, MG>;
    const int n = threadIdx.x & 15;
    const _Float16 *p = reinterpret_cast<const _Float16 *>(tile) + (tt * 16 + n) * Sh::kStride + gi * 32 * KB +
                        cb * 8 * KB + 8 * j;
    h = load_half8(p);
    l = load_half8(p + Sh::kTT * Sh::kStride);
}

// Partial sums of one block of a split tile: N f32x4 per thread, lane-major
// (consecutive threads, consecutive 16 bytes), so that storing and reloading
// them is coalesced.
template <int N>
__device__ __forceinline__ void store_partial(const f32x4 (&acc)[N], float *part)
{
#pragma unroll
    for (int k = 0; k < N; ++k) reinterpret_cast<f32x4 *>(part)[k * 512 + threadIdx.x] = acc[k];
}

// acc[k] = sum over the splits s = 0, 1, ... of the partial sums at
// part + s * stride, accumulator slot at[k] of them.
template <int N>
__device__ __forceinline__ void sum_partials(f32x4 (&acc)[N], const float *part, size_t stride, int splits,
                                             const int (&at)[N])
{
#pragma unroll
    for (int k = 0; k < N; ++k) acc[k] = reinterpret_cast<const f32x4 *>(part)[at[k] * 512 + threadIdx.x];
    for (int s = 1; s < splits; ++s) {
        const f32x4 *ps = reinterpret_cast<const f32x4 *>(part + (size_t)s * stride);
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const f32x4 v = ps[at[k] * 512 + threadIdx.x];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[k][r] += v[r];
        }
    }
}

// Where a tile's K splits are added: in the tiled kernel itself for 16-token
// tiles (a split's slab is 8 or 16 KB; two launches fewer per call, and at 16
// tokens the host takes longer to launch a call's kernels than the GPU to run
// them), in a finishing pass for larger tiles (there every split block's
// store, wait and count of a 32 or 64 KB slab, and the last one's reads,
// sit in the kernel's tail: 64 tokens 93 against 90 us, 128 tokens 174
// against 142, 256 tokens 259 against 232).
template <int NTT>
constexpr bool kSplitsInKernel = NTT == 1;

__device__ __forceinline__ float *partial_slot(float *part, int k, int r)
{
    return part + ((size_t)(4 * k + r) * 512 + threadIdx.x);
}

// K splits of a tile, reduced in the kernel.  Every split block stores its
// accumulators at agent scope (the stores go to memory, past this XCD's L2),
// waits for them, and counts itself in on the tile's counter; the block that
// completes the count adds all the splits' partial sums in split order (its
// own from registers, the others read at agent scope) and goes on to the
// tile's epilogue; the others are done.  The sum does not depend on which
// block comes last: bitwise the same result every call.  Float r of
// accumulator k of thread t sits at (4k + r) * 512 + t of a split's slab, so
// that a wave's stores and loads are 256 contiguous bytes.  `last` is LDS.
// Returns whether this block holds the tile's sum.
//
// Ordering.  The counter is a relaxed atomic, and what orders the slabs
// before it is the machine's: on gfx950 an agent-scope atomic store is a
// store with the sc1 bit, performed at the agent's coherence point rather
// than in the XCD's L2, and s_waitcnt vmcnt(0) returns once it is performed;
// an agent-scope atomic load (sc1) reads from that point.  An agent-scope
// release / acquire pair on the counter would add to exactly these steps an
// L2 write-back before the count (for prior plain stores, of which the slabs
// have none) and an L2 invalidate after it (for later plain loads, likewise
// none), and measured 4.8 us slower per 16-token call.
template <int N>
__device__ bool split_reduce(f32x4 (&acc)[N], float *part, size_t stride, int ks, int splits, unsigned *cnt,
                             int *last)
{
    float *mine = part + (size_t)ks * stride;
#pragma unroll
    for (int k = 0; k < N; ++k)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            __hip_atomic_store(partial_slot(mine, k, r), acc[k][r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores have reached memory
    __syncthreads();
    if (threadIdx.x == 0)
        *last = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)splits - 1;
    __syncthreads();
    if (!*last) return false;
    f32x4 own[N];
#pragma unroll
    for (int k = 0; k < N; ++k) own[k] = acc[k];
    // Slabs are read B at a time, all of a round's loads in flight together,
    // then added in split order.
    constexpr int B = N <= 2 ? 8 : 16 / N;   // at most 64 floats in flight a thread
    for (int s0 = 0; s0 < splits; s0 += B) {
        float v[B][N][4];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int s = min(s0 + b, splits - 1);   // past the last split: re-read it, unused
            const float *ps = part + (size_t)s * stride;
#pragma unroll
            for (int k = 0; k < N; ++k)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[b][k][r] = s == ks ? own[k][r]
                                         : __hip_atomic_load(partial_slot(const_cast<float *>(ps), k, r),
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (s0 + b >= splits) break;
#pragma unroll
            for (int k = 0; k < N; ++k)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[k][r] = s0 + b == 0 ? v[b][k][r] : acc[k][r] + v[b][k][r];
        }
    }
    return true;
}

// gate_up epilogue of a tile: hidden = SiLU(gate) * up for the wave's 16 rows
// and the tile's tokens (tot scaled by the tokens' 2^-xe), normalised per (token, H group) by a power of two,
// stored as hi/lo halves in sigma order with the factor r[t][e] * 2^e for
// down.  tot holds the gate token tiles, then the up token tiles; mx is LDS
// for [waves][NTT][16] floats.  Contains a block barrier.
template <int KB, int NTT>
__device__ __forceinline__ void gu_epilogue(const TbArgs &a, const f32x4 (&tot)[2 * NTT], int e, int rb, int tb,
                                            float *mx)
{
    constexpr int TT = 16 * NTT;
    constexpr int group = 32 * KB;
    const int d_ff = a.d_ff, T = a.T, E = a.n_experts, HG = d_ff / group;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int t0 = tb * TT;
    const int wrow0 = rb * kTileRows + wave * 16;
    // Rows of the tile: tokens (dense mode) or positions in expert e's slot list.
    const int *list = a.top_k ? a.list + (size_t)e * T : nullptr;
    const int rows = a.top_k ? a.cnt[e] : T;
    // Per-token maxima over this wave's 16 rows.
    float h[NTT][4];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pc = min(t0 + tt * 16 + 4 * q + i, rows - 1);
            const int t = list ? list[pc] / a.top_k : pc;
            const int xe = a.xe[t];
            const float gv = ldexpf(tot[tt][i], xe), uv = ldexpf(tot[NTT + tt][i], xe);
            h[tt][i] = wrow0 + n < d_ff ? silu(gv) * uv : 0.0f;
            const float m = row16_max(fabsf(h[tt][i]));
            if (n == 0) mx[(wave * NTT + tt) * 16 + 4 * q + i] = m;
        }
    __syncthreads();
    if (wrow0 >= d_ff) return;
    constexpr int wpg = group / 16;                   // waves per H group
    const int w0 = wave - wave % wpg;
    const int hg = (rb * kTileRows + w0 * 16) / group;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tl = 4 * q + i;
            float m = 0.0f;
#pragma unroll
            for (int w = 0; w < wpg; ++w) m = fmaxf(m, mx[((w0 + w) * NTT + tt) * 16 + tl]);
            const int ee = norm_exponent(m);
            const int p = t0 + tt * 16 + tl;
            if (p < rows) {
                const float v = ldexpf(h[tt][i], -ee);
                const _Float16 hv = (_Float16)v;
                const int r = wrow0 + n;
                const size_t pos = ((size_t)e * T + p) * d_ff + (r & ~7) + sigma_pos(r & 7);
                a.hh[pos] = hv;
                a.hl[pos] = (_Float16)(v - (float)hv);
                if (wave == w0 && n == 0) {
                    const float rwt = list ? a.slot_w[list[p]] : a.route_w ? a.route_w[(size_t)p * E + e] : 1.0f;
                    a.hf[((size_t)e * HG + hg) * a.t_pad + p] = ldexpf(rwt, ee);
                }
            }
        }
}

// gate_up, tiled: block (token tile, row block, expert, split).  A step is MG
// quantisation groups of d_model; one loop iteration is 4 / MG steps (four
// groups), so that the code units and scale quads start at fixed steps of it.
template <int BITS, int KB, int NTT, int MG, int SB>
__global__ __launch_bounds__(512) void k_tb_gate_up_tiled(TbArgs a)
{
    using Sh = TileShape<KB, NTT, MG>;
    using CU = CodeUnit<BITS, KB>;
    static_assert(MG == 1 || MG == 2, "a step is one or two groups");
    constexpr int kG = CU::kGroups;
    constexpr int U = 4 / MG;   // steps per iteration
    constexpr int TT = 16 * NTT;
    constexpr int group = 32 * KB;
    extern __shared__ __align__(16) unsigned char smem[];   // two tiles, then the epilogue's maxima
    __shared__ int s_last;                                  // whether this block adds the tile's K splits
    const int d_model = a.d_model, d_ff = a.d_ff, T = a.T, E = a.n_experts;
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, n = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int G = d_model / group, NS = G / MG;
    const int NTB = (T + TT - 1) / TT;
    const int RB = (d_ff + kTileRows - 1) / kTileRows;
    const int KSG = a.ks_gu;
    // Logical block order: token tile, row block, expert, split (the blocks an
    // XCD gets share codes across token tiles and activation tiles across row
    // blocks and experts).
    int b = xcd_logical(blockIdx.x, gridDim.x);
    int tb, rb, e, ks;
    if (a.top_k) {
        // Routed mode, order chunk, row block, split: chunk c is the c-th
        // token tile of the experts' slot lists, taken in expert order (the
        // grid holds an upper bound of them; blocks past the last exit).
        const int C = gridDim.x / (RB * KSG);
        int c = b % C;
        b /= C;
        rb = b % RB;
        ks = b / RB;
        for (e = 0; e < E; ++e) {
            const int nt = (a.cnt[e] + TT - 1) / TT;
            if (c < nt) break;
            c -= nt;
        }
        if (e == E) return;   // whole block, before any barrier
        tb = c;
    } else {
        tb = b % NTB;
        b /= NTB;
        rb = b % RB;
        b /= RB;
        e = b % E;
        ks = b / E;
    }
    const int t0 = tb * TT;
    // Routed mode: the tile's rows are expert e's slots.
    const int rows = a.top_k ? a.cnt[e] : T;
    if (t0 >= rows) return;   // whole block, before any barrier
    const int wrow0 = rb * kTileRows + wave * 16;   // this wave's first d_ff row
    // The split's steps: whole iterations (only the last split may end inside
    // one); the plan keeps every split non-empty.
    const int NI = (NS + U - 1) / U;
    const int s0 = U * (int)((long)ks * NI / KSG);
    const int NSS = min(U * (int)((long)(ks + 1) * NI / KSG), NS) - s0;
    const int g0 = s0 * MG;   // the split's first group

    // Lane offsets (32-bit: a matrix has at most 8192 x 8192 entries) and
    // buffer resources.
    const unsigned row = (unsigned)min(wrow0 + n, d_ff - 1);
    const unsigned crow = row * (unsigned)(d_model * BITS / 8) + 16u * (unsigned)(q % CU::kDw);
    const int cq = q / CU::kDw;   // the lane's group within a code unit
    const unsigned srow = row * (unsigned)G;
    const int cb = CU::cb(q);
    const size_t cbytes = (size_t)d_ff * d_model * BITS / 8, sbytes = (size_t)d_ff * G * SB;
    const BufRes cr[2] = {buf_res(a.gate[e].codes, cbytes), buf_res(a.up[e].codes, cbytes)};
    const BufRes sr[2] = {buf_res(a.gate[e].scales, sbytes), buf_res(a.up[e].scales, sbytes)};
    const BufRes xhr = buf_res(a.xh, (size_t)T * d_model * 2), xlr = buf_res(a.xl, (size_t)T * d_model * 2);
    TileMap<KB, NTT, MG> tm;
    tile_map<KB, NTT, MG>(tm, wave, (unsigned)d_model * 2u, t0, rows, a.top_k ? a.list + (size_t)e * T : nullptr,
                          a.top_k);

    // Loads, all issued at the start of a step and never waited for there:
    //  * activation pieces of step s into ring slot s & 1 at the start of step
    //    s - 2; stored into LDS (buffer s & 1) at the end of step s - 1;
    //  * the raw code unit and scale quad after the current ones, as soon as
    //    those have been unpacked at the start of their first step.
    // The loop is branch-free so that the compiler's load waits are exact:
    // loads past the split's last step repeat it or clamp to the last group,
    // and the steps past the end (at most U - 1) count with scale 0.
    TileRegs<KB, NTT, MG> tr[2];
    uint4 craw[2];                     // next code unit, gate and up
    unsigned sraw[2];                  // next scale quad, gate and up
    CodeWords<BITS, KB> cw[2][kG];     // current code unit
    float sc[2][4];                    // current scale quad, divided by Z
    auto load_tile = [&](TileRegs<KB, NTT, MG> &t, int s) {
        const unsigned g = (unsigned)((s0 + min(s, NSS - 1)) * MG);
        tile_load<KB, NTT, MG>(t, tm, xhr, xlr, g * (unsigned)group * 2u);
    };
    auto load_unit = [&](int u) {   // groups g0 + kG u .. of the wave's rows
        const unsigned off = crow + (unsigned)min(g0 + kG * u + cq, G - 1) * (unsigned)(16 * CU::kDw);
        craw[0] = buf_load16(cr[0], off, 0u);
        craw[1] = buf_load16(cr[1], off, 0u);
    };
    auto load_quad = [&](int k) {   // lane row q: group g0 + 4 k + q of its row
        const unsigned idx = srow + (unsigned)min(g0 + 4 * k + q, G - 1);
        sraw[0] = buf_load_scale_bits<SB>(sr[0], idx);
        sraw[1] = buf_load_scale_bits<SB>(sr[1], idx);
    };

    f32x4 tot[2 * NTT];   // gate token tiles, then up token tiles
#pragma unroll
    for (int k = 0; k < 2 * NTT; ++k) tot[k] = (f32x4){0.f, 0.f, 0.f, 0.f};

    load_unit(0);
    load_quad(0);
    load_tile(tr[0], 0);
    load_tile(tr[1], 1);
    __builtin_amdgcn_sched_barrier(0);   // keep the loads in issue order
    tile_store<KB, NTT, MG>(tr[0], tm, smem);
    __syncthreads();
    for (int base = 0; base < NSS; base += U) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int st = base + i;
            if ((i * MG) % kG == 0) {   // a code unit starts (fixed per i)
#pragma unroll
                for (int m = 0; m < 2; ++m) unit_split<BITS, KB>(craw[m], cw[m]);
                load_unit((st * MG) / kG + 1);
            }
            if (i == 0) {   // a scale quad starts: group j of it from lane row j
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        sc[m][j] = scale_value<SB>((unsigned)__builtin_amdgcn_ds_bpermute(
                                       (n + 16 * j) * 4, (int)sraw[m])) *
                                   QFormat<BITS>::kInvZ;
                load_quad(base * MG / 4 + 1);
            }
            load_tile(tr[i & 1], st + 2);
            __builtin_amdgcn_sched_barrier(0);
            const uint8_t *tile = smem + (size_t)(i & 1) * Sh::kBytes;   // base is even
#pragma unroll
            for (int gi = 0; gi < MG; ++gi) {
                const int ug = (i * MG + gi) % kG;   // group within the unit
                half8 bf[2][KB];
                float s[2];
#pragma unroll
                for (int m = 0; m < 2; ++m) {
#pragma unroll
                    for (int j = 0; j < KB; ++j) bf[m][j] = code_frag<BITS, KB>(cw[m][ug], j);
                    s[m] = st < NSS ? sc[m][i * MG + gi] : 0.0f;
                }
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                    for (int j = 0; j < KB; ++j) {
                        half8 h, l;
                        tile_frags<KB, NTT, MG>(tile, tt, gi, j, cb, h, l);
#pragma unroll
                        for (int m = 0; m < 2; ++m) {
                            acc[m] = mfma(h, bf[m][j], acc[m]);
                            acc[m] = mfma(l, bf[m][j], acc[m]);
                        }
                    }
#pragma unroll
                    for (int m = 0; m < 2; ++m)
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            tot[m * NTT + tt][r] = fmaf(s[m], acc[m][r], tot[m * NTT + tt][r]);
                }
            }
            tile_store<KB, NTT, MG>(tr[(i + 1) & 1], tm, smem + (size_t)((i + 1) & 1) * Sh::kBytes);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        }
    }

    if (KSG > 1) {
        const int tile_id = (e * RB + rb) * NTB + tb;
        constexpr size_t stride = (size_t)2 * NTT * 4 * 512;
        if constexpr (kSplitsInKernel<NTT>) {
            if (!split_reduce<2 * NTT>(tot, a.part_gu + (size_t)tile_id * KSG * stride, stride, ks, KSG,
                                       a.cnt_gu + tile_id, &s_last))
                return;   // another split of the tile finishes it
        } else {
            store_partial<2 * NTT>(tot, a.part_gu + ((size_t)tile_id * KSG + ks) * stride);
            return;   // k_tb_gu_finish adds the splits
        }
    }
    gu_epilogue<KB, NTT>(a, tot, e, rb, tb, reinterpret_cast<float *>(smem + 2 * Sh::kBytes));
}

// gate_up finish for split tiles: one block per (expert, row block, token
// tile, 16 tokens of it) adds the splits' partial sums in split order, then
// the epilogue for those 16 tokens (the NTT blocks of a tile share nothing:
// NTT times the blocks, each a fraction of the work).
template <int KB, int NTT>
__global__ __launch_bounds__(512) void k_tb_gu_finish(TbArgs a)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int TT = 16 * NTT;
    const int NTB = (a.T + TT - 1) / TT;
    const int RB = (a.d_ff + kTileRows - 1) / kTileRows;
    int tile_id, tt, e, rb, tb16;
    if (a.top_k) {
        // Routed mode: block (row block rb, chunk c) takes the c-th 16-slot
        // chunk of the experts' slot lists, taken in expert order; the grid
        // holds at least as many chunks as there can be (T top_k / 16 +
        // n_experts per row block), and blocks past the last one exit.
        const int C = gridDim.x / RB;
        rb = blockIdx.x / C;
        int c = blockIdx.x % C;
        for (e = 0; e < a.n_experts; ++e) {
            const int n16 = (a.cnt[e] + 15) >> 4;
            if (c < n16) break;
            c -= n16;
        }
        if (e == a.n_experts) return;
        tb16 = c;
        tt = c % NTT;
        tile_id = (e * RB + rb) * NTB + c / NTT;
    } else {
        tile_id = blockIdx.x / NTT;
        tt = blockIdx.x % NTT;
        const int tb = tile_id % NTB;
        rb = (tile_id / NTB) % RB;
        e = tile_id / NTB / RB;
        tb16 = tb * NTT + tt;   // the block's 16 tokens, as a 16-token tile
    }
    constexpr size_t stride = (size_t)2 * NTT * 4 * 512;
    f32x4 tot[2];
    sum_partials<2>(tot, a.part_gu + (size_t)tile_id * a.ks_gu * stride, stride, a.ks_gu, {tt, NTT + tt});
    gu_epilogue<KB, 1>(a, tot, e, rb, tb16, reinterpret_cast<float *>(smem));
}

// out rows of the wave's 16 d_model rows for the tile's tokens.
template <int NTT>
__device__ __forceinline__ void dn_store(const TbArgs &a, const f32x4 (&tot)[NTT], int rb, int tb)
{
    const int lane = threadIdx.x & 63, q = lane >> 4, n = lane & 15;
    const int wrow0 = rb * kTileRows + (threadIdx.x >> 6) * 16;
    const int t0 = tb * 16 * NTT;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + tt * 16 + 4 * q + i;
            const int r = wrow0 + n;
            if (t < a.T && r < a.d_model) a.out[(size_t)t * a.d_model + r] = tot[tt][i];
        }
}

// down, tiled: block (token tile, row block, split) sums the (expert, group)
// pairs of its split, all experts together (the router weights are in the
// hidden factors).
template <int BITS, int KB, int NTT, int SB>
__global__ __launch_bounds__(512) void k_tb_down_tiled(TbArgs a)
{
    using CU = CodeUnit<BITS, KB>;
    constexpr int kG = CU::kGroups;
    constexpr int TT = 16 * NTT;
    constexpr int group = 32 * KB;
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_last;   // whether this block adds the tile's K splits
    const int d_model = a.d_model, d_ff = a.d_ff, T = a.T, E = a.n_experts;
    constexpr size_t tb_bytes = TileShape<KB, NTT>::kBytes;
    float *fac = reinterpret_cast<float *>(smem + 2 * tb_bytes);  // [2][TT]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int Gd = d_ff / group;
    const int NTB = (T + TT - 1) / TT;
    const int KSD = a.ks_dn;
    // Logical block order: token tile, row block, split (the blocks an XCD
    // gets share codes across token tiles and hidden tiles across row blocks).
    const int RB = (d_model + kTileRows - 1) / kTileRows;
    int bid = xcd_logical(blockIdx.x, gridDim.x);
    int tb, rb, ks;   // routed mode (one split): ks is the block's expert
    if (a.top_k) {
        // Routed mode, order chunk, row block: chunk c is the c-th token tile
        // of the experts' slot lists, taken in expert order (the grid holds an
        // upper bound of them; blocks past the last exit).
        const int C = gridDim.x / RB;
        int c = bid % C;
        rb = bid / C;
        for (ks = 0; ks < E; ++ks) {
            const int nt = (a.cnt[ks] + TT - 1) / TT;
            if (c < nt) break;
            c -= nt;
        }
        if (ks == E) return;   // whole block, before any barrier
        tb = c;
    } else {
        tb = bid % NTB;
        bid /= NTB;
        rb = bid % RB;
        ks = bid / RB;
    }
    const int t0 = tb * TT;
    const int rows = a.top_k ? a.cnt[ks] : T;   // routed mode: expert ks's slots
    if (t0 >= rows) return;                      // whole block, before any barrier
    const int wrow0 = rb * kTileRows + wave * 16;
    const unsigned row = (unsigned)min(wrow0 + n, d_model - 1);
    const unsigned crow = row * (unsigned)(d_ff * BITS / 8) + 16u * (unsigned)(q % CU::kDw);
    const int cq = q / CU::kDw;
    const unsigned srow = row * (unsigned)Gd;
    const int cb = CU::cb(q);
    const size_t cbytes = (size_t)d_model * d_ff * BITS / 8, sbytes = (size_t)d_model * Gd * SB;
    const size_t hbytes = (size_t)T * d_ff * 2;   // one expert's hidden half
    const BufRes fr_res = buf_res(a.hf, (size_t)E * Gd * a.t_pad * 4);
    TileMap<KB, NTT> tm;
    tile_map<KB, NTT>(tm, wave, (unsigned)d_ff * 2u, t0, rows);
    // The block's K range, in iterations of 4 groups of one expert (IPE per
    // expert; a group index past Gd is a dead step): its split of all the
    // experts' iterations, or in routed mode those of its expert.  Step s of
    // the block is group 4 (it % IPE) + s % 4 of expert it / IPE, it = it0 + s / 4.
    const int IPE = (Gd + 3) / 4;
    const int it0 = a.top_k ? ks * IPE : (int)((long)ks * (E * IPE) / KSD);
    const int NSS = 4 * ((a.top_k ? it0 + IPE : (int)((long)(ks + 1) * (E * IPE) / KSD)) - it0);
    const unsigned flane = (unsigned)(lane & (TT - 1));   // a token of the tile (repeats for TT < 64)
    struct Pos {
        int e, g;   // expert, first group of an iteration
    };
    auto iter_pos = [&](int it) -> Pos {   // iteration it of the block (clamped to its last)
        const int ia = it0 + min(it, NSS / 4 - 1);
        const int e = ia / IPE;
        return {e, 4 * (ia - e * IPE)};
    };

    f32x4 tot[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) tot[tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Loads and rings as in gate_up: hidden pieces and the tile's factors of
    // step s in slot s % R (issued at the start of step s - R, stored to LDS at
    // the end of step s - 1); the next code unit and scale quad once the
    // current ones are unpacked.  Loads complete in issue order, so the ring's
    // depth bounds how far ahead the tile loads run; 16-token tiles, with
    // little work a step and a few registers a slot, gain from four (about a
    // tenth of the kernel's time), larger tiles and deeper code-unit rings
    // measured no gain.  Loads past the range repeat its last iteration; dead
    // steps clamp to the expert's last group; both count with scale 0.
    constexpr int R = NTT == 1 ? 4 : 2;
    TileRegs<KB, NTT> tr[R];
    float frr[R];
    uint4 craw;
    unsigned sraw;
    CodeWords<BITS, KB> cw[kG];
    float sc[4];
    auto load_tile = [&](int slot, Pos ps, int r) {   // group ps.g + r of expert ps.e
        const int g = min(ps.g + r, Gd - 1);
        const size_t ho = (size_t)ps.e * T * d_ff;
        tile_load<KB, NTT>(tr[slot], tm, buf_res(a.hh + ho, hbytes), buf_res(a.hl + ho, hbytes),
                           (unsigned)g * (unsigned)group * 2u);
        frr[slot] = __uint_as_float(
            buf_load4(fr_res, flane * 4u, (unsigned)(((size_t)ps.e * Gd + g) * a.t_pad + t0) * 4u));
    };
    auto load_unit = [&](Pos ps, int r) {   // the unit whose first group is ps.g + r
        const unsigned off = crow + (unsigned)min(ps.g + r + cq, Gd - 1) * (unsigned)(16 * CU::kDw);
        craw = buf_load16(buf_res(a.down[ps.e].codes, cbytes), off, 0u);
    };
    auto load_quad = [&](Pos ps) {
        sraw = buf_load_scale_bits<SB>(buf_res(a.down[ps.e].scales, sbytes), srow + (unsigned)min(ps.g + q, Gd - 1));
    };
    auto store_tile = [&](int slot, int buf) {
        tile_store<KB, NTT>(tr[slot], tm, smem + (size_t)buf * tb_bytes);
        fac[buf * TT + flane] = frr[slot];
    };

    {
        const Pos p0 = iter_pos(0);
        load_unit(p0, 0);
        load_quad(p0);
#pragma unroll
        for (int j = 0; j < R; ++j) load_tile(j, p0, j);
    }
    __builtin_amdgcn_sched_barrier(0);
    store_tile(0, 0);
    __syncthreads();
    for (int base = 0; base < NSS; base += 4) {
        const Pos cur = iter_pos(base / 4), nxt = iter_pos(base / 4 + 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i % kG == 0) {   // a code unit starts; load the next one
                unit_split<BITS, KB>(craw, cw);
                if (i + kG < 4)
                    load_unit(cur, i + kG);
                else
                    load_unit(nxt, 0);
            }
            if (i == 0) {   // a scale quad starts: group j of it from lane row j
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    sc[j] = scale_value<SB>((unsigned)__builtin_amdgcn_ds_bpermute((n + 16 * j) * 4, (int)sraw)) *
                            QFormat<BITS>::kInvZ;
                load_quad(nxt);
            }
            if (i + R < 4)
                load_tile(i % R, cur, i + R);
            else
                load_tile(i % R, nxt, i + R - 4);
            __builtin_amdgcn_sched_barrier(0);
            const uint8_t *tile = smem + (size_t)(i & 1) * tb_bytes;
            half8 bf[KB];
#pragma unroll
            for (int j = 0; j < KB; ++j) bf[j] = code_frag<BITS, KB>(cw[i % kG], j);
            const float s = cur.g + i < Gd ? sc[i] : 0.0f;
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KB; ++j) {
                    half8 h, l;
                    tile_frags<KB, NTT>(tile, tt, 0, j, cb, h, l);
                    acc = mfma(h, bf[j], acc);
                    acc = mfma(l, bf[j], acc);
                }
                const f32x4 f = *reinterpret_cast<const f32x4 *>(fac + (i & 1) * TT + tt * 16 + 4 * q);
#pragma unroll
                for (int r = 0; r < 4; ++r) tot[tt][r] = fmaf(s * f[r], acc[r], tot[tt][r]);
            }
            store_tile((i + 1) % R, (i + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
            __syncthreads();
        }
    }

    if (a.top_k) {
        // Routed mode: the weighted output row of each of the tile's slots.
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = t0 + tt * 16 + 4 * q + i;
                const int r = wrow0 + n;
                if (p < rows && r < d_model) a.ys[(size_t)a.list[(size_t)ks * T + p] * d_model + r] = tot[tt][i];
            }
        return;
    }
    if (KSD > 1) {
        const int tile_id = rb * NTB + tb;
        constexpr size_t stride = (size_t)NTT * 4 * 512;
        if constexpr (kSplitsInKernel<NTT>) {
            if (!split_reduce<NTT>(tot, a.part_dn + (size_t)tile_id * KSD * stride, stride, ks, KSD,
                                   a.cnt_dn + tile_id, &s_last))
                return;   // another split of the tile finishes it
        } else {
            store_partial<NTT>(tot, a.part_dn + ((size_t)tile_id * KSD + ks) * stride);
            return;   // k_tb_dn_finish adds the splits
        }
    }
    dn_store<NTT>(a, tot, rb, tb);
}

// down finish for split tiles: one block per (row block, token tile, 16
// tokens of it) adds the splits' partial sums in split order and writes out.
template <int NTT>
__global__ __launch_bounds__(512) void k_tb_dn_finish(TbArgs a)
{
    constexpr int TT = 16 * NTT;
    const int NTB = (a.T + TT - 1) / TT;
    const int tile_id = blockIdx.x / NTT, tt = blockIdx.x % NTT;
    constexpr size_t stride = (size_t)NTT * 4 * 512;
    f32x4 tot[1];
    sum_partials<1>(tot, a.part_dn + (size_t)tile_id * a.ks_dn * stride, stride, a.ks_dn, {tt});
    dn_store<1>(a, tot, tile_id / NTB, (tile_id % NTB) * NTT + tt);
}

// -------------------------------------------------------------------------
// Streaming kernels for batches of at most 16 tokens (one token tile).
//
// There a quantisation group of codes carries 16 tokens of matrix work, and
// what bounds a pass is how many code bytes each CU keeps in flight.  These
// kernels hold the tokens' activations for a long stretch of K in LDS, issue
// each wave's codes and scales a whole phase ahead of their use, and meet at
// a barrier once per phase of 16 groups (gate_up) or once per chunk (down)
// instead of once per group.
//
// gate_up: a block of 12 waves owns 3 row tiles (16 rows of gate and of up
// each) over all of d_model, so K is not split: wave (r, k) takes groups
// 4k .. 4k+3 of every 16-group phase for row tile r, and the four K quarters
// of a row tile are added in LDS at the end.  X enters each phase as f32: the
// block scales it per token by the power of two of the phase's largest |x|
// (one exponent per token and phase), splits it into f16 hi/lo halves in
// sigma order in LDS, and the phase's sums are scaled back by the same power
// of two.  The hidden rows SiLU(g) * u leave as f32.
//
// Routed mode (T <= 16, d_ff <= 1536): a gate_up block's row tiles are one
// expert's and its token rows the expert's slots, which it lists itself; a
// down block's chunk is one expert's d_ff, and it writes each slot's
// weighted row for the combine pass instead of adding the experts.
//
// down: a block of 16 waves owns 8 row tiles (128 rows of d_model) and one
// chunk of 1536 columns of one expert's d_ff (all of it at d_ff = 1536).  The
// hidden rows are scaled per (token, group) by the power of two of the
// group's largest |h| and split into hi/lo halves on the way into LDS, and the
// router weight joins that power of two in the group's factor, as in the
// tiled path.  The two K halves of a row tile are added in LDS, the chunks
// of a row group in the kernel through the row group's counter, in chunk
// order (the counters are zeroed by gate_up, which runs before down).
constexpr int kGsRows = 3, kGsK = 4, kGsWaves = kGsRows * kGsK;
constexpr int kPhaseGroups = 16;
constexpr int kDsRows = 8, kDsK = 2, kDsWaves = kDsRows * kDsK;
constexpr int kDsCols = 1536;

// A buffer load at or past this byte offset is outside every buffer here
// (extents are below 2^31) and returns zeros.
constexpr unsigned kPastExtent = 0x80000000u;

// 8 f32 values of a 32-byte piece (two 16-byte loads).
__device__ __forceinline__ void piece_values(const uint4 (&raw)[2], float (&v)[8])
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        v[4 * h + 0] = __uint_as_float(raw[h].x);
        v[4 * h + 1] = __uint_as_float(raw[h].y);
        v[4 * h + 2] = __uint_as_float(raw[h].z);
        v[4 * h + 3] = __uint_as_float(raw[h].w);
    }
}

// hi/lo halves of v * 2^-e in sigma order, stored as two 16-byte LDS writes
// (hi rounded once, as packed pairs, and widened back from them).
typedef float f32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void store_hilo(const float (&v)[8], int e, _Float16 *hi, _Float16 *lo)
{
    constexpr int kSigma[8] = {0, 4, 1, 5, 2, 6, 3, 7};   // column at each sigma position
    f32x8 sv;
#pragma unroll
    for (int i = 0; i < 8; ++i) sv[i] = ldexpf(v[kSigma[i]], -e);
    const half8 h = __builtin_convertvector(sv, half8);
    const half8 l = __builtin_convertvector(sv - __builtin_convertvector(h, f32x8), half8);
    *reinterpret_cast<half8 *>(hi) = h;
    *reinterpret_cast<half8 *>(lo) = l;
}

template <int BITS, int KB, int SB>
__global__ __launch_bounds__(64 * kGsWaves) void k_tb_gate_up_stream(TbArgs a)
{
    using CU = CodeUnit<BITS, KB>;
    constexpr int kG = CU::kGroups, kDw = CU::kDw;
    constexpr int kWG = kPhaseGroups / kGsK;   // groups of a phase per wave
    constexpr int kU = kWG / kG;               // code units of a phase per wave
    static_assert(kWG == 4 && kU * kG == kWG, "a wave takes one scale quad and whole code units per phase");
    constexpr int group = 32 * KB;
    constexpr int KC = kPhaseGroups * group;   // columns per phase
    constexpr int kStride = KC + 8;            // halfs per LDS token row
    constexpr int kTile = 2 * 16 * kStride;    // halfs per tile: hi [16][kStride], lo [16][kStride]
    constexpr int kNT = 64 * kGsWaves;
    constexpr int kPR = KC / 8;                // 8-column pieces per token row
    constexpr int kPieces = 16 * kPR;
    constexpr int kPPT = (kPieces + kNT - 1) / kNT;
    extern __shared__ __align__(16) unsigned char smem[];   // two tiles
    __shared__ unsigned s_max[3][16];                       // per phase mod 3 and token: largest |x| (bits)
    __shared__ __align__(16) int s_exp[2][16];              // per phase parity and token: its exponent
    _Float16 *tiles = reinterpret_cast<_Float16 *>(smem);

    const int d_model = a.d_model, d_ff = a.d_ff, T = a.T;
    const int lane = threadIdx.x & 63, q = lane >> 4, n = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = wave / kGsK, wk = wave % kGsK;
    const int G = d_model / group;
    const int P = (G + kPhaseGroups - 1) / kPhaseGroups;   // phases of 16 groups
    const int RT = d_ff / 16, NRT = a.n_experts * RT;

    // The wave's row tile (past the last one: a copy of it that stores
    // nothing), and the tile's token rows: the batch (dense), or the slots
    // of the block's expert, whose row tiles its blocks cover in turn
    // (routed; a block of an expert without slots has nothing to do).
    int e, rt, rows;
    bool live;
    __shared__ int s_list[16];   // routed: the expert's slots, ascending
    __shared__ int s_wcnt[4];
    const int bpe = (RT + kGsRows - 1) / kGsRows;
    if (a.top_k) {
        e = blockIdx.x / bpe;
        const int rtb = (blockIdx.x - e * bpe) * kGsRows + rl;
        live = rtb < RT;
        rt = min(rtb, RT - 1);
        // The expert's slots (T * top_k <= 256 of them, one per thread of the
        // first four waves) in ascending order, by ballot prefix counts; an
        // expert keeps at most T slots (a token's ids are distinct, so none
        // is lost).  The expert's first block publishes the list, its length
        // and the slots' flags for the down and combine passes.
        const int ns = T * a.top_k, sl = threadIdx.x;
        const bool mine = sl < 256 && sl < ns && a.ids[sl] == e;
        const unsigned long long mask = __ballot(mine);
        if (lane == 0 && wave < 4) s_wcnt[wave] = __popcll(mask);
        __syncthreads();
        int before = 0;
        for (int w = 0; w < wave && w < 4; ++w) before += s_wcnt[w];
        const int pos = before + __popcll(mask & ((1ull << lane) - 1ull));
        rows = min(s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3], T);
        if (mine && pos < T) s_list[pos] = sl;
        if (blockIdx.x % bpe == 0) {
            if (mine) {
                if (pos < T) a.list[(size_t)e * T + pos] = sl;
                a.slot_ok[sl] = pos < T;
            }
            if (threadIdx.x == 0) a.cnt[e] = rows;
        }
        __syncthreads();
        if (rows == 0) return;   // whole block (rows is the same for every thread)
    } else {
        const int rtg = blockIdx.x * kGsRows + rl;
        live = rtg < NRT;
        const int rtc = min(rtg, NRT - 1);
        e = rtc / RT;
        rt = rtc - e * RT;
        rows = T;
        // The down pass's chunk counters start every call at zero.
        for (int i = blockIdx.x * kNT + threadIdx.x; i < a.n_cnt; i += gridDim.x * kNT) a.cnt_gu[i] = 0u;
    }
    if (threadIdx.x < 48) s_max[threadIdx.x >> 4][threadIdx.x & 15] = 0u;
    const int *list = a.top_k ? s_list : nullptr;
    // Routed mode: the expert's first block keeps each position's slot
    // weight for the down pass.
    if (list && blockIdx.x % bpe == 0 && threadIdx.x < rows)
        a.hf[(size_t)e * T + threadIdx.x] = a.slot_w[list[threadIdx.x]];
    const int wrow0 = rt * 16;
    const unsigned row = (unsigned)(wrow0 + n);
    const unsigned crow = row * (unsigned)(d_model * BITS / 8) + 16u * (unsigned)(q % kDw);
    const int cq = q / kDw;
    const unsigned srow = row * (unsigned)G;
    const int cb = CU::cb(q);
    const size_t cbytes = (size_t)d_ff * d_model * BITS / 8, sbytes = (size_t)d_ff * G * SB;
    const BufRes cr[2] = {buf_res(a.gate[e].codes, cbytes), buf_res(a.up[e].codes, cbytes)};
    const BufRes sr[2] = {buf_res(a.gate[e].scales, sbytes), buf_res(a.up[e].scales, sbytes)};
    const BufRes xr = buf_res(a.x, (size_t)T * d_model * 4);

    // Loads complete in issue order, so X (an L2 read) is always issued
    // before the codes (HBM) that are not needed as soon.  Codes and scales
    // of phase ph are issued one phase ahead, once phase ph - 1's are
    // unpacked; the thread's pieces of X for phase ph go to registers two
    // phases ahead (tokens past T and columns past d_model read as zero).
    // Where all of the wave's groups of a phase exist, a code or scale load
    // is a fixed lane offset plus the phase's first group as a uniform
    // offset, and stays inside the lane's row.  Otherwise (a partial last
    // phase, or the phase after the last, which the last iteration loads)
    // each lane's group is clamped to the last one, whole offset per lane;
    // groups past the last count with scale 0 against activation columns of
    // zeros.
    uint4 craw[2][kU];
    unsigned sraw[2];
    unsigned cvo[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) cvo[u] = crow + (unsigned)((u * kG + cq) * 16 * kDw);
    const unsigned svo = (srow + (unsigned)q) * SB;
    auto load_codes = [&](int ph) {
        const int g0 = ph * kPhaseGroups + wk * kWG;
        if (g0 + kWG <= G) {   // uniform
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int u = 0; u < kU; ++u) craw[m][u] = buf_load16(cr[m], cvo[u], (unsigned)g0 * (16u * kDw));
                sraw[m] = buf_load_scale_at<SB>(sr[m], svo, (unsigned)g0 * SB);
            }
        } else {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int u = 0; u < kU; ++u)
                    craw[m][u] = buf_load16(cr[m], crow + (unsigned)min(g0 + u * kG + cq, G - 1) * (16u * kDw), 0u);
                sraw[m] = buf_load_scale_at<SB>(sr[m], (srow + (unsigned)min(g0 + q, G - 1)) * SB, 0u);
            }
        }
    };
    // Row of X behind each of the thread's pieces (-1: past the tile's rows).
    int xrow[kPPT];
#pragma unroll
    for (int k = 0; k < kPPT; ++k) {
        const int c = threadIdx.x + kNT * k, p = c / kPR;
        xrow[k] = c < kPieces && p < rows ? (list ? list[p] / a.top_k : p) : -1;
    }
    // A piece outside X gets an offset past the buffer's extent, where a
    // buffer load returns zeros.
    auto load_x = [&](uint4 (&xv)[kPPT][2], int ph) {
#pragma unroll
        for (int k = 0; k < kPPT; ++k) {
            const int c = threadIdx.x + kNT * k, b8 = c % kPR, col = ph * KC + 8 * b8;
            const bool ok = xrow[k] >= 0 && col < d_model;
            const unsigned off = ok ? (unsigned)(xrow[k] * d_model + col) * 4u : kPastExtent;
            xv[k][0] = buf_load16(xr, off, 0u);
            xv[k][1] = buf_load16(xr, off + 16u, 0u);
        }
    };
    // The per-token maxima of phase ph's X, into s_max[ph % 3] (read after
    // the next barrier).
    auto max_x = [&](const uint4 (&xv)[kPPT][2], int ph) {
        unsigned *mx = s_max[ph % 3];
#pragma unroll
        for (int k = 0; k < kPPT; ++k) {
            const int t = (threadIdx.x + kNT * k) / kPR;
            float v[8];
            piece_values(xv[k], v);
            float m = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
            if (threadIdx.x + kNT * k < kPieces) atomicMax(&mx[t], __float_as_uint(m));
        }
    };
    // Phase ph's X into tile ph & 1 as hi/lo halves scaled by the tokens'
    // exponents, which go to s_exp[ph & 1].
    auto convert_x = [&](const uint4 (&xv)[kPPT][2], int ph) {
        const unsigned *mx = s_max[ph % 3];
        _Float16 *hi = tiles + (ph & 1) * kTile, *lo = hi + 16 * kStride;
        if (threadIdx.x < 16) s_exp[ph & 1][threadIdx.x] = norm_exponent(__uint_as_float(mx[threadIdx.x]));
#pragma unroll
        for (int k = 0; k < kPPT; ++k) {
            const int c = threadIdx.x + kNT * k;
            if (c < kPieces) {
                const int t = c / kPR, b8 = c - t * kPR;
                float v[8];
                piece_values(xv[k], v);
                store_hilo(v, norm_exponent(__uint_as_float(mx[t])), hi + t * kStride + 8 * b8,
                           lo + t * kStride + 8 * b8);
            }
        }
    };

    f32x4 tot[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // gate, up
    // The MFMAs of phase ph from tile ph & 1 and the unpacked codes, added into
    // tot with the phase's exponents.
    auto compute = [&](int ph, const CodeWords<BITS, KB> (&cw)[2][kU][kG], const float (&sc)[2][4]) {
        const _Float16 *hi = tiles + (ph & 1) * kTile, *lo = hi + 16 * kStride;
        f32x4 tp[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int gi = 0; gi < kWG; ++gi) {
            const int lg = wk * kWG + gi;   // group within the phase
            half8 bf[2][KB];
            float s[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int j = 0; j < KB; ++j) bf[m][j] = code_frag<BITS, KB>(cw[m][gi / kG][gi % kG], j);
                s[m] = ph * kPhaseGroups + lg < G ? sc[m][gi] : 0.0f;
            }
            f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int off = n * kStride + lg * group + cb * 8 * KB + 8 * j;
                const half8 h = load_half8(hi + off), l = load_half8(lo + off);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    acc[m] = mfma(h, bf[m][j], acc[m]);
                    acc[m] = mfma(l, bf[m][j], acc[m]);
                }
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int r = 0; r < 4; ++r) tp[m][r] = fmaf(s[m], acc[m][r], tp[m][r]);
        }
        const int4 ex = *reinterpret_cast<const int4 *>(&s_exp[ph & 1][4 * q]);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            tot[m][0] += ldexpf(tp[m][0], ex.x);
            tot[m][1] += ldexpf(tp[m][1], ex.y);
            tot[m][2] += ldexpf(tp[m][2], ex.z);
            tot[m][3] += ldexpf(tp[m][3], ex.w);
        }
    };
    // The loaded codes and scales, unpacked.
    auto unpack = [&](CodeWords<BITS, KB> (&cw)[2][kU][kG], float (&sc)[2][4]) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int u = 0; u < kU; ++u) unit_split<BITS, KB>(craw[m][u], cw[m][u]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                sc[m][j] = scale_value<SB>((unsigned)__builtin_amdgcn_ds_bpermute((n + 16 * j) * 4, (int)sraw[m])) *
                           QFormat<BITS>::kInvZ;
        }
    };

    // Phase ph of the loop (one barrier per phase): tile ph is complete and
    // the maxima of phase ph + 1 are in; X of phase ph + 1 goes into the other
    // tile (last read in phase ph - 1) while the waves run phase ph, whose
    // codes are unpacked before phase ph + 1's take their registers.  Phase
    // ph + 2's maxima join before the barrier; s_max[ph % 3] was last read in
    // phase ph - 1 and is cleared for phase ph + 3.
    uint4 xv[kPPT][2], xv1[kPPT][2];
    __syncthreads();   // the maxima are zero
    load_x(xv, 0);
    load_x(xv1, 1);
    load_codes(0);
    max_x(xv, 0);
    max_x(xv1, 1);
    __builtin_amdgcn_sched_barrier(0);   // nothing that waits for the codes moves above a barrier
    __syncthreads();
    convert_x(xv, 0);
#pragma unroll
    for (int k = 0; k < kPPT; ++k) xv[k][0] = xv1[k][0], xv[k][1] = xv1[k][1];
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    // Branch-free, so that the compiler's load waits are exact: the loads
    // and conversions past the last phase are of phases with no columns.
    for (int p = 0; p < P; ++p) {
        convert_x(xv, p + 1);
        CodeWords<BITS, KB> cw[2][kU][kG];
        float sc[2][4];
        unpack(cw, sc);
        load_x(xv, p + 2);
        load_codes(p + 1);
        compute(p, cw, sc);
        if (threadIdx.x < 16) s_max[p % 3][threadIdx.x] = 0u;
        max_x(xv, p + 2);
        __syncthreads();
    }

    // The four K quarters of each row tile, added in LDS in quarter order
    // (the tiles are no longer read after the last barrier).
    float *red = reinterpret_cast<float *>(smem);
    if (wk > 0) {
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[(((rl * (kGsK - 1) + wk - 1) * 2 + m) * 4 + r) * 64 + lane] = tot[m][r];
    }
    __syncthreads();
    if (wk != 0 || !live) return;
#pragma unroll
    for (int w = 1; w < kGsK; ++w)
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[m][r] += red[(((rl * (kGsK - 1) + w - 1) * 2 + m) * 4 + r) * 64 + lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = 4 * q + i;   // token (dense) or position in the expert's slot list (routed)
        if (p < rows) a.hid[((size_t)e * T + p) * d_ff + wrow0 + n] = silu(tot[0][i]) * tot[1][i];
    }
}

template <int BITS, int KB, int SB>
__global__ __launch_bounds__(64 * kDsWaves) void k_tb_down_stream(TbArgs a)
{
    using CU = CodeUnit<BITS, KB>;
    constexpr int kG = CU::kGroups, kDw = CU::kDw;
    constexpr int group = 32 * KB;
    constexpr int KDG = kDsCols / group;   // groups per block
    constexpr int kWG = KDG / kDsK;        // groups per wave
    constexpr int kU = kWG / kG;           // code units per wave
    constexpr int kQ = kWG / 4;            // scale quads per wave
    static_assert(kU * kG == kWG && kQ * 4 == kWG, "a wave takes whole code units and scale quads");
    constexpr int kStride = kDsCols + 8;
    constexpr int kNT = 64 * kDsWaves;
    constexpr int kPR = kDsCols / 8;       // 8-column pieces per token row
    constexpr int kPieces = 16 * kPR;
    constexpr int kPPT = kPieces / kNT;
    static_assert(kPPT * kNT == kPieces, "every thread takes the same number of pieces");
    constexpr int kPG = group / 8;         // pieces per group
    extern __shared__ __align__(16) unsigned char smem[];   // hi [16][kStride], lo [16][kStride], factors [KDG][16]
    __shared__ int s_last;
    _Float16 *hs_hi = reinterpret_cast<_Float16 *>(smem), *hs_lo = hs_hi + 16 * kStride;
    float *fac = reinterpret_cast<float *>(smem + (size_t)2 * 16 * kStride * 2);

    const int d_model = a.d_model, d_ff = a.d_ff, T = a.T, E = a.n_experts;
    const int lane = threadIdx.x & 63, q = lane >> 4, n = lane & 15;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rl = wave / kDsK, kh = wave % kDsK;
    const int Gd = d_ff / group;
    const int SPE = (d_ff + kDsCols - 1) / kDsCols, S = E * SPE;
    const int RG = (d_model + 16 * kDsRows - 1) / (16 * kDsRows);
    // Logical order chunk, row group: the blocks an XCD gets share a chunk of
    // hidden rows.
    const int b = xcd_logical(blockIdx.x, gridDim.x);
    const int sp = b / RG, rg = b - sp * RG;
    const int e = sp / SPE, kc = sp - e * SPE;
    // Token rows of the chunk: the batch (dense), or the positions of the
    // expert's slot list (routed, one chunk per expert; none: nothing to do).
    const int rows = a.top_k ? a.cnt[e] : T;
    if (rows == 0) return;   // whole block, before any barrier
    const int wrow0 = rg * 16 * kDsRows + rl * 16;
    const unsigned row = (unsigned)min(wrow0 + n, d_model - 1);
    const unsigned crow = row * (unsigned)(d_ff * BITS / 8) + 16u * (unsigned)(q % kDw);
    const int cq = q / kDw;
    const unsigned srow = row * (unsigned)Gd;
    const int cb = CU::cb(q);
    const size_t cbytes = (size_t)d_model * d_ff * BITS / 8, sbytes = (size_t)d_model * Gd * SB;
    const BufRes cres = buf_res(a.down[e].codes, cbytes), sres = buf_res(a.down[e].scales, sbytes);

    // The chunk's hidden rows, then all of the wave's codes and scales (loads
    // complete in issue order: the hidden rows are staged while the codes
    // arrive).
    const int wg0 = kc * KDG + kh * kWG;   // the wave's first group of d_ff
    const BufRes hr = buf_res(a.hid + (size_t)e * T * d_ff, (size_t)T * d_ff * 4);
    const int c0 = kc * kDsCols;
    // Router weights of the pieces' rows, loaded with the hidden rows (a load
    // issued after the codes would be waited for behind all of them): the
    // token's weight for the expert (dense), or the slot's weight, which
    // gate_up kept by position (routed).
    const bool rwv = a.top_k || a.route_w;
    const BufRes rr = a.top_k ? buf_res(a.hf + (size_t)e * T, (size_t)T * 4)
                              : buf_res(a.route_w ? a.route_w : a.out, a.route_w ? (size_t)T * E * 4 : 4);
    uint4 hv[kPPT][2];
    unsigned rw[kPPT];
#pragma unroll
    for (int k = 0; k < kPPT; ++k) {
        const int c = threadIdx.x + kNT * k, t = c / kPR, b8 = c - t * kPR;
        const bool ok = t < rows && c0 + 8 * b8 < d_ff;
        const unsigned off = ok ? (unsigned)(t * d_ff + c0 + 8 * b8) * 4u : kPastExtent;   // zeros past X
        hv[k][0] = buf_load16(hr, off, 0u);
        hv[k][1] = buf_load16(hr, off + 16u, 0u);
        const unsigned woff = a.top_k ? (unsigned)t * 4u : (unsigned)(t * E + e) * 4u;
        rw[k] = buf_load4(rr, rwv && t < rows ? woff : 0u, 0u);
    }
    uint4 craw[kU];
    unsigned sraw[kQ];
#pragma unroll
    for (int u = 0; u < kU; ++u)
        craw[u] = buf_load16(cres, crow + (unsigned)min(wg0 + u * kG + cq, Gd - 1) * (unsigned)(16 * kDw), 0u);
#pragma unroll
    for (int k = 0; k < kQ; ++k) sraw[k] = buf_load_scale_bits<SB>(sres, srow + (unsigned)min(wg0 + 4 * k + q, Gd - 1));
    // Per (token, group): the largest |h| over the group's kPG pieces, held
    // by kPG consecutive lanes (kNT and kPR are multiples of 8).
#pragma unroll
    for (int k = 0; k < kPPT; ++k) {
        const int c = threadIdx.x + kNT * k, t = c / kPR, b8 = c - t * kPR;
        float v[8];
        piece_values(hv[k], v);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
#pragma unroll
        for (int s = 1; s < kPG; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
        const int ex = norm_exponent(m);
        store_hilo(v, ex, hs_hi + t * kStride + 8 * b8, hs_lo + t * kStride + 8 * b8);
        if (b8 % kPG == 0) {
            const float rwt = t >= rows ? 0.0f : rwv ? __uint_as_float(rw[k]) : 1.0f;
            fac[(b8 / kPG) * 16 + t] = ldexpf(rwt, ex);
        }
    }
    __builtin_amdgcn_sched_barrier(0);   // nothing that waits for the codes moves above the barrier
    __syncthreads();

    CodeWords<BITS, KB> cw[kU][kG];
#pragma unroll
    for (int u = 0; u < kU; ++u) unit_split<BITS, KB>(craw[u], cw[u]);
    f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kQ; ++k) {
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            sc[j] = scale_value<SB>((unsigned)__builtin_amdgcn_ds_bpermute((n + 16 * j) * 4, (int)sraw[k])) *
                    QFormat<BITS>::kInvZ;
#pragma unroll
        for (int j4 = 0; j4 < 4; ++j4) {
            const int gi = 4 * k + j4, lg = kh * kWG + gi;   // group of the wave, of the chunk
            half8 bf[KB];
#pragma unroll
            for (int j = 0; j < KB; ++j) bf[j] = code_frag<BITS, KB>(cw[gi / kG][gi % kG], j);
            const float s = wg0 + gi < Gd ? sc[j4] : 0.0f;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                const int off = n * kStride + lg * group + cb * 8 * KB + 8 * j;
                acc = mfma(load_half8(hs_hi + off), bf[j], acc);
                acc = mfma(load_half8(hs_lo + off), bf[j], acc);
            }
            const f32x4 f = *reinterpret_cast<const f32x4 *>(fac + lg * 16 + 4 * q);
#pragma unroll
            for (int r = 0; r < 4; ++r) tot[r] = fmaf(s * f[r], acc[r], tot[r]);
        }
    }

    // The two K halves of each row tile, added in LDS.
    __syncthreads();
    float *red = reinterpret_cast<float *>(smem);
    if (kh == 1) {
#pragma unroll
        for (int r = 0; r < 4; ++r) red[(rl * 4 + r) * 64 + lane] = tot[r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[r] += red[(rl * 4 + r) * 64 + lane];
    }

    // Routed mode: each slot's weighted output row (k_route_combine adds a
    // token's slots).
    if (a.top_k) {
        if (kh != 0) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int p = 4 * q + i, r = wrow0 + n;
            if (p < rows && r < d_model) a.ys[(size_t)a.list[(size_t)e * T + p] * d_model + r] = tot[i];
        }
        return;
    }
    // The row group's chunks, added by the last of its blocks to finish, in
    // chunk order (published and read as the tiled kernels' K splits are).
    if (S > 1) {
        float *slabs = a.part_dn + (size_t)rg * S * (kDsRows * 256);
        if (kh == 0) {
            float *mine = slabs + ((size_t)sp * kDsRows + rl) * 256;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                __hip_atomic_store(mine + r * 64 + lane, tot[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): this thread's stores have reached memory
        __syncthreads();
        if (threadIdx.x == 0)
            s_last = __hip_atomic_fetch_add(a.cnt_dn + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (unsigned)S - 1;
        __syncthreads();
        if (!s_last || kh != 0) return;
        const f32x4 own = tot;
        constexpr int B = 8;   // slabs in flight at once
        for (int s0 = 0; s0 < S; s0 += B) {
            float v[B][4];
#pragma unroll
            for (int bb = 0; bb < B; ++bb) {
                const int s = min(s0 + bb, S - 1);   // past the last chunk: re-read it, unused
                const float *ps = slabs + ((size_t)s * kDsRows + rl) * 256;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[bb][r] = s == sp ? own[r]
                                       : __hip_atomic_load(const_cast<float *>(ps) + r * 64 + lane, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            }
#pragma unroll
            for (int bb = 0; bb < B; ++bb) {
                if (s0 + bb >= S) break;
#pragma unroll
                for (int r = 0; r < 4; ++r) tot[r] = s0 + bb == 0 ? v[bb][r] : tot[r] + v[bb][r];
            }
        }
    } else if (kh != 0) {
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int t = 4 * q + i, r = wrow0 + n;
        if (t < T && r < d_model) a.out[(size_t)t * d_model + r] = tot[i];
    }
}

template <int BITS, int KB, int SB>
hipError_t launch_tb_stream(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL((k_tb_gate_up_stream<BITS, KB, SB>), dim3(pl.gu_blocks), dim3(64 * kGsWaves), pl.gu_lds,
                       st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_down_stream<BITS, KB, SB>), dim3(pl.dn_blocks), dim3(64 * kDsWaves), pl.dn_lds, st,
                       a);
    return hipGetLastError();
}

template <int BITS, int KB, int NTT, int MG, int SB>
hipError_t launch_tb_tiled(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(k_tb_prep, dim3((unsigned)a.T), dim3(256), 0, st, a.x, a.d_model, a.xh, a.xl, a.xe, a.cnt_gu,
                       a.n_cnt);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_gate_up_tiled<BITS, KB, NTT, MG, SB>), dim3(pl.gu_blocks),
                       dim3(64 * kTileWaves), pl.gu_lds, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.ks_gu > 1 && !kSplitsInKernel<NTT>) {
        hipLaunchKernelGGL((k_tb_gu_finish<KB, NTT>), dim3(pl.gu_blocks / a.ks_gu * NTT), dim3(64 * kTileWaves),
                           (size_t)kTileWaves * 16 * 4, st, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    hipLaunchKernelGGL((k_tb_down_tiled<BITS, KB, NTT, SB>), dim3(pl.dn_blocks), dim3(64 * kTileWaves),
                       pl.dn_lds, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.ks_dn > 1 && !kSplitsInKernel<NTT>) {
        hipLaunchKernelGGL(k_tb_dn_finish<NTT>, dim3(pl.dn_blocks / a.ks_dn * NTT), dim3(64 * kTileWaves), 0, st,
                           a);
        err = hipGetLastError();
    }
    return err;
}

// -------------------------------------------------------------------------
// Routed mode ("Token-Batch Fused FFN": per expert, the tokens that chose it
// run through it together).  Slot s = t*top_k + j of token t goes to expert
// ids[s].  One block per expert lists that expert's slots in ascending order
// (a ballot prefix count per 256 slots), so the lists and hence every sum
// downstream are deterministic.  An expert keeps at most T slots (a token's
// ids are distinct, so no slot is lost); slot_ok[s] marks the kept slots of
// ids in [0, n_experts).
__device__ __forceinline__ void route_bucket(const int *__restrict__ ids, int T, int top_k, int *list, int *cnt,
                                             int *slot_ok, int e)
{
    __shared__ int s_wave[4];
    const int n = T * top_k;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int base = 0;
    for (int c0 = 0; c0 < n; c0 += 256) {
        const int s = c0 + threadIdx.x;
        const bool mine = s < n && ids[s] == e;
        const unsigned long long mask = __ballot(mine);
        const int below = __popcll(mask & ((1ull << lane) - 1ull));
        if (lane == 0) s_wave[wave] = __popcll(mask);
        __syncthreads();
        int before = base;
        for (int w = 0; w < wave; ++w) before += s_wave[w];
        const int total = s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
        if (mine) {
            const int pos = before + below;
            if (pos < T) list[(size_t)e * T + pos] = s;
            slot_ok[s] = pos < T;
        }
        base += total;
        __syncthreads();
    }
    if (threadIdx.x == 0) cnt[e] = min(base, T);
}

// The routed call's first launch: blocks 0 .. n_experts - 1 list the experts'
// slots, the T blocks after them prepare the tokens (the two are independent).
__global__ __launch_bounds__(256) void k_route_prep(TbArgs a)
{
    if ((int)blockIdx.x < a.n_experts)
        route_bucket(a.ids, a.T, a.top_k, a.list, a.cnt, a.slot_ok, blockIdx.x);
    else
        prep_token(a.x, a.d_model, a.xh, a.xl, a.xe, a.cnt_gu, a.n_cnt, blockIdx.x - a.n_experts, a.T);
}

// out[t][:] = sum over the token's slots j (ascending) that were processed of
// ys[t*top_k + j][:] (each already weighted by its router weight).  Block
// (t, c) covers columns 1024 c .. 1024 c + 1023 of token t, four per thread
// (d_model is a multiple of 32, and 16-byte aligned rows of ys).
__global__ __launch_bounds__(256) void k_route_combine(const int *__restrict__ ids, const int *__restrict__ slot_ok,
                                                       const float *__restrict__ ys, int top_k, int n_experts,
                                                       int d_model, float *__restrict__ out)
{
    const int t = blockIdx.x;
    const int r = blockIdx.y * 1024 + threadIdx.x * 4;
    if (r >= d_model) return;
    float4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < top_k; ++j) {
        const int s = t * top_k + j, e = ids[s];
        if (e >= 0 && e < n_experts && slot_ok[s]) {
            const float4 v = *reinterpret_cast<const float4 *>(ys + (size_t)s * d_model + r);
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
    }
    float *o = out + (size_t)t * d_model + r;   // out is only 4-byte aligned
    o[0] = acc.x;
    o[1] = acc.y;
    o[2] = acc.z;
    o[3] = acc.w;
}

template <int BITS, int KB, int NTT, int MG, int SB>
hipError_t launch_routed_tiled(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(k_route_prep, dim3((unsigned)(a.n_experts + a.T)), dim3(256), 0, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_gate_up_tiled<BITS, KB, NTT, MG, SB>), dim3(pl.gu_blocks),
                       dim3(64 * kTileWaves), pl.gu_lds, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.ks_gu > 1 && !kSplitsInKernel<NTT>) {
        // One block per 16-slot chunk of the slot lists and row block.
        const long chunks = ((long)a.T * a.top_k + 15) / 16 + a.n_experts;
        const long rbs = (a.d_ff + kTileRows - 1) / kTileRows;
        hipLaunchKernelGGL((k_tb_gu_finish<KB, NTT>), dim3((unsigned)(rbs * chunks)), dim3(64 * kTileWaves),
                           (size_t)kTileWaves * 16 * 4, st, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    hipLaunchKernelGGL((k_tb_down_tiled<BITS, KB, NTT, SB>), dim3(pl.dn_blocks), dim3(64 * kTileWaves),
                       pl.dn_lds, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_route_combine, dim3((unsigned)a.T, (unsigned)((a.d_model + 1023) / 1024)), dim3(256), 0, st,
                       a.ids, a.slot_ok, a.ys, a.top_k, a.n_experts, a.d_model, a.out);
    return hipGetLastError();
}

// Routed mode of the streaming kernels (T <= 16, d_ff <= 1536): gate_up
// (which lists each expert's slots itself), down, combine.
template <int BITS, int KB, int SB>
hipError_t launch_routed_stream(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    hipError_t err = launch_tb_stream<BITS, KB, SB>(pl, a, st);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_route_combine, dim3((unsigned)a.T, (unsigned)((a.d_model + 1023) / 1024)), dim3(256), 0, st,
                       a.ids, a.slot_ok, a.ys, a.top_k, a.n_experts, a.d_model, a.out);
    return hipGetLastError();
}

template <int BITS, int KB, int SB>
hipError_t launch_routed_kb(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    if (pl.stream) return launch_routed_stream<BITS, KB, SB>(pl, a, st);
    if (pl.ntt == 1) {
        if (pl.mg == 2) return launch_routed_tiled<BITS, KB, 1, 2, SB>(pl, a, st);
        return launch_routed_tiled<BITS, KB, 1, 1, SB>(pl, a, st);
    }
    if (pl.ntt == 2) return launch_routed_tiled<BITS, KB, 2, 1, SB>(pl, a, st);
    return launch_routed_tiled<BITS, KB, 4, 1, SB>(pl, a, st);
}

template <int SB>
hipError_t launch_routed_fmt(int bits, const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    const int kb = a.group / 32;
    if (bits == 4) {
        if (kb == 1) return launch_routed_kb<4, 1, SB>(pl, a, st);
        if (kb == 2) return launch_routed_kb<4, 2, SB>(pl, a, st);
        return hipErrorInvalidValue;
    }
    if (kb == 2) return launch_routed_kb<2, 2, SB>(pl, a, st);
    return hipErrorInvalidValue;
}

template <int BITS, int KB, int SB>
hipError_t launch_tb_kb(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    if (pl.ntt == 1) {
        if (pl.mg == 2) return launch_tb_tiled<BITS, KB, 1, 2, SB>(pl, a, st);
        return launch_tb_tiled<BITS, KB, 1, 1, SB>(pl, a, st);
    }
    if (pl.ntt == 2) return launch_tb_tiled<BITS, KB, 2, 1, SB>(pl, a, st);
    return launch_tb_tiled<BITS, KB, 4, 1, SB>(pl, a, st);
}

template <int SB>
hipError_t launch_tb_fmt(int bits, const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    if (bits == 4) return a.group == 32 ? launch_tb_kb<4, 1, SB>(pl, a, st) : launch_tb_kb<4, 2, SB>(pl, a, st);
    return launch_tb_kb<2, 2, SB>(pl, a, st);
}

template <int SB>
hipError_t launch_stream_fmt(int bits, const TbArgs &a, const TbPlan &pl, hipStream_t st)
{
    if (bits == 4) return a.group == 32 ? launch_tb_stream<4, 1, SB>(pl, a, st) : launch_tb_stream<4, 2, SB>(pl, a, st);
    return launch_tb_stream<2, 2, SB>(pl, a, st);
}

}  // namespace

// Dynamic LDS per block: the tiled kernels keep within 64 KB (two blocks a
// CU), the streaming kernels take up to the CU's 160 KB (one block a CU).
constexpr size_t kMaxBlockLds = 64 * 1024;
constexpr size_t kMaxStreamLds = 160 * 1024;

// Streaming down grid: row groups of 128 rows x chunks of 1536 columns of
// each expert's d_ff; each block's partial sums take 8 x 256 floats.
long stream_down_blocks(int n_experts, int d_model, int d_ff)
{
    return (long)((d_model + 16 * kDsRows - 1) / (16 * kDsRows)) * n_experts * ((d_ff + kDsCols - 1) / kDsCols);
}

// Tokens per tile: 16, 32 or 64.
int tile_ntt(int T) { return T <= 16 ? 1 : T <= 32 ? 2 : 4; }

// Splits of K over blocks: the smallest power of two (at most 16) that gives
// `tiles` x splits >= `target` blocks of 8 waves.  Every split adds f32
// partial sums written to memory and read back (64 KB per split of a
// 64-token tile), so the smallest count that keeps the CUs busy is taken.
int splits_for(long tiles, long target)
{
    int s = 1;
    while (s < 16 && tiles * s < target) s *= 2;
    return s;
}

// Dense token batch: 192 blocks (three quarters of the CUs) while the tiles
// are few; from 128 tiles on, 512 (two blocks on every CU), which the work of
// a 64-token tile pays for.  Measured at 16 and 64 tokens (96 and 32 tiles),
// 192 beat 256, 384 and 512 blocks; at 256 tokens, 512 blocks (gate_up split
// in 2, down in 4) took 226 us against 240 us for 192 (gate_up not split,
// down in 2), and at 128 tokens 142 us against 146 us.
long batch_block_target(long tiles) { return tiles >= 128 ? 512 : 192; }

BatchSplits batch_splits(int n_experts, int d_model, int d_ff, int T)
{
    BatchSplits b{};
    b.ntt = tile_ntt(T);
    const long ntb = (T + 16 * b.ntt - 1) / (16 * b.ntt);
    b.gu_tiles = (long)n_experts * ((d_ff + kTileRows - 1) / kTileRows) * ntb;
    b.dn_tiles = (long)((d_model + kTileRows - 1) / kTileRows) * ntb;
    b.ks_gu = splits_for(b.gu_tiles, batch_block_target(b.gu_tiles));
    b.ks_dn = splits_for(b.dn_tiles, batch_block_target(b.dn_tiles));
    b.gu_part_floats = b.ks_gu > 1 ? (size_t)b.gu_tiles * b.ks_gu * 2 * b.ntt * 4 * 512 : 0;
    b.dn_part_floats = b.ks_dn > 1 ? (size_t)b.dn_tiles * b.ks_dn * b.ntt * 4 * 512 : 0;
    if (T <= 16)   // the streaming down pass's chunk sums (its counters are the down tiles')
        b.dn_part_floats = std::max(b.dn_part_floats, (size_t)stream_down_blocks(n_experts, d_model, d_ff) *
                                                          kDsRows * 256);
    return b;
}

bool plan_batch(int bits, int group, int d_model, int d_ff, int n_experts, int T, TbPlan *pl)
{
    if (T < 2 || n_experts < 1) return false;
    if (bits == 4 ? (group != 32 && group != 64) : group != 64) return false;
    if (d_model % group || d_ff % group) return false;
    if (T <= 16) {
        // Streaming kernels: gate_up blocks of 3 row tiles over all of K,
        // down blocks of 128 rows x one 1536-column chunk of one expert.
        TbPlan p{};
        p.stream = 1;
        p.ntt = 1;
        p.mg = 1;
        p.gu_blocks = ((long)n_experts * (d_ff / 16) + kGsRows - 1) / kGsRows;
        p.gu_lds = (size_t)2 * 2 * 16 * (kPhaseGroups * group + 8) * 2;   // two tiles of hi/lo halves
        p.dn_blocks = stream_down_blocks(n_experts, d_model, d_ff);
        p.dn_lds = (size_t)2 * 16 * (kDsCols + 8) * 2 + (size_t)(kDsCols / group) * 16 * 4;
        if (p.gu_lds > kMaxStreamLds || p.dn_lds > kMaxStreamLds) return false;
        *pl = p;
        return true;
    }
    // 16 * ntt tokens x 128 rows per 8-wave block, K split over blocks as the
    // workspace allows (at most one split per 4-group iteration).
    const BatchSplits bs = batch_splits(n_experts, d_model, d_ff, T);
    TbPlan p{};
    p.ntt = bs.ntt;
    // gate_up steps of mg groups: 2 for 16-token tiles, else 1 (1 if 2 does
    // not divide the groups of d_model).
    const int G = d_model / group;
    p.mg = p.ntt == 1 ? 2 : 1;
    while (G % p.mg) p.mg /= 2;
    p.ks_gu = std::min(bs.ks_gu, (G + 3) / 4);   // splits of whole 4-group iterations
    p.ks_dn = std::min(bs.ks_dn, n_experts * ((d_ff / group + 3) / 4));
    p.gu_blocks = bs.gu_tiles * p.ks_gu;
    p.dn_blocks = bs.dn_tiles * p.ks_dn;
    const int tt = 16 * p.ntt;
    const size_t gtile = (size_t)2 * tt * (p.mg * group + 8) * 2;
    p.gu_lds = 2 * gtile + (size_t)kTileWaves * p.ntt * 16 * 4;
    p.dn_lds = 2 * ((size_t)2 * tt * (group + 8) * 2) + 2 * tt * 4;
    if (p.gu_lds > kMaxBlockLds || p.dn_lds > kMaxBlockLds) return false;
    *pl = p;
    return true;
}

// Routed mode: tiles sized for the average slots per expert (T * top_k /
// n_experts), grids for the largest possible count (T per expert; tiles past
// an expert's count exit at once), K split chosen from the expected active
// tiles.
BatchSplits routed_splits(int n_experts, int d_model, int d_ff, int T, int top_k)
{
    BatchSplits b{};
    const long avg = ((long)T * top_k + n_experts - 1) / n_experts;
    // Lists are ragged (their lengths spread around the average), and a list's
    // last tile costs a full tile: 32-token tiles waste less of it than 64 and
    // measured faster up to an average of 96 (256 tokens x top-2 of 8: 194 ->
    // 136 us of gate_up + down, and with the grids over the actual tiles 128
    // against 112 us for the call; top-4, an average of 128: 198 against 177
    // us); at an average of 256 (top-8) 64-token tiles do better (256 against
    // 294 us), and the switch is put half way.  At an average of 32 (256
    // tokens x top-1 of 8) 32-token tiles took 94 us against 111 for 16-token
    // ones, which are kept for averages up to 16.
    b.ntt = std::min(tile_ntt(T), avg > 192 ? 4 : avg > 16 ? 2 : 1);
    const int tt = 16 * b.ntt;
    const long ntb = (T + tt - 1) / tt, ntb_avg = (std::min<long>(avg, T) + tt - 1) / tt;
    const long rbg = (d_ff + kTileRows - 1) / kTileRows;
    b.gu_tiles = (long)n_experts * rbg * ntb;
    b.dn_tiles = (long)n_experts * ((d_model + kTileRows - 1) / kTileRows) * ntb;
    // K splits for gate_up from the expected active tiles: 192 blocks, or 384
    // with 32- or 64-token tiles, whose work pays for the finishing pass (256
    // tokens x top-4 of 8: 225 -> 207 us, top-2: 150 -> 146 us; at top-1,
    // where the splits are added in the kernel, more of them were slower).
    b.ks_gu = splits_for((long)n_experts * rbg * ntb_avg, b.ntt >= 2 ? 384 : 192);
    b.ks_dn = 1;
    b.gu_part_floats = b.ks_gu > 1 ? (size_t)b.gu_tiles * b.ks_gu * 2 * b.ntt * 4 * 512 : 0;
    b.dn_part_floats = 0;
    return b;
}

bool plan_routed(int bits, int group, int d_model, int d_ff, int n_experts, int T, int top_k, TbPlan *pl)
{
    if (T < 1 || n_experts < 1 || top_k < 1) return false;
    if (!(group == 32 && bits == 4) && group != 64) return false;
    if (d_model % group || d_ff % group) return false;
    if (T <= 16 && d_ff <= kDsCols) {
        // Streaming kernels: an expert's slots are one token tile; gate_up
        // blocks of 3 row tiles of one expert, down blocks of 128 rows x one
        // expert.
        TbPlan p{};
        p.stream = 1;
        p.ntt = 1;
        p.mg = 1;
        p.gu_blocks = (long)n_experts * ((d_ff / 16 + kGsRows - 1) / kGsRows);
        p.gu_lds = (size_t)2 * 2 * 16 * (kPhaseGroups * group + 8) * 2;
        p.dn_blocks = stream_down_blocks(n_experts, d_model, d_ff);
        p.dn_lds = (size_t)2 * 16 * (kDsCols + 8) * 2 + (size_t)(kDsCols / group) * 16 * 4;
        if (p.gu_lds > kMaxStreamLds || p.dn_lds > kMaxStreamLds) return false;
        *pl = p;
        return true;
    }
    const BatchSplits bs = routed_splits(n_experts, d_model, d_ff, T, top_k);
    TbPlan p{};
    p.ntt = bs.ntt;
    const int G = d_model / group;
    p.mg = p.ntt == 1 ? 2 : 1;
    while (G % p.mg) p.mg /= 2;
    p.ks_gu = std::min(bs.ks_gu, (G + 3) / 4);   // splits of whole 4-group iterations
    p.ks_dn = 1;
    const int tt = 16 * p.ntt;
    // Grids of chunk x row block (x split): an expert's list of c slots takes
    // ceil(c / tt) token tiles, at most T top_k / tt + n_experts over all of
    // them (not n_experts x ceil(T / tt), most of which would be empty).
    const long chunks = ((long)T * top_k + tt - 1) / tt + n_experts;
    p.gu_blocks = (long)((d_ff + kTileRows - 1) / kTileRows) * p.ks_gu * chunks;
    p.dn_blocks = (long)((d_model + kTileRows - 1) / kTileRows) * chunks;
    p.gu_lds = 2 * ((size_t)2 * tt * (p.mg * group + 8) * 2) + (size_t)kTileWaves * p.ntt * 16 * 4;
    p.dn_lds = 2 * ((size_t)2 * tt * (group + 8) * 2) + 2 * tt * 4;
    if (p.gu_lds > kMaxBlockLds || p.dn_lds > kMaxBlockLds) return false;
    *pl = p;
    return true;
}

hipError_t launch_routed(int bits, const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    return a.scale_bytes == 2 ? launch_routed_fmt<2>(bits, pl, a, st) : launch_routed_fmt<4>(bits, pl, a, st);
}

hipError_t launch_batch(int bits, const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    if (pl.stream) return a.scale_bytes == 2 ? launch_stream_fmt<2>(bits, a, pl, st) : launch_stream_fmt<4>(bits, a, pl, st);
    return a.scale_bytes == 2 ? launch_tb_fmt<2>(bits, pl, a, st) : launch_tb_fmt<4>(bits, pl, a, st);
}

}  // namespace smoe
