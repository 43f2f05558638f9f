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
//  * an activation row is cut into quantisation groups; each group is scaled by
//    a power of two 2^-e chosen so every scaled value is below 1 in magnitude,
//    then written as hi + lo with hi = f16(v), lo = f16(v - hi): 22 significant
//    bits, no overflow, and the scaling is undone exactly by ldexp;
//  * v_mfma_f32_16x16x32_f16 multiplies exactly and accumulates in f32; hi and
//    lo go through two MFMAs into one accumulator per group, and the group's
//    f32 result is multiplied by ldexp(s/Z, e) into the running output.
//
// Launch sequence (one stream): k_tb_prep (X -> hi/lo + exponents),
// k_tb_gate_up (both projections, SiLU, H -> hi/lo + exponents per group of
// d_ff columns), k_tb_down (all experts summed with the router weights in a
// fixed order, so the result is deterministic; no atomics).
//
// Fragment layout of v_mfma_f32_16x16x32_f16 (lane l, q = l / 16, n = l % 16):
//   A (16 x 32):  row n, k = 8q + i for element i = 0..7      <- weight codes
//   B (32 x 16):  column n, k = 8q + i                          <- activations
//   D (16 x 16):  rows 4q + i (i = 0..3), column n              -> outputs
// Within one quantisation group of 32*KB columns, lane group q owns the 8*KB
// columns [q*8KB, (q+1)*8KB), so its codes are one contiguous load; K-block j
// uses columns q*8KB + 8j + sigma(i), sigma = (0,4,1,5,2,6,3,7).  sigma is the
// order in which the nibble unpacking below yields codes; activations are
// stored in the same order (element 8b + i holds column 8b + sigma(i)).
#include "common.h"
#include "launch.h"

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

// f16 pair (1024 + a, 1024 + b) from bytes a, b (< 16) of src picked by sel,
// shifted to (a - Z, b - Z).  Both subtractions are exact in f16.
template <int BITS>
__device__ __forceinline__ half2v code_pair(uint32_t src, uint32_t sel)
{
    const uint32_t bits = __builtin_amdgcn_perm(0x64646464u, src, sel);
    half2v h = __builtin_bit_cast(half2v, bits);
    h = h - (half2v){(_Float16)1024.0f, (_Float16)1024.0f};
    constexpr float z = QFormat<BITS>::kZ;
    return h - (half2v){(_Float16)z, (_Float16)z};
}

// Codes per lane per quantisation group: KB K-blocks of 8 codes.
template <int BITS, int KB>
struct CodeWords {
    static constexpr int kDwords = (KB * BITS + 3) / 4;  // Q4: KB dwords, Q2: KB/2 dwords
    uint32_t w[kDwords];
};

template <int BITS, int KB>
__device__ __forceinline__ void load_codes(const uint8_t *p, CodeWords<BITS, KB> &c)
{
    constexpr int n = CodeWords<BITS, KB>::kDwords;
    if constexpr (n == 1) {
        c.w[0] = *reinterpret_cast<const uint32_t *>(p);
    } else if constexpr (n == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(p);
        c.w[0] = v.x;
        c.w[1] = v.y;
    } else if constexpr (n == 4) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        c.w[0] = v.x;
        c.w[1] = v.y;
        c.w[2] = v.z;
        c.w[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < n; ++i) c.w[i] = reinterpret_cast<const uint32_t *>(p)[i];
    }
}

// A fragment of K-block j: the lane's 8 codes in sigma order as f16 (c - Z).
template <int BITS, int KB>
__device__ __forceinline__ half8 code_frag(const CodeWords<BITS, KB> &c, int j)
{
    Half8Parts f;
    if constexpr (BITS == 4) {
        // Nibbles n0..n7 of one dword: lo holds bytes (n0,n2,n4,n6), hi (n1,n3,n5,n7).
        const uint32_t d = c.w[j];
        const uint32_t lo = d & 0x0F0F0F0Fu, hi = (d >> 4) & 0x0F0F0F0Fu;
        f.v[0] = code_pair<4>(lo, 0x04020400u);  // n0, n4
        f.v[1] = code_pair<4>(hi, 0x04020400u);  // n1, n5
        f.v[2] = code_pair<4>(lo, 0x04030401u);  // n2, n6
        f.v[3] = code_pair<4>(hi, 0x04030401u);  // n3, n7
    } else {
        // 16 two-bit codes c0..c15 per dword; a_k holds bytes (c_k, c_4+k, c_8+k, c_12+k).
        const uint32_t d = c.w[j >> 1];
        const uint32_t sel = (j & 1) ? 0x04030402u : 0x04010400u;
#pragma unroll
        for (int k = 0; k < 4; ++k) f.v[k] = code_pair<2>((d >> (2 * k)) & 0x03030303u, sel);
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

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) v = fmaxf(v, __shfl_xor(v, s));
    return v;
}

// Exponent e with |m| = f * 2^e, f in [0.5, 1) (0 for m == 0): v * 2^-e < 1.
__device__ __forceinline__ int norm_exponent(float m)
{
    int e = 0;
    (void)frexpf(m, &e);
    return e;
}

// -------------------------------------------------------------------------
// X -> hi/lo halves in sigma order + one exponent per (token, group).
// One wave per (token, group).
__global__ __launch_bounds__(256) void k_tb_prep(const float *__restrict__ x, int rows, int cols,
                                                 int group, _Float16 *__restrict__ xh,
                                                 _Float16 *__restrict__ xl, int *__restrict__ xe)
{
    const int lane = threadIdx.x & 63;
    const int G = cols / group;
    const long pair = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (pair >= (long)rows * G) return;
    const long t = pair / G;
    const int g = (int)(pair % G);
    const size_t base = (size_t)t * cols + (size_t)g * group;
    float m = 0.0f;
    for (int c = lane; c < group; c += 64) m = fmaxf(m, fabsf(x[base + c]));
    const int e = norm_exponent(wave_max(m));
    for (int c = lane; c < group; c += 64) {
        const float v = ldexpf(x[base + c], -e);
        const _Float16 h = (_Float16)v;
        const size_t pos = base + (c & ~7) + sigma_pos(c & 7);
        xh[pos] = h;
        xl[pos] = (_Float16)(v - (float)h);
    }
    if (lane == 0) xe[pair] = e;
}

// -------------------------------------------------------------------------
// Gate and up for one expert, one quantisation group of d_ff rows (the block's
// H group) and 16*NTT tokens.  Wave (rw, ks): rows rw*16*RT .. +16*RT of the
// H group in both matrices, quantisation groups [ks*G/KS, (ks+1)*G/KS) of
// d_model.  Partial sums over ks are added in LDS in a fixed order.
template <int BITS, int KB, int NTT, int RT>
__global__ __launch_bounds__(512) void k_tb_gate_up(TbArgs a)
{
    extern __shared__ float lds[];
    constexpr int NM = 2;  // gate, up
    constexpr int kTiles = NM * RT * NTT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = a.ks_gu, RW = a.rw_gu;
    const int ks = wave % KS, rw = wave / KS;
    const int q = lane >> 4, n = lane & 15;
    const int group = a.group, d_model = a.d_model, d_ff = a.d_ff, T = a.T;
    const int G = d_model / group, HG = d_ff / group;
    const int NTB = (T + 16 * NTT - 1) / (16 * NTT);
    int b = blockIdx.x;
    const int tb = b % NTB;
    b /= NTB;
    const int hg = b % HG;
    const int e = b / HG;
    const int row0 = hg * group + rw * 16 * RT;
    const int t0 = tb * 16 * NTT;
    const size_t rs = (size_t)d_model * BITS / 8;
    const QPtr mats[NM] = {a.gate[e], a.up[e]};

    int tok[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) tok[tt] = min(t0 + tt * 16 + n, T - 1);

    f32x4 tot[NM][RT][NTT];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) tot[m][rt][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int gbeg = ks * G / KS, gend = (ks + 1) * G / KS;
    for (int g = gbeg; g < gend; ++g) {
        CodeWords<BITS, KB> cw[NM][RT];
        float sc[NM][RT][4];
        const size_t cofs = (size_t)(g * group + q * 8 * KB) * BITS / 8;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                load_codes(mats[m].codes + (size_t)(row0 + rt * 16 + n) * rs + cofs, cw[m][rt]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sc[m][rt][i] = mats[m].scales[(size_t)(row0 + rt * 16 + 4 * q + i) * G + g] *
                                   QFormat<BITS>::kInvZ;
            }
        half8 bh[NTT][KB], bl[NTT][KB];
        int ex[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const size_t xo = (size_t)tok[tt] * d_model + g * group + q * 8 * KB;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                bh[tt][j] = load_half8(a.xh + xo + 8 * j);
                bl[tt][j] = load_half8(a.xl + xo + 8 * j);
            }
            ex[tt] = a.xe[(size_t)tok[tt] * G + g];
        }
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                half8 af[KB];
#pragma unroll
                for (int j = 0; j < KB; ++j) af[j] = code_frag<BITS, KB>(cw[m][rt], j);
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < KB; ++j) {
                        acc = mfma(af[j], bh[tt][j], acc);
                        acc = mfma(af[j], bl[tt][j], acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        tot[m][rt][tt][i] = fmaf(ldexpf(sc[m][rt][i], ex[tt]), acc[i], tot[m][rt][tt][i]);
                }
            }
    }

    // Sum the KS partials: tot(0) + (tot(1) + (... + tot(KS-1))).
    float *buf = lds + (size_t)rw * kTiles * 4 * 64;
    if (KS > 1) {
        for (int s = KS - 1; s >= 1; --s) {
            if (ks == s) {
                int r = 0;
#pragma unroll
                for (int m = 0; m < NM; ++m)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                            for (int i = 0; i < 4; ++i, ++r) {
                                float v = tot[m][rt][tt][i];
                                if (s != KS - 1) v += buf[r * 64 + lane];
                                buf[r * 64 + lane] = v;
                            }
            }
            __syncthreads();
        }
    }

    // hidden = SiLU(gate) * up, and its per-token maximum over this wave's rows.
    float *mx = lds + (KS > 1 ? (size_t)RW * kTiles * 4 * 64 : 0);  // [RW][NTT][16]
    float h[RT][NTT][4];
    if (ks == 0) {
        int r = 0;
#pragma unroll
        for (int m = 0; m < NM; ++m)
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                    for (int i = 0; i < 4; ++i, ++r)
                        if (KS > 1) tot[m][rt][tt][i] += buf[r * 64 + lane];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            float m = 0.0f;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    h[rt][tt][i] = silu(tot[0][rt][tt][i]) * tot[1][rt][tt][i];
                    m = fmaxf(m, fabsf(h[rt][tt][i]));
                }
            m = fmaxf(m, __shfl_xor(m, 16));
            m = fmaxf(m, __shfl_xor(m, 32));
            if (q == 0) mx[(rw * NTT + tt) * 16 + n] = m;
        }
    }
    __syncthreads();
    if (ks != 0) return;

    // Normalise per (token, H group), split into hi/lo halves, store in sigma
    // order.  Lanes q and q^1 hold columns 0..3 and 4..7 of one 8-column block:
    // the even lane assembles and stores the hi block, the odd lane the lo block.
    const bool even = (q & 1) == 0;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        float m = 0.0f;
        for (int w = 0; w < RW; ++w) m = fmaxf(m, mx[(w * NTT + tt) * 16 + n]);
        const int ee = norm_exponent(m);
        const int t = t0 + tt * 16 + n;
        const bool valid = t < T;
        const size_t hrow = ((size_t)e * T + (valid ? t : 0)) * d_ff;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            uint32_t hi2[2], lo2[2];
            _Float16 hv[4], lv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float v = ldexpf(h[rt][tt][i], -ee);
                hv[i] = (_Float16)v;
                lv[i] = (_Float16)(v - (float)hv[i]);
            }
            hi2[0] = __builtin_bit_cast(uint32_t, (half2v){hv[0], hv[1]});
            hi2[1] = __builtin_bit_cast(uint32_t, (half2v){hv[2], hv[3]});
            lo2[0] = __builtin_bit_cast(uint32_t, (half2v){lv[0], lv[1]});
            lo2[1] = __builtin_bit_cast(uint32_t, (half2v){lv[2], lv[3]});
            // Send what the partner assembles: the even lane sends lo, the odd lane hi.
            const uint32_t s0 = even ? lo2[0] : hi2[0], s1 = even ? lo2[1] : hi2[1];
            const uint32_t r0 = __shfl_xor((int)s0, 16), r1 = __shfl_xor((int)s1, 16);
            const half2v m0 = __builtin_bit_cast(half2v, even ? hi2[0] : lo2[0]);
            const half2v m1 = __builtin_bit_cast(half2v, even ? hi2[1] : lo2[1]);
            const half2v p0 = __builtin_bit_cast(half2v, r0), p1 = __builtin_bit_cast(half2v, r1);
            // Block columns (0..3 from the even lane, 4..7 from the odd lane) in
            // sigma order: pairs (c0,c4), (c1,c5), (c2,c6), (c3,c7).
            const half2v c03[4] = {even ? (half2v){m0[0], p0[0]} : (half2v){p0[0], m0[0]},
                                   even ? (half2v){m0[1], p0[1]} : (half2v){p0[1], m0[1]},
                                   even ? (half2v){m1[0], p1[0]} : (half2v){p1[0], m1[0]},
                                   even ? (half2v){m1[1], p1[1]} : (half2v){p1[1], m1[1]}};
            if (valid) {
                const size_t col = (size_t)row0 + rt * 16 + 8 * (q >> 1);
                _Float16 *dst = (even ? a.hh : a.hl) + hrow + col;
                uint4 v;
                v.x = __builtin_bit_cast(uint32_t, c03[0]);
                v.y = __builtin_bit_cast(uint32_t, c03[1]);
                v.z = __builtin_bit_cast(uint32_t, c03[2]);
                v.w = __builtin_bit_cast(uint32_t, c03[3]);
                *reinterpret_cast<uint4 *>(dst) = v;
            }
        }
        if (valid && rw == 0 && q == 0) a.he[((size_t)e * T + t) * HG + hg] = ee;
    }
}

// -------------------------------------------------------------------------
// Down for 16*RT*RW rows of d_model and 16*NTT tokens, summed over all
// experts with the router weights.  Wave (rw, ks): rows rw*16*RT .. +16*RT of
// the block, (expert, group) pairs [ks*P/KS, (ks+1)*P/KS) of P = E * d_ff/group,
// taken in ascending order; partials over ks are added in LDS in a fixed order.
template <int BITS, int KB, int NTT, int RT>
__global__ __launch_bounds__(512) void k_tb_down(TbArgs a)
{
    extern __shared__ float lds[];
    constexpr int kTiles = RT * NTT;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = a.ks_dn, RW = a.rw_dn;
    const int ks = wave % KS, rw = wave / KS;
    const int q = lane >> 4, n = lane & 15;
    const int group = a.group, d_model = a.d_model, d_ff = a.d_ff, T = a.T, E = a.n_experts;
    const int Gd = d_ff / group;
    const int NTB = (T + 16 * NTT - 1) / (16 * NTT);
    const int tb = blockIdx.x % NTB, rb = blockIdx.x / NTB;
    const int row0 = (rb * RW + rw) * 16 * RT;
    const int t0 = tb * 16 * NTT;
    const size_t rs = (size_t)d_ff * BITS / 8;

    int tok[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) tok[tt] = min(t0 + tt * 16 + n, T - 1);
    int arow[RT];  // A-fragment row of each row tile (clamped), and output rows
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) arow[rt] = min(row0 + rt * 16 + n, d_model - 1);

    f32x4 tot[RT][NTT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) tot[rt][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    const int P = E * Gd;
    const int pbeg = ks * P / KS, pend = (ks + 1) * P / KS;
    for (int p = pbeg; p < pend; ++p) {
        const int e = p / Gd, g = p - e * Gd;
        const QPtr dm = a.down[e];
        CodeWords<BITS, KB> cw[RT];
        float sc[RT][4];
        const size_t cofs = (size_t)(g * group + q * 8 * KB) * BITS / 8;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            load_codes(dm.codes + (size_t)arow[rt] * rs + cofs, cw[rt]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = min(row0 + rt * 16 + 4 * q + i, d_model - 1);
                sc[rt][i] = dm.scales[(size_t)r * Gd + g] * QFormat<BITS>::kInvZ;
            }
        }
        half8 bh[NTT][KB], bl[NTT][KB];
        float fac[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const size_t hrow = ((size_t)e * T + tok[tt]) * d_ff + g * group + q * 8 * KB;
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                bh[tt][j] = load_half8(a.hh + hrow + 8 * j);
                bl[tt][j] = load_half8(a.hl + hrow + 8 * j);
            }
            const float rwt = a.route_w ? a.route_w[(size_t)tok[tt] * E + e] : 1.0f;
            fac[tt] = ldexpf(rwt, a.he[((size_t)e * T + tok[tt]) * Gd + g]);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            half8 af[KB];
#pragma unroll
            for (int j = 0; j < KB; ++j) af[j] = code_frag<BITS, KB>(cw[rt], j);
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int j = 0; j < KB; ++j) {
                    acc = mfma(af[j], bh[tt][j], acc);
                    acc = mfma(af[j], bl[tt][j], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    tot[rt][tt][i] = fmaf(sc[rt][i] * fac[tt], acc[i], tot[rt][tt][i]);
            }
        }
    }

    float *buf = lds + (size_t)rw * kTiles * 4 * 64;
    if (KS > 1) {
        for (int s = KS - 1; s >= 1; --s) {
            if (ks == s) {
                int r = 0;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i, ++r) {
                            float v = tot[rt][tt][i];
                            if (s != KS - 1) v += buf[r * 64 + lane];
                            buf[r * 64 + lane] = v;
                        }
            }
            __syncthreads();
        }
    }
    if (ks != 0) return;
    int r = 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
            const int t = t0 + tt * 16 + n;
#pragma unroll
            for (int i = 0; i < 4; ++i, ++r) {
                float v = tot[rt][tt][i];
                if (KS > 1) v += buf[r * 64 + lane];
                const int row = row0 + rt * 16 + 4 * q + i;
                if (t < T && row < d_model) a.out[(size_t)t * d_model + row] = v;
            }
        }
}

template <int BITS, int KB, int NTT, int RT>
hipError_t launch_tb_kernels(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    const int G = a.d_model / a.group;
    const long pairs = (long)a.T * G;
    hipLaunchKernelGGL(k_tb_prep, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, st, a.x, a.T, a.d_model,
                       a.group, a.xh, a.xl, a.xe);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_gate_up<BITS, KB, NTT, RT>), dim3(pl.gu_blocks), dim3(64 * pl.gu_waves),
                       pl.gu_lds, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_down<BITS, KB, NTT, RT>), dim3(pl.dn_blocks), dim3(64 * pl.dn_waves),
                       pl.dn_lds, st, a);
    return hipGetLastError();
}

template <int BITS, int KB>
hipError_t launch_tb_kb(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    if (pl.ntt == 1) return launch_tb_kernels<BITS, KB, 1, 1>(pl, a, st);
    return launch_tb_kernels<BITS, KB, 4, 2>(pl, a, st);
}

}  // namespace

// Dynamic LDS per block is kept within 64 KB.
constexpr size_t kMaxBlockLds = 64 * 1024;

bool plan_batch(int bits, int group, int d_model, int d_ff, int n_experts, int T, TbPlan *pl)
{
    if (T < 2 || n_experts < 1) return false;
    const int kb = group / 32;
    if (bits == 4 ? (kb < 1 || kb > 4) : (kb != 2 && kb != 4)) return false;
    if (d_model % group || d_ff % group) return false;
    TbPlan p{};
    p.ntt = T <= 16 ? 1 : 4;
    const int rt = p.ntt == 1 ? 1 : 2;
    const int ntb = (T + 16 * p.ntt - 1) / (16 * p.ntt);
    const int G = d_model / group;
    // gate_up: the block covers one quantisation group of d_ff rows.
    p.rw_gu = group / (16 * rt);
    if (p.rw_gu < 1 || p.rw_gu > 8 || p.rw_gu * 16 * rt != group) return false;
    const long gu_blocks = (long)n_experts * (d_ff / group) * ntb;
    // LDS: the K-split partial sums (only when K is split) and the per-token maxima.
    const size_t gu_buf = (size_t)p.rw_gu * (2 * rt * p.ntt) * 4 * 64 * 4;
    const size_t gu_max = (size_t)p.rw_gu * p.ntt * 16 * 4;
    p.ks_gu = 1;
    while (p.ks_gu < 4 && p.rw_gu * p.ks_gu * 2 <= 8 && p.ks_gu * 2 <= G &&
           gu_buf + gu_max <= kMaxBlockLds && gu_blocks * p.rw_gu * p.ks_gu < 2048)
        p.ks_gu *= 2;
    p.gu_waves = p.rw_gu * p.ks_gu;
    p.gu_blocks = gu_blocks;
    p.gu_lds = (p.ks_gu > 1 ? gu_buf : 0) + gu_max;
    // down: the block covers 16*rt*rw_dn rows of d_model; waves split the
    // (expert, group) pairs.
    p.rw_dn = p.ntt == 1 ? 1 : 2;
    const int P = n_experts * (d_ff / group);
    p.ks_dn = 8 / p.rw_dn;
    while (p.ks_dn > 1 && p.ks_dn > P) p.ks_dn /= 2;
    p.dn_waves = p.rw_dn * p.ks_dn;
    const int rows_per_block = 16 * rt * p.rw_dn;
    p.dn_blocks = (long)((d_model + rows_per_block - 1) / rows_per_block) * ntb;
    p.dn_lds = p.ks_dn > 1 ? (size_t)p.rw_dn * rt * p.ntt * 4 * 64 * 4 : 0;
    if (p.gu_lds > kMaxBlockLds || p.dn_lds > kMaxBlockLds) return false;
    *pl = p;
    return true;
}

hipError_t launch_batch(int bits, const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    const int kb = a.group / 32;
    if (bits == 4) {
        switch (kb) {
        case 1: return launch_tb_kb<4, 1>(pl, a, st);
        case 2: return launch_tb_kb<4, 2>(pl, a, st);
        case 3: return launch_tb_kb<4, 3>(pl, a, st);
        case 4: return launch_tb_kb<4, 4>(pl, a, st);
        default: return hipErrorInvalidValue;
        }
    }
    switch (kb) {
    case 2: return launch_tb_kb<2, 2>(pl, a, st);
    case 4: return launch_tb_kb<2, 4>(pl, a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace smoe
