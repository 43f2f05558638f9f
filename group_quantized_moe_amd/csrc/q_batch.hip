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
// Launch sequence (one stream): k_tb_prep (X -> hi/lo halves + per-token
// exponent), k_tb_gate_up (both projections, SiLU, hidden rows -> hi/lo halves
// + one factor per (expert, group, token) that folds the group's power of two
// and the router weight), k_tb_down (all experts summed in a fixed order, so
// the result is deterministic; no atomics).
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

// B fragment of K-block j: the lane's 8 codes in sigma order as f16 (c - Z).
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

// -------------------------------------------------------------------------
// X -> hi/lo halves in sigma order + one exponent per token.  One block per
// token.
__global__ __launch_bounds__(256) void k_tb_prep(const float *__restrict__ x, int cols, _Float16 *__restrict__ xh,
                                                 _Float16 *__restrict__ xl, int *__restrict__ xe)
{
    __shared__ float s_max[4];
    const size_t base = (size_t)blockIdx.x * cols;
    float m = 0.0f;
    for (int c = threadIdx.x; c < cols; c += blockDim.x) m = fmaxf(m, fabsf(x[base + c]));
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) m = fmaxf(m, __shfl_xor(m, s));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    m = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const int e = norm_exponent(m);
    for (int c = threadIdx.x; c < cols; c += blockDim.x) {
        const float v = ldexpf(x[base + c], -e);
        const _Float16 h = (_Float16)v;
        const size_t pos = base + (c & ~7) + sigma_pos(c & 7);
        xh[pos] = h;
        xl[pos] = (_Float16)(v - (float)h);
    }
    if (threadIdx.x == 0) xe[blockIdx.x] = e;
}

// One step of the K loop: the activation fragments of NTT token tiles and
// the codes and scales of NB row tiles, for one quantisation group.
template <int BITS, int KB, int NTT, int NB>
struct TbStage {
    half8 ah[NTT][KB], al[NTT][KB];
    CodeWords<BITS, KB> cw[NB];
    float s[NB];
};

// sum over the step's K-blocks of (hi + lo) x codes, for token tile tt and
// row tile b: one f32 accumulator per quantisation group.
template <int BITS, int KB, int NTT, int NB>
__device__ __forceinline__ f32x4 group_mfma(const TbStage<BITS, KB, NTT, NB> &st, const half8 *bf, int tt)
{
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KB; ++j) {
        acc = mfma(st.ah[tt][j], bf[j], acc);
        acc = mfma(st.al[tt][j], bf[j], acc);
    }
    return acc;
}

// -------------------------------------------------------------------------
// Gate and up for one expert, one quantisation group of d_ff rows (the
// block's "H group") and 16*NTT tokens.  Wave (rw, ks) covers rows
// rw*16*RT .. +16*RT of the H group in both matrices and quantisation groups
// [ks*G/KS, (ks+1)*G/KS) of d_model; partial sums over ks are added in LDS in
// a fixed order.  The hidden rows are normalised per (token, H group), split
// into hi/lo halves and stored with the factor r[t][e] * 2^e for down.
template <int BITS, int KB, int NTT, int RT>
__global__ __launch_bounds__(512) void k_tb_gate_up(TbArgs a)
{
    extern __shared__ float lds[];
    constexpr int NB = 2 * RT;            // gate row tiles, then up row tiles
    constexpr int kTot = NB * NTT * 4;    // accumulator floats per lane
    constexpr int DEPTH = 2;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int KS = a.ks_gu, RW = a.rw_gu;
    const int ks = wave % KS, rw = wave / KS;
    const int q = lane >> 4, n = lane & 15;
    const int group = a.group, d_model = a.d_model, d_ff = a.d_ff, T = a.T, E = a.n_experts;
    const int G = d_model / group, HG = d_ff / group;
    const int NTB = (T + 16 * NTT - 1) / (16 * NTT);
    int b = blockIdx.x;
    const int tb = b % NTB;
    b /= NTB;
    const int hg = b % HG;
    const int e = b / HG;
    const int row0 = hg * group + rw * 16 * RT;   // first d_ff row of this wave
    const int t0 = tb * 16 * NTT;
    const size_t rs = (size_t)d_model * BITS / 8;
    const uint8_t *code_base[NB];
    const float *scale_base[NB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const QPtr M = m == 0 ? a.gate[e] : a.up[e];
            const int row = row0 + rt * 16 + n;
            code_base[m * RT + rt] = M.codes + (size_t)row * rs + (size_t)(q * 8 * KB) * BITS / 8;
            scale_base[m * RT + rt] = M.scales + (size_t)row * G;
        }
    const _Float16 *xh_base[NTT], *xl_base[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
        const size_t off = (size_t)min(t0 + tt * 16 + n, T - 1) * d_model + q * 8 * KB;
        xh_base[tt] = a.xh + off;
        xl_base[tt] = a.xl + off;
    }
    using Stage = TbStage<BITS, KB, NTT, NB>;
    auto load = [&](Stage &st, int g) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                st.ah[tt][j] = load_half8(xh_base[tt] + (size_t)g * group + 8 * j);
                st.al[tt][j] = load_half8(xl_base[tt] + (size_t)g * group + 8 * j);
            }
#pragma unroll
        for (int bt = 0; bt < NB; ++bt) {
            load_codes<BITS, KB>(code_base[bt] + (size_t)g * group * BITS / 8, st.cw[bt]);
            st.s[bt] = scale_base[bt][g];
        }
    };

    f32x4 tot[NB][NTT];
#pragma unroll
    for (int bt = 0; bt < NB; ++bt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) tot[bt][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Every wave has at least one group (KS <= G).  Ring loads are
    // unconditional (past the last group they re-read it) so that waiting for
    // one stage leaves the other in flight.
    const int gbeg = ks * G / KS, gend = (ks + 1) * G / KS;
    Stage S[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) load(S[i], min(gbeg + i, gend - 1));
    for (int base = gbeg; base < gend; base += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            const int g = base + i;
            if (g < gend) {
#pragma unroll
                for (int bt = 0; bt < NB; ++bt) {
                    half8 bf[KB];
#pragma unroll
                    for (int j = 0; j < KB; ++j) bf[j] = code_frag<BITS, KB>(S[i].cw[bt], j);
                    const float s = S[i].s[bt] * QFormat<BITS>::kInvZ;
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt) {
                        const f32x4 acc = group_mfma<BITS, KB, NTT, NB>(S[i], bf, tt);
#pragma unroll
                        for (int r = 0; r < 4; ++r) tot[bt][tt][r] = fmaf(s, acc[r], tot[bt][tt][r]);
                    }
                }
            }
            load(S[i], min(g + DEPTH, gend - 1));
        }
    }

    // Sum the KS partials: tot(0) + (tot(1) + (... + tot(KS-1))).
    float *buf = lds + (size_t)rw * kTot * 64;
    if (KS > 1) {
        for (int s = KS - 1; s >= 1; --s) {
            if (ks == s) {
                int r = 0;
#pragma unroll
                for (int bt = 0; bt < NB; ++bt)
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                        for (int i = 0; i < 4; ++i, ++r) {
                            float v = tot[bt][tt][i];
                            if (s != KS - 1) v += buf[r * 64 + lane];
                            buf[r * 64 + lane] = v;
                        }
            }
            __syncthreads();
        }
    }

    // hidden = SiLU(gate) * up for tokens 4q + i of each token tile, rows n
    // of each row tile; then each token's largest |hidden| over this wave's
    // rows (a DPP row holds the 16 rows of a tile for the same 4 tokens).
    float *mx = lds + (KS > 1 ? (size_t)RW * kTot * 64 : 0);  // [RW][NTT][16]
    float h[RT][NTT][4];
    if (ks == 0) {
        int r = 0;
#pragma unroll
        for (int bt = 0; bt < NB; ++bt)
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i, ++r)
                    if (KS > 1) tot[bt][tt][i] += buf[r * 64 + lane];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = min(t0 + tt * 16 + 4 * q + i, T - 1);
                const int xe = a.xe[t];
                float m = 0.0f;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const float gv = ldexpf(tot[rt][tt][i], xe), uv = ldexpf(tot[RT + rt][tt][i], xe);
                    h[rt][tt][i] = silu(gv) * uv;
                    m = fmaxf(m, fabsf(h[rt][tt][i]));
                }
                m = row16_max(m);
                if (n == 0) mx[(rw * NTT + tt) * 16 + 4 * q + i] = m;
            }
        }
    }
    __syncthreads();
    if (ks != 0) return;

    // Normalise per (token, H group), split into hi/lo halves, store in sigma
    // order, and store each token's factor for down.
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tl = 4 * q + i;
            float m = 0.0f;
            for (int w = 0; w < RW; ++w) m = fmaxf(m, mx[(w * NTT + tt) * 16 + tl]);
            const int ee = norm_exponent(m);
            const int t = t0 + tt * 16 + tl;
            if (t < T) {
                const size_t hrow = ((size_t)e * T + t) * d_ff;
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const float v = ldexpf(h[rt][tt][i], -ee);
                    const _Float16 hv = (_Float16)v;
                    const int r = row0 + rt * 16 + n;
                    const size_t pos = hrow + (r & ~7) + sigma_pos(r & 7);
                    a.hh[pos] = hv;
                    a.hl[pos] = (_Float16)(v - (float)hv);
                }
                if (rw == 0 && n == 0) {
                    const float rwt = a.route_w ? a.route_w[(size_t)t * E + e] : 1.0f;
                    a.hf[((size_t)e * HG + hg) * a.t_pad + t] = ldexpf(rwt, ee);
                }
            }
        }
    }
}

// -------------------------------------------------------------------------
// Down for 16*RT*RW rows of d_model and 16*NTT tokens, summed over all
// experts.  Wave (rw, ks): rows rw*16*RT .. +16*RT of the block, (expert,
// group) pairs [ks*P/KS, (ks+1)*P/KS) of P = E * d_ff/group in ascending
// order; partials over ks are added in LDS in a fixed order.
template <int BITS, int KB, int NTT, int RT>
__global__ __launch_bounds__(512) void k_tb_down(TbArgs a)
{
    extern __shared__ float lds[];
    constexpr int kTot = RT * NTT * 4;
    constexpr int DEPTH = 2;
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
    size_t code_off[RT], scale_off[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int row = min(row0 + rt * 16 + n, d_model - 1);
        code_off[rt] = (size_t)row * rs + (size_t)(q * 8 * KB) * BITS / 8;
        scale_off[rt] = (size_t)row * Gd;
    }
    size_t hoff[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) hoff[tt] = (size_t)min(t0 + tt * 16 + n, T - 1) * d_ff + q * 8 * KB;

    struct Stage {
        TbStage<BITS, KB, NTT, RT> v;
        f32x4 f[NTT];  // factors of tokens 4q..4q+3 of each token tile
    };
    auto load = [&](Stage &st, int p) {
        const int e = p / Gd, g = p - e * Gd;
        const QPtr D = a.down[e];
        const size_t hb = (size_t)e * T * d_ff + (size_t)g * group;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
#pragma unroll
            for (int j = 0; j < KB; ++j) {
                st.v.ah[tt][j] = load_half8(a.hh + hb + hoff[tt] + 8 * j);
                st.v.al[tt][j] = load_half8(a.hl + hb + hoff[tt] + 8 * j);
            }
            st.f[tt] = *reinterpret_cast<const f32x4 *>(a.hf + ((size_t)e * Gd + g) * a.t_pad + t0 + tt * 16 + 4 * q);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            load_codes<BITS, KB>(D.codes + code_off[rt] + (size_t)g * group * BITS / 8, st.v.cw[rt]);
            st.v.s[rt] = D.scales[scale_off[rt] + g];
        }
    };

    f32x4 tot[RT][NTT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) tot[rt][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Every wave has at least one pair (KS <= P); unconditional ring loads.
    const int P = E * Gd;
    const int pbeg = ks * P / KS, pend = (ks + 1) * P / KS;
    Stage S[DEPTH];
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) load(S[i], min(pbeg + i, pend - 1));
    for (int base = pbeg; base < pend; base += DEPTH) {
#pragma unroll
        for (int i = 0; i < DEPTH; ++i) {
            const int p = base + i;
            if (p < pend) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    half8 bf[KB];
#pragma unroll
                    for (int j = 0; j < KB; ++j) bf[j] = code_frag<BITS, KB>(S[i].v.cw[rt], j);
                    const float s = S[i].v.s[rt] * QFormat<BITS>::kInvZ;
#pragma unroll
                    for (int tt = 0; tt < NTT; ++tt) {
                        const f32x4 acc = group_mfma<BITS, KB, NTT, RT>(S[i].v, bf, tt);
#pragma unroll
                        for (int r = 0; r < 4; ++r) tot[rt][tt][r] = fmaf(s * S[i].f[tt][r], acc[r], tot[rt][tt][r]);
                    }
                }
            }
            load(S[i], min(p + DEPTH, pend - 1));
        }
    }

    float *buf = lds + (size_t)rw * kTot * 64;
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
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i, ++r) {
                float v = tot[rt][tt][i];
                if (KS > 1) v += buf[r * 64 + lane];
                const int t = t0 + tt * 16 + 4 * q + i;
                const int row = row0 + rt * 16 + n;
                if (t < T && row < d_model) a.out[(size_t)t * d_model + row] = v;
            }
}

// -------------------------------------------------------------------------
// Tiled variants for more than 16 tokens: a block of 8 waves covers 64 tokens
// and 128 weight rows (one 16-row tile per wave).  For each quantisation group
// (gate_up) or (expert, group) pair (down), the block loads the 64 tokens'
// activation halves once, with coalesced 16-byte loads, into one of two LDS
// buffers; the waves read their MFMA fragments from LDS.  One barrier per
// step: a buffer is refilled only after every wave has passed the barrier
// that ends the step reading it.  Codes and scales are per wave, one step
// ahead in registers.
constexpr int kTileTokens = 64;
constexpr int kTileWaves = 8;
constexpr int kTilePrefetch = 3;   // steps of loads in registers (two in flight)

// The hardware hands consecutive workgroups to the 8 XCDs in turn, and each XCD
// has its own L2.  This maps the launch index to a logical one so that the
// blocks an XCD receives are consecutive logical blocks (which share weights);
// a bijection on [0, n) for any n.
__device__ __forceinline__ int xcd_logical(int b, int n)
{
    const int q = n >> 3, r = n & 7, x = b & 7, k = b >> 3;
    return x < r ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
}

// Halfs per token row of an LDS activation tile (16 bytes of padding, so that
// the 16 token rows of a fragment read fall into different banks).
__host__ __device__ constexpr int tile_stride(int group) { return group + 8; }
__host__ __device__ constexpr size_t tile_bytes(int group) { return (size_t)2 * kTileTokens * tile_stride(group) * 2; }

// Buffer loads: a resource (base, byte extent) in scalar registers, a fixed
// per-lane byte offset and a uniform byte offset per step, so that moving to the
// next step writes no vector registers.  Raw buffer (stride 0) with a 32-bit
// data format, as the memory instructions expect for untyped loads.
using BufRes = __amdgpu_buffer_rsrc_t;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

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

template <int BITS, int KB>
__device__ __forceinline__ void buf_load_codes(BufRes r, unsigned voff, unsigned soff, CodeWords<BITS, KB> &c)
{
    constexpr int n = CodeWords<BITS, KB>::kDwords;
    if constexpr (n == 4) {
        const uint4 v = buf_load16(r, voff, soff);
        c.w[0] = v.x;
        c.w[1] = v.y;
        c.w[2] = v.z;
        c.w[3] = v.w;
    } else if constexpr (n == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0);
        c.w[0] = v.x;
        c.w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < n; ++i) c.w[i] = buf_load4(r, voff + 4 * i, soff);
    }
}

// Cooperative load of one activation tile: 64 token rows x group = 32 * KB
// columns of the hi and the lo halves, KB 16-byte pieces per thread.  Piece i of
// a thread is fixed by the thread and i alone: its half (hi or lo; the same for
// the whole wave, since a half is 256 * KB pieces), its byte offset from the
// step's first column (below 2^30 for T <= 65536 and 8192 columns) and its
// place in LDS.
template <int KB>
struct TileRegs {
    uint4 v[KB];
};

template <int KB>
struct TileMap {
    unsigned off[KB];   // global byte offset of the piece within its half
    unsigned lds[KB];   // LDS byte offset of the piece within a tile buffer
    bool lo[KB];        // wave-uniform: the piece belongs to the lo half
};

template <int KB>
__device__ __forceinline__ void tile_map(TileMap<KB> &m, int wave, unsigned row_stride_bytes, int t0, int T)
{
    constexpr int group = 32 * KB, per_row = group / 8, per_half = kTileTokens * per_row;
    constexpr int st = tile_stride(group);
#pragma unroll
    for (int i = 0; i < KB; ++i) {
        const int c = threadIdx.x + 512 * i;
        const int hl = (wave * 64 + 512 * i) / per_half;
        const int rem = c - hl * per_half;
        const int tok = rem / per_row, part = rem - tok * per_row;
        m.lo[i] = hl != 0;
        m.off[i] = (unsigned)min(t0 + tok, T - 1) * row_stride_bytes + (unsigned)part * 16u;
        m.lds[i] = (unsigned)((hl * kTileTokens + tok) * st + part * 8) * 2u;
    }
}

// The pieces of the step whose first column is `col_bytes` into each row.
template <int KB>
__device__ __forceinline__ void tile_load(TileRegs<KB> &r, const TileMap<KB> &m, BufRes hi, BufRes lo,
                                          unsigned col_bytes)
{
#pragma unroll
    for (int i = 0; i < KB; ++i) r.v[i] = buf_load16(m.lo[i] ? lo : hi, m.off[i], col_bytes);
}

template <int KB>
__device__ __forceinline__ void tile_store(const TileRegs<KB> &r, const TileMap<KB> &m, _Float16 *tile)
{
#pragma unroll
    for (int i = 0; i < KB; ++i) *reinterpret_cast<uint4 *>(reinterpret_cast<uint8_t *>(tile) + m.lds[i]) = r.v[i];
}

// A fragments of token tile tt, K-block j, hi and lo, from an LDS tile.
__device__ __forceinline__ void tile_frags(const _Float16 *tile, int group, int tt, int j, int KB, half8 &h, half8 &l)
{
    const int st = tile_stride(group);
    const int lane = threadIdx.x & 63, q = lane >> 4, n = lane & 15;
    const _Float16 *p = tile + (tt * 16 + n) * st + q * 8 * KB + 8 * j;
    h = load_half8(p);
    l = load_half8(p + kTileTokens * st);
}

template <int BITS, int KB, int PF>
__global__ __launch_bounds__(512) void k_tb_gate_up_tiled(TbArgs a)
{
    constexpr int NTT = kTileTokens / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    const int group = a.group, d_model = a.d_model, d_ff = a.d_ff, T = a.T, E = a.n_experts;
    const size_t tb_bytes = tile_bytes(group);
    _Float16 *tiles = reinterpret_cast<_Float16 *>(smem);
    float *mx = reinterpret_cast<float *>(smem + 2 * tb_bytes);  // [waves][NTT][16]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int G = d_model / group, HG = d_ff / group;
    const int NTB = (T + kTileTokens - 1) / kTileTokens;
    const int RB = (d_ff + 16 * kTileWaves - 1) / (16 * kTileWaves);
    int b = xcd_logical(blockIdx.x, gridDim.x);
    const int tb = b % NTB;
    b /= NTB;
    const int rb = b % RB;
    const int e = b / RB;
    const int t0 = tb * kTileTokens;
    const int wrow0 = rb * 16 * kTileWaves + wave * 16;   // this wave's first d_ff row
    // Lane offsets (32-bit: a matrix has at most 8192 x 8192 entries) and
    // buffer resources; a step moves only the uniform offsets.
    const unsigned row = (unsigned)min(wrow0 + n, d_ff - 1);
    const unsigned coff = row * (unsigned)(d_model * BITS / 8) + (unsigned)(q * 8 * KB * BITS / 8);
    const unsigned soff = row * (unsigned)G * 4u;
    const size_t cbytes = (size_t)d_ff * d_model * BITS / 8, sbytes = (size_t)d_ff * G * 4;
    const BufRes cr[2] = {buf_res(a.gate[e].codes, cbytes), buf_res(a.up[e].codes, cbytes)};
    const BufRes sr[2] = {buf_res(a.gate[e].scales, sbytes), buf_res(a.up[e].scales, sbytes)};
    const BufRes xhr = buf_res(a.xh, (size_t)T * d_model * 2), xlr = buf_res(a.xl, (size_t)T * d_model * 2);
    TileMap<KB> tm;
    tile_map<KB>(tm, wave, (unsigned)d_model * 2u, t0, T);

    // Register ring of PF steps: the activation pieces this thread stores into
    // LDS and the wave's codes and scales, PF - 1 steps ahead of the step being
    // computed; LDS holds two steps.  The loop is branch-free so that the
    // compiler's load waits are exact: loads past the last group repeat it,
    // and the steps past the end (at most PF - 1) are computed with scale 0.
    struct GuStage {
        TileRegs<KB> tr;
        CodeWords<BITS, KB> cw[2];
        float sc[2];
    };
    GuStage S[PF];
    auto load_step = [&](GuStage &st, int g) {
        const unsigned gc = (unsigned)min(g, G - 1);
        tile_load<KB>(st.tr, tm, xhr, xlr, gc * (unsigned)group * 2u);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            buf_load_codes<BITS, KB>(cr[m], coff, gc * (unsigned)(group * BITS / 8), st.cw[m]);
            st.sc[m] = __uint_as_float(buf_load4(sr[m], soff, gc * 4u));
        }
    };

    f32x4 tot[2][NTT];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) tot[m][tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int i = 0; i < PF; ++i) load_step(S[i], i);
    tile_store<KB>(S[0].tr, tm, tiles);
    __syncthreads();
    for (int base = 0; base < G; base += PF) {
#pragma unroll
        for (int i = 0; i < PF; ++i) {
            const int g = base + i;
            const _Float16 *tile = tiles + (size_t)(g & 1) * (tb_bytes / 2);
            half8 bf[2][KB];
            float s[2];
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
                for (int j = 0; j < KB; ++j) bf[m][j] = code_frag<BITS, KB>(S[i].cw[m], j);
                s[m] = g < G ? S[i].sc[m] * QFormat<BITS>::kInvZ : 0.0f;
            }
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) {
                f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
                for (int j = 0; j < KB; ++j) {
                    half8 h, l;
                    tile_frags(tile, group, tt, j, KB, h, l);
#pragma unroll
                    for (int m = 0; m < 2; ++m) {
                        acc[m] = mfma(h, bf[m][j], acc[m]);
                        acc[m] = mfma(l, bf[m][j], acc[m]);
                    }
                }
#pragma unroll
                for (int m = 0; m < 2; ++m)
#pragma unroll
                    for (int r = 0; r < 4; ++r) tot[m][tt][r] = fmaf(s[m], acc[m][r], tot[m][tt][r]);
            }
            tile_store<KB>(S[(i + 1) % PF].tr, tm, tiles + (size_t)((g + 1) & 1) * (tb_bytes / 2));
            load_step(S[i], g + PF);
            __syncthreads();
        }
    }

    // hidden = SiLU(gate) * up; per-token maxima over this wave's 16 rows.
    float h[NTT][4];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = min(t0 + tt * 16 + 4 * q + i, T - 1);
            const int xe = a.xe[t];
            const float gv = ldexpf(tot[0][tt][i], xe), uv = ldexpf(tot[1][tt][i], xe);
            h[tt][i] = wrow0 + n < d_ff ? silu(gv) * uv : 0.0f;
            const float m = row16_max(fabsf(h[tt][i]));
            if (n == 0) mx[(wave * NTT + tt) * 16 + 4 * q + i] = m;
        }
    __syncthreads();
    if (wrow0 >= d_ff) return;
    const int wpg = group / 16;                       // waves per H group
    const int w0 = wave - wave % wpg;
    const int hg = (rb * 16 * kTileWaves + w0 * 16) / group;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tl = 4 * q + i;
            float m = 0.0f;
            for (int w = w0; w < w0 + wpg; ++w) m = fmaxf(m, mx[(w * NTT + tt) * 16 + tl]);
            const int ee = norm_exponent(m);
            const int t = t0 + tt * 16 + tl;
            if (t < T) {
                const float v = ldexpf(h[tt][i], -ee);
                const _Float16 hv = (_Float16)v;
                const int r = wrow0 + n;
                const size_t pos = ((size_t)e * T + t) * d_ff + (r & ~7) + sigma_pos(r & 7);
                a.hh[pos] = hv;
                a.hl[pos] = (_Float16)(v - (float)hv);
                if (wave == w0 && n == 0) {
                    const float rwt = a.route_w ? a.route_w[(size_t)t * E + e] : 1.0f;
                    a.hf[((size_t)e * HG + hg) * a.t_pad + t] = ldexpf(rwt, ee);
                }
            }
        }
}

// Down, tiled: block (token tile, row block, split) sums the (expert, group)
// pairs of its split; with more than one split each writes its partial sums to
// part[split][T][d_model] and k_tb_sum adds them in split order (deterministic).
template <int BITS, int KB, int PF>
__global__ __launch_bounds__(512) void k_tb_down_tiled(TbArgs a)
{
    constexpr int NTT = kTileTokens / 16;
    extern __shared__ __align__(16) unsigned char smem[];
    const int group = a.group, d_model = a.d_model, d_ff = a.d_ff, T = a.T, E = a.n_experts;
    const size_t tb_bytes = tile_bytes(group);
    _Float16 *tiles = reinterpret_cast<_Float16 *>(smem);
    float *fac = reinterpret_cast<float *>(smem + 2 * tb_bytes);  // [2][64]
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q = lane >> 4, n = lane & 15;
    const int Gd = d_ff / group;
    const int NTB = (T + kTileTokens - 1) / kTileTokens;
    const int RB = (d_model + 16 * kTileWaves - 1) / (16 * kTileWaves);
    int bid = xcd_logical(blockIdx.x, gridDim.x);
    const int tb = bid % NTB;
    bid /= NTB;
    const int rb = bid % RB;
    const int ks = bid / RB;
    const int t0 = tb * kTileTokens;
    const int wrow0 = rb * 16 * kTileWaves + wave * 16;
    const unsigned row = (unsigned)min(wrow0 + n, d_model - 1);
    const unsigned coff = row * (unsigned)(d_ff * BITS / 8) + (unsigned)(q * 8 * KB * BITS / 8);
    const unsigned soff = row * (unsigned)Gd * 4u;
    const size_t cbytes = (size_t)d_model * d_ff * BITS / 8, sbytes = (size_t)d_model * Gd * 4;
    const size_t hbytes = (size_t)T * d_ff * 2;   // one expert's hidden half
    const BufRes fr_res = buf_res(a.hf, (size_t)E * Gd * a.t_pad * 4);
    TileMap<KB> tm;
    tile_map<KB>(tm, wave, (unsigned)d_ff * 2u, t0, T);
    const int P = E * Gd;
    const int p0 = (int)((long)ks * P / a.ks_dn), p1 = (int)((long)(ks + 1) * P / a.ks_dn);
    const int NP = p1 - p0;
    float *dst = a.ks_dn > 1 ? a.part + (size_t)ks * T * d_model : a.out;

    f32x4 tot[NTT];
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) tot[tt] = (f32x4){0.f, 0.f, 0.f, 0.f};

    if (NP > 0) {
        // Register ring of PF steps (hidden tile pieces, the 64 tokens' factors,
        // the wave's codes and scale), branch-free as in gate_up: loads past
        // the split's end repeat its last pair, and those steps count with
        // scale 0.
        struct DnStage {
            TileRegs<KB> tr;
            CodeWords<BITS, KB> cw;
            float fr, sc;
        };
        DnStage S[PF];
        auto load_step = [&](DnStage &st, int i) {
            const int p = p0 + min(i, NP - 1);
            const int e = p / Gd, g = p - e * Gd;
            const size_t ho = (size_t)e * T * d_ff;
            tile_load<KB>(st.tr, tm, buf_res(a.hh + ho, hbytes), buf_res(a.hl + ho, hbytes),
                          (unsigned)g * (unsigned)group * 2u);
            st.fr = __uint_as_float(buf_load4(fr_res, (unsigned)lane * 4u,
                                              (unsigned)(((size_t)e * Gd + g) * a.t_pad + t0) * 4u));
            buf_load_codes<BITS, KB>(buf_res(a.down[e].codes, cbytes), coff, (unsigned)g * (unsigned)(group * BITS / 8),
                                     st.cw);
            st.sc = __uint_as_float(buf_load4(buf_res(a.down[e].scales, sbytes), soff, (unsigned)g * 4u));
        };
        auto store_step = [&](const DnStage &st, int buf) {
            tile_store<KB>(st.tr, tm, tiles + (size_t)buf * (tb_bytes / 2));
            fac[buf * 64 + lane] = st.fr;
        };
#pragma unroll
        for (int i = 0; i < PF; ++i) load_step(S[i], i);
        store_step(S[0], 0);
        __syncthreads();
        for (int base = 0; base < NP; base += PF) {
#pragma unroll
            for (int i = 0; i < PF; ++i) {
                const int st = base + i;
                const int buf = st & 1;
                const _Float16 *tile = tiles + (size_t)buf * (tb_bytes / 2);
                half8 bf[KB];
#pragma unroll
                for (int j = 0; j < KB; ++j) bf[j] = code_frag<BITS, KB>(S[i].cw, j);
                const float s = st < NP ? S[i].sc * QFormat<BITS>::kInvZ : 0.0f;
#pragma unroll
                for (int tt = 0; tt < NTT; ++tt) {
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < KB; ++j) {
                        half8 h, l;
                        tile_frags(tile, group, tt, j, KB, h, l);
                        acc = mfma(h, bf[j], acc);
                        acc = mfma(l, bf[j], acc);
                    }
                    const f32x4 f = *reinterpret_cast<const f32x4 *>(fac + buf * 64 + tt * 16 + 4 * q);
#pragma unroll
                    for (int r = 0; r < 4; ++r) tot[tt][r] = fmaf(s * f[r], acc[r], tot[tt][r]);
                }
                store_step(S[(i + 1) % PF], buf ^ 1);
                load_step(S[i], st + PF);
                __syncthreads();
            }
        }
    }
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + tt * 16 + 4 * q + i;
            const int r = wrow0 + n;
            if (t < T && r < d_model) dst[(size_t)t * d_model + r] = tot[tt][i];
        }
}

// out = sum over the down splits of their partial sums, in split order.  The
// partial slabs are 16-byte aligned (T * d_model is a multiple of 32); out is
// only 4-byte aligned, so it is written one float at a time.
__global__ __launch_bounds__(256) void k_tb_sum(const float *__restrict__ part, int splits, size_t count,
                                                float *__restrict__ out)
{
    const size_t n4 = count / 4;
    for (size_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        float4 acc = reinterpret_cast<const float4 *>(part)[i];
        for (int s = 1; s < splits; ++s) {
            const float4 v = reinterpret_cast<const float4 *>(part + (size_t)s * count)[i];
            acc.x += v.x;
            acc.y += v.y;
            acc.z += v.z;
            acc.w += v.w;
        }
        out[4 * i] = acc.x;
        out[4 * i + 1] = acc.y;
        out[4 * i + 2] = acc.z;
        out[4 * i + 3] = acc.w;
    }
}

template <int BITS, int KB>
hipError_t launch_tb_tiled(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(k_tb_prep, dim3((unsigned)a.T), dim3(256), 0, st, a.x, a.d_model, a.xh, a.xl, a.xe);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_gate_up_tiled<BITS, KB, kTilePrefetch>), dim3(pl.gu_blocks), dim3(64 * kTileWaves),
                       pl.gu_lds, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_down_tiled<BITS, KB, kTilePrefetch>), dim3(pl.dn_blocks), dim3(64 * kTileWaves),
                       pl.dn_lds, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.ks_dn > 1) {
        const size_t count = (size_t)a.T * a.d_model;
        const unsigned blocks = (unsigned)std::min<size_t>((count / 4 + 255) / 256 + 1, 2048);
        hipLaunchKernelGGL(k_tb_sum, dim3(blocks), dim3(256), 0, st, a.part, a.ks_dn, count, a.out);
        err = hipGetLastError();
    }
    return err;
}

template <int BITS, int KB, int NTT, int RTG, int RTD>
hipError_t launch_tb_kernels(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    hipLaunchKernelGGL(k_tb_prep, dim3((unsigned)a.T), dim3(256), 0, st, a.x, a.d_model, a.xh, a.xl, a.xe);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_gate_up<BITS, KB, NTT, RTG>), dim3(pl.gu_blocks), dim3(64 * pl.gu_waves), pl.gu_lds,
                       st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((k_tb_down<BITS, KB, NTT, RTD>), dim3(pl.dn_blocks), dim3(64 * pl.dn_waves), pl.dn_lds, st,
                       a);
    return hipGetLastError();
}

template <int BITS, int KB>
hipError_t launch_tb_kb(const TbPlan &pl, const TbArgs &a, hipStream_t st)
{
    // gate_up row tiles: 4 for 16-token tiles and 64-column groups (one wave per
    // group), else 2 (more would not fit the registers); down: 4 row tiles for
    // 16-token tiles, 2 for 32.
    if (pl.ntt == 1) {
        if constexpr (KB == 2)
            if (pl.rt_gu == 4) return launch_tb_kernels<BITS, KB, 1, 4, 4>(pl, a, st);
        return launch_tb_kernels<BITS, KB, 1, 2, 4>(pl, a, st);
    }
    if constexpr (KB <= 2)
        if (pl.ntt == kTileTokens / 16) return launch_tb_tiled<BITS, KB>(pl, a, st);
    return launch_tb_kernels<BITS, KB, 2, 2, 2>(pl, a, st);
}

}  // namespace

// Dynamic LDS per block is kept within 64 KB.
constexpr size_t kMaxBlockLds = 64 * 1024;

// Splits of the tiled down kernel's (expert, group) pairs over blocks: enough
// to give about two 8-wave blocks per compute unit, at most 8.
int batch_down_splits(int d_model, int T)
{
    if (T <= 16) return 1;
    const long blocks = (long)((d_model + 16 * kTileWaves - 1) / (16 * kTileWaves)) *
                        ((T + kTileTokens - 1) / kTileTokens);
    int s = 1;
    while (s < 8 && blocks * s < 512) s *= 2;
    return s;
}

bool plan_batch(int bits, int group, int d_model, int d_ff, int n_experts, int T, TbPlan *pl)
{
    if (T < 2 || n_experts < 1) return false;
    const int kb = group / 32;
    if (bits == 4 ? (kb < 1 || kb > 4) : (kb != 2 && kb != 4)) return false;
    if (d_model % group || d_ff % group) return false;
    TbPlan p{};
    if (T > 16 && (group == 32 || group == 64)) {
        // Tiled kernels: 64 tokens x 128 rows per 8-wave block.
        p.ntt = kTileTokens / 16;
        const long ntb = (T + kTileTokens - 1) / kTileTokens;
        const int rows = 16 * kTileWaves;
        p.gu_waves = p.dn_waves = kTileWaves;
        p.gu_blocks = (long)n_experts * ((d_ff + rows - 1) / rows) * ntb;
        p.ks_dn = std::min(batch_down_splits(d_model, T), n_experts * (d_ff / group));
        p.dn_blocks = (long)((d_model + rows - 1) / rows) * ntb * p.ks_dn;
        p.gu_lds = 2 * tile_bytes(group) + (size_t)kTileWaves * (kTileTokens / 16) * 16 * 4;
        p.dn_lds = 2 * tile_bytes(group) + 2 * 64 * 4;
        if (p.gu_lds > kMaxBlockLds || p.dn_lds > kMaxBlockLds) return false;
        *pl = p;
        return true;
    }
    p.ntt = T <= 16 ? 1 : 2;
    const int ntb = (T + 16 * p.ntt - 1) / (16 * p.ntt);
    const int G = d_model / group;
    // gate_up: the block covers one quantisation group of d_ff rows.
    p.rt_gu = (p.ntt == 1 && kb == 2) ? 4 : 2;
    p.rw_gu = group / (16 * p.rt_gu);
    if (p.rw_gu < 1 || p.rw_gu > 8 || p.rw_gu * 16 * p.rt_gu != group) return false;
    const long gu_blocks = (long)n_experts * (d_ff / group) * ntb;
    const int gu_tot = 2 * p.rt_gu * p.ntt * 4;   // accumulator floats per lane
    const size_t gu_buf = (size_t)p.rw_gu * gu_tot * 64 * 4;
    const size_t gu_max = (size_t)p.rw_gu * p.ntt * 16 * 4;
    p.ks_gu = 1;
    while (p.ks_gu < 8 && p.rw_gu * p.ks_gu * 2 <= 8 && p.ks_gu * 2 <= G && gu_buf + gu_max <= kMaxBlockLds &&
           gu_blocks * p.rw_gu * p.ks_gu < 2048)
        p.ks_gu *= 2;
    p.gu_waves = p.rw_gu * p.ks_gu;
    p.gu_blocks = gu_blocks;
    p.gu_lds = (p.ks_gu > 1 ? gu_buf : 0) + gu_max;
    // down: the block covers 16*rt*rw_dn rows of d_model; waves split the
    // (expert, group) pairs.
    const int rt_dn = p.ntt == 1 ? 4 : 2;
    p.rw_dn = 1;
    const int P = n_experts * (d_ff / group);
    const int rows_per_block = 16 * rt_dn * p.rw_dn;
    p.dn_blocks = (long)((d_model + rows_per_block - 1) / rows_per_block) * ntb;
    p.ks_dn = 1;
    while (p.ks_dn < 8 && p.ks_dn * 2 <= P && p.dn_blocks * p.ks_dn < 2048) p.ks_dn *= 2;
    p.dn_waves = p.rw_dn * p.ks_dn;
    p.dn_lds = p.ks_dn > 1 ? (size_t)p.rw_dn * rt_dn * p.ntt * 4 * 64 * 4 : 0;
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
