// Decode attention block for one token (Metal Compute Kernels page of the
// S-MoE docs, section "GPU-Resident Decode Attention"): the q/k/v
// projections, a per-head RMS norm of q and k with 1e-6 under the root, RoPE,
// k and v appended to the f32 KV cache, causal grouped-query attention of the
// new token over positions 0..pos, and the output projection.
//
// Launch sequence (one stream, no host synchronisation):
//   1. the three projections as one batched bf16 matvec launch;
//   2. k_attn_partial: one block per (32-position chunk, KV head) serves all
//      the query heads of that KV head (the group shares every K and V row it
//      stages in LDS).  It normalises and rotates those queries itself (a few
//      thousand flops per block, cheaper than a launch), and the block whose
//      chunk holds the new token also normalises and rotates k and appends k
//      and v to the caches.  Then the scores, the chunk's max and exp-sum per
//      head, and the chunk's unnormalised output rows;
//   3. k_attn_combine: blocks of 32 columns of a query head merge the chunks
//      into the attention output, summing in a fixed order (deterministic);
//   4. the output projection as a bf16 matvec.
// Everything is f32 but the rotation angles, which are formed and reduced to
// [-pi, pi] in f64: pos * base^(-2i/hd) reaches thousands of radians, where an
// f32 angle would be off by about 1e-4.
#include "common.h"
#include "launch.h"

namespace smoe {
namespace {

constexpr int kAttnChunk = 32;     // cache positions per partial block
constexpr int kAttnThreads = 512;  // 8 waves: two query heads per wave, one (head, row) score per thread

// Sums and maxima over aligned groups of W lanes (W = 32 or 64), every lane
// of a group receiving the result: DPP within 16-lane rows, then one or two
// cross-row shuffles.
__device__ __forceinline__ float wave_sum(float v) { return lane_group_sum<64>(v); }
__device__ __forceinline__ float half_sum(float v) { return lane_group_sum<32>(v); }
__device__ __forceinline__ float half_max(float v)
{
    v = fmaxf(v, dpp<0xB1>(v));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp<0x4E>(v));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp<0x141>(v));   // row_half_mirror
    v = fmaxf(v, dpp<0x140>(v));   // row_mirror
    return fmaxf(v, __shfl_xor(v, 16));
}

// RMS norm and rotation of one head's hd values held as pairs (i, i + HD/2)
// by the lanes of a wave (lane l: pairs i = l + 64 p); cs / sn are the pair
// angles' cosine and sine; lanes past the last pair hold zeros.
template <int NP>
__device__ __forceinline__ void norm_rotate(const float (&x0)[NP], const float (&x1)[NP], const float (&g0)[NP],
                                            const float (&g1)[NP], const float (&cs)[NP], const float (&sn)[NP],
                                            int hd, float (&y0)[NP], float (&y1)[NP])
{
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) ss += x0[p] * x0[p] + x1[p] * x1[p];
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)hd + 1e-6f);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const float a0 = x0[p] * inv * g0[p], a1 = x1[p] * inv * g1[p];
        y0[p] = a0 * cs[p] - a1 * sn[p];
        y1[p] = a0 * sn[p] + a1 * cs[p];
    }
}

// Chunk c of the window 0..pos for KV head g and its G query heads, with the
// norm and rotation of those queries done in the block (each of the 8 waves
// takes heads w and w + 8), and, in the block whose chunk holds pos, the norm,
// rotation and cache append of the new k and v.  LDS rows of K and V are
// padded by 4 floats so that the rows a half wave reads at one column fall in
// different banks.  Heads past G are zero rows.
template <int HD>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(AttnArgs a)
{
    constexpr int RS = HD + 4;
    constexpr int HALF = HD / 2;
    constexpr int NP = (HALF + 63) / 64;
    constexpr int GP = kMaxAttnGroup;
    __shared__ __align__(16) float Ks[kAttnChunk * RS];
    __shared__ __align__(16) float Vs[kAttnChunk * RS];
    __shared__ __align__(16) float Qs[GP * HD];
    __shared__ __align__(16) float Pt[kAttnChunk * GP];   // [j][head]
    const int c = blockIdx.x, g = blockIdx.y;
    const int G = a.n_head / a.n_kv;
    const int n_ctx = a.pos + 1;
    const int j0 = c * kAttnChunk;
    const int nj = min(kAttnChunk, n_ctx - j0);
    const int jnew = a.pos - j0;   // row of the new token in this chunk (in range only in the last chunk)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // Every global load first, so that one round trip covers them: the chunk's
    // cached K and V rows (rows past the window are zero; the new token's row
    // is computed below), and the raw queries of this wave's heads.
    constexpr int NKV = kAttnChunk * HD / 4 / kAttnThreads;   // float4 of K (and of V) per thread
    constexpr int HPW = GP / (kAttnThreads / 64);              // query heads per wave
    const float *Kg = a.k_cache + ((size_t)g * a.max_ctx + j0) * HD;
    const float *Vg = a.v_cache + ((size_t)g * a.max_ctx + j0) * HD;
    float4 kr[NKV], vr[NKV];
#pragma unroll
    for (int r = 0; r < NKV; ++r) {
        const int e = tid + r * kAttnThreads, j = e / (HD / 4), d4 = e - j * (HD / 4);
        kr[r] = vr[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < nj && j != jnew) {
            kr[r] = reinterpret_cast<const float4 *>(Kg + (size_t)j * HD)[d4];
            vr[r] = reinterpret_cast<const float4 *>(Vg + (size_t)j * HD)[d4];
        }
    }
    float qx0[HPW][NP], qx1[HPW][NP];
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        const float *src = a.q + ((size_t)g * G + min(wave + (kAttnThreads / 64) * k, G - 1)) * HD;
#pragma unroll
        for (int p = 0; p < NP; ++p) {   // lanes past the last pair hold zeros (they add nothing to the norm)
            const int i = min(lane + 64 * p, HALF - 1);
            qx0[k][p] = lane + 64 * p < HALF ? src[i] : 0.0f;
            qx1[k][p] = lane + 64 * p < HALF ? src[i + HALF] : 0.0f;
        }
    }
    // Pair angles: pos * base^(-2i/hd) formed in f64 and reduced to [-pi, pi]
    // there, so that the f32 sine and cosine see a small argument.
    float cs[NP], sn[NP], qg0[NP], qg1[NP];
    const double l2b = log2(a.rope_base);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int i = min(lane + 64 * p, HALF - 1);
        const double ang = (double)a.pos * exp2(-(2.0 * i / HD) * l2b);
        const double twopi = 6.283185307179586476925286766559;
        const float r = (float)(ang - twopi * rint(ang / twopi));
        sincosf(r, &sn[p], &cs[p]);
        qg0[p] = a.q_norm[i];
        qg1[p] = a.q_norm[i + HALF];
    }
#pragma unroll
    for (int r = 0; r < NKV; ++r) {   // row jnew is written by wave 0 below, and only there
        const int e = tid + r * kAttnThreads, j = e / (HD / 4), d4 = e - j * (HD / 4);
        if (j != jnew) {
            *reinterpret_cast<float4 *>(Ks + j * RS + 4 * d4) = kr[r];
            *reinterpret_cast<float4 *>(Vs + j * RS + 4 * d4) = vr[r];
        }
    }
#pragma unroll
    for (int k = 0; k < HPW; ++k) {
        const int hq = wave + (kAttnThreads / 64) * k;
        float y0[NP], y1[NP];
        norm_rotate<NP>(qx0[k], qx1[k], qg0, qg1, cs, sn, HD, y0, y1);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int i = lane + 64 * p;
            if (i < HALF) {
                Qs[hq * HD + i] = hq < G ? y0[p] : 0.0f;
                Qs[hq * HD + i + HALF] = hq < G ? y1[p] : 0.0f;
            }
        }
    }
    if (jnew >= 0 && jnew < kAttnChunk && wave == 0) {   // the chunk holding the new token
        float x0[NP], x1[NP], g0[NP], g1[NP], y0[NP], y1[NP];
        const float *src = a.k + (size_t)g * HD;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int i = min(lane + 64 * p, HALF - 1);
            x0[p] = lane + 64 * p < HALF ? src[i] : 0.0f;
            x1[p] = lane + 64 * p < HALF ? src[i + HALF] : 0.0f;
            g0[p] = a.k_norm[i];
            g1[p] = a.k_norm[i + HALF];
        }
        norm_rotate<NP>(x0, x1, g0, g1, cs, sn, HD, y0, y1);
        float *kd = a.k_cache + ((size_t)g * a.max_ctx + a.pos) * HD;
        float *vd = a.v_cache + ((size_t)g * a.max_ctx + a.pos) * HD;
        const float *vs = a.v + (size_t)g * HD;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            const int i = lane + 64 * p;
            if (i < HALF) {
                Ks[jnew * RS + i] = kd[i] = y0[p];
                Ks[jnew * RS + i + HALF] = kd[i + HALF] = y1[p];
            }
        }
        for (int d = lane; d < HD; d += 64) Vs[jnew * RS + d] = vd[d] = vs[d];
    }
    __syncthreads();
    // Score of head hq against row j (thread (hq, j); hq uniform over the half
    // wave), then each head's max and exp-sum over the chunk's rows.
    {
        static_assert(kAttnThreads == GP * kAttnChunk, "one (head, row) score per thread");
        const int j = tid & (kAttnChunk - 1), hq = tid / kAttnChunk;
        const float scale = 1.0f / sqrtf((float)HD);
        float dot = 0.0f;
#pragma unroll 8
        for (int d4 = 0; d4 < HD / 4; ++d4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(Ks + j * RS + 4 * d4);
            const float4 q4 = *reinterpret_cast<const float4 *>(Qs + hq * HD + 4 * d4);
            dot += k4.x * q4.x + k4.y * q4.y + k4.z * q4.z + k4.w * q4.w;
        }
        const float s = j < nj ? dot * scale : -INFINITY;
        const float m = half_max(s);
        const float p = j < nj ? expf(s - m) : 0.0f;
        const float l = half_sum(p);
        Pt[j * GP + hq] = hq < G ? p : 0.0f;
        if (j == 0 && hq < G) {
            float *ml = a.part_ml + (((size_t)g * a.n_chunks + c) * G + hq) * 2;
            ml[0] = m;
            ml[1] = l;
        }
    }
    __syncthreads();
    // Unnormalised output rows o[hq][d] = sum_j P[hq][j] V[j][d]: thread
    // (column d, head group) reads each V value once for HPT heads.
    {
        constexpr int HPT = GP * HD / kAttnThreads;   // heads per thread: 4 (HD 128) or 2 (HD 64)
        const int d = tid % HD, h0 = (tid / HD) * HPT;
        float o[HPT];
#pragma unroll
        for (int k = 0; k < HPT; ++k) o[k] = 0.0f;
#pragma unroll 8
        for (int j = 0; j < kAttnChunk; ++j) {
            const float v = Vs[j * RS + d];
#pragma unroll
            for (int k = 0; k < HPT; ++k) o[k] += Pt[j * GP + h0 + k] * v;
        }
#pragma unroll
        for (int k = 0; k < HPT; ++k)
            if (h0 + k < G) a.part_o[(((size_t)g * a.n_chunks + c) * G + h0 + k) * HD + d] = o[k];
    }
}

// Query head h, columns 32y .. 32y + 31 (block (h, y)): merge the chunks.
// att[h][d] = sum_c e^(m_c - M) o_c[d] / sum_c e^(m_c - M) l_c, M = max_c m_c.
// The 1024 threads take column d and one of P = 32 contiguous chunk ranges
// each (independent loads, all in flight), and the P range sums are added in
// range order: deterministic.  Four blocks per head of 128 (one per head,
// each thread a range of 16 chunks, took 5.7 us against 4.6 us).
constexpr int kCombineThreads = 1024;
constexpr int kCombineCols = 32;   // columns of a head per block
template <int HD>
__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(AttnArgs a)
{
    constexpr int P = kCombineThreads / kCombineCols;
    __shared__ float red[kCombineThreads / 64];
    __shared__ float part_o[P][kCombineCols];
    __shared__ float part_l[P];
    const int h = blockIdx.x, t = threadIdx.x;
    const int G = a.n_head / a.n_kv, g = h / G, hq = h - g * G;
    const int nc = (a.pos + 1 + kAttnChunk - 1) / kAttnChunk;
    const float *ml = a.part_ml + ((size_t)g * a.n_chunks * G + hq) * 2;
    const size_t cstride = (size_t)G * 2;
    float m = -INFINITY;
    for (int c = t; c < nc; c += kCombineThreads) m = fmaxf(m, ml[c * cstride]);
    m = half_max(m);
    m = fmaxf(m, __shfl_xor(m, 32));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) M = fmaxf(M, red[w]);
    const int dl = t % kCombineCols, pr = t / kCombineCols;
    const int d = blockIdx.y * kCombineCols + dl;
    const int c0 = (int)((long)pr * nc / P), c1 = (int)((long)(pr + 1) * nc / P);
    const float *po = a.part_o + ((size_t)g * a.n_chunks * G + hq) * HD + d;
    float L = 0.0f, o = 0.0f;
#pragma unroll 16
    for (int c = c0; c < c1; ++c) {
        const float w = expf(ml[c * cstride] - M);
        L += w * ml[c * cstride + 1];
        o += w * po[(size_t)c * G * HD];
    }
    part_o[pr][dl] = o;
    if (dl == 0) part_l[pr] = L;
    __syncthreads();
    if (pr == 0) {
        float os = part_o[0][dl], ls = part_l[0];
#pragma unroll
        for (int q = 1; q < P; ++q) {
            os += part_o[q][dl];
            ls += part_l[q];
        }
        a.att[(size_t)h * HD + d] = os / ls;
    }
}

template <int HD>
hipError_t launch_attn_hd(const AttnArgs &a, hipStream_t st)
{
    const int nc = (a.pos + 1 + kAttnChunk - 1) / kAttnChunk;
    hipLaunchKernelGGL(k_attn_partial<HD>, dim3(nc, a.n_kv), dim3(kAttnThreads), 0, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_attn_combine<HD>, dim3(a.n_head, HD / kCombineCols), dim3(kCombineThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int attn_chunks(int max_ctx) { return (max_ctx + kAttnChunk - 1) / kAttnChunk; }

hipError_t launch_attn_core(const AttnArgs &a, hipStream_t st)
{
    switch (a.head_dim) {
    case 64: return launch_attn_hd<64>(a, st);
    case 128: return launch_attn_hd<128>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace smoe
