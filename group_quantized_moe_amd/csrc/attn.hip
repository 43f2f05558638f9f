// Decode attention block for one token (Metal Compute Kernels page of the
// S-MoE docs, section "GPU-Resident Decode Attention"): the q/k/v
// projections, a per-head RMS norm of q and k with 1e-6 under the root, RoPE,
// k and v appended to the f32 KV cache, causal grouped-query attention of the
// new token over positions 0..pos, and the output projection.
//
// Launch sequence (one stream, no host synchronisation):
//   1. the three projections as one batched bf16 matvec launch;
//   2. k_attn_prep: one wave per head (query heads, then KV heads): RMS norm,
//      rotation, and for KV heads the cache append of k and v;
//   3. k_attn_partial: one block per (32-position chunk, KV head) serves all
//      the query heads of that KV head (the group shares every K and V row it
//      stages in LDS): scores, the chunk's max and exp-sum per head, and the
//      chunk's unnormalised output rows;
//   4. k_attn_combine: one block per query head merges the chunks into the
//      attention output, summing in a fixed order (deterministic);
//   5. the output projection as a bf16 matvec.
// Everything is f32 but the rotation angles, which are formed and reduced in
// f64: pos * base^(-2i/hd) reaches thousands of radians, where an f32 angle
// would be off by about 1e-4.
#include "common.h"
#include "launch.h"

namespace smoe {
namespace {

constexpr int kAttnChunk = 32;    // cache positions per partial block
constexpr int kAttnThreads = 256;

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Max / sum over the 32 lanes of a half wave.
__device__ __forceinline__ float half_max(float v)
{
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 32));
    return v;
}
__device__ __forceinline__ float half_sum(float v)
{
#pragma unroll
    for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 32);
    return v;
}

// One wave per head.  Lane l owns the rotation pairs i = l + 64 p (i < HD/2),
// each pair (i, i + HD/2) as the rotation takes it.
template <int HD>
__global__ __launch_bounds__(kAttnThreads) void k_attn_prep(AttnArgs a)
{
    constexpr int HALF = HD / 2;
    constexpr int NP = (HALF + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int head = blockIdx.x * (kAttnThreads / 64) + (threadIdx.x >> 6);
    const int H = a.n_head, KV = a.n_kv;
    if (head >= H + KV) return;   // whole wave; no barrier in this kernel
    const bool is_q = head < H;
    const int g = head - H;
    const float *src = is_q ? a.q + (size_t)head * HD : a.k + (size_t)g * HD;
    const float *gain = is_q ? a.q_norm : a.k_norm;
    float va[NP], vb[NP];
    float ss = 0.0f;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int i = lane + 64 * p;
        va[p] = i < HALF ? src[i] : 0.0f;
        vb[p] = i < HALF ? src[i + HALF] : 0.0f;
        ss += va[p] * va[p] + vb[p] * vb[p];
    }
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)HD + 1e-6f);
    float *dst = is_q ? a.qr + (size_t)head * HD : a.k_cache + ((size_t)g * a.max_ctx + a.pos) * HD;
    const double l2b = log2(a.rope_base);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int i = lane + 64 * p;
        if (i >= HALF) continue;
        const float x0 = va[p] * inv * gain[i], x1 = vb[p] * inv * gain[i + HALF];
        const double ang = (double)a.pos * exp2(-(2.0 * i / HD) * l2b);
        double sd, cd;
        sincos(ang, &sd, &cd);
        const float s = (float)sd, c = (float)cd;
        dst[i] = x0 * c - x1 * s;
        dst[i + HALF] = x0 * s + x1 * c;
    }
    if (!is_q) {
        const float *vs = a.v + (size_t)g * HD;
        float *vd = a.v_cache + ((size_t)g * a.max_ctx + a.pos) * HD;
        for (int d = lane; d < HD; d += 64) vd[d] = vs[d];
    }
}

// Chunk c of the window 0..pos for KV head g and its G query heads.  LDS rows
// are padded by 4 floats so that the 32 rows a half wave reads at one column
// fall in different banks.
template <int HD>
__global__ __launch_bounds__(kAttnThreads) void k_attn_partial(AttnArgs a)
{
    constexpr int RS = HD + 4;
    __shared__ __align__(16) float Ks[kAttnChunk * RS];
    __shared__ __align__(16) float Vs[kAttnChunk * RS];
    __shared__ __align__(16) float Qs[kMaxAttnGroup * HD];
    __shared__ float P[kMaxAttnGroup * kAttnChunk];
    const int c = blockIdx.x, g = blockIdx.y;
    const int G = a.n_head / a.n_kv;
    const int n_ctx = a.pos + 1;
    const int j0 = c * kAttnChunk;
    const int nj = min(kAttnChunk, n_ctx - j0);
    const int tid = threadIdx.x;
    // Stage the chunk's K and V rows (rows past the window are zero) and the group's queries.
    const float *Kg = a.k_cache + ((size_t)g * a.max_ctx + j0) * HD;
    const float *Vg = a.v_cache + ((size_t)g * a.max_ctx + j0) * HD;
    for (int e = tid; e < kAttnChunk * HD / 4; e += kAttnThreads) {
        const int j = e / (HD / 4), d4 = e - j * (HD / 4);
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        if (j < nj) {
            kv = reinterpret_cast<const float4 *>(Kg + (size_t)j * HD)[d4];
            vv = reinterpret_cast<const float4 *>(Vg + (size_t)j * HD)[d4];
        }
        *reinterpret_cast<float4 *>(Ks + j * RS + 4 * d4) = kv;
        *reinterpret_cast<float4 *>(Vs + j * RS + 4 * d4) = vv;
    }
    const float *Qg = a.qr + (size_t)g * G * HD;
    for (int e = tid; e < G * HD / 4; e += kAttnThreads)
        reinterpret_cast<float4 *>(Qs)[e] = reinterpret_cast<const float4 *>(Qg)[e];
    __syncthreads();
    // Scores and the per-head softmax pieces: thread (hq, j), j = lane % 32.
    const int j = tid & (kAttnChunk - 1);
    const float scale = 1.0f / sqrtf((float)HD);
    for (int hq = tid / kAttnChunk; hq < kMaxAttnGroup; hq += kAttnThreads / kAttnChunk) {
        // hq is uniform over the half wave, so the exits below keep half waves whole.
        if (hq >= G) break;
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
        P[hq * kAttnChunk + j] = p;
        if (j == 0) {
            float *ml = a.part_ml + (((size_t)g * a.n_chunks + c) * G + hq) * 2;
            ml[0] = m;
            ml[1] = l;
        }
    }
    __syncthreads();
    // Unnormalised output rows: o[hq][d] = sum_j P[hq][j] V[j][d].
    for (int e = tid; e < G * HD; e += kAttnThreads) {
        const int hq = e / HD, d = e - hq * HD;
        float o = 0.0f;
#pragma unroll 8
        for (int jj = 0; jj < kAttnChunk; ++jj) o += P[hq * kAttnChunk + jj] * Vs[jj * RS + d];
        a.part_o[(((size_t)g * a.n_chunks + c) * G + hq) * HD + d] = o;
    }
}

// Query head h: merge the chunks.  att[h][d] = sum_c e^(m_c - M) o_c[d] /
// sum_c e^(m_c - M) l_c, M = max_c m_c.  The 512 threads take column d and one
// of P = 512 / HD contiguous chunk ranges each (independent loads, several in
// flight), and the P range sums are added in range order: deterministic.
constexpr int kCombineThreads = 512;
template <int HD>
__global__ __launch_bounds__(kCombineThreads) void k_attn_combine(AttnArgs a)
{
    constexpr int P = kCombineThreads / HD;
    __shared__ float red[kCombineThreads / 64];
    __shared__ float part_o[P][HD];
    __shared__ float part_l[P];
    const int h = blockIdx.x, t = threadIdx.x;
    const int G = a.n_head / a.n_kv, g = h / G, hq = h - g * G;
    const int nc = (a.pos + 1 + kAttnChunk - 1) / kAttnChunk;
    const float *ml = a.part_ml + ((size_t)g * a.n_chunks * G + hq) * 2;
    const size_t cstride = (size_t)G * 2;
    float m = -INFINITY;
    for (int c = t; c < nc; c += kCombineThreads) m = fmaxf(m, ml[c * cstride]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    float M = red[0];
#pragma unroll
    for (int w = 1; w < kCombineThreads / 64; ++w) M = fmaxf(M, red[w]);
    const int d = t % HD, pr = t / HD;
    const int c0 = (int)((long)pr * nc / P), c1 = (int)((long)(pr + 1) * nc / P);
    const float *po = a.part_o + ((size_t)g * a.n_chunks * G + hq) * HD + d;
    float L = 0.0f, o = 0.0f;
#pragma unroll 8
    for (int c = c0; c < c1; ++c) {
        const float w = expf(ml[c * cstride] - M);
        L += w * ml[c * cstride + 1];
        o += w * po[(size_t)c * G * HD];
    }
    part_o[pr][d] = o;
    if (d == 0) part_l[pr] = L;
    __syncthreads();
    if (pr == 0) {
        float os = part_o[0][d], ls = part_l[0];
#pragma unroll
        for (int q = 1; q < P; ++q) {
            os += part_o[q][d];
            ls += part_l[q];
        }
        a.att[(size_t)h * HD + d] = os / ls;
    }
}

template <int HD>
hipError_t launch_attn_hd(const AttnArgs &a, hipStream_t st)
{
    const int heads = a.n_head + a.n_kv;
    hipLaunchKernelGGL(k_attn_prep<HD>, dim3((heads + 3) / 4), dim3(kAttnThreads), 0, st, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int nc = (a.pos + 1 + kAttnChunk - 1) / kAttnChunk;
    hipLaunchKernelGGL(k_attn_partial<HD>, dim3(nc, a.n_kv), dim3(kAttnThreads), 0, st, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(k_attn_combine<HD>, dim3(a.n_head), dim3(kCombineThreads), 0, st, a);
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
