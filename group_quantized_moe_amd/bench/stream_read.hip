// Measurement helpers for bench.py (not part of libsmoe.so's ABI): a plain
// streaming read of a device buffer, the bandwidth a kernel that only reads
// its bytes once can reach on this GPU at a given size (the decode group's
// two kernels are compared with it on the same number of bytes in the same
// run), and a register-only run of one matrix instruction, the rate that
// instruction sustains on this GPU (the token batch's matrix work is compared
// with it).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRateThreads = 256;
constexpr int kChains = 4;   // independent accumulators per wave

// Every wave runs kChains independent accumulator chains of one MFMA form
// `iters` times on register operands: no memory traffic, nothing but the
// matrix instruction's own issue rate.  shape 0: v_mfma_f32_16x16x32_f16
// (16384 flops), 1: v_mfma_f32_32x32x16_f16 (32768 flops).
template <int SHAPE>
__global__ __launch_bounds__(kRateThreads) void k_mfma_rate(int iters, unsigned *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const half8 a = {(_Float16)(lane * 1e-3f), (_Float16)1.0f, (_Float16)0.5f, (_Float16)0.25f,
                     (_Float16)1.0f, (_Float16)2.0f, (_Float16)0.0f, (_Float16)1.0f};
    const half8 b = a * (_Float16)0.5f;
    float tot = 0.0f;
    if constexpr (SHAPE == 0) {
        f32x4 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = (f32x4){0.0f, 0.0f, 0.0f, (float)c};
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < kChains; ++c) tot += acc[c][0] + acc[c][3];
    } else {
        f32x16 acc[kChains];
#pragma unroll
        for (int c = 0; c < kChains; ++c) {
            acc[c] = (f32x16){};
            acc[c][0] = (float)c;
        }
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < kChains; ++c) tot += acc[c][0] + acc[c][15];
    }
    if (tot == 1234.5f) sink[0] = 1u;
}

constexpr int kThreads = 256;
constexpr int kUnroll = 4;   // 16-byte loads in flight per thread per pass

// Each thread reads kUnroll 16-byte pieces per pass, a block's pieces being
// consecutive, and the grid strides over the buffer.  The XOR of everything
// read is stored only if it equals a value no input here produces, so the
// loads cannot be dropped and nothing is written.
__global__ __launch_bounds__(kThreads) void k_stream_read(const uint4 *__restrict__ p, size_t n16,
                                                          unsigned *__restrict__ sink)
{
    size_t i = (size_t)blockIdx.x * kThreads * kUnroll + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * kThreads * kUnroll;
    unsigned acc = 0;
    for (; i < n16; i += stride) {
        uint4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            v[u] = j < n16 ? p[j] : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

}  // namespace

extern "C" {

// Reads nbytes (a multiple of 16, 16-byte aligned) at p.  blocks_per_cu == 0:
// one pass, one block per kUnroll * 256 pieces; else a grid of blocks_per_cu
// blocks per compute unit striding over the buffer.  sink: one device word.
// Returns 0, or -1 for bad arguments, -2 if the launch failed.
int smoe_bench_stream_read(const void *p, size_t nbytes, unsigned *sink, int blocks_per_cu, void *stream)
{
    if (!p || !sink || nbytes == 0 || nbytes % 16 || (reinterpret_cast<uintptr_t>(p) & 15) || blocks_per_cu < 0)
        return -1;
    const size_t n16 = nbytes / 16;
    long grid;
    if (blocks_per_cu == 0) {
        grid = (long)((n16 + kThreads * kUnroll - 1) / (kThreads * kUnroll));
    } else {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
            return -2;
        grid = (long)cus * blocks_per_cu;
    }
    if (grid < 1 || grid > (1L << 30)) return -1;
    hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(kThreads), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint4 *>(p), n16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Launches the matrix-instruction run: blocks_per_cu blocks of 256 threads
// per compute unit, `iters` iterations of kChains MFMAs per wave.  Its flops
// are grid * 4 waves * iters * kChains * (16384 for shape 0, 32768 for 1).
// Returns 0, or -1 for bad arguments, -2 if the launch failed.
int smoe_bench_mfma_rate(int shape, int blocks_per_cu, int iters, unsigned *sink, void *stream)
{
    if (!sink || shape < 0 || shape > 1 || blocks_per_cu < 1 || blocks_per_cu > 64 || iters < 1) return -1;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return -2;
    const dim3 grid((unsigned)(cus * blocks_per_cu)), block(kRateThreads);
    if (shape == 0)
        hipLaunchKernelGGL(k_mfma_rate<0>, grid, block, 0, (hipStream_t)stream, iters, sink);
    else
        hipLaunchKernelGGL(k_mfma_rate<1>, grid, block, 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
