// Measurement helper for bench.py (not part of libsmoe.so's ABI): a plain
// streaming read of a device buffer, the bandwidth a kernel that only reads
// its bytes once can reach on this GPU at a given size.  The decode group's
// two kernels are compared with it on the same number of bytes in the same
// run.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

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

}  // extern "C"
